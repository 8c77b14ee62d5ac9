// Device-side helpers shared by the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bf16 values travel as their 16-bit patterns.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (the gfx950 conversion
// instruction; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// scalar load/store of an element type as fp32
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ void st(float* p, float x) { *p = x; }
__device__ __forceinline__ void st(bf16* p, float x) { p->bits = f32_to_bf16(x); }

// x rounded to element type T and back (what a store and reload of x gives)
template <typename T>
__device__ __forceinline__ float round_to(float x) { return x; }
template <>
__device__ __forceinline__ float round_to<bf16>(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// 8 consecutive elements (16 B for bf16, 32 B for fp32), 16-byte aligned
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16* p, float (&x)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> one word of two bf16 (lo in the low half), one packed conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void st8(bf16* p, const float (&x)[8]) {
    uint4 a;
    a.x = pack_bf16x2(x[0], x[1]);
    a.y = pack_bf16x2(x[2], x[3]);
    a.z = pack_bf16x2(x[4], x[5]);
    a.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = a;
}

// 4 consecutive elements
__device__ __forceinline__ void ld4(const float* p, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void ld4(const bf16* p, float (&x)[4]) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(a.x << 16);
    x[1] = __uint_as_float(a.x & 0xffff0000u);
    x[2] = __uint_as_float(a.y << 16);
    x[3] = __uint_as_float(a.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st4(bf16* p, const float (&x)[4]) {
    uint2 a;
    a.x = pack_bf16x2(x[0], x[1]);
    a.y = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2*>(p) = a;
}

// softplus(x) = log(1 + e^x) without overflow; -softplus is the log decay
__device__ __forceinline__ float softplus(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + expf(-x)); }
// sigmoid with the hardware exponential and reciprocal (about 2 ulp)
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// softplus(x) / ln 2 with the hardware base-2 exponential and logarithm
// (v_exp_f32, v_log_f32): log2(1 + e^x) = max(x, 0) log2(e) + log2(1 + 2^(-|x| log2 e)),
// and the log's argument lies in (1, 2], so it needs no range handling
__device__ __forceinline__ float softplus_log2(float x) {
    return fmaxf(x, 0.f) * kLog2e + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e));
}
__device__ __forceinline__ float softplus_fast(float x) { return softplus_log2(x) * kLn2; }

// the L2 norm's epsilon: x / sqrt(|x|^2 + eps)
constexpr float kL2Eps = 1e-6f;

// index of the sequence holding token t: the largest n with cu[n] <= t
// (empty sequences never hold a token, so ties resolve to the non-empty one)
__device__ __forceinline__ int find_seq(const int32_t* cu, int N, int64_t t) {
    int lo = 0, hi = N;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Cross-lane sums without the LDS path (a shuffle is an LDS round trip).
// x + x rotated by N lanes within each row of 16 (DPP row_ror)
template <int N>
__device__ __forceinline__ float row_ror_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
// x + x of the lane 16 away (rows 0 and 1, rows 2 and 3 exchanged): one
// v_permlane16_swap with both operands x returns the two rows of each pair
__device__ __forceinline__ float xor16_add(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + x of the lane 32 away (the two halves exchanged)
__device__ __forceinline__ float xor32_add(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over the lanes of the wave that agree in lane % S (S = 1, 2, 4, 8);
// every lane gets the sum of its class (the order of the additions differs
// between lanes, so lanes may differ in the last bit).
template <int S>
__device__ __forceinline__ float wave_sum_stride(float x) {
    static_assert(S == 1 || S == 2 || S == 4 || S == 8, "stride within a row of 16");
    if (S <= 1) x = row_ror_add<1>(x);
    if (S <= 2) x = row_ror_add<2>(x);
    if (S <= 4) x = row_ror_add<4>(x);
    x = row_ror_add<8>(x);
    return xor32_add(xor16_add(x));
}
// Sum over the whole wave, the same value in every lane (lane 0's)
__device__ __forceinline__ float wave_sum(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_sum_stride<1>(x))));
}

constexpr int kChunk = 64;  // tokens per chunk of the prefill

// Workgroup barrier for LDS traffic only.  __syncthreads() fences all memory
// at workgroup scope, which makes every wave wait for its outstanding global
// loads and stores (and LDS DMA copies) before the barrier.  This barrier
// waits only for the wave's own LDS operations (lgkmcnt 0); the compiler-only
// fences keep memory operations from moving across it.  A wave that needs
// its global->LDS copies to be visible waits for them (vmcnt) first.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// wait until this wave has no global memory operation in flight (vmcnt 0)
__device__ __forceinline__ void wait_vmem() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt and expcnt at their maxima
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace kda
