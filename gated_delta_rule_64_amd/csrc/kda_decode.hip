// Decode step of the KDA recurrence: one token per sequence, state in place.
//
// Per (sequence b, head h), with S the dk x dv fp32 state (the gated delta
// rule of the page "Ling-3.0-flash: a 124B open MoE that runs like a 5B and
// reaches for 1M tokens", section "KDA: constant-size memory over a very long
// context"):
//   S' = Diag(alpha) S;  u = S'^T k;  p = S'^T q;
//   S  = S' + beta k (v - u)^T;       o = S^T q = p + beta (q.k) (v - u);
//   y  = o * sigmoid(z).
//
// The step moves 2 x dk x dv x 4 bytes of state and a few hundred bytes of
// per-token vectors, so it is bound by HBM.  One 256-thread workgroup owns one
// (b, h): every thread holds a dk/(1024/dv) x 4 patch of the state in
// registers (64 floats at dk = dv = 128), so the state is read once and
// written once.  Rows are interleaved across row groups so that one wave's
// 16-byte loads cover adjacent full rows (contiguous, coalesced).  The two
// reductions over dk (u and p) run in registers, then across the row groups
// of a wave with lane shuffles, then across the four waves through LDS.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_profile.h"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(256) void decode_kernel(const XT* __restrict__ q,
                                                     const XT* __restrict__ k,
                                                     const XT* __restrict__ v,
                                                     const GT* __restrict__ la,
                                                     const GT* __restrict__ beta,
                                                     const XT* __restrict__ z,
                                                     float* __restrict__ state,
                                                     XT* __restrict__ out) {
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int NRG = 256 / CG;               // row groups
    constexpr int RPT = (DK + NRG - 1) / NRG;   // rows per thread
    constexpr int RG_PER_WAVE = 64 / CG;

    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_qk[4];
    __shared__ float s_red[4][CG][8];

    float* __restrict__ Sp = state + bh * (DK * DV);

    // 1. issue the whole state patch (plain loads: measured, non-temporal
    // loads of several 16-byte pieces per thread cut the read rate by a
    // quarter; the stores stay non-temporal, which measured faster)
    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) S[i] = *reinterpret_cast<const f32x4*>(Sp + r * DV + 4 * cg);
    }

    // 2. per-row vectors to LDS, q.k per wave
    float qk_part = 0.f;
    if (tid < DK) {
        const float kk = ld(k + bh * DK + tid);
        const float qq = ld(q + bh * DK + tid);
        s_k[tid] = kk;
        s_q[tid] = qq;
        s_a[tid] = expf(ld(la + bh * DK + tid));
        qk_part = kk * qq;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk_part += __shfl_xor(qk_part, off);
    if (lane == 0) s_qk[wave] = qk_part;
    const float bt = ld(beta + bh);
    __syncthreads();

    // 3. decay, then the two partial reductions over this thread's rows
    float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) {
            const float a = s_a[r], kk = s_k[r], qq = s_q[r];
            S[i].x *= a; S[i].y *= a; S[i].z *= a; S[i].w *= a;
            u[0] += S[i].x * kk; u[1] += S[i].y * kk; u[2] += S[i].z * kk; u[3] += S[i].w * kk;
            p[0] += S[i].x * qq; p[1] += S[i].y * qq; p[2] += S[i].z * qq; p[3] += S[i].w * qq;
        }
    }
    // across the row groups held by this wave
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] += __shfl_xor(u[c], off);
            p[c] += __shfl_xor(p[c], off);
        }
    }
    if ((rg % RG_PER_WAVE) == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_red[wave][cg][c] = u[c];
            s_red[wave][cg][4 + c] = p[c];
        }
    }
    __syncthreads();
    const float qk = s_qk[0] + s_qk[1] + s_qk[2] + s_qk[3];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u[c] = s_red[0][cg][c] + s_red[1][cg][c] + s_red[2][cg][c] + s_red[3][cg][c];
        p[c] = s_red[0][cg][4 + c] + s_red[1][cg][4 + c] + s_red[2][cg][4 + c] + s_red[3][cg][4 + c];
    }

    // 4. write: S = S' + beta k (v - u)^T, and the read o = p + (q.k) beta (v - u)
    float vv[4];
    ld4(v + bh * DV + 4 * cg, vv);
    float d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = bt * (vv[c] - u[c]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) {
            const float kk = s_k[r];
            f32x4 o4;
            o4.x = S[i].x + kk * d[0];
            o4.y = S[i].y + kk * d[1];
            o4.z = S[i].z + kk * d[2];
            o4.w = S[i].w + kk * d[3];
            __builtin_nontemporal_store(o4, reinterpret_cast<f32x4*>(Sp + r * DV + 4 * cg));
        }
    }
    if (rg == 0) {
        float o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = p[c] + qk * d[c];
        if (z != nullptr) {
            float zz[4];
            ld4(z + bh * DV + 4 * cg, zz);
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] *= sigmoid(zz[c]);
        }
        st4(out + bh * DV + 4 * cg, o);
    }
}

template <int DK, int DV, typename XT, typename GT>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H);
    if (grid == 0) return hipSuccess;
    LaunchTimer timer("decode", s);
    hipLaunchKernelGGL((decode_kernel<DK, DV, XT, GT>), dim3(grid), dim3(256), 0, s,
                       static_cast<const XT*>(a.q), static_cast<const XT*>(a.k),
                       static_cast<const XT*>(a.v), static_cast<const GT*>(a.la),
                       static_cast<const GT*>(a.beta), static_cast<const XT*>(a.z), a.state,
                       static_cast<XT*>(a.out));
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const DecodeArgs& a, hipStream_t s) {
    if (a.x == DT::BF16) {
        return a.gate == DT::BF16 ? launch_typed<DK, DV, bf16, bf16>(a, s)
                                  : launch_typed<DK, DV, bf16, float>(a, s);
    }
    return a.gate == DT::BF16 ? launch_typed<DK, DV, float, bf16>(a, s)
                              : launch_typed<DK, DV, float, float>(a, s);
}

template <int DK>
hipError_t launch_dk(const DecodeArgs& a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_dims<DK, 16>(a, s);
        case 32: return launch_dims<DK, 32>(a, s);
        case 64: return launch_dims<DK, 64>(a, s);
        case 128: return launch_dims<DK, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return launch_dk<16>(a, s);
        case 32: return launch_dk<32>(a, s);
        case 64: return launch_dk<64>(a, s);
        case 128: return launch_dk<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
