// Per-kernel event timing for profiling (thread-local; off unless enabled).
#include <cstring>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_profile.h"

namespace kda {
namespace {

struct Pending {
    const char* name;
    hipEvent_t start, stop;
    bool stop_recorded;  // false if recording the stop event failed (a pooled event may hold an old time)
};

struct State {
    bool on = false;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;
};

thread_local State g_state;

hipEvent_t take_event() {
    if (!g_state.pool.empty()) {
        hipEvent_t e = g_state.pool.back();
        g_state.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t s) : slot_(-1), stream_(s) {
    if (!g_state.on) return;
    hipEvent_t a = take_event(), b = take_event();
    if (a == nullptr || b == nullptr) return;
    if (hipEventRecord(a, s) != hipSuccess) return;
    g_state.pending.push_back({name, a, b, false});
    slot_ = static_cast<int>(g_state.pending.size()) - 1;
}

LaunchTimer::~LaunchTimer() {
    if (slot_ >= 0) g_state.pending[slot_].stop_recorded = hipEventRecord(g_state.pending[slot_].stop, stream_) == hipSuccess;
}

// ---------------------------------------------------------------------------
// Peak-rate probes: what the matrix cores and HBM sustain on this device,
// measured beside the published peaks.

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));

// Each wave runs `iters` rounds of four independent matrix-core products
// (16 x 16 outputs, fp32 accumulators), so the matrix core of every SIMD
// always has work queued.  Operands depend on the lane so nothing folds; one
// value per thread is written so nothing is dead.
__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float* __restrict__ out) {
    const int t = threadIdx.x;
    probe_bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(1.f + 1e-3f * static_cast<float>((t + e) & 7));
        b[e] = static_cast<__bf16>(1e-3f * static_cast<float>((t * 3 + e) & 15));
    }
    probe_f32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<int64_t>(blockIdx.x) * 256 + t] = s;
}

__global__ __launch_bounds__(256) void probe_mfma_f32_kernel(int iters, float* __restrict__ out) {
    const int t = threadIdx.x;
    const float a = 1.f + 1e-3f * static_cast<float>(t & 7), b = 1e-3f * static_cast<float>((t * 3) & 15);
    probe_f32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<int64_t>(blockIdx.x) * 256 + t] = s;
}

// Streaming read of n16 16-byte words (grid-stride), one sum per thread out.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         float* __restrict__ out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    uint32_t acc = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = static_cast<float>(acc & 0xffff);
}

}  // namespace kda

extern "C" {

int kda_probe_peak(int32_t kind, int32_t blocks, int32_t iters, const void* src, int64_t src_bytes, float* out,
                   void* stream) {
    if (blocks <= 0 || out == nullptr) return KDA_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    kda::LaunchTimer timer(kind == 0 ? "probe_mfma_bf16" : kind == 1 ? "probe_mfma_f32" : "probe_read", s);
    if (kind == 0 || kind == 1) {
        if (iters <= 0) return KDA_ERR_INVALID_ARGUMENT;
        if (kind == 0)
            hipLaunchKernelGGL(kda::probe_mfma_bf16_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
        else
            hipLaunchKernelGGL(kda::probe_mfma_f32_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
    } else if (kind == 2) {
        if (src == nullptr || src_bytes <= 0 || src_bytes % 16 != 0 ||
            reinterpret_cast<uintptr_t>(src) % 16 != 0)
            return KDA_ERR_INVALID_ARGUMENT;
        hipLaunchKernelGGL(kda::probe_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                           src_bytes / 16, out);
    } else {
        return KDA_ERR_INVALID_ARGUMENT;
    }
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_profile_enable(int on) {
    kda::g_state.on = on != 0;
    return KDA_OK;
}

int kda_profile_collect(kda_kernel_time_t* out, int max_entries) {
    using kda::g_state;
    std::vector<kda_kernel_time_t> agg;
    int status = KDA_OK;
    for (const kda::Pending& p : g_state.pending) {
        float ms = 0.f;
        if (!p.stop_recorded || hipEventSynchronize(p.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
            status = KDA_ERR_HIP;
        kda_kernel_time_t* hit = nullptr;
        for (auto& a : agg)
            if (std::strncmp(a.name, p.name, sizeof(a.name)) == 0) hit = &a;
        if (hit == nullptr) {
            kda_kernel_time_t z;
            std::memset(&z, 0, sizeof(z));
            std::strncpy(z.name, p.name, sizeof(z.name) - 1);
            agg.push_back(z);
            hit = &agg.back();
        }
        hit->launches += 1;
        hit->total_ms += ms;
        g_state.pool.push_back(p.start);
        g_state.pool.push_back(p.stop);
    }
    g_state.pending.clear();
    const int n = static_cast<int>(agg.size());
    for (int i = 0; i < n && i < max_entries; ++i) out[i] = agg[i];
    return status == KDA_OK ? n : -status;
}

}  // extern "C"
