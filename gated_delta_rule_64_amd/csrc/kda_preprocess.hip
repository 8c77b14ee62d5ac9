// Fused preprocess of the KDA token mixer: causal short conv (4 taps) on q,
// k and v, L2 norm of q and k per head, and the two gates (the page
// "Ling-3.0-flash: a 124B open MoE that runs like a 5B and reaches for 1M
// tokens", section "KDA: constant-size memory over a very long context": q
// and k pass a short conv and an L2 norm, v a conv; a softplus gate gives the
// decay and a sigmoid the write strength; 4 taps per the "Every architecture
// field" table of the page "Ling 3.0 Flash").
//
// Streaming design: the op reads each raw input once and writes each output
// once, so it is bound by HBM.  A workgroup covers 64 tokens of one head.  Its
// four waves split the work by tensor (q, k, v, gates), which keeps each
// lane's registers small (one filter, one history) and the occupancy high.
// Inside a wave, a group of 16 lanes covers a 128-channel row of one token
// with 16-byte accesses (8 channels per lane) and walks a run of 16
// consecutive tokens, keeping the three previous raw rows of its channels in
// registers: the conv reads every input row once, plus a three-row halo per
// run.  The L2 norm reduces over the 16 lanes with shuffles.  Runs respect
// sequence boundaries: history before a sequence start is the caller's conv
// state or zero.  A second tiny kernel, ordered after the first on the
// stream, rewrites the conv state, so the read of the old state never races
// with the write of the new one.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_profile.h"

namespace kda {
namespace {

constexpr int kRun = 16;                 // tokens per 16-lane group
constexpr int kTile = kRun * 4;          // tokens per workgroup (4 groups per wave)

// One lane's 8 channels of a row, as loaded (bf16: 16 B, fp32: 32 B).  Rows
// are loaded a whole batch ahead of their use and unpacked when consumed.
template <typename XT> struct Raw;
template <> struct Raw<bf16> {
    uint4 v;
    static constexpr int kBatch = 16;  // the whole 16-token run in flight
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void unpack(float (&x)[8], bool keep) const {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = keep ? __uint_as_float(w[i] << 16) : 0.f;
            x[2 * i + 1] = keep ? __uint_as_float(w[i] & 0xffff0000u) : 0.f;
        }
    }
};
template <> struct Raw<float> {
    float4 a, b;
    static constexpr int kBatch = 8;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void unpack(float (&x)[8], bool keep) const {
        const float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = keep ? y[i] : 0.f;
    }
};


template <typename XT>
struct PrepK {
    int64_t T;
    int H, dk, dv, N;
    const int32_t* cu;
    const XT *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b;
    const float* cs;
    XT *q_out, *k_out, *v_out;
    float *la_out, *beta_out;
};

// Loads are branch-free: an inactive lane or a row past the end reads a
// valid clamped address and selects zero, so the compiler can keep several
// rows in flight instead of waiting on each load inside a branch.
template <typename XT>
__device__ __forceinline__ void load_row(const XT* base, int64_t t, int64_t width, int64_t off, bool keep,
                                         float (&x)[8]) {
    ld8(base + t * width + off, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = keep ? x[i] : 0.f;
}

// history row of position tau (-3..-1) of sequence n: conv state or zero
__device__ __forceinline__ void load_hist(const float* cs, int n, int tau, int64_t cs_width, int64_t off,
                                          bool keep, float (&x)[8]) {
    if (cs != nullptr) {  // uniform over the whole launch
        ld8(cs + (static_cast<int64_t>(n) * 3 + (3 + tau)) * cs_width + off, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = keep ? x[i] : 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
}

// one of q, k, v: conv (+ L2 norm for q and k) over a run of tokens
template <typename XT>
__device__ __forceinline__ void conv_run(const PrepK<XT>& a, const XT* src, const XT* wts, XT* dst,
                                         int64_t width, int64_t off, int64_t cs_off, bool act, bool norm,
                                         int64_t t_begin, int64_t t_end) {
    float w[8][4];
    {
        float wl[32];
        ld8(wts + off * 4, *reinterpret_cast<float(*)[8]>(&wl[0]));
        ld8(wts + off * 4 + 8, *reinterpret_cast<float(*)[8]>(&wl[8]));
        ld8(wts + off * 4 + 16, *reinterpret_cast<float(*)[8]>(&wl[16]));
        ld8(wts + off * 4 + 24, *reinterpret_cast<float(*)[8]>(&wl[24]));
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[c][j] = act ? wl[c * 4 + j] : 0.f;
    }
    const int64_t cs_width = static_cast<int64_t>(a.H) * (2 * a.dk + a.dv);
    int n = a.cu ? find_seq(a.cu, a.N, t_begin) : 0;
    int64_t seq_start = a.cu ? a.cu[n] : 0;
    int64_t seq_end = a.cu ? a.cu[n + 1] : a.T;
    float hst[3][8];  // raw rows t-3, t-2, t-1
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t pos = t_begin - 3 + m;
        const bool in_seq = pos >= seq_start;
        float xi[8], xh[8];
        load_row(src, pos < 0 ? 0 : pos, width, off, act && in_seq, xi);
        const int tau = in_seq ? -1 : static_cast<int>(pos - seq_start);
        load_hist(a.cs, n, tau, cs_width, cs_off + off, act && !in_seq, xh);
#pragma unroll
        for (int i = 0; i < 8; ++i) hst[m][i] = xi[i] + xh[i];  // one of the two is zero
    }
    constexpr int kBatch = Raw<XT>::kBatch;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kBatch) {
        Raw<XT> raw[kBatch];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int64_t t = t0 + r < t_end ? t0 + r : t_end - 1;
            raw[r].load(src + t * width + off);
        }
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int64_t t = t0 + r;
            if (t >= t_end) continue;  // (not break: the loop must unroll so raw[] stays in registers)
            float xr[8];
            raw[r].unpack(xr, act);
            if (t >= seq_end) {
                // entering a later sequence: skip empty ones, restart the history
                do {
                    ++n;
                    seq_start = a.cu[n];
                    seq_end = a.cu[n + 1];
                } while (seq_end <= t);
#pragma unroll
                for (int m = 0; m < 3; ++m) load_hist(a.cs, n, m - 3, cs_width, cs_off + off, act, hst[m]);
            }
            float y[8];
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                y[c] = w[c][0] * hst[0][c] + w[c][1] * hst[1][c] + w[c][2] * hst[2][c] + w[c][3] * xr[c];
                ss += y[c] * y[c];
                hst[0][c] = hst[1][c];
                hst[1][c] = hst[2][c];
                hst[2][c] = xr[c];
            }
            if (norm) {
#pragma unroll
                for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 16);
                const float inv = 1.f / sqrtf(ss + kL2Eps);
#pragma unroll
                for (int c = 0; c < 8; ++c) y[c] *= inv;
            }
            if (act) st8(dst + t * width + off, y);
        }
    }
}

template <typename XT>
__global__ __launch_bounds__(256) void preprocess_kernel(PrepK<XT> a) {
    // heads vary fastest across workgroups, so the workgroups in flight
    // together cover whole token rows (all heads) of the [T, H*d] inputs
    const int64_t bid = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t tiles = (a.T + kTile - 1) / kTile;
    if (bid >= tiles * a.H) return;
    const int h = static_cast<int>(bid % a.H);
    const int wave = threadIdx.x >> 6;  // 0: q, 1: k, 2: v, 3: gates
    const int grp = (threadIdx.x >> 4) & 3;
    const int li = threadIdx.x & 15;
    const int64_t t_begin = (bid / a.H) * kTile + grp * kRun;
    if (t_begin >= a.T) return;  // whole 16-lane group leaves together
    const int64_t t_end = min(t_begin + kRun, a.T);
    const int64_t wk = static_cast<int64_t>(a.H) * a.dk, wv = static_cast<int64_t>(a.H) * a.dv;
    const bool aq = 8 * li < a.dk, av = 8 * li < a.dv;
    // lanes past the head size keep a valid (clamped) column and store nothing
    const int64_t off_k = static_cast<int64_t>(h) * a.dk + (aq ? 8 * li : 0);
    const int64_t off_v = static_cast<int64_t>(h) * a.dv + (av ? 8 * li : 0);
    if (wave < 3) {
        const bool is_v = wave == 2;
        const XT* src = wave == 0 ? a.q_in : (wave == 1 ? a.k_in : a.v_in);
        const XT* wts = wave == 0 ? a.w_q : (wave == 1 ? a.w_k : a.w_v);
        XT* dst = wave == 0 ? a.q_out : (wave == 1 ? a.k_out : a.v_out);
        conv_run(a, src, wts, dst, is_v ? wv : wk, is_v ? off_v : off_k, wave * wk, is_v ? av : aq, !is_v,
                 t_begin, t_end);
    } else {
        constexpr int kBatch = Raw<XT>::kBatch;
        for (int64_t t0 = t_begin; t0 < t_end; t0 += kBatch) {
            Raw<XT> raw[kBatch];
            float xb[kBatch];
#pragma unroll
            for (int r = 0; r < kBatch; ++r) {
                const int64_t t = t0 + r < t_end ? t0 + r : t_end - 1;
                raw[r].load(a.g + t * wk + off_k);
                xb[r] = ld(a.b + t * a.H + h);
            }
#pragma unroll
            for (int r = 0; r < kBatch; ++r) {
                const int64_t t = t0 + r;
                if (t >= t_end) continue;
                float x[8], la[8];
                raw[r].unpack(x, aq);
#pragma unroll
                for (int c = 0; c < 8; ++c) la[c] = -softplus_fast(x[c]);
                if (aq) st8(a.la_out + t * wk + off_k, la);
                if (li == 0) a.beta_out[t * a.H + h] = sigmoid_fast(xb[r]);
            }
        }
    }
}

// conv state after the call: the last three raw tokens of each sequence,
// reaching back into the old state for sequences shorter than three.
template <typename XT>
__global__ __launch_bounds__(256) void conv_state_kernel(PrepK<XT> a, int blocks_per_seq) {
    const int n = blockIdx.x / blocks_per_seq;
    const int64_t c = static_cast<int64_t>(blockIdx.x % blocks_per_seq) * 256 + threadIdx.x;
    const int64_t wk = static_cast<int64_t>(a.H) * a.dk, wv = static_cast<int64_t>(a.H) * a.dv;
    const int64_t width = 2 * wk + wv;
    if (c >= width) return;
    const XT* src;
    int64_t ch, stride;
    if (c < wk) { src = a.q_in; ch = c; stride = wk; }
    else if (c < 2 * wk) { src = a.k_in; ch = c - wk; stride = wk; }
    else { src = a.v_in; ch = c - 2 * wk; stride = wv; }
    const int64_t s0 = a.cu ? a.cu[n] : 0;
    const int64_t L = (a.cu ? a.cu[n + 1] : a.T) - s0;
    float* cs = const_cast<float*>(a.cs) + static_cast<int64_t>(n) * 3 * width + c;
    float old[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) old[m] = cs[m * width];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t tau = L - 3 + m;
        cs[m * width] = tau >= 0 ? ld(src + (s0 + tau) * stride + ch) : old[L + m];
    }
}

template <typename XT>
hipError_t launch_conv_state(const PrepK<XT>& k, hipStream_t s) {
    if (k.cs == nullptr || k.N <= 0) return hipSuccess;
    const int64_t width = static_cast<int64_t>(k.H) * (2 * k.dk + k.dv);
    const int bps = static_cast<int>((width + 255) / 256);
    LaunchTimer timer("conv_state", s);
    hipLaunchKernelGGL((conv_state_kernel<XT>), dim3(static_cast<unsigned>(k.N) * bps), dim3(256), 0, s, k, bps);
    return hipGetLastError();
}

template <typename XT>
PrepK<XT> prep_args(const PreprocessArgs& a) {
    PrepK<XT> k;
    k.T = a.T; k.H = a.H; k.dk = a.dk; k.dv = a.dv; k.N = a.N; k.cu = a.cu;
    k.q_in = static_cast<const XT*>(a.q_in); k.k_in = static_cast<const XT*>(a.k_in);
    k.v_in = static_cast<const XT*>(a.v_in); k.w_q = static_cast<const XT*>(a.w_q);
    k.w_k = static_cast<const XT*>(a.w_k); k.w_v = static_cast<const XT*>(a.w_v);
    k.g = static_cast<const XT*>(a.g); k.b = static_cast<const XT*>(a.b);
    k.cs = a.conv_state;
    k.q_out = static_cast<XT*>(a.q_out); k.k_out = static_cast<XT*>(a.k_out);
    k.v_out = static_cast<XT*>(a.v_out);
    k.la_out = a.la_out; k.beta_out = a.beta_out;
    return k;
}

template <typename XT>
hipError_t launch_typed(const PreprocessArgs& a, hipStream_t s) {
    const PrepK<XT> k = prep_args<XT>(a);
    if (a.T > 0) {
        const int64_t blocks = (a.T + kTile - 1) / kTile * a.H;
        const int64_t gx = blocks < (1 << 20) ? blocks : (1 << 20);
        const int64_t gy = (blocks + gx - 1) / gx;
        LaunchTimer timer("preprocess", s);
        hipLaunchKernelGGL((preprocess_kernel<XT>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), dim3(256),
                           0, s, k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_conv_state<XT>(k, s);
}

}  // namespace

hipError_t launch_preprocess(const PreprocessArgs& a, hipStream_t s) {
    return a.x == DT::BF16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

hipError_t launch_conv_state_update(const PreprocessArgs& a, hipStream_t s) {
    return a.x == DT::BF16 ? launch_conv_state<bf16>(prep_args<bf16>(a), s)
                           : launch_conv_state<float>(prep_args<float>(a), s);
}

}  // namespace kda
