// Fused preprocess of the KDA token mixer: causal short conv (4 taps) on q,
// k and v, L2 norm of q and k per head, and the two gates (the page
// "Ling-3.0-flash: a 124B open MoE that runs like a 5B and reaches for 1M
// tokens", section "KDA: constant-size memory over a very long context": q
// and k pass a short conv and an L2 norm, v a conv; a softplus gate gives the
// decay and a sigmoid the write strength; 4 taps per the "Every architecture
// field" table of the page "Ling 3.0 Flash").
//
// Streaming design: the op reads each raw input once and writes each output
// once, so it is bound by HBM.  A group of 16 lanes covers one head's 128
// channels of a token row with 16-byte accesses (8 channels per lane), and
// walks a run of 16 consecutive tokens, keeping the three previous raw rows
// of its 8 channels in registers; the conv then reads every input row once
// (plus a three-row halo per run).  The L2 norm reduces over the 16 lanes
// with shuffles.  Runs respect sequence boundaries: history before a
// sequence start is the caller's conv state or zero.  A second tiny kernel,
// ordered after the first on the stream, rewrites the conv state, so the
// read of the old state never races with the write of the new one.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kRun = 16;                 // tokens per 16-lane group
constexpr int kGroups = 16;              // groups per workgroup
constexpr int kTile = kRun * kGroups;    // tokens per workgroup
constexpr float kL2Eps = 1e-6f;

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

template <typename XT>
__device__ __forceinline__ void load_row(const XT* base, int64_t t, int64_t width, int64_t off,
                                         bool active, float (&x)[8]) {
    if (active) {
        ld8(base + t * width + off, x);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
}

// history row of position tau (< 0) of sequence n: conv state or zero
__device__ __forceinline__ void load_hist(const float* cs, int n, int tau, int64_t cs_width,
                                          int64_t off, bool active, float (&x)[8]) {
    if (active && cs != nullptr) {
        const float* p = cs + (static_cast<int64_t>(n) * 3 + (3 + tau)) * cs_width + off;
        ld8(p, x);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
}

template <typename XT>
__global__ __launch_bounds__(256) void preprocess_kernel(PrepK<XT> a) {
    const int h = blockIdx.y;
    const int grp = threadIdx.x >> 4;
    const int li = threadIdx.x & 15;
    const int64_t t_begin = static_cast<int64_t>(blockIdx.x) * kTile + grp * kRun;
    if (t_begin >= a.T) return;  // whole 16-lane group leaves together
    const int64_t t_end = min(t_begin + kRun, a.T);

    const int dk = a.dk, dv = a.dv;
    const int64_t wk = static_cast<int64_t>(a.H) * dk, wv = static_cast<int64_t>(a.H) * dv;
    const int64_t cs_width = 2 * wk + wv;
    const bool aq = 8 * li < dk;  // lane covers q/k channels
    const bool av = 8 * li < dv;  // lane covers v channels
    const int64_t off_k = static_cast<int64_t>(h) * dk + 8 * li;
    const int64_t off_v = static_cast<int64_t>(h) * dv + 8 * li;

    // conv taps of this lane's 8 channels, for q, k, v
    float wq[8][4], wkk[8][4], wvv[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wq[c][j] = aq ? ld(a.w_q + (off_k + c) * 4 + j) : 0.f;
            wkk[c][j] = aq ? ld(a.w_k + (off_k + c) * 4 + j) : 0.f;
            wvv[c][j] = av ? ld(a.w_v + (off_v + c) * 4 + j) : 0.f;
        }
    }

    int n = a.cu ? find_seq(a.cu, a.N, t_begin) : 0;
    int64_t seq_start = a.cu ? a.cu[n] : 0;
    int64_t seq_end = a.cu ? a.cu[n + 1] : a.T;

    // history rows for positions t_begin-3 .. t_begin-1 (index 0 = oldest)
    float hq[3][8], hk[3][8], hv[3][8];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t pos = t_begin - 3 + m;
        if (pos >= seq_start) {
            load_row(a.q_in, pos, wk, off_k, aq, hq[m]);
            load_row(a.k_in, pos, wk, off_k, aq, hk[m]);
            load_row(a.v_in, pos, wv, off_v, av, hv[m]);
        } else {
            const int tau = static_cast<int>(pos - seq_start);  // -3 .. -1
            load_hist(a.cs, n, tau, cs_width, off_k, aq, hq[m]);
            load_hist(a.cs, n, tau, cs_width, wk + off_k, aq, hk[m]);
            load_hist(a.cs, n, tau, cs_width, 2 * wk + off_v, av, hv[m]);
        }
    }

    for (int64_t t0 = t_begin; t0 < t_end; t0 += 4) {
        // issue four rows of loads before using any of them
        float xq[4][8], xk[4][8], xv[4][8], xg[4][8];
        float xb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + r;
            const bool in = t < t_end;
            load_row(a.q_in, t, wk, off_k, in && aq, xq[r]);
            load_row(a.k_in, t, wk, off_k, in && aq, xk[r]);
            load_row(a.v_in, t, wv, off_v, in && av, xv[r]);
            load_row(a.g, t, wk, off_k, in && aq, xg[r]);
            xb[r] = (in && li == 0) ? ld(a.b + t * a.H + h) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + r;
            if (t >= t_end) break;
            if (t >= seq_end) {
                // entering a later sequence: skip empty ones, restart history
                do {
                    ++n;
                    seq_start = a.cu[n];
                    seq_end = a.cu[n + 1];
                } while (seq_end <= t);
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    load_hist(a.cs, n, m - 3, cs_width, off_k, aq, hq[m]);
                    load_hist(a.cs, n, m - 3, cs_width, wk + off_k, aq, hk[m]);
                    load_hist(a.cs, n, m - 3, cs_width, 2 * wk + off_v, av, hv[m]);
                }
            }
            float cq[8], ck[8], cv[8];
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                cq[c] = wq[c][0] * hq[0][c] + wq[c][1] * hq[1][c] + wq[c][2] * hq[2][c] + wq[c][3] * xq[r][c];
                ck[c] = wkk[c][0] * hk[0][c] + wkk[c][1] * hk[1][c] + wkk[c][2] * hk[2][c] + wkk[c][3] * xk[r][c];
                cv[c] = wvv[c][0] * hv[0][c] + wvv[c][1] * hv[1][c] + wvv[c][2] * hv[2][c] + wvv[c][3] * xv[r][c];
                ssq += cq[c] * cq[c];
                ssk += ck[c] * ck[c];
                hq[0][c] = hq[1][c]; hq[1][c] = hq[2][c]; hq[2][c] = xq[r][c];
                hk[0][c] = hk[1][c]; hk[1][c] = hk[2][c]; hk[2][c] = xk[r][c];
                hv[0][c] = hv[1][c]; hv[1][c] = hv[2][c]; hv[2][c] = xv[r][c];
            }
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) {
                ssq += __shfl_xor(ssq, off, 16);
                ssk += __shfl_xor(ssk, off, 16);
            }
            const float iq = 1.f / sqrtf(ssq + kL2Eps);
            const float ik = 1.f / sqrtf(ssk + kL2Eps);
            float la[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                cq[c] *= iq;
                ck[c] *= ik;
                la[c] = -softplus(xg[r][c]);
            }
            if (aq) {
                st8(a.q_out + t * wk + off_k, cq);
                st8(a.k_out + t * wk + off_k, ck);
                st8(a.la_out + t * wk + off_k, la);
            }
            if (av) st8(a.v_out + t * wv + off_v, cv);
            if (li == 0) a.beta_out[t * a.H + h] = sigmoid(xb[r]);
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
hipError_t launch_typed(const PreprocessArgs& a, hipStream_t s) {
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
    if (a.T > 0) {
        const int64_t tiles = (a.T + kTile - 1) / kTile;
        hipLaunchKernelGGL((preprocess_kernel<XT>), dim3(static_cast<unsigned>(tiles), a.H), dim3(256),
                           0, s, k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.conv_state != nullptr && a.N > 0) {
        const int64_t width = static_cast<int64_t>(a.H) * (2 * a.dk + a.dv);
        const int bps = static_cast<int>((width + 255) / 256);
        hipLaunchKernelGGL((conv_state_kernel<XT>), dim3(static_cast<unsigned>(a.N) * bps), dim3(256), 0, s,
                           k, bps);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_preprocess(const PreprocessArgs& a, hipStream_t s) {
    return a.x == DT::BF16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

}  // namespace kda
