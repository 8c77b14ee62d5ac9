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

// Arguments of both forms of the step.  Unfused: q, k, v, la, beta hold the
// preprocessed token (kda_preprocess's outputs).  Fused: q_in .. b hold the
// raw projections, conv taps and gate logits, and the kernel runs the short
// conv (against the caller's conv history, which it rolls forward), the L2
// norm and the gates itself.  State (and conv history) rows are slot
// idx[b] of a pool of `slots` (idx NULL: slot b).
template <typename XT, typename GT>
struct DecK {
    int H;
    const XT *q, *k, *v;
    const GT *la, *beta;
    const XT* z;
    float* state;
    XT* out;
    // fused form
    const XT *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b;
    float* cs;
    const int32_t* idx;
    int slots;
};

template <int DK, int DV, typename XT, typename GT, bool kFused>
__global__ __launch_bounds__(256) void decode_kernel(DecK<XT, GT> a) {
    constexpr int CG = DV / 4;                  // float4 column groups
    constexpr int NRG = 256 / CG;               // row groups
    constexpr int RPT = (DK + NRG - 1) / NRG;   // rows per thread
    constexpr int RG_PER_WAVE = 64 / CG;

    const int64_t bh = blockIdx.x;
    const int H = a.H;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ float s_k[DK], s_q[DK], s_a[DK], s_v[DV];
    __shared__ float s_qk[4];
    __shared__ float s_red[4][CG][8];
    __shared__ float s_ss[2][4];

    int64_t sbh = bh;  // state row
    if (kFused) {
        const int bb = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
        const int slot = a.idx ? a.idx[bb] : bb;
        if (slot < 0 || slot >= a.slots) {  // a row without a state (padding): output 0, nothing else
            if (rg == 0) {
                const float zero[4] = {0.f, 0.f, 0.f, 0.f};
                st4(a.out + bh * DV + 4 * cg, zero);
            }
            return;
        }
        sbh = static_cast<int64_t>(slot) * H + h;
    }
    float* __restrict__ Sp = a.state + sbh * (DK * DV);

    // 1. the whole state patch, then the token's own (small) inputs.
    // Measured: this order is faster than the token's loads first (whose
    // arithmetic could then run under the state's arrival) by 7 % for the
    // fused step and 1 % for the plain one.  Plain loads for the state:
    // non-temporal loads of several 16-byte pieces per thread cut the read
    // rate by a quarter; the stores stay non-temporal, which measured faster.
    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) S[i] = *reinterpret_cast<const f32x4*>(Sp + r * DV + 4 * cg);
    }
    const int bb = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    float t_k = 0.f, t_q = 0.f, t_a = 0.f, t_v = 0.f, bt;
    // fused form: per tensor the three history values (oldest first), the
    // raw value and the four taps of this thread's channel
    float hq[8] = {}, hk[8] = {}, hv[8] = {};
    const int64_t cs_width = static_cast<int64_t>(H) * (2 * DK + DV);
    float* cs = kFused ? a.cs + (sbh / H) * 3 * cs_width : nullptr;
    auto load_conv = [&](const XT* src, const XT* w, int64_t col, float* hp, float (&r)[8]) {
        r[0] = hp[0];
        r[1] = hp[cs_width];
        r[2] = hp[2 * cs_width];
        r[3] = ld(src + col);
        float wt[4];
        ld4(w + col * 4, wt);
        r[4] = wt[0]; r[5] = wt[1]; r[6] = wt[2]; r[7] = wt[3];
    };
    // Every thread loads (lanes past dk or dv re-read a valid channel and
    // store nothing): the loads stay in one block, issued back to back.
    const int ck = tid & (DK - 1), cv = tid & (DV - 1);
    const int64_t col_k = static_cast<int64_t>(h) * DK + ck, col_v = static_cast<int64_t>(h) * DV + cv;
    if (!kFused) {
        t_k = ld(a.k + bh * DK + ck);
        t_q = ld(a.q + bh * DK + ck);
        t_a = ld(a.la + bh * DK + ck);
        t_v = ld(a.v + bh * DV + cv);
        bt = ld(a.beta + bh);
    } else {
        load_conv(a.q_in + static_cast<int64_t>(bb) * H * DK, a.w_q, col_k, cs + col_k, hq);
        load_conv(a.k_in + static_cast<int64_t>(bb) * H * DK, a.w_k, col_k,
                  cs + static_cast<int64_t>(H) * DK + col_k, hk);
        t_a = ld(a.g + static_cast<int64_t>(bb) * H * DK + col_k);
        load_conv(a.v_in + static_cast<int64_t>(bb) * H * DV, a.w_v, col_v,
                  cs + static_cast<int64_t>(2) * H * DK + col_v, hv);
        bt = ld(a.b + static_cast<int64_t>(bb) * H + h);
    }

    // 2. per-row vectors to LDS, q.k per wave
    float qk_part = 0.f;
    if (!kFused) {
        if (tid < DK) {
            s_k[tid] = t_k;
            s_q[tid] = t_q;
            s_a[tid] = expf(t_a);
            qk_part = t_k * t_q;
        }
        if (tid < DV) s_v[tid] = t_v;
    } else {
        // the token's preprocess: thread c < max(dk, dv) runs channel c of q
        // and k (c < dk) and of v (c < dv): the width-4 conv over the three
        // raw tokens before it and this one, the history rolled forward by
        // one token; the L2 norm of q and k over dk; -softplus and sigmoid
        // gates.  q^, k^, v^ are rounded to the input type, as kda_preprocess
        // stores them.
        auto roll = [&](const float (&r)[8], float* hp) {
            hp[0] = r[1];
            hp[cs_width] = r[2];
            hp[2 * cs_width] = r[3];
        };
        auto conv = [](const float (&r)[8]) { return r[4] * r[0] + r[5] * r[1] + r[6] * r[2] + r[7] * r[3]; };
        if (tid < DK) {
            roll(hq, cs + col_k);
            roll(hk, cs + static_cast<int64_t>(H) * DK + col_k);
        }
        if (tid < DV) roll(hv, cs + static_cast<int64_t>(2) * H * DK + col_v);
        const float yq = tid < DK ? conv(hq) : 0.f, yk = tid < DK ? conv(hk) : 0.f, yv = conv(hv);
        // sums of squares over dk: within each wave, then across the waves
        float sq = yq * yq, sk = yk * yk;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sq += __shfl_xor(sq, off);
            sk += __shfl_xor(sk, off);
        }
        if (lane == 0) {
            s_ss[0][wave] = sq;
            s_ss[1][wave] = sk;
        }
        bt = sigmoid_fast(bt);
        lds_barrier();  // (LDS only: outstanding loads stay in flight)
        if (tid < DK) {
            const float iq = 1.f / sqrtf(s_ss[0][0] + s_ss[0][1] + s_ss[0][2] + s_ss[0][3] + kL2Eps);
            const float ik = 1.f / sqrtf(s_ss[1][0] + s_ss[1][1] + s_ss[1][2] + s_ss[1][3] + kL2Eps);
            const float qq = round_to<XT>(yq * iq), kk = round_to<XT>(yk * ik);
            s_q[tid] = qq;
            s_k[tid] = kk;
            s_a[tid] = expf(-softplus_fast(t_a));
            qk_part = kk * qq;
        }
        if (tid < DV) s_v[tid] = round_to<XT>(yv);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk_part += __shfl_xor(qk_part, off);
    if (lane == 0) s_qk[wave] = qk_part;
    __syncthreads();

    // 3. decay, then the two partial reductions over this thread's rows
    float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) {
            const float al = s_a[r], kk = s_k[r], qq = s_q[r];
            S[i].x *= al; S[i].y *= al; S[i].z *= al; S[i].w *= al;
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
    float d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = bt * (s_v[4 * cg + c] - u[c]);
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
        if (a.z != nullptr) {
            float zz[4];
            ld4(a.z + bh * DV + 4 * cg, zz);
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] *= sigmoid(zz[c]);
        }
        st4(a.out + bh * DV + 4 * cg, o);
    }
}

template <int DK, int DV, typename XT, typename GT, bool kFused>
hipError_t launch_typed(const DecK<XT, GT>& k, int64_t grid, hipStream_t s) {
    if (grid == 0) return hipSuccess;
    LaunchTimer timer(kFused ? "decode_layer" : "decode", s);
    hipLaunchKernelGGL((decode_kernel<DK, DV, XT, GT, kFused>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, k);
    return hipGetLastError();
}

template <int DK, int DV, typename XT, typename GT>
hipError_t launch_step(const DecodeArgs& a, hipStream_t s) {
    DecK<XT, GT> k{};
    k.H = a.H;
    k.q = static_cast<const XT*>(a.q); k.k = static_cast<const XT*>(a.k); k.v = static_cast<const XT*>(a.v);
    k.la = static_cast<const GT*>(a.la); k.beta = static_cast<const GT*>(a.beta);
    k.z = static_cast<const XT*>(a.z); k.state = a.state; k.out = static_cast<XT*>(a.out);
    return launch_typed<DK, DV, XT, GT, false>(k, static_cast<int64_t>(a.B) * a.H, s);
}

template <int DK, int DV>
hipError_t launch_dims(const DecodeArgs& a, hipStream_t s) {
    if (a.x == DT::BF16) {
        return a.gate == DT::BF16 ? launch_step<DK, DV, bf16, bf16>(a, s) : launch_step<DK, DV, bf16, float>(a, s);
    }
    return a.gate == DT::BF16 ? launch_step<DK, DV, float, bf16>(a, s) : launch_step<DK, DV, float, float>(a, s);
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

template <int DK, int DV, typename XT>
hipError_t launch_layer_step(const DecodeLayerArgs& a, hipStream_t s) {
    DecK<XT, float> k{};
    k.H = a.H;
    k.z = static_cast<const XT*>(a.z); k.state = a.state; k.out = static_cast<XT*>(a.out);
    k.q_in = static_cast<const XT*>(a.q_in); k.k_in = static_cast<const XT*>(a.k_in);
    k.v_in = static_cast<const XT*>(a.v_in); k.w_q = static_cast<const XT*>(a.w_q);
    k.w_k = static_cast<const XT*>(a.w_k); k.w_v = static_cast<const XT*>(a.w_v);
    k.g = static_cast<const XT*>(a.g); k.b = static_cast<const XT*>(a.b);
    k.cs = a.conv_state; k.idx = a.state_indices; k.slots = a.slots;
    return launch_typed<DK, DV, XT, float, true>(k, static_cast<int64_t>(a.B) * a.H, s);
}

template <int DK>
hipError_t launch_layer_dk(const DecodeLayerArgs& a, hipStream_t s) {
    const bool bf = a.x == DT::BF16;
    switch (a.dv) {
        case 16: return bf ? launch_layer_step<DK, 16, bf16>(a, s) : launch_layer_step<DK, 16, float>(a, s);
        case 32: return bf ? launch_layer_step<DK, 32, bf16>(a, s) : launch_layer_step<DK, 32, float>(a, s);
        case 64: return bf ? launch_layer_step<DK, 64, bf16>(a, s) : launch_layer_step<DK, 64, float>(a, s);
        case 128: return bf ? launch_layer_step<DK, 128, bf16>(a, s) : launch_layer_step<DK, 128, float>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_layer(const DecodeLayerArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return launch_layer_dk<16>(a, s);
        case 32: return launch_layer_dk<32>(a, s);
        case 64: return launch_layer_dk<64>(a, s);
        case 128: return launch_layer_dk<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

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
