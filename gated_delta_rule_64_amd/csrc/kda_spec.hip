// Speculative multi-token verify with a deferred commit (gfx950).
//
// A serving step that verifies draft tokens runs the token mixer over 1 + n
// tokens per sequence and learns only afterwards how many of them the model
// accepts.  Rather than write a state snapshot after every draft token (n + 1
// full states per sequence and head), a call here
//   1. commits the tokens of the previous call that were accepted: their raw
//      values sit in a small per-slot draft buffer, so the conv, norm, gates
//      and state updates are simply run again for them, and the state and conv
//      history are written back once;
//   2. runs the new tokens from that state, in registers: each token's output
//      reads the state after the tokens before it (the recurrence of the
//      section "KDA: constant-size memory over a very long context" of the
//      page "Ling-3.0-flash: a 124B open MoE ..."), and the state is not
//      written; the new raw tokens go to the draft buffer for the next call.
// So a step reads and writes each state once, like a plain decode step.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_profile.h"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTok = kSpecMaxTokens;

template <typename XT>
struct SpecK {
    int H, T, slots;
    const XT *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b, *z;
    float* cs;
    float* state;
    const int32_t* idx;
    const int32_t* acc;
    XT* drafts;
    XT* out;
};

// One 256-thread workgroup per (sequence, head).  The dv columns of the state
// evolve independently, so wave w owns columns [w dv/4, (w+1) dv/4) over all
// dk rows: lane (rg, cg) holds rows rg + NRG*i, columns 4cg .. 4cg+3 of its
// wave's quarter, the reductions over rows stay inside the wave (shuffles),
// and the token loop needs no barrier.  Preprocess roles: threads 0..127 run
// channel tid of q and k, threads 128..255 channel tid-128 of v and of the
// decay logits (both wave-uniform).
template <int DK, int DV, typename XT>
__global__ __launch_bounds__(256) void spec_kernel(SpecK<XT> a) {
    constexpr int CPW = DV / 4;              // columns per wave
    constexpr int CG = CPW / 4;              // 4-column groups per wave
    constexpr int NRG = 64 / CG;             // row groups per wave
    constexpr int RPT = (DK + NRG - 1) / NRG;  // rows per lane
    constexpr int W = spec_draft_width(DK, DV);
    constexpr int NJ = 2 * kMaxTok;  // committed + new tokens at most

    const int64_t bh = blockIdx.x;
    const int H = a.H, T = a.T;
    const int bb = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = lane % CG;
    const int rg = lane / CG;
    const int col = wave * CPW + 4 * cg;  // this lane's first state column

    __shared__ float s_k[NJ][DK], s_a[NJ][DK], s_v[NJ][DV], s_q[kMaxTok][DK], s_z[kMaxTok][DV];
    __shared__ float s_beta[NJ];
    __shared__ float s_ss[NJ][2][2];
    __shared__ float s_qk[kMaxTok];

    const int slot = a.idx ? a.idx[bb] : bb;
    if (slot < 0 || slot >= a.slots) {  // padding row: zero outputs, nothing else
        if (rg == 0) {
            const float zero[4] = {0.f, 0.f, 0.f, 0.f};
            for (int t = 0; t < T; ++t) st4(a.out + ((static_cast<int64_t>(bb) * T + t) * H + h) * DV + col, zero);
        }
        return;
    }
    int na = a.acc ? a.acc[bb] : 0;
    na = na < 0 ? 0 : (na > kMaxTok ? kMaxTok : na);
    const int J = na + T;
    if (J == 0) return;  // nothing to commit, nothing to verify

    const int64_t sbh = static_cast<int64_t>(slot) * H + h;
    float* __restrict__ Sp = a.state + sbh * (DK * DV);

    // 1. the state patch (only read when there is something to commit or verify)
    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + NRG * i;
        if (r < DK) S[i] = *reinterpret_cast<const f32x4*>(Sp + r * DV + col);
    }

    // 2. where this thread's raw values live: committed token j < na in the
    // draft buffer, new token t = j - na in the inputs; its conv taps and the
    // committed conv history
    const bool lower = tid < 128;           // q, k  |  v, decay logit
    const int c = lower ? tid : tid - 128;  // channel
    const bool act0 = c < (lower ? DK : DV), act1 = c < DK;
    const int c0 = lower ? (c & (DK - 1)) : (c & (DV - 1)), c1 = c & (DK - 1);
    const int64_t cs_width = static_cast<int64_t>(H) * (2 * DK + DV);
    float* cs = a.cs + static_cast<int64_t>(slot) * 3 * cs_width;
    // conv-history columns of this thread's two tensors (the second unused by the upper half)
    float* hp0 = cs + (lower ? static_cast<int64_t>(h) * DK : static_cast<int64_t>(2) * H * DK + static_cast<int64_t>(h) * DV) + c0;
    float* hp1 = cs + static_cast<int64_t>(H) * DK + static_cast<int64_t>(h) * DK + c1;
    XT* dr = a.drafts + (static_cast<int64_t>(slot) * kMaxTok * H + h) * W;  // token j at dr + j*H*W
    const int d_off0 = lower ? c0 : 2 * DK + c0;      // q | v
    const int d_off1 = lower ? DK + c1 : 2 * DK + DV + c1;  // k | g
    const XT* in0 = lower ? a.q_in : a.v_in;
    const XT* in1 = lower ? a.k_in : a.g;
    const int64_t row0 = lower ? static_cast<int64_t>(H) * DK : static_cast<int64_t>(H) * DV;
    const int64_t col0 = lower ? static_cast<int64_t>(h) * DK + c0 : static_cast<int64_t>(h) * DV + c0;
    const int64_t col1 = static_cast<int64_t>(h) * DK + c1;
    const int64_t row1 = static_cast<int64_t>(H) * DK;
    float w0[4], w1[4], h0[3], h1[3];
    ld4((lower ? a.w_q : a.w_v) + col0 * 4, w0);
    ld4(a.w_k + col1 * 4, w1);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        h0[m] = hp0[m * cs_width];
        h1[m] = hp1[m * cs_width];
    }

    // 3. preprocess every token in order, eight token slots at a time (the
    // second eight only when there are more than eight tokens; a slot past J
    // re-reads token J-1, no extra traffic, and is ignored): conv against
    // the running history (written back to the pool once the committed tokens
    // are through), new raw tokens saved to the draft buffer, the norms'
    // partial sums, the gates.
    constexpr int NB = 8;
    const bool has_z = a.z != nullptr;
    const int64_t row_z = static_cast<int64_t>(H) * DV, col_z = static_cast<int64_t>(h) * DV + (c & (DV - 1));
    auto preprocess = [&](const int j0) {
        float x0[NB], x1[NB], xb[NB], xz[NB];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int j = j0 + jb;
            const int jj = j < J ? j : J - 1;
            // the source by selects, not branches: a load inside a branch
            // would have its value converted there, and the wait for it would
            // also wait for the state loads still in flight
            const bool draft = jj < na;
            const XT* pd = dr + static_cast<int64_t>(jj) * H * W;
            const int64_t t = static_cast<int64_t>(bb) * T + (draft ? 0 : jj - na);
            x0[jb] = ld(draft ? pd + d_off0 : in0 + t * row0 + col0);
            x1[jb] = ld(draft ? pd + d_off1 : in1 + t * row1 + col1);
            xb[jb] = ld(draft ? pd + 3 * DK + DV : a.b + t * H + h);
            // output-gate logit of a new token (any valid address otherwise)
            xz[jb] = ld(draft || !has_z ? pd : a.z + t * row_z + col_z);
        }
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int j = j0 + jb;
            if (j >= J) continue;  // (not break: the loop must unroll so x0, x1 stay in registers)
            const float y0 = w0[0] * h0[0] + w0[1] * h0[1] + w0[2] * h0[2] + w0[3] * x0[jb];
            const float y1 = lower ? w1[0] * h1[0] + w1[1] * h1[1] + w1[2] * h1[2] + w1[3] * x1[jb] : 0.f;
            h0[0] = h0[1]; h0[1] = h0[2]; h0[2] = x0[jb];
            h1[0] = h1[1]; h1[1] = h1[2]; h1[2] = x1[jb];
            if (j + 1 == na) {  // committed history
                if (act0) {
#pragma unroll
                    for (int m = 0; m < 3; ++m) hp0[m * cs_width] = h0[m];
                }
                if (lower && act1) {
#pragma unroll
                    for (int m = 0; m < 3; ++m) hp1[m * cs_width] = h1[m];
                }
            }
            if (j >= na) {  // new token: keep its raw values for the next call
                XT* p = dr + static_cast<int64_t>(j - na) * H * W;
                // Every element of a draft slot has one owner thread, which
                // both reads the committed value (first loop) and writes the
                // new one, so a slot is never rewritten by a thread other
                // than the one that read it: q / k channel c by thread c, v /
                // decay channel c by thread 128 + c, and the write logit by
                // thread 128, the thread that turns it into beta below.
                if (act0) st(p + d_off0, x0[jb]);
                if (act1) st(p + d_off1, x1[jb]);
                if (tid == 128) st(p + 3 * DK + DV, xb[jb]);
            }
            if (lower) {
                const float sk = wave_sum(act1 ? y1 * y1 : 0.f);
                const float sq = j >= na ? wave_sum(act0 ? y0 * y0 : 0.f) : 0.f;
                if (lane == 0) {
                    s_ss[j][0][wave] = sq;
                    s_ss[j][1][wave] = sk;
                }
                if (act1) {
                    s_k[j][c] = y1;
                    if (j >= na) s_q[j - na][c] = y0;
                }
            } else {
                if (act0) s_v[j][c] = round_to<XT>(y0);
                if (act0 && j >= na) s_z[j - na][c] = has_z ? sigmoid(xz[jb]) : 1.f;
                if (act1) s_a[j][c] = expf(-softplus_fast(x1[jb]));
                if (tid == 128) s_beta[j] = sigmoid_fast(xb[jb]);
            }
        }
    };
    static_assert(NJ == 2 * NB, "two batches of token slots");
    preprocess(0);
    if (J > NB) preprocess(NB);
    lds_barrier();
    // L2 norms, rounding to the input type (as kda_preprocess stores q^, k^),
    // and q^.k^ of each new token: wave w takes tokens w, w + 4, ..., its
    // lanes the channels (all four waves busy, the tokens independent)
    for (int j = wave; j < J; j += 4) {
        const float ik = __builtin_amdgcn_rsqf(s_ss[j][1][0] + s_ss[j][1][1] + kL2Eps);
        const bool vt = j >= na;
        const float iq = vt ? __builtin_amdgcn_rsqf(s_ss[j][0][0] + s_ss[j][0][1] + kL2Eps) : 0.f;
        float qk = 0.f;
        for (int ch = lane; ch < DK; ch += 64) {
            const float kk = round_to<XT>(s_k[j][ch] * ik);
            s_k[j][ch] = kk;
            if (vt) {
                const float qq = round_to<XT>(s_q[j - na][ch] * iq);
                s_q[j - na][ch] = qq;
                qk += qq * kk;
            }
        }
        if (vt) {
            qk = wave_sum(qk);
            if (lane == 0) s_qk[j - na] = qk;
        }
    }
    lds_barrier();

    // 4. the state, token by token (each wave on its own columns, no barrier):
    // decay, then u = S'^T k and p = S'^T q,
    // then S = S' + beta k (v - u)^T and, for a new token, the output
    // o = p + (q.k) beta (v - u).  One loop over all tokens keeps a single
    // copy of S in registers; a committed token computes p with k in place of
    // q (a few FMAs, no branch) and stores no output.  The committed state is
    // stored once, after the last committed token.
    for (int j = 0; j < J; ++j) {
        const bool verify = j >= na;
        const int t = j - na;
        const float* qrow = verify ? s_q[t] : s_k[j];
        float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + NRG * i;
            if (r < DK) {
                const float al = s_a[j][r], kk = s_k[j][r], qq = qrow[r];
                S[i].x *= al; S[i].y *= al; S[i].z *= al; S[i].w *= al;
                u[0] += S[i].x * kk; u[1] += S[i].y * kk; u[2] += S[i].z * kk; u[3] += S[i].w * kk;
                p[0] += S[i].x * qq; p[1] += S[i].y * qq; p[2] += S[i].z * qq; p[3] += S[i].w * qq;
            }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {  // sums over the wave's row groups
            u[cc] = wave_sum_stride<CG>(u[cc]);
            p[cc] = wave_sum_stride<CG>(p[cc]);
        }
        const float bt = s_beta[j];
        float d[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) d[cc] = bt * (s_v[j][col + cc] - u[cc]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + NRG * i;
            if (r < DK) {
                const float kk = s_k[j][r];
                S[i].x += kk * d[0]; S[i].y += kk * d[1]; S[i].z += kk * d[2]; S[i].w += kk * d[3];
            }
        }
        if (j + 1 == na) {  // the committed state
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + NRG * i;
                if (r < DK) __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(Sp + r * DV + col));
            }
        }
        if (verify && rg == 0) {
            const float qk = s_qk[t];
            float o[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) o[cc] = p[cc] + qk * d[cc];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) o[cc] *= s_z[t][col + cc];  // (1 without a gate)
            st4(a.out + ((static_cast<int64_t>(bb) * T + t) * H + h) * DV + col, o);
        }
    }
}

template <int DK, int DV, typename XT>
hipError_t launch_typed(const SpecArgs& s, hipStream_t st) {
    SpecK<XT> k{};
    k.H = s.H; k.T = s.T; k.slots = s.slots;
    k.q_in = static_cast<const XT*>(s.q_in); k.k_in = static_cast<const XT*>(s.k_in);
    k.v_in = static_cast<const XT*>(s.v_in); k.w_q = static_cast<const XT*>(s.w_q);
    k.w_k = static_cast<const XT*>(s.w_k); k.w_v = static_cast<const XT*>(s.w_v);
    k.g = static_cast<const XT*>(s.g); k.b = static_cast<const XT*>(s.b); k.z = static_cast<const XT*>(s.z);
    k.cs = s.conv_state; k.state = s.state; k.idx = s.state_indices; k.acc = s.accepted;
    k.drafts = static_cast<XT*>(s.drafts); k.out = static_cast<XT*>(s.out);
    const int64_t grid = static_cast<int64_t>(s.B) * s.H;
    if (grid == 0) return hipSuccess;
    LaunchTimer timer("spec_verify", st);
    hipLaunchKernelGGL((spec_kernel<DK, DV, XT>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, k);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const SpecArgs& s, hipStream_t st) {
    const bool bf = s.x == DT::BF16;
    switch (s.dv) {
        case 16: return bf ? launch_typed<DK, 16, bf16>(s, st) : launch_typed<DK, 16, float>(s, st);
        case 32: return bf ? launch_typed<DK, 32, bf16>(s, st) : launch_typed<DK, 32, float>(s, st);
        case 64: return bf ? launch_typed<DK, 64, bf16>(s, st) : launch_typed<DK, 64, float>(s, st);
        case 128: return bf ? launch_typed<DK, 128, bf16>(s, st) : launch_typed<DK, 128, float>(s, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_spec_verify(const SpecArgs& s, hipStream_t st) {
    switch (s.dk) {
        case 16: return launch_dk<16>(s, st);
        case 32: return launch_dk<32>(s, st);
        case 64: return launch_dk<64>(s, st);
        case 128: return launch_dk<128>(s, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
