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
//   2. runs the new tokens from that state: each token's output reads the
//      state after the tokens before it (the recurrence of the section "KDA:
//      constant-size memory over a very long context" of the page
//      "Ling-3.0-flash: a 124B open MoE ..."), and the state is not written;
//      the new raw tokens go to the draft buffer for the next call.
// So a step reads and writes each state once, like a plain decode step.
//
// The J = na + T tokens of a call (na committed, then T new) are one short
// chunk, computed in the chunked form (the exact rewrite the prefill uses).
// With S0 the slot's state and G_j the running sum of the log decays through
// token j (per key channel, base 2 here):
//   P    = X S0,  X = rows 2^{G_j} k_j (j < J), then 2^{G_{na+t}} q_t (t < T)
//   A_jl = beta_j sum_c k_jc k_lc 2^{G_jc - G_lc}                  (l < j)
//   u_j  = beta_j (v_j - P_j) - sum_{l<j} A_jl u_l        (the delta-rule writes)
//   o_t  = P_{J+t} + sum_{i <= na+t} M_ti u_i,  M_ti = sum_c q_tc k_ic 2^{G_{na+t},c - G_ic}
//   S    = Diag(2^{G_{na-1}}) S0 + sum_{i<na} (2^{G_{na-1} - G_i} * k_i) u_i^T
// (the last line is the committed state).  Every exponent is a later running
// sum minus an earlier one, taken element by element, so none is positive and
// nothing overflows however strong the decay.  The state is read once into
// registers, feeds P on the fp32 matrix cores (v_mfma_f32_16x16x4_f32) as
// their B operand, takes the rank-na update in place and is stored once; the
// token-by-token chain shrinks to the J x J solve on 16-element vectors.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_profile.h"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// buffer resource word 3 for raw (unformatted) 32-bit data on gfx9-family
// parts, and the cache-policy bit of a streaming (non-temporal) access
constexpr int kBufferDword3 = 0x00020000;
constexpr int kNonTemporal = 2;

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes from global memory straight into LDS: lane l's bytes land at
// lds_dst + 16 l (lds_dst is the same for the whole wave)
__device__ __forceinline__ void lds_copy16(const void* gsrc, char* lds_dst) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)(lds_dst), 16, 0, 0);
}

// wait until at most N of this wave's global memory operations are in flight
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kMaxTok = kSpecMaxTokens;
constexpr int kNJ = 2 * kMaxTok;  // committed + new tokens at most

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

// How the four waves share the dk x dv state for the products: NWC groups of
// columns times NWK groups of rows.  In v_mfma_f32_16x16x4_f32, lane l = 16 q + n
// gives A[n][q] and B[q][n] and receives D[4q + i][n] (i = 0..3).  Contraction
// step s of wave (wc, wk) takes state rows wk KW + SP q + s (q = 0..3) as the
// four contraction indices, and the V instructions of the step take columns
// wc 16 V + V n + j (j < V) as their sixteen result columns: each lane holds V
// adjacent floats of one row per step (16 lanes read 16 V contiguous floats
// of a row), and its A operands X[n][wk KW + SP q + s] are contiguous in s.
template <int DK, int DV>
struct SpecSplit {
    static constexpr int NWC = DV / 16 < 4 ? DV / 16 : 4;
    static constexpr int NWK = 4 / NWC;
    static constexpr int V = DV / (16 * NWC);  // adjacent columns per lane
    static constexpr int KW = DK / NWK;        // state rows per wave
    static constexpr int SP = KW / 4;          // contraction steps per wave
    static constexpr int XS = DK + 4;          // LDS row stride of X (floats)
    static constexpr int PS = DV + 4;          // LDS row stride of P
    static_assert(NWC * NWK == 4 && V >= 1 && V <= 2 && SP >= 1, "head sizes 16..128");
};

// Dynamic LDS of one workgroup, float offsets; jm = kMaxTok + T token rows at
// most, X and P padded to whole 16-row passes; XB bytes per input element.
template <int DK, int DV, int XB>
struct SpecLds {
    static constexpr int MW = DK > DV ? DK : DV;  // row width of the raw staging
    int k, G, v, q, z, beta, xp, kh, u, ab, m, st, total;
    __host__ __device__ explicit SpecLds(int T) {
        typedef SpecSplit<DK, DV> Sp;
        const int jm = kMaxTok + T, xr = 16 * ((jm + T + 15) / 16);
        const int xsz = xr * Sp::XS, psz = Sp::NWK * xr * Sp::PS;
        k = 0;                          // normalized k      [jm][DK]
        G = k + jm * DK;                // running log2 decay [jm][DK]
        v = G + jm * DK;                // v                 [jm][DV]
        q = v + jm * DV;                // normalized q      [T][DK]
        z = q + T * DK;                 // sigmoid(out gate) [T][DV]
        beta = z + T * DV;              // [kNJ]
        // from here on, space that is first written after the preprocess
        xp = beta + 16 * ((kNJ + 15) / 16);  // X, then P (16-float aligned)
        kh = xp + (xsz > psz ? xsz : psz);  // commit factors [1 + kMaxTok][DK]
        // U of the committed tokens [kMaxTok][DV]: in k's place once k is read
        u = kMaxTok * DV <= jm * DK ? k : kh + (1 + kMaxTok) * DK;
        ab = (u == k ? kh + (1 + kMaxTok) * DK : u + kMaxTok * DV);  // beta_j A_jl [kNJ][kNJ]
        m = ab + kNJ * kNJ;             // M [kMaxTok][kNJ]
        const int end = m + kMaxTok * kNJ;
        // the call's raw rows as loaded, for the preprocess: [4 jm][MW] (q, k,
        // v, g of every token), then [T][MW] output-gate logits; over X and
        // what follows it
        st = xp;
        const int st_end = st + (4 * jm + T) * MW * XB / 4;
        total = end > st_end ? end : st_end;
    }
};

// One 256-thread workgroup per (sequence, head).  Preprocess roles: threads
// 0..127 run channel tid of q and k, threads 128..255 channel tid-128 of v
// and of the decay logits (both wave-uniform).  Register budget: four
// workgroups per CU (128 VGPRs; at d = 128 one 64-bit value spills, reloaded
// only after the state has arrived), measured faster than three.
template <int DK, int DV, typename XT>
__global__ __launch_bounds__(256, 4) void spec_kernel(SpecK<XT> a) {
    typedef SpecSplit<DK, DV> Sp;
    constexpr int W = spec_draft_width(DK, DV);
    constexpr int SP = Sp::SP, V = Sp::V;
    extern __shared__ f32x4 spec_smem[];
    float* const sm = reinterpret_cast<float*>(spec_smem);

    const int64_t bh = blockIdx.x;
    const int H = a.H, T = a.T;
    const int bb = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int slot = a.idx ? a.idx[bb] : bb;
    if (slot < 0 || slot >= a.slots) {  // padding row: zero outputs, nothing else
        if (tid < DV)
            for (int t = 0; t < T; ++t) st(a.out + ((static_cast<int64_t>(bb) * T + t) * H + h) * DV + tid, 0.f);
        return;
    }
    int na = a.acc ? a.acc[bb] : 0;
    na = na < 0 ? 0 : (na > kMaxTok ? kMaxTok : na);
    const int J = na + T;
    if (J == 0) return;  // nothing to commit, nothing to verify

    const SpecLds<DK, DV, sizeof(XT)> L(T);
    float* const s_k = sm + L.k;
    float* const s_G = sm + L.G;
    float* const s_v = sm + L.v;
    float* const s_q = sm + L.q;
    float* const s_z = sm + L.z;
    float* const s_X = sm + L.xp;
    float* const s_kh = sm + L.kh;
    float* const s_U = sm + L.u;
    float* const s_ab = sm + L.ab;
    float* const s_M = sm + L.m;
    float* const s_beta = sm + L.beta;
    XT* const s_raw = reinterpret_cast<XT*>(sm + L.st);
    constexpr int MW = SpecLds<DK, DV, sizeof(XT)>::MW;

    // this lane's part of the state (see SpecSplit)
    const int wc = wave % Sp::NWC, wk = wave / Sp::NWC;
    const int ln = lane & 15, lq = lane >> 4;
    const int row0 = wk * Sp::KW + SP * lq;
    const int col0 = wc * 16 * V + V * ln;
    const int64_t sbh = static_cast<int64_t>(slot) * H + h;
    // The state patch is read and written with buffer instructions over the
    // head's dk x dv x 4 bytes: a byte offset per lane plus a per-row
    // constant, so that no 64-bit address per row is kept in registers
    // between the load and the store.
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.state + sbh * (DK * DV), 0, DK * DV * 4, kBufferDword3);
    const int Soff = 4 * (row0 * DV + col0);

    // this thread's channel of its two tensors, their conv taps and the
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
    const int64_t col0_in = lower ? static_cast<int64_t>(h) * DK + c0 : static_cast<int64_t>(h) * DV + c0;
    const int64_t col1_in = static_cast<int64_t>(h) * DK + c1;
    float w0[4], w1[4], h0[3], h1[3];
    ld4((lower ? a.w_q : a.w_v) + col0_in * 4, w0);
    ld4(a.w_k + col1_in * 4, w1);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        h0[m] = hp0[m * cs_width];
        h1[m] = hp1[m * cs_width];
    }

    // 1. The call's raw rows go to LDS first, with 16-byte copies straight
    // into LDS (q, k, v, g of every token, committed ones from the draft
    // buffer, new ones from the inputs, and the new tokens' output-gate
    // logits): a wave moves 1 KB per copy, and the per-channel preprocess
    // below reads its values from there.
    const bool has_z = a.z != nullptr;
    {
        constexpr int CPR = MW * static_cast<int>(sizeof(XT)) / 16;  // 16-byte chunks per staged row
        constexpr int EPC = 16 / static_cast<int>(sizeof(XT));       // elements per chunk
        const int nrow = 4 * J + (has_z ? T : 0);
        const int nblk = (nrow * CPR + 63) / 64;
        for (int blk = wave; blk < nblk; blk += 4) {
            const int e = 64 * blk + lane;
            const int rho = e / CPR, el = (e % CPR) * EPC;
            const XT* src = nullptr;
            int width = 0;
            if (rho < 4 * J) {
                const int j = rho >> 2, tau = rho & 3;  // q, k, v, g
                width = tau == 2 ? DV : DK;
                if (j < na) {
                    const int off = tau == 0 ? 0 : (tau == 1 ? DK : (tau == 2 ? 2 * DK : 2 * DK + DV));
                    src = dr + static_cast<int64_t>(j) * H * W + off;
                } else {
                    const int64_t t = static_cast<int64_t>(bb) * T + (j - na);
                    const XT* base = tau == 0 ? a.q_in : (tau == 1 ? a.k_in : (tau == 2 ? a.v_in : a.g));
                    src = base + (t * H + h) * width;
                }
            } else if (rho < nrow) {
                width = DV;
                src = a.z + ((static_cast<int64_t>(bb) * T + (rho - 4 * J)) * H + h) * DV;
            }
            if (el < width) lds_copy16(src + el, reinterpret_cast<char*>(s_raw) + blk * 1024);
        }
    }

    // Then the preprocess of every token in order, eight token slots at a
    // time (the second eight only when there are more than eight tokens; a
    // slot past J re-reads token J-1 and is ignored): conv against the
    // running history (written back to the pool once the committed tokens are
    // through), the norms' partial sums, the gates and the running log decay.
    constexpr int NB = 8;
    const int zc = c & (DV - 1);
    float x0[NB], x1[NB], xz[NB];
    // The write logits: lane j of wave 2 loads token j's (one load for all
    // tokens, issued with the staging copies), turns it into beta and, for a
    // new token, keeps it in the draft buffer.  A lane's store follows its own
    // load, and all of the wave's loads are one instruction, so a committed
    // logit is read before any new one replaces it.
    // (Every wave issues the load, lanes past J on token 0's address: a load
    // under a branch would be waited for inside it, before the state's loads
    // go out.)
    const int jl = lane < J ? lane : 0;
    const int64_t tl = static_cast<int64_t>(bb) * T + (jl < na ? 0 : jl - na);
    const float bj = ld(jl < na ? dr + static_cast<int64_t>(jl) * H * W + 3 * DK + DV : a.b + tl * H + h);
    auto load_batch = [&](const int j0) {
        const int tau0 = lower ? 0 : 2, tau1 = lower ? 1 : 3;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int j = j0 + jb;
            const int jj = j < J ? j : J - 1;
            x0[jb] = ld(s_raw + (4 * jj + tau0) * MW + c0);
            x1[jb] = ld(s_raw + (4 * jj + tau1) * MW + c1);
            // output-gate logit of a new token (staged only for those)
            xz[jb] = has_z && jj >= na ? ld(s_raw + (4 * J + (jj - na)) * MW + zc) : 0.f;
        }
    };
    float gl = 0.f;  // running log2 decay of channel c (upper half)
    auto compute_batch = [&](const int j0) {
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
            if (lower) {
                if (act1) {
                    s_k[j * DK + c] = y1;
                    if (j >= na) s_q[(j - na) * DK + c] = y0;
                }
            } else {
                if (act0) s_v[j * DV + c] = round_to<XT>(y0);
                if (act0 && j >= na) s_z[(j - na) * DV + c] = has_z ? sigmoid(xz[jb]) : 1.f;
                gl -= softplus_log2(x1[jb]);
                if (act1) s_G[j * DK + c] = gl;
            }
        }
    };
    static_assert(kNJ == 2 * NB, "two batches of token slots");
    // (no memory operation moves across: the counted wait below relies on
    // the state's loads being the last ones issued)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // the state, into registers, read once in two halves: the first right
    // behind the staging copies, in flight through the preprocess and the
    // norms, the second after the norms, in flight through the small
    // operands.  (All of it at once leaves the preprocess so few registers
    // that the compiler spills a state register, and waits for its load to
    // do so, right after issuing it.)
    constexpr int SA = SP > 1 ? SP / 2 : SP;  // steps loaded first
    float Sr[SP][V];
    auto load_state = [&](int s0, int s1) {
#pragma unroll
        for (int s = 0; s < SP; ++s) {
            if (s < s0 || s >= s1) continue;
            if constexpr (V == 2) {
                const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(srsrc, Soff, 4 * DV * s, 0);
                Sr[s][0] = __int_as_float(x.x);
                Sr[s][1] = __int_as_float(x.y);
            } else {
                Sr[s][0] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(srsrc, Soff, 4 * DV * s, 0));
            }
        }
    };
    load_state(0, SA);
    // the staging copies (and the write logits) have landed once no more than
    // the state's loads are in flight
    wait_vmem_but<SA>();
    if (wave == 2 && lane < J) {
        s_beta[lane] = sigmoid_fast(bj);
        if (lane >= na) st(dr + static_cast<int64_t>(lane - na) * H * W + 3 * DK + DV, bj);
    }
    lds_barrier();
    // The new tokens' raw q, k, v, g rows to the draft buffer for the next
    // call (16-byte copies out of the staging rows).  Every read of the
    // buffer's committed rows landed before the barrier above.
    {
        constexpr int EPC = 16 / static_cast<int>(sizeof(XT));
        constexpr int CPT = (3 * DK + DV) / EPC;  // chunks of one draft row's q, k, v, g
        for (int e = tid; e < T * CPT; e += 256) {
            const int t = e / CPT, el = (e % CPT) * EPC;
            const int tau = el < DK ? 0 : (el < 2 * DK ? 1 : (el < 2 * DK + DV ? 2 : 3));
            const int off = tau == 0 ? 0 : (tau == 1 ? DK : (tau == 2 ? 2 * DK : 2 * DK + DV));
            const uint4 v4 = *reinterpret_cast<const uint4*>(s_raw + (4 * (na + t) + tau) * MW + (el - off));
            *reinterpret_cast<uint4*>(dr + static_cast<int64_t>(t) * H * W + el) = v4;
        }
    }
    load_batch(0);
    compute_batch(0);
    if (J > NB) {
        load_batch(NB);
        compute_batch(NB);
    }

    lds_barrier();
    // L2 norms, rounding to the input type (as kda_preprocess stores q^, k^):
    // wave w takes tokens w, w + 4, ..., its lanes the channels (DK / 64 or
    // one each), and sums the squares across the wave
    constexpr int CPL = DK >= 64 ? DK / 64 : 1;  // channels per lane
    for (int j = wave; j < J; j += 4) {
        const bool vt = j >= na;
        const int tq = vt ? j - na : 0;
        float kv[CPL], qv[CPL], sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            const bool in = ch < DK;
            kv[i] = in ? s_k[j * DK + ch] : 0.f;
            qv[i] = in && vt ? s_q[tq * DK + ch] : 0.f;
            sk += kv[i] * kv[i];
            sq += qv[i] * qv[i];
        }
        const float ik = __builtin_amdgcn_rsqf(wave_sum(sk) + kL2Eps);
        const float iq = __builtin_amdgcn_rsqf(wave_sum(sq) + kL2Eps);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            if (ch < DK) {
                s_k[j * DK + ch] = round_to<XT>(kv[i] * ik);
                if (vt) s_q[tq * DK + ch] = round_to<XT>(qv[i] * iq);
            }
        }
    }
    lds_barrier();
    load_state(SA, SP);

    // 3. the call's small operands: X (zero rows pad it to whole 16-row
    // passes), the commit factors, and A and M, one 16-lane row per entry
    const int npass = (J + T + 15) >> 4;
    const int XR = 16 * npass;
    // (fixed trip counts, unrolled, so that each thread's LDS reads are
    // issued together rather than one round trip at a time)
    constexpr int kXPer = (32 * DK + 255) / 256;  // X elements per thread for two passes
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
        const int e = tid + 256 * m;
        const int r = e / DK, ch = e % DK;
        if (r < XR) {
            const bool isk = r < J, isq = !isk && r < J + T;
            const int gr = isk ? r : na + r - J;
            const float* vrow = isk ? s_k + r * DK : s_q + (r - J) * DK;
            const float x = (isk || isq) ? __builtin_amdgcn_exp2f(s_G[(isk || isq ? gr : 0) * DK + ch]) * vrow[ch] : 0.f;
            s_X[r * Sp::XS + ch] = x;
        }
    }
    if (na > 0) {
        // row 0: 2^{G_{na-1}}; row 1 + i: 2^{G_{na-1} - G_i} k_i (zero for i >= na)
        constexpr int kKhPer = ((1 + kMaxTok) * DK + 255) / 256;
#pragma unroll
        for (int m = 0; m < kKhPer; ++m) {
            const int e = tid + 256 * m;
            if (e >= (1 + kMaxTok) * DK) break;
            const int i = e / DK - 1, ch = e % DK;
            const float gl_c = s_G[(na - 1) * DK + ch];
            float f;
            if (i < 0) f = __builtin_amdgcn_exp2f(gl_c);
            else if (i < na) f = __builtin_amdgcn_exp2f(gl_c - s_G[i * DK + ch]) * s_k[i * DK + ch];
            else f = 0.f;
            s_kh[e] = f;
        }
    }
    {
        const int npa = J * (J - 1) / 2, npm = T * na + T * (T + 1) / 2;
        const int grp = tid >> 4, li = tid & 15;
        for (int p0 = 0; p0 < npa + npm; p0 += 16) {
            const int p = p0 + grp;
            int ra, rb;        // rows of the entry's two vectors and its running sums
            const float* va;   // its left vector (k or q)
            int dst;
            if (p < npa) {     // A_jl: j = ra, l = rb; row j starts at entry j (j - 1) / 2
                int i = static_cast<int>((1.f + __builtin_sqrtf(1.f + 8.f * p)) * 0.5f);
                i += (i * (i + 1)) / 2 <= p;   // (the float root may land one off)
                i -= (i * (i - 1)) / 2 > p;
                ra = i;
                rb = p - (i * (i - 1)) / 2;
                va = s_k + ra * DK;
                dst = ra * kNJ + rb;
            } else {           // M_ti: running sum of token na + t, i = rb; row t holds
                               // na + 1 + t entries, starting at entry t (na + 1) + t (t - 1) / 2
                const int qq = p < npa + npm ? p - npa : 0;
                const float b2 = 2.f * na + 1.f;
                int t = static_cast<int>((__builtin_sqrtf(b2 * b2 + 8.f * qq) - b2) * 0.5f);
                t = t < 0 ? 0 : t;
                t += (t + 1) * (na + 1) + ((t + 1) * t) / 2 <= qq;
                t -= t * (na + 1) + (t * (t - 1)) / 2 > qq;
                ra = na + t;
                rb = qq - (t * (na + 1) + (t * (t - 1)) / 2);
                va = s_q + t * DK;
                dst = t * kNJ + rb;
            }
            float acc = 0.f;
            if (p < npa + npm) {
#pragma unroll
                for (int m = 0; m < DK / 16; ++m) {
                    const int ch = li + 16 * m;
                    acc += va[ch] * s_k[rb * DK + ch] * __builtin_amdgcn_exp2f(s_G[ra * DK + ch] - s_G[rb * DK + ch]);
                }
            }
            acc = row_ror_add<8>(row_ror_add<4>(row_ror_add<2>(row_ror_add<1>(acc))));
            if (p < npa + npm && li == 0) {
                if (p < npa) s_ab[dst] = s_beta[ra] * acc;
                else s_M[dst] = acc;
            }
        }
    }
    lds_barrier();

    // 4. P = X S0 on the matrix cores, fp32
    f32x4 pacc[2][V];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int j = 0; j < V; ++j) pacc[pp][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        if (pp < npass) {
            const float* xa = s_X + (16 * pp + ln) * Sp::XS + row0;
            if constexpr (SP >= 4) {
                // one group of four A operands ahead (the fences keep the
                // compiler from reading them all at once, which would hold
                // SP more registers beside the state)
                f32x4 av = *reinterpret_cast<const f32x4*>(xa);
#pragma unroll
                for (int s4 = 0; s4 < SP; s4 += 4) {
                    const f32x4 an = *reinterpret_cast<const f32x4*>(xa + (s4 + 4 < SP ? s4 + 4 : s4));
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < V; ++j)
                            pacc[pp][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], Sr[s4 + e][j], pacc[pp][j], 0, 0, 0);
                    av = an;
                }
            } else {
#pragma unroll
                for (int s = 0; s < SP; ++s)
#pragma unroll
                    for (int j = 0; j < V; ++j)
                        pacc[pp][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], Sr[s][j], pacc[pp][j], 0, 0, 0);
            }
        }
    }
    lds_barrier();  // every wave is done with X: P takes its place
    float* const s_P = s_X;  // [NWK][XR][PS], the row groups' partial sums
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        if (pp < npass) {
#pragma unroll
            for (int j = 0; j < V; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_P[(wk * XR + 16 * pp + 4 * lq + i) * Sp::PS + col0 + j] = pacc[pp][j][i];
        }
    }
    lds_barrier();

    // 5. the delta-rule writes u_j by forward substitution and the outputs,
    // one column per thread.  Branch-free over the 16 token slots (slots past
    // J read row 0 and are zeroed by a select), so the compiler can issue the
    // LDS reads of all steps together instead of one step at a time.
    if (tid < DV) {
        const int cc = tid;
        float u[kNJ];
#pragma unroll
        for (int i = 0; i < kNJ; ++i) {
            const int ir = i < J ? i : 0;
            float pk = 0.f;
#pragma unroll
            for (int w = 0; w < Sp::NWK; ++w) pk += s_P[(w * XR + ir) * Sp::PS + cc];
            float r = s_beta[ir] * (s_v[ir * DV + cc] - pk);
#pragma unroll
            for (int l = 0; l < i; ++l) r -= s_ab[i * kNJ + l] * u[l];
            u[i] = i < J ? r : 0.f;
        }
        // (U of the committed tokens goes where k was: every read of k is
        // done; the commit reads rows i < na only)
#pragma unroll
        for (int i = 0; i < kMaxTok; ++i) s_U[i * DV + cc] = u[i];
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t) {
            if (t < T) {
                float o = 0.f;
#pragma unroll
                for (int w = 0; w < Sp::NWK; ++w) o += s_P[(w * XR + J + t) * Sp::PS + cc];
#pragma unroll
                for (int i = 0; i < kNJ; ++i) o += (i <= na + t ? s_M[t * kNJ + i] : 0.f) * u[i];
                st(a.out + ((static_cast<int64_t>(bb) * T + t) * H + h) * DV + cc, o * s_z[t * DV + cc]);
            }
        }
    }
    if (na == 0) return;  // nothing committed: the state stays as it is
    lds_barrier();

    // 6. the committed state, in place: S = Diag(2^{G_{na-1}}) S0 + sum_i K^_i u_i^T
    // f: the factors of this lane's rows in one row of the table (2^G, or
    // K^ of committed token i); applied four rows at a time
    auto rows4 = [&](const float* f, const int s4, float (&fv)[4]) {
        if constexpr (SP >= 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(f + row0 + s4);
            fv[0] = x.x; fv[1] = x.y; fv[2] = x.z; fv[3] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) fv[e] = s4 + e < SP ? f[row0 + s4 + e] : 0.f;
        }
    };
#pragma unroll
    for (int s4 = 0; s4 < SP; s4 += 4) {
        float fv[4];
        rows4(s_kh, s4, fv);
#pragma unroll
        for (int e = 0; e < 4 && s4 + e < SP; ++e)
#pragma unroll
            for (int j = 0; j < V; ++j) Sr[s4 + e][j] *= fv[e];
    }
#pragma unroll
    for (int i = 0; i < kMaxTok; ++i) {
        if (i < na) {
            float ui[V];
#pragma unroll
            for (int j = 0; j < V; ++j) ui[j] = s_U[i * DV + col0 + j];
#pragma unroll
            for (int s4 = 0; s4 < SP; s4 += 4) {
                float fv[4];
                rows4(s_kh + (1 + i) * DK, s4, fv);
#pragma unroll
                for (int e = 0; e < 4 && s4 + e < SP; ++e)
#pragma unroll
                    for (int j = 0; j < V; ++j) Sr[s4 + e][j] += fv[e] * ui[j];
            }
        }
    }
#pragma unroll
    for (int s = 0; s < SP; ++s) {
        if constexpr (V == 2) {
            __builtin_amdgcn_raw_buffer_store_b64(i32x2{__float_as_int(Sr[s][0]), __float_as_int(Sr[s][1])}, srsrc,
                                                  Soff, 4 * DV * s, kNonTemporal);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(Sr[s][0]), srsrc, Soff, 4 * DV * s, kNonTemporal);
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
    const size_t lds = static_cast<size_t>(SpecLds<DK, DV, sizeof(XT)>(s.T).total) * sizeof(float);
    // (above 64 KB only for fp32 inputs with many tokens at d = 128)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&spec_kernel<DK, DV, XT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("spec_verify", st);
    hipLaunchKernelGGL((spec_kernel<DK, DV, XT>), dim3(static_cast<unsigned>(grid)), dim3(256), lds, st, k);
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
