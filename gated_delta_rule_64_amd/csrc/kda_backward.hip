// Gradients of the chunked recurrence (fp32 arithmetic, any supported head
// size, fp32 or bf16 inputs; the dense 64-row products on the fp32 matrix
// cores, the rest on the vector ALUs).
//
// The forward of one chunk (the chunked form of the recurrence in
// kda_prefill_common.h; decays G, A, M, T, W, U~, Q', K^, gamma as there,
// S the state at the chunk start, Q_e = e^G * Q, K_e = e^G * K, B = Diag(beta)):
//     U = U~ - W S,   O = Q' S + M U~ = Q_e S + M U,   S_end = Diag(gamma) S + K^^T U.
// Given dO (from dy and the output gate) and dS_end, its adjoint is
//     dS      = Q'^T dO + Diag(gamma) dS_end - W^T (K^ dS_end)          (the chain)
//     dU      = M^T dO + K^ dS_end
//     dM      = dO U^T,  dQ_e = dO S^T,  dK^ = U dS_end^T,  dgamma = diag(S^T dS_end)
//     dW      = -dU S^T, dU~ = dU
//     dT      = dU~ (B V)^T + dW (B K_e)^T
//     d(B V)  = T^T dU~,  d(B K_e) = T^T dW
//     dY      = -T^T dT T^T   (Y = I + B A, T = Y^-1),  d(B A) = dY below the diagonal
// and the chain rule through A, M (products of k, q and e^{G_r - G_s}), the
// e^G factors and G = cumsum(log alpha).  Three passes:
//   1. the forward: chunk records (a tiled version of the prefill's fp32
//      record kernel) and the fp32 state pass with the state at every chunk
//      start (snapshots after every chunk);
//   2. the chain, chunks in reverse order per (sequence, head, 16 columns):
//      dS_end of every chunk, and dS at the sequence start (d initial state);
//   3. per (chunk, head) in parallel: everything else.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_prefill_common.h"
#include "kda_profile.h"

namespace kda {
namespace {

template <typename XT, typename GT>
struct BwdK {
    int64_t T;
    int H, N;
    const int32_t* cu;
    const int32_t* base;      // chunk slots per sequence (prefix sums)
    const int32_t* snap_off;  // states after full chunks: sequence n's j-th at snap_off[n] + j - 1
    const float* snaps;
    const float* rec;
    const XT *q, *k, *v, *z, *dy;
    const GT *la, *beta;
    const float* S0;
    const float* dSf;
    float* dSe;  // [slot][H][dk][dv]: dS at the end of each chunk
    float* scratch;  // [slot][H]: U, dO, dU [64][dv]; dW [64][dk]
    float *dq, *dk, *dv, *dla, *dbeta, *dz, *dS0;
};

// Threads of the per-chunk kernels.  Their LDS allows one workgroup per CU,
// and their phases are latency-bound, so both run 16 waves (measured on the
// 4096-token layer: the record kernel 1.58 -> 1.15 ms against 4 waves; the
// gradient kernel, with its products on the matrix cores, 3.17 ms with 4
// waves, 2.70 with 8, 2.38 with 16).
constexpr int kRecThreads = 1024;
constexpr int kGradThreads = 1024;
// runs of 16 terms a product of the gradient kernel keeps in flight ahead of
// the one it multiplies, where an operand comes from global memory
constexpr int kAhead = 2;

// Row stride (floats) of the 64 x 64 matrices in LDS (A, M, T, dT, P): the
// products below read 16 rows at one column and 16 columns at one row, and
// at a 64-float stride the first would land in one bank.
constexpr int MS = 68;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// How a 64-row, N-column result (N = 16 .. 128) is dealt to the NT / 64
// waves of a workgroup as 16 x 16 tiles: a wave takes RPW row tiles of CPW
// column tiles, starting at row r0 and column c0; waves past the tiles take
// none.  Every product of width N below, and the chain rule through A and M,
// use this deal, so a (row, channel) result always lives in the same lane.
template <int N, int NT>
struct Deal64 {
    static constexpr int W = NT / 64, CT = N / 16;
    static constexpr int CPW = CT >= W ? CT / W : 1;    // column tiles per wave
    static constexpr int WPC = CT >= W ? 1 : W / CT;    // waves per column tile
    static constexpr int RPW = WPC >= 4 ? 1 : 4 / WPC;  // row tiles per wave
    static constexpr int PER_LANE = RPW * CPW * 4;     // results per lane
    static_assert(CT * 16 == N && (CT >= W ? CT % W == 0 : W % CT == 0), "tile deal");
    int r0, c0;
    bool active;
    __device__ explicit Deal64(int wave) {
        const int part = CT >= W ? 0 : wave % WPC;
        active = part * RPW < 4;
        r0 = 16 * part * RPW;
        c0 = 16 * (CT >= W ? wave * CPW : wave / WPC);
    }
};

// C = A B for 64 rows and N columns (N = 16 .. 128), K terms (a multiple of
// 16), by the NT threads of the workgroup, on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: lane (g, c) = (lane / 16, lane % 16) gives
// A[c][g] and B[g][c] and holds D[4g + i][c]; fp32 products, fp32 sums),
// tiles dealt as Deal64 says, so each operand a wave loads serves several
// products.  Lane (g, c) takes the terms k0 + 4g .. k0 + 4g + 3 of every run
// of 16, four consecutive elements of a row-major A row.  A(r, k), B(k, c)
// read the operands; out(idx, r, c, acc) takes each result once, idx being
// its index among the lane's PER_LANE results (a constant once unrolled).
template <int N, int NT, int AHEAD = 1, typename FA, typename FB, typename FO>
__device__ __forceinline__ void mm64i(int K, FA A, FB B, FO out) {
    static_assert(AHEAD == 1 || AHEAD == 2, "one or two runs in flight");
    using D = Deal64<N, NT>;
    constexpr int RPW = D::RPW, CPW = D::CPW;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const D d(threadIdx.x >> 6);
    if (!d.active) return;  // (more waves than tiles; wave-uniform)
    const int r0 = d.r0, c0 = d.c0;
    f32x4 acc[RPW][CPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the operands of run k0 (terms k0 .. k0 + 15) into registers
    auto load = [&](int k0, float (&av)[RPW][4], float (&bv)[CPW][4]) {
        const int kk = k0 + 4 * g;
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) av[i][j] = A(r0 + 16 * i + c, kk + j);
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[jj][j] = B(kk + j, c0 + 16 * jj + c);
    };
    auto mma = [&](const float (&av)[RPW][4], const float (&bv)[CPW][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < RPW; ++i)
#pragma unroll
                for (int jj = 0; jj < CPW; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][j], bv[jj][j], acc[i][jj], 0, 0, 0);
    };
    float a0[RPW][4], b0[CPW][4], a1[RPW][4], b1[CPW][4];
    if constexpr (AHEAD == 1) {
        // two register sets: the next run's loads are in flight while this
        // run's products are issued (a clamped run index repeats a load that
        // is not used)
        if (K > 0) load(0, a0, b0);
#pragma unroll 1
        for (int k0 = 0; k0 < K; k0 += 32) {
            const bool two = k0 + 16 < K;
            load(two ? k0 + 16 : k0, a1, b1);
            mma(a0, b0);
            if (two) {
                load(k0 + 32 < K ? k0 + 32 : k0 + 16, a0, b0);
                mma(a1, b1);
            }
        }
    } else {
        // three register sets: the two next runs' loads are in flight while
        // this run's products are issued, for operands that come from global
        // memory (one round trip then covers two runs); the runs are
        // multiplied in the same order as above
        float a2[RPW][4], b2[CPW][4];
        auto cl = [&](int k) { return k < K ? k : K - 16; };
        if (K > 0) {
            load(0, a0, b0);
            load(cl(16), a1, b1);
        }
#pragma unroll 1
        for (int k0 = 0; k0 < K; k0 += 48) {
            load(cl(k0 + 32), a2, b2);
            mma(a0, b0);
            if (k0 + 16 < K) {
                load(cl(k0 + 48), a0, b0);
                mma(a1, b1);
                if (k0 + 32 < K) {
                    load(cl(k0 + 64), a1, b1);
                    mma(a2, b2);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out((i * CPW + jj) * 4 + e, r0 + 16 * i + 4 * g + e, c0 + 16 * jj + c, acc[i][jj][e]);
}

// Two products that share their B operand, C1 = A1 B and C2 = A2 B, in one
// pass: each run's B values are loaded once and serve both, and both
// products' runs wait on the same memory round trips.  Every sum is made in
// the same order as mm64i would make it.
template <int N, int NT, typename FA1, typename FA2, typename FB, typename FO1, typename FO2>
__device__ __forceinline__ void mm64i2(int K, FA1 A1, FA2 A2, FB B, FO1 out1, FO2 out2) {
    using D = Deal64<N, NT>;
    constexpr int RPW = D::RPW, CPW = D::CPW;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const D d(threadIdx.x >> 6);
    if (!d.active) return;
    const int r0 = d.r0, c0 = d.c0;
    f32x4 acc1[RPW][CPW], acc2[RPW][CPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj) acc1[i][jj] = acc2[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load = [&](int k0, float (&av1)[RPW][4], float (&av2)[RPW][4], float (&bv)[CPW][4]) {
        const int kk = k0 + 4 * g;
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                av1[i][j] = A1(r0 + 16 * i + c, kk + j);
                av2[i][j] = A2(r0 + 16 * i + c, kk + j);
            }
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[jj][j] = B(kk + j, c0 + 16 * jj + c);
    };
    auto mma = [&](const float (&av1)[RPW][4], const float (&av2)[RPW][4], const float (&bv)[CPW][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < RPW; ++i)
#pragma unroll
                for (int jj = 0; jj < CPW; ++jj) {
                    acc1[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[i][j], bv[jj][j], acc1[i][jj], 0, 0, 0);
                    acc2[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av2[i][j], bv[jj][j], acc2[i][jj], 0, 0, 0);
                }
    };
    float p0[RPW][4], q0[RPW][4], b0[CPW][4], p1[RPW][4], q1[RPW][4], b1[CPW][4];
    if (K > 0) load(0, p0, q0, b0);
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += 32) {
        const bool two = k0 + 16 < K;
        load(two ? k0 + 16 : k0, p1, q1, b1);
        mma(p0, q0, b0);
        if (two) {
            load(k0 + 32 < K ? k0 + 32 : k0 + 16, p0, q0, b0);
            mma(p1, q1, b1);
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = (i * CPW + jj) * 4 + e, r = r0 + 16 * i + 4 * g + e, cc = c0 + 16 * jj + c;
                out1(x, r, cc, acc1[i][jj][e]);
                out2(x, r, cc, acc2[i][jj][e]);
            }
}

// mm64i for callers that need no result index
template <int N, int NT, int AHEAD = 1, typename FA, typename FB, typename FO>
__device__ __forceinline__ void mm64(int K, FA A, FB B, FO out) {
    mm64i<N, NT, AHEAD>(K, A, B, [&](int, int r, int c, float v) { out(r, c, v); });
}

// In place, the running sum down the 64 rows of each of the DK channels of
// sG (row stride KP), by all NT threads: each sums RPS consecutive rows of
// one channel, and the segments' totals are combined through tmp (NT floats,
// distinct from sG).  The caller synchronises before and after.
template <int DK, int NT, int KP>
__device__ __forceinline__ void cumsum_rows(float* sG, float* tmp) {
    constexpr int NSEG = NT / DK, RPS = 64 / NSEG;
    static_assert(NSEG * DK == NT && NSEG * RPS == 64, "whole segments");
    const int c = threadIdx.x % DK, seg = threadIdx.x / DK;
    float v[RPS];
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        run += sG[(seg * RPS + i) * KP + c];
        v[i] = run;
    }
    tmp[seg * DK + c] = run;
    __syncthreads();
    float off = 0.f;
    for (int q = 0; q < seg; ++q) off += tmp[q * DK + c];
#pragma unroll
    for (int i = 0; i < RPS; ++i) sG[(seg * RPS + i) * KP + c] = v[i] + off;
}

// e^x for x <= 0 (a decay between two tokens of a chunk) through the
// hardware base-2 exponential; x > 0 only occurs for entries that are masked
// out, and is clamped to 0 so that nothing overflows
__device__ __forceinline__ float decay(float x) { return __builtin_amdgcn_exp2f(fminf(x, 0.f) * kLog2e); }

// Row stride (floats) of the per-chunk key, query and decay rows in LDS:
// rows stay 16-byte aligned for four-channel reads, and the 4-float pad
// puts 16 rows at one channel on distinct banks.
template <int DK>
constexpr int kKP = DK + 4;

// A diagonal 16 x 16 block whose decay over its 16 rows exceeds this (in any
// channel, natural-log units) is "steep": its factored form below would need
// e^{span}, which leaves the fp32 range near 88.
constexpr float kSpanMax = 80.f;

// (R, S) of tile i in the lower block triangle of a 64 x 64 matrix
// (16 x 16 blocks, R >= S), row-major order
__device__ __forceinline__ void lower_tile(int i, int& R, int& S) {
    R = i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0;
    S = i - R * (R + 1) / 2;
}

// A (strictly lower) and M (lower with diagonal) of a chunk,
//   A_rs = sum_c k_rc k_sc e^{G_rc - G_sc},  M_rs = sum_c q_rc k_sc e^{G_rc - G_sc},
// by 16 x 16 blocks (R, S), R >= S, one wave each (ten blocks).  The
// pairwise decay factors through the first row of block R:
//   e^{G_r - G_s} = e^{G_r - G_16R} e^{G_16R - G_s},
// so a block is a product over the channels of (K_R or Q_R) * e^{G_R - G_16R}
// and (K_S * e^{G_16R - G_S})^T, on the fp32 matrix cores.  Below the
// diagonal (R > S) both factors are at most 1, since G does not increase
// along the chunk.  On a diagonal block the right factor grows with the decay
// inside the block; where that could leave the fp32 range (a steep block)
// the block is summed pair by pair instead.  K, Q, G rows have stride kKP.
template <int DK, int NT>
__device__ __forceinline__ void am_mfma(const float* sK, const float* sQ, const float* sG, float* sA, float* sM) {
    static_assert(NT % 64 == 0 && DK % 16 == 0, "whole waves; whole runs of 16 channels");
    constexpr int KP = kKP<DK>, CW = DK / 4;  // lane (g, c) takes channels CW g .. CW g + CW - 1
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
#pragma unroll 1
    for (int tile = wave; tile < 10; tile += NT / 64) {
        int R, S;
        lower_tile(tile, R, S);
        const bool diag = R == S;
        bool steep = false;
        if (diag) {
            float span = 0.f;
            for (int ch = lane; ch < DK; ch += 64) span = fmaxf(span, sG[(16 * R) * KP + ch] - sG[(16 * R + 15) * KP + ch]);
            steep = __ballot(span >= kSpanMax) != 0;
        }
        if (!steep) {
            // v_mfma_f32_16x16x4_f32: lane (g, c) gives A[c][g] and B[g][c] and
            // holds D[4g + i][c]; the left rows are 16R + c, the right ones 16S + c
            const float* kr = sK + (16 * R + c) * KP + CW * g;
            const float* qr = sQ + (16 * R + c) * KP + CW * g;
            const float* gr = sG + (16 * R + c) * KP + CW * g;
            const float* gf = sG + (16 * R) * KP + CW * g;
            const float* ks = sK + (16 * S + c) * KP + CW * g;
            const float* gs = sG + (16 * S + c) * KP + CW * g;
            // exponent bounds: the left factor at most 1; the right one at most
            // 1 below the diagonal and e^{kSpanMax} on it (the bounds only bind
            // for decays that grow, which the inputs do not hold)
            const float rmax = diag ? kSpanMax * kLog2e : 0.f;
            f32x4 aa = {0.f, 0.f, 0.f, 0.f}, am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < CW / 4; ++u) {
                const float4 k4 = reinterpret_cast<const float4*>(kr)[u], q4 = reinterpret_cast<const float4*>(qr)[u];
                const float4 g4 = reinterpret_cast<const float4*>(gr)[u], f4 = reinterpret_cast<const float4*>(gf)[u];
                const float4 s4 = reinterpret_cast<const float4*>(ks)[u], h4 = reinterpret_cast<const float4*>(gs)[u];
                const float kv[4] = {k4.x, k4.y, k4.z, k4.w}, qv[4] = {q4.x, q4.y, q4.z, q4.w};
                const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, fv[4] = {f4.x, f4.y, f4.z, f4.w};
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, hv[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fl = __builtin_amdgcn_exp2f(fminf((gv[j] - fv[j]) * kLog2e, 0.f));
                    const float fr = __builtin_amdgcn_exp2f(fminf((fv[j] - hv[j]) * kLog2e, rmax));
                    const float b = sv[j] * fr;
                    aa = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[j] * fl, b, aa, 0, 0, 0);
                    am = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[j] * fl, b, am, 0, 0, 0);
                }
            }
            const int s_ = 16 * S + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * g + i;
                sA[r * MS + s_] = s_ < r ? aa[i] : 0.f;
                sM[r * MS + s_] = s_ <= r ? am[i] : 0.f;
            }
        } else {
            // the 136 pairs s <= r of the block, pair by pair over the channels;
            // the lane of pair (r, s), s < r, also clears (s, r)
            for (int p = lane; p < 136; p += 64) {
                int rl = static_cast<int>((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
                if ((rl + 1) * (rl + 2) / 2 <= p) ++rl;
                if (rl * (rl + 1) / 2 > p) --rl;
                const int sl = p - rl * (rl + 1) / 2, r = 16 * R + rl, s_ = 16 * R + sl;
                float av = 0.f, mv = 0.f;
                for (int ch = 0; ch < DK; ch += 4) {
                    const float4 k4 = *reinterpret_cast<const float4*>(sK + r * KP + ch);
                    const float4 q4 = *reinterpret_cast<const float4*>(sQ + r * KP + ch);
                    const float4 g4 = *reinterpret_cast<const float4*>(sG + r * KP + ch);
                    const float4 s4 = *reinterpret_cast<const float4*>(sK + s_ * KP + ch);
                    const float4 h4 = *reinterpret_cast<const float4*>(sG + s_ * KP + ch);
                    const float e0 = s4.x * decay(g4.x - h4.x), e1 = s4.y * decay(g4.y - h4.y);
                    const float e2 = s4.z * decay(g4.z - h4.z), e3 = s4.w * decay(g4.w - h4.w);
                    av += k4.x * e0 + k4.y * e1 + k4.z * e2 + k4.w * e3;
                    mv += q4.x * e0 + q4.y * e1 + q4.z * e2 + q4.w * e3;
                }
                sA[r * MS + s_] = sl < rl ? av : 0.f;
                sM[r * MS + s_] = mv;
                if (sl < rl) {
                    sA[s_ * MS + r] = 0.f;
                    sM[s_ * MS + r] = 0.f;
                }
            }
        }
        if (!diag) {  // the block (S, R) above the diagonal
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sA[(16 * S + 4 * g + i) * MS + 16 * R + c] = 0.f;
                sM[(16 * S + 4 * g + i) * MS + 16 * R + c] = 0.f;
            }
        }
    }
}

// T = (I + Diag(beta) A)^-1 (unit lower triangular) by 16 x 16 blocks.
// Wave w inverts diagonal block w by forward substitution inside the wave
// (no workgroup barrier per row); then the blocks below the diagonal follow by
// block distance d = 1, 2, 3:  T_ij = -T_ii sum_{k=j}^{i-1} (B A)_ik T_kj,
// which is Y T = I (Y = I + B A) written for block (i, j).  sTmp holds
// 3 x 16 x 16 floats.
template <int NT>
__device__ __forceinline__ void t_solve(const float* sA, const float* sB, float* sT, float* sTmp) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // zero everything above the diagonal blocks' lower triangles first
    for (int i = tid; i < 4096; i += NT) {
        const int r = i >> 6, c = i & 63;
        if (c > r || (r >> 4) != (c >> 4)) sT[r * MS + c] = r == c ? 1.f : 0.f;
    }
    if (wave < 4) {
        const int b0 = 16 * wave;
        const int c = b0 + (lane & 15);
        for (int rl = 0; rl < 16; ++rl) {
            const int r = b0 + rl;
            float acc = r == c ? 1.f : 0.f;
            if (c < r) {
                float sum = 0.f;
                for (int s_ = c; s_ < r; ++s_) sum += sA[r * MS + s_] * sT[s_ * MS + c];
                acc = -sB[r] * sum;
            }
            if (lane < 16) sT[r * MS + c] = acc;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // row r is visible to the wave
        }
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int nb = 4 - d;  // blocks (j + d, j), j = 0 .. nb-1
        // P_ij = sum_{k=j}^{i-1} (B A)_ik T_kj
        for (int e = tid; e < nb * 256; e += NT) {
            const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int ib = jb + d, r = 16 * ib + rr, c = 16 * jb + cc;
            float acc = 0.f;
            for (int k = 16 * jb; k < 16 * ib; ++k) acc += sA[r * MS + k] * sT[k * MS + c];
            sTmp[e] = sB[r] * acc;
        }
        __syncthreads();
        // T_ij = -T_ii P_ij
        for (int e = tid; e < nb * 256; e += NT) {
            const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int ib = jb + d, r = 16 * ib + rr, c = 16 * jb + cc;
            float acc = 0.f;
            for (int k = 0; k < 16; ++k) acc += sT[r * MS + 16 * ib + k] * sTmp[(jb << 8) + k * 16 + cc];
            sT[r * MS + c] = -acc;
        }
        __syncthreads();
    }
}

// ---- the chunk records of the fp32 path (W, U~, Q', K^, M U~, gamma; the
// layout in kda_prefill_common.h), with the tiled products above.  The fp32
// prefill makes its records here too, and pass 1 of the gradients remakes
// them.
template <int DK>
constexpr size_t rec_lds_bytes() {
    return (3 * 64 * kKP<DK> + 3 * 64 * MS + 64 + 768) * sizeof(float);  // K, Q, G; A, M, T; beta; T's scratch
}

template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(kRecThreads) void chunk_records_kernel(BwdK<XT, GT> a) {
    extern __shared__ __align__(16) float smem[];
    constexpr int KP = kKP<DK>;
    float* sK = smem;
    float* sQ = sK + 64 * KP;
    float* sG = sQ + 64 * KP;
    float* sA = sG + 64 * KP;
    float* sM = sA + 64 * MS;
    float* sT = sM + 64 * MS;
    float* sB = sT + 64 * MS;
    float* sTmp = sB + 64;
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    if (slot >= a.base[a.N]) return;
    const int n = find_seq(a.base, a.N, slot);
    const int64_t t0 = seq_begin(a.cu, n) + static_cast<int64_t>(slot - a.base[n]) * kChunk;
    const int L = static_cast<int>(min(static_cast<int64_t>(kChunk), seq_finish(a.cu, n, a.T) - t0));
    const GenRec R = gen_rec(DK, DV);
    float* rec = const_cast<float*>(a.rec) + (static_cast<int64_t>(slot) * a.H + h) * R.size;
    auto tok = [&](int r) { return (t0 + r) * a.H + h; };
    {
        // every load of the chunk's keys, queries and decays goes out before
        // the first is stored (padded tokens: no decay, no write)
        constexpr int NP = 64 * DK / kRecThreads;
        static_assert(NP * kRecThreads == 64 * DK, "whole passes");
        float kv[NP], qv[NP], gv[NP];
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int i = tid + it * kRecThreads, r = i / DK, c = i % DK;
            // rows past the chunk's end read row 0 (L >= 1) and drop it, so
            // no load sits under a branch that would wait for it
            const bool in = r < L;
            const int64_t o = tok(in ? r : 0) * DK + c;
            const float kr = ld(a.k + o), qr = ld(a.q + o), gr = ld(a.la + o);
            kv[it] = in ? kr : 0.f;
            qv[it] = in ? qr : 0.f;
            gv[it] = in ? gr : 0.f;
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int i = tid + it * kRecThreads, r = i / DK, c = i % DK;
            sK[r * KP + c] = kv[it];
            sQ[r * KP + c] = qv[it];
            sG[r * KP + c] = gv[it];
        }
    }
    if (tid < 64) sB[tid] = tid < L ? ld(a.beta + tok(tid)) : 0.f;
    __syncthreads();
    cumsum_rows<DK, kRecThreads, KP>(sG, sA);  // (A is made after this)
    __syncthreads();
    // K^ and gamma (G_last = G_63: padded rows add no decay)
    for (int i = tid; i < 64 * DK; i += kRecThreads) {
        const int r = i / DK, c = i % DK;
        rec[R.Kh + i] = expf(sG[63 * KP + c] - sG[r * KP + c]) * sK[r * KP + c];
    }
    if (tid < DK) rec[R.gam + tid] = expf(sG[63 * KP + tid]);
    am_mfma<DK, kRecThreads>(sK, sQ, sG, sA, sM);
    __syncthreads();
    t_solve<kRecThreads>(sA, sB, sT, sTmp);
    // W = T (B e^G K),  U~ = T (B V)
    mm64<DK, kRecThreads>(64, [&](int r, int s_) { return sT[r * MS + s_]; },
             [&](int s_, int c) { return sB[s_] * expf(sG[s_ * KP + c]) * sK[s_ * KP + c]; },
             [&](int r, int c, float acc) { rec[R.W + r * DK + c] = acc; });
    mm64<DV, kRecThreads>(64, [&](int r, int s_) { return sT[r * MS + s_]; },
             [&](int s_, int c) {
                 const float vv = ld(a.v + tok(s_ < L ? s_ : 0) * DV + c);
                 return s_ < L ? sB[s_] * vv : 0.f;
             },
             [&](int r, int c, float acc) { rec[R.U + r * DV + c] = acc; });
    __syncthreads();  // W and U~ are in the record
    // Q' = e^G Q - M W,  M U~
    mm64<DK, kRecThreads>(64, [&](int r, int s_) { return sM[r * MS + s_]; }, [&](int s_, int c) { return rec[R.W + s_ * DK + c]; },
             [&](int r, int c, float acc) {
                 rec[R.Qp + r * DK + c] = expf(sG[r * KP + c]) * sQ[r * KP + c] - acc;
             });
    mm64<DV, kRecThreads>(64, [&](int r, int s_) { return sM[r * MS + s_]; }, [&](int s_, int c) { return rec[R.U + s_ * DV + c]; },
             [&](int r, int c, float acc) { rec[R.Oi + r * DV + c] = acc; });
}

// ---- pass 2: the chain, chunks in reverse order ----
// Four waves on the fp32 matrix cores, laid out as the forward state pass:
// per chunk, wave w makes token rows 16w .. 16w + 15 of X = K^ dS and of
// dO = dy * sigmoid(z); then the waves that own rows of dS update them,
//     dS <- Diag(gamma) dS + Q'^T dO - W^T X.
// dS (the B operand of K^ dS) and X, dO (of the update) are shared through
// LDS; a wave keeps its rows of dS as matrix-core accumulators, and reloads
// each operand it takes from the record, for the next chunk, as soon as the
// products that use it are issued.
constexpr int kCS = 20;  // LDS row stride of dS, X, dO (16 columns): rows 4g + jj of lanes (g, c) hit distinct banks

template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdK<XT, GT> a) {
    constexpr int KB = DK / 16, ST = DK / 16, SPW = ST >= 4 ? ST / 4 : 1;
    __shared__ float sD[DK * kCS];
    __shared__ float sX[64 * kCS];
    __shared__ float sO[64 * kCS];
    constexpr int NSL = DV / 16;
    const SliceBlock sbk = slice_block(blockIdx.x, NSL);
    if (sbk.grp >= static_cast<int64_t>(a.N) * a.H) return;
    const int sl = sbk.sl, h = static_cast<int>(sbk.grp % a.H), n = static_cast<int>(sbk.grp / a.H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    const bool owner = wave * SPW < ST;  // (below d = 64 some waves own no rows of dS)
    auto i0 = [&](int t) { return owner ? 16 * (wave * SPW + t) : 0; };
    const GenRec R = gen_rec(DK, DV);
    const int64_t sidx = (static_cast<int64_t>(n) * a.H + h) * DK * DV;
    const int col = 16 * sl + c;
    const bool has_z = a.z != nullptr;
    const XT* zp = has_z ? a.z : a.v;  // (same [T][H][dv] layout; read but unused without a gate)
    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    const int nch = a.base[n + 1] - a.base[n];
    auto rec_of = [&](int j) { return a.rec + (static_cast<int64_t>(a.base[n] + j) * a.H + h) * R.size; };
    auto len_of = [&](int j) {
        return static_cast<int>(min(static_cast<int64_t>(kChunk), se - (sb + static_cast<int64_t>(j) * kChunk)));
    };
    // a wave's operands of one chunk
    f32x4 kA[KB];          // K^[16 wave + c][16 kb + 4g .. + 3]
    float qT[SPW][4][4];   // Q'[16 kb + 4g + jj][i0 + c]
    float wT[SPW][4][4];   // -W[16 kb + 4g + jj][i0 + c]
    float gam[SPW][4];     // gamma[i0 + 4g + e]
    float dyv[4], zv[4];   // dy, z at token 16 wave + 4g + e, column col
    auto load_k = [&](const float* rec) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            kA[kb] = *reinterpret_cast<const f32x4*>(rec + R.Kh + (16 * wave + c) * DK + 16 * kb + 4 * g);
    };
    auto load_io = [&](int j) {
        const int L = len_of(j);
        const int64_t t0 = sb + static_cast<int64_t>(j) * kChunk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t oidx = ((t0 + min(16 * wave + 4 * g + e, L - 1)) * a.H + h) * DV + col;
            dyv[e] = ld(a.dy + oidx);
            zv[e] = ld(zp + oidx);
        }
    };
    auto load_t = [&](const float* rec) {
#pragma unroll
        for (int t = 0; t < SPW; ++t) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t off = (16 * kb + 4 * g + jj) * DK + i0(t) + c;
                    qT[t][kb][jj] = rec[R.Qp + off];
                    wT[t][kb][jj] = -rec[R.W + off];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) gam[t][e] = rec[R.gam + i0(t) + 4 * g + e];
        }
    };
    // this wave's rows of dS: tile t holds rows i0(t) + 4g + e, column col
    f32x4 D[SPW];
#pragma unroll
    for (int t = 0; t < SPW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = i0(t) + 4 * g + e;
            D[t][e] = a.dSf && owner ? a.dSf[sidx + row * DV + col] : 0.f;
            if (owner) sD[row * kCS + c] = D[t][e];
        }
    if (nch > 0) {
        const float* rec = rec_of(nch - 1);
        load_k(rec);
        load_io(nch - 1);
        load_t(rec);
    }
    __syncthreads();
    for (int j = nch - 1; j >= 0; --j) {
        const int slot = a.base[n] + j;
        const int L = len_of(j);
        const int jn = max(j - 1, 0);  // (the last step reloads its own chunk, unused)
        const float* rec_next = rec_of(jn);
        // dS at this chunk's end
        if (owner) {
            float* dse = a.dSe + (static_cast<int64_t>(slot) * a.H + h) * DK * DV;
#pragma unroll
            for (int t = 0; t < SPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) dse[(i0(t) + 4 * g + e) * DV + col] = D[t][e];
        }
        // dO = dy * sigmoid(z) on the chunk's tokens, 0 on padding
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * wave + 4 * g + e;
            const float d = has_z ? dyv[e] * sigmoid(zv[e]) : dyv[e];
            sO[r * kCS + c] = r < L ? d : 0.f;
        }
        load_io(jn);
        // X = K^ dS, rows 16 wave .. + 15 (all of dS's operand values read first)
        float bd[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bd[kb][jj] = sD[(16 * kb + 4 * g + jj) * kCS + c];
        // (two accumulators, even and odd blocks of terms: two independent
        // chains of products instead of one)
        f32x4 xa2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                xa2[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kA[kb][jj], bd[kb][jj], xa2[kb & 1], 0, 0, 0);
        const f32x4 xa = xa2[0] + xa2[1];
        load_k(rec_next);
#pragma unroll
        for (int e = 0; e < 4; ++e) sX[(16 * wave + 4 * g + e) * kCS + c] = xa[e];
        __syncthreads();  // X and dO are complete; every read of dS is done
        if (owner) {
            float bo[4][4], bx[4][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    bo[kb][jj] = sO[(16 * kb + 4 * g + jj) * kCS + c];
                    bx[kb][jj] = sX[(16 * kb + 4 * g + jj) * kCS + c];
                }
            // (two accumulators a tile, Q'^T dO onto Diag(gamma) dS and W^T X
            // from zero: independent chains of products)
            f32x4 acc[SPW][2];
#pragma unroll
            for (int t = 0; t < SPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[t][0][e] = gam[t][e] * D[t][e];
                    acc[t][1][e] = 0.f;
                }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int t = 0; t < SPW; ++t) {
                        acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(qT[t][kb][jj], bo[kb][jj], acc[t][0], 0, 0, 0);
                        acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wT[t][kb][jj], bx[kb][jj], acc[t][1], 0, 0, 0);
                    }
#pragma unroll
            for (int t = 0; t < SPW; ++t) D[t] = acc[t][0] + acc[t][1];
            load_t(rec_next);
#pragma unroll
            for (int t = 0; t < SPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) sD[(i0(t) + 4 * g + e) * kCS + c] = D[t][e];
        }
        __syncthreads();  // dS is complete; every read of X and dO is done
    }
    if (a.dS0 && owner) {
#pragma unroll
        for (int t = 0; t < SPW; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.dS0[sidx + (i0(t) + 4 * g + e) * DV + col] = D[t][e];
    }
}

constexpr size_t scratch_floats(int dk, int dv) { return 3 * 64 * static_cast<size_t>(dv) + 64 * static_cast<size_t>(dk); }

template <int DK>
constexpr size_t intra_lds_bytes() {
    // K, G [64][kKP]; A, M, T, dT, P [64][MS]; beta, dbeta [64]; dG_last [DK]
    return (2 * 64 * kKP<DK> + 5 * 64 * MS + 2 * 64 + DK) * sizeof(float);
}

// ---- pass 3: per (chunk, head), every input gradient ----
template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(kGradThreads) void bwd_intra_kernel(BwdK<XT, GT> a) {
    extern __shared__ __align__(16) float smem[];
    // K and G rows padded to kKP floats: the tiles below read 4 rows at one
    // channel, which would otherwise land in one LDS bank
    constexpr int KP = kKP<DK>;
    float* sK = smem;              // [64][KP] keys
    float* sG = sK + 64 * KP;      // [64][KP] decay cumsums; at the end dG
    float* sA = sG + 64 * KP;      // [64][MS] A
    float* sM = sA + 64 * MS;      // [64][MS] M, later dM
    float* sT = sM + 64 * MS;      // [64][MS] T
    float* sdT = sT + 64 * MS;     // [64][MS] dT, later dY
    float* sP = sdT + 64 * MS;     // [64][MS] dT T^T
    float* sB = sP + 64 * MS;         // [64] beta
    float* sdB = sB + 64;          // [64] dbeta
    float* sdGl = sdB + 64;        // [DK] gradient of G_last

    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    if (slot >= a.base[a.N]) return;
    const int n = find_seq(a.base, a.N, slot);
    const int j = slot - a.base[n];
    const int64_t t0 = seq_begin(a.cu, n) + static_cast<int64_t>(j) * kChunk;
    const int L = static_cast<int>(min(static_cast<int64_t>(kChunk), seq_finish(a.cu, n, a.T) - t0));
    const GenRec R = gen_rec(DK, DV);
    const int64_t unit = static_cast<int64_t>(slot) * a.H + h;
    const float* rec = a.rec + unit * R.size;
    const float* dSe = a.dSe + unit * DK * DV;
    // the state at the chunk start
    const float* S = j == 0 ? a.S0 : a.snaps + ((static_cast<int64_t>(a.snap_off[n]) + j - 1) * a.H + h) * DK * DV;
    if (j == 0 && S != nullptr) S += (static_cast<int64_t>(n) * a.H + h) * DK * DV;
    float* scr = a.scratch + unit * scratch_floats(DK, DV);
    float* gU = scr;
    float* gdO = gU + 64 * DV;
    float* gdU = gdO + 64 * DV;
    float* gdW = gdU + 64 * DV;
    // The running sums of dq, dk, dG stay in registers: every product of
    // width DK, and the chain rule through A and M, deal element (row,
    // channel) to the same lane (Deal64), which holds it at the same index.
    constexpr int NS = Deal64<DK, kGradThreads>::PER_LANE;
    float sq[NS], sk[NS], sg[NS];
    // K_e = e^G K, for dT and d(B K_e) below
    auto ke_at = [&](int r, int c) { return expf(sG[r * KP + c]) * sK[r * KP + c]; };
    auto tok = [&](int r) { return (t0 + r) * a.H + h; };

    // ---- 0. the forward's chunk quantities: G, A, M, T.  The queries sit,
    // padded like K, in the space of T, dT, P until T is made.
    constexpr int NP = 64 * DK / kGradThreads;
    static_assert(NP * kGradThreads == 64 * DK, "whole passes");
    {
        // every load goes out before the first is stored
        float kv[NP], qv[NP], gv[NP];
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int i = tid + it * kGradThreads, r = i / DK, c = i % DK;
            // rows past the chunk's end read row 0 (L >= 1) and drop it, so
            // no load sits under a branch that would wait for it
            const bool in = r < L;
            const int64_t o = tok(in ? r : 0) * DK + c;
            const float kr = ld(a.k + o), qr = ld(a.q + o), gr = ld(a.la + o);
            kv[it] = in ? kr : 0.f;
            qv[it] = in ? qr : 0.f;
            gv[it] = in ? gr : 0.f;
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int i = tid + it * kGradThreads, r = i / DK, c = i % DK;
            sK[r * KP + c] = kv[it];
            sT[r * KP + c] = qv[it];
            sG[r * KP + c] = gv[it];
        }
    }
    if (tid < 64) {
        sB[tid] = tid < L ? ld(a.beta + tok(tid)) : 0.f;
        sdB[tid] = 0.f;
    }
    if (tid < DK) sdGl[tid] = 0.f;
    __syncthreads();
    cumsum_rows<DK, kGradThreads, KP>(sG, sA);  // (A is made after this)
    __syncthreads();
    // A (strictly lower) and M (lower with diagonal), by blocks on the matrix cores
    am_mfma<DK, kGradThreads>(sK, sT, sG, sA, sM);
    __syncthreads();  // the queries are dead; T goes where they were
    t_solve<kGradThreads>(sA, sB, sT, sP);  // (P's space is free until phase 5)

    // ---- 1. U = U~ - W S and O = Q' S + M U~ (one pass over S); dO, dz.
    // The products leave their sums in registers; every load the results
    // need (U~, M U~, dy, z) is then issued before the first store.  Taken
    // result by result, each load waited for the store before it, since the
    // compiler cannot tell the record from the scratch and output it writes.
    {
        using D1 = Deal64<DV, kGradThreads>;
        constexpr int NX = D1::PER_LANE;
        float sU[NX], sO[NX];
        int rx[NX], cx[NX];
        mm64i2<DV, kGradThreads>(S != nullptr ? DK : 0, [&](int r, int kk) { return rec[R.W + r * DK + kk]; },
                 [&](int r, int kk) { return rec[R.Qp + r * DK + kk]; },
                 [&](int kk, int c) { return S[kk * DV + c]; },
                 [&](int x, int r, int c, float acc) { sU[x] = acc; rx[x] = r; cx[x] = c; },
                 [&](int x, int, int, float acc) { sO[x] = acc; });
        const D1 d1(tid >> 6);
        if (d1.active) {
            float vu[NX], vo[NX], vdy[NX], vz[NX];
            // without a gate, z's loads read dy again (same shape) and are
            // not used: no branch between a load and the next
            const XT* zp = a.z ? a.z : a.dy;
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                const int r = rx[x], c = cx[x];
                // rows past the chunk's end read row 0 (L >= 1) and are not used
                const int64_t oidx = tok(r < L ? r : 0) * DV + c;
                vu[x] = rec[R.U + r * DV + c];
                vo[x] = rec[R.Oi + r * DV + c];
                vdy[x] = ld(a.dy + oidx);
                vz[x] = ld(zp + oidx);
            }
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                const int r = rx[x], c = cx[x];
                gU[r * DV + c] = vu[x] - sU[x];
                const float o = vo[x] + sO[x];
                float d = 0.f;
                if (r < L) {
                    if (a.z) {
                        const float sg = sigmoid(vz[x]);
                        d = vdy[x] * sg;
                        a.dz[tok(r) * DV + c] = vdy[x] * o * sg * (1.f - sg);
                    } else {
                        d = vdy[x];
                    }
                }
                gdO[r * DV + c] = d;
            }
        }
    }
    __syncthreads();
    // ---- 2. dU = M^T dO + K^ dS_end
    mm64<DV, kGradThreads, kAhead>(64, [&](int r, int s_) { return sM[s_ * MS + r]; }, [&](int s_, int c) { return gdO[s_ * DV + c]; },
             [&](int r, int c, float acc) { gdU[r * DV + c] = acc; });
    mm64<DV, kGradThreads, kAhead>(DK, [&](int r, int kk) { return rec[R.Kh + r * DK + kk]; }, [&](int kk, int c) { return dSe[kk * DV + c]; },
             [&](int r, int c, float acc) { gdU[r * DV + c] += acc; });  // (same thread, same element)
    __syncthreads();
    // ---- 3. dQ_e = dO S^T, dK^ = U dS_end^T, dW = -dU S^T; the sums of dq,
    // dk, dG start here (Q_e = e^G Q, K^ = e^{G_last - G} K)
    mm64i<DK, kGradThreads, kAhead>(S != nullptr ? DV : 0, [&](int r, int col) { return gdO[r * DV + col]; },
             [&](int col, int i) { return S[i * DV + col]; },
             [&](int x, int r, int c, float dqe) {
                 sq[x] = expf(sG[r * KP + c]) * dqe;
                 sg[x] = 0.f;  // (q's share, q e^G dQ_e, joins where q is in LDS)
             });
    mm64i<DK, kGradThreads, kAhead>(DV, [&](int r, int col) { return gU[r * DV + col]; }, [&](int col, int i) { return dSe[i * DV + col]; },
             [&](int x, int r, int c, float dkh) {
                 const float eh = expf(sG[63 * KP + c] - sG[r * KP + c]), kv = sK[r * KP + c];
                 sk[x] = eh * dkh;
                 sg[x] -= eh * kv * dkh;
                 atomicAdd(&sdGl[c], eh * kv * dkh);  // (G_last's share of K^)
             });
    mm64<DK, kGradThreads, kAhead>(S != nullptr ? DV : 0, [&](int r, int col) { return gdU[r * DV + col]; },
             [&](int col, int i) { return S[i * DV + col]; },
             [&](int r, int c, float acc) { gdW[r * DK + c] = -acc; });
    if (S != nullptr) {  // dgamma = diag(S dS_end^T); gamma = e^{G_last}
        // TPR threads per state row, each loading its columns in one batch,
        // then a sum across those lanes (a row's threads share a wave)
        constexpr int TPR = kGradThreads / DK, NCOL = (DV + TPR - 1) / TPR;
        static_assert(TPR * DK == kGradThreads && TPR <= 64, "rows dealt to lane groups");
        const int row = tid / TPR, part = tid % TPR;
        float sv[NCOL], ev[NCOL];
#pragma unroll
        for (int i = 0; i < NCOL; ++i) {
            const int col = part + TPR * i;
            sv[i] = col < DV ? S[row * DV + col] : 0.f;
            ev[i] = col < DV ? dSe[row * DV + col] : 0.f;
        }
        float dg = 0.f;
#pragma unroll
        for (int i = 0; i < NCOL; ++i) dg += sv[i] * ev[i];
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) dg += __shfl_xor(dg, off, TPR);
        if (part == 0) atomicAdd(&sdGl[row], expf(sG[63 * KP + row]) * dg);
    }
    __syncthreads();
    // ---- 4. dM = dO U^T (into M's place); dT = dU (B V)^T + dW (B K_e)^T
    mm64<64, kGradThreads, kAhead>(DV, [&](int r, int col) { return gdO[r * DV + col]; }, [&](int col, int s_) { return gU[s_ * DV + col]; },
             [&](int r, int s_, float acc) { sM[r * MS + s_] = s_ <= r ? acc : 0.f; });
    mm64<64, kGradThreads, kAhead>(DV, [&](int r, int col) { return gdU[r * DV + col]; },
             [&](int col, int s_) {
                 const float vv = ld(a.v + tok(s_ < L ? s_ : 0) * DV + col);
                 return s_ < L ? vv : 0.f;
             },
             [&](int r, int s_, float acc) { sdT[r * MS + s_] = acc; });
    mm64<64, kGradThreads>(DK, [&](int r, int kk) { return gdW[r * DK + kk]; }, [&](int kk, int s_) { return ke_at(s_, kk); },
             [&](int r, int s_, float acc) {  // (same thread, same element as just above)
                 sdT[r * MS + s_] = s_ < r ? sB[s_] * (sdT[r * MS + s_] + acc) : 0.f;
             });
    // d(B V) = T^T dU: dv, and beta's share
    mm64<DV, kGradThreads>(64, [&](int s_, int r) { return sT[r * MS + s_]; }, [&](int r, int c) { return gdU[r * DV + c]; },
             [&](int s_, int c, float acc) {
                 const float vv = ld(a.v + tok(s_ < L ? s_ : 0) * DV + c);
                 if (s_ >= L) return;
                 a.dv[tok(s_) * DV + c] = sB[s_] * acc;
                 atomicAdd(&sdB[s_], vv * acc);
             });
    // d(B K_e) = T^T dW: k's, G's and beta's shares
    mm64i<DK, kGradThreads>(64, [&](int s_, int r) { return sT[r * MS + s_]; }, [&](int r, int c) { return gdW[r * DK + c]; },
             [&](int x, int s_, int c, float acc) {
                 const float eg = expf(sG[s_ * KP + c]), ke = eg * sK[s_ * KP + c];
                 sk[x] += sB[s_] * eg * acc;
                 sg[x] += sB[s_] * ke * acc;
                 if (s_ < L) atomicAdd(&sdB[s_], ke * acc);
             });
    __syncthreads();
    // ---- 5. dY = -T^T dT T^T; d(B A) = dY below the diagonal.  The queries
    // for the chain rule through A and M are loaded now and stored once every
    // read of A and T is done.
    float qn[NP];
#pragma unroll
    for (int it = 0; it < NP; ++it) {
        const int i = tid + it * kGradThreads, r = i / DK, c = i % DK;
        const float qraw = ld(a.q + tok(r < L ? r : 0) * DK + c);  // (a load under no branch)
        qn[it] = r < L ? qraw : 0.f;
    }
    mm64<64, kGradThreads>(64, [&](int r, int s_) { return sdT[r * MS + s_]; }, [&](int s_, int c) { return sT[c * MS + s_]; },
             [&](int r, int c, float acc) { sP[r * MS + c] = acc; });
    __syncthreads();
    mm64<64, kGradThreads>(64, [&](int a_, int r) { return sT[r * MS + a_]; }, [&](int r, int c) { return sP[r * MS + c]; },
             [&](int a_, int c, float acc) { sdT[a_ * MS + c] = c < a_ ? -acc : 0.f; });
    __syncthreads();
    if (tid < 64) {  // beta's share through B A: sum_s dY_rs A_rs
        float acc = 0.f;
        for (int s_ = 0; s_ < tid; ++s_) acc += sdT[tid * MS + s_] * sA[tid * MS + s_];
        atomicAdd(&sdB[tid], acc);
    }
    __syncthreads();  // every read of A and T is done: the queries go there
    // the queries for the loops below, channels 0 .. 63 in A's space and
    // 64 .. 127 in T's (a thread's channels never straddle the two)
#pragma unroll
    for (int it = 0; it < NP; ++it) {
        const int i = tid + it * kGradThreads, r = i / DK, c = i % DK;
        (c < 64 ? sA : sT)[r * MS + (c & 63)] = qn[it];
    }
    __syncthreads();
    // ---- 6. through A (dA = B dY) and M (dM), with E_rsc = e^{G_rc - G_sc}:
    //   as row r of A and M:  dk_rc += sum_s dA_rs k_sc E,  dq_rc += sum_s dM_rs k_sc E,
    //     and dG_rc gains k_rc (the first sum) + q_rc (the second);
    //   as column s of them:  dk_sc += sum_r (dA_rs k_rc + dM_rs q_rc) E,
    //     and dG_sc loses k_sc times that sum.
    // By 16-row blocks on the fp32 matrix cores, the decay factored as in
    // am_mfma: for output rows in block B, the row sums over blocks S <= B
    // take e^{G_r - G_16B} e^{G_16B - G_s}, and the column sums over blocks
    // R >= B take e^{G_r - G_16R} e^{G_16R - G_s}.  A wave takes output tiles
    // (B, channels 16 j .. 16 j + 15) as Deal64 deals them; lane (g, c) owns
    // rows 16 B + 4 g + i of channel 16 j + c.  Where the diagonal block is
    // steep (over the tile's channels) its share is summed pair by pair.
    {
        using D = Deal64<DK, kGradThreads>;
        static_assert(D::CPW == 1, "one column tile per wave");
        const int lane = tid & 63, g = lane >> 4, c = lane & 15;
        const D dl(tid >> 6);
        const float rmax = kSpanMax * kLog2e;  // (binds on diagonal blocks only)
#pragma unroll
        for (int t = 0; t < D::RPW; ++t) {
            if (!dl.active) continue;
            const int B = dl.r0 / 16 + t, ch = dl.c0 + c;
            const float* qcol = (ch < 64 ? sA : sT) + (ch & 63);  // the queries: qcol[r * MS]
            const float gB = sG[(16 * B) * KP + ch];
            const bool steep = __ballot(gB - sG[(16 * B + 15) * KP + ch] >= kSpanMax) != 0;
            // row sums: dA_B,S (K_S e^{G_16B - G_S}) over S, and the same with dM
            f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = {0.f, 0.f, 0.f, 0.f};
            const int s_end = steep ? 16 * B : 16 * B + 16;
#pragma unroll 1
            for (int s0 = 0; s0 < s_end; s0 += 4) {
                const int s_ = s0 + g, ra = 16 * B + c;
                const float kr = sK[s_ * KP + ch] * __builtin_amdgcn_exp2f(fminf((gB - sG[s_ * KP + ch]) * kLog2e, rmax));
                xk = __builtin_amdgcn_mfma_f32_16x16x4f32(sB[ra] * sdT[ra * MS + s_], kr, xk, 0, 0, 0);
                xq = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[ra * MS + s_], kr, xq, 0, 0, 0);
            }
            float dkr[4], dqr[4], dks[4], gown[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gown[i] = sG[(16 * B + 4 * g + i) * KP + ch];
                const float fl = __builtin_amdgcn_exp2f(fminf((gown[i] - gB) * kLog2e, 0.f));
                dkr[i] = fl * xk[i];
                dqr[i] = fl * xq[i];
                dks[i] = 0.f;
            }
            // column sums: dA_R,B^T (K_R e^{G_R - G_16R}) + dM_R,B^T (Q_R e^{G_R - G_16R}),
            // then times e^{G_16R - G_s}, for each R
#pragma unroll 1
            for (int R = steep ? B + 1 : B; R < 4; ++R) {
                const float gR = sG[(16 * R) * KP + ch];
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r0 = 0; r0 < 16; r0 += 4) {
                    const int r = 16 * R + r0 + g, sc = 16 * B + c;
                    const float f = __builtin_amdgcn_exp2f(fminf((sG[r * KP + ch] - gR) * kLog2e, 0.f));
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sB[r] * sdT[r * MS + sc], sK[r * KP + ch] * f, y, 0, 0, 0);
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[r * MS + sc], qcol[r * MS] * f, y, 0, 0, 0);
                }
                const float smax = R == B ? rmax : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) dks[i] += __builtin_amdgcn_exp2f(fminf((gR - gown[i]) * kLog2e, smax)) * y[i];
            }
            if (steep) {  // the diagonal block pair by pair
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * B + 4 * g + i;
#pragma unroll 1
                    for (int u = 16 * B; u < 16 * B + 16; ++u) {
                        const float gu = sG[u * KP + ch], ku = sK[u * KP + ch];
                        if (u <= r) {  // row r, column u (dA is zero on the diagonal)
                            const float e = ku * decay(gown[i] - gu);
                            dkr[i] += sB[r] * sdT[r * MS + u] * e;
                            dqr[i] += sM[r * MS + u] * e;
                        }
                        if (u >= r)  // row u, column r
                            dks[i] += (sB[u] * sdT[u * MS + r] * ku + sM[u * MS + r] * qcol[u * MS]) * decay(gu - gown[i]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * B + 4 * g + i, x = 4 * t + i;
                const float kv = sK[r * KP + ch], qv = qcol[r * MS];
                // sq holds e^G dQ_e until here: q's share of dG through it
                sg[x] += qv * sq[x] + kv * dkr[i] + qv * dqr[i] - kv * dks[i];
                sk[x] += dkr[i] + dks[i];
                sq[x] += dqr[i];
            }
        }
    }
    __syncthreads();  // every read of sK, sG, sdT, sM is done
    // ---- 7. dla = reverse cumsum of dG (G_last is G_63); outputs
    {
        using D = Deal64<DK, kGradThreads>;
        const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
        const D dl(tid >> 6);
        if (dl.active) {
            // Every sum is taken into a register before the first store: a
            // sum the compiler left in scratch is otherwise reloaded between
            // stores, and each reload then waits for the stores before it.
            float vq[NS], vk[NS];
#pragma unroll
            for (int i = 0; i < D::RPW; ++i)
#pragma unroll
                for (int jj = 0; jj < D::CPW; ++jj)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int x = (i * D::CPW + jj) * 4 + e;
                        const int r = dl.r0 + 16 * i + 4 * g + e, c = dl.c0 + 16 * jj + cl;
                        sG[r * KP + c] = sg[x] + (r == 63 ? sdGl[c] : 0.f);
                        vq[x] = sq[x];
                        vk[x] = sk[x];
                        asm volatile("" : "+v"(vq[x]), "+v"(vk[x]));
                    }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < D::RPW; ++i)
#pragma unroll
                for (int jj = 0; jj < D::CPW; ++jj)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int x = (i * D::CPW + jj) * 4 + e;
                        const int r = dl.r0 + 16 * i + 4 * g + e, c = dl.c0 + 16 * jj + cl;
                        if (r < L) {
                            a.dq[tok(r) * DK + c] = vq[x];
                            a.dk[tok(r) * DK + c] = vk[x];
                        }
                    }
        }
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 63; r >= 0; --r) {
            acc += sG[r * KP + tid];
            if (r < L) a.dla[tok(r) * DK + tid] = acc;
        }
    }
    if (tid < L) a.dbeta[tok(tid)] = sdB[tid];
}

size_t chunk_slots_total(int64_t T, int N) { return static_cast<size_t>(chunk_slots_bound(T, N)); }

struct BwdLayout {
    size_t map, rec, snaps, snap_off, dse, scratch, total;
};

BwdLayout bwd_layout(int64_t T, int N, int H, int dk, int dv) {
    BwdLayout L;
    const size_t slots = chunk_slots_total(T, N);
    const size_t state = static_cast<size_t>(dk) * dv * 4;
    L.map = 0;
    L.rec = align_up(chunk_map_bytes(T, N), 256);
    L.snaps = align_up(L.rec + slots * H * static_cast<size_t>(gen_rec(dk, dv).size) * 4, 256);
    L.snap_off = align_up(L.snaps + static_cast<size_t>(T / kChunk) * H * state, 256);
    L.dse = align_up(L.snap_off + static_cast<size_t>(N + 1) * 4, 256);
    L.scratch = align_up(L.dse + slots * H * state, 256);
    L.total = align_up(L.scratch + slots * H * scratch_floats(dk, dv) * 4, 256);
    return L;
}

template <int DK, int DV, typename XT, typename GT>
hipError_t launch_records_typed(const BwdK<XT, GT>& k, const PrefillArgs& f, hipStream_t s) {
    const int64_t slots = chunk_slots_bound(f.T, f.N);
    if (slots == 0 || f.T == 0) return hipSuccess;
    constexpr size_t lds = rec_lds_bytes<DK>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_records_kernel<DK, DV, XT, GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("chunk_records", s);
    hipLaunchKernelGGL((chunk_records_kernel<DK, DV, XT, GT>), dim3(static_cast<unsigned>(slots), f.H),
                       dim3(kRecThreads), lds, s, k);
    return hipGetLastError();
}

template <int DK, int DV, typename XT, typename GT>
hipError_t launch_records_args(const PrefillArgs& f, hipStream_t s, const int32_t* base, float* rec) {
    BwdK<XT, GT> k{};
    k.T = f.T; k.H = f.H; k.N = f.N; k.cu = f.cu; k.base = base; k.rec = rec;
    k.q = static_cast<const XT*>(f.q); k.k = static_cast<const XT*>(f.k); k.v = static_cast<const XT*>(f.v);
    k.la = static_cast<const GT*>(f.la); k.beta = static_cast<const GT*>(f.beta);
    return launch_records_typed<DK, DV, XT, GT>(k, f, s);
}

template <int DK, int DV>
hipError_t launch_records_dims(const PrefillArgs& f, hipStream_t s, const int32_t* base, float* rec) {
    if (f.x == DT::BF16) {
        return f.gate == DT::BF16 ? launch_records_args<DK, DV, bf16, bf16>(f, s, base, rec)
                                  : launch_records_args<DK, DV, bf16, float>(f, s, base, rec);
    }
    return f.gate == DT::BF16 ? launch_records_args<DK, DV, float, bf16>(f, s, base, rec)
                              : launch_records_args<DK, DV, float, float>(f, s, base, rec);
}

template <int DK>
hipError_t launch_records_dk(const PrefillArgs& f, hipStream_t s, const int32_t* base, float* rec) {
    switch (f.dv) {
        case 16: return launch_records_dims<DK, 16>(f, s, base, rec);
        case 32: return launch_records_dims<DK, 32>(f, s, base, rec);
        case 64: return launch_records_dims<DK, 64>(f, s, base, rec);
        case 128: return launch_records_dims<DK, 128>(f, s, base, rec);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int DV, typename XT, typename GT>
hipError_t launch_bwd_typed(const BackwardArgs& b, const PrefillArgs& fa, hipStream_t s, const BwdLayout& Lo) {
    const PrefillArgs& f = b.f;
    char* ws = static_cast<char*>(f.ws);
    BwdK<XT, GT> k{};
    k.T = f.T; k.H = f.H; k.N = f.N; k.cu = f.cu;
    k.base = reinterpret_cast<const int32_t*>(ws + Lo.map);
    k.snap_off = reinterpret_cast<const int32_t*>(ws + Lo.snap_off);
    k.snaps = reinterpret_cast<const float*>(ws + Lo.snaps);
    k.rec = reinterpret_cast<const float*>(ws + Lo.rec);
    k.q = static_cast<const XT*>(f.q); k.k = static_cast<const XT*>(f.k); k.v = static_cast<const XT*>(f.v);
    k.z = static_cast<const XT*>(f.z); k.dy = static_cast<const XT*>(b.dy);
    k.la = static_cast<const GT*>(f.la); k.beta = static_cast<const GT*>(f.beta);
    k.S0 = f.S0; k.dSf = b.dS_final;
    k.dSe = reinterpret_cast<float*>(ws + Lo.dse);
    k.scratch = reinterpret_cast<float*>(ws + Lo.scratch);
    k.dq = b.dq; k.dk = b.dk; k.dv = b.dv; k.dla = b.dla; k.dbeta = b.dbeta; k.dz = b.dz; k.dS0 = b.dS0;
    const int64_t slots = chunk_slots_bound(f.T, f.N);
    {
        hipError_t e = launch_records_typed<DK, DV, XT, GT>(k, f, s);
        if (e != hipSuccess) return e;
    }
    {
        hipError_t e = launch_gen_state(fa, s, const_cast<int32_t*>(k.base), const_cast<float*>(k.rec));
        if (e != hipSuccess) return e;
    }
    {
        const int64_t blocks = slice_grid(static_cast<int64_t>(f.N) * f.H, DV / 16);
        LaunchTimer timer("bwd_chain", s);
        hipLaunchKernelGGL((bwd_chain_kernel<DK, DV, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (slots == 0 || f.T == 0) return hipSuccess;
    constexpr size_t lds = intra_lds_bytes<DK>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_intra_kernel<DK, DV, XT, GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("bwd_intra", s);
    hipLaunchKernelGGL((bwd_intra_kernel<DK, DV, XT, GT>), dim3(static_cast<unsigned>(slots), f.H), dim3(kGradThreads), lds,
                       s, k);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_dims(const BackwardArgs& b, const PrefillArgs& fa, hipStream_t s, const BwdLayout& Lo) {
    if (b.f.x == DT::BF16) {
        return b.f.gate == DT::BF16 ? launch_bwd_typed<DK, DV, bf16, bf16>(b, fa, s, Lo)
                                    : launch_bwd_typed<DK, DV, bf16, float>(b, fa, s, Lo);
    }
    return b.f.gate == DT::BF16 ? launch_bwd_typed<DK, DV, float, bf16>(b, fa, s, Lo)
                                : launch_bwd_typed<DK, DV, float, float>(b, fa, s, Lo);
}

template <int DK>
hipError_t launch_bwd_dk(const BackwardArgs& b, const PrefillArgs& fa, hipStream_t s, const BwdLayout& Lo) {
    switch (b.f.dv) {
        case 16: return launch_bwd_dims<DK, 16>(b, fa, s, Lo);
        case 32: return launch_bwd_dims<DK, 32>(b, fa, s, Lo);
        case 64: return launch_bwd_dims<DK, 64>(b, fa, s, Lo);
        case 128: return launch_bwd_dims<DK, 128>(b, fa, s, Lo);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t backward_workspace_bytes(int64_t T, int N, int H, int dk, int dv) { return bwd_layout(T, N, H, dk, dv).total; }

hipError_t launch_chunk_records(const PrefillArgs& f, hipStream_t s, const int32_t* base, float* rec) {
    switch (f.dk) {
        case 16: return launch_records_dk<16>(f, s, base, rec);
        case 32: return launch_records_dk<32>(f, s, base, rec);
        case 64: return launch_records_dk<64>(f, s, base, rec);
        case 128: return launch_records_dk<128>(f, s, base, rec);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_backward(const BackwardArgs& b, hipStream_t s) {
    const PrefillArgs& f = b.f;
    const BwdLayout Lo = bwd_layout(f.T, f.N, f.H, f.dk, f.dv);
    char* ws = static_cast<char*>(f.ws);
    int32_t* base = reinterpret_cast<int32_t*>(ws + Lo.map);
    SlotInfo* slot_info = reinterpret_cast<SlotInfo*>(ws + Lo.map + chunk_map_base_bytes(f.N));
    // 1. the forward on the fp32 path: records, and the state after every full chunk
    PrefillArgs fa = f;
    fa.out = nullptr;
    fa.S_out = nullptr;
    fa.snap.chunks = 1;
    fa.snap.out = reinterpret_cast<float*>(ws + Lo.snaps);
    fa.snap.off = reinterpret_cast<int32_t*>(ws + Lo.snap_off);
    {
        LaunchTimer timer("chunk_map", s);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, fa.cu, fa.N, fa.T, base, slot_info,
                           fa.snap.chunks, fa.snap.off);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // records (pass 1a), then the fp32 state pass over them (pass 1b), then 2. and 3.
    switch (f.dk) {
        case 16: return launch_bwd_dk<16>(b, fa, s, Lo);
        case 32: return launch_bwd_dk<32>(b, fa, s, Lo);
        case 64: return launch_bwd_dk<64>(b, fa, s, Lo);
        case 128: return launch_bwd_dk<128>(b, fa, s, Lo);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
