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
    float* scratch;  // [slot][H]: U, dO, dU [64][dv]; dW, the dq, dk, dG sums and K_e [64][dk]
    float *dq, *dk, *dv, *dla, *dbeta, *dz, *dS0;
};

// Threads of the per-chunk kernels.  Their LDS allows one workgroup per CU,
// and their phases are latency-bound, so both run 16 waves (measured on the
// 4096-token layer: the record kernel 1.58 -> 1.15 ms against 4 waves; the
// gradient kernel, with its products on the matrix cores, 3.17 ms with 4
// waves, 2.70 with 8, 2.38 with 16).
constexpr int kRecThreads = 1024;
constexpr int kGradThreads = 1024;

// Per-thread tile of a 64-row, N-column result shared by NT threads:
// TR rows x TC columns, TR * TC = 64 N / NT.
template <int N, int NT>
struct Tile64 {
    static constexpr int OUT = 64 * N / NT;
    static constexpr int TR = OUT >= 16 ? 4 : (OUT >= 8 ? 2 : 1);
    static constexpr int TC = OUT / TR;
    static constexpr int NCT = N / TC;  // column tiles
    static_assert(TR * TC == OUT && OUT >= 1 && NCT * (64 / TR) == NT, "tile shape");
};

// Row stride (floats) of the 64 x 64 matrices in LDS (A, M, T, dT, P): the
// products below read 16 rows at one column and 16 columns at one row, and
// at a 64-float stride the first would land in one bank.
constexpr int MS = 68;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// C = A B for 64 rows and N columns (N = 16 .. 128), K terms (a multiple of
// 16), by the NT threads of the workgroup, on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: lane (g, c) = (lane / 16, lane % 16) gives
// A[c][g] and B[g][c] and holds D[4g + i][c]; fp32 products, fp32 sums).
// The output's 16 x 16 tiles are dealt to the waves: a wave takes RPW row
// tiles of CPW column tiles, so each operand it loads serves several
// products.  Lane (g, c) takes the terms k0 + 4g .. k0 + 4g + 3 of every run
// of 16, four consecutive elements of a row-major A row.  A(r, k), B(k, c)
// read the operands; out(r, c, acc) takes each result once, and for equal N
// the same thread always gets the same (r, c).
template <int N, int NT, typename FA, typename FB, typename FO>
__device__ __forceinline__ void mm64(int K, FA A, FB B, FO out) {
    constexpr int W = NT / 64, CT = N / 16;
    constexpr int CPW = CT >= W ? CT / W : 1;    // column tiles per wave
    constexpr int WPC = CT >= W ? 1 : W / CT;    // waves per column tile
    constexpr int RPW = WPC >= 4 ? 1 : 4 / WPC;  // row tiles per wave
    static_assert(CT * 16 == N && (CT >= W ? CT % W == 0 : W % CT == 0), "tile deal");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const int part = CT >= W ? 0 : wave % WPC;
    if (part * RPW >= 4) return;  // (more waves than tiles; wave-uniform)
    const int r0 = 16 * part * RPW, c0 = 16 * (CT >= W ? wave * CPW : wave / WPC);
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
    // two register sets: the next run's loads are in flight while this run's
    // products are issued (a clamped run index repeats a load that is not used)
    float a0[RPW][4], b0[CPW][4], a1[RPW][4], b1[CPW][4];
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
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) out(r0 + 16 * i + 4 * g + e, c0 + 16 * jj + c, acc[i][jj][e]);
}

// e^x for x <= 0 (a decay between two tokens of a chunk) through the
// hardware base-2 exponential; x > 0 only occurs for entries that are masked
// out, and is clamped to 0 so that nothing overflows
__device__ __forceinline__ float decay(float x) { return __builtin_amdgcn_exp2f(fminf(x, 0.f) * kLog2e); }

// A (strictly lower) and M (lower with diagonal) of a chunk, by AT x AT
// tiles of (r, s) per thread (one tile, or two for 512 threads); K, Q, G
// rows padded to DK + 1 floats in LDS.
template <int DK, int NT>
__device__ __forceinline__ void am_tiles(const float* sK, const float* sQ, const float* sG, float* sA, float* sM) {
    constexpr int KP = DK + 1;
    constexpr int AT = NT == 256 ? 4 : 2, GD = 64 / AT;
    static_assert(GD * GD == NT || GD * GD == 2 * NT, "one or two tiles per thread");
    for (int tile = threadIdx.x; tile < GD * GD; tile += NT) {
        const int r0 = AT * (tile / GD), s0 = AT * (tile % GD);
        float av[AT][AT], mv[AT][AT];
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int jj = 0; jj < AT; ++jj) av[i][jj] = mv[i][jj] = 0.f;
        if (s0 <= r0 + AT - 1) {  // the tile reaches the lower triangle
            for (int c = 0; c < DK; ++c) {
                float kr[AT], qr[AT], gr[AT], ks[AT], gs[AT];
#pragma unroll
                for (int i = 0; i < AT; ++i) {
                    kr[i] = sK[(r0 + i) * KP + c];
                    qr[i] = sQ[(r0 + i) * KP + c];
                    gr[i] = sG[(r0 + i) * KP + c];
                    ks[i] = sK[(s0 + i) * KP + c];
                    gs[i] = sG[(s0 + i) * KP + c];
                }
#pragma unroll
                for (int i = 0; i < AT; ++i)
#pragma unroll
                    for (int jj = 0; jj < AT; ++jj) {
                        // e^{G_r - G_s}; above the diagonal the exponent is
                        // clamped (those entries are dropped below)
                        const float ke = ks[jj] * decay(gr[i] - gs[jj]);
                        av[i][jj] += kr[i] * ke;
                        mv[i][jj] += qr[i] * ke;
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int jj = 0; jj < AT; ++jj) {
                const int r = r0 + i, s_ = s0 + jj;
                sA[r * MS + s_] = s_ < r ? av[i][jj] : 0.f;
                sM[r * MS + s_] = s_ <= r ? mv[i][jj] : 0.f;
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
    return (3 * 64 * (DK + 1) + 3 * 64 * MS + 64 + 768) * sizeof(float);  // K, Q, G; A, M, T; beta; T's scratch
}

template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(kRecThreads) void chunk_records_kernel(BwdK<XT, GT> a) {
    extern __shared__ __align__(16) float smem[];
    constexpr int KP = DK + 1;
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
    for (int i = tid; i < 64 * DK; i += kRecThreads) {
        const int r = i / DK, c = i % DK;
        const bool in = r < L;
        sK[r * KP + c] = in ? ld(a.k + tok(r) * DK + c) : 0.f;
        sQ[r * KP + c] = in ? ld(a.q + tok(r) * DK + c) : 0.f;
        sG[r * KP + c] = in ? ld(a.la + tok(r) * DK + c) : 0.f;  // padded tokens: no decay, no write
    }
    if (tid < 64) sB[tid] = tid < L ? ld(a.beta + tok(tid)) : 0.f;
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) {
            acc += sG[r * KP + tid];
            sG[r * KP + tid] = acc;
        }
    }
    __syncthreads();
    // K^ and gamma (G_last = G_63: padded rows add no decay)
    for (int i = tid; i < 64 * DK; i += kRecThreads) {
        const int r = i / DK, c = i % DK;
        rec[R.Kh + i] = expf(sG[63 * KP + c] - sG[r * KP + c]) * sK[r * KP + c];
    }
    if (tid < DK) rec[R.gam + tid] = expf(sG[63 * KP + tid]);
    am_tiles<DK, kRecThreads>(sK, sQ, sG, sA, sM);
    __syncthreads();
    t_solve<kRecThreads>(sA, sB, sT, sTmp);
    // W = T (B e^G K),  U~ = T (B V)
    mm64<DK, kRecThreads>(64, [&](int r, int s_) { return sT[r * MS + s_]; },
             [&](int s_, int c) { return sB[s_] * expf(sG[s_ * KP + c]) * sK[s_ * KP + c]; },
             [&](int r, int c, float acc) { rec[R.W + r * DK + c] = acc; });
    mm64<DV, kRecThreads>(64, [&](int r, int s_) { return sT[r * MS + s_]; },
             [&](int s_, int c) { return s_ < L ? sB[s_] * ld(a.v + tok(s_) * DV + c) : 0.f; },
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
        f32x4 xa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) xa = __builtin_amdgcn_mfma_f32_16x16x4f32(kA[kb][jj], bd[kb][jj], xa, 0, 0, 0);
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
#pragma unroll
            for (int t = 0; t < SPW; ++t) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = gam[t][e] * D[t][e];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qT[t][kb][jj], bo[kb][jj], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wT[t][kb][jj], bx[kb][jj], acc, 0, 0, 0);
                    }
                D[t] = acc;
            }
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

constexpr size_t scratch_floats(int dk, int dv) { return 3 * 64 * static_cast<size_t>(dv) + 5 * 64 * static_cast<size_t>(dk); }

template <int DK>
constexpr size_t intra_lds_bytes() {
    // K, G [64][DK + 1]; A, M, T, dT, P [64][MS]; beta, dbeta [64]; dG_last [DK]
    return (2 * 64 * (DK + 1) + 5 * 64 * MS + 2 * 64 + DK) * sizeof(float);
}

// ---- pass 3: per (chunk, head), every input gradient ----
template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(kGradThreads) void bwd_intra_kernel(BwdK<XT, GT> a) {
    extern __shared__ __align__(16) float smem[];
    // K and G rows padded to DK + 1 floats: the tiles below read 4 rows at
    // one channel, which would otherwise land in one LDS bank
    constexpr int KP = DK + 1;
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
    // running sums of dq, dk, dG: between two barriers, element (row,
    // channel) is touched by one thread only (every product of width DK
    // gives it to the same thread), so plain read-modify-writes suffice
    float* gq = gdW + 64 * DK;
    float* gk = gq + 64 * DK;
    float* gG = gk + 64 * DK;
    float* gKe = gG + 64 * DK;
    auto tok = [&](int r) { return (t0 + r) * a.H + h; };

    // ---- 0. the forward's chunk quantities: G, A, M, T
    for (int i = tid; i < 64 * DK; i += kGradThreads) {
        const int r = i / DK, c = i % DK;
        const bool in = r < L;
        sK[r * KP + c] = in ? ld(a.k + tok(r) * DK + c) : 0.f;
        sG[r * KP + c] = in ? ld(a.la + tok(r) * DK + c) : 0.f;
    }
    if (tid < 64) {
        sB[tid] = tid < L ? ld(a.beta + tok(tid)) : 0.f;
        sdB[tid] = 0.f;
    }
    if (tid < DK) sdGl[tid] = 0.f;
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) {
            acc += sG[r * KP + tid];
            sG[r * KP + tid] = acc;
        }
    }
    __syncthreads();
    // A (strictly lower) and M (lower with diagonal) by 4 x 4 tiles of (r, s);
    // the queries sit, padded like K, in the space of T, dT, P until T is made
    {
        float* sQ = sT;
        for (int i = tid; i < 64 * DK; i += kGradThreads) {
            const int r = i / DK, c = i % DK;
            sQ[r * KP + c] = r < L ? ld(a.q + tok(r) * DK + c) : 0.f;
        }
        __syncthreads();
        am_tiles<DK, kGradThreads>(sK, sQ, sG, sA, sM);
        __syncthreads();  // the queries are dead; T goes where they were
    }
    t_solve<kGradThreads>(sA, sB, sT, sP);  // (P's space is free until phase 5)

    // ---- 1. U = U~ - W S and O = Q' S + M U~; dO, dz
    mm64<DV, kGradThreads>(S != nullptr ? DK : 0, [&](int r, int kk) { return rec[R.W + r * DK + kk]; },
             [&](int kk, int c) { return S[kk * DV + c]; },
             [&](int r, int c, float acc) { gU[r * DV + c] = rec[R.U + r * DV + c] - acc; });
    mm64<DV, kGradThreads>(S != nullptr ? DK : 0, [&](int r, int kk) { return rec[R.Qp + r * DK + kk]; },
             [&](int kk, int c) { return S[kk * DV + c]; },
             [&](int r, int c, float acc) {
                 const float o = rec[R.Oi + r * DV + c] + acc;
                 float d = 0.f;
                 if (r < L) {
                     const int64_t oidx = tok(r) * DV + c;
                     const float dy = ld(a.dy + oidx);
                     if (a.z) {
                         const float sg = sigmoid(ld(a.z + oidx));
                         d = dy * sg;
                         a.dz[oidx] = dy * o * sg * (1.f - sg);
                     } else {
                         d = dy;
                     }
                 }
                 gdO[r * DV + c] = d;
             });
    // K_e = e^G K, for dT and d(B K_e) below
    for (int e = tid; e < 64 * DK; e += kGradThreads) {
        const int r = e / DK, c = e % DK;
        gKe[e] = expf(sG[r * KP + c]) * sK[r * KP + c];
    }
    __syncthreads();
    // ---- 2. dU = M^T dO + K^ dS_end
    mm64<DV, kGradThreads>(64, [&](int r, int s_) { return sM[s_ * MS + r]; }, [&](int s_, int c) { return gdO[s_ * DV + c]; },
             [&](int r, int c, float acc) { gdU[r * DV + c] = acc; });
    mm64<DV, kGradThreads>(DK, [&](int r, int kk) { return rec[R.Kh + r * DK + kk]; }, [&](int kk, int c) { return dSe[kk * DV + c]; },
             [&](int r, int c, float acc) { gdU[r * DV + c] += acc; });  // (same thread, same element)
    __syncthreads();
    // ---- 3. dQ_e = dO S^T, dK^ = U dS_end^T, dW = -dU S^T; the sums of dq,
    // dk, dG start here (Q_e = e^G Q, K^ = e^{G_last - G} K)
    mm64<DK, kGradThreads>(S != nullptr ? DV : 0, [&](int r, int col) { return gdO[r * DV + col]; },
             [&](int col, int i) { return S[i * DV + col]; },
             [&](int r, int c, float dqe) {
                 const float eg = expf(sG[r * KP + c]);
                 const float qv = r < L ? ld(a.q + tok(r) * DK + c) : 0.f;
                 gq[r * DK + c] = eg * dqe;
                 gG[r * DK + c] = eg * qv * dqe;
             });
    mm64<DK, kGradThreads>(DV, [&](int r, int col) { return gU[r * DV + col]; }, [&](int col, int i) { return dSe[i * DV + col]; },
             [&](int r, int c, float dkh) {
                 const int e = r * DK + c;
                 const float eh = expf(sG[63 * KP + c] - sG[r * KP + c]), kv = sK[r * KP + c];
                 gk[e] = eh * dkh;
                 gG[e] -= eh * kv * dkh;
                 atomicAdd(&sdGl[c], eh * kv * dkh);  // (G_last's share of K^)
             });
    mm64<DK, kGradThreads>(S != nullptr ? DV : 0, [&](int r, int col) { return gdU[r * DV + col]; },
             [&](int col, int i) { return S[i * DV + col]; },
             [&](int r, int c, float acc) { gdW[r * DK + c] = -acc; });
    if (tid < DK) {  // dgamma = diag(S^T dS_end); gamma = e^{G_last}
        float dg = 0.f;
        if (S != nullptr)
            for (int col = 0; col < DV; ++col) dg += S[tid * DV + col] * dSe[tid * DV + col];
        atomicAdd(&sdGl[tid], expf(sG[63 * KP + tid]) * dg);
    }
    __syncthreads();
    // ---- 4. dM = dO U^T (into M's place); dT = dU (B V)^T + dW (B K_e)^T
    mm64<64, kGradThreads>(DV, [&](int r, int col) { return gdO[r * DV + col]; }, [&](int col, int s_) { return gU[s_ * DV + col]; },
             [&](int r, int s_, float acc) { sM[r * MS + s_] = s_ <= r ? acc : 0.f; });
    mm64<64, kGradThreads>(DV, [&](int r, int col) { return gdU[r * DV + col]; },
             [&](int col, int s_) { return s_ < L ? ld(a.v + tok(s_) * DV + col) : 0.f; },
             [&](int r, int s_, float acc) { sdT[r * MS + s_] = acc; });
    mm64<64, kGradThreads>(DK, [&](int r, int kk) { return gdW[r * DK + kk]; }, [&](int kk, int s_) { return gKe[s_ * DK + kk]; },
             [&](int r, int s_, float acc) {  // (same thread, same element as just above)
                 sdT[r * MS + s_] = s_ < r ? sB[s_] * (sdT[r * MS + s_] + acc) : 0.f;
             });
    // d(B V) = T^T dU: dv, and beta's share
    mm64<DV, kGradThreads>(64, [&](int s_, int r) { return sT[r * MS + s_]; }, [&](int r, int c) { return gdU[r * DV + c]; },
             [&](int s_, int c, float acc) {
                 if (s_ >= L) return;
                 a.dv[tok(s_) * DV + c] = sB[s_] * acc;
                 atomicAdd(&sdB[s_], ld(a.v + tok(s_) * DV + c) * acc);
             });
    // d(B K_e) = T^T dW: k's, G's and beta's shares
    mm64<DK, kGradThreads>(64, [&](int s_, int r) { return sT[r * MS + s_]; }, [&](int r, int c) { return gdW[r * DK + c]; },
             [&](int s_, int c, float acc) {
                 const int e = s_ * DK + c;
                 const float ke = gKe[e];
                 gk[e] += sB[s_] * expf(sG[s_ * KP + c]) * acc;
                 gG[e] += sB[s_] * ke * acc;
                 if (s_ < L) atomicAdd(&sdB[s_], ke * acc);
             });
    __syncthreads();
    // ---- 5. dY = -T^T dT T^T; d(B A) = dY below the diagonal
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
    auto qs = [&](int r, int c) -> float& { return (c < 64 ? sA : sT)[r * MS + (c & 63)]; };
    for (int i = tid; i < 64 * DK; i += kGradThreads) {
        const int r = i / DK, c = i % DK;
        qs(r, c) = r < L ? ld(a.q + tok(r) * DK + c) : 0.f;
    }
    __syncthreads();
    // ---- 6. through A (dA = B dY) and M (dM), with E_rsc = e^{G_rc - G_sc}.
    // Thread tiles of Tile64<DK>: rows R0 .. R0+TR-1, channels C0 .. C0+TC-1.
    // As row r of A and M:  dk_rc += sum_s dA_rs k_sc E,  dq_rc += sum_s dM_rs k_sc E,
    //   and dG_rc gains k_rc (the first sum) + q_rc (the second);
    // as column s of them:  dk_sc += sum_r w_rsc E with w = dA_rs k_rc + dM_rs q_rc,
    //   and dG_sc loses k_sc times that sum.
    {
        constexpr int TC = Tile64<DK, kGradThreads>::TC, NCT = Tile64<DK, kGradThreads>::NCT, TR = Tile64<DK, kGradThreads>::TR;
        const int C0 = TC * (tid % NCT), R0 = TR * (tid / NCT);
        float dkr[TR][TC], dqr[TR][TC], dks[TR][TC], gown[TR][TC];
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int jj = 0; jj < TC; ++jj) {
                dkr[i][jj] = dqr[i][jj] = dks[i][jj] = 0.f;
                gown[i][jj] = sG[(R0 + i) * KP + C0 + jj];
            }
        for (int s_ = 0; s_ < R0 + TR; ++s_) {  // row role: s <= r
            float da[TR], dm[TR], ks[TC], gs[TC];
#pragma unroll
            for (int i = 0; i < TR; ++i) {
                da[i] = sB[R0 + i] * sdT[(R0 + i) * MS + s_];  // (zero unless s < r)
                dm[i] = sM[(R0 + i) * MS + s_];                // (zero unless s <= r)
            }
#pragma unroll
            for (int jj = 0; jj < TC; ++jj) {
                ks[jj] = sK[s_ * KP + C0 + jj];
                gs[jj] = sG[s_ * KP + C0 + jj];
            }
#pragma unroll
            for (int i = 0; i < TR; ++i)
#pragma unroll
                for (int jj = 0; jj < TC; ++jj) {
                    const float ke = ks[jj] * decay(gown[i][jj] - gs[jj]);
                    dkr[i][jj] += da[i] * ke;
                    dqr[i][jj] += dm[i] * ke;
                }
        }
        for (int r2 = R0; r2 < 64; ++r2) {  // column role: r >= s
            float da[TR], dm[TR], kr[TC], qr[TC], gr[TC];
#pragma unroll
            for (int i = 0; i < TR; ++i) {
                da[i] = sB[r2] * sdT[r2 * MS + R0 + i];
                dm[i] = sM[r2 * MS + R0 + i];
            }
#pragma unroll
            for (int jj = 0; jj < TC; ++jj) {
                kr[jj] = sK[r2 * KP + C0 + jj];
                qr[jj] = qs(r2, C0 + jj);
                gr[jj] = sG[r2 * KP + C0 + jj];
            }
#pragma unroll
            for (int i = 0; i < TR; ++i)
#pragma unroll
                for (int jj = 0; jj < TC; ++jj)
                    dks[i][jj] += (da[i] * kr[jj] + dm[i] * qr[jj]) * decay(gr[jj] - gown[i][jj]);
        }
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int jj = 0; jj < TC; ++jj) {
                const int r = R0 + i, c = C0 + jj, e = r * DK + c;
                const float kv = sK[r * KP + c], qv = qs(r, c);
                gk[e] += dkr[i][jj] + dks[i][jj];
                gq[e] += dqr[i][jj];
                gG[e] += kv * dkr[i][jj] + qv * dqr[i][jj] - kv * dks[i][jj];
            }
    }
    __syncthreads();  // every read of sK, sG, sdT, sM is done
    // ---- 7. dla = reverse cumsum of dG (G_last is G_63); outputs
    for (int e = tid; e < 64 * DK; e += kGradThreads) {
        const int r = e / DK, c = e % DK;
        sG[r * KP + c] = gG[e] + (r == 63 ? sdGl[c] : 0.f);
        if (r < L) {
            a.dq[tok(r) * DK + c] = gq[e];
            a.dk[tok(r) * DK + c] = gk[e];
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
