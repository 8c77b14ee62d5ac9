// Gradients of the chunked recurrence (fp32 vector path, any supported head
// size, fp32 or bf16 inputs).
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
//   1. the forward: chunk records and the state at every chunk start
//      (snapshots after every chunk);
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
    float* scratch;  // [slot][H]: U, dO, dU [64][dv]; dW, and the dq, dk, dG sums [64][dk]
    float *dq, *dk, *dv, *dla, *dbeta, *dz, *dS0;
};

// ---- pass 2: the chain, chunks in reverse order ----
template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdK<XT, GT> a) {
    __shared__ float sD[DK * 16];  // dS, this block's 16 columns
    __shared__ float sX[64 * 16];  // K^ dS
    __shared__ float sO[64 * 16];  // dO
    constexpr int NSL = DV / 16;
    const int sl = blockIdx.x % NSL;
    const int h = (blockIdx.x / NSL) % a.H;
    const int n = blockIdx.x / (NSL * a.H);
    const int tid = threadIdx.x;
    const GenRec R = gen_rec(DK, DV);
    const int64_t sidx = (static_cast<int64_t>(n) * a.H + h) * DK * DV;
    for (int e = tid; e < DK * 16; e += 256) {
        const int i = e >> 4, c = e & 15;
        sD[e] = a.dSf ? a.dSf[sidx + i * DV + 16 * sl + c] : 0.f;
    }
    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    const int nch = a.base[n + 1] - a.base[n];
    const int r = tid >> 2, c4 = (tid & 3) * 4;
    for (int j = nch - 1; j >= 0; --j) {
        const int slot = a.base[n] + j;
        const float* rec = a.rec + (static_cast<int64_t>(slot) * a.H + h) * R.size;
        const int64_t t0 = sb + static_cast<int64_t>(j) * kChunk;
        const int L = static_cast<int>(min(static_cast<int64_t>(kChunk), se - t0));
        __syncthreads();  // dS of this chunk's end is in sD
        float* dse = a.dSe + (static_cast<int64_t>(slot) * a.H + h) * DK * DV;
        for (int e = tid; e < DK * 16; e += 256) dse[(e >> 4) * DV + 16 * sl + (e & 15)] = sD[e];
        // dO = dy * sigmoid(z) on the chunk's tokens, 0 on padding
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float d = 0.f;
            if (r < L) {
                const int64_t oidx = ((t0 + r) * a.H + h) * DV + 16 * sl + c4 + i;
                d = ld(a.dy + oidx);
                if (a.z) d *= sigmoid(ld(a.z + oidx));
            }
            sO[r * 16 + c4 + i] = d;
        }
        // X = K^ dS
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < DK; ++i) {
            const float kh = rec[R.Kh + r * DK + i];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) x[cc] += kh * sD[i * 16 + c4 + cc];
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) sX[r * 16 + c4 + cc] = x[cc];
        __syncthreads();
        // dS <- Q'^T dO + Diag(gamma) dS - W^T X
        for (int e = tid; e < DK * 16; e += 256) {
            const int i = e >> 4, c = e & 15;
            float acc = rec[R.gam + i] * sD[e];
            for (int rr = 0; rr < 64; ++rr)
                acc += rec[R.Qp + rr * DK + i] * sO[rr * 16 + c] - rec[R.W + rr * DK + i] * sX[rr * 16 + c];
            sD[e] = acc;  // (each element read and written by its own thread)
        }
    }
    __syncthreads();
    if (a.dS0) {
        for (int e = tid; e < DK * 16; e += 256) a.dS0[sidx + (e >> 4) * DV + 16 * sl + (e & 15)] = sD[e];
    }
}

constexpr size_t scratch_floats(int dk, int dv) { return 3 * 64 * static_cast<size_t>(dv) + 4 * 64 * static_cast<size_t>(dk); }

template <int DK>
constexpr size_t intra_lds_bytes() {
    // K, G [64][DK]; A, M, T, dT, P [64][64]; beta, dbeta [64]; dG_last [DK]
    return (2 * 64 * DK + 5 * 4096 + 2 * 64 + DK) * sizeof(float);
}

// ---- pass 3: per (chunk, head), every input gradient ----
template <int DK, int DV, typename XT, typename GT>
__global__ __launch_bounds__(256) void bwd_intra_kernel(BwdK<XT, GT> a) {
    extern __shared__ float smem[];
    float* sK = smem;              // [64][DK] keys
    float* sG = sK + 64 * DK;      // [64][DK] decay cumsums; at the end dG
    float* sA = sG + 64 * DK;      // [64][64] A
    float* sM = sA + 4096;         // [64][64] M, later dM
    float* sT = sM + 4096;         // [64][64] T
    float* sdT = sT + 4096;        // [64][64] dT, later dY
    float* sP = sdT + 4096;        // [64][64] dT T^T
    float* sB = sP + 4096;         // [64] beta
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
    // running sums of dq, dk, dG: element e = (row, channel) is only ever
    // touched by thread e % 256, so plain read-modify-writes suffice
    float* gq = gdW + 64 * DK;
    float* gk = gq + 64 * DK;
    float* gG = gk + 64 * DK;
    auto tok = [&](int r) { return (t0 + r) * a.H + h; };

    // ---- 0. the forward's chunk quantities: G, A, M, T
    for (int i = tid; i < 64 * DK; i += 256) {
        const int r = i / DK, c = i % DK;
        const bool in = r < L;
        sK[i] = in ? ld(a.k + tok(r) * DK + c) : 0.f;
        sG[i] = in ? ld(a.la + tok(r) * DK + c) : 0.f;
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
            acc += sG[r * DK + tid];
            sG[r * DK + tid] = acc;
        }
    }
    __syncthreads();
    for (int i = tid; i < 4096; i += 256) {
        const int r = i >> 6, s = i & 63;
        float av = 0.f, mv = 0.f;
        if (s <= r && r < L) {
            for (int c = 0; c < DK; ++c) {
                const float ks = sK[s * DK + c] * expf(sG[r * DK + c] - sG[s * DK + c]);
                av += sK[r * DK + c] * ks;
                mv += ld(a.q + tok(r) * DK + c) * ks;
            }
        }
        sA[i] = s < r ? av : 0.f;
        sM[i] = mv;
    }
    __syncthreads();
    for (int r = 0; r < 64; ++r) {
        if (tid < 64) {
            const int c = tid;
            float acc = r == c ? 1.f : 0.f;
            if (c < r) {
                float sum = 0.f;
                for (int s = c; s < r; ++s) sum += sA[r * 64 + s] * sT[s * 64 + c];
                acc = -sB[r] * sum;
            }
            sT[r * 64 + c] = acc;
        }
        __syncthreads();
    }

    // ---- 1. U = U~ - W S and O = Q' S + M U~; dO, dz
    for (int i = tid; i < 64 * DV; i += 256) {
        const int r = i / DV, c = i % DV;
        float u = rec[R.U + i], o = rec[R.Oi + i];
        if (S != nullptr) {
            for (int kk = 0; kk < DK; ++kk) {
                const float s = S[kk * DV + c];
                u -= rec[R.W + r * DK + kk] * s;
                o += rec[R.Qp + r * DK + kk] * s;
            }
        }
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
        gU[i] = u;
        gdO[i] = d;
    }
    __syncthreads();
    // ---- 2. dU = M^T dO + K^ dS_end
    for (int i = tid; i < 64 * DV; i += 256) {
        const int r = i / DV, c = i % DV;
        float acc = 0.f;
        for (int s = r; s < 64; ++s) acc += sM[s * 64 + r] * gdO[s * DV + c];
        for (int kk = 0; kk < DK; ++kk) acc += rec[R.Kh + r * DK + kk] * dSe[kk * DV + c];
        gdU[i] = acc;
    }
    __syncthreads();
    // ---- 3. per owned (row, channel): dQ_e, dK^, dW; the sums of dq, dk,
    // dG start here
    for (int e = tid; e < 64 * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        float dqe = 0.f, dkh = 0.f, dw = 0.f;
        for (int col = 0; col < DV; ++col) {
            const float s = S != nullptr ? S[c * DV + col] : 0.f;
            dqe += gdO[r * DV + col] * s;
            dkh += gU[r * DV + col] * dSe[c * DV + col];
            dw -= gdU[r * DV + col] * s;
        }
        gdW[e] = dw;
        const float g = sG[e], glast = sG[63 * DK + c];
        const float eg = expf(g), eh = expf(glast - g);
        const float qv = r < L ? ld(a.q + tok(r) * DK + c) : 0.f;
        const float kv = sK[e];
        gq[e] = eg * dqe;             // Q_e = e^G Q
        gk[e] = eh * dkh;             // K^ = e^{G_last - G} K
        gG[e] = eg * qv * dqe - eh * kv * dkh;
        atomicAdd(&sdGl[c], eh * kv * dkh);  // (G_last's share of K^)
    }
    if (tid < DK) {  // dgamma = diag(S^T dS_end); gamma = e^{G_last}
        float dg = 0.f;
        for (int col = 0; col < DV; ++col) dg += (S != nullptr ? S[tid * DV + col] : 0.f) * dSe[tid * DV + col];
        atomicAdd(&sdGl[tid], expf(sG[63 * DK + tid]) * dg);
    }
    __syncthreads();
    // ---- 4. dM = dO U^T (into M's place); dT = dU (B V)^T + dW (B K_e)^T
    for (int i = tid; i < 4096; i += 256) {
        const int r = i >> 6, s = i & 63;
        float dm = 0.f, dt = 0.f;
        if (s <= r) {
            for (int col = 0; col < DV; ++col) dm += gdO[r * DV + col] * gU[s * DV + col];
        }
        if (s < r && s < L) {
            const float bs = sB[s];
            for (int col = 0; col < DV; ++col) dt += gdU[r * DV + col] * bs * ld(a.v + tok(s) * DV + col);
            for (int kk = 0; kk < DK; ++kk)
                dt += gdW[r * DK + kk] * bs * expf(sG[s * DK + kk]) * sK[s * DK + kk];
        }
        sM[i] = dm;
        sdT[i] = dt;
    }
    // d(B V) = T^T dU: dv, and beta's share
    for (int i = tid; i < 64 * DV; i += 256) {
        const int s = i / DV, c = i % DV;
        if (s >= L) continue;
        float acc = 0.f;
        for (int r = s; r < 64; ++r) acc += sT[r * 64 + s] * gdU[r * DV + c];
        a.dv[tok(s) * DV + c] = sB[s] * acc;
        atomicAdd(&sdB[s], ld(a.v + tok(s) * DV + c) * acc);
    }
    // d(B K_e) = T^T dW: k's and G's and beta's shares
    for (int e = tid; e < 64 * DK; e += 256) {
        const int s = e / DK, c = e % DK;
        float acc = 0.f;
        for (int r = s; r < 64; ++r) acc += sT[r * 64 + s] * gdW[r * DK + c];
        const float ke = expf(sG[e]) * sK[e];  // K_e
        gk[e] += sB[s] * expf(sG[e]) * acc;
        gG[e] += sB[s] * ke * acc;
        if (s < L) atomicAdd(&sdB[s], ke * acc);
    }
    __syncthreads();
    // ---- 5. dY = -T^T dT T^T; d(B A) = dY below the diagonal
    for (int i = tid; i < 4096; i += 256) {
        const int r = i >> 6, c = i & 63;
        float acc = 0.f;
        for (int s = 0; s < 64; ++s) acc += sdT[r * 64 + s] * sT[c * 64 + s];
        sP[i] = acc;
    }
    __syncthreads();
    for (int i = tid; i < 4096; i += 256) {
        const int a_ = i >> 6, c = i & 63;
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) acc += sT[r * 64 + a_] * sP[r * 64 + c];
        sdT[i] = c < a_ ? -acc : 0.f;  // dY, strictly lower part (B A has nothing else)
    }
    __syncthreads();
    if (tid < 64) {  // beta's share through B A: sum_s dY_rs A_rs
        float acc = 0.f;
        for (int s = 0; s < tid; ++s) acc += sdT[tid * 64 + s] * sA[tid * 64 + s];
        atomicAdd(&sdB[tid], acc);
    }
    // ---- 6. through A (dA = B dY) and M (dM), with E_rsc = e^{G_rc - G_sc}
    for (int e = tid; e < 64 * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        const float gr = sG[e], kr = sK[e];
        const float qr = r < L ? ld(a.q + tok(r) * DK + c) : 0.f;
        // this element as row r of A and M (s <= r)
        float dkr = 0.f, dqr = 0.f, dgr = 0.f;
        for (int s = 0; s <= r; ++s) {
            const float ks = sK[s * DK + c] * expf(gr - sG[s * DK + c]);
            const float da = s < r ? sB[r] * sdT[r * 64 + s] : 0.f;
            const float dm = sM[r * 64 + s];
            dkr += da * ks;
            dqr += dm * ks;
            dgr += (da * kr + dm * qr) * ks;
        }
        // this element as column s = r of A and M (rows r2 >= s)
        float dks = 0.f, dgs = 0.f;
        for (int r2 = r; r2 < 64; ++r2) {
            const float E = expf(sG[r2 * DK + c] - gr);
            const float da = r2 > r ? sB[r2] * sdT[r2 * 64 + r] : 0.f;
            const float dm = sM[r2 * 64 + r];
            const float q2 = r2 < L ? ld(a.q + tok(r2) * DK + c) : 0.f;
            const float w = (da * sK[r2 * DK + c] + dm * q2) * E;
            dks += w;
            dgs -= w * kr;
        }
        gk[e] += dkr + dks;
        gq[e] += dqr;
        gG[e] += dgr + dgs;
    }
    __syncthreads();  // every read of sK, sG, sdT, sM is done
    // ---- 7. dla = reverse cumsum of dG (G_last is G_63); outputs
    for (int e = tid; e < 64 * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        sG[e] = gG[e] + (r == 63 ? sdGl[c] : 0.f);
        if (r < L) {
            a.dq[tok(r) * DK + c] = gq[e];
            a.dk[tok(r) * DK + c] = gk[e];
        }
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 63; r >= 0; --r) {
            acc += sG[r * DK + tid];
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
hipError_t launch_bwd_typed(const BackwardArgs& b, hipStream_t s, const BwdLayout& Lo) {
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
    {
        const int64_t blocks = static_cast<int64_t>(f.N) * f.H * (DV / 16);
        LaunchTimer timer("bwd_chain", s);
        hipLaunchKernelGGL((bwd_chain_kernel<DK, DV, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t slots = chunk_slots_bound(f.T, f.N);
    if (slots == 0 || f.T == 0) return hipSuccess;
    constexpr size_t lds = intra_lds_bytes<DK>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_intra_kernel<DK, DV, XT, GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("bwd_intra", s);
    hipLaunchKernelGGL((bwd_intra_kernel<DK, DV, XT, GT>), dim3(static_cast<unsigned>(slots), f.H), dim3(256), lds,
                       s, k);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_dims(const BackwardArgs& b, hipStream_t s, const BwdLayout& Lo) {
    if (b.f.x == DT::BF16) {
        return b.f.gate == DT::BF16 ? launch_bwd_typed<DK, DV, bf16, bf16>(b, s, Lo)
                                    : launch_bwd_typed<DK, DV, bf16, float>(b, s, Lo);
    }
    return b.f.gate == DT::BF16 ? launch_bwd_typed<DK, DV, float, bf16>(b, s, Lo)
                                : launch_bwd_typed<DK, DV, float, float>(b, s, Lo);
}

template <int DK>
hipError_t launch_bwd_dk(const BackwardArgs& b, hipStream_t s, const BwdLayout& Lo) {
    switch (b.f.dv) {
        case 16: return launch_bwd_dims<DK, 16>(b, s, Lo);
        case 32: return launch_bwd_dims<DK, 32>(b, s, Lo);
        case 64: return launch_bwd_dims<DK, 64>(b, s, Lo);
        case 128: return launch_bwd_dims<DK, 128>(b, s, Lo);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t backward_workspace_bytes(int64_t T, int N, int H, int dk, int dv) { return bwd_layout(T, N, H, dk, dv).total; }

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
    hipError_t e = launch_gen_forward(fa, s, base, reinterpret_cast<float*>(ws + Lo.rec));
    if (e != hipSuccess) return e;
    // 2. and 3.
    switch (f.dk) {
        case 16: return launch_bwd_dk<16>(b, s, Lo);
        case 32: return launch_bwd_dk<32>(b, s, Lo);
        case 64: return launch_bwd_dk<64>(b, s, Lo);
        case 128: return launch_bwd_dk<128>(b, s, Lo);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
