// Chunked prefill on the gfx950 matrix cores: dk = dv = 128, bf16 inputs,
// fp32 accumulation and fp32 state.  The chunk algebra (A, M, T, W, U~, Q',
// K^, gamma) is described in kda_prefill_common.h.
//
// Matrix-core instruction: v_mfma_f32_16x16x32_bf16.  With lane l = 16 g + c
// (g = 0..3, c = 0..15), the A operand (16 x 32) gives lane l the 8 values
// A[c][8g + e], the B operand (32 x 16) the values B[8g + e][c], and the
// 16 x 16 fp32 result leaves D[4g + i][c] (i = 0..3) in lane l.  Because the
// contraction index may be permuted freely as long as A and B agree, a
// result tile pair (rows 16m.. and 16m+16..) can feed the next product as its
// B operand straight from registers: slot e of lane group g stands for
// contraction index perm(g, e) = 4g + e (e < 4) or 16 + 4g + (e - 4)
// (e >= 4) inside a 32-wide step.  Matrices stored for the state pass are laid
// out so that this permuted A operand is one 16-byte load per lane.
//
// Phase 1 (mfma_intra_kernel): one 256-thread workgroup per (chunk, head).
//  - A and M tiles (16 x 16, rows in sub-block R, columns in sub-block S <= R)
//    use factored decays referenced to row b = 16R: left factor
//    e^{G_r - G_b} <= 1 and right factor e^{G_b - G_s}, which is <= 1 off the
//    diagonal.  On a diagonal sub-block the right factor grows with the decay
//    inside those 16 tokens; if any channel decays by more than e^-40 there,
//    that tile is computed exactly (pairwise e^{G_r - G_s}) on the vector ALUs.
//  - T = (I + Diag(beta) A)^-1 in fp32: diagonal 16 x 16 blocks by forward
//    substitution (one column per lane, in registers), off-diagonal blocks by
//    block substitution.
//  - W, U~, Q', M U~ on the matrix cores; outputs stored per (chunk, head).
// Phase 2 (mfma_state_kernel): one wave per (sequence, head, 16 state
//  columns); the 128 x 16 fp32 state lives in registers, the next chunk's
//  factors stream into a second LDS buffer (global_load_lds_dwordx4) while
//  the current chunk is computed.
#include "kda_prefill_common.h"
#include "kda_prefill_mfma.h"
#include "kda_profile.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// per (chunk slot, head) record, byte offsets
constexpr int R_NEGW = 0;       // -W, A-operand layout, [4 m][4 k][64 lanes][8]
constexpr int R_QP = 16384;     // Q', same layout
constexpr int R_KHT = 32768;    // K^T (dk rows x 64 tokens), [8 m][2 k][64 lanes][8]
constexpr int R_UT = 49152;     // U~, result layout per 16-column slice, [8 s][4 m][64 lanes][4]
constexpr int R_OI = 65536;     // M U~, same layout
constexpr int R_GAM = 81920;    // gamma, fp32 [128]
constexpr int REC_BYTES = 82432;

// intra-kernel LDS strides (padded rows avoid bank conflicts)
constexpr int KS = 136;  // bf16 per row of K, Q, V
constexpr int GS = 132;  // fp32 per row of G
constexpr float kDiagRange = 40.f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int perm(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

__device__ __forceinline__ float bfv(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(x[e]);
    return r;
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<__bf16>(lo[e]);
        r[4 + e] = static_cast<__bf16>(hi[e]);
    }
    return r;
}

template <typename GT>
struct MfmaK {
    int64_t T;
    int H, N;
    const int32_t* cu;
    const int32_t* base;
    const bf16 *q, *k, *v, *z;
    const GT *la, *beta;
    const float* S0;
    float* S_out;
    bf16* out;
    char* rec;
    int64_t groups;  // N * H
};

// ---------------------------------------------------------------------------
// phase 1
// ---------------------------------------------------------------------------

constexpr size_t kIntraLds = (3 * 64 * KS) * 2 + (64 * GS + 3 * 4096 + 64 + 8 * 128) * 4 + 16;

template <typename GT>
__global__ __launch_bounds__(256) void mfma_intra_kernel(MfmaK<GT> a) {
    extern __shared__ __align__(16) char smem[];
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem);
    uint16_t* sQ = sK + 64 * KS;
    uint16_t* sV = sQ + 64 * KS;
    float* sG = reinterpret_cast<float*>(sV + 64 * KS);
    float* sA = sG + 64 * GS;
    float* sM = sA + 4096;
    float* sT = sM + 4096;
    float* sB = sT + 4096;
    float* sTot = sB + 64;
    int* sFlag = reinterpret_cast<int*>(sTot + 8 * 128);
    // staging for the transposes, over buffers that are dead by then
    uint16_t* sStW = sV;                                  // [64][KS] bf16
    uint16_t* sStQ = reinterpret_cast<uint16_t*>(sA);     // [64][128] bf16

    const int slot = blockIdx.x, h = blockIdx.y;
    if (slot >= a.base[a.N]) return;
    const int n = find_seq(a.base, a.N, slot);
    const int64_t t0 = seq_begin(a.cu, n) + static_cast<int64_t>(slot - a.base[n]) * kChunk;
    const int L = static_cast<int>(min(static_cast<int64_t>(kChunk), seq_finish(a.cu, n, a.T) - t0));
    const int H = a.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    char* rec = a.rec + (static_cast<int64_t>(slot) * H + h) * REC_BYTES;

    // ---- load q, k, v (bf16 rows of 256 B) and the decay logs; zero past L
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        const int r = idx >> 4, ch = idx & 15;
        uint4 kk = make_uint4(0, 0, 0, 0), qq = kk, vv = kk;
        if (r < L) {
            const int64_t goff = ((t0 + r) * H + h) * 128 + ch * 8;
            kk = *reinterpret_cast<const uint4*>(a.k + goff);
            qq = *reinterpret_cast<const uint4*>(a.q + goff);
            vv = *reinterpret_cast<const uint4*>(a.v + goff);
        }
        *reinterpret_cast<uint4*>(sK + r * KS + ch * 8) = kk;
        *reinterpret_cast<uint4*>(sQ + r * KS + ch * 8) = qq;
        *reinterpret_cast<uint4*>(sV + r * KS + ch * 8) = vv;
    }
    const int cq = tid & 31, rg = tid >> 5;  // 4 channels x 8 rows per thread
    float x[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 8 * rg + j;
        if (r < L) {
            ld4(a.la + ((t0 + r) * H + h) * 128 + 4 * cq, x[j]);
        } else {
            x[j][0] = x[j][1] = x[j][2] = x[j][3] = 0.f;
        }
    }
    if (tid < 64) sB[tid] = tid < L ? ld(a.beta + (t0 + tid) * H + h) : 0.f;
    if (tid < 4) sFlag[tid] = 0;
    for (int i = tid; i < 2 * 4096 / 4; i += 256)
        reinterpret_cast<float4*>(sA)[i] = make_float4(0.f, 0.f, 0.f, 0.f);  // sA and sM
#pragma unroll
    for (int j = 1; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[j][e] += x[j - 1][e];
    *reinterpret_cast<float4*>(sTot + rg * 128 + 4 * cq) = make_float4(x[7][0], x[7][1], x[7][2], x[7][3]);
    __syncthreads();
    {
        float off[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q2 = 0; q2 < rg; ++q2) {
            const float4 t4 = *reinterpret_cast<const float4*>(sTot + q2 * 128 + 4 * cq);
            off[0] += t4.x; off[1] += t4.y; off[2] += t4.z; off[3] += t4.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<float4*>(sG + (8 * rg + j) * GS + 4 * cq) =
                make_float4(x[j][0] + off[0], x[j][1] + off[1], x[j][2] + off[2], x[j][3] + off[3]);
    }
    __syncthreads();
    // sub-blocks whose decay inside 16 tokens is too steep for the factored form
    if (tid < 128) {
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            const float d = sG[(16 * R) * GS + tid] - sG[(16 * R + 15) * GS + tid];
            if (d > kDiagRange) sFlag[R] = 1;  // benign race: all writers store 1
        }
    }
    __syncthreads();

    // ---- A and M: 10 tiles (R >= S), spread over the 4 waves
    {
        // tiles (R, S) per wave, one byte each (R in the high nibble), 0xFF = none
        const uint32_t code = wave == 0 ? 0xFF3000u : wave == 1 ? 0x311110u : wave == 2 ? 0x322120u : 0xFF3322u;
#pragma unroll
        for (int ti = 0; ti < 3; ++ti) {
            const uint32_t tile = (code >> (8 * ti)) & 0xFFu;
            if (tile == 0xFFu) continue;
            const int R = static_cast<int>(tile >> 4), S = static_cast<int>(tile & 15u);
            const int b = 16 * R;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = accA;
            if (R == S && sFlag[R]) {
                // exact pairwise decays
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = b + 4 * g + i, s = 16 * S + c;
                    float av = 0.f, mv = 0.f;
                    if (s <= r) {
                        for (int ch = 0; ch < 128; ++ch) {
                            const float ks = bfv(sK + s * KS + ch) * expf(sG[r * GS + ch] - sG[s * GS + ch]);
                            av += bfv(sK + r * KS + ch) * ks;
                            mv += bfv(sQ + r * KS + ch) * ks;
                        }
                    }
                    accA[i] = av;
                    accM[i] = mv;
                }
            } else {
                const int rl = b + c, sr = 16 * S + c;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    float kl[8], ql[8], kr[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int ch = 32 * ks + 8 * g + e;
                        const float gb = sG[b * GS + ch];
                        const float el = expf(sG[rl * GS + ch] - gb);
                        kl[e] = bfv(sK + rl * KS + ch) * el;
                        ql[e] = bfv(sQ + rl * KS + ch) * el;
                        kr[e] = bfv(sK + sr * KS + ch) * expf(gb - sG[sr * GS + ch]);
                    }
                    const bf16x8 bk = to_bf16x8(kr);
                    accA = mfma(to_bf16x8(kl), bk, accA);
                    accM = mfma(to_bf16x8(ql), bk, accM);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = b + 4 * g + i, s = 16 * S + c;
                sA[r * 64 + s] = s < r ? accA[i] : 0.f;
                sM[r * 64 + s] = s <= r ? accM[i] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- T = (I + Diag(beta) A)^-1
    // diagonal blocks: wave R, lane j < 16 owns column j of T_RR
    {
        const int R = wave, j = lane;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float sum = 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) sum += sA[(16 * R + r) * 64 + 16 * R + s] * t[s];
            t[r] = (r == j ? 1.f : 0.f) - sB[16 * R + r] * sum;
        }
        if (j < 16) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * R + r) * 64 + 16 * R + j] = t[r];
        }
    }
    __syncthreads();
    // off-diagonal blocks by distance d = R - S:
    //   Y = Diag(beta_R) sum_{J=S}^{R-1} A_RJ T_JS ;  T_RS = -T_RR Y
    float* sY = sTot;  // 4 x 256 floats of scratch (the cumsum totals are dead)
    for (int d = 1; d <= 3; ++d) {
        const int S = wave, R = wave + d;
        const bool active = R <= 3;
        if (active) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                float acc = 0.f;
                for (int J = S; J < R; ++J)
#pragma unroll
                    for (int kk = 0; kk < 16; ++kk)
                        acc += sA[(16 * R + r) * 64 + 16 * J + kk] * sT[(16 * J + kk) * 64 + 16 * S + c];
                sY[wave * 256 + r * 16 + c] = sB[16 * R + r] * acc;
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    acc += sT[(16 * R + r) * 64 + 16 * R + kk] * sY[wave * 256 + kk * 16 + c];
                sT[(16 * R + r) * 64 + 16 * S + c] = -acc;
            }
        }
        __syncthreads();
    }
    // upper blocks of T stay unused: every product below skips them

    // ---- W = T (beta e^G K) and U~ = T (beta V): this wave's column tiles
    f32x4 accW[2][4], accU[2][4];
    {
        bf16x8 Ta[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float tv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = 32 * ks + 8 * g + e;
                    tv[e] = col <= 16 * mt + c ? sT[(16 * mt + c) * 64 + col] : 0.f;
                }
                Ta[mt][ks] = to_bf16x8(tv);
            }
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int nt = 2 * wave + q2;
            const int ch = 16 * nt + c;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                accW[q2][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                accU[q2][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float bk[8], bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * ks + 8 * g + e;
                    const float be = sB[s];
                    bk[e] = be * expf(sG[s * GS + ch]) * bfv(sK + s * KS + ch);
                    bv[e] = be * bfv(sV + s * KS + ch);
                }
                const bf16x8 Bk = to_bf16x8(bk), Bv = to_bf16x8(bv);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (32 * ks > 16 * mt + 15) continue;  // T is lower triangular
                    accW[q2][mt] = mfma(Ta[mt][ks], Bk, accW[q2][mt]);
                    accU[q2][mt] = mfma(Ta[mt][ks], Bv, accU[q2][mt]);
                }
            }
            // U~ in result layout, per 16-column slice nt
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                uint2 p;
                p.x = pack_bf16x2(accU[q2][mt][0], accU[q2][mt][1]);
                p.y = pack_bf16x2(accU[q2][mt][2], accU[q2][mt][3]);
                *reinterpret_cast<uint2*>(rec + R_UT + ((nt * 4 + mt) * 64 + lane) * 8) = p;
            }
        }
    }
    __syncthreads();  // V is dead: its buffer becomes the staging area of W

    // ---- Q' = e^G Q - M W and M U~; stage W and Q' for the transposes
    {
        bf16x8 Mneg[4][2], Mpos[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float mv[8], mn[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = 32 * ks + perm(g, e);
                    mv[e] = sM[(16 * mt + c) * 64 + col];
                    mn[e] = -mv[e];
                }
                Mpos[mt][ks] = to_bf16x8(mv);
                Mneg[mt][ks] = to_bf16x8(mn);
            }
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int nt = 2 * wave + q2;
            const int ch = 16 * nt + c;
            bf16x8 Bw[2], Bu[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                Bw[ks] = to_bf16x8(accW[q2][2 * ks], accW[q2][2 * ks + 1]);
                Bu[ks] = to_bf16x8(accU[q2][2 * ks], accU[q2][2 * ks + 1]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 qp, oi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g + i;
                    qp[i] = expf(sG[r * GS + ch]) * bfv(sQ + r * KS + ch);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (32 * ks > 16 * mt + 15) continue;  // M is lower triangular
                    qp = mfma(Mneg[mt][ks], Bw[ks], qp);
                    oi = mfma(Mpos[mt][ks], Bu[ks], oi);
                }
                uint2 p;
                p.x = pack_bf16x2(oi[0], oi[1]);
                p.y = pack_bf16x2(oi[2], oi[3]);
                *reinterpret_cast<uint2*>(rec + R_OI + ((nt * 4 + mt) * 64 + lane) * 8) = p;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g + i;
                    sStW[r * KS + ch] = f32_to_bf16(-accW[q2][mt][i]);
                    sStQ[r * 128 + ch] = f32_to_bf16(qp[i]);
                }
            }
        }
    }
    __syncthreads();

    // ---- stores in the A-operand layout: -W, Q' (4 blocks per wave each), K^T
    {
        const int mt = wave;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int r = 16 * mt + c;
            const int c0 = 32 * ks + 4 * g;
            uint4 w4, q4;
            const uint2 wlo = *reinterpret_cast<const uint2*>(sStW + r * KS + c0);
            const uint2 whi = *reinterpret_cast<const uint2*>(sStW + r * KS + c0 + 16);
            const uint2 qlo = *reinterpret_cast<const uint2*>(sStQ + r * 128 + c0);
            const uint2 qhi = *reinterpret_cast<const uint2*>(sStQ + r * 128 + c0 + 16);
            w4 = make_uint4(wlo.x, wlo.y, whi.x, whi.y);
            q4 = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
            const int blk = (mt * 4 + ks) * 64 + lane;
            *reinterpret_cast<uint4*>(rec + R_NEGW + blk * 16) = w4;
            *reinterpret_cast<uint4*>(rec + R_QP + blk * 16) = q4;
        }
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int t = 2 * wave + q2;
            const int ch = 16 * t + c;
            const float glast = sG[63 * GS + ch];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float kv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * ks + perm(g, e);
                    kv[e] = expf(glast - sG[s * GS + ch]) * bfv(sK + s * KS + ch);
                }
                uint4 p;
                p.x = pack_bf16x2(kv[0], kv[1]);
                p.y = pack_bf16x2(kv[2], kv[3]);
                p.z = pack_bf16x2(kv[4], kv[5]);
                p.w = pack_bf16x2(kv[6], kv[7]);
                *reinterpret_cast<uint4*>(rec + R_KHT + ((t * 2 + ks) * 64 + lane) * 16) = p;
            }
        }
        if (tid < 128) reinterpret_cast<float*>(rec + R_GAM)[tid] = expf(sG[63 * GS + tid]);
    }
}

// ---------------------------------------------------------------------------
// phase 2
// ---------------------------------------------------------------------------

// LDS image of one chunk for one 16-column slice
constexpr int B_NEGW = 0;
constexpr int B_QP = 16384;
constexpr int B_KHT = 32768;
constexpr int B_UT = 49152;   // 2 KB: this slice's U~
constexpr int B_OI = 51200;   // 2 KB: this slice's M U~
constexpr int B_GAM = 53248;  // 512 B
constexpr int B_BYTES = 53760;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lds_copy16(const char* gsrc, char* lds_dst) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(gsrc), (lds_void*)(lds_dst), 16, 0, 0);
}

// issue the asynchronous copy of chunk record `r` (slice sl) into LDS buffer `buf`
__device__ __forceinline__ void prefetch_chunk(const char* r, char* buf, int sl, int lane) {
#pragma unroll
    for (int b = 0; b < 48; ++b) lds_copy16(r + b * 1024 + lane * 16, buf + b * 1024);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        lds_copy16(r + R_UT + sl * 2048 + b * 1024 + lane * 16, buf + B_UT + b * 1024);
        lds_copy16(r + R_OI + sl * 2048 + b * 1024 + lane * 16, buf + B_OI + b * 1024);
    }
    if (lane < 32) lds_copy16(r + R_GAM + lane * 16, buf + B_GAM);
}

template <typename GT>
__global__ __launch_bounds__(64) void mfma_state_kernel(MfmaK<GT> a) {
    extern __shared__ __align__(16) char smem[];
    // blockIdx -> (sequence, head, slice): the 8 slices of one (sequence, head)
    // share an XCD (workgroups are dealt round-robin over the 8 XCDs), so the
    // records they all read are cached in one L2
    const int bid = blockIdx.x;
    const int xcd = bid & 7, sl = (bid >> 3) & 7;
    const int64_t grp = static_cast<int64_t>(bid >> 6) * 8 + xcd;
    if (grp >= a.groups) return;
    const int H = a.H;
    const int n = static_cast<int>(grp / H), h = static_cast<int>(grp % H);
    const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
    const int col = 16 * sl + c;

    // state S[16t + 4g + i][col] in registers
    f32x4 S[8];
    const int64_t sidx = grp * (128 * 128);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] = a.S0 ? a.S0[sidx + (16 * t + 4 * g + i) * 128 + col] : 0.f;

    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    const int slot0 = a.base[n];
    const int nch = a.base[n + 1] - slot0;
    auto rec_of = [&](int j) { return a.rec + (static_cast<int64_t>(slot0 + j) * H + h) * REC_BYTES; };

    float zn[16];  // output-gate logits of the chunk being prefetched
    auto load_z = [&](int j) {
        const int64_t tc = sb + static_cast<int64_t>(j) * kChunk;
        const int Lc = static_cast<int>(min(static_cast<int64_t>(kChunk), se - tc));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g + i;
                zn[mt * 4 + i] = (a.z != nullptr && r < Lc) ? ld(a.z + ((tc + r) * H + h) * 128 + col) : 0.f;
            }
    };
    if (nch > 0) {
        prefetch_chunk(rec_of(0), smem, sl, lane);
        load_z(0);
    }
    for (int j = 0; j < nch; ++j) {
        __builtin_amdgcn_s_waitcnt(0);  // chunk j has landed in LDS (and its z in registers)
        __builtin_amdgcn_sched_barrier(0);
        char* buf = smem + (j & 1) * B_BYTES;
        float zc[16];
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2) zc[q2] = zn[q2];
        if (j + 1 < nch) {
            prefetch_chunk(rec_of(j + 1), smem + ((j + 1) & 1) * B_BYTES, sl, lane);
            load_z(j + 1);
        }
        const int64_t tc = sb + static_cast<int64_t>(j) * kChunk;
        const int Lc = static_cast<int>(min(static_cast<int64_t>(kChunk), se - tc));

        bf16x8 Sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Sb[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);

        // U = U~ - W S  and  O = M U~ + Q' S
        f32x4 U[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint2 up = *reinterpret_cast<const uint2*>(buf + B_UT + (mt * 64 + lane) * 8);
            const uint2 op = *reinterpret_cast<const uint2*>(buf + B_OI + (mt * 64 + lane) * 8);
            f32x4 u = {__uint_as_float(up.x << 16), __uint_as_float(up.x & 0xffff0000u),
                       __uint_as_float(up.y << 16), __uint_as_float(up.y & 0xffff0000u)};
            f32x4 o = {__uint_as_float(op.x << 16), __uint_as_float(op.x & 0xffff0000u),
                       __uint_as_float(op.y << 16), __uint_as_float(op.y & 0xffff0000u)};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int blk = (mt * 4 + ks) * 64 + lane;
                const bf16x8 wa = *reinterpret_cast<const bf16x8*>(buf + B_NEGW + blk * 16);
                const bf16x8 qa = *reinterpret_cast<const bf16x8*>(buf + B_QP + blk * 16);
                u = mfma(wa, Sb[ks], u);
                o = mfma(qa, Sb[ks], o);
            }
            U[mt] = u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g + i;
                if (r < Lc) {
                    float y = o[i];
                    if (a.z != nullptr) y *= sigmoid(zc[mt * 4 + i]);
                    a.out[((tc + r) * H + h) * 128 + col].bits = f32_to_bf16(y);
                }
            }
        }
        // S <- Diag(gamma) S + K^T U
        bf16x8 Ub[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) Ub[ks] = to_bf16x8(U[2 * ks], U[2 * ks + 1]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float4 gm = *reinterpret_cast<const float4*>(buf + B_GAM + (16 * t + 4 * g) * 4);
            S[t][0] *= gm.x;
            S[t][1] *= gm.y;
            S[t][2] *= gm.z;
            S[t][3] *= gm.w;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + B_KHT + ((t * 2 + ks) * 64 + lane) * 16);
                S[t] = mfma(ka, Ub[ks], S[t]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (a.S_out) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.S_out[sidx + (16 * t + 4 * g + i) * 128 + col] = S[t][i];
    }
}

template <typename GT>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t s, int32_t* base, char* recs) {
    MfmaK<GT> k;
    k.T = a.T; k.H = a.H; k.N = a.N; k.cu = a.cu; k.base = base;
    k.q = static_cast<const bf16*>(a.q); k.k = static_cast<const bf16*>(a.k);
    k.v = static_cast<const bf16*>(a.v); k.z = static_cast<const bf16*>(a.z);
    k.la = static_cast<const GT*>(a.la); k.beta = static_cast<const GT*>(a.beta);
    k.S0 = a.S0; k.S_out = a.S_out; k.out = static_cast<bf16*>(a.out); k.rec = recs;
    k.groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t slots = chunk_slots_bound(a.T, a.N);
    if (a.T > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_intra_kernel<GT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(kIntraLds));
        if (e != hipSuccess) return e;
        LaunchTimer timer("mfma_intra", s);
        hipLaunchKernelGGL((mfma_intra_kernel<GT>), dim3(static_cast<unsigned>(slots), a.H), dim3(256),
                           kIntraLds, s, k);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_state_kernel<GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * B_BYTES);
    if (e != hipSuccess) return e;
    const int64_t blocks = (k.groups + 7) / 8 * 64;
    LaunchTimer timer("mfma_state", s);
    hipLaunchKernelGGL((mfma_state_kernel<GT>), dim3(static_cast<unsigned>(blocks)), dim3(64), 2 * B_BYTES, s, k);
    return hipGetLastError();
}

}  // namespace

bool mfma_prefill_supports(int dk, int dv, DT x) { return dk == 128 && dv == 128 && x == DT::BF16; }

size_t mfma_record_bytes() { return REC_BYTES; }

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s, int32_t* base, char* recs) {
    return a.gate == DT::BF16 ? launch_typed<bf16>(a, s, base, recs) : launch_typed<float>(a, s, base, recs);
}

}  // namespace kda
