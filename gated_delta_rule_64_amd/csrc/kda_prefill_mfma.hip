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
// Phase 1 (mfma_intra_kernel): a persistent grid, one 512-thread workgroup
// per CU, walking the (head, chunk) units; each unit's inputs are loaded into
// registers during the previous unit.
//  - A and M tiles (16 x 16, rows in sub-block R, columns in sub-block S <= R)
//    use factored decays referenced to row b = 16R: left factor
//    e^{G_r - G_b} <= 1 and right factor e^{G_b - G_s}, which is <= 1 off the
//    diagonal.  On a diagonal sub-block the right factor grows with the decay
//    inside those 16 tokens; if any channel decays by more than e^-40 there,
//    that tile is computed exactly (pairwise e^{G_r - G_s}) on the vector ALUs.
//  - T = (I + Diag(beta) A)^-1 in fp32: diagonal 16 x 16 blocks by forward
//    substitution (one column per lane, in registers), off-diagonal blocks
//    from the inverses of the two 32 x 32 halves.
//  - W, U~, Q', M U~ on the matrix cores; outputs stored per (head, chunk).
// Phase 2 (mfma_state_kernel): per (sequence, head, group of state
//  columns), compute waves carry the fp32 state in registers through the
//  chunks in order while copy waves stream each chunk's factors into LDS.
#include <stdlib.h>

#include "kda_prefill_common.h"
#include "kda_prefill_mfma.h"
#include "kda_profile.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Record stores: non-temporal (streamed past the caches; measured faster for
// both the writer and the state pass that reads the records back).
__device__ __forceinline__ void rec_store8(char* p, uint2 v) {
    __builtin_nontemporal_store(u32x2v{v.x, v.y}, reinterpret_cast<u32x2v*>(p));
}
__device__ __forceinline__ void rec_store16(char* p, uint4 v) {
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(p));
}

// per (chunk slot, head) record, byte offsets
constexpr int R_NEGW = 0;       // -W, A-operand layout, [4 m][4 k][64 lanes][8]
constexpr int R_QP = 16384;     // Q', same layout
constexpr int R_KHT = 32768;    // K^T (dk rows x 64 tokens), [8 m][2 k][64 lanes][8]
constexpr int R_UT = 49152;     // U~, result layout per 16-column slice, [8 s][4 m][64 lanes][4]
constexpr int R_OI = 65536;     // M U~, transposed result layout: lane (g, c) holds [16m + c][16s + 4g + i]
constexpr int R_GAM = 81920;    // gamma, fp32 [128]
constexpr int REC_BYTES = 82432;

// intra-kernel LDS strides (padded rows avoid bank conflicts)
constexpr int KS = 136;  // bf16 per row of K, Q, V
constexpr int GS = 132;  // fp32 per row of G
constexpr int MS = 68;   // fp32 per row of A, M and T (16 lanes reading 16 rows hit distinct banks)
constexpr int SQS = 136; // bf16 per row of the Q' staging tile (the same bytes per row as A)
constexpr float kDiagRange = 40.f * kLog2e;  // e^40, in the log2 units G is kept in

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
    const SlotInfo* slot_info;  // first token and length of each chunk slot
    const bf16 *q, *k, *v, *z;
    const GT *la, *beta;
    const float* S0;
    float* S_out;
    bf16* out;
    char* rec;
    // fused path only: q, k, v, la and beta above hold the raw inputs (q_in,
    // k_in, v_in, decay logits g, write logits b), and these the conv taps
    // and the optional conv history
    const bf16 *w_q, *w_k, *w_v;
    const float* cs;
    int64_t slots;   // chunk slots per head in the record array
    int64_t groups;  // N * H
    bool inline_map;  // no chunk map: the kernels derive each slot from cu (N <= 64)
    Snapshots snap;  // optional states after every snap.chunks full chunks
};

// ---------------------------------------------------------------------------
// phase 1
// ---------------------------------------------------------------------------

constexpr int kIntraThreads = 512;  // 8 waves: two per SIMD
constexpr size_t kIntraLds = (3 * 64 * KS) * 2 + (64 * GS + 3 * 64 * MS + 64 + 16 * 128) * 4 + 16;

__device__ __forceinline__ void unpack8(uint4 v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ void lds8f(const float* p, float (&x)[8]) {
    const float4 u = reinterpret_cast<const float4*>(p)[0];
    const float4 v = reinterpret_cast<const float4*>(p)[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

// One int32 through the scalar cache, for addresses that are uniform across
// the wave.  The wait sits in the same asm block, so the result register is
// never read before the load has returned.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
    int32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// 16 bytes (16-byte aligned) through the scalar cache, as scalar_load
__device__ __forceinline__ i32x4 scalar_load4(const int32_t* p) {
    i32x4 v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

// Chunk slots without the chunk map, for at most 64 sequences: lane i of the
// wave gets the number of chunks in sequences 0 .. i (an inclusive scan over
// the lanes; lanes past the last sequence hold the total).  Every lane of the
// wave must be active.
__device__ __forceinline__ int chunk_prefix_lane(const int32_t* cu, int N, int64_t T) {
    const int lane = threadIdx.x & 63;
    int c = 0;
    if (lane < N) c = static_cast<int>((seq_finish(cu, lane, T) - seq_begin(cu, lane) + kChunk - 1) / kChunk);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(c, off);
        if (lane >= off) c += y;
    }
    return c;
}
// With that prefix (uniform results): the sequence that holds a slot (the
// number of sequences that end at or before it), and the slots before
// sequence n.
__device__ __forceinline__ int seq_of_slot(int incl, int64_t slot) {
    return static_cast<int>(__popcll(__ballot(incl <= slot)));
}
__device__ __forceinline__ int slots_before(int incl, int n) {
    return n > 0 ? __builtin_amdgcn_readlane(incl, n - 1) : 0;
}
// A uniform sequence boundary, through the scalar cache.
__device__ __forceinline__ int64_t seq_bound(const int32_t* cu, int n, int64_t T, bool finish) {
    if (cu == nullptr) return finish ? T : 0;
    return scalar_load(cu + n + (finish ? 1 : 0));
}

// Four consecutive gate values of one row, kept as loaded until used.
template <typename GT> struct GateRaw;
template <> struct GateRaw<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};
template <> struct GateRaw<bf16> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = e < 2 ? v.x : v.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k + 15), all lanes
// active: swaps within quads (quad_perm [1,0,3,2], [2,3,0,1]), then the
// half-row and row mirrors pair the quads and the halves.  Vector ALU only.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// (R, S) of tile i in the lower block triangle, row-major order
__device__ __forceinline__ void tile_rs(int i, int& R, int& S) {
    R = i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0;
    S = i - R * (R + 1) / 2;
}

// kFused: the unit's inputs are the raw layer inputs, and staging them
// applies the short conv, the L2 norm and the gates first (as kda_preprocess
// does, in the same fp32 arithmetic), so the preprocessed tensors never go
// through HBM.
template <typename GT, bool kFused>
__global__ __launch_bounds__(kIntraThreads) void mfma_intra_kernel(MfmaK<GT> a) {
    extern __shared__ __align__(16) char smem[];
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem);   // [64][KS] keys (bf16)
    uint16_t* sQ = sK + 64 * KS;                        // [64][KS] queries
    uint16_t* sV = sQ + 64 * KS;                        // [64][KS] values
    float* sG = reinterpret_cast<float*>(sV + 64 * KS);  // [64][GS] decay cumsums G, in log2 units (G / ln 2)
    float* sA = sG + 64 * GS;                           // [64][MS]
    float* sM = sA + 64 * MS;                           // [64][MS]
    float* sT = sM + 64 * MS;                           // [64][MS]
    float* sB = sT + 64 * MS;                           // [64] beta
    float* sTot = sB + 64;                              // [16][128] scan partials, later scratch
    int* sFlag = reinterpret_cast<int*>(sTot + 16 * 128);
    uint16_t* sStW = sV;                                // staging of -W  [64][KS]
    uint16_t* sStQ = reinterpret_cast<uint16_t*>(sA);   // staging of Q'  [64][SQS]

    const int H = a.H;
    const int ftid = threadIdx.x;  // the thread index as the prefetch uses it
    // Units are (head, chunk slot) pairs, head-major; the grid is persistent
    // (one workgroup per CU) and walks them with stride gridDim.x.
    const int incl = a.inline_map ? chunk_prefix_lane(a.cu, a.N, a.T) : 0;
    const int nslots = a.inline_map ? (a.N > 0 ? __builtin_amdgcn_readlane(incl, a.N - 1) : 0)
                                    : scalar_load(a.base + a.N);
    const int64_t units = static_cast<int64_t>(H) * nslots;
    struct Unit {
        int h, L, n;
        bool first;  // the sequence's first chunk (its conv history is the caller's)
        int64_t slot, t0;
    };
    // The unit's head, slot, first token and length.  The lookups are
    // uniform, so they go through the scalar cache (a vector load here would
    // also wait for the previous unit's record stores).
    auto unit_of = [&](int64_t v) {
        Unit u;
        // unit indices fit 32 bits (the launcher checks the bound)
        const uint32_t v32 = static_cast<uint32_t>(v), ns = static_cast<uint32_t>(nslots);
        u.h = static_cast<int>(v32 / ns);
        u.slot = v32 % ns;
        if (a.inline_map) {
            u.n = seq_of_slot(incl, u.slot);
            const int s0 = slots_before(incl, u.n);
            u.first = u.slot == s0;
            u.t0 = seq_bound(a.cu, u.n, a.T, false) + (u.slot - s0) * kChunk;
            u.L = static_cast<int>(min(static_cast<int64_t>(kChunk), seq_bound(a.cu, u.n, a.T, true) - u.t0));
            return u;
        }
        const i32x4 si = scalar_load4(reinterpret_cast<const int32_t*>(a.slot_info + u.slot));
        u.t0 = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(si[1])) << 32) |
                                    static_cast<uint32_t>(si[0]));
        u.L = si[2] & 0xffff;
        u.first = (si[2] >> 16) != 0;
        u.n = si[3];
        return u;
    };
    // This thread's share of a unit's inputs, loaded one unit ahead into
    // registers so the loads overlap the previous unit's work: rows
    // (tid + 512 i) / 16 of q, k, v (8 channels each), rows 4 rg .. 4 rg + 3 of
    // the decay logs (4 channels), and beta of row tid % 64.  Loads are
    // branch-free: rows past the chunk end read row L-1 and are zeroed on use.
    const int fcq = ftid & 31, frg = ftid >> 5;
    const int fw = __builtin_amdgcn_readfirstlane(ftid >> 6);  // the wave, as a uniform value
    uint4 pk[2], pq[2], pv[2];
    GateRaw<GT> px[4];  // decay logs (fused: decay logits) as loaded; converted when staged
    GT pb{};
    // fused path: conv taps of 2 channels and one 8-channel piece of the
    // 3-token conv history of tensor (wave mod 3), as loaded (bf16 bits, or
    // fp32 from the caller's history)
    uint4 pw = make_uint4(0, 0, 0, 0);
    uint32_t ph[8];
    // part p of a unit's loads: 0 keys, 1 queries, 2 values, 3 decay logs and beta
    auto fetch = [&](const Unit& u, int p) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = ftid + kIntraThreads * i;
            const int r = idx >> 4, ch = idx & 15;
            const int64_t goff = ((u.t0 + min(r, u.L - 1)) * H + u.h) * 128 + ch * 8;
            if (p == 0) pk[i] = *reinterpret_cast<const uint4*>(a.k + goff);
            if (p == 1) pq[i] = *reinterpret_cast<const uint4*>(a.q + goff);
            if (p == 2) pv[i] = *reinterpret_cast<const uint4*>(a.v + goff);
        }
        if (p == 3) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                px[j].load(a.la + ((u.t0 + min(4 * frg + j, u.L - 1)) * H + u.h) * 128 + 4 * fcq);
            // The last loads cover less than 512 threads' worth; every wave
            // issues them anyway, repeating another wave's (and later writes
            // the same bytes to the same LDS place).  Loads and their uses
            // under conditions that skip whole waves would leave the compiler
            // a path on which these registers still await their loads when
            // the next unit's fetch reuses them, and it would wait there.
            // The tensor a wave covers is uniform (fw is read from lane 0),
            // so choosing its pointer is a scalar select.
            pb = a.beta[(u.t0 + min(ftid & 63, u.L - 1)) * H + u.h];
            if (kFused) {
                const int tt = fw % 3;
                {  // tensor tt (q, k, v), channels 2 (tid % 64) .. + 1
                    const bf16* w = tt == 0 ? a.w_q : (tt == 1 ? a.w_k : a.w_v);
                    pw = *reinterpret_cast<const uint4*>(w + (u.h * 128 + 2 * (ftid & 63)) * 4);
                }
                {  // tensor tt, history token hr, channels 8 chh .. + 7
                    // Two 16-byte loads every time, from addresses chosen by
                    // uniform values (no branches: a load in one arm of a
                    // branch is copied out at the merge, which waits for it).
                    // Not the first chunk: the raw row t0 - 3 + hr (bf16, first
                    // load).  First chunk with a caller history: its 8 fp32
                    // values.  First chunk without: row t0, read and unused.
                    const int hr = min((ftid & 63) >> 4, 2), chh = ftid & 15;  // lanes 48.. repeat token 2
                    const bf16* x = tt == 0 ? a.q : (tt == 1 ? a.k : a.v);
                    const int64_t row = u.first ? u.t0 : u.t0 - 3 + hr;
                    const char* src = reinterpret_cast<const char*>(x + (row * H + u.h) * 128 + 8 * chh);
                    int step = 0;
                    if (u.first && a.cs != nullptr) {
                        const int64_t width = static_cast<int64_t>(H) * 384;  // q, k, v channels of all heads
                        src = reinterpret_cast<const char*>(a.cs + (static_cast<int64_t>(u.n) * 3 + hr) * width +
                                                            static_cast<int64_t>(tt) * H * 128 + u.h * 128 + 8 * chh);
                        step = 16;
                    }
                    const uint4 lo = *reinterpret_cast<const uint4*>(src);
                    const uint4 hi = *reinterpret_cast<const uint4*>(src + step);
                    ph[0] = lo.x; ph[1] = lo.y; ph[2] = lo.z; ph[3] = lo.w;
                    ph[4] = hi.x; ph[5] = hi.y; ph[6] = hi.z; ph[7] = hi.w;
                }
            }
        }
    };
    auto fetch_all = [&](const Unit& u) {
#pragma unroll
        for (int p = 0; p < 4; ++p) fetch(u, p);
    };

    // A unit's prefetched inputs into LDS (padded rows are zero: no decay, no
    // write), the first level of the decay scan, and cleared A, M and flags.
    // Runs once the LDS buffers are free.
    auto stage_inputs = [&](const Unit& u, int tid) {
        const int cq = tid & 31, rg = tid >> 5;
        const int L = u.L;
        if (!kFused) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int idx = tid + kIntraThreads * i;
                const int r = idx >> 4, ch = idx & 15;
                const uint32_t m = r < L ? 0xffffffffu : 0u;  // masks, not selects: the arrays stay in registers
                *reinterpret_cast<uint4*>(sK + r * KS + ch * 8) =
                    make_uint4(pk[i].x & m, pk[i].y & m, pk[i].z & m, pk[i].w & m);
                *reinterpret_cast<uint4*>(sQ + r * KS + ch * 8) =
                    make_uint4(pq[i].x & m, pq[i].y & m, pq[i].z & m, pq[i].w & m);
                *reinterpret_cast<uint4*>(sV + r * KS + ch * 8) =
                    make_uint4(pv[i].x & m, pv[i].y & m, pv[i].z & m, pv[i].w & m);
            }
        } else {
            // Raw rows (bf16, [64][KS] per tensor), the 3-token history (fp32
            // [3][128] per tensor) and the conv taps (fp32 [3 tensors][4 taps][128]) go to
            // buffers that are free until the gates are staged.
            uint16_t* raw = reinterpret_cast<uint16_t*>(sG);
            float* hist = reinterpret_cast<float*>(raw + 3 * 64 * KS);
            float* taps = sTot;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int idx = tid + kIntraThreads * i;
                const int r = idx >> 4, ch = idx & 15;
                const uint32_t m = r < L ? 0xffffffffu : 0u;
                *reinterpret_cast<uint4*>(raw + r * KS + ch * 8) =
                    make_uint4(pq[i].x & m, pq[i].y & m, pq[i].z & m, pq[i].w & m);
                *reinterpret_cast<uint4*>(raw + 64 * KS + r * KS + ch * 8) =
                    make_uint4(pk[i].x & m, pk[i].y & m, pk[i].z & m, pk[i].w & m);
                *reinterpret_cast<uint4*>(raw + 2 * 64 * KS + r * KS + ch * 8) =
                    make_uint4(pv[i].x & m, pv[i].y & m, pv[i].z & m, pv[i].w & m);
            }
            const int tw = __builtin_amdgcn_readfirstlane(tid >> 6) % 3;  // the tensor this wave fetched
            {
                const int tt = tw, hr = min((tid & 63) >> 4, 2), chh = tid & 15;
                // the history as fetched for this unit (see fetch): raw bf16
                // rows, the caller's fp32 values, or zeros.  Every path
                // reads all eight registers (the raw rows fill four), so none
                // is left awaiting its load when the next fetch reuses it.
                asm volatile("" ::"v"(ph[4]), "v"(ph[5]), "v"(ph[6]), "v"(ph[7]));
                float hv[8];
                if (!u.first) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hv[2 * e] = __uint_as_float(ph[e] << 16);
                        hv[2 * e + 1] = __uint_as_float(ph[e] & 0xffff0000u);
                    }
                } else {
                    const uint32_t m = a.cs != nullptr ? 0xffffffffu : 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) hv[e] = __uint_as_float(ph[e] & m);
                }
                float4* d = reinterpret_cast<float4*>(hist + (tt * 3 + hr) * 128 + 8 * chh);
                d[0] = make_float4(hv[0], hv[1], hv[2], hv[3]);
                d[1] = make_float4(hv[4], hv[5], hv[6], hv[7]);
            }
            {  // taps as [tensor][tap][channel]: a lane's 8 channels of one tap are contiguous
                const uint32_t w4[4] = {pw.x, pw.y, pw.z, pw.w};
                float* d = taps + tw * 512 + 2 * (tid & 63);
#pragma unroll
                for (int e = 0; e < 2; ++e) {  // channel 2 (tid % 64) + e, taps 0..3
                    d[0 * 128 + e] = __uint_as_float(w4[2 * e] << 16);
                    d[1 * 128 + e] = __uint_as_float(w4[2 * e] & 0xffff0000u);
                    d[2 * 128 + e] = __uint_as_float(w4[2 * e + 1] << 16);
                    d[3 * 128 + e] = __uint_as_float(w4[2 * e + 1] & 0xffff0000u);
                }
            }
            lds_barrier();
            // conv (tap 3 is the current token) of the thread's two consecutive
            // rows 2k, 2k+1 of each tensor, from the five raw rows 2k-3 .. 2k+1
            // (the first ones reach into the history), all reads of a tensor
            // issued before the arithmetic that needs them; then the L2 norm
            // of q and k over the 128 channels a 16-lane group holds
            const int ch8 = 8 * (tid & 15), r0 = 2 * (tid >> 4);
#pragma unroll
            for (int tt = 0; tt < 3; ++tt) {
                float w[4][8];
#pragma unroll
                for (int j = 0; j < 4; ++j) lds8f(taps + tt * 512 + j * 128 + ch8, w[j]);
                float xv[5][8];
                if (r0 >= 4) {  // every tap inside the chunk: one straight run of reads
#pragma unroll
                    for (int m = 0; m < 5; ++m)
                        unpack8(*reinterpret_cast<const uint4*>(raw + tt * 64 * KS + (r0 - 3 + m) * KS + ch8), xv[m]);
                } else {
#pragma unroll
                    for (int m = 0; m < 5; ++m) {
                        const int rr = r0 - 3 + m;
                        if (rr >= 0) unpack8(*reinterpret_cast<const uint4*>(raw + tt * 64 * KS + rr * KS + ch8), xv[m]);
                        else lds8f(hist + (tt * 3 + rr + 3) * 128 + ch8, xv[m]);
                    }
                }
                float y[2][8];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int c8 = 0; c8 < 8; ++c8)
                        y[i][c8] = w[0][c8] * xv[i][c8] + w[1][c8] * xv[i + 1][c8] + w[2][c8] * xv[i + 2][c8] +
                                   w[3][c8] * xv[i + 3][c8];
                if (tt < 2) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        float ss = 0.f;
#pragma unroll
                        for (int c8 = 0; c8 < 8; ++c8) ss += y[i][c8] * y[i][c8];
                        const float inv = __builtin_amdgcn_rsqf(row16_sum(ss) + kL2Eps);
#pragma unroll
                        for (int c8 = 0; c8 < 8; ++c8) y[i][c8] *= inv;
                    }
                }
                uint16_t* dst = tt == 0 ? sQ : (tt == 1 ? sK : sV);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = r0 + i;
                    const uint32_t m = r < L ? 0xffffffffu : 0u;  // padded rows: zero
                    *reinterpret_cast<uint4*>(dst + r * KS + ch8) =
                        make_uint4(pack_bf16x2(y[i][0], y[i][1]) & m, pack_bf16x2(y[i][2], y[i][3]) & m,
                                   pack_bf16x2(y[i][4], y[i][5]) & m, pack_bf16x2(y[i][6], y[i][7]) & m);
                }
            }
            lds_barrier();  // the raw rows, history and taps are dead
        }
        float x[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gv = px[j].get(e);
                // decay logs in log2 units: every use of G is 2^(difference);
                // computed for every row, padded rows masked afterwards
                const float lg = kFused ? -softplus_log2(gv) : gv * kLog2e;
                x[j][e] = 4 * rg + j < L ? lg : 0.f;
            }
        {
            const float bv = ld(&pb);
            const int bt = tid & 63;  // every wave writes the same 64 values
            sB[bt] = bt < L ? (kFused ? sigmoid_fast(bv) : bv) : 0.f;
        }
        if (tid < 4) sFlag[tid] = 0;
        for (int i = tid; i < 2 * 64 * MS / 4; i += kIntraThreads)
            reinterpret_cast<float4*>(sA)[i] = make_float4(0.f, 0.f, 0.f, 0.f);  // sA, sM
#pragma unroll
        for (int j = 1; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[j][e] += x[j - 1][e];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4*>(sG + (4 * rg + j) * GS + 4 * cq) =
                make_float4(x[j][0], x[j][1], x[j][2], x[j][3]);
        *reinterpret_cast<float4*>(sTot + rg * 128 + 4 * cq) = make_float4(x[3][0], x[3][1], x[3][2], x[3][3]);
    };

    int64_t v = blockIdx.x;
    if (v >= units) return;
    Unit nxt = unit_of(v);
    fetch_all(nxt);
    stage_inputs(nxt, ftid);
    for (;; v += gridDim.x) {
        // Lane-dependent values are rederived from an opaque copy of the thread
        // index in every unit, so the compiler does not hoist dozens of masks
        // and addresses out of the loop (they would not fit in registers).
        int tid = ftid;
        asm volatile("" : "+v"(tid));
        const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
        const int cq = tid & 31, rg = tid >> 5;
        const Unit cur = nxt;
        const int h = cur.h;
        const int64_t slot = cur.slot;
        char* rec = a.rec + (h * a.slots + slot) * REC_BYTES;  // a head's chunks are contiguous
        const bool more = v + gridDim.x < units;
        lds_barrier();
        {
            float off[4] = {0.f, 0.f, 0.f, 0.f};
            for (int q2 = 0; q2 < rg; ++q2) {
                const float4 t4 = *reinterpret_cast<const float4*>(sTot + q2 * 128 + 4 * cq);
                off[0] += t4.x; off[1] += t4.y; off[2] += t4.z; off[3] += t4.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float4* p = reinterpret_cast<float4*>(sG + (4 * rg + j) * GS + 4 * cq);
                const float4 x4 = *p;
                *p = make_float4(x4.x + off[0], x4.y + off[1], x4.z + off[2], x4.w + off[3]);
            }
        }
        lds_barrier();
        // sub-blocks whose decay inside 16 tokens is too steep for the factored form
        if (tid < 128) {
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const float d = sG[(16 * R) * GS + tid] - sG[(16 * R + 15) * GS + tid];
                if (d > kDiagRange) sFlag[R] = 1;  // benign race: every writer stores 1
            }
        }
        lds_barrier();

        // ---- A and M: 10 tiles (R >= S) of 4 contraction steps each.  Wave w
        // computes tile w whole; the steps of tiles 8 and 9 go one per wave
        // (tile 8 + w/4, step w%4), and their partial tiles are summed in a fixed
        // order afterwards, so the result does not depend on timing.
        {
            // A and M partials of tile (R, S) over contraction steps [k0, k1)
            auto tile_part = [&](int R, int S, int k0, int k1, f32x4& accA, f32x4& accM) {
                const int b = 16 * R;
                if (R == S && sFlag[R]) {
                    // exact pairwise decays (steep decay inside the block)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = b + 4 * g + i, s2 = 16 * S + c;
                        float av = 0.f, mv = 0.f;
                        if (s2 <= r) {
                            for (int ch = 32 * k0; ch < 32 * k1; ++ch) {
                                const float ks = bfv(sK + s2 * KS + ch) * exp2f(sG[r * GS + ch] - sG[s2 * GS + ch]);
                                av += bfv(sK + r * KS + ch) * ks;
                                mv += bfv(sQ + r * KS + ch) * ks;
                            }
                        }
                        accA[i] += av;
                        accM[i] += mv;
                    }
                } else {
                    const int rl = b + c, sr = 16 * S + c;
                    for (int ks = k0; ks < k1; ++ks) {
                        const int ch0 = 32 * ks + 8 * g;
                        float kl[8], ql[8], kr[8], gl[8], gb[8], gr[8];
                        unpack8(*reinterpret_cast<const uint4*>(sK + rl * KS + ch0), kl);
                        unpack8(*reinterpret_cast<const uint4*>(sQ + rl * KS + ch0), ql);
                        unpack8(*reinterpret_cast<const uint4*>(sK + sr * KS + ch0), kr);
                        lds8f(sG + rl * GS + ch0, gl);
                        lds8f(sG + b * GS + ch0, gb);
                        lds8f(sG + sr * GS + ch0, gr);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float el = __builtin_amdgcn_exp2f(gl[e] - gb[e]);  // <= 1
                            kl[e] *= el;
                            ql[e] *= el;
                            kr[e] *= __builtin_amdgcn_exp2f(gb[e] - gr[e]);
                        }
                        const bf16x8 bk = to_bf16x8(kr);
                        accA = mfma(to_bf16x8(kl), bk, accA);
                        accM = mfma(to_bf16x8(ql), bk, accM);
                    }
                }
            };
            auto store_tile = [&](int R, int S, const f32x4& accA, const f32x4& accM) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * R + 4 * g + i, s2 = 16 * S + c;
                    sA[r * MS + s2] = s2 < r ? accA[i] : 0.f;
                    sM[r * MS + s2] = s2 <= r ? accM[i] : 0.f;
                }
            };
            int R, S;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = accA;
            tile_rs(wave, R, S);
            tile_part(R, S, 0, 4, accA, accM);
            store_tile(R, S, accA, accM);
            // one step of tile 8 or 9 into a partial block in sT (free until T is built)
            const int tp = 8 + (wave >> 2), kp = wave & 3;
            tile_rs(tp, R, S);
            accA = f32x4{0.f, 0.f, 0.f, 0.f};
            accM = accA;
            tile_part(R, S, kp, kp + 1, accA, accM);
            float* part = sT + wave * 512;  // [A: 4 x 64 lanes][M: 4 x 64 lanes]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part[i * 64 + lane] = accA[i];
                part[256 + i * 64 + lane] = accM[i];
            }
            lds_barrier();
            if (wave < 2) {  // wave 0 sums tile 8, wave 1 tile 9, steps in order
                tile_rs(8 + wave, R, S);
                f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sm = sa;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float* q = sT + (4 * wave + k) * 512;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sa[i] += q[i * 64 + lane];
                        sm[i] += q[256 + i * 64 + lane];
                    }
                }
                store_tile(R, S, sa, sm);
            }
        }
        lds_barrier();

        // The next unit's loads go out in four parts, one after each of the
        // phases from here on, and land during the rest of this unit's work.
        // All workgroups run in near lockstep, so one burst of loads per unit
        // would saturate HBM while it lasts and idle it the rest of the time.
        if (more) {
            nxt = unit_of(v + gridDim.x);
            fetch(nxt, 0);
        }

        // ---- T = (I + Diag(beta) A)^-1
        // diagonal blocks: wave R < 4, lane j < 16 owns column j of T_RR in registers
        if (wave < 4) {
            const int R = wave, j = lane;
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float arow[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 v4 = *reinterpret_cast<const float4*>(sA + (16 * R + r) * MS + 16 * R + 4 * q4);
                    arow[4 * q4] = v4.x; arow[4 * q4 + 1] = v4.y; arow[4 * q4 + 2] = v4.z; arow[4 * q4 + 3] = v4.w;
                }
                float sum = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) sum += arow[s2] * t[s2];
                t[r] = (r == j ? 1.f : 0.f) - sB[16 * R + r] * sum;
            }
            if (j < 16) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sT[(16 * R + r) * MS + 16 * R + j] = t[r];
            }
        }
        lds_barrier();
        if (more) fetch(nxt, 1);
        // Off-diagonal blocks of T from the two 32 x 32 halves (L = Diag(beta) A):
        //   level 1: T_10 = -T_11 L_10 T_00,  T_32 = -T_33 L_32 T_22          (waves 0, 1)
        //   level 2: X = L_hi,lo T_lo:  X_20 = L_20 T_00 + L_21 T_10,  X_21 = L_21 T_11,
        //            X_30 = L_30 T_00 + L_31 T_10,  X_31 = L_31 T_11           (waves 0..3)
        //   level 3: T_hi,lo = -T_hi X:  T_20 = -T_22 X_20,  T_21 = -T_22 X_21,
        //            T_30 = -(T_32 X_20 + T_33 X_30),  T_31 = -(T_32 X_21 + T_33 X_31)
        // Lane (g, c) computes rows 4g .. 4g+3, column c of a 16 x 16 block.
        {
            // 16 x 16 blocks with row stride XS, XB floats apart (the scan
            // partials are dead); 20 puts the four row groups a wave writes
            // on distinct banks
            constexpr int XS = 20, XB = 16 * XS;
            float* sX = sTot;
            // acc[i] += sum_k P[4g+i][k] Q[k][c] over a 16 x 16 pair, in fp32 on
            // the matrix cores: v_mfma_f32_16x16x4_f32 takes A[c][g] and B[g][c]
            // from lane (g, c) and leaves D[4g + i][c], four steps of 4 in k
            auto mm16 = [&](const float* P, int ldp, const float* Q, int ldq, float (&acc)[4]) {
                f32x4 d = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    d = __builtin_amdgcn_mfma_f32_16x16x4f32(P[c * ldp + 4 * s4 + g], Q[(4 * s4 + g) * ldq + c], d,
                                                             0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = d[i];
            };
            if (wave < 2) {
                const int R = 2 * wave + 1, S = R - 1;
                float y[4] = {0.f, 0.f, 0.f, 0.f};
                mm16(sA + (16 * R) * MS + 16 * S, MS, sT + (16 * S) * MS + 16 * S, MS, y);
                float* Y = sX + wave * XB;
#pragma unroll
                for (int i = 0; i < 4; ++i) Y[(4 * g + i) * XS + c] = sB[16 * R + 4 * g + i] * y[i];
                // (a wave's LDS operations are performed in order: Y is complete here)
                float t[4] = {0.f, 0.f, 0.f, 0.f};
                mm16(sT + (16 * R) * MS + 16 * R, MS, Y, XS, t);
#pragma unroll
                for (int i = 0; i < 4; ++i) sT[(16 * R + 4 * g + i) * MS + 16 * S + c] = -t[i];
            }
            lds_barrier();
            const int R = 2 + (wave >> 1), S = wave & 1;  // block of waves 0..3
            if (wave < 4) {
                float x[4] = {0.f, 0.f, 0.f, 0.f};
                for (int J = S; J < 2; ++J) mm16(sA + (16 * R) * MS + 16 * J, MS, sT + (16 * J) * MS + 16 * S, MS, x);
#pragma unroll
                for (int i = 0; i < 4; ++i) sX[wave * XB + (4 * g + i) * XS + c] = sB[16 * R + 4 * g + i] * x[i];
            }
            lds_barrier();
            if (wave < 4) {
                float t[4] = {0.f, 0.f, 0.f, 0.f};
                mm16(sT + (16 * R) * MS + 32, MS, sX + S * XB, XS, t);                      // T_R2 X_2S
                if (R == 3) mm16(sT + (16 * 3) * MS + 48, MS, sX + (2 + S) * XB, XS, t);  // T_33 X_3S
#pragma unroll
                for (int i = 0; i < 4; ++i) sT[(16 * R + 4 * g + i) * MS + 16 * S + c] = -t[i];
            }
        }
        lds_barrier();
        // blocks of T above the diagonal are never written; every reader masks them

        if (more) fetch(nxt, 2);
        // ---- W = T (beta e^G K) and U~ = T (beta V): column tile nt = wave
        const int nt = wave;
        const int chn = 16 * nt + c;
        f32x4 accW[4], accU[4];
        {
            bf16x8 Ta[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int row = 16 * mt + c, col0 = 32 * ks + 8 * g;
                    float tv[8];
                    lds8f(sT + row * MS + col0, tv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) tv[e] = col0 + e <= row ? tv[e] : 0.f;
                    Ta[mt][ks] = to_bf16x8(tv);
                }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                accW[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                accU[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int s0 = 32 * ks + 8 * g;
                float bt[8], bk[8], bv[8];
                lds8f(sB + s0, bt);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s2 = s0 + e;
                    bk[e] = bt[e] * __builtin_amdgcn_exp2f(sG[s2 * GS + chn]) * bfv(sK + s2 * KS + chn);
                    bv[e] = bt[e] * bfv(sV + s2 * KS + chn);
                }
                const bf16x8 Bk = to_bf16x8(bk), Bv = to_bf16x8(bv);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (32 * ks > 16 * mt + 15) continue;  // T is lower triangular
                    accW[mt] = mfma(Ta[mt][ks], Bk, accW[mt]);
                    accU[mt] = mfma(Ta[mt][ks], Bv, accU[mt]);
                }
            }
            // U~ in result layout, slice nt
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                uint2 p;
                p.x = pack_bf16x2(accU[mt][0], accU[mt][1]);
                p.y = pack_bf16x2(accU[mt][2], accU[mt][3]);
                rec_store8(rec + R_UT + ((nt * 4 + mt) * 64 + lane) * 8, p);
            }
        }
        lds_barrier();  // V and A are dead: their buffers become the staging areas

        if (more) fetch(nxt, 3);
        // ---- Q' = e^G Q - M W and M U~; stage -W and Q' for the transposes
        {
            bf16x8 Mneg[4][2], Mpos[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const float* mrow = sM + (16 * mt + c) * MS + 32 * ks + 4 * g;
                    const float4 lo = *reinterpret_cast<const float4*>(mrow);
                    const float4 hi = *reinterpret_cast<const float4*>(mrow + 16);
                    const float mv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    float mn[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) mn[e] = -mv[e];
                    Mpos[mt][ks] = to_bf16x8(mv);
                    Mneg[mt][ks] = to_bf16x8(mn);
                }
            bf16x8 Bw[2], Bu[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                Bw[ks] = to_bf16x8(accW[2 * ks], accW[2 * ks + 1]);
                Bu[ks] = to_bf16x8(accU[2 * ks], accU[2 * ks + 1]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 qp, oi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g + i;
                    qp[i] = __builtin_amdgcn_exp2f(sG[r * GS + chn]) * bfv(sQ + r * KS + chn);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (32 * ks > 16 * mt + 15) continue;  // M is lower triangular
                    qp = mfma(Mneg[mt][ks], Bw[ks], qp);
                    // (M U~)^T = U~^T M^T: the operands swap roles, so lane (g, c)
                    // ends up with M U~[16mt + c][16nt + 4g + i]
                    oi = mfma(Bu[ks], Mpos[mt][ks], oi);
                }
                uint2 p;
                p.x = pack_bf16x2(oi[0], oi[1]);
                p.y = pack_bf16x2(oi[2], oi[3]);
                rec_store8(rec + R_OI + ((nt * 4 + mt) * 64 + lane) * 8, p);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g + i;
                    sStW[r * KS + chn] = f32_to_bf16(-accW[mt][i]);
                    sStQ[r * SQS + chn] = f32_to_bf16(qp[i]);
                }
            }
        }
        lds_barrier();

        // ---- stores in the A-operand layout: -W, Q' (2 blocks per wave each), K^T
        {
            const int mt = wave >> 1;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ks = 2 * (wave & 1) + k2;
                const int r = 16 * mt + c;
                const int c0 = 32 * ks + 4 * g;
                const uint2 wlo = *reinterpret_cast<const uint2*>(sStW + r * KS + c0);
                const uint2 whi = *reinterpret_cast<const uint2*>(sStW + r * KS + c0 + 16);
                const uint2 qlo = *reinterpret_cast<const uint2*>(sStQ + r * SQS + c0);
                const uint2 qhi = *reinterpret_cast<const uint2*>(sStQ + r * SQS + c0 + 16);
                const int blk = (mt * 4 + ks) * 64 + lane;
                rec_store16(rec + R_NEGW + blk * 16, make_uint4(wlo.x, wlo.y, whi.x, whi.y));
                rec_store16(rec + R_QP + blk * 16, make_uint4(qlo.x, qlo.y, qhi.x, qhi.y));
            }
            const int t = wave;
            const int ch = 16 * t + c;
            const float glast = sG[63 * GS + ch];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float kv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s2 = 32 * ks + perm(g, e);
                    kv[e] = __builtin_amdgcn_exp2f(glast - sG[s2 * GS + ch]) * bfv(sK + s2 * KS + ch);
                }
                uint4 p;
                p.x = pack_bf16x2(kv[0], kv[1]);
                p.y = pack_bf16x2(kv[2], kv[3]);
                p.z = pack_bf16x2(kv[4], kv[5]);
                p.w = pack_bf16x2(kv[6], kv[7]);
                rec_store16(rec + R_KHT + ((t * 2 + ks) * 64 + lane) * 16, p);
            }
            if (tid < 128) reinterpret_cast<float*>(rec + R_GAM)[tid] = exp2f(sG[63 * GS + tid]);
        }
        lds_barrier();  // every LDS buffer is free for the next unit
        // Leave before staging rather than staging conditionally: the loop's
        // back edge then comes only from a path where the staging has
        // consumed (waited for) every prefetched register, so reusing those
        // registers in the next unit needs no wait for loads in flight.
        if (!more) break;
        stage_inputs(nxt, tid);
    }
}

// ---------------------------------------------------------------------------
// phase 2
// ---------------------------------------------------------------------------

// One workgroup per (sequence, head, group of SB 16-column slices of the
// state), with three roles.  Per slice, a chain wave keeps the slice's state
// in registers and runs the recurrence, and an output wave computes the
// gated output from the state the chain wave hands over in LDS (see the
// compute section).  Inside the chunk loop they touch only LDS, reading the
// chunk's factors and writing the gated output tile to an LDS staging area.
// Four memory waves do all global traffic: they copy what a chunk needs into
// one of two LDS buffers with global_load_lds_dwordx4 and store the staged
// output as whole row pieces.  A chunk is copied in two parts: the part the
// first half of a step reads (-W, Q', the group's U~ and M U~ tiles, its gate
// logits) as soon as the compute waves are done with it two chunks back, and
// the part the second half reads (K^T, gamma) one step ahead.  Every memory
// wave issues the same number of operations every step (a wave with no piece
// of some tile makes a one-lane copy into a dump area), so a fixed count
// (vmcnt) tells when a part has landed while later ones stay in flight:
// vector memory operations of one wave retire in issue order.
// One slice per workgroup spreads a head over more CUs, which suits few
// (sequence, head) pairs; two share each copied factor between two slices.
template <int SB>
struct StateCfg {
    static_assert(SB == 1 || SB == 2, "1 or 2 slices per workgroup");
    // memory waves: each issues its share of every copy (more of them do not
    // move a chunk faster: the copies are bound by the CU's path into LDS)
    static constexpr int kMemWaves = 4;
    static constexpr int kRowBytes = 32 * SB;             // one token row of the group's columns, bf16
    static constexpr int kPieces = 2 * SB;                // 1 KB pieces of each group tile (U~, M U~, z)
    static constexpr int kPiecesPerWave = (kPieces + kMemWaves - 1) / kMemWaves;
    static constexpr int kRowsPerWave = 64 / kMemWaves;   // output rows each memory wave stores
    // LDS buffer layout, bytes.  The first 48 KB mirror the record's first 48 KB.
    static constexpr int B_NEGW = 0;                      // -W, 16 KB
    static constexpr int B_QP = 16384;                    // Q', 16 KB
    static constexpr int B_KHT = 32768;                   // K^T, 16 KB
    static constexpr int B_UT = 49152;                    // U~ of the group's slices, [SB s][4 m][64][4]
    static constexpr int B_OI = B_UT + 1024 * kPieces;    // M U~, same layout
    static constexpr int B_Z = B_OI + 1024 * kPieces;     // gate logits [64 tokens][kRowBytes], swizzled
    static constexpr int B_GAM = B_Z + 1024 * kPieces;    // gamma, fp32 [128]
    static constexpr int B_DUMP = B_GAM + 512;            // target of the one-lane filler copies, never read
    static constexpr int B_BYTES = B_DUMP + 64;
    // operations one memory wave issues per part (wave 0 issues one more in
    // the second part: gamma) and per output tile
    static constexpr int kPartA = 32 / kMemWaves + 3 * kPiecesPerWave;
    static constexpr int kPartB = 16 / kMemWaves;
    static constexpr int kRowsPerStore = 1024 / kRowBytes;  // rows of kRowBytes one 64-lane store covers
    static constexpr int kStores = (kRowsPerWave + kRowsPerStore - 1) / kRowsPerStore;
    // after the two buffers: the staged output tile, then per slice the bf16
    // state operand the chain wave hands to the output wave
    static constexpr int B_STAGE = 2 * B_BYTES;
    static constexpr int B_SBX = B_STAGE + 64 * kRowBytes;  // [SB s][4 ks][64 lanes][16 B]
    static constexpr size_t kLds = static_cast<size_t>(B_SBX) + 4096 * SB;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lds_copy16(const void* gsrc, char* lds_dst) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)(lds_dst), 16, 0, 0);
}

// 16 bytes of LDS that no LDS-DMA copy writes (the output staging area).  The
// compiler cannot tell which LDS bytes a copy in flight lands in, so before a
// plain LDS read it waits for all of them (vmcnt 0), which would drain the
// copy pipeline every step.  This read is inline asm instead, waited for
// (lgkmcnt 0) in the same block.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_read16_staged(const char* p) {
    u32x4_t v;
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void*)(p)));
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Tiles of 64 token rows x (2 SB) 16-byte pieces (gate logits, staged
// output): piece q of row r is kept at slot q ^ (r mod 2 SB), so reads and
// writes that walk 16 rows of one column group spread over the banks.
template <int SB>
__device__ __forceinline__ int tile_slot(int r, int q) { return q ^ (r & (2 * SB - 1)); }

// s_waitcnt with vmcnt(n) only (lgkmcnt and expcnt left at their maxima)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename GT, bool kGate, int NS>
__global__ __launch_bounds__(64 * (2 * NS + StateCfg<NS>::kMemWaves)) void mfma_state_kernel(MfmaK<GT> a) {
    constexpr int SB = NS;
    using C = StateCfg<SB>;
    constexpr int P = 8 / SB;            // slice groups per head
    constexpr int RB = C::kRowBytes;
    constexpr int PR = 2 * SB;           // 16-byte pieces per tile row
    constexpr int ROWS_PER_PIECE = 1024 / RB;
    extern __shared__ __align__(16) char smem[];
    char* const buf0 = smem;
    char* const buf1 = smem + C::B_BYTES;
    char* const stage = smem + C::B_STAGE;  // gated output tile, bf16 [64][RB], swizzled
    // blockIdx -> (sequence, head, part): all parts of a (sequence, head) land
    // on one XCD (workgroups are dealt round-robin over the 8 XCDs), so the
    // chunk records they share are read through one L2
    const int bid = blockIdx.x;
    const int xcd = bid & 7, part = (bid >> 3) % P;
    const int64_t grp = static_cast<int64_t>((bid >> 3) / P) * 8 + xcd;
    if (grp >= a.groups) return;
    const int H = a.H;
    const int n = static_cast<int>(grp / H), h = static_cast<int>(grp % H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;

    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    int slot0, nch;
    if (a.inline_map) {
        const int incl = chunk_prefix_lane(a.cu, a.N, a.T);
        slot0 = slots_before(incl, n);
        nch = __builtin_amdgcn_readlane(incl, n) - slot0;
    } else {
        slot0 = a.base[n];
        nch = a.base[n + 1] - slot0;
    }
    auto rec_of = [&](int j) { return a.rec + (h * a.slots + slot0 + j) * REC_BYTES; };
    auto chunk_len = [&](int j) {
        return static_cast<int>(min(static_cast<int64_t>(kChunk), se - (sb + static_cast<int64_t>(j) * kChunk)));
    };
    auto buf_of = [&](int j) { return (j & 1) ? buf1 : buf0; };

    if (wave >= 2 * NS) {
        // ---- memory waves
        if (nch == 0) return;
        const int wm = wave - 2 * NS;
        // part A of chunk min(j, nch-1): -W, Q', U~, M U~ and gate logits
        // (past the end it copies the last chunk again into the free buffer
        // the index selects, so that every step issues the same operations)
        constexpr int MW = C::kMemWaves;
        auto issue_a = [&](int jn) {
            char* buf = buf_of(jn);
            const int j = min(jn, nch - 1);
            const char* rp = rec_of(j);
#pragma unroll
            for (int i = 0; i < 32 / MW; ++i) {
                const int b = wm + MW * i;
                lds_copy16(rp + b * 1024 + lane * 16, buf + b * 1024);
            }
            const int Lc = chunk_len(j);
            const int64_t tb = sb + static_cast<int64_t>(j) * kChunk;
#pragma unroll
            for (int i = 0; i < C::kPiecesPerWave; ++i) {
                const int b = wm + MW * i;
                const bool real = b < C::kPieces;
                const int bb = real ? b : 0;
                const char* ut = rp + R_UT + part * (1024 * C::kPieces) + bb * 1024 + lane * 16;
                const char* oi = rp + R_OI + part * (1024 * C::kPieces) + bb * 1024 + lane * 16;
                // a filler copy (no piece here) moves 16 bytes from one lane:
                // it is one operation all the same, which keeps the count fixed
                if (real || lane == 0) {
                    lds_copy16(ut, real ? buf + C::B_UT + b * 1024 : buf + C::B_DUMP);
                    lds_copy16(oi, real ? buf + C::B_OI + b * 1024 : buf + C::B_DUMP);
                }
                const int r = bb * ROWS_PER_PIECE + lane / PR;
                const int q = tile_slot<SB>(r, lane % PR);  // the slot map is its own inverse
                // without a gate the tile is never read; copying keeps the count fixed
                const void* zs = kGate ? static_cast<const void*>(a.z + ((tb + min(r, Lc - 1)) * H + h) * 128 +
                                                                  16 * SB * part + 8 * q)
                                       : static_cast<const void*>(ut);
                if ((real && kGate) || lane == 0)
                    lds_copy16(zs, (real && kGate) ? buf + C::B_Z + b * 1024 : buf + C::B_DUMP);
            }
        };
        // part B of chunk min(j, nch-1): K^T and gamma
        auto issue_b = [&](int jn) {
            char* buf = buf_of(jn);
            const int j = min(jn, nch - 1);
            const char* rp = rec_of(j);
#pragma unroll
            for (int i = 0; i < 16 / MW; ++i) {
                const int b = 32 + wm + MW * i;
                lds_copy16(rp + b * 1024 + lane * 16, buf + b * 1024);
            }
            if (wm == 0 && lane < 32) lds_copy16(rp + R_GAM + lane * 16, buf + C::B_GAM);
        };
        // issue order per step j: [A_j] B(j+1) [M_j] stores(j), A(j+2).
        // Before A_j part A of chunk j must be in; after it came B(j),
        // stores(j-1) and A(j+1).  Before M_j part B of chunk j must be in;
        // after it came stores(j-1), A(j+1) and B(j+1).  (Wave 0's gamma copy
        // is left out of the counts: it waits for one operation more than
        // needed.)  In step 0 there were no stores(-1).
        constexpr int kA = C::kPartA, kB = C::kPartB, kS = C::kStores;
        issue_a(0);
        issue_b(0);
        issue_a(1);
        // store role: rows RW wm .. RW wm + RW-1, ROWS_PER_PIECE of them per
        // instruction
        constexpr int RW = C::kRowsPerWave;
        const int wq = lane % PR;
        for (int j = 0; j < nch; ++j) {
            if (j == 0) wait_vmcnt<kB + kA>(); else wait_vmcnt<kB + kS + kA>();
            lds_barrier();  // A_j: part A of chunk j is in LDS; part B of chunk j+1 may be copied
            issue_b(j + 1);
            if (j == 0) wait_vmcnt<kA + kB>(); else wait_vmcnt<kS + kA + kB>();
            lds_barrier();  // M_j: part B of chunk j is in; the output tile of chunk j is staged
            const int Lc = chunk_len(j);
            const int64_t tb = sb + static_cast<int64_t>(j) * kChunk;
#pragma unroll
            for (int i = 0; i < kS; ++i) {
                const int rl = i * ROWS_PER_PIECE + lane / PR;  // row within the wave's RW
                const int r = RW * wm + min(rl, RW - 1);
                const uint4 v = lds_read16_staged(stage + r * RB + wq * 16);
                const int q = tile_slot<SB>(r, wq);
                // rows past the end exist only in a sequence's last chunk,
                // after which no counted wait follows
                if (rl < RW && r < Lc)
                    *reinterpret_cast<uint4*>(a.out + ((tb + r) * H + h) * 128 + 16 * SB * part + 8 * q) = v;
            }
            issue_a(j + 2);
        }
        wait_vmcnt<0>();  // no copy may land after the workgroup has ended
        return;
    }

    // ---- compute waves: two per 16-column slice ls = wave / 2 of the group.
    // The chain wave (even) keeps the slice's fp32 state in registers and runs
    // the recurrence, U = U~ - W S and then S <- Diag(gamma) S + K^T U; after
    // each update it leaves the state as the bf16 matrix-core operand in LDS.
    // The output wave (odd) takes that operand for the chunk's gated output,
    // O^T = (M U~)^T + S^T Q'^T, off the recurrence's critical path: row tiles
    // 0-2; the chain wave, which has less to do before M_j, takes row tile 3.
    // Inside the chunk loop both touch only LDS.  In a step the output wave
    // reads the operand before M_j and the chain wave rewrites it after M_j.
    const int ls = wave >> 1;
    char* const sbx = smem + C::B_SBX + ls * 4096;
    const int col0 = 16 * (SB * part + ls) + c;
    auto widen = [](uint2 p) {
        return f32x4{__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xffff0000u), __uint_as_float(p.y << 16),
                     __uint_as_float(p.y & 0xffff0000u)};
    };
    // one row tile of the output: lane (g, c) holds token 16 mt + c, columns
    // 16 ls + 4 g .. + 3 (the state operand and the Q' operand swap roles)
    struct OutOps {
        uint2 op, zp;
        bf16x8 qa[4];
    };
    auto stage_off = [&](int mt) {
        // columns 16 ls + 4 g .. + 3 of the group: piece 2 ls + g/2, bytes 8 (g & 1)
        const int r = 16 * mt + c;
        return r * RB + tile_slot<SB>(r, 2 * ls + (g >> 1)) * 16 + 8 * (g & 1);
    };
    auto load_out = [&](const char* cur, int mt, OutOps& x) {
        x.op = *reinterpret_cast<const uint2*>(cur + C::B_OI + ((ls * 4 + mt) * 64 + lane) * 8);
        if (kGate) x.zp = *reinterpret_cast<const uint2*>(cur + C::B_Z + stage_off(mt));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            x.qa[ks] = *reinterpret_cast<const bf16x8*>(cur + C::B_QP + ((mt * 4 + ks) * 64 + lane) * 16);
    };
    auto out_tile = [&](int mt, const OutOps& x, const bf16x8 (&Sb)[4]) {
        f32x4 o = widen(x.op);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o = mfma(Sb[ks], x.qa[ks], o);
        if (kGate) {
            const f32x4 zf = widen(x.zp);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] *= sigmoid_fast(zf[i]);
        }
        *reinterpret_cast<uint2*>(stage + stage_off(mt)) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    };
    if ((wave & 1) == 0) {
        f32x4 S[8];  // S[t][i] = state[16t + 4g + i][col0]
        const int64_t sidx = grp * (128 * 128);
        if (a.S0 != nullptr) {  // one uniform branch: all loads in flight together
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[t][i] = a.S0[sidx + (16 * t + 4 * g + i) * 128 + col0];
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        bf16x8 Sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Sb[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
            *reinterpret_cast<bf16x8*>(sbx + (ks * 64 + lane) * 16) = Sb[ks];
        }
        for (int j = 0; j < nch; ++j) {
            const char* cur = buf_of(j);
            lds_barrier();  // A_j: part A of chunk j is in LDS
            // U = U~ - W S; the reads of row tile mt + 1 go out before the
            // products of tile mt
            struct ChainOps {
                uint2 up;
                bf16x8 wa[4];
            };
            auto load_tile = [&](int mt, ChainOps& x) {
                x.up = *reinterpret_cast<const uint2*>(cur + C::B_UT + ((ls * 4 + mt) * 64 + lane) * 8);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    x.wa[ks] = *reinterpret_cast<const bf16x8*>(cur + C::B_NEGW + ((mt * 4 + ks) * 64 + lane) * 16);
            };
            f32x4 U[4];
            ChainOps ops[2];
            OutOps oops;
            load_tile(0, ops[0]);
            load_out(cur, 3, oops);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (mt < 3) load_tile(mt + 1, ops[(mt + 1) & 1]);
                const ChainOps& x = ops[mt & 1];
                U[mt] = widen(x.up);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) U[mt] = mfma(x.wa[ks], Sb[ks], U[mt]);
            }
            out_tile(3, oops, Sb);
            lds_barrier();  // M_j: part B of chunk j is in LDS; the output wave is done with the operand
            // S <- Diag(gamma) S + K^T U, with every K^T and gamma read issued first
            bf16x8 ka[8][2];
            float4 gm[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                gm[t] = *reinterpret_cast<const float4*>(cur + C::B_GAM + (16 * t + 4 * g) * 4);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    ka[t][ks] = *reinterpret_cast<const bf16x8*>(cur + C::B_KHT + ((t * 2 + ks) * 64 + lane) * 16);
            }
            const bf16x8 Ub[2] = {to_bf16x8(U[0], U[1]), to_bf16x8(U[2], U[3])};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                S[t][0] *= gm[t].x;
                S[t][1] *= gm[t].y;
                S[t][2] *= gm[t].z;
                S[t][3] *= gm[t].w;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) S[t] = mfma(ka[t][ks], Ub[ks], S[t]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Sb[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
                *reinterpret_cast<bf16x8*>(sbx + (ks * 64 + lane) * 16) = Sb[ks];
            }
            // a full chunk that ends a snapshot interval: the state after it
            // is the sequence's m-th snapshot (this slice's columns)
            const int sc = a.snap.chunks;
            if (sc > 0 && (j + 1) % sc == 0 && chunk_len(j) == kChunk) {
                float* so = a.snap.out + ((static_cast<int64_t>(a.snap.off[n]) + (j + 1) / sc - 1) * H + h) * (128 * 128);
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) so[(16 * t + 4 * g + i) * 128 + col0] = S[t][i];
            }
        }
        if (a.S_out) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) a.S_out[sidx + (16 * t + 4 * g + i) * 128 + col0] = S[t][i];
        }
    } else {
        for (int j = 0; j < nch; ++j) {
            const char* cur = buf_of(j);
            lds_barrier();  // A_j: part A of chunk j and the state operand are in LDS; the staging tile is free
            bf16x8 Sb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) Sb[ks] = *reinterpret_cast<const bf16x8*>(sbx + (ks * 64 + lane) * 16);
            // row tiles 0-2; the reads of tile mt + 1 go out before the products of tile mt
            OutOps ops[2];
            load_out(cur, 0, ops[0]);
#pragma unroll
            for (int mt = 0; mt < 3; ++mt) {
                if (mt < 2) load_out(cur, mt + 1, ops[(mt + 1) & 1]);
                out_tile(mt, ops[mt & 1], Sb);
            }
            lds_barrier();  // M_j: the output tile is staged
        }
    }
}

template <typename GT, bool kGate, int NS>
hipError_t launch_state(const MfmaK<GT>& k, hipStream_t s) {
    using C = StateCfg<NS>;
    constexpr int P = 8 / NS;
    const void* fn = reinterpret_cast<const void*>(&mfma_state_kernel<GT, kGate, NS>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(C::kLds));
    if (e != hipSuccess) return e;
    const int64_t blocks = (k.groups + 7) / 8 * 8 * P;
    hipLaunchKernelGGL((mfma_state_kernel<GT, kGate, NS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * (2 * NS + C::kMemWaves)), C::kLds, s, k);
    return hipGetLastError();
}

// Workgroup shape of the state pass.  Few (sequence, head) pairs: spread
// each head over 8 workgroups of one 16-column slice, so every CU takes
// part.  Many: one workgroup per quarter head (two slices), so each copied
// factor serves two slices.  KDA_STATE_SHAPE=1 or 2 in the environment forces
// the number of slices per workgroup (the tests use it to cover both).
template <typename GT, bool kGate>
hipError_t launch_state_for(const MfmaK<GT>& k, hipStream_t s, int cus) {
    int ns = k.groups * 8 <= cus ? 1 : 2;
    if (const char* env = getenv("KDA_STATE_SHAPE")) {
        const int f = atoi(env);
        if (f == 1 || f == 2) ns = f;
    }
    return ns == 1 ? launch_state<GT, kGate, 1>(k, s) : launch_state<GT, kGate, 2>(k, s);
}

// the two kernels of the chunked prefill; kFused: k.q, k.k, k.v, k.la and
// k.beta hold the raw layer inputs (see MfmaK)
template <typename GT, bool kFused>
hipError_t launch_kernels(MfmaK<GT>& k, hipStream_t s) {
    const int64_t slots = chunk_slots_bound(k.T, k.N);
    k.slots = slots;
    k.groups = static_cast<int64_t>(k.N) * k.H;
    k.inline_map = mfma_inline_map(k.N, k.snap);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = max(cus, 1);
    if (k.T > 0) {
        const void* fn = reinterpret_cast<const void*>(&mfma_intra_kernel<GT, kFused>);
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kIntraLds));
        if (e != hipSuccess) return e;
        // persistent grid: one workgroup per CU (the LDS footprint allows one)
        const int64_t grid = min(slots * k.H, static_cast<int64_t>(cus));
        LaunchTimer timer(kFused ? "mfma_prep_intra" : "mfma_intra", s);
        hipLaunchKernelGGL((mfma_intra_kernel<GT, kFused>), dim3(static_cast<unsigned>(grid)), dim3(kIntraThreads),
                           kIntraLds, s, k);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    LaunchTimer timer("mfma_state", s);
    return k.z ? launch_state_for<GT, true>(k, s, cus) : launch_state_for<GT, false>(k, s, cus);
}

template <typename GT>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t s, int32_t* base, const SlotInfo* slot_info, char* recs) {
    MfmaK<GT> k{};
    k.T = a.T; k.H = a.H; k.N = a.N; k.cu = a.cu; k.base = base; k.slot_info = slot_info;
    k.q = static_cast<const bf16*>(a.q); k.k = static_cast<const bf16*>(a.k);
    k.v = static_cast<const bf16*>(a.v); k.z = static_cast<const bf16*>(a.z);
    k.la = static_cast<const GT*>(a.la); k.beta = static_cast<const GT*>(a.beta);
    k.S0 = a.S0; k.S_out = a.S_out; k.out = static_cast<bf16*>(a.out); k.rec = recs; k.snap = a.snap;
    return launch_kernels<GT, false>(k, s);
}

}  // namespace

bool mfma_prefill_supports(int dk, int dv, DT x) { return dk == 128 && dv == 128 && x == DT::BF16; }

bool mfma_inline_map(int N, const Snapshots& snap) { return N >= 1 && N <= 64 && snap.chunks == 0; }

size_t mfma_record_bytes() { return REC_BYTES; }

hipError_t launch_layer_mfma(const LayerArgs& a, hipStream_t s, int32_t* base, const SlotInfo* slot_info,
                             char* recs) {
    MfmaK<bf16> k{};
    k.T = a.T; k.H = a.H; k.N = a.N; k.cu = a.cu; k.base = base; k.slot_info = slot_info;
    k.q = static_cast<const bf16*>(a.q_in); k.k = static_cast<const bf16*>(a.k_in);
    k.v = static_cast<const bf16*>(a.v_in); k.z = static_cast<const bf16*>(a.z);
    k.la = static_cast<const bf16*>(a.g); k.beta = static_cast<const bf16*>(a.b);
    k.w_q = static_cast<const bf16*>(a.w_q); k.w_k = static_cast<const bf16*>(a.w_k);
    k.w_v = static_cast<const bf16*>(a.w_v); k.cs = a.conv_state;
    k.S0 = a.S0; k.S_out = a.S_out; k.out = static_cast<bf16*>(a.out); k.rec = recs; k.snap = a.snap;
    return launch_kernels<bf16, true>(k, s);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s, int32_t* base, const SlotInfo* slot_info,
                               char* recs) {
    return a.gate == DT::BF16 ? launch_typed<bf16>(a, s, base, slot_info, recs)
                              : launch_typed<float>(a, s, base, slot_info, recs);
}

}  // namespace kda
