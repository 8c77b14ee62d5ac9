// Pieces shared by the two chunked-prefill implementations: the chunk map and
// the workspace layout.
//
// Chunking.  Each sequence is cut into chunks of 64 tokens starting at its own
// first token (the last chunk of a sequence may be shorter).  Chunk "slots"
// are numbered sequence by sequence: sequence n owns slots
// base[n] .. base[n+1]-1 with base[n] = sum_{m<n} ceil(L_m / 64).  A one-block
// kernel computes base[] on the device, so the host never reads cu_seqlens;
// grids are sized with the bound ceil(T/64) + N and surplus blocks exit.
//
// Chunked form of the recurrence (an exact rewrite of the token-by-token
// rule, so only rounding differs).  Inside a chunk with local tokens r, s,
// decay cumsums G_r = sum_{i<=r} log alpha_i (per key channel) and S the state
// at the chunk start:
//   A_rs = sum_c k_rc k_sc e^{G_rc - G_sc}   (s < r)
//   M_rs = sum_c q_rc k_sc e^{G_rc - G_sc}   (s <= r)
//   T    = (I + Diag(beta) A)^-1             (unit lower triangular)
//   W    = T Diag(beta) (e^G * K),   U~ = T Diag(beta) V
//   U    = U~ - W S                  (the chunk's delta-rule writes)
//   O    = (e^G * Q) S + M U = Q' S + M U~,   Q' = e^G * Q - M W
//   S   <- Diag(gamma) S + K^T U,    K^ = e^{G_last - G} * K, gamma = e^{G_last}
// The state-independent parts (W, U~, Q', K^, M U~, gamma) are computed for
// all chunks in parallel and stored per (chunk slot, head); a second kernel
// walks each sequence's chunks in order carrying S in fp32.
#pragma once

#include "kda_common.h"

namespace kda {

__device__ __forceinline__ int64_t seq_begin(const int32_t* cu, int n) { return cu ? cu[n] : 0; }
__device__ __forceinline__ int64_t seq_finish(const int32_t* cu, int n, int64_t T) {
    return cu ? cu[n + 1] : T;
}

// The chunk map, built on the device by one workgroup of 1024 threads:
//   base[0..N]       prefix sums of chunks per sequence;
//   slot_info[slot]  for each used chunk slot, its first token, length and
//                    sequence (slots past base[N] are left unwritten);
//   snap_off[0..N]   (snap_chunks > 0) prefix sums of floor(len / (64
//                    snap_chunks)): where each sequence's state snapshots go.
struct SlotInfo {
    int64_t t0;
    int32_t len;  // tokens in the chunk (bits 0..15); bit 16: the sequence's first chunk
    int32_t seq;
};
static_assert(sizeof(SlotInfo) == 16, "one 16-byte record per slot");

__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* __restrict__ cu, int N,
                                                         int64_t T, int32_t* __restrict__ base,
                                                         SlotInfo* __restrict__ slot_info, int snap_chunks,
                                                         int32_t* __restrict__ snap_off);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The state passes run one workgroup per (sequence, head, 16-column slice).
// Block b -> (group = sequence * H + head, slice) such that all slices of a
// group share an XCD (workgroups are dealt round-robin over the 8 XCDs), so
// the chunk records they all read go through one L2.  The grid is rounded up
// to whole sets of 8 groups; a block past the last group has grp >= groups.
struct SliceBlock {
    int64_t grp;
    int sl;
};
__device__ __forceinline__ SliceBlock slice_block(int bid, int nsl) {
    const int q = bid >> 3;
    return {static_cast<int64_t>(q / nsl) * 8 + (bid & 7), q % nsl};
}
inline int64_t slice_grid(int64_t groups, int nsl) { return (groups + 7) / 8 * 8 * nsl; }

// Record of one (chunk slot, head) on the fp32 path, offsets in floats:
// W [64][dk], U~ [64][dv], Q' [64][dk], K^ [64][dk], M U~ [64][dv], gamma [dk]
struct GenRec {
    int64_t W, U, Qp, Kh, Oi, gam, size;
};

__host__ __device__ inline GenRec gen_rec(int dk, int dv) {
    GenRec r;
    r.W = 0;
    r.U = r.W + 64 * dk;
    r.Qp = r.U + 64 * dv;
    r.Kh = r.Qp + 64 * dk;
    r.Oi = r.Kh + 64 * dk;
    r.gam = r.Oi + 64 * dv;
    r.size = (r.gam + dk + 63) / 64 * 64;
    return r;
}

inline int64_t chunk_slots_bound(int64_t T, int N) { return (T + kChunk - 1) / kChunk + N; }

inline size_t chunk_map_base_bytes(int N) { return align_up(static_cast<size_t>(N + 1) * 4, 256); }

// base[] then slot_info[] (bounded by the slot count)
inline size_t chunk_map_bytes(int64_t T, int N) {
    return chunk_map_base_bytes(N) + align_up(static_cast<size_t>(chunk_slots_bound(T, N)) * sizeof(SlotInfo), 256);
}

}  // namespace kda
