// Host-side interface between the C ABI layer (kda_api.hip) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum class DT : int { F32 = 0, BF16 = 1 };

// Optional state snapshots from the prefill: the state after every
// `chunks` * 64 tokens of each sequence (counted from its start), written to
// out[(off[n] + m - 1), h] for the m-th snapshot of sequence n.  off[n] is
// filled by the chunk map (an exclusive scan of floor(len_n / (64 chunks))),
// off[N] = the total.
struct Snapshots {
    int chunks = 0;  // 0: none
    float* out = nullptr;
    int32_t* off = nullptr;
};

struct PreprocessArgs {
    int64_t T;
    int H, dk, dv, N;
    const int32_t* cu;  // never NULL here (the ABI layer substitutes a one-sequence map)
    DT x;
    const void *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b;
    float* conv_state;
    void *q_out, *k_out, *v_out;
    float *la_out, *beta_out;
};

struct PrefillArgs {
    int64_t T;
    int H, dk, dv, N;
    const int32_t* cu;  // may be NULL: one sequence [0, T)
    DT x, gate;
    const void *q, *k, *v, *la, *beta, *z;
    const float* S0;
    float* S_out;
    void* out;
    void* ws;
    size_t ws_bytes;
    Snapshots snap;
};

struct DecodeArgs {
    int B, H, dk, dv;
    DT x, gate;
    const void *q, *k, *v, *la, *beta, *z;
    float* state;
    void* out;
};

// One decode token per sequence with its preprocess fused in: raw q/k/v
// projections, conv taps and gate logits in the input type; fp32 gates made
// inside.  state and conv_state are pools of `slots` rows, row state_indices[b]
// (b itself when state_indices is NULL) belonging to sequence b.
struct DecodeLayerArgs {
    int B, H, dk, dv;
    DT x;
    const void *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b, *z;
    float* conv_state;
    float* state;
    int slots;
    const int32_t* state_indices;
    void* out;
};

// Speculative verify with a deferred commit: `accepted[b]` (NULL: 0) tokens of
// the previous call, kept raw in the draft buffer, are committed to the state
// and conv history of slot state_indices[b]; then T new raw tokens are run
// from that state (outputs only) and saved to the draft buffer.
constexpr int kSpecMaxTokens = 8;
// elements per (slot, token, head) in the draft buffer: raw q, k, v, decay
// logits, then the write logit, padded to 16 bytes
constexpr int spec_draft_width(int dk, int dv) { return 3 * dk + dv + 8; }
struct SpecArgs {
    int B, H, dk, dv, T;
    DT x;
    const void *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b, *z;
    float* conv_state;
    float* state;
    int slots;
    const int32_t* state_indices;
    const int32_t* accepted;
    void* drafts;
    void* out;
};

// The whole layer (preprocess + chunked prefill) with the preprocess fused
// into the chunk kernel; bf16 inputs, dk = dv = 128.
struct LayerArgs {
    int64_t T;
    int H, dk, dv, N;
    const int32_t* cu;  // may be NULL: one sequence [0, T)
    const void *q_in, *k_in, *v_in, *w_q, *w_k, *w_v, *g, *b, *z;
    float* conv_state;
    const float* S0;
    float* S_out;
    void* out;
    void* ws;
    size_t ws_bytes;
    Snapshots snap;
};

hipError_t launch_preprocess(const PreprocessArgs& a, hipStream_t s);
// only the rewrite of the conv history after a call (the last three raw tokens)
hipError_t launch_conv_state_update(const PreprocessArgs& a, hipStream_t s);
bool layer_fused_supported(int dk, int dv, DT x);
hipError_t launch_layer(const LayerArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_layer(const DecodeLayerArgs& a, hipStream_t s);
hipError_t launch_spec_verify(const SpecArgs& a, hipStream_t s);

// Gradients of the chunked recurrence: everything kda_prefill_chunked takes,
// the output and final-state gradients, and where the input gradients go
// (all fp32).  dz only with z; dS0 may be NULL.
struct BackwardArgs {
    PrefillArgs f;  // the forward call's arguments (out, S_out unused)
    const void* dy;  // [T, H, dv], x dtype
    const float* dS_final;  // NULL: zero
    float *dq, *dk, *dv, *dla, *dbeta, *dz, *dS0;
};
size_t backward_workspace_bytes(int64_t T, int N, int H, int dk, int dv);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
// the fp32 chunked forward alone (phase 1 records, phase 2 state pass), and
// its state pass alone over records already made
hipError_t launch_gen_forward(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec);
hipError_t launch_gen_state(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec);
// the fp32 path's chunk records (phase 1) alone
hipError_t launch_chunk_records(const PrefillArgs& a, hipStream_t s, const int32_t* base, float* rec);

// chunked prefill: workspace layout and the two implementations
bool prefill_uses_mfma(int dk, int dv, DT x);
size_t prefill_workspace_bytes(int64_t T, int N, int H, int dk, int dv, DT x);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

}  // namespace kda
