/*
 * libkda -- the Kimi Delta Attention (KDA) token mixer on AMD Instinct
 * MI355X (gfx950).  Plain C ABI: every tensor argument is a raw device
 * pointer plus sizes; no framework types cross this boundary.
 *
 * What is computed.  KDA is the gated delta-rule linear attention of the page
 * "Ling-3.0-flash: a 124B open MoE that runs like a 5B and reaches for 1M
 * tokens", section "KDA: constant-size memory over a very long context".  Per
 * sequence and head it keeps a fixed dk x dv state S (fp32 here).  For each
 * token t, with alpha_t the per-key-channel decay, beta_t the write strength:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,           y_t = o_t * sigmoid(z_t)  (when a gate is given)
 * (that section's own equation is missing from the page text; this is the
 * update its prose describes: decay as the erase, a delta-rule write, a read
 * with the query).  Before the recurrence q and k pass through a width-4
 * causal short conv and an L2 norm, v through a conv, alpha comes from a
 * softplus gate and beta from a sigmoid (same section; the conv width and the
 * 32 x 128 head shape are in the "Every architecture field" table of the page
 * "Ling 3.0 Flash", llm-architectures-explained).
 *
 * Conventions shared by every call.
 *  - Memory: every tensor pointer is a device pointer on the current HIP
 *    device, owned by the caller.  The library never allocates, frees or
 *    retains caller memory; scratch comes from a caller-provided workspace.
 *  - Layout: tensors are dense, row-major, fastest index last, 16-byte
 *    aligned.  [T, H, d] means token-major, then head, then channel.
 *  - Aliasing: only the recurrent state may alias (final_state may equal
 *    initial_state; the decode state is updated in place).  Any other overlap
 *    is rejected with KDA_ERR_INVALID_ARGUMENT.
 *  - Execution: calls enqueue work on `stream` (a hipStream_t; NULL is the
 *    null stream) and return without synchronising.  Host-side validation
 *    checks sizes, pointers, alignment and dtypes; the contents of cu_seqlens
 *    are trusted (non-decreasing, cu_seqlens[0] = 0, cu_seqlens[N] = T_tot).
 *  - Errors: calls return a status and never abort or throw.  After a non-OK
 *    return, outputs are undefined; kda_last_error_detail() gives a
 *    thread-local sentence naming the failing argument or HIP call.
 *  - Supported shapes: dk, dv in {16, 32, 64, 128}; H >= 1; N >= 1;
 *    T_tot >= 0 and below 2^31; sequences of length 0 are allowed.
 *  - Thread safety: no global mutable state; the error text and the optional
 *    kernel-timing records (kda_profile_enable) are per host thread.
 *  - Types: every call returns a kda_status_t value as a plain int, takes
 *    each dtype as an int32_t holding a kda_dtype_t value, and takes the
 *    stream as a void* holding a hipStream_t.  They are the same bits on the
 *    ABI; plain types keep this header free of the HIP headers, so a caller
 *    can bind it from any language (the Python binding uses ctypes).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,   /* bad size, NULL or misaligned pointer, overlap */
    KDA_ERR_UNSUPPORTED = 2,        /* valid request this build does not implement */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} kda_status_t;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype_t;

/* Static text for a status code; never NULL. */
const char* kda_status_string(int status);

/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* kda_last_error_detail(void);

/* ABI version of this header (major * 100 + minor). */
int kda_abi_version(void);

/*
 * kda_preprocess -- fused short conv, L2 norm and gates for a packed batch.
 * These are the steps the section "KDA: constant-size memory over a very
 * long context" of the page "Ling-3.0-flash: a 124B open MoE ..." applies
 * before the recurrence: q and k through a short causal conv and an L2 norm,
 * v through a conv, the decay from a softplus gate and the write strength
 * from a sigmoid (the conv width of 4 is in the "Every architecture field"
 * table of the page "Ling 3.0 Flash").
 *
 * For every sequence n (tokens cu_seqlens[n] .. cu_seqlens[n+1]-1), head h
 * and channel c:
 *   conv:  x~_t[c] = sum_{j=0..3} w[c][j] * x_{t-3+j}[c]   (tap 3 = current
 *          token; no bias, no activation).  Positions before the sequence
 *          start read conv_state[n] (oldest first) if given, else zero.
 *   norm:  q^ = q~ / sqrt(|q~|^2 + 1e-6) over the head's dk channels; same
 *          for k; v^ = v~.
 *   gates: log_alpha = -softplus(g) per key channel; beta = sigmoid(b) per head.
 * Arguments:
 *   T_tot, H, dk, dv     sizes; cu_seqlens: device int32 [N+1], or NULL for a
 *                        single sequence (then N must be 1);
 *   x_dtype              dtype of q_in, k_in, v_in, w_*, g_alpha, b_beta and
 *                        of q_out, k_out, v_out;
 *   q_in, k_in  [T_tot, H*dk];  v_in [T_tot, H*dv]   projected inputs;
 *   w_q, w_k    [H*dk, 4];      w_v  [H*dv, 4]       conv taps;
 *   g_alpha     [T_tot, H*dk]   decay logits;  b_beta [T_tot, H] write logits;
 *   conv_state  NULL, or fp32 [N, 3, H*(2*dk+dv)] (q channels, then k, then v):
 *               read as the history of each sequence, then overwritten with
 *               the last three raw tokens of that sequence (reaching back into
 *               the old history for sequences shorter than three);
 *   q_out, k_out [T_tot, H, dk]; v_out [T_tot, H, dv] (x_dtype);
 *   log_alpha_out fp32 [T_tot, H, dk]; beta_out fp32 [T_tot, H].
 */
int kda_preprocess(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                   const int32_t* cu_seqlens, int32_t N, int32_t x_dtype,
                   const void* q_in, const void* k_in, const void* v_in,
                   const void* w_q, const void* w_k, const void* w_v,
                   const void* g_alpha, const void* b_beta,
                   float* conv_state,
                   void* q_out, void* k_out, void* v_out,
                   float* log_alpha_out, float* beta_out,
                   void* stream);

/*
 * Bytes of workspace kda_prefill_chunked needs for these sizes.  The bound
 * does not depend on the sequence lengths: it counts ceil(T_tot/64) + N
 * chunk slots (each sequence's chunks start at its own first token).
 * Returns 0 for unsupported or invalid sizes.
 */
size_t kda_prefill_workspace_bytes(int64_t T_tot, int32_t N, int32_t H, int32_t dk,
                                   int32_t dv, int32_t x_dtype);

/*
 * kda_prefill_chunked -- the recurrence over a packed batch of preprocessed
 * tokens, in chunks of 64 tokens.  The recurrence is the constant-size state
 * update and query read of the section "KDA: constant-size memory over a very
 * long context" of the page "Ling-3.0-flash: a 124B open MoE ...", with the
 * sigmoid output gate of the same section.  The result is that of the
 * token-by-token recurrence above (chunking changes only rounding): within a chunk the
 * writes are collected into a WY-style form (a unit-lower-triangular solve
 * over the chunk's keys) and the fp32 state is carried across chunks in
 * order, per sequence and head.
 * Arguments:
 *   cu_seqlens  device int32 [N+1], or NULL for a single sequence (N = 1);
 *   x_dtype     dtype of q, k, v, out_gate and out;
 *   gate_dtype  dtype of log_alpha and beta;
 *   q, k        [T_tot, H, dk] (L2-normalised keys keep every write a
 *               contraction);  v [T_tot, H, dv];
 *   log_alpha   [T_tot, H, dk], entries <= 0;  beta [T_tot, H];
 *   out_gate    NULL, or [T_tot, H, dv] logits z: out = o * sigmoid(z);
 *   initial_state NULL (zeros) or fp32 [N, H, dk, dv];
 *   final_state NULL (not wanted) or fp32 [N, H, dk, dv]; may equal
 *               initial_state (then updated in place);
 *   out         [T_tot, H, dv] (x_dtype);
 *   workspace   device scratch of at least kda_prefill_workspace_bytes()
 *               bytes, 256-byte aligned; contents on entry are ignored.
 * Sizes: H x (T_tot/64 + 1 + N) must stay below 2^32 (KDA_ERR_UNSUPPORTED
 * otherwise).
 */
int kda_prefill_chunked(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                        const int32_t* cu_seqlens, int32_t N,
                        int32_t x_dtype, int32_t gate_dtype,
                        const void* q, const void* k, const void* v,
                        const void* log_alpha, const void* beta,
                        const void* out_gate,
                        const float* initial_state, float* final_state,
                        void* out,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * kda_prefill_layer -- kda_preprocess followed by kda_prefill_chunked in one
 * call, for bf16 inputs with dk = dv = 128 (the Ling-shaped heads): the
 * short conv, the L2 norm and the gates run inside the chunk kernel, so the
 * preprocessed q, k, v, log-decay and beta never go through device memory.
 * The result equals the two-call path up to rounding order.
 * Arguments: those of kda_preprocess for the raw inputs (q_in .. b_beta,
 * conv_state: read as the history, then replaced by the last three raw
 * tokens of each sequence) and of kda_prefill_chunked for the rest
 * (out_gate, initial_state, final_state, out, workspace sized by
 * kda_prefill_workspace_bytes with the same sizes).  Other head sizes or
 * dtypes return KDA_ERR_UNSUPPORTED: use the two calls.
 */
int kda_prefill_layer(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                      const int32_t* cu_seqlens, int32_t N, int32_t x_dtype,
                      const void* q_in, const void* k_in, const void* v_in,
                      const void* w_q, const void* w_k, const void* w_v,
                      const void* g_alpha, const void* b_beta,
                      float* conv_state,
                      const void* out_gate,
                      const float* initial_state, float* final_state,
                      void* out,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * kda_prefill_layer_noalloc -- kda_prefill_layer for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  Same computation, arguments and
 * errors as kda_prefill_layer, without the workspace: the call uses a fixed
 * scratch array of KDA_NOALLOC_SCRATCH_BYTES inside the library instead, and
 * allocates nothing (no hipMalloc, hipFree or allocating routine).
 *  - Each GPU the library runs on holds its own copy of the array, from the
 *    library's load until the process ends.  The first call on a device
 *    looks the copy up (no allocation); a caller that captures graphs can
 *    make that first call before capturing (T_tot = 0 is enough).
 *  - Sizes whose kda_prefill_workspace_bytes() exceeds
 *    KDA_NOALLOC_SCRATCH_BYTES are rejected with KDA_ERR_WORKSPACE_TOO_SMALL
 *    before any device work (at H = 32, d = 128, one sequence fits up to
 *    1,536 tokens).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero).  Calls that
 *    overlap on one GPU (two host threads, or two streams) race on it and
 *    give undefined results: serialise them.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_prefill_layer_noalloc(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                              const int32_t* cu_seqlens, int32_t N, int32_t x_dtype,
                              const void* q_in, const void* k_in, const void* v_in,
                              const void* w_q, const void* w_k, const void* w_v,
                              const void* g_alpha, const void* b_beta,
                              float* conv_state,
                              const void* out_gate,
                              const float* initial_state, float* final_state,
                              void* out,
                              void* stream);

/*
 * State snapshots for prefix reuse: kda_prefill_chunked_snap and
 * kda_prefill_layer_snap are kda_prefill_chunked and kda_prefill_layer that
 * also write the state of each sequence after every snap_interval tokens
 * (counted from the sequence's start), so a prefix cache can resume a later
 * request from the longest cached prefix (the prefix caching of the page
 * "Ling-3.0-flash: a 124B open MoE ..."; for KDA the whole per-sequence
 * memory at a prefix is this fixed-size state plus the last three raw
 * tokens, which the caller has).  Snapshot m (m = 1 .. floor(len_n /
 * snap_interval)) of sequence n is the state after its first m *
 * snap_interval tokens (starting from initial_state[n] if given).
 * Extra arguments:
 *   snap_interval  tokens between snapshots, a positive multiple of 64;
 *   snapshots      fp32 [snap_capacity, H, dk, dv]; snapshot m of sequence n
 *                  is row snap_offsets[n] + m - 1;
 *   snap_capacity  rows available, at least T_tot / snap_interval (which
 *                  bounds the total); else KDA_ERR_INVALID_ARGUMENT;
 *   snap_offsets   device int32 [N + 1], written: the exclusive prefix sums
 *                  of floor(len_n / snap_interval); snap_offsets[N] = total.
 * The computation and every other output are those of the plain call.
 */
int kda_prefill_chunked_snap(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                             const int32_t* cu_seqlens, int32_t N,
                             int32_t x_dtype, int32_t gate_dtype,
                             const void* q, const void* k, const void* v,
                             const void* log_alpha, const void* beta,
                             const void* out_gate,
                             const float* initial_state, float* final_state,
                             void* out,
                             void* workspace, size_t workspace_bytes,
                             int32_t snap_interval, float* snapshots,
                             int64_t snap_capacity, int32_t* snap_offsets,
                             void* stream);
int kda_prefill_layer_snap(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                           const int32_t* cu_seqlens, int32_t N, int32_t x_dtype,
                           const void* q_in, const void* k_in, const void* v_in,
                           const void* w_q, const void* w_k, const void* w_v,
                           const void* g_alpha, const void* b_beta,
                           float* conv_state,
                           const void* out_gate,
                           const float* initial_state, float* final_state,
                           void* out,
                           void* workspace, size_t workspace_bytes,
                           int32_t snap_interval, float* snapshots,
                           int64_t snap_capacity, int32_t* snap_offsets,
                           void* stream);

/*
 * Gradients of kda_prefill_chunked (training).  For a loss whose gradients
 * with respect to the outputs y and the final states are dy and dS_final,
 * returns the gradients with respect to every input of the recurrence: q, k,
 * v, log_alpha, beta, the output-gate logits and the initial states.  They
 * are the adjoint of the chunked form (the recurrence of the section "KDA:
 * constant-size memory over a very long context" of the page "Ling-3.0-flash:
 * a 124B open MoE ..."; the pages train KDA from the first step), computed in
 * three passes: the forward again with the state kept at every chunk start,
 * the state gradient carried backwards over each sequence's chunks, and every
 * other gradient per chunk in parallel.  The gradient of the decay logits g
 * follows as dlog_alpha * -sigmoid(g), since log_alpha = -softplus(g).
 * Arguments: those of kda_prefill_chunked (any supported head size, both
 * dtypes; the output and final state are not recomputed), plus
 *   dy            [T_tot, H, dv] (x_dtype);
 *   dS_final      NULL (zero) or fp32 [N, H, dk, dv];
 *   grad_q, grad_k, grad_log_alpha [T_tot, H, dk], grad_v [T_tot, H, dv],
 *   grad_beta [T_tot, H]: fp32 outputs;
 *   grad_out_gate fp32 [T_tot, H, dv], required exactly when out_gate is given;
 *   grad_initial_state  NULL or fp32 [N, H, dk, dv].
 *   workspace     at least kda_backward_workspace_bytes(T_tot, N, H, dk, dv)
 *                 bytes, 256-byte aligned.
 */
size_t kda_backward_workspace_bytes(int64_t T_tot, int32_t N, int32_t H,
                                    int32_t dk, int32_t dv);
int kda_prefill_backward(int64_t T_tot, int32_t H, int32_t dk, int32_t dv,
                         const int32_t* cu_seqlens, int32_t N,
                         int32_t x_dtype, int32_t gate_dtype,
                         const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta,
                         const void* out_gate,
                         const float* initial_state,
                         const void* dy, const float* dS_final,
                         float* grad_q, float* grad_k, float* grad_v,
                         float* grad_log_alpha, float* grad_beta,
                         float* grad_out_gate, float* grad_initial_state,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * kda_decode_step -- one token per sequence, state updated in place: the
 * decode-time form of the recurrence of the section "KDA: constant-size
 * memory over a very long context" of the page "Ling-3.0-flash: a 124B open
 * MoE ..." (each new token costs the same fixed state read and write,
 * whatever the context length).
 * For each (b, h):  S' = Diag(alpha) S;  u = S'^T k;  S <- S' + beta k (v - u)^T;
 *                   o = S^T q;  out = o * sigmoid(z) (or o without a gate).
 * The state is read once and written once.
 * Arguments:
 *   q, k [B, H, dk], v [B, H, dv] (x_dtype), preprocessed;
 *   log_alpha [B, H, dk], beta [B, H] (gate_dtype);
 *   out_gate NULL or [B, H, dv] logits (x_dtype);
 *   state fp32 [B, H, dk, dv], in place;  out [B, H, dv] (x_dtype).
 */
int kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv,
                    int32_t x_dtype, int32_t gate_dtype,
                    const void* q, const void* k, const void* v,
                    const void* log_alpha, const void* beta,
                    const void* out_gate,
                    float* state, void* out,
                    void* stream);

/*
 * kda_decode_layer -- one token per sequence through the whole token mixer:
 * kda_preprocess for that token (conv against the caller's conv history, L2
 * norm, gates) fused with kda_decode_step, so a serving loop makes one call
 * per layer and token.  The preprocessed q, k, v are rounded to x_dtype
 * before the step (as kda_preprocess stores them); the gates stay fp32.
 * The result equals kda_preprocess (T_tot = B, N = B, cu_seqlens = 0..B)
 * followed by kda_decode_step with gate_dtype KDA_F32, up to rounding order.
 * States live in a pool: sequence b uses row state_indices[b] of state and
 * of conv_state (row b when state_indices is NULL, then state_slots must be
 * B).  This is the decode-time form of the recurrence and the conv in the
 * section "KDA: constant-size memory over a very long context" of the page
 * "Ling-3.0-flash: a 124B open MoE ...".
 * Arguments:
 *   q_in, k_in [B, H, dk], v_in [B, H, dv], g_alpha [B, H, dk], b_beta [B, H]
 *                 raw projections and gate logits of the new token (x_dtype);
 *   w_q, w_k [H*dk, 4], w_v [H*dv, 4]   conv taps (x_dtype), as kda_preprocess;
 *   conv_state    fp32 [state_slots, 3, H*(2*dk + dv)]: per slot the last
 *                 three raw tokens (oldest first; q, then k, then v columns),
 *                 the layout kda_preprocess reads and writes; rolled forward
 *                 by one token in place;
 *   out_gate      NULL or [B, H, dv] logits (x_dtype);
 *   state         fp32 [state_slots, H, dk, dv], updated in place;
 *   state_slots   rows in the two pools (>= 0);
 *   state_indices NULL or device int32 [B].  An entry outside
 *                 [0, state_slots) marks a padding row: its out row is set to
 *                 zero and no state is read or written.  Valid entries must be
 *                 distinct (two rows on one slot race); with the environment
 *                 variable KDA_DEBUG_CHECK=1 the call copies the indices to the
 *                 host, synchronising the stream, and rejects duplicates;
 *   out           [B, H, dv] (x_dtype).
 * Pool rows that no valid entry names are neither read nor written.
 */
int kda_decode_layer(int32_t B, int32_t H, int32_t dk, int32_t dv,
                     int32_t x_dtype,
                     const void* q_in, const void* k_in, const void* v_in,
                     const void* w_q, const void* w_k, const void* w_v,
                     const void* g_alpha, const void* b_beta,
                     float* conv_state,
                     const void* out_gate,
                     float* state, int32_t state_slots,
                     const int32_t* state_indices,
                     void* out,
                     void* stream);

/*
 * Speculative decoding: verify 1 + n draft tokens per sequence, commit later.
 *
 * The decoding on the page "Ling-3.0-flash: a 124B open MoE ..." proposes
 * three draft tokens per step (multi-token prediction) and verifies them in
 * one pass; how many are accepted is known only after that pass.  Each call
 * of kda_spec_verify, per sequence b and its pool row s = state_indices[b]:
 *   1. commits: the first accepted[b] tokens of the previous call on slot s
 *      (kept raw in the draft buffer) go through the conv (against the
 *      slot's conv history), the L2 norm, the gates and the recurrence, as
 *      kda_decode_layer would run them one by one; the slot's state and conv
 *      history are written back, holding those tokens;
 *   2. verifies: the T new raw tokens run from that state in order (token t's
 *      output reads the state after tokens 0..t), and their outputs are
 *      written; the state and conv history are NOT advanced by them.  Their
 *      raw values replace the slot's draft buffer, for the next call to commit.
 * So each call reads and writes the state once.  A call with T = 0 only
 * commits (use it to bring a slot up to date, e.g. when a sequence leaves
 * speculative mode).  The recurrence is that of kda_decode_step (section
 * "KDA: constant-size memory over a very long context" of the same page).
 * Arguments:
 *   B, T          sequences and new tokens per sequence (0 <= T <= 8);
 *   q_in, k_in [B, T, H, dk], v_in [B, T, H, dv], g_alpha [B, T, H, dk],
 *   b_beta [B, T, H]   raw projections and gate logits (x_dtype);
 *   w_q, w_k, w_v, conv_state, state, state_slots, state_indices
 *                 as for kda_decode_layer (pools of state_slots rows);
 *   out_gate      NULL or [B, T, H, dv] (x_dtype);
 *   accepted      NULL (commit nothing) or device int32 [B]: how many of the
 *                 previous call's tokens on that slot to commit, in
 *                 [0, that call's T]; values are clamped to [0, 8], and a
 *                 count above the previous T commits stale buffer contents;
 *   drafts        per slot kda_spec_draft_bytes(H, dk, dv, x_dtype) bytes
 *                 of device memory, owned by the caller, opaque (raw tokens
 *                 of the last call, in x_dtype: every call on one buffer
 *                 must use the same x_dtype, a commit-only call included);
 *                 contents matter only where accepted > 0;
 *   out           [B, T, H, dv] (x_dtype).
 * Padding rows (index outside the pool) get zero outputs and touch nothing.
 * A row with accepted = 0 and T = 0 is a no-op.
 */
size_t kda_spec_draft_bytes(int32_t H, int32_t dk, int32_t dv, int32_t x_dtype);
int kda_spec_verify(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                    int32_t x_dtype,
                    const void* q_in, const void* k_in, const void* v_in,
                    const void* w_q, const void* w_k, const void* w_v,
                    const void* g_alpha, const void* b_beta,
                    float* conv_state,
                    const void* out_gate,
                    float* state, int32_t state_slots,
                    const int32_t* state_indices,
                    const int32_t* accepted,
                    void* drafts,
                    void* out,
                    void* stream);

/*
 * Kernel timing for profiling tools (not needed for normal use).
 * kda_profile_enable(1) makes every later call on the calling host thread
 * bracket each kernel it launches with a pair of HIP events recorded on the
 * call's stream; kda_profile_enable(0) stops it.  kda_profile_collect()
 * waits for the recorded events, sums them per kernel name since the last
 * collect, writes at most max_entries records to `out` and returns the number
 * of distinct kernels (or -KDA_ERR_HIP if an event failed).  Event objects
 * are pooled per thread; no device memory is allocated.
 */
typedef struct kda_kernel_time {
    char name[48];
    int64_t launches;
    double total_ms;
} kda_kernel_time_t;

int kda_profile_enable(int on);
int kda_profile_collect(kda_kernel_time_t* out, int max_entries);

/*
 * Peak-rate probes for measurement tools (not part of the token mixer): what
 * this device sustains, to report beside the published peaks.  Launches
 * `blocks` workgroups of 256 threads on `stream`:
 *   kind 0  each wave issues iters x 4 bf16 matrix-core products of
 *           16 x 16 x 32 (16,384 flops each): blocks * 4 * iters * 4 * 16384
 *           flops in all;
 *   kind 1  the same with fp32 products of 16 x 16 x 4 (2,048 flops each);
 *   kind 2  reads src_bytes (a multiple of 16, 16-byte aligned device memory
 *           at src) once, grid-stride.
 * out: device fp32 [blocks * 256], written (a checksum per thread).  Returns
 * KDA_ERR_INVALID_ARGUMENT for bad arguments.  The launch is timed by
 * kda_profile_enable like any kernel of the library ("probe_mfma_bf16",
 * "probe_mfma_f32", "probe_read").
 */
int kda_probe_peak(int32_t kind, int32_t blocks, int32_t iters, const void* src, int64_t src_bytes,
                   float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
