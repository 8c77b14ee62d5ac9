// C ABI of libkda: argument validation, status codes and dispatch to the
// kernels.  See include/kda.h for the contract of every entry point.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_detail[0] = '\0';
    return KDA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(KDA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

bool valid_head_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_dtype(int32_t t) { return t == KDA_F32 || t == KDA_BF16; }
size_t dsize(int32_t t) { return t == KDA_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const char* name;
    const void* p;
    size_t bytes;
    bool writes;
};

// Rejects NULL/misaligned pointers and any overlap that involves a written
// buffer (read-only inputs may share memory with each other).
int check_spans(const std::vector<Span>& v) {
    for (const Span& s : v) {
        if (s.bytes == 0) continue;
        if (s.p == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", s.name);
        if (!aligned16(s.p)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", s.name);
    }
    for (size_t i = 0; i < v.size(); ++i) {
        for (size_t j = i + 1; j < v.size(); ++j) {
            const Span &a = v[i], &b = v[j];
            if (a.bytes == 0 || b.bytes == 0 || !(a.writes || b.writes)) continue;
            const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
            if (a0 < b0 + b.bytes && b0 < a0 + a.bytes)
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", a.name, b.name);
        }
    }
    return KDA_OK;
}

int check_sizes(int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t N) {
    if (T < 0 || T >= (int64_t(1) << 31)) return fail(KDA_ERR_INVALID_ARGUMENT, "T_tot=%lld out of range [0, 2^31)", (long long)T);
    if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H=%d out of range [1, 65535]", H);
    if (N < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "N=%d must be >= 1", N);
    if (!valid_head_dim(dk) || !valid_head_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head sizes are 16, 32, 64, 128", dk, dv);
    return KDA_OK;
}

// Optional host-side check of cu_seqlens contents (synchronises the stream).
int debug_check_cu(const int32_t* cu, int32_t N, int64_t T, hipStream_t s) {
    const char* env = getenv("KDA_DEBUG_CHECK");
    if (cu == nullptr || env == nullptr || strcmp(env, "1") != 0) return KDA_OK;
    std::vector<int32_t> h(static_cast<size_t>(N) + 1);
    hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "copy of cu_seqlens for KDA_DEBUG_CHECK");
    if (h[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0]=%d, expected 0", h[0]);
    for (int32_t n = 0; n < N; ++n)
        if (h[n + 1] < h[n]) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d", n);
    if (h[N] != T) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[N]=%d, expected T_tot=%lld", h[N], (long long)T);
    return KDA_OK;
}

// Optional host-side check that the valid entries of state_indices are
// distinct (synchronises the stream).
int debug_check_indices(const int32_t* idx, int32_t B, int32_t slots, hipStream_t s) {
    const char* env = getenv("KDA_DEBUG_CHECK");
    if (idx == nullptr || B == 0 || env == nullptr || strcmp(env, "1") != 0) return KDA_OK;
    std::vector<int32_t> h(static_cast<size_t>(B));
    hipError_t e = hipMemcpyAsync(h.data(), idx, h.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "copy of state_indices for KDA_DEBUG_CHECK");
    std::vector<int32_t> seen(static_cast<size_t>(slots), -1);
    for (int32_t b = 0; b < B; ++b) {
        const int32_t i = h[b];
        if (i < 0 || i >= slots) continue;
        if (seen[i] >= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices[%d] = state_indices[%d] = %d", seen[i], b, i);
        seen[i] = b;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        default: return "KDA_ERR_UNKNOWN";
    }
}

const char* kda_last_error_detail(void) { return g_detail; }

int kda_abi_version(void) { return 104; }

int kda_preprocess(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                   int32_t x_dtype, const void* q_in, const void* k_in, const void* v_in, const void* w_q,
                   const void* w_k, const void* w_v, const void* g_alpha, const void* b_beta,
                   float* conv_state, void* q_out, void* k_out, void* v_out, float* log_alpha_out,
                   float* beta_out, void* stream) {
    int st = check_sizes(T_tot, H, dk, dv, N);
    if (st != KDA_OK) return st;
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (cu_seqlens == nullptr && N != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but N=%d", N);
    const size_t xs = dsize(x_dtype);
    const size_t T = static_cast<size_t>(T_tot);
    const size_t qk = T * H * dk, vv = T * H * dv;
    const size_t cs_bytes = conv_state ? static_cast<size_t>(N) * 3 * H * (2 * dk + dv) * 4 : 0;
    std::vector<Span> sp = {
        {"q_in", q_in, qk * xs, false}, {"k_in", k_in, qk * xs, false}, {"v_in", v_in, vv * xs, false},
        {"w_q", w_q, static_cast<size_t>(H) * dk * 4 * xs, false},
        {"w_k", w_k, static_cast<size_t>(H) * dk * 4 * xs, false},
        {"w_v", w_v, static_cast<size_t>(H) * dv * 4 * xs, false},
        {"g_alpha", g_alpha, qk * xs, false}, {"b_beta", b_beta, T * H * xs, false},
        {"conv_state", conv_state, cs_bytes, true},
        {"q_out", q_out, qk * xs, true}, {"k_out", k_out, qk * xs, true}, {"v_out", v_out, vv * xs, true},
        {"log_alpha_out", log_alpha_out, qk * 4, true}, {"beta_out", beta_out, T * H * 4, true},
    };
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    // b_beta rows are H elements: only the base needs 16-byte alignment when H*xs is a multiple of 16;
    // the kernel reads it one element at a time, so relax the check to element alignment.
    sp[7].bytes = 0;
    if (T * H > 0 && (b_beta == nullptr || (reinterpret_cast<uintptr_t>(b_beta) % xs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "b_beta is NULL or misaligned");
    st = check_spans(sp);
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu(cu_seqlens, N, T_tot, s);
    if (st != KDA_OK) return st;
    kda::PreprocessArgs a;
    a.T = T_tot; a.H = H; a.dk = dk; a.dv = dv; a.N = N; a.cu = cu_seqlens;
    a.x = static_cast<kda::DT>(x_dtype);
    a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.w_q = w_q; a.w_k = w_k; a.w_v = w_v;
    a.g = g_alpha; a.b = b_beta; a.conv_state = conv_state;
    a.q_out = q_out; a.k_out = k_out; a.v_out = v_out; a.la_out = log_alpha_out; a.beta_out = beta_out;
    hipError_t e = kda::launch_preprocess(a, s);
    if (e != hipSuccess) return hip_fail(e, "preprocess launch");
    return ok();
}

size_t kda_prefill_workspace_bytes(int64_t T_tot, int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t x_dtype) {
    if (T_tot < 0 || T_tot >= (int64_t(1) << 31) || N < 1 || H < 1 || H > 65535 || !valid_head_dim(dk) ||
        !valid_head_dim(dv) || !valid_dtype(x_dtype))
        return 0;
    return kda::prefill_workspace_bytes(T_tot, N, H, dk, dv, static_cast<kda::DT>(x_dtype));
}

}  // extern "C"

namespace {

// A request for state snapshots from the prefill (the *_snap entry points).
struct SnapReq {
    int32_t interval;
    float* out;
    int64_t capacity;
    int32_t* offsets;
};

// Validates a snapshot request and adds its outputs to the overlap check.
int check_snap(const SnapReq* r, int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, std::vector<Span>& sp,
               kda::Snapshots& out) {
    out = kda::Snapshots{};
    if (r == nullptr) return KDA_OK;
    if (r->interval < 64 || r->interval % 64 != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "snap_interval=%d is not a positive multiple of 64", r->interval);
    const int64_t most = T / r->interval;  // sum over sequences of floor(len / interval) is at most this
    if (r->capacity < most)
        return fail(KDA_ERR_INVALID_ARGUMENT, "snap_capacity=%lld < T_tot / snap_interval = %lld",
                    static_cast<long long>(r->capacity), static_cast<long long>(most));
    sp.push_back({"snapshots", r->out, static_cast<size_t>(most) * H * dk * dv * 4, true});
    sp.push_back({"snap_offsets", r->offsets, static_cast<size_t>(N + 1) * 4, true});
    out.chunks = r->interval / 64;
    out.out = r->out;
    out.off = r->offsets;
    return KDA_OK;
}

int prefill_chunked_impl(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                         int32_t x_dtype, int32_t gate_dtype, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const void* out_gate,
                         const float* initial_state, float* final_state, void* out, void* workspace,
                         size_t workspace_bytes, void* stream, const SnapReq* snap) {
    int st = check_sizes(T_tot, H, dk, dv, N);
    if (st != KDA_OK) return st;
    if ((T_tot / 64 + 1 + N) * static_cast<int64_t>(H) > 0xffffffffll)
        return fail(KDA_ERR_UNSUPPORTED, "H x (T_tot/64 + N) = %lld chunk units exceed 2^32 - 1",
                    static_cast<long long>((T_tot / 64 + 1 + N) * static_cast<int64_t>(H)));
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (!valid_dtype(gate_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "gate_dtype=%d is not KDA_F32 or KDA_BF16", gate_dtype);
    if (cu_seqlens == nullptr && N != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but N=%d", N);
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    const size_t need = kda_prefill_workspace_bytes(T_tot, N, H, dk, dv, x_dtype);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL or not 256-byte aligned");
    const size_t xs = dsize(x_dtype), gs = dsize(gate_dtype);
    const size_t T = static_cast<size_t>(T_tot);
    const size_t qk = T * H * dk, vv = T * H * dv;
    const size_t state = static_cast<size_t>(N) * H * dk * dv * 4;
    if (final_state != nullptr && initial_state != nullptr && final_state != initial_state) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(initial_state), b0 = reinterpret_cast<uintptr_t>(final_state);
        if (a0 < b0 + state && b0 < a0 + state)
            return fail(KDA_ERR_INVALID_ARGUMENT, "final_state partially overlaps initial_state");
    }
    std::vector<Span> sp = {
        {"q", q, qk * xs, false}, {"k", k, qk * xs, false}, {"v", v, vv * xs, false},
        {"log_alpha", log_alpha, qk * gs, false},
        {"out_gate", out_gate, out_gate ? vv * xs : 0, false},
        {"initial_state", initial_state, (initial_state && initial_state != final_state) ? state : 0, false},
        {"final_state", final_state, final_state ? state : 0, true},
        {"out", out, vv * xs, true},
        {"workspace", workspace, need, true},
    };
    kda::Snapshots snaps;
    st = check_snap(snap, T_tot, N, H, dk, dv, sp, snaps);
    if (st != KDA_OK) return st;
    st = check_spans(sp);
    if (st != KDA_OK) return st;
    if (T * H > 0 && (beta == nullptr || (reinterpret_cast<uintptr_t>(beta) % gs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "beta is NULL or misaligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu(cu_seqlens, N, T_tot, s);
    if (st != KDA_OK) return st;
    kda::PrefillArgs a;
    a.T = T_tot; a.H = H; a.dk = dk; a.dv = dv; a.N = N; a.cu = cu_seqlens;
    a.x = static_cast<kda::DT>(x_dtype); a.gate = static_cast<kda::DT>(gate_dtype);
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.z = out_gate;
    a.S0 = initial_state; a.S_out = final_state; a.out = out; a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.snap = snaps;
    hipError_t e = kda::launch_prefill(a, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

int prefill_layer_impl(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                       int32_t x_dtype, const void* q_in, const void* k_in, const void* v_in, const void* w_q,
                       const void* w_k, const void* w_v, const void* g_alpha, const void* b_beta,
                       float* conv_state, const void* out_gate, const float* initial_state, float* final_state,
                       void* out, void* workspace, size_t workspace_bytes, void* stream, const SnapReq* snap) {
    int st = check_sizes(T_tot, H, dk, dv, N);
    if (st != KDA_OK) return st;
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (!kda::layer_fused_supported(dk, dv, static_cast<kda::DT>(x_dtype)))
        return fail(KDA_ERR_UNSUPPORTED, "kda_prefill_layer covers dk = dv = 128 with bf16 inputs (got dk=%d, dv=%d, "
                    "x_dtype=%d); use kda_preprocess + kda_prefill_chunked", dk, dv, x_dtype);
    if ((T_tot / 64 + 1 + N) * static_cast<int64_t>(H) > 0xffffffffll)
        return fail(KDA_ERR_UNSUPPORTED, "H x (T_tot/64 + N) = %lld chunk units exceed 2^32 - 1",
                    static_cast<long long>((T_tot / 64 + 1 + N) * static_cast<int64_t>(H)));
    if (cu_seqlens == nullptr && N != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but N=%d", N);
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    const size_t need = kda_prefill_workspace_bytes(T_tot, N, H, dk, dv, x_dtype);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL or not 256-byte aligned");
    const size_t xs = dsize(x_dtype);
    const size_t T = static_cast<size_t>(T_tot);
    const size_t qk = T * H * dk, vv = T * H * dv;
    const size_t state = static_cast<size_t>(N) * H * dk * dv * 4;
    const size_t cs_bytes = conv_state ? static_cast<size_t>(N) * 3 * H * (2 * dk + dv) * 4 : 0;
    if (final_state != nullptr && initial_state != nullptr && final_state != initial_state) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(initial_state), b0 = reinterpret_cast<uintptr_t>(final_state);
        if (a0 < b0 + state && b0 < a0 + state)
            return fail(KDA_ERR_INVALID_ARGUMENT, "final_state partially overlaps initial_state");
    }
    std::vector<Span> sp = {
        {"q_in", q_in, qk * xs, false}, {"k_in", k_in, qk * xs, false}, {"v_in", v_in, vv * xs, false},
        {"w_q", w_q, static_cast<size_t>(H) * dk * 4 * xs, false},
        {"w_k", w_k, static_cast<size_t>(H) * dk * 4 * xs, false},
        {"w_v", w_v, static_cast<size_t>(H) * dv * 4 * xs, false},
        {"g_alpha", g_alpha, qk * xs, false},
        {"conv_state", conv_state, cs_bytes, true},
        {"out_gate", out_gate, out_gate ? vv * xs : 0, false},
        {"initial_state", initial_state, (initial_state && initial_state != final_state) ? state : 0, false},
        {"final_state", final_state, final_state ? state : 0, true},
        {"out", out, vv * xs, true},
        {"workspace", workspace, need, true},
    };
    kda::Snapshots snaps;
    st = check_snap(snap, T_tot, N, H, dk, dv, sp, snaps);
    if (st != KDA_OK) return st;
    st = check_spans(sp);
    if (st != KDA_OK) return st;
    // b_beta rows are H elements, read one at a time: element alignment suffices
    if (T * H > 0 && (b_beta == nullptr || (reinterpret_cast<uintptr_t>(b_beta) % xs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "b_beta is NULL or misaligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu(cu_seqlens, N, T_tot, s);
    if (st != KDA_OK) return st;
    kda::LayerArgs a{};
    a.T = T_tot; a.H = H; a.dk = dk; a.dv = dv; a.N = N; a.cu = cu_seqlens;
    a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.w_q = w_q; a.w_k = w_k; a.w_v = w_v;
    a.g = g_alpha; a.b = b_beta; a.z = out_gate; a.conv_state = conv_state;
    a.S0 = initial_state; a.S_out = final_state; a.out = out; a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.snap = snaps;
    hipError_t e = kda::launch_layer(a, s);
    if (e != hipSuccess) return hip_fail(e, "layer launch");
    return ok();
}

}  // namespace

extern "C" {

int kda_prefill_chunked(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                        int32_t x_dtype, int32_t gate_dtype, const void* q, const void* k, const void* v,
                        const void* log_alpha, const void* beta, const void* out_gate,
                        const float* initial_state, float* final_state, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return prefill_chunked_impl(T_tot, H, dk, dv, cu_seqlens, N, x_dtype, gate_dtype, q, k, v, log_alpha, beta,
                                out_gate, initial_state, final_state, out, workspace, workspace_bytes, stream,
                                nullptr);
}

int kda_prefill_chunked_snap(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens,
                             int32_t N, int32_t x_dtype, int32_t gate_dtype, const void* q, const void* k,
                             const void* v, const void* log_alpha, const void* beta, const void* out_gate,
                             const float* initial_state, float* final_state, void* out, void* workspace,
                             size_t workspace_bytes, int32_t snap_interval, float* snapshots,
                             int64_t snap_capacity, int32_t* snap_offsets, void* stream) {
    const SnapReq r{snap_interval, snapshots, snap_capacity, snap_offsets};
    return prefill_chunked_impl(T_tot, H, dk, dv, cu_seqlens, N, x_dtype, gate_dtype, q, k, v, log_alpha, beta,
                                out_gate, initial_state, final_state, out, workspace, workspace_bytes, stream, &r);
}

int kda_prefill_layer(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                      int32_t x_dtype, const void* q_in, const void* k_in, const void* v_in, const void* w_q,
                      const void* w_k, const void* w_v, const void* g_alpha, const void* b_beta,
                      float* conv_state, const void* out_gate, const float* initial_state, float* final_state,
                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_layer_impl(T_tot, H, dk, dv, cu_seqlens, N, x_dtype, q_in, k_in, v_in, w_q, w_k, w_v, g_alpha,
                              b_beta, conv_state, out_gate, initial_state, final_state, out, workspace,
                              workspace_bytes, stream, nullptr);
}

int kda_prefill_layer_snap(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                           int32_t x_dtype, const void* q_in, const void* k_in, const void* v_in, const void* w_q,
                           const void* w_k, const void* w_v, const void* g_alpha, const void* b_beta,
                           float* conv_state, const void* out_gate, const float* initial_state,
                           float* final_state, void* out, void* workspace, size_t workspace_bytes,
                           int32_t snap_interval, float* snapshots, int64_t snap_capacity,
                           int32_t* snap_offsets, void* stream) {
    const SnapReq r{snap_interval, snapshots, snap_capacity, snap_offsets};
    return prefill_layer_impl(T_tot, H, dk, dv, cu_seqlens, N, x_dtype, q_in, k_in, v_in, w_q, w_k, w_v, g_alpha,
                              b_beta, conv_state, out_gate, initial_state, final_state, out, workspace,
                              workspace_bytes, stream, &r);
}

int kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t x_dtype, int32_t gate_dtype,
                    const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                    const void* out_gate, float* state, void* out, void* stream) {
    if (B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
    if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H=%d out of range [1, 65535]", H);
    if (!valid_head_dim(dk) || !valid_head_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head sizes are 16, 32, 64, 128", dk, dv);
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (!valid_dtype(gate_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "gate_dtype=%d is not KDA_F32 or KDA_BF16", gate_dtype);
    if (static_cast<int64_t>(B) * H >= (int64_t(1) << 31)) return fail(KDA_ERR_INVALID_ARGUMENT, "B*H too large");
    const size_t xs = dsize(x_dtype), gs = dsize(gate_dtype);
    const size_t BH = static_cast<size_t>(B) * H;
    std::vector<Span> sp = {
        {"q", q, BH * dk * xs, false}, {"k", k, BH * dk * xs, false}, {"v", v, BH * dv * xs, false},
        {"log_alpha", log_alpha, BH * dk * gs, false},
        {"out_gate", out_gate, out_gate ? BH * dv * xs : 0, false},
        {"state", state, BH * dk * dv * 4, true},
        {"out", out, BH * dv * xs, true},
    };
    int st = check_spans(sp);
    if (st != KDA_OK) return st;
    if (BH > 0 && (beta == nullptr || (reinterpret_cast<uintptr_t>(beta) % gs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "beta is NULL or misaligned");
    kda::DecodeArgs a;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv;
    a.x = static_cast<kda::DT>(x_dtype); a.gate = static_cast<kda::DT>(gate_dtype);
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.z = out_gate; a.state = state; a.out = out;
    hipError_t e = kda::launch_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

int kda_decode_layer(int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t x_dtype, const void* q_in,
                     const void* k_in, const void* v_in, const void* w_q, const void* w_k, const void* w_v,
                     const void* g_alpha, const void* b_beta, float* conv_state, const void* out_gate,
                     float* state, int32_t state_slots, const int32_t* state_indices, void* out, void* stream) {
    if (B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
    if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H=%d out of range [1, 65535]", H);
    if (!valid_head_dim(dk) || !valid_head_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head sizes are 16, 32, 64, 128", dk, dv);
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (static_cast<int64_t>(B) * H >= (int64_t(1) << 31)) return fail(KDA_ERR_INVALID_ARGUMENT, "B*H too large");
    if (state_indices == nullptr && state_slots != B)
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices is NULL but state_slots=%d != B=%d", state_slots, B);
    if (state_slots < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "state_slots=%d must be >= 0", state_slots);
    if (static_cast<int64_t>(state_slots) * H >= (int64_t(1) << 31))
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_slots*H too large");
    const size_t xs = dsize(x_dtype);
    const size_t BH = static_cast<size_t>(B) * H, SH = static_cast<size_t>(state_slots) * H;
    const bool any = BH > 0;  // nothing is read or written when B == 0
    std::vector<Span> sp = {
        {"q_in", q_in, BH * dk * xs, false}, {"k_in", k_in, BH * dk * xs, false}, {"v_in", v_in, BH * dv * xs, false},
        {"w_q", w_q, any ? static_cast<size_t>(H) * dk * 4 * xs : 0, false},
        {"w_k", w_k, any ? static_cast<size_t>(H) * dk * 4 * xs : 0, false},
        {"w_v", w_v, any ? static_cast<size_t>(H) * dv * 4 * xs : 0, false},
        {"g_alpha", g_alpha, BH * dk * xs, false},
        {"out_gate", out_gate, out_gate ? BH * dv * xs : 0, false},
        {"conv_state", conv_state, any ? SH * 3 * (2 * dk + dv) * 4 : 0, true},
        {"state", state, any ? SH * dk * dv * 4 : 0, true},
        {"out", out, BH * dv * xs, true},
    };
    int st = check_spans(sp);
    if (st != KDA_OK) return st;
    if (any && (b_beta == nullptr || (reinterpret_cast<uintptr_t>(b_beta) % xs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "b_beta is NULL or misaligned");
    if (any && state_indices != nullptr && (reinterpret_cast<uintptr_t>(state_indices) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices is not 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_indices(state_indices, B, state_slots, s);
    if (st != KDA_OK) return st;
    kda::DecodeLayerArgs a;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv; a.x = static_cast<kda::DT>(x_dtype);
    a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.w_q = w_q; a.w_k = w_k; a.w_v = w_v;
    a.g = g_alpha; a.b = b_beta; a.z = out_gate;
    a.conv_state = conv_state; a.state = state; a.slots = state_slots; a.state_indices = state_indices; a.out = out;
    hipError_t e = kda::launch_decode_layer(a, s);
    if (e != hipSuccess) return hip_fail(e, "decode layer launch");
    return ok();
}

size_t kda_spec_draft_bytes(int32_t H, int32_t dk, int32_t dv, int32_t x_dtype) {
    if (H < 1 || H > 65535 || !valid_head_dim(dk) || !valid_head_dim(dv) || !valid_dtype(x_dtype)) return 0;
    return static_cast<size_t>(kda::kSpecMaxTokens) * H * kda::spec_draft_width(dk, dv) * dsize(x_dtype);
}

int kda_spec_verify(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t x_dtype, const void* q_in,
                    const void* k_in, const void* v_in, const void* w_q, const void* w_k, const void* w_v,
                    const void* g_alpha, const void* b_beta, float* conv_state, const void* out_gate,
                    float* state, int32_t state_slots, const int32_t* state_indices, const int32_t* accepted,
                    void* drafts, void* out, void* stream) {
    if (B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
    if (T < 0 || T > kda::kSpecMaxTokens)
        return fail(KDA_ERR_INVALID_ARGUMENT, "T=%d out of range [0, %d]", T, kda::kSpecMaxTokens);
    if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H=%d out of range [1, 65535]", H);
    if (!valid_head_dim(dk) || !valid_head_dim(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d, dv=%d: supported head sizes are 16, 32, 64, 128", dk, dv);
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (static_cast<int64_t>(B) * H >= (int64_t(1) << 31)) return fail(KDA_ERR_INVALID_ARGUMENT, "B*H too large");
    if (state_slots < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "state_slots=%d must be >= 0", state_slots);
    if (state_indices == nullptr && state_slots != B)
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices is NULL but state_slots=%d != B=%d", state_slots, B);
    if (static_cast<int64_t>(state_slots) * H >= (int64_t(1) << 31))
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_slots*H too large");
    const size_t xs = dsize(x_dtype);
    const size_t BTH = static_cast<size_t>(B) * T * H, SH = static_cast<size_t>(state_slots) * H;
    const bool any = B > 0;
    std::vector<Span> sp = {
        {"q_in", q_in, BTH * dk * xs, false}, {"k_in", k_in, BTH * dk * xs, false},
        {"v_in", v_in, BTH * dv * xs, false},
        {"w_q", w_q, any ? static_cast<size_t>(H) * dk * 4 * xs : 0, false},
        {"w_k", w_k, any ? static_cast<size_t>(H) * dk * 4 * xs : 0, false},
        {"w_v", w_v, any ? static_cast<size_t>(H) * dv * 4 * xs : 0, false},
        {"g_alpha", g_alpha, BTH * dk * xs, false},
        {"out_gate", out_gate, out_gate ? BTH * dv * xs : 0, false},
        {"conv_state", conv_state, any ? SH * 3 * (2 * dk + dv) * 4 : 0, true},
        {"state", state, any ? SH * dk * dv * 4 : 0, true},
        {"drafts", drafts, any ? static_cast<size_t>(state_slots) * kda_spec_draft_bytes(H, dk, dv, x_dtype) : 0, true},
        {"out", out, BTH * dv * xs, true},
    };
    int st = check_spans(sp);
    if (st != KDA_OK) return st;
    if (BTH > 0 && (b_beta == nullptr || (reinterpret_cast<uintptr_t>(b_beta) % xs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "b_beta is NULL or misaligned");
    if (any && state_indices != nullptr && (reinterpret_cast<uintptr_t>(state_indices) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices is not 4-byte aligned");
    if (any && accepted != nullptr && (reinterpret_cast<uintptr_t>(accepted) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "accepted is not 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_indices(state_indices, B, state_slots, s);
    if (st != KDA_OK) return st;
    kda::SpecArgs a;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv; a.T = T; a.x = static_cast<kda::DT>(x_dtype);
    a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.w_q = w_q; a.w_k = w_k; a.w_v = w_v;
    a.g = g_alpha; a.b = b_beta; a.z = out_gate;
    a.conv_state = conv_state; a.state = state; a.slots = state_slots; a.state_indices = state_indices;
    a.accepted = accepted; a.drafts = drafts; a.out = out;
    hipError_t e = kda::launch_spec_verify(a, s);
    if (e != hipSuccess) return hip_fail(e, "speculative verify launch");
    return ok();
}

size_t kda_backward_workspace_bytes(int64_t T_tot, int32_t N, int32_t H, int32_t dk, int32_t dv) {
    if (T_tot < 0 || T_tot >= (int64_t(1) << 31) || N < 1 || H < 1 || H > 65535 || !valid_head_dim(dk) ||
        !valid_head_dim(dv))
        return 0;
    return kda::backward_workspace_bytes(T_tot, N, H, dk, dv);
}

int kda_prefill_backward(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens, int32_t N,
                         int32_t x_dtype, int32_t gate_dtype, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const void* out_gate,
                         const float* initial_state, const void* dy, const float* dS_final, float* dq, float* dk_,
                         float* dv_, float* dlog_alpha, float* dbeta, float* dz, float* dS0, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int st = check_sizes(T_tot, H, dk, dv, N);
    if (st != KDA_OK) return st;
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    if (!valid_dtype(gate_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "gate_dtype=%d is not KDA_F32 or KDA_BF16", gate_dtype);
    if (cu_seqlens == nullptr && N != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but N=%d", N);
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    if ((out_gate == nullptr) != (dz == nullptr))
        return fail(KDA_ERR_INVALID_ARGUMENT, "dz must be given exactly when out_gate is");
    const size_t need = kda_backward_workspace_bytes(T_tot, N, H, dk, dv);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL or not 256-byte aligned");
    const size_t xs = dsize(x_dtype), gs = dsize(gate_dtype);
    const size_t T = static_cast<size_t>(T_tot);
    const size_t qk = T * H * dk, vv = T * H * dv;
    const size_t state = static_cast<size_t>(N) * H * dk * dv * 4;
    std::vector<Span> sp = {
        {"q", q, qk * xs, false}, {"k", k, qk * xs, false}, {"v", v, vv * xs, false},
        {"log_alpha", log_alpha, qk * gs, false},
        {"out_gate", out_gate, out_gate ? vv * xs : 0, false},
        {"initial_state", initial_state, initial_state ? state : 0, false},
        {"dy", dy, vv * xs, false},
        {"dS_final", dS_final, dS_final ? state : 0, false},
        {"dq", dq, qk * 4, true}, {"dk", dk_, qk * 4, true}, {"dv", dv_, vv * 4, true},
        {"dlog_alpha", dlog_alpha, qk * 4, true}, {"dbeta", dbeta, T * H * 4, true},
        {"dz", dz, dz ? vv * 4 : 0, true}, {"dS0", dS0, dS0 ? state : 0, true},
        {"workspace", workspace, need, true},
    };
    // beta and dbeta rows are H elements, accessed one at a time: element alignment suffices
    sp[12].bytes = 0;
    st = check_spans(sp);
    if (st != KDA_OK) return st;
    if (T * H > 0 && (beta == nullptr || (reinterpret_cast<uintptr_t>(beta) % gs) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "beta is NULL or misaligned");
    if (T * H > 0 && (dbeta == nullptr || (reinterpret_cast<uintptr_t>(dbeta) & 3u) != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "dbeta is NULL or misaligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu(cu_seqlens, N, T_tot, s);
    if (st != KDA_OK) return st;
    kda::BackwardArgs b{};
    kda::PrefillArgs& a = b.f;
    a.T = T_tot; a.H = H; a.dk = dk; a.dv = dv; a.N = N; a.cu = cu_seqlens;
    a.x = static_cast<kda::DT>(x_dtype); a.gate = static_cast<kda::DT>(gate_dtype);
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.z = out_gate;
    a.S0 = initial_state; a.ws = workspace; a.ws_bytes = workspace_bytes;
    b.dy = dy; b.dS_final = dS_final;
    b.dq = dq; b.dk = dk_; b.dv = dv_; b.dla = dlog_alpha; b.dbeta = dbeta; b.dz = dz; b.dS0 = dS0;
    hipError_t e = kda::launch_backward(b, s);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kda_prefill_layer_noalloc: the layer prefill with its workspace in a fixed
// device array instead of caller memory.  Each GPU the library runs on holds
// its own copy of the array until the process ends; every call on that GPU
// shares it (the last call's contents stay; nothing in it needs to start at
// zero, since every record is written before it is read).  Calls that overlap
// on one GPU race on it.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch` per device ordinal

// The current device's copy of `scratch`.  In host code the array's name is a
// host-side stand-in, not a device address, so its device address is looked
// up once per device, with that device current, and only that pointer ever
// reaches a kernel.
int noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KDA_ERR_UNSUPPORTED, "device ordinal %d: the no-allocation scratch is kept for devices 0..%d",
                    dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the no-allocation scratch");
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
            return fail(KDA_ERR_HIP, "the no-allocation scratch has no 256-byte aligned device address");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_prefill_layer_noalloc(int64_t T_tot, int32_t H, int32_t dk, int32_t dv, const int32_t* cu_seqlens,
                              int32_t N, int32_t x_dtype, const void* q_in, const void* k_in, const void* v_in,
                              const void* w_q, const void* w_k, const void* w_v, const void* g_alpha,
                              const void* b_beta, float* conv_state, const void* out_gate,
                              const float* initial_state, float* final_state, void* out, void* stream) {
    // the size limit first, before any device work
    int st = check_sizes(T_tot, H, dk, dv, N);
    if (st != KDA_OK) return st;
    if (!valid_dtype(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_dtype=%d is not KDA_F32 or KDA_BF16", x_dtype);
    const size_t need = kda_prefill_workspace_bytes(T_tot, N, H, dk, dv, x_dtype);
    if (need > static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                    "kda_prefill_layer_noalloc: T_tot=%lld, N=%d, H=%d need %zu bytes of scratch, more than its "
                    "fixed %zu; use kda_prefill_layer with a workspace",
                    static_cast<long long>(T_tot), N, H, need, static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != KDA_OK) return st;
    return prefill_layer_impl(T_tot, H, dk, dv, cu_seqlens, N, x_dtype, q_in, k_in, v_in, w_q, w_k, w_v, g_alpha,
                              b_beta, conv_state, out_gate, initial_state, final_state, out, ws,
                              static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES), stream, nullptr);
}

}  // extern "C"
