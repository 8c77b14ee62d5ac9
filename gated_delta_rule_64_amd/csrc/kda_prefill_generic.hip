// Chunked prefill, general path: any dk, dv in {16, 32, 64, 128}, fp32 or
// bf16 inputs, all arithmetic in fp32 on the vector ALUs.  It serves fp32
// inputs (where bf16 matrix-core operands would lose the precision the
// caller asked for) and head sizes the matrix-core path does not cover.
// The chunk algebra is described in kda_prefill_common.h.
//
// Every pairwise decay e^{G_r - G_s} (r >= s, so the exponent is <= 0) is
// evaluated directly, so no factor can overflow whatever the decay rates.
#include "kda_prefill_common.h"
#include "kda_internal.h"
#include "kda_profile.h"
#include "kda_prefill_mfma.h"

namespace kda {

__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* __restrict__ cu, int N,
                                                         int64_t T, int32_t* __restrict__ base,
                                                         SlotInfo* __restrict__ slot_info, int snap_chunks,
                                                         int32_t* __restrict__ snap_off) {
    // Both counts of a sequence (chunks in the low word, snapshots in the
    // high word) go through one 64-bit scan: the chunk total stays below
    // 2^26, so no carry crosses into the high word.
    __shared__ int64_t buf[1024];
    __shared__ int64_t wsum[16];
    __shared__ int64_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    // sequences in blocks of 1024, one per thread
    for (int start = 0; start < N; start += 1024) {
        const int i = start + tid;
        int64_t c = 0;
        if (i < N) {
            const int64_t L = seq_finish(cu, i, T) - seq_begin(cu, i);
            c = (L + kChunk - 1) / kChunk;
            if (snap_chunks > 0) c |= (L / (static_cast<int64_t>(kChunk) * snap_chunks)) << 32;
        }
        // inclusive scan: within each wave by lane shuffles, then over the
        // 16 wave totals in wave 0
        int64_t x = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        if (wave == 0) {
            int64_t w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const int64_t y = __shfl_up(w, off);
                if (lane >= off) w += y;
            }
            if (lane < 16) wsum[lane] = w;
        }
        __syncthreads();
        buf[tid] = x + (wave > 0 ? wsum[wave - 1] : 0);
        __syncthreads();
        const int64_t carry = carry_s;
        const int32_t carry_c = static_cast<int32_t>(carry & 0xffffffff);
        if (i < N) {
            const int64_t excl = carry + buf[tid] - c;
            base[i] = static_cast<int32_t>(excl & 0xffffffff);
            if (snap_chunks > 0) snap_off[i] = static_cast<int32_t>(excl >> 32);
        }
        // the block's slots, spread over all threads: slot carry + s belongs
        // to the first sequence j of the block whose inclusive count exceeds s
        auto chunks_to = [&](int k) { return static_cast<int32_t>(buf[k] & 0xffffffff); };
        const int32_t total = chunks_to(1023);
        for (int32_t s = tid; s < total; s += 1024) {
            int lo = 0, hi = 1023;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (chunks_to(mid) > s) hi = mid; else lo = mid + 1;
            }
            const int n = start + lo;
            const int32_t j = s - (lo > 0 ? chunks_to(lo - 1) : 0);  // chunk index inside the sequence
            SlotInfo si;
            si.t0 = seq_begin(cu, n) + static_cast<int64_t>(j) * kChunk;
            si.len = static_cast<int32_t>(min(static_cast<int64_t>(kChunk), seq_finish(cu, n, T) - si.t0)) |
                     (j == 0 ? (1 << 16) : 0);
            si.seq = n;
            slot_info[carry_c + s] = si;
        }
        __syncthreads();
        if (tid == 1023) carry_s = carry + buf[1023];
        __syncthreads();
    }
    if (tid == 0) {
        base[N] = static_cast<int32_t>(carry_s & 0xffffffff);
        if (snap_chunks > 0) snap_off[N] = static_cast<int32_t>(carry_s >> 32);
    }
}

namespace {

template <typename XT, typename GT>
struct GenK {
    int64_t T;
    int H, dk, dv, N;
    const int32_t* cu;
    const int32_t* base;
    const XT *q, *k, *v, *z;
    const GT *la, *beta;
    const float* S0;
    float* S_out;
    XT* out;
    float* rec;
    Snapshots snap;
};

// ---- phase 1, the records, is chunk_records_kernel (kda_backward.hip) ----

// ---- phase 2: per (sequence, head, 16 state columns), chunks in order ----
// One chunk's record matrix [64][dk] (16-byte aligned) into LDS rows of
// dk + 1 floats (the padding keeps reads of one channel over many rows, or
// of many rows at one channel, off a single bank).
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int dk) {
    const int kp = dk + 1;
    for (int i = threadIdx.x; i < 16 * dk; i += 256) {
        const int r = (4 * i) / dk, c = (4 * i) % dk;
        const float4 v = *reinterpret_cast<const float4*>(src + r * dk + c);
        float* d = dst + r * kp + c;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
}

size_t gen_state_lds_bytes(int dk) { return (2 * 64 * static_cast<size_t>(dk + 1) + 16 * dk + 64 * 16) * 4; }

template <typename XT, typename GT>
__global__ __launch_bounds__(256) void gen_state_kernel(GenK<XT, GT> a) {
    extern __shared__ float gsm[];
    const int dk = a.dk, dv = a.dv, kp = dk + 1;
    float* sWK = gsm;              // [64][kp]: W, then K^
    float* sQp = sWK + 64 * kp;    // [64][kp]: Q'
    float* sS = sQp + 64 * kp;     // [dk][16]: this block's 16 state columns
    float* sU = sS + 16 * dk;      // [64][16]
    const int nsl = dv / 16;
    const int sl = blockIdx.x % nsl;
    const int h = (blockIdx.x / nsl) % a.H;
    const int n = blockIdx.x / (nsl * a.H);
    const int tid = threadIdx.x;
    const GenRec R = gen_rec(dk, dv);
    const int64_t sidx = (static_cast<int64_t>(n) * a.H + h) * dk * dv;
    for (int e = tid; e < dk * 16; e += 256) {
        const int c = e >> 4, j = e & 15;
        sS[e] = a.S0 ? a.S0[sidx + c * dv + 16 * sl + j] : 0.f;
    }
    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    const int nch = a.base[n + 1] - a.base[n];
    const int r = tid >> 2, c4 = (tid & 3) * 4;
    for (int j = 0; j < nch; ++j) {
        const float* rec = a.rec + (static_cast<int64_t>(a.base[n] + j) * a.H + h) * R.size;
        const int64_t t0 = sb + static_cast<int64_t>(j) * kChunk;
        const int L = static_cast<int>(min(static_cast<int64_t>(kChunk), se - t0));
        __syncthreads();  // the last chunk's reads of sWK are done
        stage_rows(sWK, rec + R.W, dk);
        stage_rows(sQp, rec + R.Qp, dk);
        __syncthreads();
        // U = U~ - W S, O = Q' S + M U~ (row r, columns c4 .. c4+3)
        float u[4], o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = rec[R.U + r * dv + 16 * sl + c4 + i];
            o[i] = rec[R.Oi + r * dv + 16 * sl + c4 + i];
        }
        for (int c = 0; c < dk; ++c) {
            const float w = sWK[r * kp + c], qp = sQp[r * kp + c];
            const float4 s4 = *reinterpret_cast<const float4*>(sS + c * 16 + c4);
            u[0] -= w * s4.x; u[1] -= w * s4.y; u[2] -= w * s4.z; u[3] -= w * s4.w;
            o[0] += qp * s4.x; o[1] += qp * s4.y; o[2] += qp * s4.z; o[3] += qp * s4.w;
        }
        if (r < L && a.out != nullptr) {  // (no output: a forward pass run for its records and states)
            const int64_t oidx = ((t0 + r) * a.H + h) * dv + 16 * sl + c4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y = o[i];
                if (a.z) y *= sigmoid(ld(a.z + oidx + i));
                st(a.out + oidx + i, y);
            }
        }
        __syncthreads();  // every read of W and of S is done
#pragma unroll
        for (int i = 0; i < 4; ++i) sU[r * 16 + c4 + i] = u[i];
        stage_rows(sWK, rec + R.Kh, dk);
        __syncthreads();
        // S <- Diag(gamma) S + K^T U (channel c, columns j4 .. j4+3); a full
        // chunk that ends a snapshot interval: the state after it is the m-th snapshot
        const int sc = a.snap.chunks;
        const bool snap = sc > 0 && (j + 1) % sc == 0 && L == kChunk;
        float* snap_out = snap ? a.snap.out + ((static_cast<int64_t>(a.snap.off[n]) + (j + 1) / sc - 1) * a.H + h) *
                                                  dk * dv
                               : nullptr;
        for (int e = tid; e < dk * 4; e += 256) {
            const int c = e >> 2, j4 = (e & 3) * 4;
            const float gm = rec[R.gam + c];
            float acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gm * sS[c * 16 + j4 + i];
            for (int rr = 0; rr < 64; ++rr) {
                const float kh = sWK[rr * kp + c];
                const float4 u4 = *reinterpret_cast<const float4*>(sU + rr * 16 + j4);
                acc[0] += kh * u4.x; acc[1] += kh * u4.y; acc[2] += kh * u4.z; acc[3] += kh * u4.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sS[c * 16 + j4 + i] = acc[i];  // (each element read and written by its own thread)
                if (snap) snap_out[c * dv + 16 * sl + j4 + i] = acc[i];
            }
        }
    }
    __syncthreads();
    if (a.S_out) {
        for (int e = tid; e < dk * 16; e += 256) {
            const int c = e >> 4, jj = e & 15;
            a.S_out[sidx + c * dv + 16 * sl + jj] = sS[e];
        }
    }
}

template <typename XT, typename GT>
hipError_t launch_gen_typed(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec) {
    GenK<XT, GT> k;
    k.T = a.T; k.H = a.H; k.dk = a.dk; k.dv = a.dv; k.N = a.N; k.cu = a.cu; k.base = base;
    k.q = static_cast<const XT*>(a.q); k.k = static_cast<const XT*>(a.k);
    k.v = static_cast<const XT*>(a.v); k.z = static_cast<const XT*>(a.z);
    k.la = static_cast<const GT*>(a.la); k.beta = static_cast<const GT*>(a.beta);
    k.S0 = a.S0; k.S_out = a.S_out; k.out = static_cast<XT*>(a.out); k.rec = rec; k.snap = a.snap;
    {
        hipError_t e = launch_chunk_records(a, s, base, rec);
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = static_cast<int64_t>(a.N) * a.H * (a.dv / 16);
    const size_t lds = gen_state_lds_bytes(a.dk);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gen_state_kernel<XT, GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("gen_state", s);
    hipLaunchKernelGGL((gen_state_kernel<XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), lds, s, k);
    return hipGetLastError();
}

}  // namespace

template <typename XT, typename GT>
hipError_t launch_gen_state_typed(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec) {
    GenK<XT, GT> k;
    k.T = a.T; k.H = a.H; k.dk = a.dk; k.dv = a.dv; k.N = a.N; k.cu = a.cu; k.base = base;
    k.q = static_cast<const XT*>(a.q); k.k = static_cast<const XT*>(a.k);
    k.v = static_cast<const XT*>(a.v); k.z = static_cast<const XT*>(a.z);
    k.la = static_cast<const GT*>(a.la); k.beta = static_cast<const GT*>(a.beta);
    k.S0 = a.S0; k.S_out = a.S_out; k.out = static_cast<XT*>(a.out); k.rec = rec; k.snap = a.snap;
    const int64_t blocks = static_cast<int64_t>(a.N) * a.H * (a.dv / 16);
    const size_t lds = gen_state_lds_bytes(a.dk);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gen_state_kernel<XT, GT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    LaunchTimer timer("gen_state", s);
    hipLaunchKernelGGL((gen_state_kernel<XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), lds, s, k);
    return hipGetLastError();
}

hipError_t launch_gen_state(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec) {
    if (a.x == DT::BF16) {
        return a.gate == DT::BF16 ? launch_gen_state_typed<bf16, bf16>(a, s, base, rec)
                                  : launch_gen_state_typed<bf16, float>(a, s, base, rec);
    }
    return a.gate == DT::BF16 ? launch_gen_state_typed<float, bf16>(a, s, base, rec)
                              : launch_gen_state_typed<float, float>(a, s, base, rec);
}

hipError_t launch_gen_forward(const PrefillArgs& a, hipStream_t s, int32_t* base, float* rec) {
    if (a.x == DT::BF16) {
        return a.gate == DT::BF16 ? launch_gen_typed<bf16, bf16>(a, s, base, rec)
                                  : launch_gen_typed<bf16, float>(a, s, base, rec);
    }
    return a.gate == DT::BF16 ? launch_gen_typed<float, bf16>(a, s, base, rec)
                              : launch_gen_typed<float, float>(a, s, base, rec);
}

bool prefill_uses_mfma(int dk, int dv, DT x) { return mfma_prefill_supports(dk, dv, x); }

size_t prefill_workspace_bytes(int64_t T, int N, int H, int dk, int dv, DT x) {
    const size_t slots = static_cast<size_t>(chunk_slots_bound(T, N));
    const size_t rec = prefill_uses_mfma(dk, dv, x) ? mfma_record_bytes()
                                                    : static_cast<size_t>(gen_rec(dk, dv).size) * 4;
    return chunk_map_bytes(T, N) + slots * static_cast<size_t>(H) * rec;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    int32_t* base = static_cast<int32_t*>(a.ws);
    SlotInfo* slot_info = reinterpret_cast<SlotInfo*>(static_cast<char*>(a.ws) + chunk_map_base_bytes(a.N));
    char* recs = static_cast<char*>(a.ws) + chunk_map_bytes(a.T, a.N);
    hipError_t e;
    {
        LaunchTimer timer("chunk_map", s);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.T, base, slot_info,
                           a.snap.chunks, a.snap.off);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if (prefill_uses_mfma(a.dk, a.dv, a.x)) return launch_prefill_mfma(a, s, base, slot_info, recs);
    return launch_gen_forward(a, s, base, reinterpret_cast<float*>(recs));
}

bool layer_fused_supported(int dk, int dv, DT x) { return prefill_uses_mfma(dk, dv, x); }

hipError_t launch_layer(const LayerArgs& a, hipStream_t s) {
    int32_t* base = static_cast<int32_t*>(a.ws);
    SlotInfo* slot_info = reinterpret_cast<SlotInfo*>(static_cast<char*>(a.ws) + chunk_map_base_bytes(a.N));
    char* recs = static_cast<char*>(a.ws) + chunk_map_bytes(a.T, a.N);
    hipError_t e;
    {
        LaunchTimer timer("chunk_map", s);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.T, base, slot_info,
                           a.snap.chunks, a.snap.off);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    e = launch_layer_mfma(a, s, base, slot_info, recs);
    if (e != hipSuccess) return e;
    // the chunk kernel has read the old conv history; now it is replaced
    PreprocessArgs p{};
    p.T = a.T; p.H = a.H; p.dk = a.dk; p.dv = a.dv; p.N = a.N; p.cu = a.cu; p.x = DT::BF16;
    p.q_in = a.q_in; p.k_in = a.k_in; p.v_in = a.v_in; p.conv_state = a.conv_state;
    return launch_conv_state_update(p, s);
}

}  // namespace kda
