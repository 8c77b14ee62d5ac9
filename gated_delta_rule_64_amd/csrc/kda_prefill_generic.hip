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
// Four waves on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane (g, c) =
// (lane / 16, lane % 16) gives A[c][g] and B[g][c] and holds D[4g + e][c];
// here the MFMA's term g of step jj is term 4g + jj of a run of 16).  Per
// chunk, wave w makes token rows 16w .. 16w + 15 of
//     U = U~ - W S   and   O = Q' S + M U~,
// then the waves that own state rows update them:  S <- Diag(gamma) S + K^T U.
// A wave keeps its state rows as matrix-core accumulators; S (the B operand
// of W S and Q' S) and U (of K^T U) are shared through LDS.  Each operand a
// wave takes from the record is reloaded, for the next chunk, as soon as the
// products that use it are issued, so its load overlaps the rest of the step.
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGS = 20;  // LDS row stride of S and U (16 columns): rows 4g + jj of lanes (g, c) fall in distinct banks

template <int DK>
struct GenOps {
    static constexpr int KB = DK / 16;                // 16-term runs of W S
    static constexpr int ST = DK / 16;                // 16-row tiles of S
    static constexpr int SPW = ST >= 4 ? ST / 4 : 1;  // state tiles per wave
    float kh[SPW][4][4];  // K^[16 kb + 4g + jj][i0 + c]
    float gam[SPW][4];    // gamma[i0 + 4g + e]
    float u[4], oi[4];    // U~, M U~ at [16 wave + 4g + e][16 sl + c]
    float z[4];           // gate logits of the same outputs
};

template <int DK, typename XT, typename GT>
__global__ __launch_bounds__(256) void gen_state_kernel(GenK<XT, GT> a) {
    using Ops = GenOps<DK>;
    constexpr int KB = Ops::KB, ST = Ops::ST, SPW = Ops::SPW;
    __shared__ float sS[DK * kGS];
    __shared__ float sU[64 * kGS];
    const int dv = a.dv, nsl = dv / 16;
    const SliceBlock sbk = slice_block(blockIdx.x, nsl);
    if (sbk.grp >= static_cast<int64_t>(a.N) * a.H) return;
    const int sl = sbk.sl, h = static_cast<int>(sbk.grp % a.H), n = static_cast<int>(sbk.grp / a.H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    const bool owner = wave * SPW < ST;  // (below d = 64 some waves own no state rows)
    const GenRec R = gen_rec(DK, dv);
    const int64_t sidx = (static_cast<int64_t>(n) * a.H + h) * DK * dv;
    const int col = 16 * sl + c;
    auto i0 = [&](int t) { return owner ? 16 * (wave * SPW + t) : 0; };
    const int64_t sb = seq_begin(a.cu, n), se = seq_finish(a.cu, n, a.T);
    const int nch = a.base[n + 1] - a.base[n];
    const bool has_z = a.z != nullptr;
    const XT* zp = has_z ? a.z : a.v;  // (same [T][H][dv] layout; read but unused without a gate)
    auto rec_of = [&](int j) { return a.rec + (static_cast<int64_t>(a.base[n] + j) * a.H + h) * R.size; };
    auto len_of = [&](int j) {
        return static_cast<int>(min(static_cast<int64_t>(kChunk), se - (sb + static_cast<int64_t>(j) * kChunk)));
    };
    Ops o;
    // W, Q' at row 16 wave + c, terms 16 kb + 4g .. + 3: two register sets,
    // chunk j in set j % 2, so the next chunk's loads are issued a whole step
    // before they are used
    f32x4 w0[KB], q0[KB], w1[KB], q1[KB];
    auto load_wq = [&](const float* rec, f32x4 (&w)[KB], f32x4 (&q)[KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t off = (16 * wave + c) * DK + 16 * kb + 4 * g;
            w[kb] = *reinterpret_cast<const f32x4*>(rec + R.W + off);
            q[kb] = *reinterpret_cast<const f32x4*>(rec + R.Qp + off);
        }
    };
    auto load_rows = [&](const float* rec, int j) {  // U~, M U~, gate logits
        const int L = len_of(j);
        const int64_t t0 = sb + static_cast<int64_t>(j) * kChunk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * wave + 4 * g + e;
            o.u[e] = rec[R.U + r * dv + col];
            o.oi[e] = rec[R.Oi + r * dv + col];
            o.z[e] = ld(zp + ((t0 + min(r, L - 1)) * a.H + h) * dv + col);
        }
    };
    auto load_k = [&](const float* rec) {
#pragma unroll
        for (int t = 0; t < SPW; ++t) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o.kh[t][kb][jj] = rec[R.Kh + (16 * kb + 4 * g + jj) * DK + i0(t) + c];
#pragma unroll
            for (int e = 0; e < 4; ++e) o.gam[t][e] = rec[R.gam + i0(t) + 4 * g + e];
        }
    };
    // the state rows of this wave: tile t holds rows i0(t) + 4g + e, column col
    f32x4 S[SPW];
#pragma unroll
    for (int t = 0; t < SPW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = i0(t) + 4 * g + e;
            S[t][e] = a.S0 && owner ? a.S0[sidx + row * dv + col] : 0.f;
            if (owner) sS[row * kGS + c] = S[t][e];
        }
    if (nch > 0) {
        const float* rec = rec_of(0);
        load_wq(rec, w0, q0);
        load_rows(rec, 0);
        load_k(rec);
    }
    __syncthreads();
    auto step = [&](int j, f32x4 (&w)[KB], f32x4 (&q)[KB], f32x4 (&wn)[KB], f32x4 (&qn)[KB]) {
        const int L = len_of(j);
        const int64_t t0 = sb + static_cast<int64_t>(j) * kChunk;
        const float* rec_next = rec_of(min(j + 1, nch - 1));  // (the last step reloads its own chunk, unused)
        load_wq(rec_next, wn, qn);
        // U and O rows 16 wave .. + 15
        // (all of S's operand values are read from LDS before the products start)
        float bs[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bs[kb][jj] = sS[(16 * kb + 4 * g + jj) * kGS + c];
        f32x4 ua = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                ua = __builtin_amdgcn_mfma_f32_16x16x4f32(w[kb][jj], bs[kb][jj], ua, 0, 0, 0);
                oa = __builtin_amdgcn_mfma_f32_16x16x4f32(q[kb][jj], bs[kb][jj], oa, 0, 0, 0);
            }
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sU[(16 * wave + 4 * g + e) * kGS + c] = o.u[e] - ua[e];
            const float out = o.oi[e] + oa[e];
            y[e] = has_z ? out * sigmoid_fast(o.z[e]) : out;
        }
        load_rows(rec_next, min(j + 1, nch - 1));
        if (a.out != nullptr) {  // (no output: a forward pass run for its records and states)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * wave + 4 * g + e;
                if (r < L) st(a.out + ((t0 + r) * a.H + h) * dv + col, y[e]);
            }
        }
        __syncthreads();  // U is complete; every read of S is done
        // a full chunk that ends a snapshot interval: the state after it is the m-th snapshot
        const int sc = a.snap.chunks;
        const bool snap = sc > 0 && (j + 1) % sc == 0 && L == kChunk;
        if (owner) {
            float bu[4][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) bu[kb][jj] = sU[(16 * kb + 4 * g + jj) * kGS + c];
#pragma unroll
            for (int t = 0; t < SPW; ++t) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = o.gam[t][e] * S[t][e];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o.kh[t][kb][jj], bu[kb][jj], acc, 0, 0, 0);
                S[t] = acc;
            }
            load_k(rec_next);
#pragma unroll
            for (int t = 0; t < SPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) sS[(i0(t) + 4 * g + e) * kGS + c] = S[t][e];
            if (snap) {
                float* so = a.snap.out + ((static_cast<int64_t>(a.snap.off[n]) + (j + 1) / sc - 1) * a.H + h) * DK * dv;
#pragma unroll
                for (int t = 0; t < SPW; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) so[(i0(t) + 4 * g + e) * dv + col] = S[t][e];
            }
        }
        __syncthreads();  // S is complete; every read of U is done
    };
    for (int j = 0; j < nch; j += 2) {
        step(j, w0, q0, w1, q1);
        if (j + 1 < nch) step(j + 1, w1, q1, w0, q0);
    }
    if (a.S_out && owner) {
#pragma unroll
        for (int t = 0; t < SPW; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.S_out[sidx + (i0(t) + 4 * g + e) * dv + col] = S[t][e];
    }
}

template <typename XT, typename GT>
hipError_t launch_gen_state_kernel(const GenK<XT, GT>& k, hipStream_t s) {
    const int64_t blocks = slice_grid(static_cast<int64_t>(k.N) * k.H, k.dv / 16);
    LaunchTimer timer("gen_state", s);
    switch (k.dk) {
        case 16: hipLaunchKernelGGL((gen_state_kernel<16, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k); break;
        case 32: hipLaunchKernelGGL((gen_state_kernel<32, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k); break;
        case 64: hipLaunchKernelGGL((gen_state_kernel<64, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k); break;
        case 128: hipLaunchKernelGGL((gen_state_kernel<128, XT, GT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
    return launch_gen_state_kernel(k, s);
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
    return launch_gen_state_kernel(k, s);
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
    const bool mfma = prefill_uses_mfma(a.dk, a.dv, a.x);
    if (!mfma || !mfma_inline_map(a.N, a.snap)) {
        LaunchTimer timer("chunk_map", s);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.T, base, slot_info,
                           a.snap.chunks, a.snap.off);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (mfma) return launch_prefill_mfma(a, s, base, slot_info, recs);
    return launch_gen_forward(a, s, base, reinterpret_cast<float*>(recs));
}

bool layer_fused_supported(int dk, int dv, DT x) { return prefill_uses_mfma(dk, dv, x); }

hipError_t launch_layer(const LayerArgs& a, hipStream_t s) {
    int32_t* base = static_cast<int32_t*>(a.ws);
    SlotInfo* slot_info = reinterpret_cast<SlotInfo*>(static_cast<char*>(a.ws) + chunk_map_base_bytes(a.N));
    char* recs = static_cast<char*>(a.ws) + chunk_map_bytes(a.T, a.N);
    hipError_t e;
    if (!mfma_inline_map(a.N, a.snap)) {
        LaunchTimer timer("chunk_map", s);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.T, base, slot_info,
                           a.snap.chunks, a.snap.off);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = launch_layer_mfma(a, s, base, slot_info, recs);
    if (e != hipSuccess) return e;
    // the chunk kernel has read the old conv history; now it is replaced
    PreprocessArgs p{};
    p.T = a.T; p.H = a.H; p.dk = a.dk; p.dv = a.dv; p.N = a.N; p.cu = a.cu; p.x = DT::BF16;
    p.q_in = a.q_in; p.k_in = a.k_in; p.v_in = a.v_in; p.conv_state = a.conv_state;
    return launch_conv_state_update(p, s);
}

}  // namespace kda
