// Per-kernel event timing for profiling (thread-local; off unless enabled).
#include <cstring>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_profile.h"

namespace kda {
namespace {

struct Pending {
    const char* name;
    hipEvent_t start, stop;
    bool stop_recorded;  // false if recording the stop event failed (a pooled event may hold an old time)
};

struct State {
    bool on = false;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;
};

thread_local State g_state;

hipEvent_t take_event() {
    if (!g_state.pool.empty()) {
        hipEvent_t e = g_state.pool.back();
        g_state.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t s) : slot_(-1), stream_(s) {
    if (!g_state.on) return;
    hipEvent_t a = take_event(), b = take_event();
    if (a == nullptr || b == nullptr) return;
    if (hipEventRecord(a, s) != hipSuccess) return;
    g_state.pending.push_back({name, a, b, false});
    slot_ = static_cast<int>(g_state.pending.size()) - 1;
}

LaunchTimer::~LaunchTimer() {
    if (slot_ >= 0) g_state.pending[slot_].stop_recorded = hipEventRecord(g_state.pending[slot_].stop, stream_) == hipSuccess;
}

}  // namespace kda

extern "C" {

int kda_profile_enable(int on) {
    kda::g_state.on = on != 0;
    return KDA_OK;
}

int kda_profile_collect(kda_kernel_time_t* out, int max_entries) {
    using kda::g_state;
    std::vector<kda_kernel_time_t> agg;
    int status = KDA_OK;
    for (const kda::Pending& p : g_state.pending) {
        float ms = 0.f;
        if (!p.stop_recorded || hipEventSynchronize(p.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
            status = KDA_ERR_HIP;
        kda_kernel_time_t* hit = nullptr;
        for (auto& a : agg)
            if (std::strncmp(a.name, p.name, sizeof(a.name)) == 0) hit = &a;
        if (hit == nullptr) {
            kda_kernel_time_t z;
            std::memset(&z, 0, sizeof(z));
            std::strncpy(z.name, p.name, sizeof(z.name) - 1);
            agg.push_back(z);
            hit = &agg.back();
        }
        hit->launches += 1;
        hit->total_ms += ms;
        g_state.pool.push_back(p.start);
        g_state.pool.push_back(p.stop);
    }
    g_state.pending.clear();
    const int n = static_cast<int>(agg.size());
    for (int i = 0; i < n && i < max_entries; ++i) out[i] = agg[i];
    return status == KDA_OK ? n : -status;
}

}  // extern "C"
