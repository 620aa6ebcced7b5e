// rse_trace.hip -- per-kernel timing with HIP events (measurement support).
//
// While a trace is active, launch sites of the traced kernel bracket the
// launch with two events on the launch stream; rse_trace_stop synchronises
// them and sums the elapsed times.  Events come from a fixed pool created on
// first use.
#include <mutex>
#include <vector>

#include "rse_host.h"

namespace {

constexpr int POOL = 4096;

struct Trace {
    std::mutex mu;
    int kernel = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;   // 2 * POOL events
};

Trace& trace() {
    static Trace t;
    return t;
}

}  // namespace

namespace rse_host {

int g_trace_kernel = 0;

void trace_mark(int kernel, hipStream_t s, bool after) {
    Trace& t = trace();
    std::lock_guard<std::mutex> lk(t.mu);
    if (t.kernel != kernel || t.ev.empty()) return;
    if (!after) {
        if (t.used >= POOL) return;
        hipEventRecord(t.ev[2 * t.used], s);
    } else {
        if (t.used >= POOL) return;
        hipEventRecord(t.ev[2 * t.used + 1], s);
        ++t.used;
    }
}

}  // namespace rse_host

extern "C" {

int rse_trace_start(int32_t kernel) {
    if (kernel < RSE_K_PROBE || kernel > RSE_K_INTERACT) return RSE_ERR_INVALID_ARG;
    Trace& t = trace();
    std::lock_guard<std::mutex> lk(t.mu);
    if (t.ev.empty()) {
        t.ev.resize(2 * POOL);
        for (auto& e : t.ev)
            if (hipEventCreate(&e) != hipSuccess) return RSE_ERR_HIP;
    }
    t.kernel = kernel;
    t.used = 0;
    rse_host::g_trace_kernel = kernel;
    return RSE_OK;
}

int rse_trace_stop(int64_t* n_launches_out, double* total_ms_out) {
    Trace& t = trace();
    std::lock_guard<std::mutex> lk(t.mu);
    rse_host::g_trace_kernel = 0;
    double tot = 0.0;
    for (int i = 0; i < t.used; ++i) {
        if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess) return RSE_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return RSE_ERR_HIP;
        tot += ms;
    }
    if (n_launches_out) *n_launches_out = t.used;
    if (total_ms_out) *total_ms_out = tot;
    t.kernel = 0;
    t.used = 0;
    return RSE_OK;
}

}  // extern "C"
