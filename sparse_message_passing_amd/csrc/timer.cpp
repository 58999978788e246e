// timer.cpp -- per-kernel launch timing with HIP events (measurement only).
//
// While timing is on, every instrumented launch whose key matches the wanted
// key (or every one, for an empty key) is bracketed by two events recorded on
// the stream it is launched on, so the recorded interval is that kernel's
// execution on the device.  The events come from a pool created when timing
// starts (nothing is allocated while launches are being timed); launches
// beyond the pool's capacity are counted as dropped and make the result call
// fail instead of returning a partial sum.

#include <atomic>
#include <cstring>
#include <mutex>
#include <set>

#include "internal.h"

namespace gnnmp {

namespace {

struct Rec {
    std::string key;
    int slot;
};

struct TimerState {
    std::mutex mu;
    std::string want;
    std::vector<hipEvent_t> pool;  // 2 * capacity events: start, end of each slot
    std::vector<Rec> recs;
    std::set<std::string> seen;
    int64_t dropped = 0;
};

std::atomic<bool> g_on{false};

TimerState& state() {
    static TimerState s;
    return s;
}

void release_pool(TimerState& s) {
    for (hipEvent_t e : s.pool) (void)hipEventDestroy(e);
    s.pool.clear();
    s.recs.clear();
    s.seen.clear();
    s.dropped = 0;
}

}  // namespace

bool timer_on() { return g_on.load(std::memory_order_relaxed); }

int timer_begin(const std::string& key, hipStream_t st) {
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (!timer_on()) return -1;
    s.seen.insert(key);
    if (!s.want.empty() && key != s.want) return -1;
    const int slot = static_cast<int>(s.recs.size());
    if (2 * static_cast<size_t>(slot) + 1 >= s.pool.size()) {
        ++s.dropped;
        return -1;
    }
    if (hipEventRecord(s.pool[2 * slot], st) != hipSuccess) {
        ++s.dropped;
        return -1;
    }
    s.recs.push_back(Rec{key, slot});
    return slot;
}

void timer_end(int slot, hipStream_t st) {
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (slot < 0 || 2 * static_cast<size_t>(slot) + 1 >= s.pool.size()) return;
    if (hipEventRecord(s.pool[2 * slot + 1], st) != hipSuccess) ++s.dropped;
}

ScopedTimer::ScopedTimer(hipStream_t st, const char* fmt, ...) : st_(st) {
    if (!timer_on()) return;
    char buf[160];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    slot_ = timer_begin(buf, st);
}

ScopedTimer::~ScopedTimer() {
    if (slot_ >= 0) timer_end(slot_, st_);
}

}  // namespace gnnmp

using namespace gnnmp;

extern "C" {

gnn_status_t gnn_timer_start(const char* key, int64_t capacity) {
    GNN_REQUIRE(capacity >= 1 && capacity <= (int64_t(1) << 20), "gnn_timer_start: capacity must be in [1, 2^20]");
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    g_on.store(false);
    release_pool(s);
    s.want = key ? key : "";
    s.pool.resize(static_cast<size_t>(2 * capacity), nullptr);
    for (hipEvent_t& e : s.pool) {
        const hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            e = nullptr;
            release_pool(s);
            return hip_fail(err, "gnn_timer_start: hipEventCreate");
        }
    }
    g_on.store(true);
    return GNN_OK;
}

gnn_status_t gnn_timer_stop(void) {
    g_on.store(false);
    return GNN_OK;
}

gnn_status_t gnn_timer_result(const char* key, int64_t* launches, double* total_ms) {
    GNN_REQUIRE(key && launches && total_ms, "gnn_timer_result: NULL argument");
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (s.dropped)
        return fail(GNN_ERR_WORKSPACE, "gnn_timer_result: " + std::to_string(s.dropped) +
                                           " launches were not timed (event pool too small)");
    int64_t cnt = 0;
    double tot = 0.0;
    for (const Rec& r : s.recs) {
        if (r.key != key) continue;
        GNN_HIP(hipEventSynchronize(s.pool[2 * r.slot + 1]));
        float ms = 0.0f;
        GNN_HIP(hipEventElapsedTime(&ms, s.pool[2 * r.slot], s.pool[2 * r.slot + 1]));
        tot += ms;
        ++cnt;
    }
    *launches = cnt;
    *total_ms = tot;
    return GNN_OK;
}

gnn_status_t gnn_timer_keys(char* buf, size_t len) {
    GNN_REQUIRE(buf && len >= 1, "gnn_timer_keys: need a buffer");
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    std::string all;
    for (const std::string& k : s.seen) all += k + "\n";
    if (all.size() + 1 > len) return fail(GNN_ERR_WORKSPACE, "gnn_timer_keys: buffer too small");
    std::memcpy(buf, all.c_str(), all.size() + 1);
    return GNN_OK;
}

gnn_status_t gnn_timer_release(void) {
    TimerState& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    g_on.store(false);
    release_pool(s);
    return GNN_OK;
}

}  // extern "C"
