// Kernel timer (see timer.hpp and pkv_timer_enable / pkv_timer_read in pkv.h).
#include "timer.hpp"

#include <atomic>
#include <mutex>
#include <vector>

#include "status.hpp"

namespace pkv {
namespace {

struct EntryEvents {
    std::vector<LaunchEvents> pool;   // created on demand, reused after each read
    size_t used = 0;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
EntryEvents g_entries[PKV_TIMER_ENTRIES];

}  // namespace

LaunchEvents timer_events(int entry) {
    if (!g_on.load(std::memory_order_relaxed) || entry < 0 || entry >= PKV_TIMER_ENTRIES)
        return {nullptr, nullptr};
    std::lock_guard<std::mutex> lock(g_mu);
    EntryEvents& e = g_entries[entry];
    if (e.used == e.pool.size()) {
        LaunchEvents ev{nullptr, nullptr};
        if (hipEventCreate(&ev.start) != hipSuccess) return {nullptr, nullptr};
        if (hipEventCreate(&ev.stop) != hipSuccess) {
            (void)hipEventDestroy(ev.start);
            return {nullptr, nullptr};
        }
        e.pool.push_back(ev);
    }
    return e.pool[e.used++];
}

}  // namespace pkv

extern "C" int pkv_timer_enable(int32_t enable) {
    std::lock_guard<std::mutex> lock(pkv::g_mu);
    pkv::g_on.store(enable != 0);
    for (auto& e : pkv::g_entries) e.used = 0;
    return pkv::ok();
}

extern "C" int pkv_timer_read(int32_t entry, double* total_ms, int64_t* launches) {
    using pkv::fail;
    if (entry < 0 || entry >= PKV_TIMER_ENTRIES || !total_ms || !launches)
        return fail(PKV_EINVAL, "pkv_timer_read: bad entry or NULL output");
    std::lock_guard<std::mutex> lock(pkv::g_mu);
    pkv::EntryEvents& e = pkv::g_entries[entry];
    double sum = 0.0;
    for (size_t i = 0; i < e.used; ++i) {
        float ms = 0.f;
        hipError_t err = hipEventSynchronize(e.pool[i].stop);
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, e.pool[i].start, e.pool[i].stop);
        if (err != hipSuccess)
            return fail(PKV_EHIP, "pkv_timer_read: %s", hipGetErrorString(err));
        sum += ms;
    }
    *total_ms = sum;
    *launches = int64_t(e.used);
    e.used = 0;
    return pkv::ok();
}
