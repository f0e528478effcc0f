// host_threads.h -- the worker pool of libecf8's host encoders (internal).
#pragma once

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <thread>
#include <vector>

namespace ecf8_host {

// Threads for `items` units of work, at least min_per_worker each; ECF8_THREADS
// overrides the hardware count, capped at 64.
inline int worker_count(uint64_t items, uint64_t min_per_worker)
{
    unsigned hw = std::thread::hardware_concurrency();
    if (hw == 0) hw = 1;
    if (const char* env = std::getenv("ECF8_THREADS")) {
        int v = std::atoi(env);
        if (v > 0) hw = (unsigned)v;
    }
    hw = std::min(hw, 64u);
    uint64_t by_work = std::max<uint64_t>(1, items / std::max<uint64_t>(1, min_per_worker));
    return (int)std::min<uint64_t>(hw, by_work);
}

// fn(0) .. fn(workers - 1), the first on the calling thread.
template <class F>
void run_parallel(int workers, F&& fn)
{
    if (workers <= 1) {
        fn(0);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(workers - 1);
    for (int w = 1; w < workers; ++w) pool.emplace_back([&, w] { fn(w); });
    fn(0);
    for (auto& t : pool) t.join();
}

}  // namespace ecf8_host
