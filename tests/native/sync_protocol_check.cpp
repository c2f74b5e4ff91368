// CPU model of the library's cross-workgroup wait protocol (the arrival
// counters of nvfp4_kernels.hip and the host's slot bookkeeping of
// nvfp4_api.cpp), run with one thread per workgroup to check the protocol's
// logic: zero-first (the first workgroups clear the outputs and arrive; the
// others wait for them before their first atomic max), the grid-wide wait
// (every workgroup arrives after its atomics; the last arrival publishes the
// slot's final count to flag words, which the others poll, one of several
// per workgroup), slots reused
// by later launches with host-tracked bases, and the bounded wait that gives
// up and records the failure in an error word the next call reports.
//
// Each launch draws fresh per-workgroup values; after the grid-wide wait
// every workgroup must read exactly the maximum over all workgroups, and
// after the launch the outputs must equal it (a maximum combined before the
// zeroing, or read before the last arrival, would show).  Random short
// sleeps shuffle the interleavings.  Prints "OK <n> launches" on success.
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

namespace {

constexpr int kSlots = 4;                  // few slots, so they are reused often
std::atomic<uint64_t> g_count[kSlots];     // the device counters (never reset)
std::atomic<uint32_t> g_err{0};            // the pinned error word
constexpr int kFlagLines = 4;              // flag words per slot (fewer than workgroups)
std::atomic<uint64_t> g_flag[kSlots][kFlagLines];   // published final counts (never reset)

struct SyncArg { uint64_t base; int slot; };

// host side: slots in turn, each advanced by its launch's arrivals
struct Host {
    uint64_t next = 0, count[kSlots] = {};
    bool fail_next = false;
    SyncArg take(uint64_t arrivals) {
        const int s = (int)(next++ % kSlots);
        SyncArg a{count[s], s};
        if (fail_next) { a.base += (uint64_t)1 << 40; fail_next = false; }
        count[s] += arrivals;
        return a;
    }
};

void arrive(const SyncArg& s) { g_count[s.slot].fetch_add(1, std::memory_order_release); }

// one poller; false when the bound passed (the error word is then set)
bool poll(const SyncArg& s, uint64_t n, std::chrono::milliseconds bound) {
    const auto t0 = std::chrono::steady_clock::now();
    while (g_count[s.slot].load(std::memory_order_acquire) < s.base + n) {
        if (std::chrono::steady_clock::now() - t0 > bound) { g_err.store(1); return false; }
        std::this_thread::yield();
    }
    return true;
}

// the grid-wide wait: arrive; the last arrival publishes base + n to every
// flag word of the slot, the others poll word g % kFlagLines; false when the
// bound passed (the error word is then set)
bool grid_wait(const SyncArg& s, uint64_t n, int g, std::chrono::milliseconds bound) {
    const uint64_t target = s.base + n;
    const uint64_t old = g_count[s.slot].fetch_add(1, std::memory_order_acq_rel);
    if (old + 1 == target) {
        for (auto& f : g_flag[s.slot]) f.store(target, std::memory_order_release);
        return true;
    }
    const auto t0 = std::chrono::steady_clock::now();
    while (g_flag[s.slot][g % kFlagLines].load(std::memory_order_acquire) < target) {
        if (std::chrono::steady_clock::now() - t0 > bound) { g_err.store(1); return false; }
        std::this_thread::yield();
    }
    return true;
}

void atomic_max(std::atomic<uint32_t>& a, uint32_t v) {
    uint32_t cur = a.load(std::memory_order_relaxed);
    while (cur < v && !a.compare_exchange_weak(cur, v, std::memory_order_relaxed)) {}
}

// one launch of G workgroups over an output of n entries, zw of which zero it
bool launch(Host& host, int G, int zw, std::vector<std::atomic<uint32_t>>& out, std::mt19937& rng, bool expect_fail,
            std::chrono::milliseconds bound) {
    const SyncArg zs = host.take((uint64_t)zw), bs = host.take((uint64_t)G);
    std::vector<uint32_t> val(G);
    for (auto& v : val) v = 1u + (uint32_t)(rng() % 1000000u);
    uint32_t expect = 0;
    for (uint32_t v : val) expect = v > expect ? v : expect;
    std::vector<int> delay(G);
    for (auto& d : delay) d = (int)(rng() % 200);
    std::atomic<int> bad{0}, gave_up{0};
    const int n = (int)out.size();
    auto wg = [&](int g) {
        std::this_thread::sleep_for(std::chrono::microseconds(delay[g]));
        if (g < zw) {   // zero-first: a slice each, then arrive
            for (int i = g; i < n; i += zw) out[i].store(0, std::memory_order_relaxed);
            arrive(zs);
        }
        // as in the kernels: a zero wait that gave up skips the atomics but the
        // workgroup still arrives, so the slot's count stays what the host assumed
        if (poll(zs, (uint64_t)zw, bound)) {
            for (int i = 0; i < n; ++i) atomic_max(out[i], val[g] - (uint32_t)(i % 3));
        } else {
            gave_up.fetch_add(1);
        }
        if (!grid_wait(bs, (uint64_t)G, g, bound)) { gave_up.fetch_add(1); return; }
        for (int i = 0; i < n; ++i)
            if (out[i].load(std::memory_order_relaxed) != expect - (uint32_t)(i % 3)) bad.fetch_add(1);
    };
    std::vector<std::thread> th;
    for (int g = 0; g < G; ++g) th.emplace_back(wg, g);
    for (auto& t : th) t.join();
    if (expect_fail) return gave_up.load() > 0 && g_err.exchange(0) == 1;
    if (gave_up.load() != 0 || g_err.load() != 0 || bad.load() != 0) return false;
    for (int i = 0; i < n; ++i)
        if (out[i].load() != expect - (uint32_t)(i % 3)) return false;
    return true;
}

}  // namespace

int main() {
    std::mt19937 rng(12345);
    Host host;
    std::vector<std::atomic<uint32_t>> out(257);
    for (auto& o : out) o.store(0xFFFFFFFFu);   // stale contents: the zeroing must clear them
    int launches = 0;
    for (int it = 0; it < 60; ++it) {
        const int G = 8 + (int)(rng() % 57), zw = 1 + (int)(rng() % 3);
        if (!launch(host, G, zw, out, rng, false, std::chrono::milliseconds(5000))) {
            std::printf("FAIL launch %d (G=%d zw=%d)\n", it, G, zw);
            return 1;
        }
        ++launches;
        if (it % 20 == 19) {   // a forced failure: the waits give up, the error word is set and read once
            host.fail_next = true;
            if (!launch(host, 16, 1, out, rng, true, std::chrono::milliseconds(50))) {
                std::printf("FAIL forced give-up after launch %d\n", it);
                return 1;
            }
            ++launches;
        }
    }
    std::printf("OK %d launches\n", launches);
    return 0;
}
