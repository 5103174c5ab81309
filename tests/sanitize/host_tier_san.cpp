// Host-only exercise of the decode-host cache core (host_tier_core.h) for the
// address, undefined-behaviour and thread sanitizers (built with g++ by
// tests/test_sanitizers.py, no HIP).  Random layer-step histories run on 1, 2,
// 3 and 5 worker threads, directly and through the dispatcher thread (each job
// first waits for a flag that another thread sets, standing in for the GPU
// event that follows the plan); generated blocks and trims come in between.
// Every run must leave exactly the cache of the one-thread direct run: slot
// contents, last-use stamps, union map, cache bytes and counters.  A budget
// too small for the working sets must fail the same way in every run.
// Exit status 0 on success; a sanitizer report aborts the process.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <thread>
#include <vector>

#include "host_tier_core.h"

using oasis::tier::Cache;

namespace {

struct Step {
    long long step;
    std::vector<int32_t> count, src, slots;  // [R][H], [R][H][K], [R][H][K]
};

// Each head keeps K distinct blocks; a step admits up to K new ones per head
// (the plan's sources) into random slots.
std::vector<Step> history(unsigned seed, int R, int H, int K, int n_blk, int steps) {
    std::mt19937 rng(seed);
    std::vector<int32_t> res((size_t)R * H * K);
    for (int u = 0; u < R * H; ++u) {
        std::vector<int> perm(n_blk);
        for (int b = 0; b < n_blk; ++b) perm[b] = b;
        std::shuffle(perm.begin(), perm.end(), rng);
        for (int k = 0; k < K; ++k) res[(size_t)u * K + k] = perm[k];
    }
    std::vector<Step> out;
    for (int t = 0; t < steps; ++t) {
        Step s;
        s.step = t + 1;
        s.count.assign((size_t)R * H, 0);
        s.src.assign((size_t)R * H * K, -1);
        for (int u = 0; u < R * H; ++u) {
            int32_t* row = &res[(size_t)u * K];
            const int c = t == 0 ? K : (int)(rng() % (K + 1));
            int n = 0;
            for (int tries = 0; n < c && tries < 64 * K; ++tries) {
                const int b = (int)(rng() % n_blk);
                bool have = false;
                for (int k = 0; k < K; ++k) have = have || row[k] == b;
                if (have && t > 0) continue;
                const int slot = t == 0 ? n : (int)(rng() % K);
                if (t > 0) row[slot] = b;
                s.src[(size_t)u * K + n] = t == 0 ? row[n] : b;
                ++n;
            }
            s.count[u] = n;
        }
        s.slots = res;
        out.push_back(std::move(s));
    }
    return out;
}

struct Snapshot {
    std::vector<int32_t> slot_blk, map;
    std::vector<int64_t> last;
    std::vector<uint8_t> bytes;
    int64_t stats[5];
    std::vector<int> status;
};

Snapshot run(const std::vector<Step>& hist, int R, int H, int K, int n_blk, int cap,
             size_t block_bytes, const std::vector<uint8_t>& remote, int workers,
             bool dispatched) {
    std::vector<uint8_t> cache((size_t)R * cap * block_bytes, 0xA5);
    std::vector<int32_t> map((size_t)R * n_blk, 7);
    std::vector<int32_t> capacity(R, cap);
    Cache c;
    if (!oasis::tier::cache_init(c, R, H, K, n_blk, capacity.data(), cap, block_bytes,
                                 remote.data(), cache.data(), map.data())) {
        std::fprintf(stderr, "cache_init rejected its arguments\n");
        std::exit(2);
    }
    for (uint8_t x : cache)
        if (x) {
            std::fprintf(stderr, "cache_init did not zero the cache\n");
            std::exit(2);
        }
    if (oasis::tier::cache_set_workers(c, workers) != oasis::tier::kOk) std::exit(2);
    Snapshot snap;
    struct Job {
        const Step* s;
        std::atomic<int>* ready;
        int* status;
    };
    std::vector<int> status(hist.size(), 0);
    auto extras = [&](const Step& s) {  // generated blocks and periodic trims between steps
        if (s.step == 5)
            for (int r = 0; r < R; ++r) (void)oasis::tier::cache_add_generated(c, r, n_blk - 1 - r, s.step, s.slots.data());
        if (s.step % 7 == 0) {
            std::vector<int32_t> target(R, cap / 2);
            (void)oasis::tier::cache_trim(c, target.data(), s.slots.data());
        }
    };
    // Steps go in groups of 4; the generated blocks and trims of a group's
    // steps follow the group (both modes, so their results must agree).
    const size_t group = 4;
    if (!dispatched) {
        for (size_t g0 = 0; g0 < hist.size(); g0 += group) {
            const size_t g1 = std::min(hist.size(), g0 + group);
            for (size_t i = g0; i < g1; ++i)
                status[i] = oasis::tier::cache_fetch(c, hist[i].step, hist[i].count.data(),
                                                     hist[i].src.data(), hist[i].slots.data());
            for (size_t i = g0; i < g1; ++i) extras(hist[i]);
        }
    } else {
        oasis::tier::Dispatcher<Job> d;
        if (!d.start([] {}, [&](const Job& j) {
                for (int spin = 0; j.ready->load(std::memory_order_acquire) == 0; ++spin)
                    std::this_thread::yield();  // the producer sets it: the wait ends
                *j.status = oasis::tier::cache_fetch(c, j.s->step, j.s->count.data(),
                                                     j.s->src.data(), j.s->slots.data());
                return *j.status;
            }))
            std::exit(2);
        std::vector<std::unique_ptr<std::atomic<int>>> flags;
        for (size_t i = 0; i < hist.size(); ++i) flags.emplace_back(new std::atomic<int>(0));
        // A producer thread releases each group's flags after a short delay,
        // while the dispatcher already waits on them.  Host calls between
        // groups drain the queue first, as the library's entry points do.
        for (size_t g0 = 0; g0 < hist.size(); g0 += group) {
            const size_t g1 = std::min(hist.size(), g0 + group);
            for (size_t i = g0; i < g1; ++i) d.submit(Job{&hist[i], flags[i].get(), &status[i]});
            std::thread producer([&, g0, g1] {
                for (size_t i = g0; i < g1; ++i) {
                    std::this_thread::sleep_for(std::chrono::microseconds(50));
                    flags[i]->store(1, std::memory_order_release);
                }
            });
            (void)d.drain();
            producer.join();
            for (size_t i = g0; i < g1; ++i) extras(hist[i]);
        }
        d.finish();
    }
    snap.slot_blk = c.slot_blk;
    snap.last.assign(c.last.begin(), c.last.end());
    snap.map = map;
    snap.bytes = cache;
    oasis::tier::cache_state(c, nullptr, nullptr, snap.stats, 0);
    snap.stats[4] = 0;  // host time differs between runs
    snap.status = status;
    oasis::tier::stop_pool(c);
    // consistency of the union map with the slots
    for (int r = 0; r < R; ++r)
        for (int s = 0; s < cap; ++s) {
            const int b = c.slot_blk[(size_t)r * cap + s];
            if (b >= 0 && map[(size_t)r * n_blk + b] != s) {
                std::fprintf(stderr, "map and slots disagree (r %d slot %d)\n", r, s);
                std::exit(3);
            }
        }
    return snap;
}

bool same(const Snapshot& a, const Snapshot& b) {
    for (int i = 0; i < 5; ++i)
        if (a.stats[i] != b.stats[i]) return false;
    return a.slot_blk == b.slot_blk && a.last == b.last && a.map == b.map && a.bytes == b.bytes &&
           a.status == b.status;
}

int check_case(unsigned seed, int R, int H, int K, int n_blk, int cap, bool expect_fail) {
    const size_t block_bytes = 40;
    std::vector<uint8_t> remote((size_t)R * n_blk * block_bytes);
    std::mt19937 rng(seed * 7 + 1);
    for (auto& x : remote) x = (uint8_t)(rng() & 0xff);
    const auto hist = history(seed, R, H, K, n_blk, 24);
    const Snapshot ref = run(hist, R, H, K, n_blk, cap, block_bytes, remote, 1, false);
    bool failed = false;
    for (int st : ref.status) failed = failed || st != oasis::tier::kOk;
    if (failed != expect_fail || (ref.stats[2] > 0) != expect_fail) {
        std::fprintf(stderr, "case seed %u: failure %d, expected %d\n", seed, (int)failed, (int)expect_fail);
        return 1;
    }
    for (int w : {1, 2, 3, 5})
        for (bool disp : {false, true}) {
            if (w == 1 && !disp) continue;
            const Snapshot s = run(hist, R, H, K, n_blk, cap, block_bytes, remote, w, disp);
            if (!same(ref, s)) {
                std::fprintf(stderr, "case seed %u: %d workers%s differs from one thread\n", seed, w,
                             disp ? " (dispatcher)" : "");
                return 1;
            }
        }
    std::printf("case seed %u R %d H %d K %d n_blk %d cap %d: %lld fetched, %lld evicted, %lld failed\n",
                seed, R, H, K, n_blk, cap, (long long)ref.stats[0], (long long)ref.stats[1],
                (long long)ref.stats[2]);
    return 0;
}

}  // namespace

int main() {
    int bad = 0;
    bad += check_case(1, 3, 2, 4, 48, 2 * 4 + 12, false);
    bad += check_case(2, 5, 4, 3, 40, 4 * 3 + 6, false);
    bad += check_case(3, 2, 8, 2, 64, 8 * 2 + 9, false);
    bad += check_case(4, 4, 4, 4, 40, 9, true);  // budget below the working sets
    std::printf(bad ? "FAILED\n" : "ok\n");
    return bad ? 1 : 0;
}
