// Decode-host block cache: the CPU state and work behind the oasis_host_tier_*
// entry points, in plain C++ (no HIP), so the same code also builds host-only
// under the address, undefined-behaviour and thread sanitizers.
//
// Sources: OasisKV paperpeel v2 text, §3.2.1 (ii) (the decode host fetches
// whole blocks -- every KV head's entries -- for the union of the heads'
// selections), §3.2.2 (union block mapping: remote block -> decode-host slot,
// per request) and §3.2.3 (per-request budget; least recently used prompt
// blocks are evicted while generated blocks and the current working set are
// kept; evicted blocks are fetched again when selected).
//
// Cache: per request r, cap[r] slots of block_bytes in `cache`, the block each
// slot holds (-1 free), its last use, and the union map map[r][b] = slot of
// remote block b (-1 absent).  A fetch of one layer-step splits the requests
// over a pool of host threads: worker w of W takes r = w, w+W, ... with scratch
// of its own, so the result does not depend on W.
// Dispatcher: an in-order job queue served by one thread (the library's jobs
// wait for a GPU event, fetch, and launch the gather); the first error of a
// job is kept (sticky) for the caller's drain.
#pragma once

#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <deque>
#include <mutex>
#include <thread>
#include <vector>

namespace oasis {
namespace tier {

constexpr int kOk = 0;       // OASIS_OK
constexpr int kInval = -1;   // OASIS_EINVAL
constexpr int kThread = -4;  // OASIS_EHIP (a thread could not be started)

// Per-thread working memory of a fetch: epoch marks over one request's
// blocks, that request's union, and counters (summed by the state query).
struct Scratch {
    std::vector<unsigned> in_union;  // [n_blk] epoch marks
    std::vector<unsigned> in_keep;   // [n_blk] epoch marks
    std::vector<int> uni;
    unsigned epoch = 0;
    long long fetched = 0, evicted = 0, failed = 0;

    void begin_request() {
        if (++epoch == 0) {  // wrapped: old marks could match again
            std::fill(in_union.begin(), in_union.end(), 0u);
            std::fill(in_keep.begin(), in_keep.end(), 0u);
            epoch = 1;
        }
        uni.clear();
    }
};

struct Cache {
    int R = 0, H = 0, K = 0, n_blk = 0, cap_max = 0;
    size_t block_bytes = 0;
    std::vector<int> cap;            // [R]
    const uint8_t* remote = nullptr;  // [R][n_blk][block_bytes]
    uint8_t* cache = nullptr;         // [R][cap_max][block_bytes]
    int32_t* map = nullptr;           // [R][n_blk]
    std::vector<int> slot_blk;       // [R][cap_max], -1 free
    std::vector<long long> last;     // [R][cap_max]
    std::vector<uint8_t> generated;  // [R][n_blk]
    std::vector<Scratch> scr;        // [workers]; scr[0] is the calling thread's
    long long base_fetched = 0, base_evicted = 0, base_failed = 0;  // of retired scratch
    long long fetch_ns = 0;          // host time inside fetches
    // worker pool (threads 1..W-1; the calling thread is worker 0)
    std::vector<std::thread> pool;
    std::mutex mu;
    std::condition_variable go, done;
    long long job_gen = 0;
    int job_left = 0, job_status = 0;
    bool stop = false;
    long long job_step = 0;
    const int32_t *job_count = nullptr, *job_src = nullptr, *job_slots = nullptr;
};

inline void init_scratch(Cache& t, int W) {
    for (const Scratch& x : t.scr) {
        t.base_fetched += x.fetched;
        t.base_evicted += x.evicted;
        t.base_failed += x.failed;
    }
    t.scr.assign(W, Scratch{});
    for (Scratch& x : t.scr) {
        x.in_union.assign(t.n_blk, 0u);
        x.in_keep.assign(t.n_blk, 0u);
        x.uni.reserve((size_t)t.H * t.K);
    }
}

// Validates the arguments and sets up the state; false on a bad argument.
// Every cache byte is written once here from the host: pinned pages the host
// has not written cost a fault per page on first touch (about 8x the copy of
// a whole block), which would otherwise land inside the fetches.
inline bool cache_init(Cache& t, int R, int H, int K, int n_blk, const int32_t* capacity,
                       int cap_max, size_t block_bytes, const void* remote, void* cache,
                       int32_t* map) {
    if (R <= 0 || H <= 0 || K <= 0 || n_blk <= 0 || cap_max <= 0 || block_bytes == 0 ||
        !capacity || !remote || !cache || !map)
        return false;
    for (int r = 0; r < R; ++r)
        if (capacity[r] < 0 || capacity[r] > cap_max) return false;
    t.R = R;
    t.H = H;
    t.K = K;
    t.n_blk = n_blk;
    t.cap_max = cap_max;
    t.block_bytes = block_bytes;
    t.cap.assign(capacity, capacity + R);
    t.remote = static_cast<const uint8_t*>(remote);
    t.cache = static_cast<uint8_t*>(cache);
    t.map = map;
    t.slot_blk.assign((size_t)R * cap_max, -1);
    t.last.assign((size_t)R * cap_max, -1);
    t.generated.assign((size_t)R * n_blk, 0);
    init_scratch(t, 1);
    for (size_t i = 0; i < (size_t)R * n_blk; ++i) map[i] = -1;
    std::memset(cache, 0, (size_t)R * cap_max * block_bytes);
    return true;
}

// The unprotected slot of request r with the smallest (last use, slot), -1 if none.
inline int victim(Cache& t, Scratch& x, int r) {
    int best = -1;
    long long best_last = 0;
    for (int s = 0; s < t.cap[r]; ++s) {
        const int b = t.slot_blk[(size_t)r * t.cap_max + s];
        if (b < 0 || x.in_keep[b] == x.epoch || t.generated[(size_t)r * t.n_blk + b]) continue;
        const long long l = t.last[(size_t)r * t.cap_max + s];
        if (best < 0 || l < best_last) {  // ties: the lower slot (first seen) wins
            best = s;
            best_last = l;
        }
    }
    return best;
}

// Slot for block b of request r: the lowest free slot, else the least
// recently used evictable one (-1 if none).
inline int place(Cache& t, Scratch& x, int r, int b) {
    int s = -1;
    for (int i = 0; i < t.cap[r]; ++i)
        if (t.slot_blk[(size_t)r * t.cap_max + i] < 0) {
            s = i;
            break;
        }
    if (s < 0) {
        s = victim(t, x, r);
        if (s < 0) return -1;
        const int old = t.slot_blk[(size_t)r * t.cap_max + s];
        t.map[(size_t)r * t.n_blk + old] = -1;
        ++x.evicted;
    }
    t.slot_blk[(size_t)r * t.cap_max + s] = b;
    t.map[(size_t)r * t.n_blk + b] = s;
    return s;
}

// Marks request r's HBM working set (slot_block rows of every head) as kept.
inline void keep_working_set(const Cache& t, Scratch& x, int r, const int32_t* slot_block) {
    if (!slot_block) return;
    for (size_t i = 0; i < (size_t)t.H * t.K; ++i) {
        const int b = slot_block[(size_t)r * t.H * t.K + i];
        if (b >= 0 && b < t.n_blk) x.in_keep[b] = x.epoch;
    }
}

// One layer-step of the requests r = w, w+W, ...: union of the planned
// sources, fetch of the absent blocks, last-use stamps.  Returns kOk, or kInval
// when a request's budget held no evictable block (that request's remaining
// blocks are skipped; `failed` counts them).
inline int fetch_share(Cache& t, int w, int W, long long step, const int32_t* count,
                       const int32_t* src, const int32_t* slots) {
    Scratch& x = t.scr[w];
    int st = kOk;
    for (int r = w; r < t.R; r += W) {
        x.begin_request();
        for (int g = 0; g < t.H; ++g) {
            const size_t u = (size_t)r * t.H + g;
            const int n = std::min(std::max(count[u], 0), t.K);
            for (int i = 0; i < n; ++i) {
                const int b = src[u * t.K + i];
                if (b < 0 || b >= t.n_blk || x.in_union[b] == x.epoch) continue;
                x.in_union[b] = x.epoch;
                x.in_keep[b] = x.epoch;
                x.uni.push_back(b);
            }
        }
        keep_working_set(t, x, r, slots);
        for (int b : x.uni) {
            if (t.map[(size_t)r * t.n_blk + b] >= 0) continue;
            const int s = place(t, x, r, b);
            if (s < 0) {
                ++x.failed;
                st = kInval;
                continue;
            }
            std::memcpy(t.cache + ((size_t)r * t.cap_max + s) * t.block_bytes,
                        t.remote + ((size_t)r * t.n_blk + b) * t.block_bytes, t.block_bytes);
            ++x.fetched;
        }
        for (int b : x.uni) {
            const int s = t.map[(size_t)r * t.n_blk + b];
            if (s >= 0) t.last[(size_t)r * t.cap_max + s] = step;
        }
    }
    return st;
}

// `seen` starts at the job generation current when the worker was spawned
// (no job in flight then): the counter keeps running across pool restarts,
// and a job posted before this thread first takes the lock must still run.
inline void worker_main(Cache* t, int w, long long seen) {
    std::unique_lock<std::mutex> lk(t->mu);
    for (;;) {
        t->go.wait(lk, [&] { return t->stop || t->job_gen != seen; });
        if (t->stop) return;
        seen = t->job_gen;
        const int W = (int)t->scr.size();
        const long long step = t->job_step;
        const int32_t *count = t->job_count, *src = t->job_src, *slots = t->job_slots;
        lk.unlock();
        const int st = fetch_share(*t, w, W, step, count, src, slots);
        lk.lock();
        if (st != kOk) t->job_status = st;
        if (--t->job_left == 0) t->done.notify_one();
    }
}

inline void stop_pool(Cache& t) {
    {
        std::lock_guard<std::mutex> lk(t.mu);
        t.stop = true;
    }
    t.go.notify_all();
    for (std::thread& th : t.pool) th.join();
    t.pool.clear();
    t.stop = false;
}

// Every request of one layer-step, split over the pool.
inline int cache_fetch(Cache& t, long long step, const int32_t* count, const int32_t* src,
                       const int32_t* slots) {
    const auto t0 = std::chrono::steady_clock::now();
    const int W = (int)t.scr.size();
    int st;
    if (W == 1) {
        st = fetch_share(t, 0, 1, step, count, src, slots);
    } else {
        {
            std::lock_guard<std::mutex> lk(t.mu);
            t.job_step = step;
            t.job_count = count;
            t.job_src = src;
            t.job_slots = slots;
            t.job_status = kOk;
            t.job_left = W - 1;
            ++t.job_gen;
        }
        t.go.notify_all();
        st = fetch_share(t, 0, W, step, count, src, slots);
        std::unique_lock<std::mutex> lk(t.mu);
        t.done.wait(lk, [&] { return t.job_left == 0; });
        if (t.job_status != kOk) st = t.job_status;
    }
    t.fetch_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                      std::chrono::steady_clock::now() - t0).count();
    return st;
}

// Restarts the pool with W threads (1..64).  kThread if a thread could not be
// started (the cache is then left with one worker).
inline int cache_set_workers(Cache& t, int W) {
    if (W < 1 || W > 64) return kInval;
    stop_pool(t);
    init_scratch(t, W);
    try {
        for (int w = 1; w < W; ++w) t.pool.emplace_back(worker_main, &t, w, t.job_gen);
    } catch (...) {
        stop_pool(t);
        init_scratch(t, 1);
        return kThread;
    }
    return kOk;
}

inline int cache_add_generated(Cache& t, int req, int block, long long step,
                               const int32_t* slot_block) {
    if (req < 0 || req >= t.R || block < 0 || block >= t.n_blk) return kInval;
    Scratch& x = t.scr[0];
    x.begin_request();
    keep_working_set(t, x, req, slot_block);
    int s = t.map[(size_t)req * t.n_blk + block];
    if (s < 0 && (s = place(t, x, req, block)) < 0) {
        ++x.failed;
        return kInval;
    }
    t.generated[(size_t)req * t.n_blk + block] = 1;
    t.last[(size_t)req * t.cap_max + s] = step;
    return kOk;
}

// Periodic pass: evict, by the victim order, until request r holds at most
// target[r] blocks (protected blocks stay, so fewer may go).
inline int cache_trim(Cache& t, const int32_t* target, const int32_t* slot_block) {
    if (!target) return kInval;
    Scratch& x = t.scr[0];
    for (int r = 0; r < t.R; ++r) {
        x.begin_request();
        keep_working_set(t, x, r, slot_block);
        int live = 0;
        for (int s = 0; s < t.cap[r]; ++s) live += t.slot_blk[(size_t)r * t.cap_max + s] >= 0;
        while (live > target[r]) {
            const int s = victim(t, x, r);
            if (s < 0) break;
            const size_t i = (size_t)r * t.cap_max + s;
            t.map[(size_t)r * t.n_blk + t.slot_blk[i]] = -1;
            t.slot_blk[i] = -1;
            t.last[i] = -1;
            ++x.evicted;
            --live;
        }
    }
    return kOk;
}

// slot_block_out / last_out [R][cap_max] (either may be null); stats_out[5] =
// blocks fetched, blocks evicted, blocks that found no slot, `steps`, host
// nanoseconds spent inside fetches.
inline void cache_state(const Cache& t, int32_t* slot_block_out, int64_t* last_out,
                        int64_t* stats_out, long long steps) {
    const size_t n = (size_t)t.R * t.cap_max;
    if (slot_block_out)
        for (size_t i = 0; i < n; ++i) slot_block_out[i] = t.slot_blk[i];
    if (last_out)
        for (size_t i = 0; i < n; ++i) last_out[i] = t.last[i];
    if (stats_out) {
        long long f = t.base_fetched, e = t.base_evicted, x = t.base_failed;
        for (const Scratch& s : t.scr) {
            f += s.fetched;
            e += s.evicted;
            x += s.failed;
        }
        stats_out[0] = f;
        stats_out[1] = e;
        stats_out[2] = x;
        stats_out[3] = steps;
        stats_out[4] = t.fetch_ns;
    }
}

// In-order jobs served by one thread: run(job) returns a status; the first
// non-kOk one is kept until the owner is destroyed.
template <class Job>
class Dispatcher {
public:
    ~Dispatcher() { finish(); }

    bool running() const { return th_.joinable(); }

    // Starts the thread: init() once on it, then run(job) for each job.
    template <class Init, class Run>
    bool start(Init init, Run run) {
        if (th_.joinable()) return true;
        stopping_ = false;
        try {
            th_ = std::thread([this, init, run]() mutable {
                init();
                std::unique_lock<std::mutex> lk(mu_);
                for (;;) {
                    go_.wait(lk, [&] { return stopping_ || !jobs_.empty(); });
                    if (jobs_.empty()) return;  // stop requested and drained
                    const Job j = jobs_.front();
                    jobs_.pop_front();
                    lk.unlock();
                    const int st = run(j);
                    lk.lock();
                    if (st != kOk && status_ == kOk) status_ = st;
                    ++issued_;
                    issued_cv_.notify_all();
                }
            });
        } catch (...) {
            return false;
        }
        return true;
    }

    void submit(const Job& j) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            jobs_.push_back(j);
            ++submitted_;
        }
        go_.notify_one();
    }

    // Waits until every submitted job has run; returns the sticky status.
    int drain() {
        std::unique_lock<std::mutex> lk(mu_);
        issued_cv_.wait(lk, [&] { return issued_ == submitted_; });
        return status_;
    }

    // Runs what was submitted, then ends the thread.
    void finish() {
        if (!th_.joinable()) return;
        {
            std::lock_guard<std::mutex> lk(mu_);
            stopping_ = true;
        }
        go_.notify_all();
        th_.join();
    }

private:
    std::deque<Job> jobs_;
    std::thread th_;
    std::mutex mu_;
    std::condition_variable go_, issued_cv_;
    long long submitted_ = 0, issued_ = 0;
    int status_ = kOk;
    bool stopping_ = false;
};

}  // namespace tier
}  // namespace oasis
