// Decode-host block cache between a remote KV store and the GPU's resident
// slots, and the gather that reads the GPU's planned blocks through it.
//
// Sources: OasisKV paperpeel v2 text, §3.2.1 (ii) (the decode host fetches
// whole blocks -- every KV head's entries -- for the union of the heads'
// selections, even when one head alone selects a block), §3.2.2 (a union
// block mapping records where each selected remote block sits in decode-host
// memory; the GPU gather reads the head slices through it) and §3.2.3 (a
// per-request budget of f_Host*P + F blocks; least recently used prompt blocks
// are evicted while generated blocks and the current working set are kept;
// evicted blocks stay in remote memory and are fetched again when selected).
//
// Layouts (caller-owned memory; whole blocks of H interleaved K|V records):
//   remote  [R][n_blk][H][rec]   rec = tile_stride elements (K tile, V tile)
//   cache   [R][cap_max][H][rec] pinned host memory the GPU can address
//   map     [R][n_blk] int32     cache slot of a remote block, -1 if absent;
//                                pinned, read by the gather kernel
// The manager's state (slots, last use, generated flags) lives in this
// object; its work is plain CPU code, run either directly (host call) or by
// the tier's dispatcher thread, which takes submitted layer-steps in order:
// wait on the host for the event that follows the plan, copy the plan back,
// fetch, then launch the mapped gather on the caller's copy stream and record
// the caller's event after it.  No GPU queue ever waits on host memory; the
// caller orders later GPU work on that event once the host call
// oasis_host_tier_wait_issued says it has been recorded.  Requests are
// independent (each owns its rows of every array), so a fetch may split them
// over a small pool of host threads: worker w of W takes r = w, w+W, ... with
// scratch of its own, and the result does not depend on W.
#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "oasis_internal.h"

namespace oasis {

// Per-thread working memory of a fetch: epoch marks over one request's
// blocks, that request's union, and counters (summed by the state query).
struct TierScratch {
    std::vector<unsigned> in_union;   // [n_blk] epoch marks
    std::vector<unsigned> in_keep;    // [n_blk] epoch marks
    std::vector<int> uni;
    unsigned epoch = 0;
    long long fetched = 0, evicted = 0, failed = 0;

    void begin_request() {
        if (++epoch == 0) {           // wrapped: old marks could match again
            std::fill(in_union.begin(), in_union.end(), 0u);
            std::fill(in_keep.begin(), in_keep.end(), 0u);
            epoch = 1;
        }
        uni.clear();
    }
};

// One submitted layer-step (see oasis_host_tier_submit).
struct TierJob {
    const int32_t *plan_count, *plan_src, *plan_dst, *slot_block;  // device
    const void *dev_k, *dev_v, *dev_map;                            // device views
    void *res_k, *res_v;
    int tile_u4;
    long long stride_u4;
    hipEvent_t after, done;
    hipStream_t copy_stream;
};

}  // namespace oasis

struct oasis_host_tier {
    int R, H, K, n_blk, cap_max;
    size_t block_bytes;
    std::vector<int> cap;             // [R]
    const uint8_t* remote;            // [R][n_blk][block_bytes]
    uint8_t* cache;                   // [R][cap_max][block_bytes]
    int32_t* map;                     // [R][n_blk]
    std::vector<int> slot_blk;        // [R][cap_max], -1 free
    std::vector<long long> last;      // [R][cap_max]
    std::vector<uint8_t> generated;   // [R][n_blk]
    std::vector<oasis::TierScratch> scr;  // [workers]; scr[0] is the calling thread's
    long long clock = 0;              // stream-ordered calls stamp with their own counter
    long long base_fetched = 0, base_evicted = 0, base_failed = 0;  // of retired scratch
    long long fetch_ns = 0;           // host time inside fetch calls
    // dispatcher: submitted jobs, its thread, pinned staging of the plan and a
    // private non-blocking stream for copying it back (set up on first submit)
    std::deque<oasis::TierJob> jobs;
    std::thread dispatcher;
    std::mutex dmu;
    std::condition_variable dgo, dissued;
    long long submitted = 0, issued = 0;
    int async_status = 0;             // first error of a dispatched job (sticky)
    bool dstop = false;
    int device = -1;
    hipStream_t dstream = nullptr;
    int32_t* st_count = nullptr;      // [R][H]
    int32_t* st_src = nullptr;        // [R][H][K]
    int32_t* st_slots = nullptr;      // [R][H][K]
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

namespace oasis {

static int tier_victim(oasis_host_tier* t, TierScratch& x, int r) {
    int best = -1;
    long long best_last = 0;
    for (int s = 0; s < t->cap[r]; ++s) {
        const int b = t->slot_blk[(size_t)r * t->cap_max + s];
        if (b < 0 || x.in_keep[b] == x.epoch || t->generated[(size_t)r * t->n_blk + b]) continue;
        const long long l = t->last[(size_t)r * t->cap_max + s];
        if (best < 0 || l < best_last) {  // ties: the lower slot (first seen) wins
            best = s;
            best_last = l;
        }
    }
    return best;
}

// Slot for block b of request r: the lowest free slot, else the least
// recently used evictable one (-1 if none).
static int tier_place(oasis_host_tier* t, TierScratch& x, int r, int b) {
    int s = -1;
    for (int i = 0; i < t->cap[r]; ++i)
        if (t->slot_blk[(size_t)r * t->cap_max + i] < 0) {
            s = i;
            break;
        }
    if (s < 0) {
        s = tier_victim(t, x, r);
        if (s < 0) return -1;
        const int old = t->slot_blk[(size_t)r * t->cap_max + s];
        t->map[(size_t)r * t->n_blk + old] = -1;
        ++x.evicted;
    }
    t->slot_blk[(size_t)r * t->cap_max + s] = b;
    t->map[(size_t)r * t->n_blk + b] = s;
    return s;
}

// One layer-step of the requests r = w, w+W, ...: union of the planned
// sources, fetch of the absent blocks, last-use stamps.  Returns OASIS_OK or
// OASIS_EINVAL when a request's budget held no evictable block (that
// request's remaining blocks are skipped; failed counts them).
static int fetch_share(oasis_host_tier* t, int w, int W, long long step, const int32_t* count,
                       const int32_t* src, const int32_t* slots) {
    TierScratch& x = t->scr[w];
    int st = OASIS_OK;
    for (int r = w; r < t->R; r += W) {
        x.begin_request();
        for (int g = 0; g < t->H; ++g) {
            const size_t u = (size_t)r * t->H + g;
            const int n = count[u] < t->K ? count[u] : t->K;
            for (int i = 0; i < n; ++i) {
                const int b = src[u * t->K + i];
                if (b < 0 || b >= t->n_blk || x.in_union[b] == x.epoch) continue;
                x.in_union[b] = x.epoch;
                x.in_keep[b] = x.epoch;
                x.uni.push_back(b);
            }
            if (slots)
                for (int k = 0; k < t->K; ++k) {
                    const int b = slots[u * t->K + k];
                    if (b >= 0 && b < t->n_blk) x.in_keep[b] = x.epoch;
                }
        }
        for (int b : x.uni) {
            if (t->map[(size_t)r * t->n_blk + b] >= 0) continue;
            const int s = tier_place(t, x, r, b);
            if (s < 0) {
                ++x.failed;
                st = OASIS_EINVAL;
                continue;
            }
            std::memcpy(t->cache + ((size_t)r * t->cap_max + s) * t->block_bytes,
                        t->remote + ((size_t)r * t->n_blk + b) * t->block_bytes, t->block_bytes);
            ++x.fetched;
        }
        for (int b : x.uni) {
            const int s = t->map[(size_t)r * t->n_blk + b];
            if (s >= 0) t->last[(size_t)r * t->cap_max + s] = step;
        }
    }
    return st;
}

// `seen` starts at the job generation current when the worker was spawned
// (no job in flight then): the counter keeps running across pool restarts,
// and a job posted before this thread first takes the lock must still run.
static void tier_worker(oasis_host_tier* t, int w, long long seen) {
    std::unique_lock<std::mutex> lk(t->mu);
    for (;;) {
        t->go.wait(lk, [&] { return t->stop || t->job_gen != seen; });
        if (t->stop) return;
        seen = t->job_gen;
        const int W = (int)t->scr.size();
        const long long step = t->job_step;
        const int32_t *count = t->job_count, *src = t->job_src, *slots = t->job_slots;
        lk.unlock();
        const int st = fetch_share(t, w, W, step, count, src, slots);
        lk.lock();
        if (st != OASIS_OK) t->job_status = st;
        if (--t->job_left == 0) t->done.notify_one();
    }
}

static void stop_pool(oasis_host_tier* t) {
    {
        std::lock_guard<std::mutex> lk(t->mu);
        t->stop = true;
    }
    t->go.notify_all();
    for (std::thread& th : t->pool) th.join();
    t->pool.clear();
    t->stop = false;
}

// Every request of one layer-step, split over the pool.
static int tier_fetch(oasis_host_tier* t, long long step, const int32_t* count,
                      const int32_t* src, const int32_t* slots) {
    const auto t0 = std::chrono::steady_clock::now();
    const int W = (int)t->scr.size();
    int st;
    if (W == 1) {
        st = fetch_share(t, 0, 1, step, count, src, slots);
    } else {
        {
            std::lock_guard<std::mutex> lk(t->mu);
            t->job_step = step;
            t->job_count = count;
            t->job_src = src;
            t->job_slots = slots;
            t->job_status = OASIS_OK;
            t->job_left = W - 1;
            ++t->job_gen;
        }
        t->go.notify_all();
        st = fetch_share(t, 0, W, step, count, src, slots);
        std::unique_lock<std::mutex> lk(t->mu);
        t->done.wait(lk, [&] { return t->job_left == 0; });
        if (t->job_status != OASIS_OK) st = t->job_status;
    }
    t->fetch_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                       std::chrono::steady_clock::now() - t0).count();
    return st;
}


static void init_scratch(oasis_host_tier* t, int W) {
    for (const TierScratch& x : t->scr) {
        t->base_fetched += x.fetched;
        t->base_evicted += x.evicted;
        t->base_failed += x.failed;
    }
    t->scr.assign(W, TierScratch{});
    for (TierScratch& x : t->scr) {
        x.in_union.assign(t->n_blk, 0u);
        x.in_keep.assign(t->n_blk, 0u);
        x.uni.reserve((size_t)t->H * t->K);
    }
}

// ------------------------------------------------------------ mapped gather
// As copy_blocks_kernel, with the source tile of (unit u = (r, g), block b)
// at cache slot map[r][b] of request r (entries whose block is absent are
// skipped).
constexpr int kMapCopySplit = 2;
constexpr int kMapCopyThreads = 64;

__global__ void __launch_bounds__(kMapCopyThreads)
copy_mapped_kernel(const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
                   const int32_t* __restrict__ map, int H, int n_blk, int cap_max,
                   uint4* __restrict__ res_k, uint4* __restrict__ res_v, int K, int tile_u4,
                   long long stride_u4, const int32_t* __restrict__ plan_count,
                   const int32_t* __restrict__ plan_src, const int32_t* __restrict__ plan_dst) {
    const size_t u = blockIdx.y;
    const size_t r = u / H, g = u - (u / H) * H;
    const int n = min(plan_count[u], K);
    for (int i = blockIdx.x; i < n; i += kMapCopySplit) {
        const int src = plan_src[u * K + i];
        const int dst = plan_dst[u * K + i];
        if (src < 0 || src >= n_blk || dst < 0 || dst >= K) continue;
        const int slot = map[r * n_blk + src];
        if (slot < 0 || slot >= cap_max) continue;
        const size_t so = ((r * cap_max + slot) * H + g) * (size_t)stride_u4;
        const uint4* sk = src_k + so;
        const uint4* sv = src_v + so;
        uint4* dk = res_k + (u * K + dst) * (size_t)stride_u4;
        uint4* dv = res_v + (u * K + dst) * (size_t)stride_u4;
        for (unsigned t = threadIdx.x; t < (unsigned)tile_u4; t += kMapCopyThreads) dk[t] = sk[t];
        for (unsigned t = threadIdx.x; t < (unsigned)tile_u4; t += kMapCopyThreads) dv[t] = sv[t];
    }
}

static int device_view(const void* p, const void** out) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EINVAL;
    }
    if (attr.type == hipMemoryTypeHost) {
        if (!attr.devicePointer) return OASIS_EINVAL;
        *out = attr.devicePointer;
        return OASIS_OK;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
        attr.type == hipMemoryTypeUnified) {
        *out = p;
        return OASIS_OK;
    }
    return OASIS_EINVAL;
}

// The gather of one layer-step: units = R*H (<= 65535, checked by callers).
static int launch_mapped(int units, int H, int n_blk, int cap_max, int K, const TierJob& j) {
    hipLaunchKernelGGL(copy_mapped_kernel, dim3(kMapCopySplit, (unsigned)units),
                       dim3(kMapCopyThreads), 0, j.copy_stream,
                       reinterpret_cast<const uint4*>(j.dev_k),
                       reinterpret_cast<const uint4*>(j.dev_v),
                       reinterpret_cast<const int32_t*>(j.dev_map), H, n_blk, cap_max,
                       reinterpret_cast<uint4*>(j.res_k), reinterpret_cast<uint4*>(j.res_v), K,
                       j.tile_u4, j.stride_u4, j.plan_count, j.plan_src, j.plan_dst);
    return launch_status();
}

// One job: the attention that read the slots (and wrote the plan) is done
// once `after` completes; then plan back, fetch, gather, `done`.
static int run_job(oasis_host_tier* t, const TierJob& j) {
    const size_t nc = (size_t)t->R * t->H * sizeof(int32_t), ns = nc * t->K;
    if (hipEventSynchronize(j.after) != hipSuccess ||
        hipMemcpyAsync(t->st_count, j.plan_count, nc, hipMemcpyDeviceToHost, t->dstream) !=
            hipSuccess ||
        hipMemcpyAsync(t->st_src, j.plan_src, ns, hipMemcpyDeviceToHost, t->dstream) !=
            hipSuccess ||
        hipMemcpyAsync(t->st_slots, j.slot_block, ns, hipMemcpyDeviceToHost, t->dstream) !=
            hipSuccess ||
        hipStreamSynchronize(t->dstream) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EHIP;
    }
    // A request whose budget held no evictable block leaves some planned
    // blocks absent (EINVAL, counted as failed).  The gather still runs and
    // `done` is still recorded, so no stream waits forever, but the slots of
    // the absent blocks keep stale tiles: the status goes to the caller
    // through oasis_host_tier_wait_issued.
    const int fst = tier_fetch(t, ++t->clock, t->st_count, t->st_src, t->st_slots);
    const int st = launch_mapped(t->R * t->H, t->H, t->n_blk, t->cap_max, t->K, j);
    if (st != OASIS_OK) return st;
    if (hipEventRecord(j.done, j.copy_stream) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EHIP;
    }
    return fst;
}

static void dispatcher_main(oasis_host_tier* t) {
    (void)hipSetDevice(t->device);
    std::unique_lock<std::mutex> lk(t->dmu);
    for (;;) {
        t->dgo.wait(lk, [&] { return t->dstop || !t->jobs.empty(); });
        if (t->jobs.empty()) return;  // stop requested and drained
        const TierJob j = t->jobs.front();
        t->jobs.pop_front();
        lk.unlock();
        const int st = run_job(t, j);
        lk.lock();
        if (st != OASIS_OK && t->async_status == OASIS_OK) t->async_status = st;
        ++t->issued;
        t->dissued.notify_all();
    }
}

// Host calls on the tier first let the dispatcher issue every submitted job
// (it uses the same state); returns that jobs' sticky status.
static int drain(oasis_host_tier* t) {
    std::unique_lock<std::mutex> lk(t->dmu);
    t->dissued.wait(lk, [&] { return t->issued == t->submitted; });
    return t->async_status;
}

static void stop_dispatcher(oasis_host_tier* t) {
    if (!t->dispatcher.joinable()) return;
    {
        std::lock_guard<std::mutex> lk(t->dmu);
        t->dstop = true;
    }
    t->dgo.notify_all();
    t->dispatcher.join();
}

}  // namespace oasis

using namespace oasis;

extern "C" oasis_host_tier* oasis_host_tier_create(int32_t batch, int32_t n_kv_heads,
                                                   int32_t top_k, int32_t n_blk,
                                                   const int32_t* capacity, int32_t cap_max,
                                                   size_t block_bytes, const void* remote,
                                                   void* cache, int32_t* map) {
    if (batch <= 0 || n_kv_heads <= 0 || top_k <= 0 || n_blk <= 0 || cap_max <= 0 ||
        block_bytes == 0 || !capacity || !remote || !cache || !map)
        return nullptr;
    for (int r = 0; r < batch; ++r)
        if (capacity[r] < 0 || capacity[r] > cap_max) return nullptr;
    oasis_host_tier* t = new (std::nothrow) oasis_host_tier;
    if (!t) return nullptr;
    t->R = batch;
    t->H = n_kv_heads;
    t->K = top_k;
    t->n_blk = n_blk;
    t->cap_max = cap_max;
    t->block_bytes = block_bytes;
    t->cap.assign(capacity, capacity + batch);
    t->remote = static_cast<const uint8_t*>(remote);
    t->cache = static_cast<uint8_t*>(cache);
    t->map = map;
    t->slot_blk.assign((size_t)batch * cap_max, -1);
    t->last.assign((size_t)batch * cap_max, -1);
    t->generated.assign((size_t)batch * n_blk, 0);
    init_scratch(t, 1);
    for (size_t i = 0; i < (size_t)batch * n_blk; ++i) map[i] = -1;
    // Every cache byte written once from the host: pinned pages the host has
    // not written yet cost a fault per page on first touch (about 8x the copy
    // of a whole block), which would otherwise land inside the fetches.
    std::memset(cache, 0, (size_t)batch * cap_max * block_bytes);
    return t;
}

extern "C" int oasis_host_tier_set_workers(oasis_host_tier* t, int32_t n_workers) {
    if (!t || n_workers < 1 || n_workers > 64) return OASIS_EINVAL;
    (void)drain(t);
    stop_pool(t);
    init_scratch(t, n_workers);
    try {
        for (int w = 1; w < n_workers; ++w) t->pool.emplace_back(tier_worker, t, w, t->job_gen);
    } catch (...) {
        stop_pool(t);
        init_scratch(t, 1);
        return OASIS_EHIP;
    }
    return OASIS_OK;
}

extern "C" void oasis_host_tier_destroy(oasis_host_tier* t) {
    if (!t) return;
    stop_dispatcher(t);  // runs what was submitted, then ends
    stop_pool(t);
    if (t->dstream) (void)hipStreamDestroy(t->dstream);
    if (t->st_count) (void)hipHostFree(t->st_count);
    if (t->st_src) (void)hipHostFree(t->st_src);
    if (t->st_slots) (void)hipHostFree(t->st_slots);
    delete t;
}

extern "C" int oasis_host_tier_fetch(oasis_host_tier* t, int64_t step, const int32_t* plan_count,
                                     const int32_t* plan_src, const int32_t* slot_block) {
    if (!t || !plan_count || !plan_src) return OASIS_EINVAL;
    (void)drain(t);
    return tier_fetch(t, step, plan_count, plan_src, slot_block);
}

extern "C" int oasis_host_tier_submit(oasis_host_tier* t, const oasis_shape* s,
                                      const void* cache_k, const void* cache_v, void* res_k,
                                      void* res_v, const int32_t* plan_count,
                                      const int32_t* plan_src, const int32_t* plan_dst,
                                      const int32_t* slot_block, hipEvent_t after,
                                      hipStream_t copy_stream, hipEvent_t done) {
    if (!t) return OASIS_EINVAL;
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (!cache_k || !cache_v || !res_k || !res_v || !plan_count || !plan_src || !plan_dst ||
        !slot_block || !after || !done || s->batch != t->R || s->n_kv_heads != t->H)
        return OASIS_EINVAL;
    const int eb = s->dtype == OASIS_F32 ? 4 : 2;
    const size_t tile_bytes = (size_t)s->block_size * s->head_dim * eb;
    const size_t rec_bytes = (size_t)tile_stride_of(s) * eb;
    if (tile_bytes % 16 || rec_bytes % 16 || (long long)t->R * t->H > 65535)
        return OASIS_EUNSUPPORTED;
    // The cache's records must tile its blocks exactly: H records per block.
    if (rec_bytes * t->H != t->block_bytes) return OASIS_EINVAL;
    TierJob j{};
    if (device_view(cache_k, &j.dev_k) != OASIS_OK || device_view(cache_v, &j.dev_v) != OASIS_OK ||
        device_view(t->map, &j.dev_map) != OASIS_OK)
        return OASIS_EINVAL;
    j.plan_count = plan_count;
    j.plan_src = plan_src;
    j.plan_dst = plan_dst;
    j.slot_block = slot_block;
    j.res_k = res_k;
    j.res_v = res_v;
    j.tile_u4 = (int)(tile_bytes / 16);
    j.stride_u4 = (long long)(rec_bytes / 16);
    j.after = after;
    j.done = done;
    j.copy_stream = copy_stream;
    if (!t->dispatcher.joinable()) {  // first submit: staging, private stream, thread
        const size_t nc = (size_t)t->R * t->H * sizeof(int32_t), ns = nc * t->K;
        if (hipGetDevice(&t->device) != hipSuccess) {
            (void)hipGetLastError();
            return OASIS_EHIP;
        }
        if (!t->st_count) {  // all three buffers or none
            int32_t *c = nullptr, *sr = nullptr, *sl = nullptr;
            if (hipHostMalloc((void**)&c, nc) != hipSuccess ||
                hipHostMalloc((void**)&sr, ns) != hipSuccess ||
                hipHostMalloc((void**)&sl, ns) != hipSuccess) {
                (void)hipGetLastError();
                if (c) (void)hipHostFree(c);
                if (sr) (void)hipHostFree(sr);
                if (sl) (void)hipHostFree(sl);
                return OASIS_EHIP;
            }
            t->st_count = c;
            t->st_src = sr;
            t->st_slots = sl;
        }
        if (!t->dstream && hipStreamCreateWithFlags(&t->dstream, hipStreamNonBlocking) !=
                               hipSuccess) {
            (void)hipGetLastError();
            t->dstream = nullptr;
            return OASIS_EHIP;
        }
        try {
            t->dstop = false;
            t->dispatcher = std::thread(dispatcher_main, t);
        } catch (...) {
            return OASIS_EHIP;
        }
    }
    {
        std::lock_guard<std::mutex> lk(t->dmu);
        t->jobs.push_back(j);
        ++t->submitted;
    }
    t->dgo.notify_one();
    return OASIS_OK;
}

extern "C" int oasis_host_tier_wait_issued(oasis_host_tier* t) {
    if (!t) return OASIS_EINVAL;
    return drain(t);
}

extern "C" int oasis_host_tier_add_generated(oasis_host_tier* t, int32_t req, int32_t block,
                                             int64_t step, const int32_t* slot_block) {
    if (!t || req < 0 || req >= t->R || block < 0 || block >= t->n_blk) return OASIS_EINVAL;
    (void)drain(t);
    TierScratch& x = t->scr[0];
    x.begin_request();
    if (slot_block)
        for (size_t i = 0; i < (size_t)t->H * t->K; ++i) {
            const int b = slot_block[(size_t)req * t->H * t->K + i];
            if (b >= 0 && b < t->n_blk) x.in_keep[b] = x.epoch;
        }
    int s = t->map[(size_t)req * t->n_blk + block];
    if (s < 0 && (s = tier_place(t, x, req, block)) < 0) {
        ++x.failed;
        return OASIS_EINVAL;
    }
    t->generated[(size_t)req * t->n_blk + block] = 1;
    t->last[(size_t)req * t->cap_max + s] = step;
    return OASIS_OK;
}

extern "C" int oasis_host_tier_trim(oasis_host_tier* t, const int32_t* target,
                                    const int32_t* slot_block) {
    if (!t || !target) return OASIS_EINVAL;
    (void)drain(t);
    TierScratch& x = t->scr[0];
    for (int r = 0; r < t->R; ++r) {
        x.begin_request();
        if (slot_block)
            for (size_t i = 0; i < (size_t)t->H * t->K; ++i) {
                const int b = slot_block[(size_t)r * t->H * t->K + i];
                if (b >= 0 && b < t->n_blk) x.in_keep[b] = x.epoch;
            }
        int live = 0;
        for (int s = 0; s < t->cap[r]; ++s) live += t->slot_blk[(size_t)r * t->cap_max + s] >= 0;
        while (live > target[r]) {
            const int s = tier_victim(t, x, r);
            if (s < 0) break;
            const size_t i = (size_t)r * t->cap_max + s;
            t->map[(size_t)r * t->n_blk + t->slot_blk[i]] = -1;
            t->slot_blk[i] = -1;
            t->last[i] = -1;
            ++x.evicted;
            --live;
        }
    }
    return OASIS_OK;
}

extern "C" int oasis_host_tier_state(const oasis_host_tier* t, int32_t* slot_block_out,
                                     int64_t* last_out, int64_t* stats_out) {
    if (!t) return OASIS_EINVAL;
    (void)drain(const_cast<oasis_host_tier*>(t));  // the lock and wait only
    const size_t n = (size_t)t->R * t->cap_max;
    if (slot_block_out)
        for (size_t i = 0; i < n; ++i) slot_block_out[i] = t->slot_blk[i];
    if (last_out)
        for (size_t i = 0; i < n; ++i) last_out[i] = t->last[i];
    if (stats_out) {
        long long f = t->base_fetched, e = t->base_evicted, x = t->base_failed;
        for (const TierScratch& s : t->scr) {
            f += s.fetched;
            e += s.evicted;
            x += s.failed;
        }
        stats_out[0] = f;
        stats_out[1] = e;
        stats_out[2] = x;
        stats_out[3] = t->clock;
        stats_out[4] = t->fetch_ns;
    }
    return OASIS_OK;
}

extern "C" int oasis_copy_blocks_mapped(const oasis_shape* s, const void* cache_k,
                                        const void* cache_v, int32_t cap_max, const int32_t* map,
                                        int32_t n_blk, void* res_k, void* res_v, int32_t top_k,
                                        const int32_t* plan_count, const int32_t* plan_src,
                                        const int32_t* plan_dst, hipStream_t stream) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (!cache_k || !cache_v || !map || !res_k || !res_v || !plan_count || !plan_src ||
        !plan_dst || cap_max <= 0 || n_blk <= 0 || top_k <= 0 || top_k > 65535)
        return OASIS_EINVAL;
    const int eb = s->dtype == OASIS_F32 ? 4 : 2;
    const size_t tile_bytes = (size_t)s->block_size * s->head_dim * eb;
    if (tile_bytes % 16) return OASIS_EUNSUPPORTED;
    const long long units = (long long)s->batch * s->n_kv_heads;
    if (units > 65535) return OASIS_EUNSUPPORTED;
    TierJob j{};
    if (device_view(cache_k, &j.dev_k) != OASIS_OK || device_view(cache_v, &j.dev_v) != OASIS_OK ||
        device_view(map, &j.dev_map) != OASIS_OK)
        return OASIS_EINVAL;
    j.res_k = res_k;
    j.res_v = res_v;
    j.tile_u4 = int(tile_bytes / 16);
    j.stride_u4 = tile_stride_of(s) * eb / 16;
    j.plan_count = plan_count;
    j.plan_src = plan_src;
    j.plan_dst = plan_dst;
    j.copy_stream = stream;
    return launch_mapped((int)units, s->n_kv_heads, n_blk, cap_max, top_k, j);
}
