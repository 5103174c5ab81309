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
// The manager's state (slots, last use, generated flags) and its work are
// plain C++ in host_tier_core.h (no HIP), run either directly (host call) or by
// the tier's dispatcher thread, which takes submitted layer-steps in order:
// wait on the host for the event that follows the plan, copy the plan back,
// fetch, then launch the mapped gather on the caller's copy stream and record
// the caller's event after it.  No GPU queue ever waits on host memory; the
// caller orders later GPU work on that event once the host call
// oasis_host_tier_wait_issued says it has been recorded.  Requests are
// independent (each owns its rows of every array), so a fetch may split them
// over a small pool of host threads: worker w of W takes r = w, w+W, ... with
// scratch of its own, and the result does not depend on W.
#include <new>

#include "host_tier_core.h"
#include "oasis_internal.h"

static_assert(oasis::tier::kOk == OASIS_OK && oasis::tier::kInval == OASIS_EINVAL &&
                  oasis::tier::kThread == OASIS_EHIP,
              "status codes of the cache core");

namespace oasis {

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
    oasis::tier::Cache c;                     // slots, map, LRU state, worker pool
    oasis::tier::Dispatcher<oasis::TierJob> d;  // stream-ordered jobs (set up on first submit)
    long long clock = 0;                      // stream-ordered calls stamp with their own counter
    int device = -1;
    hipStream_t dstream = nullptr;            // private stream for copying the plan back
    int32_t* st_count = nullptr;              // [R][H] pinned staging of the plan
    int32_t* st_src = nullptr;                // [R][H][K]
    int32_t* st_slots = nullptr;              // [R][H][K]
};

namespace oasis {

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
    const tier::Cache& c = t->c;
    const size_t nc = (size_t)c.R * c.H * sizeof(int32_t), ns = nc * c.K;
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
    const int fst = tier::cache_fetch(t->c, ++t->clock, t->st_count, t->st_src, t->st_slots);
    const int st = launch_mapped(c.R * c.H, c.H, c.n_blk, c.cap_max, c.K, j);
    if (st != OASIS_OK) return st;
    if (hipEventRecord(j.done, j.copy_stream) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EHIP;
    }
    return fst;
}

// Host calls on the tier first let the dispatcher issue every submitted job
// (it uses the same state); returns those jobs' sticky status.
static int drain(oasis_host_tier* t) { return t->d.running() ? t->d.drain() : OASIS_OK; }

}  // namespace oasis

using namespace oasis;

extern "C" oasis_host_tier* oasis_host_tier_create(int32_t batch, int32_t n_kv_heads,
                                                   int32_t top_k, int32_t n_blk,
                                                   const int32_t* capacity, int32_t cap_max,
                                                   size_t block_bytes, const void* remote,
                                                   void* cache, int32_t* map) {
    oasis_host_tier* t = new (std::nothrow) oasis_host_tier;
    if (!t) return nullptr;
    if (!tier::cache_init(t->c, batch, n_kv_heads, top_k, n_blk, capacity, cap_max, block_bytes,
                          remote, cache, map)) {
        delete t;
        return nullptr;
    }
    return t;
}

extern "C" int oasis_host_tier_set_workers(oasis_host_tier* t, int32_t n_workers) {
    if (!t || n_workers < 1 || n_workers > 64) return OASIS_EINVAL;
    (void)drain(t);
    return tier::cache_set_workers(t->c, n_workers);
}

extern "C" void oasis_host_tier_destroy(oasis_host_tier* t) {
    if (!t) return;
    t->d.finish();  // runs what was submitted, then ends
    tier::stop_pool(t->c);
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
    return tier::cache_fetch(t->c, step, plan_count, plan_src, slot_block);
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
    const tier::Cache& c = t->c;
    if (!cache_k || !cache_v || !res_k || !res_v || !plan_count || !plan_src || !plan_dst ||
        !slot_block || !after || !done || s->batch != c.R || s->n_kv_heads != c.H)
        return OASIS_EINVAL;
    const int eb = s->dtype == OASIS_F32 ? 4 : 2;
    const size_t tile_bytes = (size_t)s->block_size * s->head_dim * eb;
    const size_t rec_bytes = (size_t)tile_stride_of(s) * eb;
    if (tile_bytes % 16 || rec_bytes % 16 || (long long)c.R * c.H > 65535)
        return OASIS_EUNSUPPORTED;
    // The cache's records must tile its blocks exactly: H records per block.
    if (rec_bytes * c.H != c.block_bytes) return OASIS_EINVAL;
    TierJob j{};
    if (device_view(cache_k, &j.dev_k) != OASIS_OK || device_view(cache_v, &j.dev_v) != OASIS_OK ||
        device_view(c.map, &j.dev_map) != OASIS_OK)
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
    if (!t->d.running()) {  // first submit: staging, private stream, thread
        const size_t nc = (size_t)c.R * c.H * sizeof(int32_t), ns = nc * c.K;
        if (hipGetDevice(&t->device) != hipSuccess) {
            (void)hipGetLastError();
            return OASIS_EHIP;
        }
        if (!t->st_count) {  // all three buffers or none
            int32_t *cn = nullptr, *sr = nullptr, *sl = nullptr;
            if (hipHostMalloc((void**)&cn, nc) != hipSuccess ||
                hipHostMalloc((void**)&sr, ns) != hipSuccess ||
                hipHostMalloc((void**)&sl, ns) != hipSuccess) {
                (void)hipGetLastError();
                if (cn) (void)hipHostFree(cn);
                if (sr) (void)hipHostFree(sr);
                if (sl) (void)hipHostFree(sl);
                return OASIS_EHIP;
            }
            t->st_count = cn;
            t->st_src = sr;
            t->st_slots = sl;
        }
        if (!t->dstream && hipStreamCreateWithFlags(&t->dstream, hipStreamNonBlocking) !=
                               hipSuccess) {
            (void)hipGetLastError();
            t->dstream = nullptr;
            return OASIS_EHIP;
        }
        const int dev = t->device;
        if (!t->d.start([dev] { (void)hipSetDevice(dev); },
                        [t](const TierJob& job) { return run_job(t, job); }))
            return OASIS_EHIP;
    }
    t->d.submit(j);
    return OASIS_OK;
}

extern "C" int oasis_host_tier_wait_issued(oasis_host_tier* t) {
    if (!t) return OASIS_EINVAL;
    return drain(t);
}

extern "C" int oasis_host_tier_add_generated(oasis_host_tier* t, int32_t req, int32_t block,
                                             int64_t step, const int32_t* slot_block) {
    if (!t) return OASIS_EINVAL;
    (void)drain(t);
    return tier::cache_add_generated(t->c, req, block, step, slot_block);
}

extern "C" int oasis_host_tier_trim(oasis_host_tier* t, const int32_t* target,
                                    const int32_t* slot_block) {
    if (!t || !target) return OASIS_EINVAL;
    (void)drain(t);
    return tier::cache_trim(t->c, target, slot_block);
}

extern "C" int oasis_host_tier_state(const oasis_host_tier* t, int32_t* slot_block_out,
                                     int64_t* last_out, int64_t* stats_out) {
    if (!t) return OASIS_EINVAL;
    oasis_host_tier* m = const_cast<oasis_host_tier*>(t);  // the wait only
    (void)drain(m);
    tier::cache_state(t->c, slot_block_out, last_out, stats_out, t->clock);
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
