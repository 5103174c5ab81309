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
// object; its work is plain CPU code, run either directly (host call) or in
// stream order (after the plan is copied back, before the gather).
#include <cstring>
#include <new>
#include <vector>

#include "oasis_internal.h"

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
    std::vector<unsigned> in_union;   // [n_blk] epoch marks
    std::vector<unsigned> in_keep;    // [n_blk] epoch marks
    std::vector<int> uni;             // scratch: one request's union
    unsigned epoch = 0;
    long long clock = 0;              // stream-ordered calls stamp with their own counter
    long long fetched = 0, evicted = 0, failed = 0;
    // pinned staging of the stream-ordered variant (allocated on first use)
    int32_t* st_count = nullptr;      // [R][H]
    int32_t* st_src = nullptr;        // [R][H][K]
    int32_t* st_slots = nullptr;      // [R][H][K]
};

namespace oasis {

static int tier_victim(oasis_host_tier* t, int r) {
    int best = -1;
    long long best_last = 0;
    for (int s = 0; s < t->cap[r]; ++s) {
        const int b = t->slot_blk[(size_t)r * t->cap_max + s];
        if (b < 0 || t->in_keep[b] == t->epoch || t->generated[(size_t)r * t->n_blk + b]) continue;
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
static int tier_place(oasis_host_tier* t, int r, int b) {
    int s = -1;
    for (int i = 0; i < t->cap[r]; ++i)
        if (t->slot_blk[(size_t)r * t->cap_max + i] < 0) {
            s = i;
            break;
        }
    if (s < 0) {
        s = tier_victim(t, r);
        if (s < 0) return -1;
        const int old = t->slot_blk[(size_t)r * t->cap_max + s];
        t->map[(size_t)r * t->n_blk + old] = -1;
        ++t->evicted;
    }
    t->slot_blk[(size_t)r * t->cap_max + s] = b;
    t->map[(size_t)r * t->n_blk + b] = s;
    return s;
}

// One layer-step: union of the planned sources per request, fetch of the
// absent blocks, last-use stamps.  Returns OASIS_OK or OASIS_EINVAL when a
// request's budget held no evictable block (that request's remaining blocks
// are skipped; failed counts them).
static int tier_fetch(oasis_host_tier* t, long long step, const int32_t* count,
                      const int32_t* src, const int32_t* slots) {
    int st = OASIS_OK;
    for (int r = 0; r < t->R; ++r) {
        ++t->epoch;
        t->uni.clear();
        for (int g = 0; g < t->H; ++g) {
            const size_t u = (size_t)r * t->H + g;
            const int n = count[u] < t->K ? count[u] : t->K;
            for (int i = 0; i < n; ++i) {
                const int b = src[u * t->K + i];
                if (b < 0 || b >= t->n_blk || t->in_union[b] == t->epoch) continue;
                t->in_union[b] = t->epoch;
                t->in_keep[b] = t->epoch;
                t->uni.push_back(b);
            }
            if (slots)
                for (int k = 0; k < t->K; ++k) {
                    const int b = slots[u * t->K + k];
                    if (b >= 0 && b < t->n_blk) t->in_keep[b] = t->epoch;
                }
        }
        for (int b : t->uni) {
            if (t->map[(size_t)r * t->n_blk + b] >= 0) continue;
            const int s = tier_place(t, r, b);
            if (s < 0) {
                ++t->failed;
                st = OASIS_EINVAL;
                continue;
            }
            std::memcpy(t->cache + ((size_t)r * t->cap_max + s) * t->block_bytes,
                        t->remote + ((size_t)r * t->n_blk + b) * t->block_bytes, t->block_bytes);
            ++t->fetched;
        }
        for (int b : t->uni) {
            const int s = t->map[(size_t)r * t->n_blk + b];
            if (s >= 0) t->last[(size_t)r * t->cap_max + s] = step;
        }
    }
    return st;
}

static void tier_host_fn(void* p) {
    oasis_host_tier* t = static_cast<oasis_host_tier*>(p);
    (void)tier_fetch(t, ++t->clock, t->st_count, t->st_src, t->st_slots);
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
    const int n = plan_count[u];
    for (int i = blockIdx.x; i < n; i += kMapCopySplit) {
        const int src = plan_src[u * K + i];
        const int dst = plan_dst[u * K + i];
        if (src < 0 || src >= n_blk) continue;
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
    t->in_union.assign(n_blk, 0);
    t->in_keep.assign(n_blk, 0);
    for (size_t i = 0; i < (size_t)batch * n_blk; ++i) map[i] = -1;
    return t;
}

extern "C" void oasis_host_tier_destroy(oasis_host_tier* t) {
    if (!t) return;
    if (t->st_count) (void)hipHostFree(t->st_count);
    if (t->st_src) (void)hipHostFree(t->st_src);
    if (t->st_slots) (void)hipHostFree(t->st_slots);
    delete t;
}

extern "C" int oasis_host_tier_fetch(oasis_host_tier* t, int64_t step, const int32_t* plan_count,
                                     const int32_t* plan_src, const int32_t* slot_block) {
    if (!t || !plan_count || !plan_src) return OASIS_EINVAL;
    return tier_fetch(t, step, plan_count, plan_src, slot_block);
}

extern "C" int oasis_host_tier_enqueue_fetch(oasis_host_tier* t, const int32_t* plan_count,
                                             const int32_t* plan_src, const int32_t* slot_block,
                                             hipStream_t stream) {
    if (!t || !plan_count || !plan_src || !slot_block) return OASIS_EINVAL;
    const size_t nc = (size_t)t->R * t->H * 4, ns = nc * t->K;
    if (!t->st_count) {
        if (hipHostMalloc((void**)&t->st_count, nc) != hipSuccess ||
            hipHostMalloc((void**)&t->st_src, ns) != hipSuccess ||
            hipHostMalloc((void**)&t->st_slots, ns) != hipSuccess) {
            (void)hipGetLastError();
            return OASIS_EHIP;
        }
    }
    if (hipMemcpyAsync(t->st_count, plan_count, nc, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(t->st_src, plan_src, ns, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(t->st_slots, slot_block, ns, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipLaunchHostFunc(stream, tier_host_fn, t) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EHIP;
    }
    return OASIS_OK;
}

extern "C" int oasis_host_tier_add_generated(oasis_host_tier* t, int32_t req, int32_t block,
                                             int64_t step, const int32_t* slot_block) {
    if (!t || req < 0 || req >= t->R || block < 0 || block >= t->n_blk) return OASIS_EINVAL;
    ++t->epoch;
    if (slot_block)
        for (size_t i = 0; i < (size_t)t->H * t->K; ++i) {
            const int b = slot_block[(size_t)req * t->H * t->K + i];
            if (b >= 0 && b < t->n_blk) t->in_keep[b] = t->epoch;
        }
    int s = t->map[(size_t)req * t->n_blk + block];
    if (s < 0 && (s = tier_place(t, req, block)) < 0) {
        ++t->failed;
        return OASIS_EINVAL;
    }
    t->generated[(size_t)req * t->n_blk + block] = 1;
    t->last[(size_t)req * t->cap_max + s] = step;
    return OASIS_OK;
}

extern "C" int oasis_host_tier_trim(oasis_host_tier* t, const int32_t* target,
                                    const int32_t* slot_block) {
    if (!t || !target) return OASIS_EINVAL;
    for (int r = 0; r < t->R; ++r) {
        ++t->epoch;
        if (slot_block)
            for (size_t i = 0; i < (size_t)t->H * t->K; ++i) {
                const int b = slot_block[(size_t)r * t->H * t->K + i];
                if (b >= 0 && b < t->n_blk) t->in_keep[b] = t->epoch;
            }
        int live = 0;
        for (int s = 0; s < t->cap[r]; ++s) live += t->slot_blk[(size_t)r * t->cap_max + s] >= 0;
        while (live > target[r]) {
            const int s = tier_victim(t, r);
            if (s < 0) break;
            const size_t i = (size_t)r * t->cap_max + s;
            t->map[(size_t)r * t->n_blk + t->slot_blk[i]] = -1;
            t->slot_blk[i] = -1;
            t->last[i] = -1;
            ++t->evicted;
            --live;
        }
    }
    return OASIS_OK;
}

extern "C" int oasis_host_tier_state(const oasis_host_tier* t, int32_t* slot_block_out,
                                     int64_t* last_out, int64_t* stats_out) {
    if (!t) return OASIS_EINVAL;
    const size_t n = (size_t)t->R * t->cap_max;
    if (slot_block_out)
        for (size_t i = 0; i < n; ++i) slot_block_out[i] = t->slot_blk[i];
    if (last_out)
        for (size_t i = 0; i < n; ++i) last_out[i] = t->last[i];
    if (stats_out) {
        stats_out[0] = t->fetched;
        stats_out[1] = t->evicted;
        stats_out[2] = t->failed;
        stats_out[3] = t->clock;
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
    const void *dk = nullptr, *dv = nullptr, *dm = nullptr;
    if (device_view(cache_k, &dk) != OASIS_OK || device_view(cache_v, &dv) != OASIS_OK ||
        device_view(map, &dm) != OASIS_OK)
        return OASIS_EINVAL;
    hipLaunchKernelGGL(copy_mapped_kernel, dim3(kMapCopySplit, (unsigned)units),
                       dim3(kMapCopyThreads), 0, stream, reinterpret_cast<const uint4*>(dk),
                       reinterpret_cast<const uint4*>(dv), reinterpret_cast<const int32_t*>(dm),
                       s->n_kv_heads, n_blk, cap_max, reinterpret_cast<uint4*>(res_k),
                       reinterpret_cast<uint4*>(res_v), top_k, int(tile_bytes / 16),
                       tile_stride_of(s) * eb / 16, plan_count, plan_src, plan_dst);
    return launch_status();
}
