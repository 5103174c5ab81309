// Gather of planned block-head tiles from the full per-head store (pinned host
// memory read over PCIe, or device memory) into the resident HBM slots.
//
// Sources: OasisKV paperpeel v2 text, §3.2.1 (a gather kernel running on the
// GPU reads the selected per-head entries straight from pinned host memory and
// writes them into HBM) and §4.1 Implementation (the full KV cache lives in
// pinned CPU memory; the gather writes directly into the resident GPU pages).
//
// One workgroup per (plan entry, KV head, request); entries at or past the
// unit's plan_count exit at once.  Each thread moves 16-byte words of the K
// tile and of the V tile, so one workgroup keeps 2*tile bytes of reads in
// flight; the device-resident plan is consumed without a host round trip.
#include "oasis_internal.h"

namespace oasis {

__global__ void __launch_bounds__(256)
copy_blocks_kernel(const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
                   uint4* __restrict__ res_k, uint4* __restrict__ res_v, int H, int n_blk_max,
                   int K, int tile_u4, long long stride_u4, const int32_t* __restrict__ plan_count,
                   const int32_t* __restrict__ plan_src, const int32_t* __restrict__ plan_dst) {
    const int i = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const size_t u = (size_t)r * H + g;
    if (i >= plan_count[u]) return;
    const int src = plan_src[u * K + i];
    const int dst = plan_dst[u * K + i];
    const size_t so = (u * n_blk_max + src) * (size_t)stride_u4;
    const size_t d_o = (u * K + dst) * (size_t)stride_u4;
    for (int t = threadIdx.x; t < tile_u4; t += 256) {
        const uint4 a = src_k[so + t];
        const uint4 b = src_v[so + t];
        res_k[d_o + t] = a;
        res_v[d_o + t] = b;
    }
}

}  // namespace oasis

using namespace oasis;

// GPU-side address of a source store.  Device and managed memory are used as
// they are; pinned host memory must be mapped for the GPU (hipHostMalloc or a
// pinned torch tensor) and is translated to its device address.  Anything
// else (pageable host memory) is rejected here, before a kernel could touch it.
static int device_view(const void* p, const void** out) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EINVAL;
    }
    switch (attr.type) {
        case hipMemoryTypeDevice:
        case hipMemoryTypeManaged:
        case hipMemoryTypeUnified:
        case hipMemoryTypeArray:
            *out = p;
            return OASIS_OK;
        case hipMemoryTypeHost:
            if (!attr.devicePointer) return OASIS_EINVAL;
            *out = attr.devicePointer;
            return OASIS_OK;
        default:
            return OASIS_EINVAL;
    }
}

extern "C" int oasis_copy_blocks(const oasis_shape* s, const void* src_k, const void* src_v,
                                 int32_t n_blk_max, void* res_k, void* res_v, int32_t top_k,
                                 const int32_t* plan_count, const int32_t* plan_src,
                                 const int32_t* plan_dst, hipStream_t stream) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (!src_k || !src_v || !res_k || !res_v || !plan_count || !plan_src || !plan_dst ||
        n_blk_max <= 0 || top_k <= 0 || top_k > 65535)
        return OASIS_EINVAL;
    const size_t tile_bytes = (size_t)s->block_size * s->head_dim * (s->dtype == OASIS_F32 ? 4 : 2);
    if (tile_bytes % 16) return OASIS_EUNSUPPORTED;
    const void* dk = nullptr;
    const void* dv = nullptr;
    if (device_view(src_k, &dk) != OASIS_OK || device_view(src_v, &dv) != OASIS_OK)
        return OASIS_EINVAL;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(top_k, s->n_kv_heads, s->batch), dim3(256), 0,
                       stream, reinterpret_cast<const uint4*>(dk),
                       reinterpret_cast<const uint4*>(dv), reinterpret_cast<uint4*>(res_k),
                       reinterpret_cast<uint4*>(res_v), s->n_kv_heads, n_blk_max, top_k,
                       int(tile_bytes / 16),
                       tile_stride_of(s) * (s->dtype == OASIS_F32 ? 4 : 2) / 16, plan_count,
                       plan_src, plan_dst);
    return launch_status();
}

extern "C" const char* oasis_status_string(int status) {
    switch (status) {
        case OASIS_OK: return "ok";
        case OASIS_EINVAL: return "invalid argument";
        case OASIS_EUNSUPPORTED: return "unsupported dtype, head dim, block size or group size";
        case OASIS_EWORKSPACE: return "workspace missing or too small";
        case OASIS_EHIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

extern "C" int oasis_version(void) { return 100; }
