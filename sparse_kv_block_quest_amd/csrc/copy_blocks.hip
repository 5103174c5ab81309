// Gather of planned block-head tiles from the full per-head store (pinned host
// memory read over PCIe, or device memory) into the resident HBM slots.
//
// Sources: OasisKV paperpeel v2 text, §3.2.1 (a gather kernel running on the
// GPU reads the selected per-head entries straight from pinned host memory and
// writes them into HBM) and §4.1 Implementation (the full KV cache lives in
// pinned CPU memory; the gather writes directly into the resident GPU pages).
//
// Workgroup (j, u), one wave, moves plan entries j, j + S, j + 2S, ... of
// unit u (S = kCopySplit).  Offsets are uniform, so they stay in scalar
// registers, and a lane carries one 16-byte word at a time: the kernel needs
// about 10 VGPRs.  That lets copy waves share a SIMD with two waves of the
// fused step kernel when the copy runs beside it on another stream, and a
// small grid (2 waves per unit) keeps few SIMDs busy with waits on PCIe while
// still holding enough reads in flight to fill the link.  The device-resident
// plan is consumed without a host round trip.
#include "oasis_internal.h"

namespace oasis {

constexpr int kCopySplit = 2;
constexpr int kCopyThreads = 64;

__global__ void __launch_bounds__(kCopyThreads)
copy_blocks_kernel(const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
                   uint4* __restrict__ res_k, uint4* __restrict__ res_v, int n_blk_max,
                   int K, int tile_u4, long long stride_u4, const int32_t* __restrict__ plan_count,
                   const int32_t* __restrict__ plan_src, const int32_t* __restrict__ plan_dst) {
    const size_t u = blockIdx.y;
    const int n = min(plan_count[u], K);
    for (int i = blockIdx.x; i < n; i += kCopySplit) {
        const int src = plan_src[u * K + i];
        const int dst = plan_dst[u * K + i];
        // an entry naming a block or slot outside the stores is skipped
        if ((unsigned)src >= (unsigned)n_blk_max || (unsigned)dst >= (unsigned)K) continue;
        const uint4* sk = src_k + (u * n_blk_max + src) * (size_t)stride_u4;
        const uint4* sv = src_v + (u * n_blk_max + src) * (size_t)stride_u4;
        uint4* dk = res_k + (u * K + dst) * (size_t)stride_u4;
        uint4* dv = res_v + (u * K + dst) * (size_t)stride_u4;
        for (unsigned t = threadIdx.x; t < (unsigned)tile_u4; t += kCopyThreads) dk[t] = sk[t];
        for (unsigned t = threadIdx.x; t < (unsigned)tile_u4; t += kCopyThreads) dv[t] = sv[t];
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
    const long long units = (long long)s->batch * s->n_kv_heads;
    if (units > 65535) return OASIS_EUNSUPPORTED;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(kCopySplit, (unsigned)units), dim3(kCopyThreads), 0,
                       stream, reinterpret_cast<const uint4*>(dk),
                       reinterpret_cast<const uint4*>(dv), reinterpret_cast<uint4*>(res_k),
                       reinterpret_cast<uint4*>(res_v), n_blk_max, top_k,
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
