// Per-block min/max key summaries (Quest-style compressed keys).
//
// Sources: OasisKV, signal-papers reader text, paragraph on ranking
// non-resident blocks (coordinate-wise minimum and maximum of the keys of each
// logical block); metallab.ai summary, Fig. 7 caption (per-block min/max
// pooling); paperpeel v2 text, §4.1 (two summary rows per 16-token block).
//
// Mapping: a block's B key rows are D*e bytes each (one K tile; tiles are
// tile_stride elements apart in the store).  LPR = D*e/16 lanes share
// one block; lane c owns the 16-byte column chunk c of every row, walks the B
// rows with 16-byte loads (one coalesced D*e-byte segment per row per lane
// group) and writes its chunk of the min row and of the max row.  Min/max of
// exactly representable values is exact, so bf16 results are bit-identical to
// a reference in any precision.  HBM-bound: reads B*D*e and writes 2*D*e
// bytes per block.
#include "oasis_internal.h"

namespace oasis {

template <int DT, int D, int B>
__global__ void __launch_bounds__(256)
build_summaries_kernel(const uint8_t* __restrict__ keys, uint8_t* __restrict__ summ,
                       const int32_t* __restrict__ seq_len, int H, int n_blk_max,
                       int blk_begin, int n_range, long long total_lanes, long long tile_u4) {
    constexpr int EB = Elem<DT>::bytes;
    constexpr int VEC = 16 / EB;
    constexpr int LPR = D / VEC;           // lanes per block
    constexpr int ROW_U4 = D * EB / 16;    // uint4 per key row (== LPR)
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= total_lanes) return;
    const int c = int(gid % LPR);
    const long long item = gid / LPR;
    const int b = blk_begin + int(item % n_range);
    const long long unit = item / n_range;
    const int r = int(unit / H);
    const int n_full = seq_len ? seq_len[r] / B : n_blk_max;
    if (b >= n_full) return;

    const uint4* src = reinterpret_cast<const uint4*>(keys) + (unit * n_blk_max + b) * tile_u4 + c;
    float lo[VEC], hi[VEC];
    {
        float v[VEC];
        unpack16<DT>(load_stream(src), v);
#pragma unroll
        for (int e = 0; e < VEC; ++e) lo[e] = hi[e] = v[e];
    }
    constexpr int CH = B < 16 ? B : 16;  // rows loaded per batch
#pragma unroll 1
    for (int i0 = 0; i0 < B; i0 += CH) {
        uint4 raw[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) raw[i] = load_stream(src + (long long)(i0 + i) * ROW_U4);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            float v[VEC];
            unpack16<DT>(raw[i], v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                lo[e] = v[e] < lo[e] ? v[e] : lo[e];
                hi[e] = v[e] > hi[e] ? v[e] : hi[e];
            }
        }
    }
    uint4* dst = reinterpret_cast<uint4*>(summ) + ((unit * n_blk_max + b) * 2) * ROW_U4 + c;
    dst[0] = pack16_exact<DT>(lo);
    dst[ROW_U4] = pack16_exact<DT>(hi);
}

template <int DT, int D>
static void launch_summaries_d(int B, const void* keys, void* summ, const int32_t* seq_len,
                               int H, int n_blk_max, int blk_begin, int n_range,
                               long long total_lanes, long long tile_u4, hipStream_t st) {
    dim3 grid((unsigned)((total_lanes + 255) / 256));
    auto k8 = reinterpret_cast<const uint8_t*>(keys);
    auto s8 = reinterpret_cast<uint8_t*>(summ);
#define OASIS_SUMM_CASE(BB)                                                                   \
    case BB:                                                                                  \
        hipLaunchKernelGGL((build_summaries_kernel<DT, D, BB>), grid, dim3(256), 0, st, k8, s8, \
                           seq_len, H, n_blk_max, blk_begin, n_range, total_lanes, tile_u4); \
        break;
    switch (B) {
        OASIS_SUMM_CASE(1)
        OASIS_SUMM_CASE(2)
        OASIS_SUMM_CASE(4)
        OASIS_SUMM_CASE(8)
        OASIS_SUMM_CASE(16)
        OASIS_SUMM_CASE(32)
        OASIS_SUMM_CASE(64)
        default:
            break;
    }
#undef OASIS_SUMM_CASE
}

}  // namespace oasis

using namespace oasis;

extern "C" int oasis_build_summaries(const oasis_shape* s, const void* keys, int32_t n_blk_max,
                                     const int32_t* seq_len, int32_t blk_begin, int32_t blk_end,
                                     void* summaries, hipStream_t stream) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (!keys || !summaries || n_blk_max <= 0 || blk_begin < 0 || blk_end < blk_begin)
        return OASIS_EINVAL;
    if (blk_end > n_blk_max) blk_end = n_blk_max;
    const int n_range = blk_end - blk_begin;
    if (n_range <= 0) return OASIS_OK;
    const int D = s->head_dim;
    const int lpr = D * (s->dtype == OASIS_F32 ? 4 : 2) / 16;
    const long long total = (long long)s->batch * s->n_kv_heads * n_range * lpr;
    const int H = s->n_kv_heads, B = s->block_size;
    const long long tu4 = tile_stride_of(s) * (s->dtype == OASIS_F32 ? 4 : 2) / 16;
    if (s->dtype == OASIS_F32) {
        if (D == 64)
            launch_summaries_d<OASIS_F32, 64>(B, keys, summaries, seq_len, H, n_blk_max,
                                              blk_begin, n_range, total, tu4, stream);
        else
            launch_summaries_d<OASIS_F32, 128>(B, keys, summaries, seq_len, H, n_blk_max,
                                               blk_begin, n_range, total, tu4, stream);
    } else {
        if (D == 64)
            launch_summaries_d<OASIS_BF16, 64>(B, keys, summaries, seq_len, H, n_blk_max,
                                               blk_begin, n_range, total, tu4, stream);
        else
            launch_summaries_d<OASIS_BF16, 128>(B, keys, summaries, seq_len, H, n_blk_max,
                                                blk_begin, n_range, total, tu4, stream);
    }
    return launch_status();
}

// ------------------------------------------------------------ token append
// Growing contexts: request r's new token (position pos[r], skipped if
// negative) goes into the K tile row and the V tile column of its block, for
// every KV head; a token that completes its block also rebuilds that block's
// summary rows (the same min / max as build_summaries_kernel).  Sources:
// OasisKV paperpeel v2 text, §3.2.1 (newly generated blocks join each head's
// working set) and Fig. 6 (per-block min / max key summaries in HBM).
// One thread per (unit, dim): the K writes of a unit are one contiguous row;
// the block's other B-1 keys of the column were written by earlier launches.
template <int DT>
__global__ void __launch_bounds__(256)
append_kv_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
                 const int32_t* __restrict__ pos, void* __restrict__ kt, void* __restrict__ vt,
                 void* __restrict__ summ, int H, int D, int B, int n_blk_max, long long stride,
                 long long total) {
    using E = typename Elem<DT>::type;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const long long u = i / D;
    const int d = (int)(i - u * D);
    const int r = (int)(u / H);
    // The new token does not depend on pos: its loads go out with pos's, so a
    // thread waits for one round trip before its stores (and, for a token that
    // completes its block, for one more before the summary stores).
    const int p = pos[r];
    const E kx = reinterpret_cast<const E*>(k_new)[i];
    const E vx = reinterpret_cast<const E*>(v_new)[i];
    if (p < 0 || p / B >= n_blk_max) return;  // no token, or past the store
    const int b = p / B, t = p - b * B;
    const size_t tile = ((size_t)u * n_blk_max + b) * (size_t)stride;
    if (summ && t == B - 1) {
        float lo = load_elem<DT>(&kx, 0), hi = lo;
        for (int j0 = 0; j0 < B - 1; j0 += 16) {  // rows written by earlier launches:
            float x[16];                            // 16 loads in flight, then reduce
#pragma unroll
            for (int k = 0; k < 16; ++k)
                x[k] = j0 + k < B - 1 ? load_elem<DT>(kt, tile + (size_t)(j0 + k) * D + d) : lo;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                lo = fminf(lo, x[k]);
                hi = fmaxf(hi, x[k]);
            }
        }
        reinterpret_cast<E*>(kt)[tile + (size_t)t * D + d] = kx;
        reinterpret_cast<E*>(vt)[tile + (size_t)d * B + t] = vx;
        const size_t so = ((size_t)u * n_blk_max + b) * 2 * D + d;
        store_elem<DT>(summ, so, lo);
        store_elem<DT>(summ, so + D, hi);
        return;
    }
    reinterpret_cast<E*>(kt)[tile + (size_t)t * D + d] = kx;
    reinterpret_cast<E*>(vt)[tile + (size_t)d * B + t] = vx;
}

extern "C" int oasis_append_kv(const oasis_shape* s, const void* k_new, const void* v_new,
                               const int32_t* pos, void* k_tiles, void* v_tiles,
                               int32_t n_blk_max, void* summaries, hipStream_t stream) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (!k_new || !v_new || !pos || !k_tiles || !v_tiles || n_blk_max <= 0) return OASIS_EINVAL;
    const long long total = (long long)s->batch * s->n_kv_heads * s->head_dim;
    const dim3 grid((unsigned)((total + 255) / 256));
    const long long stride = tile_stride_of(s);
    if (s->dtype == OASIS_F32)
        hipLaunchKernelGGL(append_kv_kernel<OASIS_F32>, grid, dim3(256), 0, stream, k_new, v_new,
                           pos, k_tiles, v_tiles, summaries, s->n_kv_heads, s->head_dim,
                           s->block_size, n_blk_max, stride, total);
    else
        hipLaunchKernelGGL(append_kv_kernel<OASIS_BF16>, grid, dim3(256), 0, stream, k_new, v_new,
                           pos, k_tiles, v_tiles, summaries, s->n_kv_heads, s->head_dim,
                           s->block_size, n_blk_max, stride, total);
    return launch_status();
}
