// Summary scan (upper-bound block scores) and per-KV-head top-K.
//
// Score: OasisKV paperpeel v2 text, §3.1, equation s_b(alpha) at alpha = 1,
// summed over the query heads of one KV head's group (selection is per KV head:
// signal-papers reader text, paragraph on ranking non-resident blocks).
// Written per coordinate as sum_h sum_d max(q_hd*max_bd, q_hd*min_bd), which
// factorises into P_g . max_b + N_g . min_b with P_g = sum_h max(q_h, 0) and
// N_g = sum_h min(q_h, 0); the scan therefore reads each block's two summary
// rows once for all stacked query rows and costs 2*D FMAs per row per block
// whatever the group size.
//
// Top-K: v2 §3.3.1 (prediction ranks the compressed keys into the per-head
// block set); reader text (every KV head ranks all logical blocks on its own).
// Ranked by (score descending, block ascending).  Implemented as an MSB-first
// 8-bit radix select over order-preserving uint32 keys held in LDS, an
// index-ordered compaction of the threshold ties, and a counting rank of the
// K survivors: every step is integer work on fixed keys, so the result is
// deterministic and exact for the fp32 scores it is given.
#include "oasis_internal.h"

namespace oasis {

// ------------------------------------------------------------------ scan
// grid (chunks, H, R); 256 threads.  LPR lanes share one block (one 16-byte
// chunk of the min row and of the max row each); a wave covers 64/LPR blocks
// per pass.  P/N for all stacked rows of this KV head sit in registers.
template <int DT, int D, int NQ>
__global__ void __launch_bounds__(256)
block_scores_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ summ,
                    const int32_t* __restrict__ n_blk, float* __restrict__ scores, int Hq,
                    int H, int n_blk_max, int chunk) {
    constexpr int EB = Elem<DT>::bytes;
    constexpr int VEC = 16 / EB;
    constexpr int LPR = D / VEC;
    constexpr int BPP = 256 / LPR;  // blocks per pass of the workgroup
    __shared__ float pn_s[NQ][2][D];
    const int g = blockIdx.y, r = blockIdx.z;
    const int G = Hq / H;
    for (int idx = threadIdx.x; idx < NQ * D; idx += 256) {
        const int j = idx / D, d = idx % D;
        float p = 0.f, n = 0.f;
        for (int h = 0; h < G; ++h) {
            const float x = load_elem<DT>(q, (((size_t)r * NQ + j) * Hq + g * G + h) * D + d);
            p += x > 0.f ? x : 0.f;
            n += x < 0.f ? x : 0.f;
        }
        pn_s[j][0][d] = p;
        pn_s[j][1][d] = n;
    }
    __syncthreads();
    const int c = threadIdx.x % LPR;
    float P[NQ][VEC], N[NQ][VEC];
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            P[j][e] = pn_s[j][0][c * VEC + e];
            N[j][e] = pn_s[j][1][c * VEC + e];
        }
    const int n_r = n_blk ? min(max(n_blk[r], 0), n_blk_max) : n_blk_max;
    const int b_begin = blockIdx.x * chunk;
    const int b_end = min(b_begin + chunk, n_blk_max);
    const size_t unit = (size_t)r * H + g;
    const uint4* base = reinterpret_cast<const uint4*>(summ) + unit * n_blk_max * 2 * LPR + c;
    const int n_pass = (b_end - b_begin + BPP - 1) / BPP;
    for (int it = 0; it < n_pass; ++it) {
        const int b = b_begin + it * BPP + threadIdx.x / LPR;
        const bool in_range = b < b_end;
        const bool valid = in_range && b < n_r;
        float acc[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) acc[j] = 0.f;
        if (valid) {
            const uint4 mn_raw = base[(size_t)b * 2 * LPR];
            const uint4 mx_raw = base[(size_t)b * 2 * LPR + LPR];
            float mn[VEC], mx[VEC];
            unpack16<DT>(mn_raw, mn);
            unpack16<DT>(mx_raw, mx);
#pragma unroll
            for (int j = 0; j < NQ; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    acc[j] = fmaf(P[j][e], mx[e], acc[j]);
                    acc[j] = fmaf(N[j][e], mn[e], acc[j]);
                }
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1)
#pragma unroll
            for (int j = 0; j < NQ; ++j) acc[j] += __shfl_xor(acc[j], off, LPR);
        if (in_range && c == 0) {
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                scores[(((size_t)r * NQ + j) * H + g) * n_blk_max + b] =
                    valid ? acc[j] : -__builtin_inff();
        }
    }
}

// ------------------------------------------------------------------ top-K
constexpr int kTopkThreads = 512;
constexpr int kTopkLdsMax = 12288;  // scores staged in LDS up to this many blocks

// Inclusive prefix sum of one value per thread over the workgroup (NT threads).
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    if (lane == 63) wave_tot[w] = v;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += wave_tot[i];
    __syncthreads();
    return v + base;
}

// grid (H, NQ, R).  One workgroup ranks one (request, row, KV head) problem.
__global__ void __launch_bounds__(kTopkThreads)
topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ n_blk, int n_blk_max,
            int NQ, int H, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score,
            int stage_lds) {
    constexpr int NT = kTopkThreads;
    extern __shared__ float s_lds[];
    __shared__ int hist[256];
    __shared__ int wave_tot[NT / 64];
    __shared__ int sh_digit, sh_greater;
    __shared__ uint32_t sel_key[1024];
    __shared__ int sel_idx[1024];
    const int g = blockIdx.x, j = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x;
    const int n = n_blk ? min(max(n_blk[r], 0), n_blk_max) : n_blk_max;
    const float* src = scores + (((size_t)r * NQ + j) * H + g) * n_blk_max;
    if (stage_lds) {
        for (int i = tid; i < n; i += NT) s_lds[i] = src[i];
        __syncthreads();
        src = s_lds;
    }
    const size_t out_base = (((size_t)r * NQ + j) * H + g) * K;
    const int Kp = min(K, n);

    // MSB-first radix select of the Kp-th largest key.
    uint32_t prefix = 0, mask = 0;
    int remaining = Kp;
    for (int shift = 24; shift >= 0 && Kp > 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint32_t k = float_key(src[i]);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        // Suffix sums over digits (largest digit first).
        const int cnt = tid < 256 ? hist[255 - tid] : 0;
        const int cum = block_inclusive_scan<NT>(cnt, wave_tot);
        if (tid < 256 && cum >= remaining && cum - cnt < remaining) {
            sh_digit = 255 - tid;
            sh_greater = cum - cnt;
        }
        __syncthreads();
        prefix |= uint32_t(sh_digit) << shift;
        mask |= 255u << shift;
        remaining -= sh_greater;
        __syncthreads();
    }
    // prefix is now the Kp-th largest key T; take every key > T and the first
    // `remaining` keys == T in block order.
    const int per = (n + NT - 1) / NT;
    const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
    int n_eq = 0;
    if (Kp > 0)
        for (int i = i0; i < i1; ++i) n_eq += float_key(src[i]) == prefix;
    const int eq_before = block_inclusive_scan<NT>(n_eq, wave_tot) - n_eq;
    int n_sel = 0;
    if (Kp > 0) {
        int e = eq_before;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = float_key(src[i]);
            if (k > prefix) ++n_sel;
            else if (k == prefix) n_sel += (e++ < remaining);
        }
    }
    int pos = block_inclusive_scan<NT>(n_sel, wave_tot) - n_sel;
    if (Kp > 0) {
        int e = eq_before;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = float_key(src[i]);
            bool take = k > prefix;
            if (k == prefix) take = (e++ < remaining);
            if (take) {
                sel_key[pos] = k;
                sel_idx[pos] = i;
                ++pos;
            }
        }
    }
    __syncthreads();
    // Counting rank of every survivor under (key desc, block asc).
    for (int a = tid; a < Kp; a += NT) {
        const uint32_t ka = sel_key[a];
        const int ia = sel_idx[a];
        int rank = 0;
        for (int b = 0; b < Kp; ++b) {
            const uint32_t kb = sel_key[b];
            rank += (kb > ka) || (kb == ka && sel_idx[b] < ia);
        }
        topk_idx[out_base + rank] = ia;
        if (topk_score) topk_score[out_base + rank] = src[ia];
    }
    for (int a = Kp + tid; a < K; a += NT) {
        topk_idx[out_base + a] = -1;
        if (topk_score) topk_score[out_base + a] = -__builtin_inff();
    }
}

template <int DT, int D>
static void launch_scores(int nq, const void* q, const void* summ, const int32_t* n_blk,
                          float* scores, int R, int Hq, int H, int n_blk_max, hipStream_t st) {
    const int chunk = 256;
    dim3 grid((n_blk_max + chunk - 1) / chunk, H, R);
    auto q8 = reinterpret_cast<const uint8_t*>(q);
    auto s8 = reinterpret_cast<const uint8_t*>(summ);
    if (nq == 1)
        hipLaunchKernelGGL((block_scores_kernel<DT, D, 1>), grid, dim3(256), 0, st, q8, s8, n_blk,
                           scores, Hq, H, n_blk_max, chunk);
    else
        hipLaunchKernelGGL((block_scores_kernel<DT, D, 2>), grid, dim3(256), 0, st, q8, s8, n_blk,
                           scores, Hq, H, n_blk_max, chunk);
}

}  // namespace oasis

using namespace oasis;

static int score_topk_check(const oasis_shape* s, int32_t n_blk_max, int32_t top_k) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (n_blk_max <= 0 || top_k <= 0 || top_k > 1024) return OASIS_EINVAL;
    if (n_blk_max > 32768) return OASIS_EUNSUPPORTED;
    return OASIS_OK;
}

extern "C" size_t oasis_score_topk_workspace(const oasis_shape* s, int32_t n_blk_max,
                                             int32_t top_k) {
    if (score_topk_check(s, n_blk_max, top_k) != OASIS_OK) return 0;
    return align_up((size_t)s->batch * s->n_q * s->n_kv_heads * n_blk_max * sizeof(float), 256);
}

extern "C" int oasis_score_topk(const oasis_shape* s, const void* q, const void* summaries,
                                int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                                int32_t* topk_idx, float* topk_score, float* scores,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = score_topk_check(s, n_blk_max, top_k);
    if (st != OASIS_OK) return st;
    if (!q || !summaries || !topk_idx) return OASIS_EINVAL;
    float* sc = scores;
    if (!sc) {
        if (!workspace || workspace_bytes < oasis_score_topk_workspace(s, n_blk_max, top_k))
            return OASIS_EWORKSPACE;
        sc = reinterpret_cast<float*>(workspace);
    }
    const int R = s->batch, Hq = s->n_q_heads, H = s->n_kv_heads, D = s->head_dim;
    if (s->dtype == OASIS_F32) {
        if (D == 64)
            launch_scores<OASIS_F32, 64>(s->n_q, q, summaries, n_blk, sc, R, Hq, H, n_blk_max, stream);
        else
            launch_scores<OASIS_F32, 128>(s->n_q, q, summaries, n_blk, sc, R, Hq, H, n_blk_max, stream);
    } else {
        if (D == 64)
            launch_scores<OASIS_BF16, 64>(s->n_q, q, summaries, n_blk, sc, R, Hq, H, n_blk_max, stream);
        else
            launch_scores<OASIS_BF16, 128>(s->n_q, q, summaries, n_blk, sc, R, Hq, H, n_blk_max, stream);
    }
    const int stage = n_blk_max <= kTopkLdsMax;
    const size_t lds = stage ? (size_t)n_blk_max * sizeof(float) : 0;
    hipLaunchKernelGGL(topk_kernel, dim3(H, s->n_q, R), dim3(kTopkThreads), lds, stream, sc, n_blk,
                       n_blk_max, s->n_q, H, top_k, topk_idx, topk_score, stage);
    return launch_status();
}
