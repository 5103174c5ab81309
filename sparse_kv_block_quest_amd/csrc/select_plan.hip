// Capped least-recently-selected KV selection and transfer plan.
//
// Sources: OasisKV, signal-papers reader text, paragraphs on the capped
// eviction policy (intersect predicted and resident sets, rank resident blocks
// outside the prediction by their last-selected step, pair each admitted block
// with one eviction target, at most C pairs per KV head per step) and on
// partial transfer at admission (the first working set comes from the first
// generated token's query); paperpeel v2 text, §3.3.2 (the cap applies once the
// first working set is fully seeded; exactly K blocks stay resident per head).
//
// One workgroup per (request, KV head) unit, one thread per slot / predicted
// rank.  Membership tests and the victim ordering are O(K) counting loops over
// LDS, so the plan is integer-only, deterministic and uses no atomics.
#include "oasis_internal.h"

namespace oasis {

constexpr int kPlanMaxK = 1024;

__global__ void __launch_bounds__(kPlanMaxK)
select_plan_kernel(int H, int NQ, int pred_row, int K, const int32_t* __restrict__ topk_idx,
                   const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                   int32_t* slot_block_out, int32_t* slot_stamp_out, int step, int cap,
                   int32_t* __restrict__ plan_count, int32_t* __restrict__ plan_src,
                   int32_t* __restrict__ plan_dst, int32_t* __restrict__ plan_evicted) {
    __shared__ int32_t P[kPlanMaxK];
    __shared__ int32_t blk[kPlanMaxK];
    __shared__ int32_t stamp[kPlanMaxK];
    __shared__ uint8_t hit[kPlanMaxK];
    __shared__ uint8_t miss[kPlanMaxK];
    __shared__ int32_t victim_of_rank[kPlanMaxK];
    __shared__ int32_t missing_of_rank[kPlanMaxK];
    __shared__ int32_t new_blk[kPlanMaxK];
    __shared__ int32_t new_stamp[kPlanMaxK];
    const int g = blockIdx.x, r = blockIdx.y;
    const int t = threadIdx.x;
    const size_t unit = (size_t)r * H + g;
    const size_t so = unit * K;
    const bool act = t < K;

    int empty = 0;
    if (act) {
        P[t] = topk_idx[(((size_t)r * NQ + pred_row) * H + g) * K + t];
        blk[t] = slot_block_in[so + t];
        stamp[t] = slot_stamp_in[so + t];
        empty = blk[t] == -1;
    }
    const int seeding = __syncthreads_or(empty);

    if (act) {
        const int32_t b = blk[t];
        int h = 0;
        if (b >= 0)
            for (int i = 0; i < K; ++i) h |= (P[i] == b);
        hit[t] = (uint8_t)h;
        const int32_t p = P[t];
        int res = 0;
        if (p >= 0)
            for (int s = 0; s < K; ++s) res |= (blk[s] == p);
        miss[t] = (uint8_t)(p >= 0 && !res);
    }
    __syncthreads();

    int n_missing = 0, n_victims = 0;
    if (act) {
        // Rank of this slot among the victims, ordered by (stamp, slot).
        const int32_t st = stamp[t];
        int vrank = 0;
        for (int s = 0; s < K; ++s) {
            if (hit[s]) continue;
            ++n_victims;
            vrank += (stamp[s] < st) || (stamp[s] == st && s < t);
        }
        if (!hit[t]) victim_of_rank[vrank] = t;
        // Rank of this predicted block among the missing ones, in P order.
        int mrank = 0;
        for (int i = 0; i < K; ++i) {
            n_missing += miss[i];
            mrank += (i < t) && miss[i];
        }
        if (miss[t]) missing_of_rank[mrank] = P[t];
        new_blk[t] = blk[t];
        new_stamp[t] = hit[t] ? step : stamp[t];
    }
    __syncthreads();

    int n = min(n_missing, n_victims);
    if (!seeding) n = min(n, cap);
    if (act) {
        if (t < n) {
            const int dst = victim_of_rank[t];
            const int src = missing_of_rank[t];
            plan_src[so + t] = src;
            plan_dst[so + t] = dst;
            if (plan_evicted) plan_evicted[so + t] = blk[dst];
            new_blk[dst] = src;
            new_stamp[dst] = step;
        } else {
            plan_src[so + t] = -1;
            plan_dst[so + t] = -1;
            if (plan_evicted) plan_evicted[so + t] = -1;
        }
    }
    __syncthreads();
    if (act) {
        slot_block_out[so + t] = new_blk[t];
        slot_stamp_out[so + t] = new_stamp[t];
    }
    if (t == 0) plan_count[unit] = n;
}

}  // namespace oasis

using namespace oasis;

extern "C" int oasis_select_plan(int32_t batch, int32_t n_kv_heads, int32_t n_q, int32_t pred_row,
                                 int32_t top_k, const int32_t* topk_idx,
                                 const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                                 int32_t* slot_block_out, int32_t* slot_stamp_out, int32_t step,
                                 int32_t cap, int32_t* plan_count, int32_t* plan_src,
                                 int32_t* plan_dst, int32_t* plan_evicted, hipStream_t stream) {
    if (batch <= 0 || n_kv_heads <= 0 || (n_q != 1 && n_q != 2) || pred_row < 0 ||
        pred_row >= n_q || top_k <= 0 || top_k > kPlanMaxK || cap < 0)
        return OASIS_EINVAL;
    if (!topk_idx || !slot_block_in || !slot_stamp_in || !slot_block_out || !slot_stamp_out ||
        !plan_count || !plan_src || !plan_dst)
        return OASIS_EINVAL;
    const int threads = (top_k + 63) / 64 * 64;
    hipLaunchKernelGGL(select_plan_kernel, dim3(n_kv_heads, batch), dim3(threads), 0, stream,
                       n_kv_heads, n_q, pred_row, top_k, topk_idx, slot_block_in, slot_stamp_in,
                       slot_block_out, slot_stamp_out, step, cap, plan_count, plan_src, plan_dst,
                       plan_evicted);
    return launch_status();
}
