// Entry points of the per-layer lookahead path built on step_device.h:
// oasis_lookahead_step (scan + top-K + plan fused with the attention of the
// current resident set in one launch), oasis_score_topk (scan + top-K only),
// oasis_sparse_attn (attention only) and oasis_select_plan (plan only).
#include <mutex>

#include "step_device.h"

namespace oasis {

// Capped plan of every unit from an existing top-K tensor.  One workgroup per
// unit; the predicted row is staged in LDS and handed to plan_unit.
__global__ void __launch_bounds__(kNT)
plan_kernel(int H, int NQ, int pred_row, int K, const int32_t* __restrict__ topk_idx,
            const int32_t* slot_blk_in, const int32_t* slot_stamp_in, int32_t* slot_blk_out,
            int32_t* slot_stamp_out, int step, int cap, const int32_t* __restrict__ ins_blk,
            int32_t* __restrict__ plan_count,
            int32_t* __restrict__ plan_src, int32_t* __restrict__ plan_dst,
            int32_t* __restrict__ plan_evicted) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int u = blockIdx.x;
    const int r = u / H, g = u - (u / H) * H;
    const int K4 = pad4(K);
    LdsCursor cur{lds};
    int* P = cur.take<int>(K4);
    const PlanLds L = carve_plan(cur, K4);
    const int32_t* row = topk_idx + (((size_t)r * NQ + pred_row) * H + g) * K;
    for (int i = threadIdx.x; i < K4; i += kNT) P[i] = i < K ? row[i] : -1;
    const size_t so = (size_t)u * K;
    plan_load(slot_blk_in + so, slot_stamp_in + so, K, L);
    __syncthreads();
    plan_unit(P, K, slot_blk_out + so, slot_stamp_out + so, step, cap, ins_blk ? ins_blk[r] : -1,
              plan_count + u, plan_src + so, plan_dst + so,
              plan_evicted ? plan_evicted + so : nullptr, L);
}

static size_t plan_lds_bytes(int K) {
    return ((size_t)pad4(K) * 4 + 15) / 16 * 16 + plan_lds_size(K);  // P, then the plan state
}

// ------------------------------------------------------------ launching
static int set_lds(const void* kern, size_t lds) {
    if (lds <= 65536) return OASIS_OK;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
        hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EUNSUPPORTED;
    }
    return OASIS_OK;
}

template <int DT, int D, int NQ, int ATT, int NRG, bool SCAN, bool TOK = false>
static int launch_step(const StepArgs& a, size_t lds, hipStream_t st) {
    const long long per_xcd = (long long)((a.U + 7) / 8) *
                              ((SCAN ? a.scan_items : 0) + (ATT != kAttnNone ? a.attn_items : 0));
    const long long grid = 8 * per_xcd;
    if (grid == 0) return OASIS_OK;
    if (grid > 0x7fffffffLL) return OASIS_EUNSUPPORTED;
    auto kern = step_kernel<DT, D, NQ, ATT, NRG, SCAN, TOK>;
    int rc = set_lds(reinterpret_cast<const void*>(kern), lds);
    if (rc != OASIS_OK) return rc;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kNT), lds, st, a);
    return launch_status();
}

// Rows one attention item computes.
static int item_rows(const StepArgs& a) { return a.RGN > 1 ? a.G : a.NR; }

// Second launch of split units (see finish_kernel); nothing when no unit is split.
template <int DT, int D, int NQ>
static int launch_finish(const StepArgs& a, hipStream_t st) {
    const int sel = a.scan_items > 1 ? 1 : 0;
    const int mrg = (a.attn_items > 0 && a.S > 1) ? 1 : 0;
    if (!sel && !mrg) return OASIS_OK;
    const long long grid = 8LL * ((a.U + 7) / 8) * (sel * NQ + mrg * a.RGN);
    if (grid > 0x7fffffffLL) return OASIS_EUNSUPPORTED;
    // rows held in registers: wide workgroups (more waves per SIMD for the
    // latency-bound selection, plan and merge); otherwise kNT threads
    const bool wide = !sel || a.n_blk_max <= kSelRowMax;
    const int nt = wide ? kFinishNT : kNT;
    const size_t lds = finish_lds_bytes(a.K, a.n_blk_max, sel != 0, nt);
    auto kern = wide ? finish_kernel<DT, D, NQ, kFinishNT> : finish_kernel<DT, D, NQ, kNT>;
    int rc = set_lds(reinterpret_cast<const void*>(kern), lds);
    if (rc != OASIS_OK) return rc;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(nt), lds, st, a, sel, mrg);
    return launch_status();
}

template <int DT, int D, int NQ, int ATT, int NRG, bool SCAN, bool TOK = false>
static int launch_both(const StepArgs& a, size_t lds, hipStream_t st) {
    int rc = launch_step<DT, D, NQ, ATT, NRG, SCAN, TOK>(a, lds, st);
    if (rc != OASIS_OK) return rc;
    return launch_finish<DT, D, NQ>(a, st);
}

// Fused scan + attention launch: choose the instantiation (TOK: a new token
// per request is appended in the same launch).
template <int DT, int D, int NQ>
static int launch_fused(const StepArgs& a, int att, size_t lds, hipStream_t st) {
    if (a.pos) {
        if (att == kAttnMfma) {
            if constexpr (DT == OASIS_BF16) {
                if (item_rows(a) <= 16)
                    return launch_both<DT, D, NQ, kAttnMfma, 1, true, true>(a, lds, st);
                return launch_both<DT, D, NQ, kAttnMfma, 2, true, true>(a, lds, st);
            }
            return OASIS_EUNSUPPORTED;
        }
        return launch_both<DT, D, NQ, kAttnValu, 1, true, true>(a, lds, st);
    }
    if (att == kAttnMfma) {
        if constexpr (DT == OASIS_BF16) {
            if (item_rows(a) <= 16) return launch_both<DT, D, NQ, kAttnMfma, 1, true>(a, lds, st);
            return launch_both<DT, D, NQ, kAttnMfma, 2, true>(a, lds, st);
        }
        return OASIS_EUNSUPPORTED;
    }
    return launch_both<DT, D, NQ, kAttnValu, 1, true>(a, lds, st);
}

template <int DT, int D>
static int launch_attn_only(const StepArgs& a, int att, size_t lds, hipStream_t st) {
    if (att == kAttnMfma) {
        if constexpr (DT == OASIS_BF16) {
            if (item_rows(a) <= 16) return launch_both<DT, D, 1, kAttnMfma, 1, false>(a, lds, st);
            return launch_both<DT, D, 1, kAttnMfma, 2, false>(a, lds, st);
        }
        return OASIS_EUNSUPPORTED;
    }
    return launch_both<DT, D, 1, kAttnValu, 1, false>(a, lds, st);
}

enum class Role { kScan, kAttn, kFused };

static int dispatch(const StepArgs& a, int dtype, int D, int NQ, int att, Role role, size_t lds,
                    hipStream_t st) {
#define OASIS_DT_D(DT, DD)                                                                    \
    if (role == Role::kAttn) return launch_attn_only<DT, DD>(a, att, lds, st);                \
    if (role == Role::kScan) {                                                                \
        if (NQ == 1) return launch_both<DT, DD, 1, kAttnNone, 1, true>(a, lds, st);           \
        return launch_both<DT, DD, 2, kAttnNone, 1, true>(a, lds, st);                        \
    }                                                                                         \
    if (NQ == 1) return launch_fused<DT, DD, 1>(a, att, lds, st);                             \
    return launch_fused<DT, DD, 2>(a, att, lds, st);
    if (dtype == OASIS_F32) {
        if (D == 64) { OASIS_DT_D(OASIS_F32, 64) }
        OASIS_DT_D(OASIS_F32, 128)
    }
    if (D == 64) { OASIS_DT_D(OASIS_BF16, 64) }
    OASIS_DT_D(OASIS_BF16, 128)
#undef OASIS_DT_D
}

// ------------------------------------------------------------ workspace
struct WsLayout {
    size_t scores, part_ml, part_acc, total;
};

// Scratch of one call: global scores when a unit's scan is split or its scores
// do not fit in LDS (and the caller passed no scores buffer), and attention
// partials when units are split.
static bool scores_in_lds(const oasis_shape* s, int n_blk_max, const StepPlan& p, int NS) {
    (void)s;
    return p.NC == 1 && (size_t)NS * n_blk_max * 4 <= kScoreLdsMax;
}

// Scored rows: the query rows, or 2 when three rows average their two drafts.
static int scored_rows(const oasis_shape* s, const oasis_step_opts* o) {
    return (o && o->draft_avg) ? 2 : s->n_q;
}

static WsLayout ws_layout(const oasis_shape* s, int n_blk_max, bool scan, bool own_scores,
                          bool attn, const StepPlan& p, int NS) {
    WsLayout L{0, 0, 0, 0};
    const size_t U = (size_t)s->batch * s->n_kv_heads;
    const int NR = s->n_q * (s->n_q_heads / s->n_kv_heads);
    size_t off = 0;
    if (scan && own_scores && !scores_in_lds(s, n_blk_max, p, NS)) {
        L.scores = off;
        off += align_up((size_t)s->batch * NS * s->n_kv_heads * n_blk_max * 4, 256);
    }
    if (attn && p.S > 1) {
        L.part_ml = off;
        off += align_up(U * p.S * NR * 2 * 4, 256);
        L.part_acc = off;
        off += align_up(U * p.S * NR * (size_t)s->head_dim * 4, 256);
    }
    L.total = off;
    return L;
}

static int elem_bytes(const oasis_shape* s) { return s->dtype == OASIS_F32 ? 4 : 2; }

static int scan_check(const oasis_shape* s, int32_t n_blk_max, int32_t top_k,
                      const oasis_step_opts* o) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (n_blk_max <= 0 || top_k <= 0 || top_k > kMaxTopK) return OASIS_EINVAL;
    // Three query rows only as (normal, draft a, draft b) with the drafts averaged.
    const bool avg = o && o->draft_avg;
    if (avg != (s->n_q == 3)) return OASIS_EINVAL;
    if (o && o->use_alpha && !(o->alpha >= 0.f && o->alpha < 1e30f)) return OASIS_EINVAL;
    if (n_blk_max > 32768) return OASIS_EUNSUPPORTED;
    return OASIS_OK;
}

static void fill_variant(StepArgs& a, const oasis_shape* s, const oasis_step_opts* o) {
    a.NS = scored_rows(s, o);
    a.draft_avg = (o && o->draft_avg) ? 1 : 0;
    a.use_alpha = (o && o->use_alpha) ? 1 : 0;
    a.alpha = a.use_alpha ? o->alpha : 1.f;
}

static int attn_check(const oasis_shape* s, int32_t n_sel) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (n_sel < 0) return OASIS_EINVAL;
    if (s->n_q * (s->n_q_heads / s->n_kv_heads) > kMaxRows) return OASIS_EUNSUPPORTED;
    return OASIS_OK;
}

static int pick_attn(const oasis_shape* s, int impl, int* att) {
    const bool mfma_ok = s->dtype == OASIS_BF16 && s->block_size % 16 == 0;
    if (impl < 0 || impl > 2) return OASIS_EINVAL;
    if (impl == 2 && !mfma_ok) return OASIS_EUNSUPPORTED;
    const bool use = impl == 0 ? mfma_ok : impl == 2;
    *att = use ? kAttnMfma : kAttnValu;
    return OASIS_OK;
}

// Row groups of the attention: a unit with more than 16 rows (both query rows
// of a wide GQA group) on the MFMA path runs one item per query row, G <= 16
// rows each, instead of one item of two 16-row MFMA blocks.  Not with an
// appended token (that item also writes the token into the store).
static int row_groups(const oasis_shape* s, int att, bool tok) {
    const int G = s->n_q_heads / s->n_kv_heads;
    return (att == kAttnMfma && !tok && s->n_q > 1 && s->n_q * G > 16 && G <= 16) ? s->n_q : 1;
}

static void fill_shape(StepArgs& a, const oasis_shape* s) {
    a = StepArgs{};
    a.R = s->batch;
    a.NQ = s->n_q;
    a.Hq = s->n_q_heads;
    a.H = s->n_kv_heads;
    a.G = s->n_q_heads / s->n_kv_heads;
    a.NR = a.NQ * a.G;
    a.D = s->head_dim;
    a.B = s->block_size;
    a.U = s->batch * s->n_kv_heads;
    a.NS = s->n_q;
    a.alpha = 1.f;
    a.pred_row = -1;
    a.RGN = 1;
}

static void fill_attn(StepArgs& a, const oasis_shape* s, const void* q, const void* k_tiles,
                      const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                      int64_t unit_stride, const int32_t* tail_tile, const int32_t* tail_len,
                      float scale, void* out, float* lse, const StepPlan& p, int rgn, uint8_t* ws,
                      const WsLayout& L) {
    a.q = reinterpret_cast<const uint8_t*>(q);
    a.RGN = rgn;
    a.kt = reinterpret_cast<const uint8_t*>(k_tiles);
    a.vt = reinterpret_cast<const uint8_t*>(v_tiles);
    a.table = tile_table;
    a.n_sel = n_sel;
    a.unit_stride = unit_stride;
    a.tile_stride = tile_stride_of(s);
    a.tail_tile = tail_tile;
    a.tail_len = tail_len;
    const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)s->head_dim);
    a.scale_log2 = sc * kLog2e;
    a.out = out;
    a.lse = lse;
    a.S = p.S;
    a.per_split = p.per_split;
    a.attn_items = p.S * rgn;
    if (p.S > 1) {
        a.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
        a.part_acc = reinterpret_cast<float*>(ws + L.part_acc);
    }
}

static void fill_scan(StepArgs& a, const oasis_shape* s, const void* q, const void* summaries,
                      int32_t n_blk_max, const int32_t* n_blk, int32_t top_k, int32_t* topk_idx,
                      float* topk_score, float* scores, const StepPlan& p, uint8_t* ws,
                      const WsLayout& L) {
    a.q = reinterpret_cast<const uint8_t*>(q);
    a.summ = reinterpret_cast<const uint8_t*>(summaries);
    a.n_blk_max = n_blk_max;
    a.n_blk = n_blk;
    a.K = top_k;
    a.topk_idx = topk_idx;
    a.topk_score = topk_score;
    a.scores_lds = scores_in_lds(s, n_blk_max, p, a.NS) ? 1 : 0;
    a.scores = scores ? scores : (a.scores_lds ? nullptr : reinterpret_cast<float*>(ws + L.scores));
    a.NC = p.NC;
    a.chunk = p.chunk;
    a.scan_items = p.NC;
}

static size_t lds_for(const StepArgs& a, Role role, int att) {
    size_t b = 0;
    if (role != Role::kAttn)
        b = scan_lds_bytes(a.NS, a.D, a.K, a.scores_lds ? a.NS * a.n_blk_max : 0);
    if (role != Role::kScan) {
        const size_t t = attn_lds_bytes(att, item_rows(a), a.D, a.per_split > 0 ? a.per_split : 1,
                                        a.pos != nullptr);
        b = t > b ? t : b;
    }
    return b;
}

static bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

}  // namespace oasis

using namespace oasis;

// ================================================================ score + top-K
extern "C" size_t oasis_score_topk_workspace(const oasis_shape* s, int32_t n_blk_max,
                                             int32_t top_k, const oasis_step_opts* opts) {
    if (scan_check(s, n_blk_max, top_k, opts) != OASIS_OK) return 0;
    const StepPlan p = plan_items(s->batch * s->n_kv_heads, n_blk_max, 0, s->head_dim,
                                  s->block_size, elem_bytes(s), true, false,
                                  opts ? opts->scan_chunks : 0, 0);
    return ws_layout(s, n_blk_max, true, true, false, p, scored_rows(s, opts)).total;
}

extern "C" int oasis_score_topk(const oasis_shape* s, const void* q, const void* summaries,
                                int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                                int32_t* topk_idx, float* topk_score, float* scores,
                                const oasis_step_opts* opts, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    int st = scan_check(s, n_blk_max, top_k, opts);
    if (st != OASIS_OK) return st;
    if (!q || !summaries || !topk_idx) return OASIS_EINVAL;
    if (opts && opts->scan_chunks < 0) return OASIS_EINVAL;
    const StepPlan p = plan_items(s->batch * s->n_kv_heads, n_blk_max, 0, s->head_dim,
                                  s->block_size, elem_bytes(s), true, false,
                                  opts ? opts->scan_chunks : 0, 0);
    const int NS = scored_rows(s, opts);
    const WsLayout L = ws_layout(s, n_blk_max, true, scores == nullptr, false, p, NS);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return OASIS_EWORKSPACE;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    StepArgs a;
    fill_shape(a, s);
    fill_variant(a, s, opts);
    fill_scan(a, s, q, summaries, n_blk_max, n_blk, top_k, topk_idx, topk_score, scores, p, ws, L);
    return dispatch(a, s->dtype, s->head_dim, NS, kAttnNone, Role::kScan,
                    lds_for(a, Role::kScan, kAttnNone), stream);
}

// ================================================================ attention
extern "C" size_t oasis_sparse_attn_workspace(const oasis_shape* s, int32_t n_sel) {
    if (attn_check(s, n_sel) != OASIS_OK) return 0;
    // the larger of the layouts with and without row groups (impl decides)
    size_t best = 0;
    for (int rgn : {1, row_groups(s, kAttnMfma, false)}) {
        const StepPlan p = plan_items(s->batch * s->n_kv_heads, 0, n_sel, s->head_dim,
                                      s->block_size, elem_bytes(s), false, true, 0, 0, rgn);
        const size_t t = ws_layout(s, 0, false, false, true, p, s->n_q).total;
        best = t > best ? t : best;
    }
    return best;
}

extern "C" int oasis_sparse_attn_impl(const oasis_shape* s, const void* q, const void* k_tiles,
                                      const void* v_tiles, const int32_t* tile_table,
                                      int32_t n_sel, int64_t unit_stride,
                                      const int32_t* tail_tile, const int32_t* tail_len,
                                      float scale, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, int32_t impl, hipStream_t stream) {
    int st = attn_check(s, n_sel);
    if (st != OASIS_OK) return st;
    if (!q || !k_tiles || !v_tiles || !out || unit_stride < 0) return OASIS_EINVAL;
    if (n_sel > 0 && !tile_table) return OASIS_EINVAL;
    int att;
    if ((st = pick_attn(s, impl, &att)) != OASIS_OK) return st;
    const int rgn = row_groups(s, att, false);
    const StepPlan p = plan_items(s->batch * s->n_kv_heads, 0, n_sel, s->head_dim, s->block_size,
                                  elem_bytes(s), false, true, 0, 0, rgn);
    const WsLayout L = ws_layout(s, 0, false, false, true, p, s->n_q);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return OASIS_EWORKSPACE;
    StepArgs a;
    fill_shape(a, s);
    fill_attn(a, s, q, k_tiles, v_tiles, tile_table, n_sel, unit_stride, tail_tile, tail_len,
              scale, out, lse, p, rgn, reinterpret_cast<uint8_t*>(workspace), L);
    return dispatch(a, s->dtype, s->head_dim, s->n_q, att, Role::kAttn,
                    lds_for(a, Role::kAttn, att), stream);
}

extern "C" int oasis_sparse_attn(const oasis_shape* s, const void* q, const void* k_tiles,
                                 const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                                 int64_t unit_stride, const int32_t* tail_tile,
                                 const int32_t* tail_len, float scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return oasis_sparse_attn_impl(s, q, k_tiles, v_tiles, tile_table, n_sel, unit_stride, tail_tile,
                                  tail_len, scale, out, lse, workspace, workspace_bytes, 0, stream);
}

// ================================================================ plan
extern "C" int oasis_select_plan(int32_t batch, int32_t n_kv_heads, int32_t n_q, int32_t pred_row,
                                 int32_t top_k, const int32_t* topk_idx,
                                 const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                                 int32_t* slot_block_out, int32_t* slot_stamp_out, int32_t step,
                                 int32_t cap, const int32_t* ins_blk, int32_t* plan_count,
                                 int32_t* plan_src, int32_t* plan_dst, int32_t* plan_evicted,
                                 hipStream_t stream) {
    if (batch <= 0 || n_kv_heads <= 0 || (n_q != 1 && n_q != 2) || pred_row < 0 ||
        pred_row >= n_q || top_k <= 0 || top_k > kMaxTopK || cap < 0)
        return OASIS_EINVAL;
    if (!topk_idx || !slot_block_in || !slot_stamp_in || !slot_block_out || !slot_stamp_out ||
        !plan_count || !plan_src || !plan_dst)
        return OASIS_EINVAL;
    const long long U = (long long)batch * n_kv_heads;
    if (U > 0x7fffffffLL) return OASIS_EINVAL;
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)U), dim3(kNT), plan_lds_bytes(top_k), stream,
                       n_kv_heads, n_q, pred_row, top_k, topk_idx, slot_block_in, slot_stamp_in,
                       slot_block_out, slot_stamp_out, step, cap, ins_blk, plan_count, plan_src,
                       plan_dst, plan_evicted);
    return launch_status();
}

// ================================================================ fused step
static int step_check(const oasis_shape* s, int32_t n_blk_max, int32_t top_k, int32_t n_sel,
                      const oasis_step_opts* o) {
    int st = scan_check(s, n_blk_max, top_k, o);
    if (st != OASIS_OK) return st;
    return attn_check(s, n_sel);
}

static StepPlan step_plan(const oasis_shape* s, int32_t n_blk_max, int32_t n_sel,
                          const oasis_step_opts* o, int rgn) {
    return plan_items(s->batch * s->n_kv_heads, n_blk_max, n_sel, s->head_dim, s->block_size,
                      elem_bytes(s), true, true, o ? o->scan_chunks : 0, o ? o->attn_splits : 0,
                      rgn);
}

extern "C" size_t oasis_lookahead_step_workspace(const oasis_shape* s, int32_t n_blk_max,
                                                 int32_t top_k, int32_t n_sel,
                                                 const oasis_step_opts* opts) {
    if (step_check(s, n_blk_max, top_k, n_sel, opts) != OASIS_OK) return 0;
    // the larger of the layouts with and without row groups (the attention
    // path and the appended token decide)
    size_t best = 0;
    for (int rgn : {1, row_groups(s, kAttnMfma, false)}) {
        const size_t t = ws_layout(s, n_blk_max, true, true, true,
                                   step_plan(s, n_blk_max, n_sel, opts, rgn),
                                   scored_rows(s, opts)).total;
        best = t > best ? t : best;
    }
    return best;
}

// The fused layer-step; with `tok` (k_new, v_new, pos) also the append of
// one token per request (oasis_lookahead_step_append).
struct NewToken {
    const void* k_new;
    const void* v_new;
    const int32_t* pos;
};

static int lookahead(
    const oasis_shape* s, const void* q, const void* summaries, int32_t n_blk_max,
    const int32_t* n_blk, int32_t top_k, int32_t* topk_idx, float* topk_score, float* scores,
    const int32_t* slot_block_in, const int32_t* slot_stamp_in, int32_t* slot_block_out,
    int32_t* slot_stamp_out, int32_t step, int32_t cap, int32_t pred_row, const int32_t* ins_blk,
    int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst, int32_t* plan_evicted,
    const void* k_tiles, const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
    int64_t unit_stride, const int32_t* tail_tile, const int32_t* tail_len, float scale, void* out,
    float* lse, const oasis_step_opts* opts, void* workspace, size_t workspace_bytes,
    hipStream_t stream, const NewToken* tok) {
    int st = step_check(s, n_blk_max, top_k, n_sel, opts);
    if (st != OASIS_OK) return st;
    const int NS = scored_rows(s, opts);
    if (!q || !summaries || !topk_idx || !slot_block_in || !slot_stamp_in || !slot_block_out ||
        !slot_stamp_out || !plan_count || !plan_src || !plan_dst || !k_tiles || !v_tiles || !out)
        return OASIS_EINVAL;
    if (n_sel > 0 && !tile_table) return OASIS_EINVAL;
    if (pred_row < 0 || pred_row >= NS || cap < 0 || unit_stride < 0) return OASIS_EINVAL;
    if (opts && (opts->scan_chunks < 0 || opts->attn_splits < 0)) return OASIS_EINVAL;
    // The plan rewrites slots while attention reads the tile table: the
    // new slot tables must not overlap it.
    const size_t U = (size_t)s->batch * s->n_kv_heads;
    if (n_sel > 0 && (overlaps(slot_block_out, U * top_k * 4, tile_table, U * n_sel * 4) ||
                      overlaps(slot_stamp_out, U * top_k * 4, tile_table, U * n_sel * 4)))
        return OASIS_EINVAL;
    int att;
    if ((st = pick_attn(s, opts ? opts->attn_impl : 0, &att)) != OASIS_OK) return st;
    const int rgn = row_groups(s, att, tok != nullptr);
    const StepPlan p = step_plan(s, n_blk_max, n_sel, opts, rgn);
    const WsLayout L = ws_layout(s, n_blk_max, true, scores == nullptr, true, p, NS);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return OASIS_EWORKSPACE;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    StepArgs a;
    fill_shape(a, s);
    fill_variant(a, s, opts);
    fill_scan(a, s, q, summaries, n_blk_max, n_blk, top_k, topk_idx, topk_score, scores, p, ws, L);
    fill_attn(a, s, q, k_tiles, v_tiles, tile_table, n_sel, unit_stride, tail_tile, tail_len, scale,
              out, lse, p, rgn, ws, L);
    a.do_plan = 1;
    a.pred_row = pred_row;
    a.step = step;
    a.cap = cap;
    a.ins_blk = ins_blk;
    a.slot_blk_in = slot_block_in;
    a.slot_stamp_in = slot_stamp_in;
    a.slot_blk_out = slot_block_out;
    a.slot_stamp_out = slot_stamp_out;
    a.plan_count = plan_count;
    a.plan_src = plan_src;
    a.plan_dst = plan_dst;
    a.plan_evicted = plan_evicted;
    if (tok) {
        a.k_new = reinterpret_cast<const uint8_t*>(tok->k_new);
        a.v_new = reinterpret_cast<const uint8_t*>(tok->v_new);
        a.pos = tok->pos;
        a.kt_w = const_cast<uint8_t*>(a.kt);
        a.vt_w = const_cast<uint8_t*>(a.vt);
        a.summ_w = const_cast<uint8_t*>(a.summ);
    }
    return dispatch(a, s->dtype, s->head_dim, NS, att, Role::kFused,
                    lds_for(a, Role::kFused, att), stream);
}

extern "C" int oasis_lookahead_step(
    const oasis_shape* s, const void* q, const void* summaries, int32_t n_blk_max,
    const int32_t* n_blk, int32_t top_k, int32_t* topk_idx, float* topk_score, float* scores,
    const int32_t* slot_block_in, const int32_t* slot_stamp_in, int32_t* slot_block_out,
    int32_t* slot_stamp_out, int32_t step, int32_t cap, int32_t pred_row, const int32_t* ins_blk,
    int32_t* plan_count,
    int32_t* plan_src, int32_t* plan_dst, int32_t* plan_evicted, const void* k_tiles,
    const void* v_tiles, const int32_t* tile_table, int32_t n_sel, int64_t unit_stride,
    const int32_t* tail_tile, const int32_t* tail_len, float scale, void* out, float* lse,
    const oasis_step_opts* opts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return lookahead(s, q, summaries, n_blk_max, n_blk, top_k, topk_idx, topk_score, scores,
                            slot_block_in, slot_stamp_in, slot_block_out, slot_stamp_out, step, cap,
                            pred_row, ins_blk, plan_count, plan_src, plan_dst, plan_evicted,
                            k_tiles, v_tiles, tile_table, n_sel, unit_stride, tail_tile, tail_len,
                            scale, out, lse, opts, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int oasis_lookahead_step_append(
    const oasis_shape* s, const void* q, void* summaries, int32_t n_blk_max,
    const int32_t* n_blk, int32_t top_k, int32_t* topk_idx, float* topk_score, float* scores,
    const int32_t* slot_block_in, const int32_t* slot_stamp_in, int32_t* slot_block_out,
    int32_t* slot_stamp_out, int32_t step, int32_t cap, int32_t pred_row, const int32_t* ins_blk,
    int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst, int32_t* plan_evicted,
    void* k_tiles, void* v_tiles, const int32_t* tile_table, int32_t n_sel, int64_t unit_stride,
    const void* k_new, const void* v_new, const int32_t* pos, float scale, void* out, float* lse,
    const oasis_step_opts* opts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!k_new || !v_new || !pos || unit_stride != n_blk_max) return OASIS_EINVAL;
    // the token's rows are read as 16-byte vectors
    if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
        return OASIS_EINVAL;
    const NewToken tok{k_new, v_new, pos};
    return lookahead(s, q, summaries, n_blk_max, n_blk, top_k, topk_idx, topk_score, scores,
                            slot_block_in, slot_stamp_in, slot_block_out, slot_stamp_out, step, cap,
                            pred_row, ins_blk, plan_count, plan_src, plan_dst, plan_evicted,
                            k_tiles, v_tiles, tile_table, n_sel, unit_stride, nullptr, nullptr,
                            scale, out, lse, opts, workspace, workspace_bytes, stream, &tok);
}

// ================================================================ fused step, no allocation
// oasis_lookahead_step_noalloc: the split-unit scratch (block scores, attention
// partials) lives in this file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy for the life of
// the process; the host reaches it only through the address
// hipGetSymbolAddress returns on that device (the array's name is a host-side
// stand-in, not a device address).  Every call on one GPU shares the array.
static __device__ __align__(256) unsigned char scratch[OASIS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // per device, set on the first call there
}  // namespace

// Device address of `scratch` on the current device (looked up once per device,
// with that device current).
static int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return OASIS_EHIP;
    }
    if (dev < 0 || dev >= kScratchDevices) return OASIS_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return OASIS_EHIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return OASIS_OK;
}

extern "C" int oasis_lookahead_step_noalloc(
    const oasis_shape* s, const void* q, const void* summaries, int32_t n_blk_max,
    const int32_t* n_blk, int32_t top_k, int32_t* topk_idx, float* topk_score, float* scores,
    const int32_t* slot_block_in, const int32_t* slot_stamp_in, int32_t* slot_block_out,
    int32_t* slot_stamp_out, int32_t step, int32_t cap, int32_t pred_row, const int32_t* ins_blk,
    int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst, int32_t* plan_evicted,
    const void* k_tiles, const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
    int64_t unit_stride, const int32_t* tail_tile, const int32_t* tail_len, float scale, void* out,
    float* lse, const oasis_step_opts* opts, hipStream_t stream) {
    int st = step_check(s, n_blk_max, top_k, n_sel, opts);
    if (st != OASIS_OK) return st;
    // The scratch this call needs (0 when every unit fits one launch), checked
    // against the array's size before anything touches the GPU.
    const size_t need = oasis_lookahead_step_workspace(s, n_blk_max, top_k, n_sel, opts);
    if (need > (size_t)OASIS_NOALLOC_SCRATCH_BYTES) return OASIS_EWORKSPACE;
    void* ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != OASIS_OK) return st;
    if (stream && need > 0) {  // the scratch address belongs to the current device
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return OASIS_EHIP;
        }
        if (sdev != cur) return OASIS_EINVAL;
    }
    return lookahead(s, q, summaries, n_blk_max, n_blk, top_k, topk_idx, topk_score, scores,
                     slot_block_in, slot_stamp_in, slot_block_out, slot_stamp_out, step, cap,
                     pred_row, ins_blk, plan_count, plan_src, plan_dst, plan_evicted, k_tiles,
                     v_tiles, tile_table, n_sel, unit_stride, tail_tile, tail_len, scale, out,
                     lse, opts, ws, need > 0 ? (size_t)OASIS_NOALLOC_SCRATCH_BYTES : 0, stream,
                     nullptr);
}
