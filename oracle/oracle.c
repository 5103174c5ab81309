/*
 * oracle.c -- plain CPU reference of the lookahead sparse-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares no
 * code with the HIP library.  Plain loops, double precision throughout,
 * OpenMP only across independent (request, KV head) units.  No blocking,
 * fusion or reordering beyond what each definition states.
 *
 * Source tags (pages about "OasisKV: Scaling In-Decode KV Cache Beyond HBM
 * with Lookahead Sparse Prefetching"):
 *   [v2]     paperpeel.com text of the paper (arXiv v2)
 *   [reader] signal-papers reader text (earlier version, no headings)
 *   [metal]  metallab.ai summary page
 * See oracle.h for the layouts.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oro_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following calls (timing runs on one host core). */
int oro_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return oro_num_threads();
}

/* Number of full blocks of request r. */
static int full_blocks(const int32_t* seq_len, int r, int B, int n_blk_max) {
    long L = seq_len ? (long)seq_len[r] : (long)n_blk_max * B;
    return (int)(L / B);
}

/*
 * Quest-style key summaries: for every full logical block of B keys, the
 * coordinate-wise minimum and maximum of its keys, per KV head.
 * [reader] paragraph on ranking non-resident blocks (min/max per logical
 * block); [metal] Fig. 7 caption (per-block min/max pooling); [v2] §4.1
 * (two summary rows per block).  The trailing partial block has no summary.
 * Only blocks in [blk_begin, blk_end) are written.
 */
int oro_build_summaries(int R, int H, int D, int B, int n_blk_max,
                        const double* keys, const int32_t* seq_len,
                        int blk_begin, int blk_end, double* summ) {
    if (R <= 0 || H <= 0 || D <= 0 || B <= 0 || n_blk_max <= 0 || !keys || !summ)
        return -1;
    for (int r = 0; r < R; ++r) {
        long L = seq_len ? (long)seq_len[r] : (long)n_blk_max * B;
        if (L < 0 || L > (long)n_blk_max * B) return -1;
    }
    if (blk_begin < 0) blk_begin = 0;
    if (blk_end > n_blk_max) blk_end = n_blk_max;
#pragma omp parallel for collapse(2) schedule(static)
    for (int r = 0; r < R; ++r) {
        for (int g = 0; g < H; ++g) {
            int n_r = full_blocks(seq_len, r, B, n_blk_max);
            int end = blk_end < n_r ? blk_end : n_r;
            for (int b = blk_begin; b < end; ++b) {
                const double* blk = keys + (((size_t)r * H + g) * n_blk_max + b) * (size_t)B * D;
                double* mn = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 0) * D;
                double* mx = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 1) * D;
                for (int d = 0; d < D; ++d) {
                    double lo = blk[d], hi = blk[d];
                    for (int i = 1; i < B; ++i) {
                        double v = blk[(size_t)i * D + d];
                        if (v < lo) lo = v;
                        if (v > hi) hi = v;
                    }
                    mn[d] = lo;
                    mx[d] = hi;
                }
            }
        }
    }
    return 0;
}

/*
 * Token append of a growing context: request r's new token (position pos[r],
 * skipped if negative) is written for every KV head into keys / values
 * ([R][H][n_blk_max*B][D], token-major here).  When the token is the last of
 * its block (pos % B == B - 1) and summ is given, that block's summary rows
 * are rebuilt from its B keys (coordinate-wise min and max, as in
 * oro_build_summaries).  [v2] §3.2.1 (newly generated blocks join the
 * working set) and Fig. 6 (per-block min/max key summaries kept in HBM);
 * [reader] paragraph on compressed-key updates.
 */
int oro_append_kv(int R, int H, int D, int B, int n_blk_max, double* keys, double* values,
                  const double* k_new, const double* v_new, const int32_t* pos, double* summ) {
    if (R <= 0 || H <= 0 || D <= 0 || B <= 0 || n_blk_max <= 0 || !keys || !values || !k_new ||
        !v_new || !pos)
        return -1;
    for (int r = 0; r < R; ++r)
        if (pos[r] >= (long)n_blk_max * B) return -1;
    for (int r = 0; r < R; ++r) {
        const long p = pos[r];
        if (p < 0) continue;
        const long b = p / B;
        for (int g = 0; g < H; ++g) {
            const size_t u = (size_t)r * H + g;
            double* krow = keys + (u * (size_t)n_blk_max * B + (size_t)p) * D;
            double* vrow = values + (u * (size_t)n_blk_max * B + (size_t)p) * D;
            for (int d = 0; d < D; ++d) {
                krow[d] = k_new[u * D + d];
                vrow[d] = v_new[u * D + d];
            }
            if (summ && p % B == B - 1) {
                const double* blk = keys + (u * (size_t)n_blk_max + (size_t)b) * (size_t)B * D;
                double* mn = summ + ((u * (size_t)n_blk_max + (size_t)b) * 2 + 0) * D;
                double* mx = summ + ((u * (size_t)n_blk_max + (size_t)b) * 2 + 1) * D;
                for (int d = 0; d < D; ++d) {
                    double lo = blk[d], hi = blk[d];
                    for (int i = 1; i < B; ++i) {
                        double v = blk[(size_t)i * D + d];
                        if (v < lo) lo = v;
                        if (v > hi) hi = v;
                    }
                    mn[d] = lo;
                    mx[d] = hi;
                }
            }
        }
    }
    return 0;
}

/*
 * Upper-bound block score, per KV head g and query row j:
 *   s_b = sum over the query heads h of group g, sum over d, of
 *         max(q_hd * max_bd, q_hd * min_bd).
 * This is [v2] §3.1, equation s_b(alpha), at alpha = 1 with c = (max+min)/2
 * and r = (max-min)/2, written per coordinate (Quest's bound).  The sum runs
 * over the query heads that share KV head g, because selection is per KV head
 * ([reader] paragraph on ranking non-resident blocks).  No 1/sqrt(D) factor.
 * Blocks at or beyond the request's full-block count get -inf.
 */
int oro_block_scores(int R, int n_q, int Hq, int H, int D, int n_blk_max,
                     const double* q, const double* summ, const int32_t* n_blk,
                     double* scores) {
    if (R <= 0 || n_q <= 0 || Hq <= 0 || H <= 0 || D <= 0 || n_blk_max <= 0 ||
        Hq % H != 0 || !q || !summ || !scores)
        return -1;
    const int G = Hq / H;
#pragma omp parallel for collapse(3) schedule(static)
    for (int r = 0; r < R; ++r) {
        for (int j = 0; j < n_q; ++j) {
            for (int g = 0; g < H; ++g) {
                int n_r = n_blk ? n_blk[r] : n_blk_max;
                if (n_r > n_blk_max) n_r = n_blk_max;
                double* out = scores + (((size_t)r * n_q + j) * H + g) * n_blk_max;
                for (int b = 0; b < n_blk_max; ++b) {
                    if (b >= n_r) {
                        out[b] = -INFINITY;
                        continue;
                    }
                    const double* mn = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 0) * D;
                    const double* mx = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 1) * D;
                    double s = 0.0;
                    for (int h = g * G; h < (g + 1) * G; ++h) {
                        const double* qh = q + (((size_t)r * n_q + j) * Hq + h) * D;
                        for (int d = 0; d < D; ++d) {
                            double a = qh[d] * mx[d];
                            double c = qh[d] * mn[d];
                            s += (a > c) ? a : c;
                        }
                    }
                    out[b] = s;
                }
            }
        }
    }
    return 0;
}

/*
 * Scoring variants ([v2] §3.1 equation s_b(alpha); §4.2.3 on the composition
 * with speculative decoding):
 *   s_b(alpha) = sum over the query heads h of group g of
 *                q_h . c_b + alpha * |q_h| . r_b,
 *   c_b = (max_b + min_b) / 2, r_b = (max_b - min_b) / 2  (coordinate-wise),
 * with alpha = 1 taken in the per-coordinate max form of oro_block_scores.
 * draft_avg: q holds n_q_in = 3 rows (normal, draft a, draft b); the scored
 * rows are row 0 and the element-wise mean of rows 1 and 2 (the two draft
 * queries averaged before scoring), so scores has 2 rows.
 */
int oro_block_scores_variant(int R, int n_q_in, int Hq, int H, int D, int n_blk_max,
                             const double* q, const double* summ, const int32_t* n_blk,
                             double alpha, int draft_avg, double* scores) {
    if (R <= 0 || n_q_in <= 0 || Hq <= 0 || H <= 0 || D <= 0 || n_blk_max <= 0 ||
        Hq % H != 0 || !q || !summ || !scores || (draft_avg && n_q_in != 3))
        return -1;
    const int G = Hq / H;
    const int n_s = draft_avg ? 2 : n_q_in;
#pragma omp parallel for collapse(3) schedule(static)
    for (int r = 0; r < R; ++r) {
        for (int j = 0; j < n_s; ++j) {
            for (int g = 0; g < H; ++g) {
                int n_r = n_blk ? n_blk[r] : n_blk_max;
                if (n_r > n_blk_max) n_r = n_blk_max;
                double* qs = (double*)malloc(sizeof(double) * (size_t)G * D);
                for (int h = 0; h < G; ++h)
                    for (int d = 0; d < D; ++d) {
                        const size_t hh = (size_t)g * G + h;
                        if (draft_avg && j == 1) {
                            const double a = q[(((size_t)r * n_q_in + 1) * Hq + hh) * D + d];
                            const double b = q[(((size_t)r * n_q_in + 2) * Hq + hh) * D + d];
                            qs[(size_t)h * D + d] = (a + b) / 2.0;
                        } else {
                            qs[(size_t)h * D + d] = q[(((size_t)r * n_q_in + j) * Hq + hh) * D + d];
                        }
                    }
                double* out = scores + (((size_t)r * n_s + j) * H + g) * n_blk_max;
                for (int b = 0; b < n_blk_max; ++b) {
                    if (b >= n_r) {
                        out[b] = -INFINITY;
                        continue;
                    }
                    const double* mn = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 0) * D;
                    const double* mx = summ + ((((size_t)r * H + g) * n_blk_max + b) * 2 + 1) * D;
                    double s = 0.0;
                    for (int h = 0; h < G; ++h) {
                        const double* qh = qs + (size_t)h * D;
                        for (int d = 0; d < D; ++d) {
                            if (alpha == 1.0) {
                                const double a = qh[d] * mx[d];
                                const double c = qh[d] * mn[d];
                                s += (a > c) ? a : c;
                            } else {
                                const double cen = (mx[d] + mn[d]) / 2.0;
                                const double rad = (mx[d] - mn[d]) / 2.0;
                                s += qh[d] * cen + alpha * fabs(qh[d]) * rad;
                            }
                        }
                    }
                    out[b] = s;
                }
                free(qs);
            }
        }
    }
    return 0;
}

typedef struct {
    double s;
    int32_t b;
} cand_t;

/* Ranking order: higher score first, then lower block index. */
static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->b > b->b) - (a->b < b->b);
}

/*
 * Per-KV-head top-K: for each (r, j, g), sort the request's full blocks by
 * (score descending, block ascending) and keep the first min(K, n_r).  Output
 * is ranked; unused positions get block -1 and score -inf.
 * [v2] §2.1 (top-K selection produces a per-head block set) and §3.3.1
 * (prediction stage ranks compressed keys); [reader] paragraph on ranking all
 * logical blocks independently for every KV head.
 */
int oro_topk(int R, int n_q, int H, int n_blk_max, const double* scores,
             const int32_t* n_blk, int K, int32_t* topk_idx, double* topk_score) {
    if (R <= 0 || n_q <= 0 || H <= 0 || n_blk_max <= 0 || K <= 0 || !scores || !topk_idx)
        return -1;
#pragma omp parallel for collapse(3) schedule(static)
    for (int r = 0; r < R; ++r) {
        for (int j = 0; j < n_q; ++j) {
            for (int g = 0; g < H; ++g) {
                int n_r = n_blk ? n_blk[r] : n_blk_max;
                if (n_r > n_blk_max) n_r = n_blk_max;
                if (n_r < 0) n_r = 0;
                const double* s = scores + (((size_t)r * n_q + j) * H + g) * n_blk_max;
                cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_r > 0 ? n_r : 1));
                for (int b = 0; b < n_r; ++b) {
                    c[b].s = s[b];
                    c[b].b = b;
                }
                qsort(c, (size_t)n_r, sizeof(cand_t), cand_cmp);
                size_t o = (((size_t)r * n_q + j) * H + g) * K;
                for (int i = 0; i < K; ++i) {
                    topk_idx[o + i] = i < n_r ? c[i].b : -1;
                    if (topk_score) topk_score[o + i] = i < n_r ? c[i].s : -INFINITY;
                }
                free(c);
            }
        }
    }
    return 0;
}

typedef struct {
    int32_t stamp;
    int32_t slot;
} victim_t;

/* Least recently selected first; ties by lower slot. */
static int victim_cmp(const void* pa, const void* pb) {
    const victim_t* a = (const victim_t*)pa;
    const victim_t* b = (const victim_t*)pb;
    if (a->stamp != b->stamp) return (a->stamp > b->stamp) - (a->stamp < b->stamp);
    return (a->slot > b->slot) - (a->slot < b->slot);
}

/*
 * Capped least-recently-selected selection, per unit (r, g):
 *   P      = ranked predicted blocks of row pred_row (entries >= 0)
 *   seeding: any slot empty (block -1) at entry -> no cap
 *   hits   : slots whose block is in P get stamp = step
 *   missing: P's blocks not resident, in P's rank order
 *   victims: slots whose block is not in P (empty ones included), ordered by
 *            (stamp ascending, slot ascending)
 *   n      = min(|missing|, |victims|, seeding ? unbounded : cap)
 *   pair i < n: src = missing[i], dst = victims[i], evicted = old block;
 *            the slot takes the new block with stamp = step.
 * Everything else stays as it was.  Plan entries i >= n are set to -1.
 *
 * Newly generated block (ins_blk[r] >= 0, optional): after the admissions the
 * block completed by request r's last token joins every KV head's resident
 * set, outside the cap.  If it is already resident its slot's stamp becomes
 * step; otherwise it replaces the slot with the smallest (stamp, slot) and is
 * recorded as plan entry n (count n + 1).  If that slot was itself admitted by
 * this plan (every slot then carries stamp = step), the insertion takes over
 * that entry instead: its source becomes the new block and the count stays.
 * [v2] §3.2.1 (newly generated blocks replace existing entries independently
 * for each KV head); the victim order is the plan's own (least recently
 * selected first).
 * [reader] paragraphs on the capped eviction policy (intersect, rank by
 * last-selected step, pair admitted blocks with eviction targets, at most C
 * pairs per KV head) and on partial transfer (first working set from the
 * first generated token's query); [v2] §3.3.2 (the cap applies after the
 * first working set has been fully seeded; exactly K blocks per head).
 */
int oro_select_plan(int R, int H, int n_q, int pred_row, int K,
                    const int32_t* topk_idx, int32_t* slot_block,
                    int32_t* slot_stamp, int step, int cap, const int32_t* ins_blk,
                    int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst,
                    int32_t* plan_evicted) {
    if (R <= 0 || H <= 0 || n_q <= 0 || K <= 0 || pred_row < 0 || pred_row >= n_q ||
        cap < 0 || !topk_idx || !slot_block || !slot_stamp || !plan_count || !plan_src ||
        !plan_dst)
        return -1;
    for (int r = 0; r < R; ++r) {
        for (int g = 0; g < H; ++g) {
            const int32_t* P = topk_idx + (((size_t)r * n_q + pred_row) * H + g) * K;
            int32_t* blk = slot_block + ((size_t)r * H + g) * K;
            int32_t* stamp = slot_stamp + ((size_t)r * H + g) * K;
            size_t po = ((size_t)r * H + g) * K;

            int seeding = 0;
            for (int s = 0; s < K; ++s)
                if (blk[s] == -1) seeding = 1;

            int* hit = (int*)calloc((size_t)K, sizeof(int));
            for (int s = 0; s < K; ++s) {
                if (blk[s] < 0) continue;
                for (int i = 0; i < K; ++i)
                    if (P[i] >= 0 && P[i] == blk[s]) hit[s] = 1;
            }
            for (int s = 0; s < K; ++s)
                if (hit[s]) stamp[s] = step;

            int32_t* missing = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
            int n_missing = 0;
            for (int i = 0; i < K; ++i) {
                if (P[i] < 0) continue;
                int resident = 0;
                for (int s = 0; s < K; ++s)
                    if (blk[s] == P[i]) resident = 1;
                if (!resident) missing[n_missing++] = P[i];
            }

            victim_t* victims = (victim_t*)malloc(sizeof(victim_t) * (size_t)K);
            int n_victims = 0;
            for (int s = 0; s < K; ++s) {
                if (hit[s]) continue;
                victims[n_victims].stamp = stamp[s];
                victims[n_victims].slot = s;
                ++n_victims;
            }
            qsort(victims, (size_t)n_victims, sizeof(victim_t), victim_cmp);

            int n = n_missing < n_victims ? n_missing : n_victims;
            if (!seeding && n > cap) n = cap;

            for (int i = 0; i < K; ++i) {
                plan_src[po + i] = -1;
                plan_dst[po + i] = -1;
                if (plan_evicted) plan_evicted[po + i] = -1;
            }
            for (int i = 0; i < n; ++i) {
                int dst = victims[i].slot;
                plan_src[po + i] = missing[i];
                plan_dst[po + i] = dst;
                if (plan_evicted) plan_evicted[po + i] = blk[dst];
                blk[dst] = missing[i];
                stamp[dst] = step;
            }
            const int32_t ins = ins_blk ? ins_blk[r] : -1;
            if (ins >= 0) {
                int at = -1;
                for (int s = 0; s < K; ++s)
                    if (blk[s] == ins) at = s;
                if (at >= 0) {
                    stamp[at] = step;
                } else {
                    int v = 0;
                    for (int s = 1; s < K; ++s)
                        if (stamp[s] < stamp[v] || (stamp[s] == stamp[v] && s < v)) v = s;
                    int entry = -1;
                    for (int i = 0; i < n; ++i)
                        if (plan_dst[po + i] == v) entry = i;
                    if (entry >= 0) {
                        plan_src[po + entry] = ins;
                    } else {
                        plan_src[po + n] = ins;
                        plan_dst[po + n] = v;
                        if (plan_evicted) plan_evicted[po + n] = blk[v];
                        ++n;
                    }
                    blk[v] = ins;
                    stamp[v] = step;
                }
            }
            plan_count[(size_t)r * H + g] = n;
            free(hit);
            free(missing);
            free(victims);
        }
    }
    return 0;
}

/*
 * Transfer of planned block-head tiles: the K tile and the V tile of every
 * (src -> dst) pair move from the full per-head store to the resident slots.
 * [v2] §3.2.1 (the gather reads selected per-head entries from pinned host
 * memory and writes them into HBM) and §4.1 Implementation.
 */
int oro_copy_blocks(int R, int H, int n_blk_max, int K, long tile_bytes,
                    const uint8_t* host_k, const uint8_t* host_v,
                    uint8_t* res_k, uint8_t* res_v, const int32_t* plan_count,
                    const int32_t* plan_src, const int32_t* plan_dst) {
    if (R <= 0 || H <= 0 || n_blk_max <= 0 || K <= 0 || tile_bytes <= 0 || !host_k ||
        !host_v || !res_k || !res_v || !plan_count || !plan_src || !plan_dst)
        return -1;
    for (int u = 0; u < R * H; ++u) {
        int n = plan_count[u];
        if (n < 0 || n > K) return -1;
        for (int i = 0; i < n; ++i) {
            int src = plan_src[(size_t)u * K + i];
            int dst = plan_dst[(size_t)u * K + i];
            if (src < 0 || src >= n_blk_max || dst < 0 || dst >= K) return -1;
            size_t so = ((size_t)u * n_blk_max + src) * (size_t)tile_bytes;
            size_t d_o = ((size_t)u * K + dst) * (size_t)tile_bytes;
            memcpy(res_k + d_o, host_k + so, (size_t)tile_bytes);
            memcpy(res_v + d_o, host_v + so, (size_t)tile_bytes);
        }
    }
    return 0;
}

/*
 * Decode attention of every stacked query row over the unit's selected tiles
 * plus the active local block:
 *   T   = the B tokens of every tile (r*H+g)*unit_stride + table[r][g][s]
 *         with table entry >= 0, plus the first tail_len[r] tokens of tile
 *         (r*H+g)*unit_stride + tail_tile[r][g] when both are given and >= 0
 *   z_i = scale * q . k_i          (g = h / (Hq/H); scale <= 0 -> 1/sqrt(D))
 *   o   = sum_i exp(z_i - z_max) v_i / sum_i exp(z_i - z_max)
 *   lse = z_max + log(sum_i exp(z_i - z_max));   T empty -> o = 0, lse = -inf
 * [v2] §3.1 and Fig. 6 (one call over one resident working set returns the
 * outputs of both stacked queries) and §4.1 (each head also attends its
 * active local block: K + 1 blocks).
 */
int oro_sparse_attn(int R, int n_q, int Hq, int H, int D, int B,
                    const double* q, const double* k_tiles,
                    const double* v_tiles, long n_tiles,
                    const int32_t* tile_table, int n_sel, long unit_stride,
                    const int32_t* tail_tile, const int32_t* tail_len,
                    double scale, double* out, double* lse) {
    if (R <= 0 || n_q <= 0 || Hq <= 0 || H <= 0 || D <= 0 || B <= 0 || Hq % H != 0 ||
        n_sel < 0 || unit_stride < 0 || !q || !k_tiles || !v_tiles || !out)
        return -1;
    if (n_sel > 0 && !tile_table) return -1;
    const int G = Hq / H;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)D);
    const int use_tail = tail_tile != NULL && tail_len != NULL;
    int bad = 0;
#pragma omp parallel for collapse(3) schedule(static) reduction(| : bad)
    for (int r = 0; r < R; ++r) {
        for (int j = 0; j < n_q; ++j) {
            for (int h = 0; h < Hq; ++h) {
                const int g = h / G;
                const size_t unit = (size_t)r * H + g;
                const double* qh = q + (((size_t)r * n_q + j) * Hq + h) * D;
                double* o = out + (((size_t)r * n_q + j) * Hq + h) * D;
                long max_tok = (long)n_sel * B + B;
                double* z = (double*)malloc(sizeof(double) * (size_t)max_tok);
                long* tok = (long*)malloc(sizeof(long) * (size_t)max_tok);
                long n_tok = 0;
                for (int s = 0; s < n_sel; ++s) {
                    int32_t t = tile_table[unit * n_sel + s];
                    if (t < 0) continue;
                    long id = (long)unit * unit_stride + t;
                    if (id >= n_tiles) { bad = 1; continue; }
                    for (int i = 0; i < B; ++i) tok[n_tok++] = id * B + i;
                }
                if (use_tail) {
                    int32_t t = tail_tile[unit];
                    int32_t L = tail_len[r];
                    if (t >= 0 && L > 0) {
                        long id = (long)unit * unit_stride + t;
                        if (id >= n_tiles || L > B) bad = 1;
                        else
                            for (int i = 0; i < L; ++i) tok[n_tok++] = id * B + i;
                    }
                }
                for (long i = 0; i < n_tok; ++i) {
                    const double* k = k_tiles + (size_t)tok[i] * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += qh[d] * k[d];
                    z[i] = scale * dot;
                }
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                if (n_tok == 0) {
                    if (lse) lse[((size_t)r * n_q + j) * Hq + h] = -INFINITY;
                } else {
                    double zmax = z[0];
                    for (long i = 1; i < n_tok; ++i)
                        if (z[i] > zmax) zmax = z[i];
                    double sum = 0.0;
                    for (long i = 0; i < n_tok; ++i) {
                        double w = exp(z[i] - zmax);
                        sum += w;
                        const double* v = v_tiles + (size_t)tok[i] * D;
                        for (int d = 0; d < D; ++d) o[d] += w * v[d];
                    }
                    for (int d = 0; d < D; ++d) o[d] /= sum;
                    if (lse) lse[((size_t)r * n_q + j) * Hq + h] = zmax + log(sum);
                }
                free(z);
                free(tok);
            }
        }
    }
    return bad ? -1 : 0;
}
