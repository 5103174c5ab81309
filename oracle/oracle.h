/*
 * oracle.h -- plain CPU reference of the lookahead sparse-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * Every floating-point quantity is double precision.  Callers pass the exact
 * values of their fp32 / bf16 tensors widened to double.
 *
 * Sources (web pages about "OasisKV: Scaling In-Decode KV Cache Beyond HBM
 * with Lookahead Sparse Prefetching"):
 *   [v2]     the paperpeel.com text of the paper (arXiv v2, sections numbered)
 *   [reader] the signal-papers reader text (earlier version, no headings)
 *   [metal]  the metallab.ai summary page (figure captions of the earlier version)
 *
 * Layouts (all contiguous, row-major):
 *   keys      [R][H][n_blk_max*B][D]       (= tiles [R][H][n_blk_max][B][D])
 *   summ      [R][H][n_blk_max][2][D]       row 0 = coordinate-wise min, row 1 = max
 *   q         [R][n_q][Hq][D]               query head h reads KV head h / (Hq/H)
 *   scores    [R][n_q][H][n_blk_max]
 *   topk      [R][n_q][H][K]
 *   slots     [R][H][K]
 *   plan      count [R][H], src/dst/evicted [R][H][K]
 *   tiles     [n_tiles][B][D]               tile id = (r*H+g)*unit_stride + local
 *   out       [R][n_q][Hq][D], lse [R][n_q][Hq]
 *
 * Return value: 0 on success, -1 on a bad argument.
 */
#ifndef OASIS_ORACLE_H
#define OASIS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oro_build_summaries(int R, int H, int D, int B, int n_blk_max,
                        const double* keys, const int32_t* seq_len,
                        int blk_begin, int blk_end, double* summ);

int oro_append_kv(int R, int H, int D, int B, int n_blk_max, double* keys, double* values,
                  const double* k_new, const double* v_new, const int32_t* pos, double* summ);

int oro_block_scores(int R, int n_q, int Hq, int H, int D, int n_blk_max,
                     const double* q, const double* summ, const int32_t* n_blk,
                     double* scores);

int oro_block_scores_variant(int R, int n_q_in, int Hq, int H, int D, int n_blk_max,
                             const double* q, const double* summ, const int32_t* n_blk,
                             double alpha, int draft_avg, double* scores);

int oro_topk(int R, int n_q, int H, int n_blk_max, const double* scores,
             const int32_t* n_blk, int K, int32_t* topk_idx, double* topk_score);

int oro_select_plan(int R, int H, int n_q, int pred_row, int K,
                    const int32_t* topk_idx, int32_t* slot_block,
                    int32_t* slot_stamp, int step, int cap, const int32_t* ins_blk,
                    int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst,
                    int32_t* plan_evicted);

int oro_copy_blocks(int R, int H, int n_blk_max, int K, long tile_bytes,
                    const uint8_t* host_k, const uint8_t* host_v,
                    uint8_t* res_k, uint8_t* res_v, const int32_t* plan_count,
                    const int32_t* plan_src, const int32_t* plan_dst);

int oro_sparse_attn(int R, int n_q, int Hq, int H, int D, int B,
                    const double* q, const double* k_tiles,
                    const double* v_tiles, long n_tiles,
                    const int32_t* tile_table, int n_sel, long unit_stride,
                    const int32_t* tail_tile, const int32_t* tail_len,
                    double scale, double* out, double* lse);

int oro_num_threads(void);
int oro_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
