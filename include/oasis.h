/*
 * oasis.h -- C ABI of liboasis.so, the MI355X (gfx950) hot path of lookahead
 * sparse-KV decode attention.
 *
 * Per layer and decode step the path (1) keeps Quest-style min/max key
 * summaries per logical block, (2) scans them with the stacked normal and
 * draft queries to bound every block's attention score per KV head, (3) takes
 * a per-head top-K, (4) diffs the prediction against the resident set into a
 * capped least-recently-selected transfer plan, (5) copies planned tiles from
 * pinned host memory into HBM, and (6) runs paged GQA decode attention of both
 * stacked queries over the resident tiles in one call.  Around it: the append
 * of each decode step's token (growing contexts) and a decode-host cache of
 * whole blocks in front of a remote KV store.
 *
 * Sources (web pages about "OasisKV: Scaling In-Decode KV Cache Beyond HBM
 * with Lookahead Sparse Prefetching"):
 *   [v2]     the paperpeel.com text of the paper (arXiv v2, numbered sections)
 *   [reader] the signal-papers reader text (earlier version, no headings;
 *            cited by paragraph topic)
 *   [metal]  the metallab.ai summary page (figure captions)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller unless stated otherwise.
 *    The kernel entry points allocate nothing, keep no state between calls and
 *    never synchronise: every call validates its host-side arguments, enqueues
 *    its kernels on `stream` and returns.  They are thread-safe.  The one
 *    exception is the decode-host block cache (oasis_host_tier_*), a
 *    caller-created host object with its own threads, staging and stream.
 *  - All arrays are dense and row-major in the layouts given below.
 *  - dtype (oasis_shape.dtype) applies to q, keys, values, summaries and out.
 *    Scores, lse and all accumulation are fp32.
 *  - Ids that address memory are range-checked where they are used: a tile
 *    table entry or active-block tile outside [0, unit_stride), a token
 *    position past the store, and a plan entry whose source block or
 *    destination slot lies outside its store are skipped (the entry is
 *    treated as empty), so a corrupt id cannot make a kernel touch memory
 *    outside the caller's buffers.  Other device-side preconditions are NOT
 *    checked and violating them is undefined behaviour: distinct ids in one
 *    table row, finite inputs, buffers at least as large as stated.
 *  - Notation: R batch, n_q stacked query rows (1 or 2; row 0 = normal query
 *    of step t, row 1 = draft query of step t+1; 3 with two drafts, see
 *    oasis_step_opts), n_s scored rows (n_q, or 2 when the two drafts are
 *    averaged), Hq query heads, H KV heads,
 *    G = Hq / H (query head h reads KV head h / G), D head dim, B block size,
 *    K top-K = resident slots per KV head, unit = one (request r, KV head g)
 *    pair with index u = r*H + g.
 *  - Tiles: a K tile holds the B keys of one block of one KV head, token-major
 *    [B][D].  A V tile holds the same block's values DIM-major [D][B] (value
 *    of token i, dim d at d*B + i).  Tile t of a store starts t * tile_stride
 *    elements after the store's base (oasis_shape.tile_stride; B*D when 0).
 */
#ifndef OASIS_H
#define OASIS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OASIS_OK 0
#define OASIS_EINVAL (-1)       /* null required pointer, bad size or index argument */
#define OASIS_EUNSUPPORTED (-2) /* dtype / head_dim / block size / group size not built */
#define OASIS_EWORKSPACE (-3)   /* workspace missing or smaller than the query says */
#define OASIS_EHIP (-4)         /* a kernel launch failed (hipGetLastError) */

typedef enum { OASIS_F32 = 0, OASIS_BF16 = 1 } oasis_dtype;

typedef struct oasis_shape {
    int32_t batch;       /* R >= 1 */
    int32_t n_q;         /* stacked query rows: 1, 2, or 3 (see oasis_step_opts.draft_avg) */
    int32_t n_q_heads;   /* Hq >= 1, multiple of n_kv_heads */
    int32_t n_kv_heads;  /* H >= 1 */
    int32_t head_dim;    /* D: 64 or 128 */
    int32_t block_size;  /* B: power of two, 1..64 (16 in every measured workload) */
    int32_t dtype;       /* oasis_dtype */
    int64_t tile_stride; /* elements from one K (or V) tile to the next in a tile store;
                            0 = B*D (dense).  2*B*D with v = k + B*D interleaves each
                            block-head's K and V tiles into one 2*B*D-element record, which
                            the attention gathers as one contiguous piece.  Otherwise
                            >= B*D and a multiple of 16 bytes. */
} oasis_shape;

/*
 * Tuning and scoring variants of oasis_score_topk and oasis_lookahead_step.  A
 * NULL pointer or zero fields mean: automatic tuning, the exact bound, no
 * draft averaging.
 *   use_alpha, alpha  score s_b(alpha) = sum_h q_h.c_b + alpha*|q_h|.r_b with
 *                     c_b, r_b the block's centre and radius ([v2] §3.1,
 *                     equation s_b(alpha)); alpha = 1 is the exact bound used
 *                     otherwise; 0 <= alpha < 1e30
 *   draft_avg         q holds three rows (normal, draft a, draft b; n_q = 3):
 *                     the two draft queries are averaged element-wise before
 *                     scoring ([v2] §4.2.3, composition with speculative
 *                     decoding), so the scored rows are row 0 and the mean
 *                     (top-K and scores have 2 rows; attention still covers
 *                     all three rows).  Required exactly when n_q = 3.
 */
typedef struct oasis_step_opts {
    int32_t scan_chunks; /* workgroups that share one unit's summary scan (0 = auto) */
    int32_t attn_splits; /* workgroups that share one unit's attention (0 = auto) */
    int32_t attn_impl;   /* 0 automatic, 1 VALU, 2 MFMA (as oasis_sparse_attn_impl) */
    int32_t use_alpha;   /* 1: score s_b(alpha) with the alpha below */
    float alpha;
    int32_t draft_avg;   /* 1: three query rows, drafts averaged before scoring */
} oasis_step_opts;

/* Human-readable text of a status code.  Never NULL; static storage. */
const char* oasis_status_string(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int oasis_version(void);

/*
 * Build per-block key summaries.
 * Defines: for every unit u and full block b (b < floor(L_r / B)) in
 * [blk_begin, blk_end), summaries[u][b][0][d] = min over the block's B keys of
 * key[d] and summaries[u][b][1][d] = max (coordinate-wise; exact, no rounding).
 * [reader] paragraph on ranking non-resident blocks (coordinate-wise min and
 * max of the keys of each logical block); [metal] Fig. 7 caption (per-block
 * min/max pooling); [v2] §4.1 (two summary rows per 16-token block, 1/16 of
 * the KV cache).
 *   s          shape; uses batch, n_kv_heads, head_dim, block_size, dtype
 *   keys       K tile store of the layer, tile (u*n_blk_max + b) = block b of
 *              unit u, [B][D] (dtype), tiles tile_stride apart
 *   n_blk_max  blocks per unit in `keys` and `summaries`
 *   seq_len    [R] int32 context lengths, or NULL = n_blk_max*B for every
 *              request; each must be in [0, n_blk_max*B]
 *   blk_begin, blk_end  block range to (re)build; clipped to [0, full blocks);
 *              an incremental update after a block completes passes [b, b+1)
 *   summaries  [R][H][n_blk_max][2][D] (dtype) output; entries outside the
 *              range and the trailing partial block are not written
 * Errors: EINVAL (null pointer, sizes <= 0, blk_begin > blk_end),
 *         EUNSUPPORTED (dtype, D, B), EHIP.
 */
int oasis_build_summaries(const oasis_shape* s, const void* keys, int32_t n_blk_max,
                          const int32_t* seq_len, int32_t blk_begin, int32_t blk_end,
                          void* summaries, hipStream_t stream);

/*
 * Append one token per request to a growing context: for every KV head, the
 * new key row goes into row t of the K tile and the new value into column t
 * of the V tile of block b, where b = pos[r] / B and t = pos[r] % B.  A token
 * that completes its block (t == B - 1) also rebuilds that block's summary
 * rows (coordinate-wise min and max of its B keys, exactly as
 * oasis_build_summaries) when `summaries` is not NULL.  [v2] §3.2.1 (newly
 * generated blocks join each KV head's working set) and Fig. 6 (per-block
 * min/max key summaries kept in HBM); [reader] paragraph on compressed-key
 * updates.  The context's other tokens must already be in the tiles.
 *   s          shape; uses batch, n_kv_heads, head_dim, block_size, dtype,
 *              tile_stride
 *   k_new, v_new  [R][H][D] (dtype) the new token's key and value per KV head
 *   pos        [R] int32 token position (< n_blk_max*B), or -1 to skip
 *   k_tiles, v_tiles  the tile stores (as oasis_sparse_attn: K tiles [B][D],
 *              V tiles [D][B]), tile (u*n_blk_max + b) for unit u; device
 *              memory or mapped pinned host memory
 *   summaries  [R][H][n_blk_max][2][D] (dtype) or NULL
 * Errors: EINVAL, EUNSUPPORTED, EHIP.
 */
int oasis_append_kv(const oasis_shape* s, const void* k_new, const void* v_new,
                    const int32_t* pos, void* k_tiles, void* v_tiles, int32_t n_blk_max,
                    void* summaries, hipStream_t stream);

/*
 * Workspaces.  When a unit's work is split over several workgroups (small
 * batches, long contexts), the partial results (block scores, attention
 * partials) go through a caller-owned scratch buffer and a second, small
 * launch merges them.  The *_workspace() queries give its size for a shape;
 * 0 means none is needed (or the shape is invalid, which the call reports).
 * A size covers every attention path the call may take for the shape (MFMA or
 * VALU, with or without an appended token): units of more than 16 query rows
 * (two rows of a GQA group above 8) run one attention item per query row on the
 * MFMA path, which splits them differently.  The content need not be
 * initialised.  One workspace serves one call at a
 * time: calls that may overlap in time (other streams) need their own.
 *
 * Workspace bytes oasis_score_topk needs.
 */
size_t oasis_score_topk_workspace(const oasis_shape* s, int32_t n_blk_max, int32_t top_k,
                                  const oasis_step_opts* opts);

/*
 * Score every full block with every stacked query row and keep the top-K per
 * (request, row, KV head).
 * Score: s[r][j][g][b] = sum over the query heads h of group g and over d of
 *   max(q[r][j][h][d] * max_b[d], q[r][j][h][d] * min_b[d])
 * which is [v2] §3.1 equation s_b(alpha) at alpha = 1 (c = (max+min)/2,
 * r = (max-min)/2), i.e. an upper bound of sum_h q_h . k for every key k of
 * the block.  Computed in fp32 as P_g . max_b + N_g . min_b with
 * P_g = sum_h max(q_h, 0), N_g = sum_h min(q_h, 0), so the scan cost does not
 * grow with the group size.  No 1/sqrt(D) factor.
 * Top-K: the min(K, n_r) full blocks with the largest fp32 score, ranked by
 * (score descending, block ascending); positions past n_r hold block -1 and
 * score -inf.  [v2] §3.3.1 (prediction ranks the compressed keys into the
 * per-head set); [reader] paragraph on ranking all logical blocks
 * independently for every KV head.
 *   q           [R][n_q][Hq][D] (dtype)
 *   summaries   [R][H][n_blk_max][2][D] (dtype)
 *   n_blk       [R] int32 full-block counts (0..n_blk_max), or NULL = n_blk_max
 *   top_k       K, 1..1024
 *   topk_idx    [R][n_s][H][K] int32 output
 *   topk_score  [R][n_s][H][K] fp32 output, or NULL
 *   scores      [R][n_s][H][n_blk_max] fp32 output of every block score
 *               (-inf past n_r), or NULL (then the workspace holds them)
 *   opts        scoring variants (alpha, draft averaging) and scan tuning, or
 *               NULL (see oasis_step_opts)
 *   workspace   device buffer of at least oasis_score_topk_workspace() bytes
 *               (NULL when that is 0; see Workspaces above)
 * Limits: n_blk_max <= 32768.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int oasis_score_topk(const oasis_shape* s, const void* q, const void* summaries,
                     int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                     int32_t* topk_idx, float* topk_score, float* scores,
                     const oasis_step_opts* opts, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Capped least-recently-selected selection and transfer plan, per unit:
 *   P       = the ranked blocks of top-K row `pred_row` (entries >= 0)
 *   seeding = some slot is empty (block -1) on entry; then no cap applies
 *   hit     : a slot whose block is in P gets stamp `step`
 *   missing = P's blocks that are not resident, in P's rank order
 *   victims = slots whose block is not in P (empty slots included), ordered
 *             by (stamp ascending, slot ascending)
 *   n       = min(|missing|, |victims|, seeding ? unbounded : cap)
 *   pair i < n: plan_src[i] = missing[i], plan_dst[i] = victims[i],
 *             plan_evicted[i] = the slot's old block; the slot then holds
 *             missing[i] with stamp `step`.  Entries i >= n are -1.
 * Every other slot keeps its block and stamp.  [reader] paragraphs on the
 * capped eviction policy and on partial transfer at admission; [v2] §3.3.2
 * (at most f_HBM*K admissions per head per step once the first working set
 * is seeded; exactly K resident blocks per head).
 * Newly completed block (ins_blk[r] >= 0): after the admissions, the block
 * that request r's last token completed joins every KV head's set outside
 * the cap ([v2] §3.2.1: newly generated blocks replace existing entries
 * independently per KV head).  If resident, its slot's stamp becomes `step`;
 * otherwise it takes the slot with the smallest (stamp, slot) and is plan
 * entry n (count n + 1), or, when that slot was admitted by this very plan,
 * that entry's source becomes the new block (count unchanged).
 *   topk_idx         [R][n_q][H][K] int32 (distinct entries per row; -1 pad)
 *   slot_block_in    [R][H][K] int32 resident block per slot (-1 = empty)
 *   slot_stamp_in    [R][H][K] int32 last step the slot's block was selected
 *   slot_block_out, slot_stamp_out  [R][H][K] outputs; may alias the inputs
 *   ins_blk          [R] int32 block each request just completed (-1 none),
 *                    or NULL for none; a block id the top-K rows never hold
 *   plan_count       [R][H] int32 output
 *   plan_src, plan_dst [R][H][K] int32 outputs
 *   plan_evicted     [R][H][K] int32 output or NULL
 * Integer-only and deterministic; no atomics.
 * Errors: EINVAL (pred_row outside [0, n_q), cap < 0, K outside 1..1024,
 *         null pointers), EHIP.
 */
int oasis_select_plan(int32_t batch, int32_t n_kv_heads, int32_t n_q, int32_t pred_row,
                      int32_t top_k, const int32_t* topk_idx, const int32_t* slot_block_in,
                      const int32_t* slot_stamp_in, int32_t* slot_block_out,
                      int32_t* slot_stamp_out, int32_t step, int32_t cap,
                      const int32_t* ins_blk, int32_t* plan_count, int32_t* plan_src,
                      int32_t* plan_dst, int32_t* plan_evicted, hipStream_t stream);

/*
 * Gather planned block-head tiles into the resident store: for every unit u
 * and i < plan_count[u], copy K tile src_k[u][plan_src[u][i]] to
 * res_k[u][plan_dst[u][i]] and the same for V (B*D*elem bytes each, layout
 * preserved).  [v2] §3.2.1 (a gather kernel on the GPU reads the selected
 * per-head entries from pinned host memory over PCIe and writes them into
 * HBM) and §4.1 Implementation.  Run it on a background stream ordered after
 * the attention that last read the destination slots.
 *   src_k, src_v  [R][H][n_blk_max] tiles (tile_stride apart); device memory or
 *                 pinned host memory the GPU can address (hipHostMalloc / pinned
 *                 torch)
 *   res_k, res_v  [R][H][top_k] tiles in device memory, same tile_stride
 *   plan_*        as written by oasis_select_plan (device memory)
 * Errors: EINVAL, EUNSUPPORTED, EHIP.
 */
int oasis_copy_blocks(const oasis_shape* s, const void* src_k, const void* src_v,
                      int32_t n_blk_max, void* res_k, void* res_v, int32_t top_k,
                      const int32_t* plan_count, const int32_t* plan_src,
                      const int32_t* plan_dst, hipStream_t stream);

/*
 * Decode-host block cache (the one stateful object of this library; created
 * and destroyed by the caller, one per layer).  [v2] §3.2.1 (ii) (the decode
 * host fetches whole blocks, every KV head's entries, for the union of the
 * heads' selections), §3.2.2 (union block mapping: remote block -> decode-host
 * block, per request) and §3.2.3 (per-request budget f_Host*P + F blocks; least
 * recently used prompt blocks are evicted while generated blocks and the
 * current working set are kept; evicted blocks are fetched again when
 * selected).  Policy: a request's union is its planned source blocks in
 * (head, entry) order, each once; an absent block takes the lowest free slot,
 * else evicts the slot with the smallest (last use, slot) among blocks that are
 * not generated, not in the request's HBM working set and not in the union.
 * Memory (caller-owned, alive until destroy):
 *   remote    [R][n_blk][block_bytes] whole blocks: H interleaved K|V records
 *             (read by the host; pinned pages the host has never touched
 *             fault on first read, so fill it from the host)
 *   cache     [R][cap_max][block_bytes] pinned host memory (the GPU reads it);
 *             create zeroes it, which also maps every page for the host
 *   map       [R][n_blk] int32 pinned host memory: cache slot of each remote
 *             block, -1 if absent (written by the tier, read by the gather)
 *   capacity  [R] slots per request (<= cap_max)
 * Returns NULL on a bad argument.  Calls on one tier must not overlap (a
 * stream-ordered fetch counts as a call until its stream has passed it).
 */
typedef struct oasis_host_tier oasis_host_tier;
oasis_host_tier* oasis_host_tier_create(int32_t batch, int32_t n_kv_heads, int32_t top_k,
                                        int32_t n_blk, const int32_t* capacity, int32_t cap_max,
                                        size_t block_bytes, const void* remote, void* cache,
                                        int32_t* map);
void oasis_host_tier_destroy(oasis_host_tier* t);

/* Split each fetch's requests over n_workers host threads (1..64; 1, the
 * default, runs on the calling thread).  Requests own disjoint state, so the
 * result does not depend on n_workers.  [v2] §3.2.1 (ii) (remote fetch is CPU
 * gather, transfer and scatter of whole blocks).  Errors: EINVAL, EHIP (a
 * thread could not be started; the tier is left with one worker). */
int oasis_host_tier_set_workers(oasis_host_tier* t, int32_t n_workers);

/* One layer-step on the CPU, now: fetch the absent blocks of every request's
 * union of plan_src[r][g][i < plan_count[r][g]] (host arrays, [R][H] and
 * [R][H][K]) and stamp the union with `step`; slot_block [R][H][K] (host, or
 * NULL) is the HBM working set after the plan.  EINVAL if a request's budget
 * held no evictable block (its blocks that did not fit are counted as failed). */
int oasis_host_tier_fetch(oasis_host_tier* t, int64_t step, const int32_t* plan_count,
                          const int32_t* plan_src, const int32_t* slot_block);

/*
 * One layer-step's remote fetch and local gather, asynchronously (the
 * remote-fetch and local-fetch stages of the per-layer prefetch pipeline,
 * [v2] §3.3 and Fig. 8).  Queues a job for the tier's dispatcher thread and
 * returns.  The dispatcher takes jobs in order: it waits on the host for
 * `after` (recorded by the caller after the step that wrote the plan and last
 * read the slots), copies plan_count / plan_src / slot_block back, fetches as
 * oasis_host_tier_fetch (stamped with the tier's own step counter), launches
 * oasis_copy_blocks_mapped(s, cache_k, cache_v, cap_max, map, ...) on
 * copy_stream and records `done` on copy_stream after it.  No GPU queue waits
 * on host memory.
 *   s            shape of the resident store (batch = R, n_kv_heads = H; one
 *                block is H records of tile_stride elements = block_bytes)
 *   cache_k/_v   the cache's K and V tiles (pinned host memory)
 *   res_k/_v     resident slots [R][H][top_k] (device memory)
 *   plan_*       as written by oasis_select_plan; slot_block [R][H][top_k] is
 *                the slot table after the plan (device memory)
 *   after, done  caller events; `done` must not be waited on before
 *                oasis_host_tier_wait_issued has returned for this job
 * The plan, slot table and `after` must stay unchanged until `done` is
 * issued.  Host calls that change the tier (fetch, add_generated, trim,
 * set_workers) or read it (state) first wait until every submitted job is
 * issued; before one that changes the cache, the caller also waits for the
 * `done` of the gathers still reading it.
 * Errors: EINVAL, EUNSUPPORTED, EHIP (setting up the dispatcher); errors of
 * a dispatched job are returned by oasis_host_tier_wait_issued.
 */
int oasis_host_tier_submit(oasis_host_tier* t, const oasis_shape* s, const void* cache_k,
                           const void* cache_v, void* res_k, void* res_v,
                           const int32_t* plan_count, const int32_t* plan_src,
                           const int32_t* plan_dst, const int32_t* slot_block, hipEvent_t after,
                           hipStream_t copy_stream, hipEvent_t done);

/* Host wait until every submitted job has been issued (its `done` recorded).
 * Returns OASIS_OK or the first error of a dispatched job (sticky): EHIP for a
 * failed copy-back or launch, EINVAL when a fetch found a request's budget
 * without an evictable block (as oasis_host_tier_fetch; the gather still ran
 * and `done` was recorded, but the planned slots of the blocks that did not
 * fit hold stale tiles, so the caller must treat the step as failed). */
int oasis_host_tier_wait_issued(oasis_host_tier* t);

/* A block generated on the decode node (already written to the cache slot
 * this returns through the map) joins request `req`'s cache, never evicted. */
int oasis_host_tier_add_generated(oasis_host_tier* t, int32_t req, int32_t block, int64_t step,
                                  const int32_t* slot_block);

/* Periodic pass: evict, by the same order, until request r holds at most
 * target[r] blocks (protected blocks stay, so fewer may go). */
int oasis_host_tier_trim(oasis_host_tier* t, const int32_t* target, const int32_t* slot_block);

/* Snapshot: slot_block_out [R][cap_max] (block per slot, -1 free) and
 * last_out [R][cap_max] (either may be NULL); stats_out[5] = blocks fetched,
 * blocks evicted, blocks that found no slot, stream-ordered steps run, host
 * nanoseconds spent inside fetches. */
int oasis_host_tier_state(const oasis_host_tier* t, int32_t* slot_block_out, int64_t* last_out,
                          int64_t* stats_out);

/*
 * oasis_copy_blocks reading its sources through the decode-host cache: the
 * tile of unit u = (r, g) for block b is record g of cache slot map[r][b]
 * (entries whose block is absent are skipped).  cache_k, cache_v: the cache's
 * K and V tiles (v = k + B*D with tile_stride 2*B*D); map as above; res_*,
 * top_k and plan_* as oasis_copy_blocks.  [v2] §3.2.2 (the gather copies each
 * head's slice of the mapped decode-host block into the GPU page).
 * Errors: EINVAL, EUNSUPPORTED, EHIP.
 */
int oasis_copy_blocks_mapped(const oasis_shape* s, const void* cache_k, const void* cache_v,
                             int32_t cap_max, const int32_t* map, int32_t n_blk, void* res_k,
                             void* res_v, int32_t top_k, const int32_t* plan_count,
                             const int32_t* plan_src, const int32_t* plan_dst, hipStream_t stream);

/* Workspace bytes oasis_sparse_attn needs for this shape (see Workspaces above). */
size_t oasis_sparse_attn_workspace(const oasis_shape* s, int32_t n_sel);

/*
 * Paged GQA decode attention of all stacked query rows over each unit's
 * selected tiles plus its active local block, in one call.
 * Tokens of unit u: the B tokens of tile u*unit_stride + tile_table[u][s] for
 * every s < n_sel with entry >= 0, plus the first tail_len[r] tokens of tile
 * u*unit_stride + tail_tile[u] when both arrays are given and the entry >= 0.
 *   z_i = scale * q[r][j][h] . k_i   (g = h / G)
 *   out[r][j][h] = sum_i exp(z_i - m) v_i / sum_i exp(z_i - m),  m = max z
 *   lse[r][j][h] = m + log(sum_i exp(z_i - m))
 * A unit with no tokens gets out = 0 and lse = -inf.  Both rows attend the
 * same tile set.  [v2] §3.1 and Fig. 6 (one attention call over one resident
 * working set returns the outputs of the normal and the draft query) and
 * §4.1 (each head also attends its active local block: K + 1 blocks).
 *   q           [R][n_q][Hq][D] (dtype)
 *   k_tiles     tile store, K tiles [B][D];  v_tiles  V tiles [D][B]
 *   tile_table  [R][H][n_sel] int32 unit-local tile indices, -1 = skip
 *               (entries outside [0, unit_stride) are skipped too)
 *   unit_stride tiles per unit in the store: K for a resident set of K slots
 *               per head, n_blk_max when the full cache is the store
 *   tail_tile   [R][H] int32 unit-local tile index of the active block, or NULL
 *   tail_len    [R] int32 valid tokens of the active block (0..B), or NULL
 *   scale       softmax scale; <= 0 means 1/sqrt(D)
 *   out         [R][n_q][Hq][D] (dtype); bf16 rounds to nearest even
 *   lse         [R][n_q][Hq] fp32, or NULL
 *   workspace   at least oasis_sparse_attn_workspace() bytes (NULL if 0)
 * Limits: n_q * G <= 32.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int oasis_sparse_attn(const oasis_shape* s, const void* q, const void* k_tiles,
                      const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                      int64_t unit_stride, const int32_t* tail_tile, const int32_t* tail_len,
                      float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * oasis_sparse_attn with an explicit choice of split kernel, for measuring one
 * against the other: impl 0 = automatic (MFMA for bf16 with B a multiple of
 * 16, VALU otherwise), 1 = VALU kernel (any dtype and B), 2 = MFMA kernel
 * (EUNSUPPORTED unless bf16 and B % 16 == 0).  Results of 1 and 2 agree
 * within the bf16 tolerance; the MFMA kernel rounds softmax weights to bf16.
 */
int oasis_sparse_attn_impl(const oasis_shape* s, const void* q, const void* k_tiles,
                           const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                           int64_t unit_stride, const int32_t* tail_tile,
                           const int32_t* tail_len, float scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, int32_t impl,
                           hipStream_t stream);

/* Workspace bytes of oasis_lookahead_step (see Workspaces above). */
size_t oasis_lookahead_step_workspace(const oasis_shape* s, int32_t n_blk_max, int32_t top_k,
                                      int32_t n_sel, const oasis_step_opts* opts);

/*
 * One layer of one decode step, in a single launch when every unit fits one
 * scan and one attention workgroup (at least 256 units): the attention of both
 * stacked query rows over the current resident working set, and, from the same
 * queries, the summary scan, the per-KV-head top-K of every row and the capped
 * least-recently-selected plan that makes the next step's working set.
 * [v2] §3.1 and Fig. 6 (the normal and draft queries share one attention call
 * over the resident set; the draft query ranks the summaries to predict the
 * next per-head set) and §3.3.1 (prediction and selection of step t+1 run
 * while step t decodes); the two halves have no data dependence within a step.
 *
 * Results equal, bit for bit on the integer outputs,
 *   oasis_sparse_attn(q, k_tiles, v_tiles, tile_table, n_sel, unit_stride,
 *                     tail_tile, tail_len, scale, out, lse)
 *   oasis_score_topk(q, summaries, n_blk_max, n_blk, top_k,
 *                    topk_idx, topk_score, scores, opts)
 *   oasis_select_plan(R, H, n_s, pred_row, top_k, topk_idx, slot_block_in,
 *                     slot_stamp_in, slot_block_out, slot_stamp_out, step,
 *                     cap, ins_blk, plan_count, plan_src, plan_dst, plan_evicted)
 * run in that order (arguments as documented there; the resident set holds
 * K = top_k slots per KV head).  In the full-cache layout (unit_stride =
 * n_blk_max) the caller passes slot_block_in as tile_table; the plan's outputs
 * must then go to other buffers (double-buffer the slot tables), because the
 * attention still reads the old table while the plan writes the new one:
 * slot_block_out / slot_stamp_out overlapping tile_table is EINVAL.
 *   opts       tuning, or NULL
 *   workspace  at least oasis_lookahead_step_workspace() bytes (NULL if 0)
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP.
 */
int oasis_lookahead_step(const oasis_shape* s, const void* q, const void* summaries,
                         int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                         int32_t* topk_idx, float* topk_score, float* scores,
                         const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                         int32_t* slot_block_out, int32_t* slot_stamp_out, int32_t step,
                         int32_t cap, int32_t pred_row, const int32_t* ins_blk,
                         int32_t* plan_count, int32_t* plan_src,
                         int32_t* plan_dst, int32_t* plan_evicted, const void* k_tiles,
                         const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                         int64_t unit_stride, const int32_t* tail_tile, const int32_t* tail_len,
                         float scale, void* out, float* lse, const oasis_step_opts* opts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * oasis_lookahead_step with the decode step's new token appended in the same
 * launch (a growing context, [v2] §3.2.1 (i): each generated token's KV joins
 * its active block, and a block it fills becomes a summarised, selectable
 * block).  Results equal
 *   oasis_append_kv(s, k_new, v_new, pos, k_tiles, v_tiles, n_blk_max, summaries)
 *   oasis_lookahead_step(..., unit_stride = n_blk_max, tail_tile[r][g] = pos[r] / B,
 *                        tail_len[r] = pos[r] % B + 1, ...)
 * (no active block for a request with pos[r] < 0): the stores, summaries and
 * integer outputs bit for bit, attention up to rounding (the new token joins
 * each row's softmax after the resident tiles and the stored part of the
 * active block, read from k_new / v_new).
 *   k_new, v_new  [R][H][D] the token's key and value (dtype), 16-byte aligned
 *   pos           [R] int32 its position, < 0 = none
 *   k_tiles, v_tiles, summaries  the full cache (written: the token's row and
 *                 column, the summary of a block the token completes)
 *   unit_stride   must equal n_blk_max (EINVAL otherwise)
 *   n_blk         must not count the active block (n_blk[r] <= pos[r] / B); the
 *                 plan's ins_blk is the caller's, as in oasis_lookahead_step
 * Other arguments as oasis_lookahead_step.  Errors: EINVAL, EUNSUPPORTED,
 * EWORKSPACE, EHIP.
 */
int oasis_lookahead_step_append(const oasis_shape* s, const void* q, void* summaries,
                                int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                                int32_t* topk_idx, float* topk_score, float* scores,
                                const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                                int32_t* slot_block_out, int32_t* slot_stamp_out, int32_t step,
                                int32_t cap, int32_t pred_row, const int32_t* ins_blk,
                                int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst,
                                int32_t* plan_evicted, void* k_tiles, void* v_tiles,
                                const int32_t* tile_table, int32_t n_sel, int64_t unit_stride,
                                const void* k_new, const void* v_new, const int32_t* pos,
                                float scale, void* out, float* lse, const oasis_step_opts* opts,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the per-GPU scratch array behind oasis_lookahead_step_noalloc. */
#define OASIS_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * oasis_lookahead_step for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not call hipMalloc,
 * harnesses that forbid allocation): the same arguments, results and errors
 * without workspace / workspace_bytes.  The scratch of split units lives in a
 * library-owned device array of OASIS_NOALLOC_SCRATCH_BYTES per GPU (16 MiB,
 * held by every GPU the library runs on until the process ends); its device
 * address is looked up once per device, on the first call with that device
 * current.  The call allocates nothing.  The caller still passes every input
 * and output.
 *   EWORKSPACE  the shape needs more scratch than the array holds, i.e.
 *               oasis_lookahead_step_workspace() > OASIS_NOALLOC_SCRATCH_BYTES
 *               (checked on the host before any launch)
 *   EINVAL      as oasis_lookahead_step, or `stream` belongs to a device other
 *               than the current one while the shape needs scratch
 *   EHIP        the scratch address could not be looked up, or a launch failed
 * Every call on one GPU uses the same array and leaves its contents there (no
 * call needs it zeroed): calls that may overlap in time on one GPU (several
 * streams or host threads) race on it and must be serialised by the caller.
 */
int oasis_lookahead_step_noalloc(const oasis_shape* s, const void* q, const void* summaries,
                                 int32_t n_blk_max, const int32_t* n_blk, int32_t top_k,
                                 int32_t* topk_idx, float* topk_score, float* scores,
                                 const int32_t* slot_block_in, const int32_t* slot_stamp_in,
                                 int32_t* slot_block_out, int32_t* slot_stamp_out, int32_t step,
                                 int32_t cap, int32_t pred_row, const int32_t* ins_blk,
                                 int32_t* plan_count, int32_t* plan_src, int32_t* plan_dst,
                                 int32_t* plan_evicted, const void* k_tiles, const void* v_tiles,
                                 const int32_t* tile_table, int32_t n_sel, int64_t unit_stride,
                                 const int32_t* tail_tile, const int32_t* tail_len, float scale,
                                 void* out, float* lse, const oasis_step_opts* opts,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* OASIS_H */
