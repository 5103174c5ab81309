// Device code of the per-layer lookahead step, shared by the fused step kernel
// and by the standalone score/top-K and attention entry points.
//
// Sources (web pages about "OasisKV: Scaling In-Decode KV Cache Beyond HBM with
// Lookahead Sparse Prefetching"):
//  - summary scan: paperpeel v2 text, §3.1, equation s_b(alpha) at alpha = 1,
//    summed over the query heads that share one KV head (selection is per KV
//    head: signal-papers reader text, paragraph on ranking non-resident
//    blocks);
//  - top-K: v2 §3.3.1 (the prediction stage ranks the compressed keys into the
//    per-head block set);
//  - plan: reader text, paragraphs on the capped eviction policy and on
//    partial transfer at admission; v2 §3.3.2 (cap applies once the first
//    working set is seeded; exactly K blocks stay resident per head);
//  - attention: v2 §3.1 and Fig. 6 (one attention call over one resident
//    working set returns the outputs of both stacked queries), §4.1 (each head
//    also attends its active local block).
//
// Work decomposition.  A unit is one (request r, KV head g) pair, u = r*H + g.
// The main launch is a 1-D grid of 256-thread workgroups (the second launch of
// split units uses 1,024 threads when the score rows fit in registers).
// Consecutive workgroup ids
// go round robin over the 8 XCDs, so id w runs on XCD w % 8; every item of
// unit u gets an id on XCD u % 8, which keeps a unit's partial results in one
// L2.  Per XCD, scan items come first.
//  - scan item (u, c): scores of blocks [c*chunk, (c+1)*chunk) for every
//    stacked row.  When one item covers the whole unit (NC = 1) its scores
//    stay in LDS and the same workgroup selects the top-K of every row and, in
//    the fused step, builds the plan.  Otherwise the scores go to global
//    memory and a second, small launch (finish_kernel) selects and plans.
//  - attention item (u, s): online softmax over split s of the unit's tile
//    table (the last split also takes the active block).  With one split the
//    item writes the outputs; with S > 1 it writes a partial (max, sum, acc)
//    that finish_kernel merges (in an order fixed by S).
// Workgroups of one launch never exchange data: on this multi-XCD part every
// device-scope release writes back a whole L2, which costs more than a second
// launch, so the kernel boundary is the only synchronisation.
#pragma once

#include "oasis_internal.h"

namespace oasis {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 256;        // threads of every step workgroup
constexpr int kMaxTopK = 1024;  // largest K (resident slots per KV head)
constexpr int kMaxRows = 32;    // n_q * G rows one attention item handles
constexpr int kScanUnroll = 8;  // block passes in flight per scan thread
constexpr int kTopkKPT = 16;    // top-K keys per thread held in registers
constexpr int kFinishKPT = 32;  // the same in the selection launch, rows over kSelRowMax blocks
constexpr int kTopkGroup = 8;   // keys re-read per group beyond the register-held ones
constexpr int kStageVec = 8;    // 16-byte score loads in flight per thread when staging
constexpr int kMaxSplitEntries = 1024;  // tile-table entries of one attention item
constexpr int kSummRows = 16;   // stored rows of a completed block staged for its summary
constexpr size_t kScoreLdsMax = 65536;  // scores of a whole unit kept in LDS up to this size

enum { kAttnNone = 0, kAttnMfma = 1, kAttnValu = 2 };

struct StepArgs {
    // shape
    int R, NQ, Hq, H, G, NR, D, B, U;
    int NS;            // scored rows (NQ, or 2 when three query rows average their drafts)
    const uint8_t* q;  // [R][NQ][Hq][D]
    // scan + top-K
    const uint8_t* summ;  // [R][H][n_blk_max][2][D]
    int n_blk_max;
    const int32_t* n_blk;  // [R] or null
    int K;
    int32_t* topk_idx;   // [R][NS][H][K]
    float* topk_score;   // [R][NS][H][K] or null
    float* scores;       // [R][NS][H][n_blk_max] global scores, or null (NC = 1 only)
    int NC, chunk;       // scan items per unit, blocks per item
    int scores_lds;      // NC = 1 and the unit's scores fit in LDS
    // plan
    int do_plan, pred_row, step, cap;
    const int32_t* ins_blk;  // [R] newly completed block per request (-1 none) or null
    int draft_avg;           // q rows: normal, draft a, draft b; scored: row 0, mean of 1 and 2
    int use_alpha;           // score s_b(alpha) instead of the exact bound (alpha = 1)
    float alpha;
    const int32_t* slot_blk_in;
    const int32_t* slot_stamp_in;
    int32_t* slot_blk_out;
    int32_t* slot_stamp_out;
    int32_t* plan_count;
    int32_t* plan_src;
    int32_t* plan_dst;
    int32_t* plan_evicted;
    // attention
    const uint8_t* kt;  // K tiles [.][B][D]
    const uint8_t* vt;  // V tiles [.][D][B]
    const int32_t* table;  // [U][n_sel]
    int n_sel;
    long long unit_stride;
    long long tile_stride;  // elements between consecutive tiles of the K / V stores
    const int32_t* tail_tile;  // [U] or null
    const int32_t* tail_len;   // [R] or null
    float scale_log2;
    void* out;   // [R][NQ][Hq][D]
    float* lse;  // [R][NQ][Hq] or null
    int S, per_split;
    int RGN;          // row groups per unit: 1, or NQ (one per query row, G rows each)
    float* part_ml;   // [RGN][U][S][rows][2]
    float* part_acc;  // [RGN][U][S][rows][D]
    // roles enabled in this launch: items per unit (0 = role off)
    int scan_items, attn_items;
    // new token per request (launches instantiated with TOK only): its K row
    // and V column land in tile pos/B (a full-cache store), it is attended
    // from these inputs, and a block it completes gets its summary
    const uint8_t* k_new;  // [R][H][D]
    const uint8_t* v_new;  // [R][H][D]
    const int32_t* pos;    // [R], < 0 = none
    uint8_t* kt_w;         // writable views of kt, vt and summ
    uint8_t* vt_w;
    uint8_t* summ_w;
};

// ------------------------------------------------------------ utilities
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for the
// wave's outstanding global stores, which under a full HBM read stream cost
// microseconds; the select / plan code exchanges data through LDS only and
// leaves its global stores in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-wide inclusive scans over the 64 lanes by DPP: row shifts by 1, 2, 4
// and 8 lanes scan each row of 16, then the row broadcasts of lanes 15 and 31
// carry the row totals into the following rows.  Lanes without a source keep
// the identity.  One VALU op per step, no LDS round trip.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t ident, Op op) {
    const int id = (int)ident;
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
    return v;
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    return wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// Minimum / maximum over the wave, the same in every lane.
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    v = wave_incl_scan(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive prefix sums over the workgroup of N values per thread.
template <int N, int NT = kNT>
__device__ __forceinline__ void block_scan(const uint32_t (&v)[N], uint32_t (&excl)[N],
                                           uint32_t (&total)[N], uint32_t* buf /*[NT / 64][N]*/) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) inc[i] = wave_incl_sum(v[i]);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i) buf[w * N + i] = inc[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t base = 0, tot = 0;
#pragma unroll
        for (int ww = 0; ww < NT / 64; ++ww) {
            const uint32_t x = buf[ww * N + i];
            base += ww < w ? x : 0u;
            tot += x;
        }
        excl[i] = inc[i] - v[i] + base;
        total[i] = tot;
    }
    lds_barrier();
}

// ------------------------------------------------------------ LDS carving
struct LdsCursor {
    unsigned char* p;
    template <typename T>
    __device__ __forceinline__ T* take(size_t n) {
        T* r = reinterpret_cast<T*>(p);
        p += (n * sizeof(T) + 15) & ~size_t(15);
        return r;
    }
};

__host__ __device__ inline int pad4(int k) { return (k + 3) & ~3; }

// LDS bytes carve_plan takes.
__host__ __device__ inline size_t plan_lds_size(int K) {
    const size_t k4 = (size_t)pad4(K);
    auto a16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    return a16(k4 * 4) * 9 + a16(k4 * 8) + a16(80 * 4) + a16(18 * 8);
}

// LDS bytes of a scan item (P/N rows, top-K, plan, and the unit's scores when
// they stay in LDS), mirrored by the carving in scan_item / finish_kernel.
__host__ __device__ inline size_t scan_lds_bytes(int NQ, int D, int K, int n_scores) {
    auto a16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    const size_t kp = (size_t)pad4(K);
    size_t b = a16(NQ * 2 * D * 4);                                     // pn
    b += a16(NQ * 512 * 4) + a16(4 * 2 * 4) + a16(16 * 4);             // hist, scan, sh
    b += a16(NQ * kp * 4) * 2 + a16(kp * 4);                            // sel key/idx, P
    b += plan_lds_size(K);                                              // plan
    b += a16((size_t)n_scores * 4);                                     // scores
    return b;
}

// ============================================================ summary scan
// Scores of blocks [c*chunk, (c+1)*chunk) of unit u for all NQ rows, written to
// dst (row j at dst + j*drs; LDS or global).
// LPR lanes share one block: lane cl owns the 16-byte chunk cl of the min row
// and of the max row.  The loop is software-pipelined: the next UNR blocks of
// every lane group are in flight while the current ones are reduced.
template <int DT, int D, int NQ>
__device__ __forceinline__ void scan_blocks(const StepArgs& a, int u, int c, float* pn, float* dst,
                                            size_t drs) {
    constexpr int EB = Elem<DT>::bytes;
    constexpr int VEC = 16 / EB;
    constexpr int LPR = D / VEC;     // lanes per summary row
    constexpr int BPP = kNT / LPR;   // blocks per workgroup pass
    constexpr int UNR = kScanUnroll;
    const int tid = threadIdx.x;
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int cl = tid % LPR, lb = tid / LPR;
    const int n_r = a.n_blk ? min(max(a.n_blk[r], 0), a.n_blk_max) : a.n_blk_max;
    const int b_begin = c * a.chunk;
    const int b_end = min(b_begin + a.chunk, a.n_blk_max);
    const int v_end = min(b_end, n_r);
    const uint4* base = reinterpret_cast<const uint4*>(a.summ) + (size_t)u * a.n_blk_max * 2 * LPR + cl;
    // Every lane loads on every pass (blocks past the chunk are clamped into
    // the unit's rows and their results discarded), so the number of loads
    // in flight is the same on every path and the prefetch is never drained.
    auto load = [&](int b0, uint4 (&mn)[UNR], uint4 (&mx)[UNR]) {
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int b = min(b0 + k * BPP + lb, b_end - 1);
            mn[k] = load_stream(base + (size_t)b * 2 * LPR);
            mx[k] = load_stream(base + (size_t)b * 2 * LPR + LPR);
        }
    };
    // The first summaries do not depend on q: they are in flight while the
    // group's P/N vectors are formed.
    uint4 mnA[UNR], mxA[UNR], mnB[UNR], mxB[UNR];
    load(b_begin, mnA, mxA);
    // P_g = sum_h max(q_h, 0), N_g = sum_h min(q_h, 0) over the group's heads
    // (scored row j; with draft averaging row 1 is the mean of query rows 1
    // and 2).  s_b(alpha) = P'.max + N'.min with P' = ((1+alpha)P + (1-alpha)N)/2
    // and N' = ((1-alpha)P + (1+alpha)N)/2, the centre/radius form rewritten.
    for (int idx = tid; idx < NQ * D; idx += kNT) {
        const int j = idx / D, d = idx - (idx / D) * D;
        const bool avg = a.draft_avg && j == 1;
        float p = 0.f, n = 0.f;
        for (int h = 0; h < a.G; ++h) {
            const size_t hd = ((size_t)g * a.G + h) * D + d;
            float x = load_elem<DT>(a.q, ((size_t)r * a.NQ + j) * a.Hq * D + hd);
            if (avg) x = 0.5f * (x + load_elem<DT>(a.q, ((size_t)r * a.NQ + 2) * a.Hq * D + hd));
            p += x > 0.f ? x : 0.f;
            n += x < 0.f ? x : 0.f;
        }
        if (a.use_alpha) {
            const float pp = 0.5f * ((1.f + a.alpha) * p + (1.f - a.alpha) * n);
            n = 0.5f * ((1.f - a.alpha) * p + (1.f + a.alpha) * n);
            p = pp;
        }
        pn[(j * 2) * D + d] = p;
        pn[(j * 2 + 1) * D + d] = n;
    }
    lds_barrier();
    float P[NQ][VEC], N[NQ][VEC];
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            P[j][e] = pn[(j * 2) * D + cl * VEC + e];
            N[j][e] = pn[(j * 2 + 1) * D + cl * VEC + e];
        }
    auto process = [&](int b0, const uint4 (&mn)[UNR], const uint4 (&mx)[UNR]) {
        float acc[UNR][NQ];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            float lo[VEC], hi[VEC];
            unpack16<DT>(mn[k], lo);
            unpack16<DT>(mx[k], hi);
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                float sacc = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    sacc = fmaf(P[j][e], hi[e], sacc);
                    sacc = fmaf(N[j][e], lo[e], sacc);
                }
                acc[k][j] = sacc;
            }
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1)
#pragma unroll
            for (int k = 0; k < UNR; ++k)
#pragma unroll
                for (int j = 0; j < NQ; ++j) acc[k][j] += __shfl_xor(acc[k][j], off, 64);
        if (cl == 0) {
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const int b = b0 + k * BPP + lb;
                if (b < b_end) {
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        dst[j * drs + b] = b < v_end ? acc[k][j] : -__builtin_inff();
                }
            }
        }
    };
    // Ping-pong over two register buffers (no copies of in-flight loads).
    constexpr int STEP = BPP * UNR;
    int b0 = b_begin;
    // sched_barrier keeps every load of the next buffer issued before the
    // current buffer's arithmetic (the scheduler would otherwise interleave
    // them and wait on the current buffer with part of the prefetch unsent).
    while (b0 < b_end) {
        load(b0 + STEP, mnB, mxB);  // past the chunk: re-reads its last block
        __builtin_amdgcn_sched_barrier(0);
        process(b0, mnA, mxA);
        b0 += STEP;
        if (b0 >= b_end) break;
        load(b0 + STEP, mnA, mxA);
        __builtin_amdgcn_sched_barrier(0);
        process(b0, mnB, mxB);
        b0 += STEP;
    }
}

// ============================================================ top-K
struct TopkLds {
    int* hist;          // [NQ][2][256] (double-buffered)
    uint32_t* scanbuf;  // [4][2]
    int* sh;            // [NQ][4]
    uint32_t* sel_key;  // [NQ][Kp4]
    int* sel_idx;       // [NQ][Kp4]
    int* P;             // [Kp4] ranked blocks of the plan's row (-1 pad)
    unsigned long long* ek;  // [NQ][Kp4] (key, position) rank keys; GROUPED selections only
};

// Ranked top-K of NQ score rows (row j at sc + j*rs, n valid entries each; LDS
// or global): the min(K, n) largest by (score desc, block asc).  The rows are
// selected concurrently, each by its own group of kNT/NQ threads (whole
// waves) holding up to kTopkKPT consecutive keys each in registers.  Radix
// select on order-preserving uint32 keys: the bits every key of a row shares
// are found first (min / max), then each pass resolves the next 8 bits below
// them through a 256-bin LDS histogram (two buffers, so a pass needs two
// barriers), until the threshold key's bin holds exactly the keys still to
// take.  The threshold ties are compacted in block order and the survivors
// ranked by counting.  Integer work only, so the result is exact for the fp32
// scores given.
// With `padded`, row j of `sc` holds key i at i + i / per (per = keys of one
// thread): a thread's keys then start one bank apart from its neighbour's, so
// the loads of a key by all threads at once are conflict-free.
template <int NQ, int KPT = kTopkKPT, bool GROUPED = false>
__device__ void topk_rows(const float* sc, size_t rs, int n, int K, int32_t* oidx, float* oscore,
                          size_t ors, int pred_row, const TopkLds& L, bool padded = false) {
    constexpr int TPR = kNT / NQ;  // threads per row
    constexpr int WPR = TPR / 64;  // waves per row
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int j = tid / TPR, t = tid - (tid / TPR) * TPR;  // row, thread within row
    const int wr = wv - j * WPR;                           // wave within the row group
    const int Kp = min(K, n);
    const int K4 = pad4(K);
    const float* row = sc + j * rs;
    int32_t* orow = oidx + j * ors;
    float* srow = oscore ? oscore + j * ors : nullptr;
    for (int a = Kp + t; a < K; a += TPR) {
        orow[a] = -1;
        if (srow) srow[a] = -__builtin_inff();
    }
    if (j == pred_row)
        for (int a = Kp + t; a < K4; a += TPR) L.P[a] = -1;
    if (Kp <= 0) {
        lds_barrier();
        return;
    }
    const int per = (n + TPR - 1) / TPR;
    const int i0 = min(t * per, n), i1 = min(i0 + per, n);
    // Where key i of this thread's range sits in the row; with GROUPED,
    // out-of-range keys read entry 0 (always present), so every load is
    // unconditional and all of them are in flight together.
    const int pad = padded ? t : 0;
    auto at = [&](int i) { return i < i1 ? i + pad : 0; };
    uint32_t key[KPT];
    if constexpr (GROUPED) {
        float f[KPT];
#pragma unroll
        for (int e = 0; e < KPT; ++e) f[e] = row[at(i0 + e)];
#pragma unroll
        for (int e = 0; e < KPT; ++e) key[e] = (i0 + e < i1) ? float_key(f[e]) : 0u;
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e) key[e] = (i0 + e < i1) ? float_key(row[i0 + pad + e]) : 0u;
    }
    // Visit this thread's keys in block order; keys beyond the register-held
    // ones are re-read (GROUPED: kTopkGroup loads in flight at a time, for the
    // selection launch; one at a time where registers are scarce).
#define OASIS_FOR_KEYS(BODY)                                                      \
    {                                                                             \
        _Pragma("unroll") for (int e_ = 0; e_ < KPT; ++e_) {                      \
            if (i0 + e_ < i1) {                                                   \
                const uint32_t kk = key[e_];                                      \
                const int ii = i0 + e_;                                           \
                BODY                                                              \
            }                                                                     \
        }                                                                         \
        for (int ib_ = i0 + KPT; GROUPED && ib_ < i1; ib_ += kTopkGroup) {        \
            float f_[kTopkGroup];                                                 \
            _Pragma("unroll") for (int e_ = 0; e_ < kTopkGroup; ++e_)             \
                f_[e_] = row[at(ib_ + e_)];                                       \
            _Pragma("unroll") for (int e_ = 0; e_ < kTopkGroup; ++e_) {           \
                if (ib_ + e_ < i1) {                                              \
                    const uint32_t kk = float_key(f_[e_]);                        \
                    const int ii = ib_ + e_;                                      \
                    BODY                                                          \
                }                                                                 \
            }                                                                     \
        }                                                                         \
        for (int ii = i0 + KPT; !GROUPED && ii < i1; ++ii) {                      \
            const uint32_t kk = float_key(row[ii + pad]);                         \
            BODY                                                                  \
        }                                                                         \
    }

    // Bits shared by every key of a row: min and max over the row group.
    uint32_t lo = 0xffffffffu, hi = 0u;
    OASIS_FOR_KEYS({
        (void)ii;
        lo = kk < lo ? kk : lo;
        hi = kk > hi ? kk : hi;
    })
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
        L.scanbuf[wv * 2] = lo;
        L.scanbuf[wv * 2 + 1] = hi;
    }
    for (int i = tid; i < NQ * 256; i += kNT) L.hist[(i >> 8) * 512 + (i & 255)] = 0;
    lds_barrier();
    // Every thread derives the starting state of every row (to know when all
    // rows are done) and keeps the full state of its own row.
    bool done_all[NQ];
    uint32_t prefix = 0, mask = 0;
    int hb = 0;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
        uint32_t l2 = 0xffffffffu, h2 = 0u;
#pragma unroll
        for (int w = jj * WPR; w < (jj + 1) * WPR; ++w) {
            const uint32_t x = L.scanbuf[w * 2], y = L.scanbuf[w * 2 + 1];
            l2 = x < l2 ? x : l2;
            h2 = y > h2 ? y : h2;
        }
        const int b = l2 == h2 ? 0 : 32 - __clz(l2 ^ h2);  // low bits not shared
        done_all[jj] = b == 0;
        if (jj == j) {
            hb = b;
            mask = b >= 32 ? 0u : (0xffffffffu << b);
            prefix = h2 & mask;
        }
    }
    int remaining = Kp;
    bool done = hb == 0;
    int buf = 0;
    for (;;) {
        bool all = true;
#pragma unroll
        for (int jj = 0; jj < NQ; ++jj) all = all && done_all[jj];
        if (all) break;
        int* hist = L.hist + j * 512 + buf * 256;
        const int w8 = hb < 8 ? hb : 8;
        const int shift = hb - w8;
        const uint32_t dm = (1u << w8) - 1u;
        if (!done) {
            OASIS_FOR_KEYS({
                (void)ii;
                if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & dm], 1);
            })
        }
        lds_barrier();
        if (!done && wr == 0) {
            // Lane l holds digits 255-4l .. 252-4l, so a prefix over lanes is a
            // suffix (largest digits first) over digits.
            int c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = hist[255 - (4 * lane + e)];
            const int local = c[0] + c[1] + c[2] + c[3];
            const int inc = (int)wave_incl_sum((uint32_t)local);
            int before = inc - local;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (before < remaining && before + c[e] >= remaining) {
                    const int rem2 = remaining - before;
                    L.sh[j * 4 + 0] = 255 - (4 * lane + e);
                    L.sh[j * 4 + 1] = before;
                    L.sh[j * 4 + 3] = (c[e] == rem2 || shift == 0) ? 1 : 0;
                }
                before += c[e];
            }
        }
        // The other buffer is cleared for the next pass meanwhile.
        for (int i = tid; i < NQ * 256; i += kNT)
            L.hist[(i >> 8) * 512 + (buf ^ 1) * 256 + (i & 255)] = 0;
        lds_barrier();
        if (!done) {
            prefix |= uint32_t(L.sh[j * 4 + 0]) << shift;
            mask |= dm << shift;
            hb = shift;
            remaining -= L.sh[j * 4 + 1];
            done = L.sh[j * 4 + 3] != 0;
        }
#pragma unroll
        for (int jj = 0; jj < NQ; ++jj)
            if (!done_all[jj]) done_all[jj] = L.sh[jj * 4 + 3] != 0;
        buf ^= 1;
    }
    // Take every key above the threshold prefix and the first `remaining`
    // keys equal to it, in block order: exclusive counts within the row group.
    // GROUPED with every key in registers: bit masks of the keys above / at the
    // threshold, so the take below visits only those keys (few per thread).
    const bool masks = GROUPED && per <= KPT && KPT <= 32;
    uint32_t mgt = 0, meq = 0;
    uint32_t gt = 0, eq = 0;
    if (masks) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const uint32_t mk = key[e] & mask;
            const bool in = i0 + e < i1;
            mgt |= uint32_t(in && mk > prefix) << e;
            meq |= uint32_t(in && mk == prefix) << e;
        }
        gt = __builtin_popcount(mgt);
        eq = __builtin_popcount(meq);
    } else {
        OASIS_FOR_KEYS({
            (void)ii;
            const uint32_t mk = kk & mask;
            gt += mk > prefix;
            eq += mk == prefix;
        })
    }
    uint32_t ig = wave_incl_sum(gt), ie = wave_incl_sum(eq);
    if (lane == 63) {
        L.scanbuf[wv * 2] = ig;
        L.scanbuf[wv * 2 + 1] = ie;
    }
    lds_barrier();
    for (int w = j * WPR; w < wv; ++w) {
        ig += L.scanbuf[w * 2];
        ie += L.scanbuf[w * 2 + 1];
    }
    int pos = int(ig - gt) + min(int(ie - eq), remaining);
    int eqb = int(ie - eq);
    uint32_t* skey = L.sel_key + j * K4;
    int* sidx = L.sel_idx + j * K4;
    if (masks) {
        // the threshold ties this thread may take, lowest positions first
        const int take_eq = max(0, min(int(eq), remaining - eqb));
        uint32_t m = mgt;
        uint32_t me = meq;
        for (int q = 0; q < take_eq; ++q) {
            m |= me & (0u - me);  // lowest set bit
            me &= me - 1u;
        }
        while (m) {
            const int e = __builtin_ctz(m);
            m &= m - 1u;
            // the key again from the staged row (a register array is not
            // indexed by a run-time position)
            skey[pos] = float_key(row[i0 + pad + e]);
            sidx[pos] = i0 + e;
            ++pos;
        }
    } else {
        OASIS_FOR_KEYS({
            const uint32_t mk = kk & mask;
            bool take = mk > prefix;
            if (mk == prefix) {
                take = eqb < remaining;
                ++eqb;
            }
            if (take) {
                skey[pos] = kk;
                sidx[pos] = ii;
                ++pos;
            }
        })
    }
#undef OASIS_FOR_KEYS
    for (int a = Kp + t; a < K4; a += TPR) {
        skey[a] = 0u;
        sidx[a] = -1;
    }
    lds_barrier();
    // Counting rank under (key desc, position asc); survivors sit in block order.
    if constexpr (GROUPED) {
        // One 64-bit compare per survivor: the key above the complement of its
        // position (padding 0 sorts last; every real key is above 2^32).
        unsigned long long* ek = L.ek + (size_t)j * K4;
        for (int a = t; a < K4; a += TPR)
            ek[a] = a < Kp ? ((unsigned long long)skey[a] << 32) | (0xffffffffu - (uint32_t)a) : 0ull;
        lds_barrier();
        const ulonglong2* e2 = reinterpret_cast<const ulonglong2*>(ek);
        for (int a = t; a < Kp; a += TPR) {
            const unsigned long long ea = ek[a];
            int rank = 0;
#pragma unroll 8
            for (int i = 0; i < K4 / 2; ++i) {
                const ulonglong2 x = e2[i];
                rank += (x.x > ea) + (x.y > ea);
            }
            const int bi = sidx[a];
            orow[rank] = bi;
            if (srow) srow[rank] = key_float((uint32_t)(ea >> 32));
            if (j == pred_row) L.P[rank] = bi;
        }
        lds_barrier();
        return;
    }
    const uint4* kv = reinterpret_cast<const uint4*>(skey);
    for (int a = t; a < Kp; a += TPR) {
        const uint32_t ka = skey[a];
        int rank = 0;
#pragma unroll 8
        for (int b4 = 0; b4 < K4 / 4; ++b4) {
            const uint4 x = kv[b4];
            const int b = b4 * 4;
            rank += (x.x > ka) + ((x.x == ka) & (b + 0 < a));
            rank += (x.y > ka) + ((x.y == ka) & (b + 1 < a));
            rank += (x.z > ka) + ((x.z == ka) & (b + 2 < a));
            rank += (x.w > ka) + ((x.w == ka) & (b + 3 < a));
        }
        const int bi = sidx[a];
        orow[rank] = bi;
        if (srow) srow[rank] = key_float(ka);
        if (j == pred_row) L.P[rank] = bi;
    }
    lds_barrier();
}

// ------------------------------------------------------------ one long row
// Top-K of one score row of up to kSelRowMax entries in global memory, by one
// workgroup of NT threads (the selection launch of split units; the ranked
// list is the pages' per-head block set, v2 §3.3.1).  Thread t
// holds the keys of blocks t, t + NT, ... in registers, loaded straight from
// memory (coalesced, all in flight).  Each block's key is 64-bit: the
// order-preserving uint32 of its score above the complement of its block
// index (13 bits), so every key is distinct and larger means (higher score,
// then lower block).  Radix passes of 8 bits below the bits every key shares
// narrow the bin of the K-th key until that bin and the bins above hold at
// most `cmax` keys (one pass on score rows of the measured shapes: ~140-170
// keys); those are compacted to LDS and ranked by counting, four adjacent
// lanes per candidate when the workgroup has them.  Integer work only: exact
// for the fp32 scores given, ties by ascending block.
constexpr int kSelIdxBits = 13;
constexpr int kSelRowMax = 1 << kSelIdxBits;  // longest row held in registers
constexpr uint32_t kSelIdxMax = (1u << kSelIdxBits) - 1u;
constexpr int kSelCandMax = kMaxTopK + 128;  // largest candidate list
constexpr int kFinishNT = 1024;              // threads of a selection-launch workgroup

struct SelLds {
    int* hist;                 // [2][256]
    int* pos;                  // [256]: first candidate slot of each digit of the first pass
    uint32_t* red;             // [64]: per wave (min, max) [0, 32), candidate counts [32, 48)
    int* sh;                   // [4]
    unsigned long long* cand;  // [kSelCandMax + 2]
};

__device__ __forceinline__ SelLds carve_sel(LdsCursor& cur) {
    SelLds L;
    L.hist = cur.take<int>(512);
    L.pos = cur.take<int>(256);
    L.red = cur.take<uint32_t>(64);
    L.sh = cur.take<int>(4);
    L.cand = cur.take<unsigned long long>(kSelCandMax + 2);
    return L;
}
__host__ __device__ inline size_t sel_lds_bytes() {
    return 512 * 4 + 256 * 4 + 64 * 4 + 16 + (size_t)(kSelCandMax + 2) * 8 + 64;
}

// Issue the loads of a row's scores (raw bits; no use, so nothing waits yet).
template <int NT>
__device__ __forceinline__ void sel_load(const float* row, int n, uint32_t (&key)[kSelRowMax / NT]) {
    const int last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int q = 0; q < kSelRowMax / NT; ++q)
        key[q] = __float_as_uint(row[min(q * NT + (int)threadIdx.x, last)]);
}

// Ranked top-K of the row whose score bits sel_load put in `key`: block
// indices to orow[0..K) (-1 past n), scores to srow (if any), and the ranked
// blocks to P (LDS, -1 padded to pad4(K); if any) for the plan.
// `hook` runs work of the caller's that needs no selection result inside the
// selection's first LDS phase: before() ahead of its first barrier, after()
// right after it (another barrier follows before the selection returns).
// With P, each ranked block's rank also goes to mark_p[block] (if mark_p).
struct NoHook {
    __device__ void before() const {}
    __device__ void after() const {}
};

template <int NT, class Hook = NoHook>
__device__ __forceinline__ void select_row(uint32_t (&key)[kSelRowMax / NT], int n, int K,
                                           int32_t* orow, float* srow, int* P, const SelLds& L,
                                           const Hook& hook = Hook(), uint16_t* mark_p = nullptr) {
    constexpr int KPT = kSelRowMax / NT;
    constexpr int NW = NT / 64;
    static_assert(KPT * NT == kSelRowMax && NT >= 256, "one index field per held key");
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int Kp = min(K, n);
    for (int a = max(Kp, 0) + t; a < K; a += NT) {
        orow[a] = -1;
        if (srow) srow[a] = -__builtin_inff();
    }
    if (P)
        for (int a = max(Kp, 0) + t; a < pad4(K); a += NT) P[a] = -1;
    if (Kp <= 0) {
        hook.before();
        lds_barrier();
        hook.after();
        lds_barrier();
        return;
    }
    const int nv = n > t ? (n - t + NT - 1) / NT : 0;  // keys q < nv are blocks < n
    const uint32_t low0 = kSelIdxMax - (uint32_t)t;   // index field of key 0
    auto comp = [&](int q) {
        return ((unsigned long long)key[q] << kSelIdxBits) | (unsigned long long)(low0 - NT * q);
    };
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        key[q] = float_key(__uint_as_float(key[q]));
        const bool v = q < nv;
        lo = v && key[q] < lo ? key[q] : lo;
        hi = v && key[q] > hi ? key[q] : hi;
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
        L.red[wv * 2] = lo;
        L.red[wv * 2 + 1] = hi;
    }
    for (int i = t; i < 512; i += NT) L.hist[i] = 0;
    hook.before();
    lds_barrier();
    hook.after();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        lo = L.red[w * 2] < lo ? L.red[w * 2] : lo;
        hi = L.red[w * 2 + 1] > hi ? L.red[w * 2 + 1] : hi;
    }
    const int cmax = min(Kp + 128, kSelCandMax);
    // Bits below hb are not shared by every key (the index field never is).
    int hb = (lo == hi ? 0 : 32 - __clz(lo ^ hi)) + kSelIdxBits;
    unsigned long long mask = ~((1ull << hb) - 1ull);
    unsigned long long prefix = ((unsigned long long)hi << kSelIdxBits) & mask;
    int above = 0, remaining = Kp, cnt = n;
    int npass = 0, d1 = 0, shift1 = 0;  // passes run; the first pass's digit and shift
    if (n <= cmax) {
        prefix = 0ull;  // every block is a candidate
    } else {
        int buf = 0;
        for (;;) {
            const int w8 = hb < 8 ? hb : 8;
            const int shift = hb - w8;
            const uint32_t dm = (1u << w8) - 1u;
            int* hist = L.hist + buf * 256;
            if (shift >= kSelIdxBits) {
                // digits and prefix in the score bits: 32-bit work
                const int ks = shift - kSelIdxBits;
                const uint32_t m32 = (uint32_t)(mask >> kSelIdxBits);
                const uint32_t p32 = (uint32_t)(prefix >> kSelIdxBits);
#pragma unroll
                for (int q = 0; q < KPT; ++q)
                    if (q < nv && (key[q] & m32) == p32) atomicAdd(&hist[(key[q] >> ks) & dm], 1);
            } else {
#pragma unroll
                for (int q = 0; q < KPT; ++q) {
                    const unsigned long long c = comp(q);
                    if (q < nv && (c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> shift) & dm], 1);
                }
            }
            lds_barrier();
            if (wv == 0) {
                // lane l holds digits 255-4l .. 252-4l: a prefix over lanes is
                // a suffix (largest digits first) over digits
                int c[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] = hist[255 - (4 * lane + e)];
                const int local = c[0] + c[1] + c[2] + c[3];
                int before = (int)wave_incl_sum((uint32_t)local) - local;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (before < remaining && before + c[e] >= remaining) {
                        L.sh[0] = 255 - (4 * lane + e);
                        L.sh[1] = before;
                        L.sh[2] = c[e];
                    }
                    if (npass == 0) L.pos[255 - (4 * lane + e)] = before;  // keys of larger digits
                    before += c[e];
                }
            }
            for (int i = t; i < 256; i += NT) L.hist[(buf ^ 1) * 256 + i] = 0;  // next pass's buffer
            lds_barrier();
            const int d = L.sh[0], before = L.sh[1];
            cnt = L.sh[2];
            if (npass == 0) {
                d1 = d;
                shift1 = shift;
            }
            ++npass;
            prefix |= (unsigned long long)d << shift;
            mask |= (unsigned long long)dm << shift;
            hb = shift;
            above += before;
            remaining -= before;
            if (above + cnt <= cmax || hb == 0) break;
            buf ^= 1;
        }
    }
    // Candidates: every key at or above the bin's lower edge.
    const int C = n <= cmax ? n : above + cnt;
    if (npass == 1) {
        // One pass: every key shares the first pass's region, so the candidates
        // are the keys of digits >= d1, and the digit's exclusive suffix count
        // is where its keys start (their order within a digit does not matter:
        // the ranking below orders them).
        // (the first pass always takes 8 bits: hb >= the index field's 13)
#pragma unroll
        for (int q = 0; q < KPT; ++q) {
            const int dg = shift1 >= kSelIdxBits
                               ? (int)((key[q] >> (shift1 - kSelIdxBits)) & 255u)
                               : (int)((uint32_t)(comp(q) >> shift1) & 255u);
            if (q < nv && dg >= d1) L.cand[atomicAdd(&L.pos[dg], 1)] = comp(q);
        }
        if (t == 0) L.cand[C] = 0ull;  // pairs are read two at a time; 0 is below every key
        lds_barrier();
    } else {
        // Otherwise compacted in thread order.
        uint32_t cm = 0;
        if ((prefix & kSelIdxMax) == 0) {  // the edge has no index bits: compare scores only
            const uint32_t p32 = (uint32_t)(prefix >> kSelIdxBits);
#pragma unroll
            for (int q = 0; q < KPT; ++q) cm |= uint32_t(q < nv && key[q] >= p32) << q;
        } else {
#pragma unroll
            for (int q = 0; q < KPT; ++q) cm |= uint32_t(q < nv && comp(q) >= prefix) << q;
        }
        const uint32_t mine = (uint32_t)__builtin_popcount(cm);
        const uint32_t inc = wave_incl_sum(mine);
        if (lane == 63) L.red[32 + wv] = inc;
        lds_barrier();
        uint32_t pos = inc - mine;
#pragma unroll
        for (int w = 0; w < NW; ++w) pos += w < wv ? L.red[32 + w] : 0u;
#pragma unroll
        for (int q = 0; q < KPT; ++q)
            if ((cm >> q) & 1u) L.cand[pos++] = comp(q);
        if (t == 0) L.cand[C] = 0ull;  // pairs are read two at a time; 0 is below every key
        lds_barrier();
    }
    // Counting rank among the candidates.
    const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(L.cand);
    const int C2 = (C + 1) >> 1;
    auto emit = [&](unsigned long long e, int rank) {
        if (rank < Kp) {
            const int bi = (int)(kSelIdxMax - (uint32_t)(e & kSelIdxMax));
            orow[rank] = bi;
            if (srow) srow[rank] = key_float((uint32_t)(e >> kSelIdxBits));
            if (P) {
                P[rank] = bi;
                if (mark_p) mark_p[bi] = (uint16_t)rank;
            }
        }
    };
    if (4 * C <= NT) {
        // lanes 4a .. 4a+3 rank candidate a, each over every fourth pair
        const int a = t >> 2, part = t & 3;
        const unsigned long long e = L.cand[a < C ? a : 0];
        int rank = 0;
        for (int i = part; i < C2; i += 4) {
            const ulonglong2 x = c2[i];
            rank += (x.x > e) + (x.y > e);
        }
        rank += __shfl_xor(rank, 1, 64);
        rank += __shfl_xor(rank, 2, 64);
        if (a < C && part == 0) emit(e, rank);
    } else {
        for (int a = t; a < C; a += NT) {
            const unsigned long long e = L.cand[a];
            int rank = 0;
#pragma unroll 8
            for (int i = 0; i < C2; ++i) {
                const ulonglong2 x = c2[i];
                rank += (x.x > e) + (x.y > e);
            }
            emit(e, rank);
        }
    }
    lds_barrier();
}

// ============================================================ plan
struct PlanLds {
    int* blk;      // [K4]
    int* stamp;    // [K4]
    int* hit;      // [K4]
    int* miss;     // [K4]
    long long* ekey;  // [K4]
    int* missing_of_rank;  // [K4]
    int* victim_of_rank;   // [K4]
    int* new_blk;          // [K4]
    int* new_stamp;        // [K4]
    int* rank_of_slot;     // [K4] victim rank of a slot (K for hits)
    uint32_t* scanbuf;     // [80]: block scans [0, 48), inserted count [48], empty flags [56, 72)
    int* order;            // [K4] slots by (stamp, slot) (plan_order; FAST plans only)
    uint16_t* mark_p;      // [n_blk] rank of a predicted block (FAST plans only; unchecked garbage elsewhere)
    uint16_t* mark_b;      // [n_blk] slot of a resident block (likewise)
    unsigned long long* ins_key;  // [18]: oldest (stamp, slot) key; slot holding the new block;
                                  // [2, 2 + waves) each wave's oldest key
};

__device__ __forceinline__ PlanLds carve_plan(LdsCursor& cur, int K4) {
    PlanLds L;
    L.blk = cur.take<int>(K4);
    L.stamp = cur.take<int>(K4);
    L.hit = cur.take<int>(K4);
    L.miss = cur.take<int>(K4);
    L.ekey = cur.take<long long>(K4);
    L.missing_of_rank = cur.take<int>(K4);
    L.victim_of_rank = cur.take<int>(K4);
    L.new_blk = cur.take<int>(K4);
    L.new_stamp = cur.take<int>(K4);
    L.rank_of_slot = cur.take<int>(K4);
    L.scanbuf = cur.take<uint32_t>(80);
    L.ins_key = cur.take<unsigned long long>(18);
    L.order = nullptr;
    L.mark_p = L.mark_b = nullptr;
    return L;
}

// The FAST plan's extra state: the slot order and the block marks of n_blk blocks.
__device__ __forceinline__ void carve_plan_fast(LdsCursor& cur, int K4, int n_blk, PlanLds& L) {
    L.order = cur.take<int>(K4);
    L.mark_p = cur.take<uint16_t>(n_blk);
    L.mark_b = cur.take<uint16_t>(n_blk);
}
__host__ __device__ inline size_t plan_fast_lds_size(int K, int n_blk) {
    auto a16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    return a16((size_t)pad4(K) * 4) + 2 * a16((size_t)n_blk * 2);
}

// Stage one unit's slot tables in LDS (no barrier: plan_unit's callers pass
// at least one before plan_unit reads them).  Issued early, so the loads
// overlap other work.
template <int NT = kNT>
__device__ __forceinline__ void plan_load(const int32_t* blk_in, const int32_t* stamp_in, int K,
                                          const PlanLds& L) {
    const int K4 = pad4(K);
    for (int s = threadIdx.x; s < K4; s += NT) {
        L.blk[s] = s < K ? blk_in[s] : -1;
        L.stamp[s] = s < K ? stamp_in[s] : 0;
    }
}

// Slots in (stamp, slot) order, oldest first (L.order[rank] = slot), whether
// any slot is empty (the seeding plan), and each resident block's slot in
// L.mark_b: all depend on the slot tables only, so a FAST plan has them
// before its predicted list exists.  Run as a selection hook: before() needs
// the staged tables (plan_load, its loads waited for) and a barrier after it,
// after() counts each slot's rank (four adjacent lanes per slot when the
// workgroup has them, each over a quarter of the keys).
template <int NT>
struct PlanOrderHook {
    const PlanLds& L;
    int K, n_blk;
    __device__ void before() const {
        const int tid = threadIdx.x;
        const int K4 = pad4(K);
        int empty = 0;
        for (int s = tid; s < K4; s += NT) {
            const int bb = s < K ? L.blk[s] : -1;
            L.ekey[s] = s < K ? (long long)(((unsigned long long)(long long)L.stamp[s] << 32) | (unsigned)s)
                              : 0x7fffffffffffffffLL;
            empty |= s < K && bb == -1;
            if (bb >= 0 && bb < n_blk) L.mark_b[bb] = (uint16_t)s;
        }
        const bool wave_empty = __ballot(empty) != 0;
        if ((tid & 63) == 0) L.scanbuf[56 + (tid >> 6)] = wave_empty;
    }
    __device__ void after() const {
        const int tid = threadIdx.x;
        const int K4 = pad4(K);
        const longlong2* E2 = reinterpret_cast<const longlong2*>(L.ekey);
        if (NT >= 4 * K4) {
            const int s = tid >> 2, part = tid & 3;
            const int q = K4 / 8;  // pairs per quarter; the last quarter takes the rest
            const int i0 = part * q, i1 = part == 3 ? K4 / 2 : i0 + q;
            int r = 0;
            if (s < K) {
                const long long e = L.ekey[s];
                for (int i = i0; i < i1; ++i) {
                    const longlong2 x = E2[i];
                    r += (x.x < e) + (x.y < e);
                }
            }
            r += __shfl_xor(r, 1, 64);
            r += __shfl_xor(r, 2, 64);
            if (s < K && part == 0) L.order[r] = s;
            return;
        }
        for (int s = tid; s < K; s += NT) {
            const long long e = L.ekey[s];
            int r = 0;
#pragma unroll 8
            for (int i = 0; i < K4 / 2; ++i) {
                const longlong2 x = E2[i];
                r += (x.x < e) + (x.y < e);
            }
            L.order[r] = s;
        }
    }
};

// Capped least-recently-selected plan of one unit from the ranked predicted
// list P (LDS, -1 padded) and the staged slot tables, then the insertion of
// the request's newly completed block `ins` (-1 = none): outside the cap it
// refreshes its slot if resident, else takes the slot with the smallest
// (stamp, slot) after the admissions, taking over that slot's admission if it
// had one.  The outputs may alias the slot tables the stage was loaded from.
// FAST (after plan_order, block ids below n_blk): membership through marks
// indexed by block (each list writes its index at its blocks' marks, then a
// block is in a list iff the entry its mark names holds it, so stale marks
// are harmless and no atomics are needed), and the victims' order from the
// slot order by the same block scan as the missing blocks.  Otherwise
// membership compares every pair and the victims are ranked by counting.
template <bool FAST = false, int NT = kNT>
__device__ void plan_unit(const int* P, int K, int32_t* blk_out, int32_t* stamp_out, int step,
                          int cap, int ins, int32_t* cnt_out, int32_t* src_out, int32_t* dst_out,
                          int32_t* ev_out, const PlanLds& L, int n_blk = 0) {
    const int tid = threadIdx.x;
    const int K4 = pad4(K);
    int seeding = 0;
    uint32_t n_missing = 0, n_hits = 0;
    bool admitted = false;  // the FAST one-wave path admits the missing blocks itself
    if (FAST && K <= 256) {
        // The marks are in place (mark_b from the slot-order hook, mark_p from
        // the ranking): every thread tests membership, then one wave scans
        // (lane l takes items 4l .. 4l+3: predicted ranks, slots, slots in
        // (stamp, slot) order).
        for (int w = 0; w < NT / 64; ++w) seeding |= L.scanbuf[56 + w] != 0;
        for (int it = tid; it < K; it += NT) {
            const int bb = L.blk[it];
            int hit = 0;
            if (bb >= 0 && bb < n_blk) {
                const int i = L.mark_p[bb];
                hit = i < K && P[i] == bb;
            }
            L.hit[it] = hit;
            L.new_blk[it] = bb;
            L.new_stamp[it] = hit ? step : L.stamp[it];
            const int pb = P[it];
            int found = 0;
            if (pb >= 0 && pb < n_blk) {
                const int sl = L.mark_b[pb];
                found = sl < K && L.blk[sl] == pb;
            }
            L.miss[it] = pb >= 0 && !found;
        }
        lds_barrier();
        if (tid < 64) {
            uint32_t f0[4], f1[4], f2[4];
            int so[4];
            uint32_t c0 = 0, c1 = 0, c2 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * tid + e;
                const bool ok = i < K;
                so[e] = ok ? L.order[i] : 0;
                f0[e] = ok ? (uint32_t)L.miss[i] : 0u;
                f1[e] = ok ? (uint32_t)L.hit[i] : 0u;
                f2[e] = ok ? (uint32_t)(L.hit[so[e]] == 0) : 0u;
                c0 += f0[e];
                c1 += f1[e];
                c2 += f2[e];
            }
            const uint32_t i0 = wave_incl_sum(c0), i1 = wave_incl_sum(c1), i2 = wave_incl_sum(c2);
            uint32_t e0 = i0 - c0, e2 = i2 - c2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * tid + e;
                if (f0[e]) L.missing_of_rank[e0++] = P[i];
                if (i < K) {
                    if (f2[e]) L.victim_of_rank[e2] = so[e];
                    L.rank_of_slot[so[e]] = f2[e] ? (int)e2 : K;
                    e2 += f2[e];
                }
            }
            if (tid == 63) {
                L.scanbuf[0] = i0;
                L.scanbuf[1] = i1;
            }
            if (tid == 0) L.ins_key[1] = ~0ull;  // for the insertion below
            // The same wave admits the missing blocks: its lanes' LDS writes
            // above are seen by its reads below (one wave's LDS operations
            // complete in order), so no workgroup barrier sits in between.
            const int nm = (int)__builtin_amdgcn_readlane((int)i0, 63);
            const int nh = (int)__builtin_amdgcn_readlane((int)i1, 63);
            int na = min(nm, K - nh);
            bool seed_w = false;
            for (int w = 0; w < NT / 64; ++w) seed_w |= L.scanbuf[56 + w] != 0;
            if (!seed_w) na = min(na, cap);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            for (int i = tid; i < na; i += 64) {
                const int dst = L.victim_of_rank[i];
                L.new_blk[dst] = L.missing_of_rank[i];
                L.new_stamp[dst] = step;
            }
        }
        admitted = true;
        lds_barrier();
        n_missing = L.scanbuf[0];
        n_hits = L.scanbuf[1];
    } else {
        if constexpr (FAST) {
            // Membership both ways through the marks (16-bit stores, one writer
            // per mark except for blocks held twice, which then agree).
            for (int it = tid; it < K; it += NT) {
                const int pb = P[it], bb = L.blk[it];
                if (pb >= 0 && pb < n_blk) L.mark_p[pb] = (uint16_t)it;
                if (bb >= 0 && bb < n_blk) L.mark_b[bb] = (uint16_t)it;
            }
            lds_barrier();
            for (int w = 0; w < NT / 64; ++w) seeding |= L.scanbuf[56 + w] != 0;
            for (int it = tid; it < K; it += NT) {
                const int bb = L.blk[it];
                int hit = 0;
                if (bb >= 0 && bb < n_blk) {
                    const int i = L.mark_p[bb];
                    hit = i < K && P[i] == bb;
                }
                L.hit[it] = hit;
                const int pb = P[it];
                int found = 0;
                if (pb >= 0 && pb < n_blk) {
                    const int sl = L.mark_b[pb];
                    found = sl < K && L.blk[sl] == pb;
                }
                L.miss[it] = pb >= 0 && !found;
            }
            lds_barrier();
        } else {
            int empty = 0;
            for (int s = tid; s < K; s += NT) empty |= L.blk[s] == -1;
            const bool wave_empty = __ballot(empty) != 0;
            if ((tid & 63) == 0) L.scanbuf[56 + (tid >> 6)] = wave_empty;
            lds_barrier();
            for (int w = 0; w < NT / 64; ++w) seeding |= L.scanbuf[56 + w] != 0;
            // Membership both ways: slot s is a hit if its block is predicted; rank i
            // is missing if its block is not resident.  Items [0, K) are slots,
            // [K, 2K) predicted ranks.
            const int4* P4 = reinterpret_cast<const int4*>(P);
            const int4* B4 = reinterpret_cast<const int4*>(L.blk);
            for (int it = tid; it < 2 * K; it += NT) {
                const bool slot = it < K;
                const int idx = slot ? it : it - K;
                const int v = slot ? L.blk[idx] : P[idx];
                const int4* other = slot ? P4 : B4;
                int found = 0;
                if (v >= 0) {
#pragma unroll 8
                    for (int i = 0; i < K4 / 4; ++i) {
                        const int4 x = other[i];
                        found |= (x.x == v) | (x.y == v) | (x.z == v) | (x.w == v);
                    }
                }
                if (slot)
                    L.hit[idx] = found;
                else
                    L.miss[idx] = v >= 0 && !found;
            }
            lds_barrier();
        }
        // Missing blocks in rank order, victims counted (FAST: victims in slot
        // order, so the scan also gives each non-hit slot its victim rank).
        if constexpr (FAST) {
            uint32_t n_vict = 0;
            for (int base = 0; base < K; base += NT) {
                const int i = base + tid;
                const int so = i < K ? L.order[i] : 0;
                uint32_t v[3] = {i < K ? (uint32_t)L.miss[i] : 0u, i < K ? (uint32_t)L.hit[i] : 0u,
                                 i < K ? (uint32_t)(L.hit[so] == 0) : 0u};
                uint32_t ex[3], tot[3];
                block_scan<3, NT>(v, ex, tot, L.scanbuf);
                if (v[0]) L.missing_of_rank[n_missing + ex[0]] = P[i];
                if (i < K) {
                    if (v[2]) L.victim_of_rank[n_vict + ex[2]] = so;
                    L.rank_of_slot[so] = v[2] ? (int)(n_vict + ex[2]) : K;
                }
                n_missing += tot[0];
                n_hits += tot[1];
                n_vict += tot[2];
            }
            for (int s = tid; s < K; s += NT) {
                L.new_blk[s] = L.blk[s];
                L.new_stamp[s] = L.hit[s] ? step : L.stamp[s];
            }
            lds_barrier();
        } else {
            for (int base = 0; base < K; base += NT) {
                const int i = base + tid;
                uint32_t v[2] = {i < K ? (uint32_t)L.miss[i] : 0u, i < K ? (uint32_t)L.hit[i] : 0u};
                uint32_t ex[2], tot[2];
                block_scan<2, NT>(v, ex, tot, L.scanbuf);
                if (v[0]) L.missing_of_rank[n_missing + ex[0]] = P[i];
                n_missing += tot[0];
                n_hits += tot[1];
            }
            for (int s = tid; s < K4; s += NT)
                L.ekey[s] = (s < K && !L.hit[s])
                                ? (long long)(((unsigned long long)(long long)L.stamp[s] << 32) | (unsigned)s)
                                : 0x7fffffffffffffffLL;
            lds_barrier();
            // Victims ordered by (stamp, slot): counting rank over the 64-bit keys.
            for (int s = tid; s < K; s += NT) {
                if (!L.hit[s]) {
                    const long long e = L.ekey[s];
                    int r = 0;
                    const longlong2* E2 = reinterpret_cast<const longlong2*>(L.ekey);
#pragma unroll 8
                    for (int i = 0; i < K4 / 2; ++i) {
                        const longlong2 x = E2[i];
                        r += (x.x < e) + (x.y < e);
                    }
                    L.victim_of_rank[r] = s;
                    L.rank_of_slot[s] = r;
                } else {
                    L.rank_of_slot[s] = K;
                }
                L.new_blk[s] = L.blk[s];
                L.new_stamp[s] = L.hit[s] ? step : L.stamp[s];
            }
            lds_barrier();
        }
    }
    const int n_victims = K - (int)n_hits;
    int n = min((int)n_missing, n_victims);
    if (!seeding) n = min(n, cap);
    if (!admitted) {
        for (int i = tid; i < n; i += NT) {
            const int dst = L.victim_of_rank[i];
            L.new_blk[dst] = L.missing_of_rank[i];
            L.new_stamp[dst] = step;
        }
        if (ins >= 0 && tid == 0) L.ins_key[1] = ~0ull;
        lds_barrier();
    }
    if (ins >= 0) {  // uniform: one value per request
        // The oldest (stamp, slot) after the admissions: a minimum per thread,
        // per wave (DPP, high words first, then the low words of the lanes
        // holding the smallest high word), then over the waves.
        unsigned long long best = ~0ull;
        for (int s = tid; s < K; s += NT) {
            // Stamps are >= -1: the offset keeps the unsigned order of (stamp, slot).
            const unsigned long long key =
                ((unsigned long long)((long long)L.new_stamp[s] + 0x80000000LL) << 32) | (unsigned)s;
            best = key < best ? key : best;
            if (L.new_blk[s] == ins) L.ins_key[1] = (unsigned)s;  // at most one slot
        }
        const uint32_t bh = (uint32_t)(best >> 32);
        const uint32_t mh = wave_min(bh);
        const uint32_t ml = wave_min(bh == mh ? (uint32_t)best : 0xffffffffu);
        if ((tid & 63) == 0) L.ins_key[2 + (tid >> 6)] = ((unsigned long long)mh << 32) | ml;
        lds_barrier();
        if (tid == 0) {
            unsigned long long oldest = L.ins_key[2];
#pragma unroll
            for (int ww = 1; ww < NT / 64; ++ww)
                oldest = L.ins_key[2 + ww] < oldest ? L.ins_key[2 + ww] : oldest;
            L.ins_key[0] = oldest;
            const unsigned long long at = L.ins_key[1];
            if (at != ~0ull) {
                L.new_stamp[(int)at] = step;
            } else {
                const int v = (int)(L.ins_key[0] & 0xffffffffu);
                const int e = L.rank_of_slot[v];
                if (e < n) {  // v was admitted by this plan: its entry brings the new block
                    L.missing_of_rank[e] = ins;
                } else {
                    L.missing_of_rank[n] = ins;
                    L.victim_of_rank[n] = v;
                    ++n;
                }
                L.new_blk[v] = ins;
                L.new_stamp[v] = step;
            }
            L.scanbuf[48] = (uint32_t)n;
        }
        lds_barrier();
        n = (int)L.scanbuf[48];
    }
    for (int i = tid; i < K; i += NT) {
        if (i < n) {
            const int dst = L.victim_of_rank[i];
            src_out[i] = L.missing_of_rank[i];
            dst_out[i] = dst;
            if (ev_out) ev_out[i] = L.blk[dst];
        } else {
            src_out[i] = -1;
            dst_out[i] = -1;
            if (ev_out) ev_out[i] = -1;
        }
    }
    for (int s = tid; s < K; s += NT) {
        blk_out[s] = L.new_blk[s];
        stamp_out[s] = L.new_stamp[s];
    }
    if (tid == 0) *cnt_out = n;
}

__device__ __forceinline__ TopkLds carve_topk(LdsCursor& cur, int NQ, int K4) {
    TopkLds T;
    T.hist = cur.take<int>(NQ * 512);
    T.scanbuf = cur.take<uint32_t>(4 * 2);
    T.sh = cur.take<int>(16);
    T.sel_key = cur.take<uint32_t>((size_t)NQ * K4);
    T.sel_idx = cur.take<int>((size_t)NQ * K4);
    T.P = cur.take<int>(K4);
    T.ek = nullptr;
    return T;
}

// Top-K of every row of unit u from `sc` (row stride rs), then, in the fused
// step, the plan of the unit from row pred_row.
template <int NQ>
__device__ void select_unit(const StepArgs& a, int u, const float* sc, size_t rs,
                            const TopkLds& T, const PlanLds& Pl) {
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int n_r = a.n_blk ? min(max(a.n_blk[r], 0), a.n_blk_max) : a.n_blk_max;
    const size_t ors = (size_t)a.H * a.K;
    const size_t ob = ((size_t)r * NQ * a.H + g) * a.K;
    topk_rows<NQ>(sc, rs, n_r, a.K, a.topk_idx + ob, a.topk_score ? a.topk_score + ob : nullptr,
                  ors, a.do_plan ? a.pred_row : -1, T);
    if (!a.do_plan) return;
    const size_t so = (size_t)u * a.K;
    plan_unit(T.P, a.K, a.slot_blk_out + so, a.slot_stamp_out + so, a.step, a.cap,
              a.ins_blk ? a.ins_blk[r] : -1, a.plan_count + u, a.plan_src + so, a.plan_dst + so,
              a.plan_evicted ? a.plan_evicted + so : nullptr, Pl);
}

// ============================================================ scan item
template <int DT, int D, int NQ>
__device__ void scan_item(const StepArgs& a, int u, int c, unsigned char* lds) {
    LdsCursor cur{lds};
    float* pn = cur.take<float>(NQ * 2 * D);
    const int K4 = pad4(a.K);
    const TopkLds T = carve_topk(cur, NQ, K4);
    const PlanLds Pl = carve_plan(cur, K4);
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    float* gsc = a.scores ? a.scores + ((size_t)r * NQ * a.H + g) * a.n_blk_max : nullptr;
    const size_t grs = (size_t)a.H * a.n_blk_max;
    if (a.NC > 1) {  // one chunk of a split unit: scores to global, selection later
        scan_blocks<DT, D, NQ>(a, u, c, pn, gsc, grs);
        return;
    }
    if (a.do_plan) plan_load(a.slot_blk_in + (size_t)u * a.K, a.slot_stamp_in + (size_t)u * a.K, a.K, Pl);
    if (a.scores_lds) {
        float* lsc = cur.take<float>((size_t)NQ * a.n_blk_max);
        scan_blocks<DT, D, NQ>(a, u, 0, pn, lsc, a.n_blk_max);
        lds_barrier();
        if (gsc)  // the caller asked for every block score
            for (int i = threadIdx.x; i < NQ * a.n_blk_max; i += kNT) {
                const int j = i / a.n_blk_max, b = i - j * a.n_blk_max;
                gsc[j * grs + b] = lsc[i];
            }
        select_unit<NQ>(a, u, lsc, a.n_blk_max, T, Pl);
    } else {
        scan_blocks<DT, D, NQ>(a, u, 0, pn, gsc, grs);
        __syncthreads();
        select_unit<NQ>(a, u, gsc, grs, T, Pl);
    }
}

// ============================================================ attention
// Split of one unit: table entries [e0, e1); the last split also owns the
// active block (tail_len tokens of tile tail_tile).
struct SplitRange {
    int e0, e1, tail_tile, tail_len;
};

template <bool TOK = false>
__device__ __forceinline__ SplitRange split_range(const StepArgs& a, int u, int sp) {
    SplitRange s;
    s.e0 = min(sp * a.per_split, a.n_sel);
    s.e1 = min(s.e0 + a.per_split, a.n_sel);
    s.tail_tile = -1;
    s.tail_len = 0;
    if constexpr (TOK) {  // the tokens of the active block before the new one
        if (sp == a.S - 1) {
            const int p = a.pos[u / a.H];
            if (p >= 0 && p / a.B < a.unit_stride && p % a.B > 0) {
                s.tail_tile = p / a.B;
                s.tail_len = p % a.B;
            }
        }
        return s;
    }
    if (sp == a.S - 1 && a.tail_tile && a.tail_len) {
        const int r = u / a.H;
        const int tt = a.tail_tile[u];
        const int tl = min(a.tail_len[r], a.B);
        if (tt >= 0 && tt < a.unit_stride && tl > 0) {
            s.tail_tile = tt;
            s.tail_len = tl;
        }
    }
    return s;
}

// LDS of an attention item: table slice + final (m, l, acc) of the item, plus
// the kernel-specific staging below, plus (tok) the appended token's stage.
__host__ __device__ inline size_t attn_lds_bytes(int att, int NR, int D, int per_split,
                                                 bool tok = false) {
    auto a16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    size_t b = a16((size_t)per_split * 4) + a16(NR * 4) * 2 + a16((size_t)NR * D * 4);
    if (tok) b += a16((size_t)NR * D * 4) + a16((size_t)D * 4) * 2 +
                  a16((size_t)kSummRows * D * 4);  // TokStage (raw elements, fp32 at most)
    if (att == kAttnMfma) {
        b += a16(3 * NR * 4) * 2 + a16((size_t)3 * NR * D * 4) + a16((size_t)4 * 16 * D * 2);
    } else {
        b += a16((size_t)kMaxRows * D * 4) + a16(16 * (D + 1) * 4) + a16((size_t)D * 17 * 4) +
             a16(kMaxRows * 16 * 4) + a16(kMaxRows * 4) * 3;
    }
    return b;
}

struct AttnFin {
    float* m;    // [NR] running max, log2 domain
    float* l;    // [NR] sum of exp2(z - m)
    float* acc;  // [NR][D] unnormalised output
};

// Rows of a unit one attention item computes: [row0, row0 + nr), partials in
// buffer group grp.  With row groups (RGN > 1, wide GQA groups) each query row
// j is its own item of the G rows of head group g, so an item needs one
// 16-row MFMA block and the kernel keeps two waves per SIMD; the item pair
// of a split reads the same tiles back to back on one XCD.
struct RowWin {
    int row0, nr, grp;
};

__device__ __forceinline__ RowWin row_win(const StepArgs& a, int grp) {
    return a.RGN > 1 ? RowWin{grp * a.G, a.G, grp} : RowWin{0, a.NR, 0};
}

// The appended token of a growing context (launches instantiated with TOK):
// what its online-softmax step and its summary need -- the unit's query rows,
// the token's key and value, and the active block's stored keys (used when
// the token completes the block, B <= kSummRows + 1) -- loaded as 16-byte
// vectors in the round trip the attention item makes anyway before its first
// tile, and kept in LDS as raw elements, so the step after the loop issues no
// load (under the launch's full HBM stream a round trip there costs several
// microseconds at the end of the critical path).  Every load is issued before
// the first LDS store, unconditionally with its index clamped (a guarded load
// compiles to a branch that waits for it).
struct TokStage {
    const uint8_t* q;     // [NR][D] the unit's query rows (LDS, raw elements)
    const uint8_t* k;     // [D] the new key
    const uint8_t* v;     // [D] the new value
    const uint8_t* rows;  // [B-1][D] stored keys of the active block
    int active;           // this item appends a token (uniform)
    int summ;             // the token completes its block: 0 no, 1 rows staged, 2 load them
    int blk, slot;        // the token's block and its row in the block
};

template <int DT, int D>
__device__ __forceinline__ TokStage tok_prefetch(const StepArgs& a, int u, int sp, LdsCursor& cur) {
    constexpr int EB = Elem<DT>::bytes;
    constexpr int RV = D * EB / 16;  // 16-byte vectors per row of D elements
    uint4* q = cur.take<uint4>((size_t)a.NR * RV);
    uint4* k = cur.take<uint4>(RV);
    uint4* v = cur.take<uint4>(RV);
    uint4* rows = cur.take<uint4>((size_t)kSummRows * D * 4 / 16);
    TokStage ts;
    ts.q = reinterpret_cast<const uint8_t*>(q);
    ts.k = reinterpret_cast<const uint8_t*>(k);
    ts.v = reinterpret_cast<const uint8_t*>(v);
    ts.rows = reinterpret_cast<const uint8_t*>(rows);
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int p = a.pos[r];
    ts.active = sp == a.S - 1 && p >= 0 && p / a.B < a.unit_stride;
    ts.summ = 0;
    ts.blk = ts.slot = 0;
    if (!ts.active) return ts;
    const int tid = threadIdx.x;
    const int b = p / a.B, t = p - (p / a.B) * a.B;
    ts.blk = b;
    ts.slot = t;
    if (t == a.B - 1) ts.summ = a.B - 1 <= kSummRows ? 1 : 2;
    // query rows: for each query row group j the G heads' rows are contiguous
    constexpr int QPT = (kMaxRows * D * 4 / 16 + kNT - 1) / kNT;  // q vectors per thread at most
    const int nqv = a.NR * RV, gv = a.G * RV;
    const uint4* qsrc = reinterpret_cast<const uint4*>(a.q) +
                        ((size_t)r * a.NQ * a.Hq + (size_t)g * a.G) * RV;
    const size_t qj = (size_t)a.Hq * RV;
    uint4 qv[QPT];
#pragma unroll
    for (int e = 0; e < QPT; ++e) {
        const int i = min(tid + e * kNT, nqv - 1);
        const int j = (i >= gv) + (i >= 2 * gv);  // n_q <= 3
        qv[e] = qsrc[(size_t)j * qj + (i - j * gv)];
    }
    const int kvi = min(tid, RV - 1);
    const uint4 kx = reinterpret_cast<const uint4*>(a.k_new)[(size_t)u * RV + kvi];
    const uint4 vx = reinterpret_cast<const uint4*>(a.v_new)[(size_t)u * RV + kvi];
    constexpr int RPT = (kSummRows * D * 4 / 16 + kNT - 1) / kNT;  // row vectors per thread at most
    const int nrv = min(a.B - 1, kSummRows) * RV;
    const uint4* rsrc = reinterpret_cast<const uint4*>(
        a.kt + ((size_t)u * a.unit_stride + b) * (size_t)a.tile_stride * EB);
    uint4 rv[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) rv[e] = rsrc[min(tid + e * kNT, max(nrv - 1, 0))];
#pragma unroll
    for (int e = 0; e < QPT; ++e)
        if (tid + e * kNT < nqv) q[tid + e * kNT] = qv[e];
    if (tid < RV) {
        k[tid] = kx;
        v[tid] = vx;
    }
    if (ts.summ == 1) {
#pragma unroll
        for (int e = 0; e < RPT; ++e)
            if (tid + e * kNT < nrv) rows[tid + e * kNT] = rv[e];
    }
    return ts;
}

// MFMA split (bf16, B % 16 == 0).  Per 16-token sub-tile:
//   S^T[16 tok][16 rows] = K_sub[16][D] * Q^T  (v_mfma_f32_16x16x32_bf16, q in
//   registers),
//   O^T[D][rows] += V^T * P^T                  (v_mfma_f32_16x16x16_bf16; the A
//   operand is 4 consecutive tokens of one dim, contiguous in a [D][B] V tile).
// The K operand wants 16 tokens x 16 bytes per instruction, i.e. 16 separate
// 64-byte pieces of the tile; such loads stream ~30% slower than contiguous
// ones on this part.  K is therefore loaded contiguously (lane i of load j
// takes bytes [1024 j + 16 i, +16)) and passed through a per-wave LDS stage:
// 16-byte chunk c of token t goes to slot 16 c + (t ^ c), which makes both the
// contiguous writes (one token, 16 chunks) and the operand reads (one chunk,
// 16 tokens) hit 16 distinct bank groups.
// The 4 waves take sub-tiles round robin and keep their next two sub-tiles in
// flight in registers while the current one is computed.  P is rounded to bf16.
// Returns the appended token's stage (TOK; inactive otherwise).
template <int D, int NRG, bool TOK>
__device__ TokStage attn_item_mfma(const StepArgs& a, int u, int sp, const RowWin& win,
                                   LdsCursor& cur, const AttnFin& F, int* tbl) {
    constexpr int KB = D / 32;
    constexpr int DB = D / 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int NR = win.nr, B = a.B;
    constexpr int CPR = D * 2 / 16;  // 16-byte chunks per K row (KB loads of 1 KiB per sub-tile)
    float* lm = cur.take<float>(3 * NR);
    float* ll = cur.take<float>(3 * NR);
    float* la = cur.take<float>((size_t)3 * NR * D);
    uint4* kst = cur.take<uint4>((size_t)4 * 16 * CPR) + (size_t)w * 16 * CPR;  // this wave's stage

    bf16x8_t qv[NRG][KB];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        const int row = rg * 16 + l16;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qv[rg][kb] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        if (row < NR) {
            const int grow = win.row0 + row;
            const int j = grow / a.G, hh = grow - (grow / a.G) * a.G;
            const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(
                a.q + ((((size_t)r * a.NQ + j) * a.Hq + (size_t)g * a.G + hh) * D) * 2);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qv[rg][kb] = qp[kb * 4 + lg];
        }
    }
    // The unit's tile table goes to LDS while the q loads above are in
    // flight (one round trip for both before the first tile load), and so
    // does an appended token's stage.
    TokStage ts{};
    if constexpr (TOK) ts = tok_prefetch<OASIS_BF16, D>(a, u, sp, cur);
    const SplitRange sr = split_range<TOK>(a, u, sp);
    for (int i = threadIdx.x; i < sr.e1 - sr.e0; i += kNT)
        tbl[i] = a.table[(size_t)u * a.n_sel + sr.e0 + i];
    __syncthreads();
    float m[NRG], lsum[NRG];
    f32x4_t acc[NRG][DB];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        m[rg] = -__builtin_inff();
        lsum[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int spe = B / 16;
    const int n_entry_sub = (sr.e1 - sr.e0) * spe;
    const int n_sub = n_entry_sub + (sr.tail_len + 15) / 16;
    const size_t tile_elems = (size_t)a.tile_stride;

    // Loads of sub-tile st (the table lives in LDS).  Every call issues the
    // same loads whether or not st is a real sub-tile (a -1 entry, or past
    // the end): then the compiler's count of loads in flight is exact and it
    // waits only for the buffer being consumed, never for the prefetch.  A
    // placeholder call reads one 16-byte piece of the unit's first tile.
    auto fetch = [&](int st, bf16x8_t (&kv)[KB], bf16x4_t (&vv)[DB]) -> int {
        int tile = 0, sub = 0, ntok = 0;
        if (st < n_entry_sub) {
            const int e = st / spe;
            tile = tbl[e];
            sub = st - e * spe;
            // ids outside the unit's tiles are skipped like -1 entries
            ntok = (tile >= 0 && tile < a.unit_stride) ? 16 : 0;
        } else if (st < n_sub) {
            tile = sr.tail_tile;
            sub = st - n_entry_sub;
            ntok = min(16, sr.tail_len - sub * 16);
        }
        const bool real = ntok > 0;
        const size_t t64 = (size_t)((long long)u * a.unit_stride + (real ? tile : 0));
        const uint8_t* kbase = a.kt + (t64 * tile_elems + (real ? (size_t)sub * 16 * D : 0)) * 2;
        const uint8_t* vbase = a.vt + (t64 * tile_elems + (real ? (size_t)sub * 16 : 0)) * 2;
#pragma unroll
        for (int j = 0; j < KB; ++j)
            kv[j] = load_stream(
                reinterpret_cast<const bf16x8_t*>(kbase + (real ? ((size_t)j * 64 + lane) * 16 : 0)));
#pragma unroll
        for (int db = 0; db < DB; ++db)
            vv[db] = load_stream(reinterpret_cast<const bf16x4_t*>(
                vbase + (real ? ((size_t)(db * 16 + l16) * B + lg * 4) * 2 : 0)));
        return ntok;
    };

    // One 16-token sub-tile: stage K, S = K q^T, online softmax, O += V^T P^T.
    auto compute = [&](const bf16x8_t (&kc)[KB], bf16x4_t (&vc)[DB], int ntok) {
        if (ntok < 16) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lg * 4 + e >= ntok) vc[db][e] = 0;
        }
        // Contiguous K chunks -> swizzled stage -> MFMA operand layout.
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
            const int t = jj * (64 / CPR) + lane / CPR, c = lane % CPR;
            kst[c * 16 + (t ^ (c & 15))] = *reinterpret_cast<const uint4*>(&kc[jj]);
        }
        bf16x8_t kop[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int c = kb * 4 + lg;
            const uint4 x = kst[c * 16 + (l16 ^ (c & 15))];
            kop[kb] = *reinterpret_cast<const bf16x8_t*>(&x);
        }
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb], qv[rg][kb], sc, 0, 0, 0);
            // sc[e] = score of token lg*4+e for row l16.
            float tmax = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[e] = (lg * 4 + e < ntok) ? sc[e] * a.scale_log2 : -__builtin_inff();
                tmax = fmaxf(tmax, sc[e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mnew = fmaxf(m[rg], tmax);
            // A row that has seen no token yet keeps m = -inf: weight 0, no NaN.
            const bool none = mnew == -__builtin_inff();
            const float corr = none ? 1.f : exp2f(m[rg] - mnew);
            float p[4];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = none ? 0.f : exp2f(sc[e] - mnew);
                psum += p[e];
            }
            lsum[rg] = lsum[rg] * corr + psum;
            m[rg] = mnew;
            bf16x4_t pb;
            pb[0] = (short)f32_to_bf16_bits(p[0]);
            pb[1] = (short)f32_to_bf16_bits(p[1]);
            pb[2] = (short)f32_to_bf16_bits(p[2]);
            pb[3] = (short)f32_to_bf16_bits(p[3]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[rg][db] *= corr;
                acc[rg][db] =
                    __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vc[db], pb, acc[rg][db], 0, 0, 0);
            }
        }
    };
    // Three register buffers in rotation (unrolled, so no buffer is ever
    // copied): two sub-tiles of this wave are in flight while the third is
    // computed.  Copying a prefetched buffer into a "current" one would make
    // the wave wait for the prefetch at every step; compute() runs for
    // placeholder sub-tiles too (ntok = 0 masks every token), so no path
    // leaves a buffer's loads unconsumed.  sched_barrier keeps each buffer's
    // loads issued before the arithmetic on the previous one.
    bf16x8_t kA[KB], kB[KB], kC[KB], kD[KB];
    bf16x4_t vA[DB], vB[DB], vC[DB], vD[DB];
    int st = w;
    int nA = fetch(st, kA, vA);
    int nB = fetch(st + 4, kB, vB);
    int nC = fetch(st + 8, kC, vC);
    int nD = 0;
    while (st < n_sub) {
        nD = fetch(st + 12, kD, vD);
        __builtin_amdgcn_sched_barrier(0);
        compute(kA, vA, nA);
        st += 4;
        if (st >= n_sub) break;
        nA = fetch(st + 12, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        compute(kB, vB, nB);
        st += 4;
        if (st >= n_sub) break;
        nB = fetch(st + 12, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        compute(kC, vC, nC);
        st += 4;
        if (st >= n_sub) break;
        nC = fetch(st + 12, kC, vC);
        __builtin_amdgcn_sched_barrier(0);
        compute(kD, vD, nD);
        st += 4;
    }
    // Row sums: the 4 lane groups hold disjoint tokens of the same rows.
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        lsum[rg] += __shfl_xor(lsum[rg], 16, 64);
        lsum[rg] += __shfl_xor(lsum[rg], 32, 64);
    }
    // Waves 1..3 park their state, wave 0 combines in wave order.
    if (w > 0) {
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
            const int row = rg * 16 + l16;
            if (row < NR) {
                if (lg == 0) {
                    lm[(w - 1) * NR + row] = m[rg];
                    ll[(w - 1) * NR + row] = lsum[rg];
                }
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        la[((size_t)(w - 1) * NR + row) * D + db * 16 + lg * 4 + e] = acc[rg][db][e];
            }
        }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
            const int row = rg * 16 + l16;
            if (row >= NR) continue;
            float mw[3];
            float M = m[rg];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                mw[k] = lm[k * NR + row];
                M = fmaxf(M, mw[k]);
            }
            const float f0 = (m[rg] == -__builtin_inff()) ? 0.f : exp2f(m[rg] - M);
            float fk[3];
            float Lr = lsum[rg] * f0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                fk[k] = (mw[k] == -__builtin_inff()) ? 0.f : exp2f(mw[k] - M);
                Lr += ll[k * NR + row] * fk[k];
            }
            if (lg == 0) {
                F.m[row] = M;
                F.l[row] = Lr;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x4_t o = acc[rg][db] * f0;
#pragma unroll
                for (int k = 0; k < 3; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] += fk[k] * la[((size_t)k * NR + row) * D + db * 16 + lg * 4 + e];
                *reinterpret_cast<f32x4_t*>(F.acc + (size_t)row * D + db * 16 + lg * 4) = o;
            }
        }
    }
    __syncthreads();
    return ts;
}

// VALU split (any dtype and block size): 16-token sub-tiles of K and V staged
// in LDS as fp32, scalar FMAs.
template <int DT, int D, bool TOK>
__device__ void attn_item_valu(const StepArgs& a, int u, int sp, LdsCursor& cur, const AttnFin& F,
                               const int* tbl) {
    constexpr int ST = 16;
    constexpr int OPT = kMaxRows * D / kNT;
    float* qs = cur.take<float>((size_t)kMaxRows * D);     // [row][D]
    float* ks = cur.take<float>((size_t)ST * (D + 1));     // [tok][D+1]
    float* vs = cur.take<float>((size_t)D * (ST + 1));     // [D][ST+1]
    float* ps = cur.take<float>((size_t)kMaxRows * ST);    // [row][ST]
    float* m_s = cur.take<float>(kMaxRows);
    float* l_s = cur.take<float>(kMaxRows);
    float* c_s = cur.take<float>(kMaxRows);
    const int tid = threadIdx.x;
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int NR = a.NR, B = a.B;
    for (int i = tid; i < NR * D; i += kNT) {
        const int row = i / D, d = i - (i / D) * D;
        const int j = row / a.G, hh = row - (row / a.G) * a.G;
        qs[row * D + d] =
            load_elem<DT>(a.q, (((size_t)r * a.NQ + j) * a.Hq + (size_t)g * a.G + hh) * D + d) *
            a.scale_log2;
    }
    if (tid < NR) {
        m_s[tid] = -__builtin_inff();
        l_s[tid] = 0.f;
    }
    float acc[OPT];
#pragma unroll
    for (int k = 0; k < OPT; ++k) acc[k] = 0.f;
    __syncthreads();
    const SplitRange sr = split_range<TOK>(a, u, sp);
    const int sub_tokens = B < ST ? B : ST;
    const int spe = B / sub_tokens;
    const int n_entry_sub = (sr.e1 - sr.e0) * spe;
    const int n_sub = n_entry_sub + (sr.tail_len + sub_tokens - 1) / sub_tokens;
    const size_t tile_elems = (size_t)a.tile_stride;
    for (int st = 0; st < n_sub; ++st) {
        int tile, sub, nt;
        if (st < n_entry_sub) {
            tile = tbl[st / spe];
            sub = st - (st / spe) * spe;
            nt = sub_tokens;
            if (tile < 0 || tile >= a.unit_stride) continue;  // -1 or out of range: skipped
        } else {
            tile = sr.tail_tile;
            sub = st - n_entry_sub;
            nt = min(sub_tokens, sr.tail_len - sub * sub_tokens);
        }
        const size_t base = (size_t)((long long)u * a.unit_stride + tile) * tile_elems;
        const int t0 = sub * sub_tokens;
        for (int i = tid; i < nt * D; i += kNT) {
            const int tt = i / D, d = i - (i / D) * D;
            ks[tt * (D + 1) + d] = load_elem<DT>(a.kt, base + (size_t)(t0 + tt) * D + d);
        }
        for (int i = tid; i < D * nt; i += kNT) {
            const int d = i / nt, tt = i - (i / nt) * nt;
            vs[d * (ST + 1) + tt] = load_elem<DT>(a.vt, base + (size_t)d * B + t0 + tt);
        }
        __syncthreads();
        for (int p = tid; p < NR * ST; p += kNT) {
            const int row = p / ST, tt = p - (p / ST) * ST;
            float z = -__builtin_inff();
            if (tt < nt) {
                z = 0.f;
                for (int d = 0; d < D; ++d) z = fmaf(qs[row * D + d], ks[tt * (D + 1) + d], z);
            }
            ps[row * ST + tt] = z;
        }
        __syncthreads();
        if (tid < NR) {
            float mx = m_s[tid];
            for (int tt = 0; tt < nt; ++tt) mx = fmaxf(mx, ps[tid * ST + tt]);
            const float corr = exp2f(m_s[tid] - mx);
            float sum = 0.f;
            for (int tt = 0; tt < nt; ++tt) {
                const float pv = exp2f(ps[tid * ST + tt] - mx);
                ps[tid * ST + tt] = pv;
                sum += pv;
            }
            l_s[tid] = l_s[tid] * corr + sum;
            m_s[tid] = mx;
            c_s[tid] = corr;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < OPT; ++k) {
            const int o = tid + k * kNT;
            if (o < NR * D) {
                const int row = o / D, d = o - (o / D) * D;
                float v = acc[k] * c_s[row];
                for (int tt = 0; tt < nt; ++tt) v = fmaf(ps[row * ST + tt], vs[d * (ST + 1) + tt], v);
                acc[k] = v;
            }
        }
        __syncthreads();
    }
    if (tid < NR) {
        F.m[tid] = m_s[tid];
        F.l[tid] = l_s[tid];
    }
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int o = tid + k * kNT;
        if (o < NR * D) F.acc[o] = acc[k];
    }
    __syncthreads();
}

// Output row of stacked row `row` (j * G + h within the group) of unit u.
__device__ __forceinline__ size_t attn_out_row(const StepArgs& a, int u, int row) {
    const int r = u / a.H, g = u - (u / a.H) * a.H;
    const int j = row / a.G, hh = row - (row / a.G) * a.G;
    return ((size_t)r * a.NQ + j) * a.Hq + (size_t)g * a.G + hh;
}

// Output of an attention item: normalised outputs when the unit has one
// split, else the split's partial (max, sum, acc) for finish_kernel.
template <int DT, int D>
__device__ void attn_emit(const StepArgs& a, int u, int sp, const RowWin& win, const AttnFin& F) {
    const int tid = threadIdx.x;
    const int NR = win.nr;
    if (a.S == 1) {
        for (int o = tid; o < NR * D; o += kNT) {
            const int row = o / D, d = o - (o / D) * D;
            const float L = F.l[row];
            store_elem<DT>(a.out, attn_out_row(a, u, win.row0 + row) * D + d,
                           L > 0.f ? F.acc[o] / L : 0.f);
        }
        if (a.lse && tid < NR) {
            const float L = F.l[tid];
            a.lse[attn_out_row(a, u, win.row0 + tid)] =
                L > 0.f ? (F.m[tid] + log2f(L)) * kLn2 : -__builtin_inff();
        }
        return;
    }
    const size_t pb = (((size_t)win.grp * a.U + u) * a.S + sp) * NR;
    for (int o = tid; o < NR * D; o += kNT) a.part_acc[pb * D + o] = F.acc[o];
    if (tid < NR) {
        a.part_ml[(pb + tid) * 2 + 0] = F.m[tid];
        a.part_ml[(pb + tid) * 2 + 1] = F.l[tid];
    }
}

// LSE merge of the S partials of unit u.  The partials come from another
// launch, so every round trip reaches the L2 of another XCD or HBM; the merge
// keeps them few.  Four adjacent threads own a 16-byte output piece, each a
// quarter of the splits; the accumulator loads of their first piece are
// issued before anything else, since they do not depend on the row maxima.
// (m, l) pairs lie [s][row], so thread t reads row t % NR of the splits
// t / NR, t / NR + NT / NR, ...: coalesced, one round trip; the row maxima,
// then the sums of exp2(m - M) * l, are reduced per row through LDS, and the
// weights exp2(m - M) of every (split, row) kept in LDS when they fit
// (kMergeW).  Each output then sums its splits' weighted accumulators (in
// split order within a quarter, the quarters as (0 + 1) + (2 + 3)) and divides
// by the row's sum.
constexpr int kMergeBatch = 16;  // 16-byte accumulator loads a merge thread keeps in flight
constexpr int kMergeW = 4096;    // (split, row) weights kept in LDS

template <int DT, int D, int NT = kNT>
__device__ void attn_merge_unit(const StepArgs& a, int u, const RowWin& win, float* Mr, float* Lr,
                                float* red, float* W) {
    const int tid = threadIdx.x;
    const int NR = win.nr, S = a.S;
    constexpr int D4 = D / 4;
    const int n4 = NR * D4;
    const int nsub = NT / NR;                 // threads per row
    const int nred = min(nsub, S);            // of those, the ones holding a split
    const int row_t = tid % NR, sub = tid / NR;
    const size_t ub = (size_t)win.grp * a.U + u;  // this item's partials: [S][NR]
    const float* ml = a.part_ml + ub * S * NR * 2;
    const float4* pa = reinterpret_cast<const float4*>(a.part_acc + ub * S * NR * D);
    const float ninf = -__builtin_inff();
    const bool keep_w = S * NR <= kMergeW;
    // tpo adjacent threads (4, or 2 when S < 4) share an output piece, each
    // summing a contiguous range of `per` splits; the ranges are then added in
    // a fixed tree.  The order depends on S only, so stacked rows merge exactly
    // as single rows.
    const int tpo = S >= 4 ? 4 : 2;
    const int per = (S + tpo - 1) / tpo;
    const int part = tid % tpo;
    const int s_lo = min(part * per, S), s_hi = min(s_lo + per, S);
    constexpr int MB = NT >= 1024 ? kMergeBatch / 2 : kMergeBatch;  // within 128 VGPRs at 1024
    float4 v[MB];
    auto load_batch = [&](int o4, int s0) {
#pragma unroll
        for (int e = 0; e < MB; ++e)
            v[e] = pa[(size_t)max(min(s0 + e, s_hi - 1), 0) * n4 + o4];
    };
    if (tid / tpo < n4) load_batch(tid / tpo, s_lo);
    // With S <= nsub a thread holds at most one (m, l) pair: read it once.
    const bool one = S <= nsub;
    float2 pr1 = make_float2(ninf, 0.f);
    if (one && sub < S) pr1 = reinterpret_cast<const float2*>(ml)[(size_t)sub * NR + row_t];
    float mx = pr1.x;
    if (!one)
        for (int s = sub; s < S; s += nsub) mx = fmaxf(mx, ml[((size_t)s * NR + row_t) * 2]);
    red[tid] = mx;
    __syncthreads();
    if (tid < NR) {
        float M = ninf;
        for (int k = 0; k < nred; ++k) M = fmaxf(M, red[tid + k * NR]);
        Mr[tid] = M;
    }
    __syncthreads();
    float sm = 0.f;
    if (one) {
        if (sub < S) {
            const float M = Mr[row_t];
            const float w = (M != ninf && pr1.x != ninf) ? exp2f(pr1.x - M) : 0.f;
            if (keep_w) W[sub * NR + row_t] = w;
            if (w != 0.f) sm += w * pr1.y;
        }
    } else if (sub < nsub) {
        const float M = Mr[row_t];
        for (int s = sub; s < S; s += nsub) {
            const size_t pr = ((size_t)s * NR + row_t) * 2;
            const float ms = ml[pr];
            const float w = (M != ninf && ms != ninf) ? exp2f(ms - M) : 0.f;
            if (keep_w) W[s * NR + row_t] = w;
            if (w != 0.f) sm += w * ml[pr + 1];
        }
    }
    red[tid] = sm;
    __syncthreads();
    if (tid < NR) {
        float L = 0.f;
        for (int k = 0; k < nred; ++k) L += red[tid + k * NR];
        Lr[tid] = L;
        const float M = Mr[tid];
        if (a.lse) a.lse[attn_out_row(a, u, win.row0 + tid)] = L > 0.f ? (M + log2f(L)) * kLn2 : ninf;
    }
    __syncthreads();  // Mr / Lr / W ready
    // Every thread of a group runs the same iterations (the shuffles below).
    for (int o4 = tid / tpo; o4 < n4; o4 += NT / tpo) {
        const int row = o4 / D4, d = (o4 - row * D4) * 4;
        const float M = Mr[row], L = Lr[row];
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = s_lo; s0 < s_hi; s0 += MB) {
            if (s0 > s_lo || o4 != tid / tpo) load_batch(o4, s0);
#pragma unroll
            for (int e = 0; e < MB; ++e) {
                const int sp = s0 + e;
                float w = 0.f;
                if (sp < s_hi) {
                    if (keep_w) {
                        w = W[sp * NR + row];
                    } else {
                        const float ms = ml[((size_t)sp * NR + row) * 2];
                        w = (M != ninf && ms != ninf) ? exp2f(ms - M) : 0.f;
                    }
                }
                if (w != 0.f) {
                    acc[0] = fmaf(w, v[e].x, acc[0]);
                    acc[1] = fmaf(w, v[e].y, acc[1]);
                    acc[2] = fmaf(w, v[e].z, acc[2]);
                    acc[3] = fmaf(w, v[e].w, acc[3]);
                }
            }
        }
        // ranges in order: (0 + 1) + (2 + 3)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float o = __shfl_xor(acc[c], 1, 64);
            acc[c] = (part & 1) ? o + acc[c] : acc[c] + o;
            if (tpo == 4) {
                o = __shfl_xor(acc[c], 2, 64);
                acc[c] = (part & 2) ? o + acc[c] : acc[c] + o;
            }
        }
        if (part == 0) {
            const size_t ob = attn_out_row(a, u, win.row0 + row) * D + d;
            float r[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) r[c] = L > 0.f ? acc[c] / L : 0.f;
            store4<DT>(a.out, ob, r);
        }
    }
}

// The new token of unit u's request joins the item's final state: one more
// key for every row (an online-softmax step in the log2 domain: z = scale *
// log2(e) * q.k), then its K row and V column go into the active tile, and a
// block it completes gets its summary (min / max over the B-1 stored rows and
// the token, as oasis_append_kv computes it; the scan of this launch does not
// read it, the block being the active one).  Inputs come from the item's
// TokStage.  Wave w owns rows w, w+4, ...; the state update touches LDS only,
// so an LDS barrier orders it before the output, and the stores are left in
// flight (a full barrier would wait for them).
template <int DT, int D>
__device__ void attn_new_token(const StepArgs& a, int u, const AttnFin& F, const TokStage& ts) {
    using E = typename Elem<DT>::type;
    if (!ts.active) return;
    constexpr int PL = (D + 63) / 64;  // dims per lane
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    constexpr int RW = kMaxRows / (kNT / 64);  // rows per wave at most
    const int b = ts.blk, t = ts.slot;
    const size_t tile = ((size_t)u * a.unit_stride + b) * (size_t)a.tile_stride;
    float kx[PL], vx[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int d = lane + 64 * i;
        kx[i] = d < D ? load_elem<DT>(ts.k, d) : 0.f;
        vx[i] = d < D ? load_elem<DT>(ts.v, d) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int row = w + k * (kNT / 64);
        if (row >= a.NR) break;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int d = lane + 64 * i;
            if (d < D) part = fmaf(load_elem<DT>(ts.q, (size_t)row * D + d), kx[i], part);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        const float z = part * a.scale_log2;
        const float mo = F.m[row], lo = F.l[row];
        const float M = fmaxf(mo, z);
        const float cf = (mo == -__builtin_inff()) ? 0.f : exp2f(mo - M);
        const float pz = exp2f(z - M);
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int d = lane + 64 * i;
            if (d < D) F.acc[(size_t)row * D + d] = fmaf(F.acc[(size_t)row * D + d], cf, pz * vx[i]);
        }
        if (lane == 0) {
            F.m[row] = M;
            F.l[row] = fmaf(lo, cf, pz);
        }
    }
    lds_barrier();
    // The token's K row and V column go into its tile from the staged copies
    // (the same elements as k_new / v_new; no load after the loop).
    for (int d = threadIdx.x; d < D; d += kNT) {
        const float knew = load_elem<DT>(ts.k, d);
        reinterpret_cast<E*>(a.kt_w)[tile + (size_t)t * D + d] = reinterpret_cast<const E*>(ts.k)[d];
        reinterpret_cast<E*>(a.vt_w)[tile + (size_t)d * a.B + t] = reinterpret_cast<const E*>(ts.v)[d];
        if (ts.summ) {
            float lo = knew, hi = knew;
            for (int j = 0; j < a.B - 1; ++j) {
                const float x = ts.summ == 1 ? load_elem<DT>(ts.rows, (size_t)j * D + d)
                                             : load_elem<DT>(a.kt, tile + (size_t)j * D + d);
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
            const size_t so = ((size_t)u * a.n_blk_max + b) * 2 * D + d;
            store_elem<DT>(a.summ_w, so, lo);
            store_elem<DT>(a.summ_w, so + D, hi);
        }
    }
}

template <int DT, int D, int ATT, int NRG, bool TOK>
__device__ void attn_item(const StepArgs& a, int u, int sp, int grp, unsigned char* lds) {
    LdsCursor cur{lds};
    const RowWin win = row_win(a, grp);
    int* tbl = cur.take<int>(a.per_split > 0 ? a.per_split : 1);
    AttnFin F;  // the item's rows (attn_lds_bytes sizes LDS for them)
    F.m = cur.take<float>(win.nr);
    F.l = cur.take<float>(win.nr);
    F.acc = cur.take<float>((size_t)win.nr * D);
    TokStage ts{};
    if constexpr (ATT == kAttnMfma) {
        // stages the table (and the token) after loading q
        ts = attn_item_mfma<D, NRG, TOK>(a, u, sp, win, cur, F, tbl);
    } else {
        if constexpr (TOK) ts = tok_prefetch<DT, D>(a, u, sp, cur);
        const SplitRange sr = split_range<TOK>(a, u, sp);
        for (int i = threadIdx.x; i < sr.e1 - sr.e0; i += kNT)
            tbl[i] = a.table[(size_t)u * a.n_sel + sr.e0 + i];
        __syncthreads();
        attn_item_valu<DT, D, TOK>(a, u, sp, cur, F, tbl);
    }
    if constexpr (TOK) attn_new_token<DT, D>(a, u, F, ts);
    attn_emit<DT, D>(a, u, sp, win, F);
}

// ============================================================ the kernels
// Main launch.  Roles present are fixed at compile time (SCAN, ATT !=
// kAttnNone); the number of items per unit of each role comes from the
// arguments.
template <int DT, int D, int NQ, int ATT, int NRG, bool SCAN, bool TOK = false>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(NRG == 1 ? 2 : 1))) step_kernel(StepArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int w = blockIdx.x;
    const int x = w & 7;
    int k = w >> 3;
    const int nu = a.U > x ? (a.U - x + 7) / 8 : 0;  // units on this XCD
    if constexpr (SCAN) {
        const int ns = nu * a.scan_items;
        if (k < ns) {
            const int i = k / a.scan_items, c = k - (k / a.scan_items) * a.scan_items;
            scan_item<DT, D, NQ>(a, x + 8 * i, c, lds);
            return;
        }
        k -= ns;
    }
    if constexpr (ATT != kAttnNone) {
        if (k < nu * a.attn_items) {
            const int i = k / a.attn_items, s = k - (k / a.attn_items) * a.attn_items;
            // a split's row groups are adjacent items (same tiles, same XCD)
            const int sp = a.RGN > 1 ? s / a.RGN : s, grp = a.RGN > 1 ? s - sp * a.RGN : 0;
            attn_item<DT, D, ATT, NRG, TOK>(a, x + 8 * i, sp, grp, lds);
        }
    }
}

// A split unit's score row is staged in LDS (padded) for its selection up to
// this size.
__host__ __device__ inline bool finish_scores_in_lds(int n_blk_max) {
    return (size_t)n_blk_max * 4 <= kScoreLdsMax;
}
__host__ __device__ inline size_t finish_scores_lds(int n_blk_max) {
    return finish_scores_in_lds(n_blk_max) ? (size_t)n_blk_max + kNT : 0;
}

// Second launch for split units: top-K (+ plan) from the global scores when
// NC > 1 (`select` items, one per unit and scored row), LSE merge of the
// attention partials when S > 1 (`merge` items, one per unit and row group).
// Same XCD mapping as the main launch.  NT = kFinishNT when every row fits
// in registers (n_blk_max <= kSelRowMax), else kNT (rows staged or re-read).
template <int DT, int D, int NQ, int NT>
__global__ void __launch_bounds__(NT) finish_kernel(StepArgs a, int select_items, int merge_items) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int w = blockIdx.x;
    const int x = w & 7;
    int k = w >> 3;
    const int nu = a.U > x ? (a.U - x + 7) / 8 : 0;
    LdsCursor cur{lds};
    if (select_items) {
        // One item per (unit, scored row): the row's NT threads hold its keys;
        // the item of row pred_row also plans the unit.
        if (k < nu * NQ) {
            const int u = x + 8 * (k / NQ), j = k - (k / NQ) * NQ;
            const int K4 = pad4(a.K);
            const bool plan = a.do_plan && j == a.pred_row;
            const int r = u / a.H, g = u - (u / a.H) * a.H;
            const float* gsc = a.scores + (((size_t)r * NQ + j) * a.H + g) * a.n_blk_max;
            const int n_r = a.n_blk ? min(max(a.n_blk[r], 0), a.n_blk_max) : a.n_blk_max;
            const size_t ors = (size_t)a.H * a.K;
            const size_t ob = (((size_t)r * NQ + j) * a.H + g) * a.K;
            int* P = cur.take<int>(K4);
            PlanLds Pl = carve_plan(cur, K4);
            if constexpr (NT != kNT) {
                // The slot tables' loads, then the scores' (all in flight).
                carve_plan_fast(cur, K4, a.n_blk_max, Pl);
                const SelLds S = carve_sel(cur);
                if (plan)
                    plan_load<NT>(a.slot_blk_in + (size_t)u * a.K, a.slot_stamp_in + (size_t)u * a.K,
                                  a.K, Pl);
                uint32_t key[kSelRowMax / NT];
                sel_load<NT>(gsc, n_r, key);
                int32_t* oi = a.topk_idx + ob;
                float* os = a.topk_score ? a.topk_score + ob : nullptr;
                if (plan)  // the slot order and resident marks ride in the selection's first phase
                    select_row<NT>(key, n_r, a.K, oi, os, P, S, PlanOrderHook<NT>{Pl, a.K, a.n_blk_max},
                                   Pl.mark_p);
                else
                    select_row<NT>(key, n_r, a.K, oi, os, nullptr, S);
                if (plan) {
                    const size_t so = (size_t)u * a.K;
                    plan_unit<true, NT>(P, a.K, a.slot_blk_out + so, a.slot_stamp_out + so, a.step, a.cap,
                                    a.ins_blk ? a.ins_blk[r] : -1, a.plan_count + u, a.plan_src + so,
                                    a.plan_dst + so, a.plan_evicted ? a.plan_evicted + so : nullptr,
                                    Pl, a.n_blk_max);
                }
                return;
            } else {
            if (plan)
                plan_load(a.slot_blk_in + (size_t)u * a.K, a.slot_stamp_in + (size_t)u * a.K, a.K, Pl);
            {
                TopkLds T = carve_topk(cur, 1, K4);
                T.P = P;
                T.ek = cur.take<unsigned long long>(K4);
                const float* lsc_row = nullptr;
                bool padded = false;
                if (finish_scores_in_lds(a.n_blk_max)) {
                    // The row goes to LDS in coalesced loads, padded for the
                    // selection's conflict-free loads of every key into registers.
                    const int per = max(1, (n_r + kNT - 1) / kNT);
                    float* lsc = cur.take<float>((size_t)a.n_blk_max + kNT);
                    if ((a.n_blk_max & 3) == 0 && (reinterpret_cast<uintptr_t>(gsc) & 15) == 0) {
                        // 16-byte loads, kStageVec of them in flight per thread
                        const int n4 = (n_r + 3) >> 2;
                        const float4* g4 = reinterpret_cast<const float4*>(gsc);
                        for (int i0 = 0; i0 < n4; i0 += kStageVec * kNT) {
                            float4 v[kStageVec];
#pragma unroll
                            for (int e = 0; e < kStageVec; ++e) {
                                const int i = i0 + e * kNT + threadIdx.x;
                                if (i < n4) v[e] = g4[i];
                            }
#pragma unroll
                            for (int e = 0; e < kStageVec; ++e) {
                                const int i = i0 + e * kNT + threadIdx.x;
                                if (i < n4) {
                                    const float f[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
                                    for (int c = 0; c < 4; ++c) {
                                        const int bb = 4 * i + c;
                                        if (bb < n_r) lsc[bb + bb / per] = f[c];
                                    }
                                }
                            }
                        }
                    } else {
#pragma unroll 8
                        for (int i = threadIdx.x; i < n_r; i += kNT) lsc[i + i / per] = gsc[i];
                    }
                    __syncthreads();
                    lsc_row = lsc;
                    padded = true;
                }
                // one call site (rows this long are rare): the row is read
                // through generic addresses, LDS or global
                topk_rows<1, kFinishKPT, true>(padded ? lsc_row : gsc, 0, n_r, a.K, a.topk_idx + ob,
                                               a.topk_score ? a.topk_score + ob : nullptr, ors,
                                               plan ? 0 : -1, T, padded);
            }
            if (plan) {
                const size_t so = (size_t)u * a.K;
                plan_unit(P, a.K, a.slot_blk_out + so, a.slot_stamp_out + so, a.step, a.cap,
                          a.ins_blk ? a.ins_blk[r] : -1, a.plan_count + u, a.plan_src + so,
                          a.plan_dst + so, a.plan_evicted ? a.plan_evicted + so : nullptr, Pl);
            }
            return;
            }
        }
        k -= nu * NQ;
    }
    if (merge_items && k < nu * a.RGN) {
        float* Mr = cur.take<float>(kMaxRows);
        float* Lr = cur.take<float>(kMaxRows);
        float* red = cur.take<float>(NT);
        float* W = cur.take<float>(kMergeW);
        const int i = k / a.RGN, grp = k - (k / a.RGN) * a.RGN;
        attn_merge_unit<DT, D, NT>(a, x + 8 * i, row_win(a, grp), Mr, Lr, red, W);
    }
}

// LDS of finish_kernel: a select item's top-K and plan state (+ its score row
// when finish_scores_in_lds), a merge item's reduction buffers.
__host__ __device__ inline size_t finish_lds_bytes(int K, int n_blk_max, bool sel, int nt) {
    const size_t m = 2 * 16 * ((kMaxRows * 4 + 15) / 16) + (size_t)nt * 4 + kMergeW * 4;
    if (!sel) return m;
    const size_t p = ((size_t)pad4(K) * 4 + 15) / 16 * 16 + plan_lds_size(K);  // P, plan
    const size_t s = p + (n_blk_max <= kSelRowMax
                              ? plan_fast_lds_size(K, n_blk_max) + sel_lds_bytes()
                              : scan_lds_bytes(1, 0, K, (int)finish_scores_lds(n_blk_max)) +
                                    ((size_t)pad4(K) * 8 + 15) / 16 * 16);  // top-K state, rank keys
    return s > m ? s : m;
}

// ============================================================ host helpers
struct StepPlan {
    int NC, chunk, S, per_split;
};

constexpr int kMinSplitTiles = 8;     // automatic split: tiles per attention item at least
constexpr int kMinChunkBlocks = 256;  // automatic split: blocks per scan item at least

// Items per unit.  With at least 256 units (one per CU) every unit gets one
// scan item and one attention item: no partials, one launch.  Smaller batches
// split units until about 512 main workgroups (two per CU) are in flight:
// the attention takes its share of the items by bytes (at least kMinSplitTiles
// tiles per split), the scan the items left (at least kMinChunkBlocks blocks
// each; below these an item's fixed costs outweigh its share of the stream);
// the split units then take a second, small launch.
// With rgn row groups every split is rgn items, each reading the split's tiles.
inline StepPlan plan_items(int U, int n_blk_max, int n_sel, int D, int B, int eb, bool scan,
                           bool attn, int want_nc, int want_s, int rgn = 1) {
    StepPlan p{0, 0, 0, 0};
    const double scan_b = scan ? (double)n_blk_max * 2 * D * eb : 0.0;
    const double attn_b = attn ? (double)n_sel * 2 * B * D * eb * rgn : 0.0;
    const int items = U >= 256 ? (scan ? 1 : 0) + (attn ? 1 : 0) : (511 + U) / U;
    const double tot = scan_b + attn_b > 0 ? scan_b + attn_b : 1.0;
    if (attn) {
        int s = want_s > 0 ? want_s : (U >= 256 ? 1 : (int)(items * attn_b / tot / rgn + 0.5));
        if (want_s <= 0 && s > (n_sel + kMinSplitTiles - 1) / kMinSplitTiles)
            s = (n_sel + kMinSplitTiles - 1) / kMinSplitTiles;
        const int min_s = (n_sel + kMaxSplitEntries - 1) / kMaxSplitEntries;
        if (s < min_s) s = min_s;
        if (n_sel > 0 && s > n_sel) s = n_sel;
        if (s < 1) s = 1;
        const int per = n_sel > 0 ? (n_sel + s - 1) / s : 0;
        p.per_split = per;
        p.S = per > 0 ? (n_sel + per - 1) / per : 1;
    }
    if (scan) {
        // the scan takes the items the attention leaves (all items fit at once)
        const int left = items - (attn ? p.S * rgn : 0);
        int nc = want_nc > 0 ? want_nc
                             : (U >= 256 ? 1 : (attn ? left : (int)(items * scan_b / tot + 0.5)));
        const int max_nc = want_nc > 0 ? n_blk_max : (n_blk_max + kMinChunkBlocks - 1) / kMinChunkBlocks;
        if (nc > max_nc) nc = max_nc;
        if (nc < 1) nc = 1;
        const int chunk = (n_blk_max + nc - 1) / nc;
        p.chunk = chunk;
        p.NC = (n_blk_max + chunk - 1) / chunk;
    }
    return p;
}

}  // namespace oasis
