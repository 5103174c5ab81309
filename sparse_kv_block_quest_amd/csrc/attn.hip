// Paged GQA decode attention of the stacked normal + draft query rows over the
// resident selected tiles plus the active local block, split-K with an LSE
// merge.
//
// Sources: OasisKV paperpeel v2 text, §3.1 and Fig. 6 (one attention call over
// one resident working set returns the outputs of both stacked queries) and
// §4.1 (each head also attends its active local block: K + 1 blocks).
//
// Work split: one workgroup per (split, KV head, request).  A split owns a
// contiguous range of the unit's tile table (the last split also owns the
// active block).  Its 4 waves share the split's 16-token sub-tiles round
// robin, each keeping an online softmax (running max in the log2 domain, sum,
// output accumulator) for all n_q*G rows of the unit; the waves are combined
// in LDS and the split's partial (max, sum, acc) goes to the workspace.
// attn_merge_kernel then combines the splits of every row in split order.
//
// Two split kernels:
//  - attn_split_mfma (bf16, B a multiple of 16): per sub-tile,
//    S^T[16 tok][16 rows] = K_sub[16][D] * Q^T via v_mfma_f32_16x16x32_bf16
//    (K rows straight from HBM into the A operand, q held in registers), then
//    O^T[D][rows] += V^T * P^T via v_mfma_f32_16x16x16_bf16, whose A operand is
//    4 consecutive tokens of one dim: contiguous because V tiles are stored
//    dim-major [D][B].  P is rounded to bf16 for the product.
//  - attn_split_valu (any dtype / B): K and V sub-tiles staged in LDS as fp32,
//    scalar FMAs.  Used for fp32 and for block sizes below 16.
#include "oasis_internal.h"

namespace oasis {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
    const uint8_t* q;
    const uint8_t* kt;
    const uint8_t* vt;
    const int32_t* table;
    const int32_t* tail_tile;
    const int32_t* tail_len;
    float* ws_ml;   // [U][S][NR][2]  (max in log2 domain, sum)
    float* ws_acc;  // [U][S][NR][D]
    long long unit_stride;
    int n_sel;
    int Hq, H, G, NQ, NR, B;
    int n_split, per_split;
    float scale_log2;
};

// Sub-tile list of one split: table entries [e0, e1) contribute B/ST sub-tiles
// each, the active block (last split only) ceil(tail/ST).
struct SplitRange {
    int e0, e1, tail_tile, tail_len, n_sub, sub_per_entry;
};

template <int ST>
__device__ __forceinline__ SplitRange split_range(const AttnArgs& a, size_t u, int r, int sp) {
    SplitRange s;
    s.e0 = min(sp * a.per_split, a.n_sel);
    s.e1 = min(s.e0 + a.per_split, a.n_sel);
    s.sub_per_entry = a.B / ST;
    s.tail_tile = -1;
    s.tail_len = 0;
    if (sp == a.n_split - 1 && a.tail_tile && a.tail_len) {
        const int tt = a.tail_tile[u];
        const int tl = min(a.tail_len[r], a.B);
        if (tt >= 0 && tl > 0) {
            s.tail_tile = tt;
            s.tail_len = tl;
        }
    }
    s.n_sub = (s.e1 - s.e0) * s.sub_per_entry + (s.tail_len + ST - 1) / ST;
    return s;
}

// --------------------------------------------------------------- MFMA path
template <int D, int NRG>
__global__ void __launch_bounds__(256) attn_split_mfma(AttnArgs a) {
    constexpr int KB = D / 32;  // QK MFMAs per sub-tile and row group
    constexpr int DB = D / 16;  // PV MFMAs per sub-tile and row group
    extern __shared__ float lds[];
    const int sp = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const size_t u = (size_t)r * a.H + g;
    const int B = a.B;

    bf16x8_t qv[NRG][KB];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        const int row = rg * 16 + l16;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qv[rg][kb] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        if (row < a.NR) {
            const int j = row / a.G, hh = row % a.G;
            const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(
                a.q + ((((size_t)r * a.NQ + j) * a.Hq + (size_t)g * a.G + hh) * D) * 2);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qv[rg][kb] = qp[kb * 4 + lg];
        }
    }
    float m[NRG], lsum[NRG];
    f32x4_t acc[NRG][DB];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        m[rg] = -__builtin_inff();
        lsum[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const SplitRange sr = split_range<16>(a, u, r, sp);
    const int n_entry_sub = (sr.e1 - sr.e0) * sr.sub_per_entry;
    const size_t tile_elems = (size_t)B * D;
    for (int st = w; st < sr.n_sub; st += 4) {
        int tile, sub, ntok;
        if (st < n_entry_sub) {
            tile = a.table[u * a.n_sel + sr.e0 + st / sr.sub_per_entry];
            sub = st % sr.sub_per_entry;
            ntok = 16;
            if (tile < 0) continue;
        } else {
            tile = sr.tail_tile;
            sub = st - n_entry_sub;
            ntok = min(16, sr.tail_len - sub * 16);
        }
        const size_t tid64 = (size_t)(u * a.unit_stride + tile);
        const uint8_t* kbase = a.kt + (tid64 * tile_elems + (size_t)sub * 16 * D) * 2;
        const uint8_t* vbase = a.vt + (tid64 * tile_elems + (size_t)sub * 16) * 2;
        bf16x8_t kv[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            kv[kb] = *reinterpret_cast<const bf16x8_t*>(kbase + ((size_t)l16 * D + kb * 32 + lg * 8) * 2);
        bf16x4_t vv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
            vv[db] = *reinterpret_cast<const bf16x4_t*>(vbase + ((size_t)(db * 16 + l16) * B + lg * 4) * 2);
        if (ntok < 16) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lg * 4 + e >= ntok) vv[db][e] = 0;
        }
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg) {
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[kb], qv[rg][kb], s, 0, 0, 0);
            // s[e] = scaled score of token lg*4+e for row l16.
            float tmax = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[e] = (lg * 4 + e < ntok) ? s[e] * a.scale_log2 : -__builtin_inff();
                tmax = fmaxf(tmax, s[e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mnew = fmaxf(m[rg], tmax);
            const float corr = exp2f(m[rg] - mnew);
            float p[4];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2f(s[e] - mnew);
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
                acc[rg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv[db], pb, acc[rg][db], 0, 0, 0);
            }
        }
    }
    // Row sums: the 4 lane groups hold disjoint tokens of the same rows.
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
        lsum[rg] += __shfl_xor(lsum[rg], 16, 64);
        lsum[rg] += __shfl_xor(lsum[rg], 32, 64);
    }
    // Combine the 4 waves: waves 1..3 park their state in LDS, wave 0 merges.
    const int NR = a.NR;
    float* lm = lds;                    // [3][NR]
    float* ll = lds + 3 * NR;           // [3][NR]
    float* la = lds + 6 * NR;           // [3][NR][D]
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
    if (w != 0) return;
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
        float L = lsum[rg] * f0;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            fk[k] = (mw[k] == -__builtin_inff()) ? 0.f : exp2f(mw[k] - M);
            L += ll[k * NR + row] * fk[k];
        }
        const size_t prow = (u * a.n_split + sp) * NR + row;
        if (lg == 0) {
            a.ws_ml[prow * 2 + 0] = M;
            a.ws_ml[prow * 2 + 1] = L;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            f32x4_t o = acc[rg][db] * f0;
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] += fk[k] * la[((size_t)k * NR + row) * D + db * 16 + lg * 4 + e];
            *reinterpret_cast<f32x4_t*>(a.ws_acc + prow * D + db * 16 + lg * 4) = o;
        }
    }
}

// --------------------------------------------------------------- VALU path
constexpr int kValuRows = 32;

template <int DT, int D>
__global__ void __launch_bounds__(256) attn_split_valu(AttnArgs a) {
    constexpr int ST = 16;                      // tokens per staged sub-tile
    constexpr int OPT = kValuRows * D / 256;    // outputs per thread (upper bound)
    __shared__ float qs[kValuRows][D];
    __shared__ float ks[ST][D + 1];
    __shared__ float vs[D][ST + 1];
    __shared__ float ps[kValuRows][ST];
    __shared__ float m_s[kValuRows], l_s[kValuRows], c_s[kValuRows];
    const int sp = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x;
    const size_t u = (size_t)r * a.H + g;
    const int NR = a.NR, B = a.B;
    for (int i = tid; i < NR * D; i += 256) {
        const int row = i / D, d = i % D;
        const int j = row / a.G, hh = row % a.G;
        qs[row][d] = load_elem<DT>(a.q, (((size_t)r * a.NQ + j) * a.Hq + (size_t)g * a.G + hh) * D + d) *
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

    const int sub_tokens = B < ST ? B : ST;
    const int spe = B / sub_tokens;
    const int e0 = min(sp * a.per_split, a.n_sel);
    const int e1 = min(e0 + a.per_split, a.n_sel);
    int tail_tile = -1, tail_len = 0;
    if (sp == a.n_split - 1 && a.tail_tile && a.tail_len) {
        const int tt = a.tail_tile[u];
        const int tl = min(a.tail_len[r], B);
        if (tt >= 0 && tl > 0) {
            tail_tile = tt;
            tail_len = tl;
        }
    }
    const int n_entry_sub = (e1 - e0) * spe;
    const int n_sub = n_entry_sub + (tail_len + sub_tokens - 1) / sub_tokens;
    const size_t tile_elems = (size_t)B * D;
    for (int st = 0; st < n_sub; ++st) {
        int tile, sub, nt;
        if (st < n_entry_sub) {
            tile = a.table[u * a.n_sel + e0 + st / spe];
            sub = st % spe;
            nt = sub_tokens;
            if (tile < 0) continue;
        } else {
            tile = tail_tile;
            sub = st - n_entry_sub;
            nt = min(sub_tokens, tail_len - sub * sub_tokens);
        }
        const size_t base = (size_t)(u * a.unit_stride + tile) * tile_elems;
        const int t0 = sub * sub_tokens;
        for (int i = tid; i < nt * D; i += 256) {
            const int tt = i / D, d = i % D;
            ks[tt][d] = load_elem<DT>(a.kt, base + (size_t)(t0 + tt) * D + d);
        }
        for (int i = tid; i < D * nt; i += 256) {
            const int d = i / nt, tt = i % nt;
            vs[d][tt] = load_elem<DT>(a.vt, base + (size_t)d * B + t0 + tt);
        }
        __syncthreads();
        for (int p = tid; p < NR * ST; p += 256) {
            const int row = p / ST, tt = p % ST;
            float z = -__builtin_inff();
            if (tt < nt) {
                z = 0.f;
                for (int d = 0; d < D; ++d) z = fmaf(qs[row][d], ks[tt][d], z);
            }
            ps[row][tt] = z;
        }
        __syncthreads();
        if (tid < NR) {
            float mx = m_s[tid];
            for (int tt = 0; tt < nt; ++tt) mx = fmaxf(mx, ps[tid][tt]);
            const float corr = exp2f(m_s[tid] - mx);
            float sum = 0.f;
            for (int tt = 0; tt < nt; ++tt) {
                const float pv = exp2f(ps[tid][tt] - mx);
                ps[tid][tt] = pv;
                sum += pv;
            }
            l_s[tid] = l_s[tid] * corr + sum;
            m_s[tid] = mx;
            c_s[tid] = corr;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < OPT; ++k) {
            const int o = tid + k * 256;
            if (o < NR * D) {
                const int row = o / D, d = o % D;
                float v = acc[k] * c_s[row];
                for (int tt = 0; tt < nt; ++tt) v = fmaf(ps[row][tt], vs[d][tt], v);
                acc[k] = v;
            }
        }
        __syncthreads();
    }
    const size_t pbase = (u * a.n_split + sp) * NR;
    if (tid < NR) {
        a.ws_ml[(pbase + tid) * 2 + 0] = m_s[tid];
        a.ws_ml[(pbase + tid) * 2 + 1] = l_s[tid];
    }
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
        const int o = tid + k * 256;
        if (o < NR * D) a.ws_acc[pbase * D + o] = acc[k];
    }
}

// -------------------------------------------------------------- LSE merge
// One wave per output row (r, j, h); 4 rows per workgroup.  Splits are
// combined in split order.
template <int DT, int D>
__global__ void __launch_bounds__(256)
attn_merge_kernel(const float* __restrict__ ws_ml, const float* __restrict__ ws_acc, int n_rows,
                  int NQ, int Hq, int H, int G, int NR, int S, void* __restrict__ out,
                  float* __restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int row_id = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row_id >= n_rows) return;
    const int h = row_id % Hq;
    const int j = (row_id / Hq) % NQ;
    const int r = row_id / (Hq * NQ);
    const int g = h / G;
    const int nr = j * G + (h - g * G);
    const size_t u = (size_t)r * H + g;
    float M = -__builtin_inff();
    for (int s = 0; s < S; ++s) M = fmaxf(M, ws_ml[((u * S + s) * NR + nr) * 2]);
    constexpr int PER = D / 64;
    float o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = 0.f;
    float L = 0.f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < S; ++s) {
            const size_t pr = (u * S + s) * NR + nr;
            const float ms = ws_ml[pr * 2];
            if (ms == -__builtin_inff()) continue;
            const float f = exp2f(ms - M);
            L += f * ws_ml[pr * 2 + 1];
#pragma unroll
            for (int k = 0; k < PER; ++k) o[k] = fmaf(f, ws_acc[pr * D + lane + 64 * k], o[k]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t ob = (size_t)row_id * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) store_elem<DT>(out, ob + lane + 64 * k, o[k] * inv);
    if (lse && lane == 0) lse[row_id] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -__builtin_inff();
}

// ------------------------------------------------------------------ host
enum { kImplAuto = 0, kImplValu = 1, kImplMfma = 2 };

static void attn_split_plan(long long units, int n_sel, int B, int* S_out, int* per_out) {
    if (n_sel <= 0) {
        *S_out = 1;
        *per_out = 0;
        return;
    }
    const int spe = B >= 16 ? B / 16 : 1;
    const long long total_sub = (long long)n_sel * spe;
    long long S = (total_sub + 31) / 32;
    const long long S_max = total_sub >= 4 ? total_sub / 4 : 1;
    if (S < 1) S = 1;
    while (S < S_max && units * S < 1024) S = S * 2 < S_max ? S * 2 : S_max;
    if (S > n_sel) S = n_sel;
    const int per = (int)((n_sel + S - 1) / S);
    *per_out = per;
    *S_out = (n_sel + per - 1) / per;
}

}  // namespace oasis

using namespace oasis;

static int attn_check(const oasis_shape* s, int32_t n_sel) {
    int st = check_shape(s);
    if (st != OASIS_OK) return st;
    if (n_sel < 0) return OASIS_EINVAL;
    const int G = s->n_q_heads / s->n_kv_heads;
    if (s->n_q * G > 32) return OASIS_EUNSUPPORTED;
    return OASIS_OK;
}

extern "C" size_t oasis_sparse_attn_workspace(const oasis_shape* s, int32_t n_sel) {
    if (attn_check(s, n_sel) != OASIS_OK) return 0;
    const long long units = (long long)s->batch * s->n_kv_heads;
    int S, per;
    attn_split_plan(units, n_sel, s->block_size, &S, &per);
    const int NR = s->n_q * (s->n_q_heads / s->n_kv_heads);
    const size_t rows = (size_t)units * S * NR;
    return align_up(rows * 2 * sizeof(float), 256) + align_up(rows * s->head_dim * sizeof(float), 256);
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
    if (impl < kImplAuto || impl > kImplMfma) return OASIS_EINVAL;
    const size_t need = oasis_sparse_attn_workspace(s, n_sel);
    if (!workspace || workspace_bytes < need) return OASIS_EWORKSPACE;
    const int R = s->batch, H = s->n_kv_heads, Hq = s->n_q_heads, D = s->head_dim;
    const int B = s->block_size, G = Hq / H, NR = s->n_q * G;
    const long long units = (long long)R * H;
    int S, per;
    attn_split_plan(units, n_sel, B, &S, &per);
    const bool mfma_ok = s->dtype == OASIS_BF16 && B % 16 == 0;
    bool use_mfma = impl == kImplAuto ? mfma_ok : impl == kImplMfma;
    if (use_mfma && !mfma_ok) return OASIS_EUNSUPPORTED;

    AttnArgs a;
    a.q = reinterpret_cast<const uint8_t*>(q);
    a.kt = reinterpret_cast<const uint8_t*>(k_tiles);
    a.vt = reinterpret_cast<const uint8_t*>(v_tiles);
    a.table = tile_table;
    a.tail_tile = tail_tile;
    a.tail_len = tail_len;
    const size_t rows = (size_t)units * S * NR;
    a.ws_ml = reinterpret_cast<float*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                        align_up(rows * 2 * sizeof(float), 256));
    a.unit_stride = unit_stride;
    a.n_sel = n_sel;
    a.Hq = Hq;
    a.H = H;
    a.G = G;
    a.NQ = s->n_q;
    a.NR = NR;
    a.B = B;
    a.n_split = S;
    a.per_split = per;
    const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
    a.scale_log2 = sc * kLog2e;

    dim3 grid(S, H, R);
    if (use_mfma) {
        const size_t lds = (size_t)(6 * NR + 3 * NR * D) * sizeof(float);
        if (NR <= 16) {
            if (D == 64) hipLaunchKernelGGL((attn_split_mfma<64, 1>), grid, dim3(256), lds, stream, a);
            else hipLaunchKernelGGL((attn_split_mfma<128, 1>), grid, dim3(256), lds, stream, a);
        } else {
            if (D == 64) hipLaunchKernelGGL((attn_split_mfma<64, 2>), grid, dim3(256), lds, stream, a);
            else hipLaunchKernelGGL((attn_split_mfma<128, 2>), grid, dim3(256), lds, stream, a);
        }
    } else {
        if (s->dtype == OASIS_F32) {
            if (D == 64) hipLaunchKernelGGL((attn_split_valu<OASIS_F32, 64>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((attn_split_valu<OASIS_F32, 128>), grid, dim3(256), 0, stream, a);
        } else {
            if (D == 64) hipLaunchKernelGGL((attn_split_valu<OASIS_BF16, 64>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((attn_split_valu<OASIS_BF16, 128>), grid, dim3(256), 0, stream, a);
        }
    }
    const int n_rows = R * s->n_q * Hq;
    dim3 mgrid((n_rows + 3) / 4);
    if (s->dtype == OASIS_F32) {
        if (D == 64) hipLaunchKernelGGL((attn_merge_kernel<OASIS_F32, 64>), mgrid, dim3(256), 0, stream, a.ws_ml, a.ws_acc, n_rows, s->n_q, Hq, H, G, NR, S, out, lse);
        else hipLaunchKernelGGL((attn_merge_kernel<OASIS_F32, 128>), mgrid, dim3(256), 0, stream, a.ws_ml, a.ws_acc, n_rows, s->n_q, Hq, H, G, NR, S, out, lse);
    } else {
        if (D == 64) hipLaunchKernelGGL((attn_merge_kernel<OASIS_BF16, 64>), mgrid, dim3(256), 0, stream, a.ws_ml, a.ws_acc, n_rows, s->n_q, Hq, H, G, NR, S, out, lse);
        else hipLaunchKernelGGL((attn_merge_kernel<OASIS_BF16, 128>), mgrid, dim3(256), 0, stream, a.ws_ml, a.ws_acc, n_rows, s->n_q, Hq, H, G, NR, S, out, lse);
    }
    return launch_status();
}

extern "C" int oasis_sparse_attn(const oasis_shape* s, const void* q, const void* k_tiles,
                                 const void* v_tiles, const int32_t* tile_table, int32_t n_sel,
                                 int64_t unit_stride, const int32_t* tail_tile,
                                 const int32_t* tail_len, float scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return oasis_sparse_attn_impl(s, q, k_tiles, v_tiles, tile_table, n_sel, unit_stride, tail_tile,
                                  tail_len, scale, out, lse, workspace, workspace_bytes, kImplAuto,
                                  stream);
}
