// Internal helpers shared by the gfx950 kernels of liboasis.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oasis.h"

namespace oasis {

// ---------------------------------------------------------------- elements
template <int DT>
struct Elem;
template <>
struct Elem<OASIS_F32> {
    static constexpr int bytes = 4;
    using type = uint32_t;  // raw bits of one element
};
template <>
struct Elem<OASIS_BF16> {
    static constexpr int bytes = 2;
    using type = uint16_t;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Loads of data a launch reads exactly once (summaries, K and V tiles):
// non-temporal, so the lines stream through the caches instead of being kept
// as if they would be reused.  On this part that raised the fused step's
// streaming rate by about 7% against ordinary loads (same values, cache
// policy only).
template <class T>
__device__ __forceinline__ T load_stream(const T* p) {
    return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// Widen the 16 bytes of `v` into 16/bytes floats (exact).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
    if constexpr (DT == OASIS_F32) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    } else {
        out[0] = bf16_lo(v.x);
        out[1] = bf16_hi(v.x);
        out[2] = bf16_lo(v.y);
        out[3] = bf16_hi(v.y);
        out[4] = bf16_lo(v.z);
        out[5] = bf16_hi(v.z);
        out[6] = bf16_lo(v.w);
        out[7] = bf16_hi(v.w);
    }
}

// Narrow 16/bytes floats that are exactly representable back into 16 bytes.
template <int DT>
__device__ __forceinline__ uint4 pack16_exact(const float* in) {
    uint4 v;
    if constexpr (DT == OASIS_F32) {
        v.x = __float_as_uint(in[0]);
        v.y = __float_as_uint(in[1]);
        v.z = __float_as_uint(in[2]);
        v.w = __float_as_uint(in[3]);
    } else {
        v.x = (__float_as_uint(in[0]) >> 16) | (__float_as_uint(in[1]) & 0xffff0000u);
        v.y = (__float_as_uint(in[2]) >> 16) | (__float_as_uint(in[3]) & 0xffff0000u);
        v.z = (__float_as_uint(in[4]) >> 16) | (__float_as_uint(in[5]) & 0xffff0000u);
        v.w = (__float_as_uint(in[6]) >> 16) | (__float_as_uint(in[7]) & 0xffff0000u);
    }
    return v;
}

// Load one element as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
    if constexpr (DT == OASIS_F32) {
        return reinterpret_cast<const float*>(base)[i];
    } else {
        return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[i]) << 16);
    }
}

// Store one float as an element (bf16: round to nearest even).
template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t i, float f) {
    if constexpr (DT == OASIS_F32) {
        reinterpret_cast<float*>(base)[i] = f;
    } else {
        reinterpret_cast<uint16_t*>(base)[i] = uint16_t(f32_to_bf16_bits(f));
    }
}

// Four consecutive elements from element i (i a multiple of 4): one vector
// store when the address allows it, else four.
template <int DT>
__device__ __forceinline__ void store4(void* base, size_t i, const float (&f)[4]) {
    if constexpr (DT == OASIS_F32) {
        float* p = reinterpret_cast<float*>(base) + i;
        if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
            *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
            return;
        }
    } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(base) + i;
        if ((reinterpret_cast<uintptr_t>(p) & 7) == 0) {
            const uint32_t lo = f32_to_bf16_bits(f[0]) | (f32_to_bf16_bits(f[1]) << 16);
            const uint32_t hi = f32_to_bf16_bits(f[2]) | (f32_to_bf16_bits(f[3]) << 16);
            *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
            return;
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) store_elem<DT>(base, i + c, f[c]);
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
// -0 and +0 compare equal, so they get one key (adding +0 turns -0 into +0).
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ host checks
inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Shape fields every kernel family relies on.  Returns an oasis status.
inline int check_shape(const oasis_shape* s) {
    if (!s) return OASIS_EINVAL;
    if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 ||
        s->block_size <= 0)
        return OASIS_EINVAL;
    if (s->n_q < 1 || s->n_q > 3) return OASIS_EINVAL;
    if (s->n_q_heads % s->n_kv_heads != 0) return OASIS_EINVAL;
    if (s->dtype != OASIS_F32 && s->dtype != OASIS_BF16) return OASIS_EUNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return OASIS_EUNSUPPORTED;
    if (!is_pow2(s->block_size) || s->block_size > 64) return OASIS_EUNSUPPORTED;
    if (s->tile_stride != 0) {
        const long long eb = s->dtype == OASIS_F32 ? 4 : 2;
        if (s->tile_stride < (long long)s->block_size * s->head_dim || (s->tile_stride * eb) % 16)
            return OASIS_EINVAL;
    }
    return OASIS_OK;
}

// Elements from one tile of a K / V store to the next.
inline long long tile_stride_of(const oasis_shape* s) {
    return s->tile_stride ? s->tile_stride : (long long)s->block_size * s->head_dim;
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? OASIS_OK : OASIS_EHIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace oasis
