// Device-side building blocks shared by the gfx950 kernels: element types, 8-wide operand
// fragments, the 16x16x32 matrix-core step, DPP row reductions and conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lra {

typedef uint16_t bf16;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------------
// conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16 b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 / fp16, round to nearest even (one v_cvt_pk_* instruction on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
constexpr float kF16Max = 65504.f;
// the fp16 halves of a 32-bit word, widened exactly
__device__ __forceinline__ float f16_lo(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[0]); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[1]); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------------------------------------
// Vector of N consecutive elements held by one lane, loaded with the widest aligned accesses.
template <typename T, int N> struct Vec;

template <int N> struct Vec<float, N> {
    static_assert(N % 4 == 0 || N == 2 || N == 1, "fp32 vector width");
    float v[N];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) {
                float4 t = reinterpret_cast<const float4*>(p)[i];
                v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            }
        } else if constexpr (N == 2) {
            float2 t = *reinterpret_cast<const float2*>(p);
            v[0] = t.x; v[1] = t.y;
        } else {
            v[0] = *p;
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = 0.f;
    }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};

template <int N> struct Vec<bf16, N> {
    static_assert(N % 2 == 0, "bf16 vector width");
    uint32_t w[N / 2];
    __device__ __forceinline__ void load(const bf16* p) {
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N / 8; ++i) {
                uint4 t = reinterpret_cast<const uint4*>(p)[i];
                w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
            }
        } else if constexpr (N == 4) {
            uint2 t = *reinterpret_cast<const uint2*>(p);
            w[0] = t.x; w[1] = t.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) w[i] = 0u;
    }
    __device__ __forceinline__ float get(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
};

// ---------------------------------------------------------------------------------------------
// One 16x16x32 matrix-core step on 8-element operand fragments.
// Lane l holds row/column (l % 16) and reduction slots 8*(l/16) .. 8*(l/16)+7 of both operands; the
// hardware pairs A's and B's slots identically, so any assignment of k indices to slots that is the
// same for both operands yields the full dot product. Output: lane l, register j holds
// C[4*(l/16) + j][l % 16].
//   bf16: one v_mfma_f32_16x16x32_bf16.
//   fp32: eight v_mfma_f32_16x16x4_f32, the e-th taking element e of every lane.
__device__ __forceinline__ f32x4 mma16x16x32(const Vec<bf16, 8>& a, const Vec<bf16, 8>& b, f32x4 c) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.w);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.w);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// the same step on fp16 operands (8 halves per lane, bit patterns in 4 dwords)
struct H8 {
    uint32_t w[4];
};
// 16x16x16 bf16 step (4 values per lane): A lane (row n, group q) holds A[n][4q..4q+3], B lane
// (column n, group q) holds B[4q..4q+3][n], C lane (n, q) holds C[4q+j][n]
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma16x16x16_bf16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                     c, 0, 0, 0);
}
// the same 16x16x16 step on fp16 operands (4 halves per lane in 2 dwords)
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma16x16x16_f16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16x16x32_f16(const H8& a, const H8& b, f32x4 c) {
    f16x8_t av = __builtin_bit_cast(f16x8_t, a.w);
    f16x8_t bv = __builtin_bit_cast(f16x8_t, b.w);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

// the fp16 step on 16-bit vectors whose words hold fp16 bit patterns
__device__ __forceinline__ f32x4 mma16x16x32_f16(const Vec<bf16, 8>& a, const Vec<bf16, 8>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a.w), __builtin_bit_cast(f16x8_t, b.w), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16x16x32(const Vec<float, 8>& a, const Vec<float, 8>& b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------------------------------------
// Cross-lane helpers (wave64). DPP row operations act inside each row of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// all-reduce over the 16 lanes of a row: xor 1, xor 2 (quad permutes), then rotate by 4 and 8
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x128>(v);
    return v;
}
// max over lanes l and l ^ 16 / l ^ 32 on the VALU (gfx950 permlane swaps: no LDS round trip).
// A swap with both operands = x leaves (x_l, x_partner) in the result pair, in some order.
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS transpose read of 16-bit elements (gfx950). Within each group of 16 lanes, let M[j] be the
// four consecutive elements at lane j's address; lane i receives M[i/4 + 4k][i%4] in element k.
// Pointing lane j at row key(j/4), columns c0 + 4*(j%4) .. +3 of a row-major [key][col] tile gives
// lane i the column c0 + i of rows key(0..3): four reduction slots of a matrix-core operand.
typedef short lds_s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
    const lds_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) lds_s16x4*)(p));
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// compiler-level ordering point for LDS traffic that stays inside one wave
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_wave_barrier(); }

}  // namespace lra
