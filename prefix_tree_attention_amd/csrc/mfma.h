// Internal: CDNA4 (gfx950) MFMA fragment types and helpers for the bf16
// attention kernels.
//
// v_mfma_f32_16x16x32_bf16, D = A * B + C with A 16x32, B 32x16, C/D 16x16:
//   A operand: lane l holds row (l % 16), k = 8 (l / 16) + 0..7
//   B operand: lane l holds column (l % 16), k = 8 (l / 16) + 0..7
//   C/D:       lane l holds column (l % 16), rows 4 (l / 16) + 0..3
// So a C fragment read "by column" has the same per-lane shape as an A or B
// operand whose row/column index is that column and whose k index runs over
// C's rows -- which lets a score tile feed the next product without a
// shuffle, provided the k order is permuted consistently on both operands.
//
// v_mfma_f32_32x32x16_bf16, D = A * B + C with A 32x16, B 16x32, C/D 32x32:
//   A operand: lane l holds row (l % 32), k = 8 (l / 32) + 0..7
//   B operand: lane l holds column (l % 32), k = 8 (l / 32) + 0..7
//   C/D:       lane l, register r holds column (l % 32),
//              row 8 (r / 4) + 4 (l / 32) + r % 4
// (both layouts checked element by element on gfx950 with random integer
// operands).  For a k-step of 16 C rows starting at 16m, lane l holds rows
// 16m + 4 (l / 32) + 0..3 in registers 8m + 0..3 and rows
// 16m + 8 + 4 (l / 32) + 0..3 in registers 8m + 4..7: eight values that
// serve as a B operand over those rows in that k order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace treeattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The value of lane l ^ 32 beside this lane's, by one v_permlane32_swap
// (lanes 32-63 of the first copy trade places with lanes 0-31 of the
// second): {x of lanes 0-31 in both halves, x of lanes 32-63 in both
// halves}, so an elementwise max or sum of the two is the lane-pair result
// with no LDS permute.
struct LanePair {
    float lo, hi;
};
__device__ __forceinline__ LanePair lane_pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Eight floats -> one bf16x8 operand.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& lo, const f32x4& hi) {
    const f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Rotary embedding of N element pairs (x1[u], x2[u]) = (x_j, x_{j + D/2}),
// j = j0 + u, by a table row of (cos, sin) float pairs cs[u]; the rotation
// arithmetic of the standalone pass (rope.hip): forward
//   (x1 c - x2 s, x2 c + x1 s), inverse (the gradient map) (x1 c + x2 s, x2 c - x1 s).
template <bool kInverse>
__device__ __forceinline__ void rope_pair(float& x1, float& x2, float c, float s) {
    const float a = x1, b = x2;
    if constexpr (kInverse) {
        x1 = __builtin_fmaf(a, c, b * s);
        x2 = __builtin_fmaf(b, c, -a * s);
    } else {
        x1 = __builtin_fmaf(a, c, -b * s);
        x2 = __builtin_fmaf(b, c, a * s);
    }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// Transpose a 4 (rows) x 8 (bf16 columns) register block: rows[r] holds 8
// consecutive bf16 of row r; returns, for column j, the 4 values of that
// column packed into 8 bytes (row 0 in the low half of word 0).
__device__ __forceinline__ void transpose4x8(const u32x4 rows[4], u32x2 cols[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1, sh = (j & 1) * 16;
        const uint32_t a = (rows[0][w] >> sh) & 0xffffu, b = (rows[1][w] >> sh) & 0xffffu;
        const uint32_t c = (rows[2][w] >> sh) & 0xffffu, d = (rows[3][w] >> sh) & 0xffffu;
        cols[j][0] = a | (b << 16);
        cols[j][1] = c | (d << 16);
    }
}

}  // namespace treeattn
