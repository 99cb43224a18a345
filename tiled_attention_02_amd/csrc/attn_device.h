// Device-side helpers shared by the libattn kernels (gfx950 / CDNA4 only).
//
// Operand layouts of the two matrix-core instructions used here (C = A*B,
// fp32 accumulate, lane l of a 64-wide wavefront, element e of 8):
//   v_mfma_f32_32x32x16_{bf16,f16}:
//     A[i = l%32][k = 8*(l/32)+e],  B[k = 8*(l/32)+e][j = l%32]
//     C register r (16 per lane): row 8*(r/4) + 4*(l/32) + r%4, column l%32
//   v_mfma_f32_16x16x32_{bf16,f16}:
//     A[i = l%16][k = 8*(l/16)+e],  B[k = 8*(l/16)+e][j = l%16]
//     C register r (4 per lane): row 4*(l/16) + r, column l%16
//   v_mfma_f32_16x16x16_{bf16,f16} (4 elements per lane):
//     A[i = l%16][k = 4*(l/16)+e],  B[k = 4*(l/16)+e][j = l%16], C as above
// Any permutation of the contraction index k applied to both A and B leaves
// C unchanged; the kernels use that freedom to make every lane's operand one
// contiguous 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element-type tags. Storage is raw 16-bit; arithmetic happens in the MFMA
// (inputs) and in fp32 (everything else).
struct BF16 {
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // 16x16x16: A[i = l%16][k = 4*(l/16)+e], B[k = 4*(l/16)+e][j = l%16], e < 4
  static __device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 against {1, 1}): sums the
  // rounded values exactly as the matrix core sees them
  static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
  }
  // the two values of a packed pair as fp32 (exact)
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
  // E4M3 codes in bytes 2*HI, 2*HI + 1 of w -> packed pair (low half from the
  // lower byte). Exact: every E4M3 value is a bf16 value.
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_e4m3x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
  static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
  // E4M3 codes in bytes 2*HI, 2*HI + 1 of w -> packed pair. Exact: every E4M3
  // value is an fp16 value.
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_e4m3x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
  }
};

// Eight E4M3 codes (two dwords, code e in byte e) -> eight 16-bit values in
// element order: one MFMA operand fragment.
template <class T>
__device__ __forceinline__ u32x4 e4m3x8(u32x2 w) {
  return u32x4{T::template from_e4m3x2<false>(w[0]), T::template from_e4m3x2<true>(w[0]),
               T::template from_e4m3x2<false>(w[1]), T::template from_e4m3x2<true>(w[1])};
}

// Rotary embedding of 8 column pairs (i, i + D/2) of one row, in place: x1
// holds columns i .. i+7, x2 columns i + D/2 .. i + D/2 + 7, c / s the
// cosines and sines of those 8 frequencies at the row's position (fp32, from
// the caller's table). Computed in fp32, rounded once to the 16-bit type:
//   x1' = x1 c - x2 s,   x2' = x2 c + x1 s.
template <class T>
__device__ __forceinline__ void rope8(u32x4& x1, u32x4& x2, const float* c, const float* s) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = T::lo(x1[w]), a1 = T::hi(x1[w]), b0 = T::lo(x2[w]), b1 = T::hi(x2[w]);
    const float c0 = c[2 * w], c1 = c[2 * w + 1], s0 = s[2 * w], s1 = s[2 * w + 1];
    x1[w] = T::pack2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    x2[w] = T::pack2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
  }
}

// Max / sum of a value with the same lane in the other half of the wavefront
// (lane l <-> lane l^32) through v_permlane32_swap: swap(x, x) returns the
// lower half's values in r[0] and the upper half's in r[1] on every lane.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
// max(x, x of lane l ^ 16) through v_permlane16_swap (rows of 16 lanes: the
// odd rows of the first operand trade places with the even rows of the
// second, so swap(x, x) gives each lane pair's even-row value in r[0] and its
// odd-row value in r[1]); no LDS round trip, unlike a bpermute.
__device__ __forceinline__ float row_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace attn
