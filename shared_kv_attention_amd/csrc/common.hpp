// Device helpers shared by the gfx950 kernels of libyoco: vector types,
// MFMA wrappers that present one "fragment of 8 elements per lane" interface
// for bf16 and f32, DPP row reductions and element conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yoco {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Fourth word of a raw buffer resource on gfx9-family chips: data format
// 32 bits (field [18:15] = 4), no index stride, no swizzle, no thread-id
// addressing.  Untyped buffer loads read bytes at base + offset and return
// zeros for offsets at or past the resource's size.
constexpr int kBufferFlags = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element traits.  A "fragment" is the 8 consecutive-k operand elements one
// lane feeds to a matrix-core step: bf16 -> one 16-byte vector, f32 -> 8 floats.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<bf16> {
  using frag = bf16x8;
  static constexpr int bytes = 2;
};
template <> struct Elem<float> {
  using frag = f32x8;
  static constexpr int bytes = 4;
};

// 32x32 output tile, 16-deep k step.  Operand lane layout (checked on gfx950):
//   lane l supplies A[row = l%32][k = 8*(l/32) + j] and B[k = 8*(l/32) + j][col = l%32],
//   j = 0..7; the result element i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// f32: v_mfma_f32_32x32x2f32 takes k = l/32 from each lane; issuing it once per
// fragment element j covers k = {j, 8+j}; the 8 issues cover all 16 k.
__device__ __forceinline__ f32x16 mma32(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// 16x16 output tile, 32-deep k step.  lane l supplies A[row = l%16][k = 8*(l/16) + j]
// and B[k = 8*(l/16) + j][col = l%16]; result element i is C[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Two OCP e4m3fn codes (bytes 0 and 1 of `w`, or 2 and 3 when hi) -> two floats.
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Four values -> four OCP e4m3fn codes (byte i = code of x[i]) with the
// per-head scale s: x / s as one correctly rounded float32 division, clamped
// to +-448 (saturation), then the hardware's round-to-nearest-even conversion.
__device__ __forceinline__ uint32_t encode_e4m3_x4(float x0, float x1, float x2, float x3, float s) {
  const float y0 = fminf(fmaxf(__fdiv_rn(x0, s), -448.f), 448.f);
  const float y1 = fminf(fmaxf(__fdiv_rn(x1, s), -448.f), 448.f);
  const float y2 = fminf(fmaxf(__fdiv_rn(x2, s), -448.f), 448.f);
  const float y3 = fminf(fmaxf(__fdiv_rn(x3, s), -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers
// ---------------------------------------------------------------------------
// DPP control words (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum / max over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<kDppQuadSwap1>(x);
  x += dpp_f32<kDppQuadSwap2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}
// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) << 2), __float_as_int(x)));
}

// Maximum / sum of the values held by lanes l and l ^ 32, on both lanes
// (v_permlane32_swap exchanges the two halves of the wave in the VALU; the
// sum is formed in the same order, low half first, on both lanes).
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A pointer that is the same on every lane, as a scalar value.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Rotary position embedding of one channel pair (x0, x1) = channels (2i, 2i+1)
// of a head at position p: the angle p * theta^(-2i/d) is formed and reduced
// modulo 2 pi in double precision (positions reach 2^20 and more, where a
// single-precision angle would be off by a sizeable fraction of a radian),
// then rotated with single-precision sine and cosine of the reduced angle.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rope_inv_freq(int i, int d, double log2_theta) {
  return exp2(-(2.0 * i / d) * log2_theta);
}
__device__ __forceinline__ void rope_pair(float& x0, float& x1, double angle) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double r = angle - kTwoPi * rint(angle * (1.0 / kTwoPi));
  float s, c;
  sincosf((float)r, &s, &c);
  const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

}  // namespace yoco
