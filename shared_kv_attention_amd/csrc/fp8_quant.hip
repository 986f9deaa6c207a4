// Quantisation of a K or V tensor into the 8-bit (OCP fp8-e4m3fn) cache.
//
// The pages motivate an 8-bit cache (YOCO podcast transcript, segments 1 and
// 24) but fix no format; the format used here: one float32 scale per KV head
// over all (batch, position, channel), s_h = amax_h / 448 (1 for an all-zero
// head), code = round-to-nearest-even e4m3fn of x / s_h (one IEEE float32
// division), saturated to +-448.
//
// Three launches, no atomics on floats and no memset (so the sequence can be
// captured in a HIP graph): clear the per-head maxima, reduce |x| per head
// (integer atomicMax on the bit patterns of non-negative floats, which order
// like the values), then encode with hardware RNE conversion after clamping.
#include "common.hpp"
#include "launch.hpp"

namespace yoco {

__global__ void quant_clear_kernel(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

// grid (blocks per slab, Hkv, B); 256 threads; 8 elements per thread per step.
template <typename T>
__global__ __launch_bounds__(256) void quant_amax_kernel(QuantArgs a) {
  __shared__ float red[4];
  const int h = blockIdx.y, b = blockIdx.z;
  const T* base = static_cast<const T*>(a.kv) + (size_t)(b * a.Hkv + h) * a.slab;
  const long long n8 = a.slab / 8;
  float m = 0.f;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    float x[8];
    load8<T>(base + i * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  }
  // wave max via DPP rows, then across rows and waves through LDS
  m = row16_max(m);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(a.amax_bits + h, __float_as_uint(mm));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void quant_encode_kernel(QuantArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const float amax = __uint_as_float(a.amax_bits[h]);
  const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
  if (blockIdx.x == 0 && b == 0 && threadIdx.x == 0) a.scale[h] = s;
  const size_t off = (size_t)(b * a.Hkv + h) * a.slab;
  const T* base = static_cast<const T*>(a.kv) + off;
  uint8_t* out = a.codes + off;
  const long long n8 = a.slab / 8;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    float x[8];
    load8<T>(base + i * 8, x);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(__fdiv_rn(x[e], s), -448.f), 448.f);
    u32x2 w;
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    w[0] = (uint32_t)lo;
    w[1] = (uint32_t)hi;
    *reinterpret_cast<u32x2*>(out + i * 8) = w;
  }
}

hipError_t launch_quant_fp8(const QuantArgs& a, bool is_bf16, hipStream_t stream) {
  hipLaunchKernelGGL(quant_clear_kernel, dim3((a.Hkv + 255) / 256), dim3(256), 0, stream, a.amax_bits, a.Hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n8 = a.slab / 8;
  long long per_slab = (n8 + 256 * 4 - 1) / (256 * 4);   // ~4 steps per thread
  if (per_slab > 1024) per_slab = 1024;
  if (per_slab < 1) per_slab = 1;
  dim3 grid((unsigned)per_slab, a.Hkv, a.B);
  if (is_bf16)
    hipLaunchKernelGGL((quant_amax_kernel<bf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((quant_amax_kernel<float>), grid, dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (is_bf16)
    hipLaunchKernelGGL((quant_encode_kernel<bf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((quant_encode_kernel<float>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace yoco
