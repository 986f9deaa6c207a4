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
  const long long stride = (long long)gridDim.x * 256;
  float m = 0.f;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  // four chunks per thread in flight, then the remainder one at a time
  for (; i + 3 * stride < n8; i += 4 * stride) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(base + (i + u * stride) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[u][e]));
  }
  for (; i < n8; i += stride) {
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

// Codes of slab (b, h) go to codes + (b * Hkv + h) * dst_slab + dst_off: a
// tensor quantised whole (dst_slab = slab, dst_off = 0), or rows written into
// a larger cache at an offset.  The scale is set from the maxima (and
// written), or given (rows appended to a cache whose scales are set).
template <typename T>
__global__ __launch_bounds__(256) void quant_encode_kernel(QuantArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  float s;
  if (a.scale_given) {
    s = a.scale[h];
  } else {
    const float amax = __uint_as_float(a.amax_bits[h]);
    s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
    if (blockIdx.x == 0 && b == 0 && threadIdx.x == 0) a.scale[h] = s;
  }
  const T* base = static_cast<const T*>(a.kv) + (size_t)(b * a.Hkv + h) * a.slab;
  uint8_t* out = a.codes + (size_t)(b * a.Hkv + h) * a.dst_slab + a.dst_off;
  const long long n8 = a.slab / 8;
  const long long stride = (long long)gridDim.x * 256;
  auto put = [&](long long j, const float* x) __attribute__((always_inline)) {
    u32x2 w;
    w[0] = encode_e4m3_x4(x[0], x[1], x[2], x[3], s);
    w[1] = encode_e4m3_x4(x[4], x[5], x[6], x[7], s);
    *reinterpret_cast<u32x2*>(out + j * 8) = w;
  };
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  // four chunks per thread in flight, then the remainder one at a time
  for (; i + 3 * stride < n8; i += 4 * stride) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(base + (i + u * stride) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) put(i + u * stride, x[u]);
  }
  for (; i < n8; i += stride) {
    float x[8];
    load8<T>(base + i * 8, x);
    put(i, x);
  }
}

// A few looping workgroups per CU over the whole tensor (1024 for bf16
// input, 256 for float32, whose threads move twice the bytes per chunk;
// measured best of 256 to 8192), each over its share of a slab.  Every
// workgroup of the maxima pass ends in one atomic on its head's word, so a
// grid of many small workgroups would also queue thousands of atomics on
// each of Hkv words.
static dim3 quant_grid(const QuantArgs& a, bool is_bf16) {
  const long long n8 = a.slab / 8;
  const long long slabs = (long long)a.B * a.Hkv;
  long long per_slab = (n8 + 256 * 4 - 1) / (256 * 4);   // at least ~4 chunks per thread
  const long long total = is_bf16 ? 1024 : 256;
  const long long cap = (total + slabs - 1) / slabs;
  if (per_slab > cap) per_slab = cap;
  if (per_slab < 1) per_slab = 1;
  return dim3((unsigned)per_slab, a.Hkv, a.B);
}

hipError_t launch_quant_clear(uint32_t* amax_bits, int n, hipStream_t stream) {
  hipLaunchKernelGGL(quant_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, amax_bits, n);
  return hipGetLastError();
}

hipError_t launch_quant_amax(const QuantArgs& a, bool is_bf16, hipStream_t stream) {
  if (is_bf16)
    hipLaunchKernelGGL((quant_amax_kernel<bf16>), quant_grid(a, true), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((quant_amax_kernel<float>), quant_grid(a, false), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_encode(const QuantArgs& a, bool is_bf16, hipStream_t stream) {
  if (is_bf16)
    hipLaunchKernelGGL((quant_encode_kernel<bf16>), quant_grid(a, true), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((quant_encode_kernel<float>), quant_grid(a, false), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantArgs& a, bool is_bf16, hipStream_t stream) {
  hipError_t e = launch_quant_clear(a.amax_bits, a.Hkv, stream);
  if (e != hipSuccess) return e;
  e = launch_quant_amax(a, is_bf16, stream);
  if (e != hipSuccess) return e;
  return launch_quant_encode(a, is_bf16, stream);
}

}  // namespace yoco
