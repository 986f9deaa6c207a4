// Achievable-peak microbenchmarks of the chip the library runs on: a
// streaming HBM read and register-resident bf16 matrix-core loops (operands
// of ones, and operands that change every instruction).  They
// report what this MI355X reaches at its clock under load, beside the spec
// figures (8 TB/s, 2.5 PFLOP/s dense bf16) the kernels are also measured
// against.  Both compute a checkable result so that nothing can be
// optimised away: the read sums the 32-bit words it loads, the matrix loop
// accumulates products of exactly representable operands.
#include "common.hpp"
#include "launch.hpp"

namespace yoco {

// Each workgroup streams one contiguous 1/gridDim of the buffer (16-byte
// chunks, 8 in flight per thread, non-temporal loads) -- on MI355X this
// pattern reaches ~7.1 TB/s where a grid-stride loop over the whole buffer
// stays near 6 TB/s -- and writes one wrapping 32-bit sum of the words it
// read.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, long long n_chunks,
                                                        uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[256];
  const long long per = (n_chunks + gridDim.x - 1) / gridDim.x;
  const long long lo = per * blockIdx.x;
  const long long hi = lo + per < n_chunks ? lo + per : n_chunks;
  long long i = lo + threadIdx.x;
  uint32_t s = 0;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  for (; i < hi; i += 256) {
    const u32x4 v = src[i];
    s += v[0] + v[1] + v[2] + v[3];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Each wave runs `iters` rounds of 8 independent 32x32x16 bf16 MFMAs on
// operands of ones: every accumulator element gains 16 per MFMA, so after
// the loop each equals 16 * iters exactly (iters <= 2^20).  Lane 0 of each
// wave writes the sum of its 8 accumulators' first elements.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ out) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (bf16)1.0f;
    b[j] = (bf16)1.0f;
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mma32(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0];
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

// The same loop with operands that change every instruction, as real data's
// do (the matrix core then draws more power, and the clock drops): each lane
// holds 8 A and 8 B fragments of integers in [-127, 127] (exact in bf16)
// drawn from a hash of its position, with B fragment 4 + j the negation of
// fragment j.  Accumulator i takes a[i] times b[(i + u) % 8] for u = 0..7 in
// every round of 8, which adds a[i] times (the sum of all 8 B fragments) =
// exactly 0 (every partial sum is an integer below 2^21), so each wave
// writes exactly 0.
__device__ __forceinline__ uint32_t peak_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void peak_mfma_toggle_kernel(int iters, float* __restrict__ out) {
  bf16x8 a[8], b[8];
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = peak_hash(seed + 8u * s + e);
      a[s][e] = (bf16)(float)((int)(h % 255u) - 127);
      if (s < 4) b[s][e] = (bf16)(float)((int)((h >> 8) % 255u) - 127);
    }
  }
#pragma unroll
  for (int s = 4; s < 8; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) b[s][e] = -b[s - 4][e];
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = mma32(a[i], b[(i + u) & 7], acc[i]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s += fabsf(acc[i][e]);
  }
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

hipError_t launch_peak_read(const void* src, long long bytes, uint32_t* partial, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     bytes / 16, partial);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(int iters, float* out, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma_toggle(int iters, float* out, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(peak_mfma_toggle_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace yoco
