// Gated retention, the self-decoder's other choice: chunkwise prefill and
// the recurrent decode step, plus the per-head GroupNorm with swish gate.
//
// What is computed (paperlayer.ai summary of "You Only Cache Once", section 3
// Gated Retention and appendix B; YOCO podcast transcript, segment 16): per
// head, with a data-dependent scalar decay gamma_n = sigmoid(z_n)^(1/tau),
//   S_n = gamma_n S_{n-1} + k_n^T v_n,   o_n = q_n S_n      (d x d state S).
// The chunkwise form splits the sequence into chunks of C positions; with L
// the log decay accumulated from the chunk start (inclusive),
//   o_n = sum_{m in chunk, m <= n} (q_n . k_m) e^{L_n - L_m} v_m + e^{L_n} q_n R,
//   R  <- e^{L_last} R + sum_{m in chunk} e^{L_last - L_m} k_m^T v_m.
//
// Design (MI355X-first): instead of one workgroup walking a head's chunks in
// order (only B*H workgroups), the prefill runs four launches that are each
// parallel over chunks:
//  1. gates:  per chunk, log2 decay prefix sums and the chunk's total decay;
//  2. state:  per chunk, dR = K^T (V scaled by e^{L_last - L_m}) on the
//             matrix cores (both operands read transposed from LDS);
//  3. scan:   per (head, state element), R_c = e^{L_last} R_{c-1} + dR_c in
//             float32, storing the state entering every chunk;
//  4. output: per (chunk, 128 query rows), an attention-like tile loop with
//             decay weights e^{L_n - L_m} (formed per pair from the
//             difference, so a strong gate can never overflow) instead of a
//             softmax, and the cross-chunk term R^T Q^T on the same
//             accumulator.
#include "common.hpp"
#include "launch.hpp"
#include "tile_lds.hpp"

namespace yoco {

template <int D>
struct GretCfg {
  static constexpr int CH = D * 2 / 16;   // 16-byte chunks per bf16 row
  static constexpr int NC = D / 16;       // 16-deep k steps over d
  static constexpr int NDB = D / 32;      // 32-wide blocks of d
  static constexpr int BK = 64;           // key rows per LDS tile
  static constexpr int TILE = BK * D * 2; // bytes of one K or V tile
};

// log2 of the decay: log2(sigmoid(z)) / tau, without overflow.
__device__ __forceinline__ float gate_log2(float z, float inv_tau) {
  const float ls = fminf(z, 0.f) - log1pf(__expf(-fabsf(z)));   // natural log of sigmoid(z)
  return ls * kLog2e * inv_tau;
}

// ---------------------------------------------------------------------------
// 1. per-chunk inclusive prefix sums of log2 decay; total decay per chunk
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gret_gate_kernel(GretArgs a) {
  __shared__ float buf[256];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int n = c * a.chunk + t;
  const bool valid = t < a.chunk && n < a.N;
  float x = valid ? gate_log2(a.gate[(size_t)bh * a.N + n], a.inv_tau) : 0.f;
  buf[t] = x;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const float y = t >= off ? buf[t - off] : 0.f;
    __syncthreads();
    x += y;
    buf[t] = x;
    __syncthreads();
  }
  if (valid) a.lg2[(size_t)bh * a.N + n] = x;
  const int last = min(a.chunk, a.N - c * a.chunk) - 1;
  if (t == last) a.lam[(size_t)bh * a.nc + c] = __builtin_amdgcn_exp2f(x);
}

// Stage rows [r0, r0 + BK) of a [N, D] bf16 matrix into an LDS tile with the
// transposed-read swizzle; rows >= N (or outside the chunk) become zero.  If
// scale is given, row r is multiplied by scale(r) (float32, then bf16 RNE).
template <int D, typename F>
__device__ __forceinline__ void stage_rows_v(char* tile, const bf16* src, int r0, int rows_valid, F scale,
                                             bool scaled) {
  using C = GretCfg<D>;
  for (int slot = threadIdx.x; slot < C::BK * C::CH; slot += 256) {
    const int row = slot / C::CH, pch = slot % C::CH;   // physical chunk pch holds logical chunk pch ^ swz
    const int lch = pch ^ swz_v<C::CH>(row);
    u32x4 w{0, 0, 0, 0};
    if (row < rows_valid) {
      w = *reinterpret_cast<const u32x4*>(src + (size_t)(r0 + row) * D + lch * 8);
      if (scaled) {
        const float f = scale(row);
        bf16x8 v = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * f);
        w = __builtin_bit_cast(u32x4, v);
      }
    }
    *reinterpret_cast<u32x4*>(tile + row * C::CH * 16 + pch * 16) = w;
  }
}

// ---------------------------------------------------------------------------
// 2. per-chunk state contribution dR[dk][dv] = sum_m K[m][dk] V[m][dv] w_m
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void gret_state_kernel(GretArgs a) {
  using C = GretCfg<D>;
  __shared__ __attribute__((aligned(16))) char kt[C::TILE], vt[C::TILE];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = c * a.chunk, clen = min(a.chunk, a.N - c0);
  const bf16* kb = static_cast<const bf16*>(a.k) + ((size_t)bh * a.N + c0) * D;
  const bf16* vb = static_cast<const bf16*>(a.v) + ((size_t)bh * a.N + c0) * D;
  const float* lg = a.lg2 + (size_t)bh * a.N + c0;
  const float l_last = lg[clen - 1];

  constexpr int TILES = C::NDB * C::NDB, TPW = TILES / 4 > 0 ? TILES / 4 : 1;
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
  const bool active = w * TPW < TILES;

  for (int r0 = 0; r0 < clen; r0 += C::BK) {
    const int rows = min(C::BK, clen - r0);
    stage_rows_v<D>(kt, kb, r0, rows, [](int) { return 1.f; }, false);
    stage_rows_v<D>(vt, vb, r0, rows, [&](int row) { return __builtin_amdgcn_exp2f(l_last - lg[r0 + row]); }, true);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tt = w * TPW + i, dkb = tt / C::NDB, dvb = tt % C::NDB;
#pragma unroll
        for (int s = 0; s < C::BK / 16; ++s)
          acc[i] = mma32(lds_frag_vt<bf16, C::CH>(kt, s, dkb, l), lds_frag_vt<bf16, C::CH>(vt, s, dvb, l), acc[i]);
      }
    }
    __syncthreads();
  }
  if (active) {
    float* dst = a.dR + ((size_t)bh * a.nc + c) * D * D;
    const int g = l >> 5;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = w * TPW + i, dkb = tt / C::NDB, dvb = tt % C::NDB;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int dk = dkb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
        dst[dk * D + dvb * 32 + (l & 31)] = acc[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. scan over chunks: rin_c = R_{c-1} (bf16), R_c = lam_c R_{c-1} + dR_c
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gret_scan_kernel(GretArgs a) {
  const int bh = blockIdx.y;
  const int DD = a.d * a.d;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= DD) return;
  float R = a.state_in ? a.state_in[(size_t)bh * DD + e] : 0.f;
  for (int c = 0; c < a.nc; ++c) {
    static_cast<bf16*>(a.rin)[((size_t)bh * a.nc + c) * DD + e] = (bf16)R;
    R = a.lam[(size_t)bh * a.nc + c] * R + a.dR[((size_t)bh * a.nc + c) * DD + e];
  }
  if (a.state_out) a.state_out[(size_t)bh * DD + e] = R;
}

// ---------------------------------------------------------------------------
// 4. outputs of 128 query rows of one chunk
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void gret_out_kernel(GretArgs a) {
  using C = GretCfg<D>;
  __shared__ __attribute__((aligned(16))) char kt[C::TILE], vt[C::TILE], rt[D * D * 2];
  __shared__ float lgt[C::BK];
  const int nrb = a.chunk / 128;
  const int c = blockIdx.x / nrb, rb = blockIdx.x % nrb, bh = blockIdx.y;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 5, r32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = c * a.chunk, clen = min(a.chunk, a.N - c0);
  const int q0 = c0 + rb * 128;                 // first query row of the workgroup
  if (q0 >= a.N) return;                        // whole workgroup past the end (uniform)
  const int wq0 = q0 + 32 * w;                  // first row of this wave
  const int n = wq0 + r32;                      // this lane's query row
  const bool row_ok = n < a.N;
  const bool wave_live = wq0 < a.N;
  const size_t hrow = (size_t)bh * a.N;

  // query fragments (as for attention: row n, dims 16c + 8g + j)
  bf16x8 qf[C::NC];
  {
    const bf16* qrow = static_cast<const bf16*>(a.q) + (hrow + (row_ok ? n : q0)) * D;
#pragma unroll
    for (int cc = 0; cc < C::NC; ++cc)
      qf[cc] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * g) : bf16x8{};
  }
  const float l_n = row_ok ? a.lg2[hrow + n] : 0.f;

  // cross-chunk term: O^T = R^T Q^T, then column n scaled by 2^{L_n}
  const bf16* rsrc = static_cast<const bf16*>(a.rin) + ((size_t)bh * a.nc + c) * D * D;
  stage_rows_v<D>(rt, rsrc, 0, D, [](int) { return 1.f; }, false);
  if constexpr (D > 64) stage_rows_v<D>(rt + 64 * D * 2, rsrc, 64, 64, [](int) { return 1.f; }, false);
  __syncthreads();
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    acc[db] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < C::NC; ++cc) acc[db] = mma32(lds_frag_vt<bf16, C::CH>(rt, cc, db, l), qf[cc], acc[db]);
  }
  {
    const float f = __builtin_amdgcn_exp2f(l_n);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] *= f;
  }

  // inner-chunk term over key tiles [c0, last row of the workgroup]
  const int k_end = min(q0 + 127, a.N - 1);     // last key any row here can see
  const int pw1 = min(wq0 + 31, a.N - 1);       // last row of this wave
  const bf16* kbase = static_cast<const bf16*>(a.k) + hrow * D;
  const bf16* vbase = static_cast<const bf16*>(a.v) + hrow * D;
  for (int k0 = c0; k0 <= k_end; k0 += C::BK) {
    const int rows = min(C::BK, min(c0 + clen, k_end + 1) - k0);
    __syncthreads();   // the previous tile (or R) is no longer read
    // K tile with the K swizzle (read as the A operand in row order sigma)
    for (int slot = tid; slot < C::BK * C::CH; slot += 256) {
      const int row = slot / C::CH, pch = slot % C::CH;
      const int lch = pch ^ swz_k<C::CH>(row);
      u32x4 v4{0, 0, 0, 0};
      if (row < rows) v4 = *reinterpret_cast<const u32x4*>(kbase + (size_t)(k0 + row) * D + lch * 8);
      *reinterpret_cast<u32x4*>(kt + row * C::CH * 16 + pch * 16) = v4;
    }
    stage_rows_v<D>(vt, vbase + (size_t)k0 * D, 0, rows, [](int) { return 1.f; }, false);
    if (tid < C::BK) lgt[tid] = tid < rows ? a.lg2[hrow + k0 + tid] : 0.f;
    __syncthreads();
    if (!wave_live || k0 > pw1) continue;       // every key of the tile is after this wave's rows

    // S^T = K Q^T; element i of block kb <-> key k0 + kb*32 + 16*(i/8) + 8g + i%8
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int krow = kb * 32 + sigma(r32);
#pragma unroll
      for (int cc = 0; cc < C::NC; ++cc) s[kb] = mma32(lds_frag_k<bf16, C::CH>(kt, krow, cc, g), qf[cc], s[kb]);
    }
    // decay weights, masked by m <= n (a select: 2^{L_n - L_m} may overflow above the diagonal)
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
        const float wgt = s[kb][i] * __builtin_amdgcn_exp2f(l_n - lgt[off]);
        const float p = (k0 + off <= n) ? wgt : 0.f;
        pf[2 * kb + (i >> 3)][i & 7] = (bf16)p;
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) acc[db] = mma32(lds_frag_vt<bf16, C::CH>(vt, cc, db, l), pf[cc], acc[db]);
    }
  }

  if (row_ok) {
    bf16* orow = static_cast<bf16*>(a.o) + (hrow + n) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)acc[db][4 * qd + e];
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * qd + 4 * g) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// recurrent step: S <- gamma S + k^T v; o = q S   (state float32 [dk][dv])
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void gret_decode_kernel(GretDecodeArgs a) {
  const int bh = blockIdx.y;
  const int j = blockIdx.x * 64 + threadIdx.x;   // this lane's dv column
  const T* q = static_cast<const T*>(a.q) + (size_t)bh * a.d;
  const T* k = static_cast<const T*>(a.k) + (size_t)bh * a.d;
  const T* v = static_cast<const T*>(a.v) + (size_t)bh * a.d;
  const float gam = __builtin_amdgcn_exp2f(gate_log2(a.gate[bh], a.inv_tau));
  const float vj = to_f32(v[j]);
  float* S = a.state + (size_t)bh * a.d * a.d + j;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < a.d; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float sn = fmaf(gam, S[(size_t)(i + u) * a.d], to_f32(k[i + u]) * vj);
      S[(size_t)(i + u) * a.d] = sn;
      acc[u] = fmaf(to_f32(q[i + u]), sn, acc[u]);
    }
  }
  static_cast<T*>(a.o)[(size_t)bh * a.d + j] = from_f32<T>((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// ---------------------------------------------------------------------------
// per-head GroupNorm (over d channels) times swish(g); one wave per (b, n, h)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gret_norm_kernel(GretNormArgs a) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, n, h) flattened
  const long long rows = (long long)a.B * a.N * a.H;
  if (row >= rows) return;
  const int l = threadIdx.x & 63;
  const int h = (int)(row % a.H);
  const long long bn = row / a.H;
  const int n = (int)(bn % a.N), b = (int)(bn / a.N);
  const T* y = static_cast<const T*>(a.y) + (((size_t)b * a.H + h) * a.N + n) * a.d;
  const T* gg = static_cast<const T*>(a.g) + ((size_t)bn * a.H + h) * a.d;
  T* out = static_cast<T*>(a.out) + ((size_t)bn * a.H + h) * a.d;
  const int per = a.d / 64;   // 1 or 2 channels per lane
  float x[2] = {0.f, 0.f};
  float s = 0.f;
  for (int e = 0; e < per; ++e) {
    x[e] = to_f32(y[l * per + e]);
    s += x[e];
  }
  auto wave_sum = [&](float v) {
    v = row16_sum(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  };
  const float mean = wave_sum(s) / (float)a.d;
  float q2 = 0.f;
  for (int e = 0; e < per; ++e) q2 += (x[e] - mean) * (x[e] - mean);
  const float rstd = 1.f / sqrtf(wave_sum(q2) / (float)a.d + a.eps);
  for (int e = 0; e < per; ++e) {
    const float gv = to_f32(gg[l * per + e]);
    const float sw = gv / (1.f + __expf(-gv));
    out[l * per + e] = from_f32<T>(sw * (x[e] - mean) * rstd);
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_gret_prefill(const GretArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gret_gate_kernel, dim3(a.nc, a.B * a.H), dim3(256), 0, stream, a);
  if (a.d == 128) hipLaunchKernelGGL(gret_state_kernel<128>, dim3(a.nc, a.B * a.H), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gret_state_kernel<64>, dim3(a.nc, a.B * a.H), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(gret_scan_kernel, dim3((a.d * a.d + 255) / 256, a.B * a.H), dim3(256), 0, stream, a);
  const int nblk = a.nc * (a.chunk / 128);
  if (a.d == 128) hipLaunchKernelGGL(gret_out_kernel<128>, dim3(nblk, a.B * a.H), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gret_out_kernel<64>, dim3(nblk, a.B * a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gret_decode(const GretDecodeArgs& a, bool is_bf16, hipStream_t stream) {
  const dim3 grid(a.d / 64, a.B * a.H);
  if (is_bf16) hipLaunchKernelGGL(gret_decode_kernel<bf16>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(gret_decode_kernel<float>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gret_norm(const GretNormArgs& a, bool is_bf16, hipStream_t stream) {
  const long long rows = (long long)a.B * a.N * a.H;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (is_bf16) hipLaunchKernelGGL(gret_norm_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gret_norm_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace yoco
