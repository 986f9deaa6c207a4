// Global KV projection: K, V = RMSNorm(X) W_K^T, RMSNorm(X) W_V^T, written
// once into the head-major shared cache.
//
// What is computed (YOCO podcast transcript, segment 12: the self-decoder
// output is normalised once and projected by a single pair of matrices into
// the shared keys and values; paperlayer.ai summary of "You Only Cache Once",
// section 2): for token t, n_t = x_t / sqrt(mean(x_t^2) + eps) * gamma and
// K[b, h, pos0 + t, c] = n_t . W_K[h*d + c], V likewise.
//
// Design (MI355X-first):
//  * One GEMM for both matrices: the output "features" are the 2*Hkv*d rows
//    of [W_K; W_V]; the product is formed transposed, C^T = W X^T, on
//    32x32x16 bf16 MFMA (32x32x2 f32 for float32), so each lane's results
//    belong to one token and 4 consecutive channels of one head -- the
//    epilogue scales by that token's RMS factor and stores 4 channels at a
//    time straight into [B, Hkv, n_cap, d].
//  * The normalisation is fused: the threads that stage X tiles into LDS
//    accumulate the row sums of squares from the very values they move, so X
//    is read once; the per-row factor is applied to the float32 accumulator.
//    A norm gain gamma, when given, multiplies X during staging.
//  * 128x128 output tile per 256-thread workgroup, 64-element k steps (32 for
//    float32), LDS double buffering with XOR-swizzled 16-byte chunks.
#include "common.hpp"
#include "launch.hpp"

namespace yoco {

template <typename T>
struct ProjCfg {
  static constexpr int E = Elem<T>::bytes;
  static constexpr int BM = 128;                 // features per tile
  static constexpr int BN = 128;                 // tokens per tile
  static constexpr int BKK = 128 / E;            // k elements per stage (128-byte rows)
  static constexpr int CH = 8;                   // 16-byte chunks per tile row
  static constexpr int PER_T = 128 * CH / 256;   // chunks per thread per operand (= 4)
  static constexpr int NKS = BKK / 16;           // matrix-core k steps per stage
  static constexpr int TILE_BYTES = 128 * 128;
};

// XOR swizzle of the 16-byte chunk index within a 128-byte tile row: the 32
// rows a wave reads at once spread over all banks whether the LDS serves 8
// or 16 lanes of 16-byte accesses per cycle.
__device__ __forceinline__ int swz8(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_row(const char* tile, int row, int kc, int g) {
  const char* rowp = tile + row * 128;
  const int sw = swz8(row);
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    const int ch = 2 * kc + g;
    f = *reinterpret_cast<const bf16x8*>(rowp + ((ch ^ sw) << 4));
  } else {
    const int ch = 4 * kc + 2 * g;
    f32x4 a = *reinterpret_cast<const f32x4*>(rowp + ((ch ^ sw) << 4));
    f32x4 b = *reinterpret_cast<const f32x4*>(rowp + (((ch + 1) ^ sw) << 4));
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// Square-sum of the elements in a raw 16-byte chunk.
template <typename T>
__device__ __forceinline__ float chunk_sumsq(u32x4 w) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
    // products of bf16 values are exact in float32: x0^2 + x1^2 per instruction
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = w[i];   // element to a scalar first (bit_cast of a vector element mis-compiles)
      const bf16x2 x = __builtin_bit_cast(bf16x2, wi);
      s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = __uint_as_float(w[i]);
      s = fmaf(x, x, s);
    }
  }
  return s;
}

// x * gamma, rounded back to T, for one 16-byte chunk.
template <typename T>
__device__ __forceinline__ u32x4 chunk_scale(u32x4 w, u32x4 gw) {
  if constexpr (sizeof(T) == 2) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16) * __uint_as_float(gw[i] << 16);
      const float hi = __uint_as_float(w[i] & 0xFFFF0000u) * __uint_as_float(gw[i] & 0xFFFF0000u);
      bf16x2 p{(bf16)lo, (bf16)hi};
      r[i] = __builtin_bit_cast(uint32_t, p);
    }
    return r;
  } else {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(__uint_as_float(w[i]) * __uint_as_float(gw[i]));
    return r;
  }
}

template <typename T>
__global__ __launch_bounds__(256, 2) void kv_proj_kernel(ProjArgs a) {
  using C = ProjCfg<T>;
  // two buffer sets as distinct LDS objects, alternated statically (the k
  // loop is unrolled by two) so that the asynchronous W loads into one set are
  // never mistaken for writes to the set being read
  __shared__ __attribute__((aligned(16))) char wbuf0[C::TILE_BYTES], xbuf0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char wbuf1[C::TILE_BYTES], xbuf1[C::TILE_BYTES];
  __shared__ float rs_lds[C::BN];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, r32 = l & 31;
  const int wf = w >> 1, wt = w & 1;
  const int HD = a.Hkv * a.d;
  const int F = 2 * HD;
  const int M = a.B * a.N;
  // Workgroup -> (token tile, feature tile).  With the feature tiles split
  // evenly over the 8 XCDs (workgroups are dealt to XCDs round-robin), each
  // XCD keeps its slice of W in its own L2 while all XCDs stream the same
  // token tiles of X at the same time (X is read from HBM about once).
  const int nft = F / C::BM;
  const int ntt = (M + C::BN - 1) / C::BN;
  const int id = blockIdx.x;
  int tt, ft;
  if (nft % 8 == 0) {
    const int per = nft / 8, xcd = id & 7, sl = id >> 3;
    ft = xcd * per + sl % per;
    tt = sl / per;
  } else {
    ft = id % nft;
    tt = id / nft;
  }
  const int t0 = tt * C::BN;
  const int f0 = ft * C::BM;
  (void)ntt;

  // staging: chunk slot P = 256 r + tid of a tile holds row P / 8 at physical
  // chunk P % 8 (logical chunk (P % 8) ^ swizzle(row)).  W goes global -> LDS
  // directly (each wave instruction fills 64 consecutive slots); X passes
  // through registers because the row sums of squares (and the optional gain)
  // are taken on the way.  Rows past the end are clamped to the last row
  // (finite data; such tokens are never written).
  const int srow0 = tid >> 3, sch = tid & 7;
  const char* wsrc[C::PER_T];
  const char* xrow[C::PER_T];
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) {
    const int slot = 256 * r + 64 * w + l;          // == 256 r + tid
    const int row = slot >> 3, pch = slot & 7;
    const int frow = f0 + row;                        // F is a multiple of 128: always valid
    const void* wmat = frow < HD ? a.w_k : a.w_v;
    const int fr = frow < HD ? frow : frow - HD;
    wsrc[r] = static_cast<const char*>(wmat) + (size_t)fr * a.D * C::E + ((pch ^ swz8(row)) << 4);
    const int trow = min(t0 + srow0 + 32 * r, M - 1);
    xrow[r] = static_cast<const char*>(a.x) + (size_t)trow * a.D * C::E + sch * 16;
  }
  float ss[C::PER_T];
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) ss[r] = 0.f;

  u32x4 xr[C::PER_T];
  auto load_stage = [&](int ks, char* wdst) {
    const size_t koff = (size_t)ks * C::BKK * C::E;
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(wsrc[r] + koff),
                                       (__attribute__((address_space(3))) void*)(wdst + (256 * r + 64 * w) * 16),
                                       16, 0, 0);
      xr[r] = *reinterpret_cast<const u32x4*>(xrow[r] + koff);
    }
  };
  auto store_stage = [&](char* xdst, int ks) {
    u32x4 gw{0, 0, 0, 0};
    if (a.norm_w != nullptr)
      gw = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.norm_w) + (size_t)ks * C::BKK * C::E + sch * 16);
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int row = srow0 + 32 * r;
      ss[r] += chunk_sumsq<T>(xr[r]);
      const u32x4 xv = a.norm_w != nullptr ? chunk_scale<T>(xr[r], gw) : xr[r];
      *reinterpret_cast<u32x4*>(xdst + row * 128 + ((sch ^ swz8(row)) << 4)) = xv;
    }
  };
  // W's LDS writes land asynchronously: wait for them before the barrier
  auto landed = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x16{};

  const int nks = a.D / C::BKK;
  // one k stage: multiply from (wt_tile, xt_tile) while stage ks+1 is staged into (wn, xn)
  auto kstep = [&](int ks, const char* wt_tile, const char* xt_tile, char* wn, char* xn) __attribute__((always_inline)) {
    const bool has_next = ks + 1 < nks;
    if (has_next) load_stage(ks + 1, wn);
#pragma unroll
    for (int kc = 0; kc < C::NKS; ++kc) {
      typename Elem<T>::frag af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = lds_frag_row<T>(wt_tile, wf * 64 + i * 32 + r32, kc, g);
        bfr[i] = lds_frag_row<T>(xt_tile, wt * 64 + i * 32 + r32, kc, g);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mma32(af[i], bfr[jj], acc[i][jj]);
    }
    if (has_next) {
      store_stage(xn, ks + 1);
      landed();
    }
    __syncthreads();
  };
  load_stage(0, wbuf0);
  store_stage(xbuf0, 0);
  landed();
  __syncthreads();
  for (int ks = 0; ks < nks; ks += 2) {
    kstep(ks, wbuf0, xbuf0, wbuf1, xbuf1);
    if (ks + 1 < nks) kstep(ks + 1, wbuf1, xbuf1, wbuf0, xbuf0);
  }

  // Row factors: the 8 threads of a staging row group hold partial sums.
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) {
    float s = ss[r];
    s += dpp_f32<kDppQuadSwap1>(s);
    s += dpp_f32<kDppQuadSwap2>(s);
    s += dpp_f32<kDppRowHalfMirror>(s);
    if (sch == 0) rs_lds[srow0 + 32 * r] = 1.0f / sqrtf(s / (float)a.D + a.eps);
  }
  __syncthreads();

  // Epilogue: acc[i][jj][e] = C^T[feature f0 + wf*64 + i*32 + 8*(e/4) + 4g + e%4][token t0 + wt*64 + jj*32 + r32]
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tl = wt * 64 + jj * 32 + r32;
    const int tok = t0 + tl;
    if (tok >= M) continue;
    const float rs = rs_lds[tl];
    const int bb = tok / a.N, n = tok % a.N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int f = f0 + wf * 64 + i * 32 + 8 * qd + 4 * g;
        if (f >= F) continue;
        const int which = f >= HD;
        const int fr = which ? f - HD : f;
        const int hh = fr / a.d, c = fr % a.d;
        T* dst = static_cast<T*>(which ? a.v_out : a.k_out) +
                 ((size_t)(bb * a.Hkv + hh) * a.n_cap + a.pos0 + n) * a.d + c;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][jj][4 * qd + e] * rs;
        if (a.rope_log2_theta != 0.0 && !which) {   // keys only, at their cache position
          const long long p = a.pos0 + n;
          rope_pair(v[0], v[1], (double)p * rope_inv_freq(c >> 1, a.d, a.rope_log2_theta));
          rope_pair(v[2], v[3], (double)p * rope_inv_freq((c >> 1) + 1, a.d, a.rope_log2_theta));
        }
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)v[e];
          *reinterpret_cast<bf16x4*>(dst) = v4;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

hipError_t launch_kv_proj(const ProjArgs& a, bool is_bf16, hipStream_t stream) {
  const int F = 2 * a.Hkv * a.d;
  const int M = a.B * a.N;
  dim3 grid((unsigned)(((long long)(M + 127) / 128) * (F / 128)));
  if (is_bf16)
    hipLaunchKernelGGL((kv_proj_kernel<bf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((kv_proj_kernel<float>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace yoco
