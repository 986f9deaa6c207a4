// Position-wise layers of a YOCO block on the matrix cores: the pre-norm
// Q/K/V projection, the SwiGLU feed-forward's gate/up product, and the
// residual products (attention output projection, feed-forward down
// projection).
//
// What is computed (YOCO podcast transcript, segment 12: each layer runs its
// attention on the normalised input plus a residual, followed by a SwiGLU
// feed-forward; a cross-decoder layer keeps only its own query projection):
// with n_t = x_t / sqrt(mean(x_t^2) + eps) * gamma for token t,
//   QKV:     q[b, h, t, c] = n_t . W_q[h*d + c]   (k, v likewise, head-major)
//   SwiGLU:  h_t[j] = silu(n_t . W_gate[j]) * (n_t . W_up[j]),  silu(z) = z sigmoid(z)
//   residual: y_t += a_t W^T, where a_t is a row of a [B, N, K] matrix or the
//            concatenation over heads of a head-major [B, H, N, K/H] tensor
//            (the attention output feeding W_o).
//
// Design (MI355X-first), one kernel template per tile shape for the three forms:
//  * C^T = W X^T on 32x32x16 bf16 MFMA (32x32x2 f32 for float32).  Each
//    lane's results are 4 consecutive features of one token, so every
//    epilogue stores 4 contiguous values.
//  * bf16 with at least 512 tokens: the wide tile further below (256 x 256,
//    4 waves of 128 x 128, a 4-stage ring of direct loads).  float32, and
//    bf16 with fewer tokens (one-token decode steps, where a wide tile would
//    leave most of the chip idle): 128 features x 128 tokens per 256-thread
//    workgroup, 4 waves of 64 x 64, k in stages of 128 bytes per row,
//    double-buffered LDS in distinct objects with XOR-swizzled 16-byte chunks.
//  * W tiles go global -> LDS directly; X passes through registers, where the
//    RMSNorm sum of squares is taken from the values being moved (X is read
//    once) and the row factor is applied to the float32 accumulator.  The
//    head-major gather of the attention output is a per-stage address.
//  * SwiGLU: a tile's 128 weight rows are 32 gate rows, the 32 matching up
//    rows, and again, so one wave holds gate and up of the same (feature,
//    token) pairs in two accumulators and the activation is formed in
//    registers; the hidden activations are written once.
//  * Feature tiles are split evenly over the 8 XCDs when they divide, so each
//    XCD keeps its slice of W in its own L2 while the token tiles stream.
#include "common.hpp"
#include "launch.hpp"

namespace yoco {

template <typename T>
struct LinCfg {
  static constexpr int E = Elem<T>::bytes;
  static constexpr int BKK = 128 / E;            // k elements per stage (128-byte rows)
  static constexpr int PER_T = 128 * 8 / 256;    // 16-byte chunks per thread per operand (= 4)
  static constexpr int NKS = BKK / 16;           // matrix-core k steps per stage
  static constexpr int TILE_BYTES = 128 * 128;
};

// 16-byte chunk swizzle within a 128-byte row: the 32 rows a wave reads at
// once spread over all LDS banks.
__device__ __forceinline__ int lin_swz(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag lin_frag(const char* tile, int row, int kc, int g) {
  const char* rowp = tile + row * 128;
  const int sw = lin_swz(row);
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    f = *reinterpret_cast<const bf16x8*>(rowp + (((2 * kc + g) ^ sw) << 4));
  } else {
    const int ch = 4 * kc + 2 * g;
    f32x4 a = *reinterpret_cast<const f32x4*>(rowp + ((ch ^ sw) << 4));
    f32x4 b = *reinterpret_cast<const f32x4*>(rowp + (((ch + 1) ^ sw) << 4));
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

template <typename T>
__device__ __forceinline__ float lin_sumsq(u32x4 w) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = w[i];
      const bf16x2 x = __builtin_bit_cast(bf16x2, wi);
      s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);   // bf16 squares are exact in float32
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

template <typename T>
__device__ __forceinline__ u32x4 lin_gain(u32x4 w, u32x4 gw) {
  u32x4 r;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16) * __uint_as_float(gw[i] << 16);
      const float hi = __uint_as_float(w[i] & 0xFFFF0000u) * __uint_as_float(gw[i] & 0xFFFF0000u);
      bf16x2 p{(bf16)lo, (bf16)hi};
      r[i] = __builtin_bit_cast(uint32_t, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(__uint_as_float(w[i]) * __uint_as_float(gw[i]));
  }
  return r;
}

// z * sigmoid(z); the fast division is exact enough for float32 and bf16 outputs
// (a denominator that overflows gives 0, the limit for z -> -inf)
__device__ __forceinline__ float silu_f32(float z) { return __fdividef(z, 1.f + __expf(-z)); }

template <typename T>
__device__ __forceinline__ void store4(T* dst, float v0, float v1, float v2, float v3) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v{(bf16)v0, (bf16)v1, (bf16)v2, (bf16)v3};
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
  }
}

template <typename T>
__device__ __forceinline__ f32x4 load4(const T* src) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(src);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(src);
  }
}

// Rotary embedding of channels c .. c+3 (pairs (c, c+1) and (c+2, c+3)) of a
// head at position p.
__device__ __forceinline__ void rope4(float& v0, float& v1, float& v2, float& v3, int c, int d, long long p,
                                      double log2_theta) {
  rope_pair(v0, v1, (double)p * rope_inv_freq(c >> 1, d, log2_theta));
  rope_pair(v2, v3, (double)p * rope_inv_freq((c >> 1) + 1, d, log2_theta));
}

template <typename T, int MODE>
__global__ __launch_bounds__(256, 2) void linear_kernel(LinArgs a) {
  using C = LinCfg<T>;
  __shared__ __attribute__((aligned(16))) char wbuf0[C::TILE_BYTES], xbuf0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char wbuf1[C::TILE_BYTES], xbuf1[C::TILE_BYTES];
  __shared__ float rs_lds[128];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, r32 = l & 31;
  const int wf = w >> 1, wt = w & 1;
  const int M = a.B * a.N;
  // features per tile: 128 weight rows; for SwiGLU they are 64 hidden features
  constexpr int FPT = MODE == kLinSwiGLU ? 64 : 128;
  const int nft = (a.F + FPT - 1) / FPT;
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
  const int t0 = tt * 128;

  // staging: chunk slot P = 256 r + tid holds tile row P / 8 at physical
  // chunk P % 8; rows past the end are clamped (finite data, never stored)
  const int srow0 = tid >> 3, sch = tid & 7;
  const char* wsrc[C::PER_T];
  size_t xoff[C::PER_T];
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) {
    const int slot = 256 * r + 64 * w + l;
    const int row = slot >> 3, pch = slot & 7;
    const void* wm;
    int fr;
    if constexpr (MODE == kLinSwiGLU) {
      const int hf = min(ft * 64 + (row >> 6) * 32 + (row & 31), a.F - 1);
      wm = (row & 32) ? a.w1 : a.w0;
      fr = hf;
    } else {
      const int f = min(ft * 128 + row, a.F - 1);
      if (MODE == kLinQKV && f >= a.f2) { wm = a.w2; fr = f - a.f2; }
      else if (MODE == kLinQKV && f >= a.f1) { wm = a.w1; fr = f - a.f1; }
      else { wm = a.w0; fr = f; }
    }
    wsrc[r] = static_cast<const char*>(wm) + (size_t)fr * a.K * C::E + ((pch ^ lin_swz(row)) << 4);
    const int trow = min(t0 + srow0 + 32 * r, M - 1);
    if (a.x_heads > 0) {
      const int dh = a.K / a.x_heads, bb = trow / a.N, n = trow % a.N;
      xoff[r] = ((size_t)bb * a.x_heads * a.N + n) * dh * C::E + sch * 16;
    } else {
      xoff[r] = (size_t)trow * a.K * C::E + sch * 16;
    }
  }
  const char* xbase = static_cast<const char*>(a.x);
  auto x_stage_off = [&](int ks) -> size_t {
    const int k0 = ks * C::BKK;
    if (a.x_heads > 0) {
      const int dh = a.K / a.x_heads, h = k0 / dh, c0 = k0 % dh;
      return ((size_t)h * a.N * dh + c0) * C::E;
    }
    return (size_t)k0 * C::E;
  };

  float ss[C::PER_T];
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) ss[r] = 0.f;
  u32x4 xr[C::PER_T];
  auto load_stage = [&](int ks, char* wdst) {
    const size_t koff = (size_t)ks * C::BKK * C::E;
    const size_t xo = x_stage_off(ks);
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(wsrc[r] + koff),
                                       (__attribute__((address_space(3))) void*)(wdst + (256 * r + 64 * w) * 16),
                                       16, 0, 0);
      xr[r] = *reinterpret_cast<const u32x4*>(xbase + xoff[r] + xo);
    }
  };
  const bool norm = MODE != kLinResidual && a.norm;
  auto store_stage = [&](char* xdst, int ks) {
    u32x4 gw{0, 0, 0, 0};
    const bool gain = norm && a.norm_w != nullptr;
    if (gain)
      gw = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.norm_w) + (size_t)ks * C::BKK * C::E + sch * 16);
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int row = srow0 + 32 * r;
      if (norm) ss[r] += lin_sumsq<T>(xr[r]);
      const u32x4 xv = gain ? lin_gain<T>(xr[r], gw) : xr[r];
      *reinterpret_cast<u32x4*>(xdst + row * 128 + ((sch ^ lin_swz(row)) << 4)) = xv;
    }
  };
  // the direct W writes into LDS land asynchronously: wait before the barrier
  auto landed = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x16{};

  const int nks = a.K / C::BKK;
  auto kstep = [&](int ks, const char* wt_tile, const char* xt_tile, char* wn, char* xn) __attribute__((always_inline)) {
    const bool has_next = ks + 1 < nks;
    if (has_next) load_stage(ks + 1, wn);
#pragma unroll
    for (int kc = 0; kc < C::NKS; ++kc) {
      typename Elem<T>::frag af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = lin_frag<T>(wt_tile, wf * 64 + i * 32 + r32, kc, g);
        bfr[i] = lin_frag<T>(xt_tile, wt * 64 + i * 32 + r32, kc, g);
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

  if (norm) {
    // the 8 threads of a staging row hold partial sums of squares
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      float s = ss[r];
      s += dpp_f32<kDppQuadSwap1>(s);
      s += dpp_f32<kDppQuadSwap2>(s);
      s += dpp_f32<kDppRowHalfMirror>(s);
      if (sch == 0) rs_lds[srow0 + 32 * r] = 1.0f / sqrtf(s / (float)a.K + a.eps);
    }
    __syncthreads();
  }

  // acc[i][jj][e] = C^T[tile row wf*64 + i*32 + 8*(e/4) + 4g + e%4][token t0 + wt*64 + jj*32 + r32]
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tl = wt * 64 + jj * 32 + r32;
    const int tok = t0 + tl;
    if (tok >= M) continue;
    const float rs = norm ? rs_lds[tl] : 1.f;
    const int bb = tok / a.N, n = tok % a.N;
    if constexpr (MODE == kLinSwiGLU) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int hf = ft * 64 + wf * 32 + 8 * qd + 4 * g;
        if (hf >= a.F) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = silu_f32(acc[0][jj][4 * qd + e] * rs) * (acc[1][jj][4 * qd + e] * rs);
        store4<T>(static_cast<T*>(a.y0) + (size_t)tok * a.F + hf, v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int f = ft * 128 + wf * 64 + i * 32 + 8 * qd + 4 * g;
          if (f >= a.F) continue;
          float v0 = acc[i][jj][4 * qd] * rs, v1 = acc[i][jj][4 * qd + 1] * rs;
          float v2 = acc[i][jj][4 * qd + 2] * rs, v3 = acc[i][jj][4 * qd + 3] * rs;
          if constexpr (MODE == kLinQKV) {
            void* out;
            int fr, H;
            size_t rows = (size_t)a.N, row0 = 0;
            if (f >= a.f2) { out = a.y2; fr = f - a.f2; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
            else if (f >= a.f1) { out = a.y1; fr = f - a.f1; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
            else { out = a.y0; fr = f; H = a.h0; }
            const int hh = fr / a.d, c = fr % a.d;
            if (a.rope_log2_theta != 0.0 && f < a.f2) rope4(v0, v1, v2, v3, c, a.d, a.rope_pos0 + n, a.rope_log2_theta);
            store4<T>(static_cast<T*>(out) + (((size_t)bb * H + hh) * rows + row0 + n) * a.d + c, v0, v1, v2, v3);
          } else {
            T* dst = static_cast<T*>(a.y0) + (size_t)tok * a.F + f;
            const f32x4 old = load4<T>(dst);
            store4<T>(dst, old[0] + v0, old[1] + v1, old[2] + v2, old[3] + v3);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 form with a wide tile: TM = 64 NI weight rows (192 or 256) x TN
// tokens (256 or 128) per workgroup, 4 waves of TM/2 x TN/2 (an NI x TN/64
// block of 32x32 MFMA tiles, the accumulators in the matrix-core register
// file), k in stages of 32 through a 4-stage LDS ring filled by direct global
// -> LDS loads three stages ahead.  At 256 x 256 a wave reads 8 fragments per
// k step for 16 MFMAs (0.5 KB of LDS per MFMA, half the 64 x 64 tile's), and
// the loads in flight cover the HBM latency.  The row count per tile is
// chosen per shape so that the tiles fill whole rounds of the chip: the 3B
// block's 3072-wide products make 16 x 16 tiles of 192 x 256 (one round
// instead of three quarters of one with 256 x 256), its Q/K/V product (5120
// rows) 27 x 16 (1.7 rounds instead of 1.25).  (320-row tiles would make one
// round of the latter but need more than 512 registers per lane.)  The RMSNorm sums of
// squares are taken from the staged token rows in LDS; a norm gain is staged
// with each k slice and applied to the token fragments in registers (x * gamma
// rounded to bf16, as in the 128 x 128 form).
// ---------------------------------------------------------------------------
namespace wide {
constexpr int BK = 32;                  // k per stage: 64 bytes per row
constexpr int NST = 4;                  // ring stages
constexpr int GB = 256;                 // per-wave gain slice of one stage (64 bytes used)
template <int TM, int TN>
constexpr int stage_bytes() { return TM * 64 + TN * 64 + 4 * GB; }   // weight rows, token rows, gain
template <int TM, int TN>
constexpr int lds_bytes() { return NST * stage_bytes<TM, TN>() + 512 * 4; }   // ring, then rs[256], ssp[256]
}  // namespace wide

// 16-byte chunk swizzle for 64-byte rows: rows r, r+4, r+8, r+12 (which share
// a group of banks) hold a given chunk at four different positions.
__device__ __forceinline__ int wswz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ bf16x8 wide_frag(const char* op, int row, int kc, int g) {
  return *reinterpret_cast<const bf16x8*>(op + row * 64 + (((2 * kc + g) ^ wswz(row)) << 4));
}

// One direct global -> LDS load of 16 bytes per lane: lane l writes LDS bytes
// [m0 + 16 l, m0 + 16 l + 16).  Written in inline assembly so that the
// compiler's wait insertion does not drain the ring before every LDS read (it
// cannot tell the four stages apart); the ring's waits are explicit.
__device__ __forceinline__ void dma16(const void* src, unsigned m0) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(m0)
      : "memory");
}
__device__ __forceinline__ void dma4(const void* src, unsigned m0) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(m0)
      : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// TN tokens per tile (256, or 128 when that keeps more of the chip busy),
// NI 32-row blocks per wave: 4 waves as 2 (weight-row halves of TM / 2) x 2
// (token halves of TN / 2).
template <int MODE, bool GAIN, int TN, int NI>
__global__ __launch_bounds__(256, 1) void linear_wide_kernel(LinArgs a) {
  using namespace wide;
  constexpr int TM = 64 * NI;             // weight rows per tile
  constexpr int OPW = TM * 64;            // the weight operand of one stage (bytes)
  static_assert(MODE != kLinSwiGLU || NI == 4, "the SwiGLU row interleave is laid out for 256 rows");
  constexpr int STB = stage_bytes<TM, TN>();
  constexpr int NJ = TN / 64;             // 32-token blocks per wave
  constexpr int XR = TN / 64;             // token-operand loads per thread per stage
  constexpr int TPT = 256 / TN;           // threads per token for the norm sums
  extern __shared__ __attribute__((aligned(16))) char ring[];
  float* rs_lds = reinterpret_cast<float*>(ring + NST * STB);
  float* ssp_lds = rs_lds + 256;
  constexpr bool NORM = MODE != kLinResidual;
  constexpr int PER = NI + XR + (GAIN ? 1 : 0);   // loads per thread per stage
  constexpr int NR = NI > XR ? NI : XR;            // staging slots per thread

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 5, r32 = l & 31;
  const int wf = w >> 1, wt = w & 1;
  const int M = a.B * a.N;
  constexpr int FPT = MODE == kLinSwiGLU ? 128 : TM;   // output features per tile
  const int nft = (a.F + FPT - 1) / FPT;
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
  const int t0 = tt * TN;

  // staging addresses: slot P = 256 r + tid of an operand holds row P / 4 at
  // physical chunk P % 4 (logical chunk (P % 4) ^ wswz(row)); rows past the
  // end are clamped (finite data, never stored)
  const char* wsrc[NI];
  const char* xsrc[XR];
  const int dh = a.x_heads > 0 ? a.K / a.x_heads : a.K;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int slot = 256 * r + tid;
    const int row = slot >> 2, lch = (slot & 3) ^ wswz(row);
    if (r < NI) {
      const void* wm;
      int fr;
      if constexpr (MODE == kLinSwiGLU) {
        const int blk = (row >> 5) & 3;
        fr = min(ft * 128 + (row >> 7) * 64 + (blk >> 1) * 32 + (row & 31), a.F - 1);
        wm = (blk & 1) ? a.w1 : a.w0;
      } else {
        const int f = min(ft * TM + row, a.F - 1);
        if (MODE == kLinQKV && f >= a.f2) { wm = a.w2; fr = f - a.f2; }
        else if (MODE == kLinQKV && f >= a.f1) { wm = a.w1; fr = f - a.f1; }
        else { wm = a.w0; fr = f; }
      }
      wsrc[r] = static_cast<const char*>(wm) + (size_t)fr * a.K * 2 + lch * 16;
    }
    if (r < XR) {
      const int trow = min(t0 + row, M - 1);
      if (a.x_heads > 0) {
        const int bb = trow / a.N, n = trow % a.N;
        xsrc[r] = static_cast<const char*>(a.x) + ((size_t)bb * a.x_heads * a.N + n) * dh * 2 + lch * 16;
      } else {
        xsrc[r] = static_cast<const char*>(a.x) + (size_t)trow * a.K * 2 + lch * 16;
      }
    }
  }
  const unsigned ring_base = (unsigned)(uintptr_t)ring;
  const int nks = a.K / BK;
  auto issue = [&](int ks) {
    const unsigned sb = ring_base + (unsigned)((ks & (NST - 1)) * STB);
    const size_t wo = (size_t)ks * BK * 2;
    size_t xo = wo;
    if (a.x_heads > 0) {
      const int k0 = ks * BK, h = k0 / dh, c0 = k0 % dh;
      xo = ((size_t)h * a.N * dh + c0) * 2;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + (unsigned)((256 * r + 64 * w) * 16));
      if (r < NI) dma16(wsrc[r] + wo, m0);
      if (r < XR) dma16(xsrc[r] + xo, m0 + OPW);
    }
    if constexpr (GAIN) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + (unsigned)(OPW + TN * 64 + w * GB));
      dma4(static_cast<const char*>(a.norm_w) + wo + 4 * min(l, 15), m0);
    }
  };

  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  float ss = 0.f;

  // Fragments of one k step (16 deep) of a stage: NI weight-row blocks, NJ token blocks.
  struct Frags {
    bf16x8 a[NI], b[NJ];
  };
  auto read_frags = [&](int ks, int kc, Frags& f) __attribute__((always_inline)) {
    const char* S = ring + (ks & (NST - 1)) * STB;
#pragma unroll
    for (int i = 0; i < NI; ++i) f.a[i] = wide_frag(S, wf * (TM / 2) + i * 32 + r32, kc, g);
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[j] = wide_frag(S + OPW, wt * (TN / 2) + j * 32 + r32, kc, g);
    if constexpr (GAIN) {
      const bf16x8 gm = *reinterpret_cast<const bf16x8*>(S + OPW + TN * 64 + w * GB + (kc * 16 + 8 * g) * 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) f.b[j][e] = (bf16)((float)f.b[j][e] * (float)gm[e]);
    }
  };
  auto mma_frags = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mma32(f.a[i], f.b[j], acc[i][j]);
  };
  // stage ks has landed (in every wave) once at most min(2, nks - 1 - ks)
  // later stages are in flight and the waves have met
  auto landed = [&](int ks) __attribute__((always_inline)) {
    const int ahead = min(2, nks - 1 - ks);
    if (ahead == 2) vm_wait<2 * PER>();
    else if (ahead == 1) vm_wait<PER>();
    else vm_wait<0>();
    lds_barrier();
  };
  // sums of squares of the staged token rows: token tid % TN, chunks of part tid / TN
  auto norm_sums = [&](int ks) __attribute__((always_inline)) {
    if constexpr (NORM) {
      const char* Xt = ring + (ks & (NST - 1)) * STB + OPW;
      const int tk = tid % TN, part = tid / TN;
#pragma unroll
      for (int cc = 0; cc < 4 / TPT; ++cc) {
        const int c = part * (4 / TPT) + cc;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Xt + tk * 64 + ((c ^ wswz(tk)) << 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wi = v[i];
          const bf16x2 x = __builtin_bit_cast(bf16x2, wi);
          ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
        }
      }
    }
  };

  // Pipeline: the fragments of the next k step are read while the current
  // one's MFMAs run; the wait for the next stage (and the refill of the slot
  // every wave has finished reading) sits between a stage's two k steps.  The
  // last stage is peeled off so that the loop body has no join of LDS read
  // streams (a join makes the compiler drain the prefetched fragments).  The
  // scheduling groups alternate MFMAs with the next block's LDS reads, one
  // read per MFMA, so the reads neither queue up in bursts nor leave the
  // matrix core idle.
  issue(0);
  if (nks > 1) issue(1);
  if (nks > 2) issue(2);
  landed(0);
  Frags f0, f1;
  read_frags(0, 0, f0);
  constexpr int NM = NI * NJ;                                // MFMAs per k step
  constexpr int NR0 = NI + NJ + (NORM ? 4 / TPT : 0);        // LDS reads in the first half
  constexpr int NR1 = NI + NJ;
  static_assert(NR0 <= NM && NR1 <= NM, "one read per MFMA");
  for (int ks = 0; ks + 1 < nks; ++ks) {
    read_frags(ks, 1, f1);
    norm_sums(ks);
    mma_frags(f0);
#pragma unroll
    for (int q = 0; q < NR0; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR0, 0);
    landed(ks + 1);                     // also: every wave is done with stage ks - 1
    if (ks + 3 < nks) issue(ks + 3);    // into the slot of stage ks - 1
    read_frags(ks + 1, 0, f0);
    mma_frags(f1);
#pragma unroll
    for (int q = 0; q < NR1; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR1, 1);
  }
  read_frags(nks - 1, 1, f1);
  mma_frags(f0);
  norm_sums(nks - 1);
  mma_frags(f1);

  if constexpr (NORM) {
    ssp_lds[tid] = ss;
    lds_barrier();
    if (tid < TN) {
      float t = 0.f;
#pragma unroll
      for (int pp = 0; pp < TPT; ++pp) t += ssp_lds[pp * TN + tid];
      rs_lds[tid] = 1.0f / sqrtf(t / (float)a.K + a.eps);
    }
    lds_barrier();
  }

  // acc[i][j][e] = C^T[tile row wf*TM/2 + i*32 + 8*(e/4) + 4g + e%4][token t0 + wt*TN/2 + j*32 + r32]
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int tl = wt * (TN / 2) + j * 32 + r32;
    const int tok = t0 + tl;
    if (tok >= M) continue;
    const float rs = NORM ? rs_lds[tl] : 1.f;
    const int bb = tok / a.N, n = tok % a.N;
    if constexpr (MODE == kLinSwiGLU) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int hf = ft * 128 + wf * 64 + (i >> 1) * 32 + 8 * qd + 4 * g;
          if (hf >= a.F) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = silu_f32(acc[i][j][4 * qd + e] * rs) * (acc[i + 1][j][4 * qd + e] * rs);
          store4<bf16>(static_cast<bf16*>(a.y0) + (size_t)tok * a.F + hf, v[0], v[1], v[2], v[3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int f = ft * TM + wf * (TM / 2) + i * 32 + 8 * qd + 4 * g;
          if (f >= a.F) continue;
          float v0 = acc[i][j][4 * qd] * rs, v1 = acc[i][j][4 * qd + 1] * rs;
          float v2 = acc[i][j][4 * qd + 2] * rs, v3 = acc[i][j][4 * qd + 3] * rs;
          if constexpr (MODE == kLinQKV) {
            void* out;
            int fr, H;
            size_t rows = (size_t)a.N, row0 = 0;
            if (f >= a.f2) { out = a.y2; fr = f - a.f2; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
            else if (f >= a.f1) { out = a.y1; fr = f - a.f1; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
            else { out = a.y0; fr = f; H = a.h0; }
            const int hh = fr / a.d, c = fr % a.d;
            if (a.rope_log2_theta != 0.0 && f < a.f2) rope4(v0, v1, v2, v3, c, a.d, a.rope_pos0 + n, a.rope_log2_theta);
            store4<bf16>(static_cast<bf16*>(out) + (((size_t)bb * H + hh) * rows + row0 + n) * a.d + c, v0, v1, v2, v3);
          } else {
            bf16* dst = static_cast<bf16*>(a.y0) + (size_t)tok * a.F + f;
            const f32x4 old = load4<bf16>(dst);
            store4<bf16>(dst, old[0] + v0, old[1] + v1, old[2] + v2, old[3] + v3);
          }
        }
      }
    }
  }
}

// Number of compute units (queried once per process; every GPU it runs on is
// the same model).
static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <int MODE, bool GAIN, int TN, int NI>
static void launch_wide(const LinArgs& a, long long tiles, hipStream_t stream) {
  constexpr int lds = wide::lds_bytes<64 * NI, TN>();
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_wide_kernel<MODE, GAIN, TN, NI>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr_set = true;
  }
  hipLaunchKernelGGL((linear_wide_kernel<MODE, GAIN, TN, NI>), dim3((unsigned)tiles), dim3(256), lds, stream, a);
}

// Tile shape per problem: the one with the best expected rate -- a per-CU
// rate for the shape (from its LDS bytes per MFMA: 256 x 256 1.0, 192 x 256
// 0.95, 256 x 128 0.9) times the useful fraction of its padded tiles times
// the fraction of the last round's CUs that are busy (one workgroup per CU).
template <int MODE, bool GAIN>
static void launch_wide_tn(const LinArgs& a, hipStream_t stream) {
  const long long M = (long long)a.B * a.N, cus = cu_count();
  struct Shape { int tm, tn; double rate; };
  const Shape shapes[] = {{256, 256, 1.0}, {256, 128, 0.9}, {192, 256, 0.95}};
  int best = 0;
  double best_eff = -1.0;
  long long best_tiles = 0;
  for (int i = 0; i < 3; ++i) {
    const Shape& sh = shapes[i];
    if (MODE == kLinSwiGLU && sh.tm != 256) continue;
    const int fpt = MODE == kLinSwiGLU ? 128 : sh.tm;
    const long long nft = (a.F + fpt - 1) / fpt, ntt = (M + sh.tn - 1) / sh.tn, tiles = nft * ntt;
    const double useful = (double)a.F / (double)(nft * fpt) * (double)M / (double)(ntt * sh.tn);
    const double eff = sh.rate * useful * (double)tiles / (double)(((tiles + cus - 1) / cus) * cus);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = i;
      best_tiles = tiles;
    }
  }
  switch (best) {
    case 0: launch_wide<MODE, GAIN, 256, 4>(a, best_tiles, stream); break;
    case 1: launch_wide<MODE, GAIN, 128, 4>(a, best_tiles, stream); break;
    default: if constexpr (MODE != kLinSwiGLU) launch_wide<MODE, GAIN, 256, 3>(a, best_tiles, stream); break;
  }
}

// ---------------------------------------------------------------------------
// bf16 form for a handful of tokens (one-token decode steps, the early-exit
// last row): the product is bound by reading W once, so a workgroup takes 16
// weight rows and spreads their K range over 16 waves (every load in flight at
// once); each wave forms a 16 x 16 block (16 rows x the tokens, padded to 16)
// on 16x16x32 MFMA, the 16 partial blocks are summed in LDS, and the epilogue
// runs per (row, token).  SwiGLU: the 16 rows are 8 gate rows and the 8
// matching up rows.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 16;
constexpr int kSkinnyMaxTokens = 64;

template <int MODE, bool GAIN>
__global__ __launch_bounds__(1024, 1) void linear_skinny_kernel(LinArgs a) {
  __shared__ float part[kSkinnyWaves][256];
  __shared__ float ssp[kSkinnyWaves][64];
  __shared__ float rs[16];
  constexpr bool NORM = MODE != kLinResidual;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int lr = l & 15, lk = l >> 4;   // MFMA lane roles: row / token l % 16, k group l / 16
  const int M = a.B * a.N;
  const int tg0 = blockIdx.y * 16;
  const int fg = blockIdx.x;

  // A operand: weight row of MFMA row lr
  const bf16* wrow;
  if constexpr (MODE == kLinSwiGLU) {
    const int hf = min(fg * 8 + (lr & 7), a.F - 1);
    wrow = static_cast<const bf16*>(lr >= 8 ? a.w1 : a.w0) + (size_t)hf * a.K;
  } else {
    const int f = min(fg * 16 + lr, a.F - 1);
    const void* wm;
    int fr;
    if (MODE == kLinQKV && f >= a.f2) { wm = a.w2; fr = f - a.f2; }
    else if (MODE == kLinQKV && f >= a.f1) { wm = a.w1; fr = f - a.f1; }
    else { wm = a.w0; fr = f; }
    wrow = static_cast<const bf16*>(wm) + (size_t)fr * a.K;
  }
  // B operand: token tg0 + lr (zero when past the end)
  const int tok = tg0 + lr;
  const bool tok_ok = tok < M;
  const int tcl = min(tok, M - 1);
  const int dh = a.x_heads > 0 ? a.K / a.x_heads : a.K;
  const bf16* xrow = static_cast<const bf16*>(a.x) +
                     (a.x_heads > 0 ? ((size_t)(tcl / a.N) * a.x_heads * a.N + tcl % a.N) * dh : (size_t)tcl * a.K);
  auto xat = [&](int k) -> const bf16* {   // element k of this token's row
    if (a.x_heads > 0) return xrow + (size_t)(k / dh) * a.N * dh + k % dh;
    return xrow + k;
  };

  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float ssl = 0.f;
  const int nk = a.K / 32;
  constexpr int U = 4;
  for (int ks0 = w; ks0 < nk; ks0 += kSkinnyWaves * U) {
    bf16x8 wa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * kSkinnyWaves;
      const int k = (ks < nk ? ks : nk - 1) * 32 + lk * 8;
      wa[u] = *reinterpret_cast<const bf16x8*>(wrow + k);
      xb[u] = *reinterpret_cast<const bf16x8*>(xat(k));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * kSkinnyWaves;
      if (ks >= nk) break;
      bf16x8 x = tok_ok ? xb[u] : bf16x8{};
      if constexpr (NORM) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 p{x[e], x[e + 1]};
          ssl = __builtin_amdgcn_fdot2_f32_bf16(p, p, ssl, false);
        }
      }
      if constexpr (GAIN) {
        const bf16x8 gm = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.norm_w) + ks * 32 + lk * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * (float)gm[e]);
      }
      acc = mma16(wa[u], x, acc);
    }
  }
  // acc[i] = C[row 4*lk + i][token lr]
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w][(4 * lk + i) * 16 + lr] = acc[i];
  ssp[w][l] = ssl;
  __syncthreads();
  if (NORM && tid < 16) {
    float t = 0.f;
    for (int ww = 0; ww < kSkinnyWaves; ++ww)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) t += ssp[ww][g4 * 16 + tid];
    rs[tid] = 1.0f / sqrtf(t / (float)a.K + a.eps);
  }
  __syncthreads();
  // epilogue: thread e -> (row e / 16, token e % 16)
  const int row = tid >> 4, t = tid & 15, tk = tg0 + t;
  if (tid >= (MODE == kLinSwiGLU ? 128 : 256) || tk >= M) return;
  auto sum_rows = [&](int r) {
    float v = 0.f;
    for (int ww = 0; ww < kSkinnyWaves; ++ww) v += part[ww][r * 16 + t];
    return NORM ? v * rs[t] : v;
  };
  const int bb = tk / a.N, n = tk % a.N;
  if constexpr (MODE == kLinSwiGLU) {
    const int hf = fg * 8 + row;
    if (hf < a.F) {
      const float gt = sum_rows(row), up = sum_rows(row + 8);
      static_cast<bf16*>(a.y0)[(size_t)tk * a.F + hf] = (bf16)(silu_f32(gt) * up);
    }
  } else {
    const int f = fg * 16 + row;
    if (f >= a.F) return;
    float v = sum_rows(row);
    if constexpr (MODE == kLinQKV) {
      void* out;
      int fr, H;
      size_t rows = (size_t)a.N, row0 = 0;
      if (f >= a.f2) { out = a.y2; fr = f - a.f2; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
      else if (f >= a.f1) { out = a.y1; fr = f - a.f1; H = a.h1; rows = a.kv_rows; row0 = a.kv_pos0; }
      else { out = a.y0; fr = f; H = a.h0; }
      const int hh = fr / a.d, c = fr % a.d;
      if (a.rope_log2_theta != 0.0 && f < a.f2) {
        // the pair partner (channel c ^ 1) is row ^ 1 of the same group of 16
        float x0 = (c & 1) ? sum_rows(row ^ 1) : v, x1 = (c & 1) ? v : sum_rows(row ^ 1);
        const double ang = (double)(a.rope_pos0 + n) * rope_inv_freq(c >> 1, a.d, a.rope_log2_theta);
        rope_pair(x0, x1, ang);
        v = (c & 1) ? x1 : x0;
      }
      static_cast<bf16*>(out)[(((size_t)bb * H + hh) * rows + row0 + n) * a.d + c] = (bf16)v;
    } else {
      bf16* dst = static_cast<bf16*>(a.y0) + (size_t)tk * a.F + f;
      *dst = (bf16)((float)*dst + v);
    }
  }
}

hipError_t launch_linear(const LinArgs& a, int mode, bool is_bf16, hipStream_t stream) {
  const int M = a.B * a.N;
  if (is_bf16 && M <= kSkinnyMaxTokens) {
    const int groups = mode == kLinSwiGLU ? (a.F + 7) / 8 : (a.F + 15) / 16;
    const dim3 grid((unsigned)groups, (unsigned)((M + 15) / 16));
    const bool gain = mode != kLinResidual && a.norm_w != nullptr;
#define YOCO_SK(MD, G) hipLaunchKernelGGL((linear_skinny_kernel<MD, G>), grid, dim3(1024), 0, stream, a)
    if (mode == kLinQKV) { if (gain) YOCO_SK(kLinQKV, true); else YOCO_SK(kLinQKV, false); }
    else if (mode == kLinSwiGLU) { if (gain) YOCO_SK(kLinSwiGLU, true); else YOCO_SK(kLinSwiGLU, false); }
    else YOCO_SK(kLinResidual, false);
#undef YOCO_SK
    return hipGetLastError();
  }
  if (is_bf16 && M >= 256) {
    const bool gain = mode != kLinResidual && a.norm_w != nullptr;
    if (mode == kLinQKV) { if (gain) launch_wide_tn<kLinQKV, true>(a, stream); else launch_wide_tn<kLinQKV, false>(a, stream); }
    else if (mode == kLinSwiGLU) { if (gain) launch_wide_tn<kLinSwiGLU, true>(a, stream); else launch_wide_tn<kLinSwiGLU, false>(a, stream); }
    else launch_wide_tn<kLinResidual, false>(a, stream);
    return hipGetLastError();
  }
  const int fpt = mode == kLinSwiGLU ? 64 : 128;
  const long long tiles = (long long)((M + 127) / 128) * ((a.F + fpt - 1) / fpt);
  const dim3 grid((unsigned)tiles);
#define YOCO_LIN(T, MD) hipLaunchKernelGGL((linear_kernel<T, MD>), grid, dim3(256), 0, stream, a)
  if (is_bf16) {   // 65 to 255 tokens: the 128 x 128 tile keeps more workgroups busy
    if (mode == kLinQKV) YOCO_LIN(bf16, kLinQKV);
    else if (mode == kLinSwiGLU) YOCO_LIN(bf16, kLinSwiGLU);
    else YOCO_LIN(bf16, kLinResidual);
  } else {
    if (mode == kLinQKV) YOCO_LIN(float, kLinQKV);
    else if (mode == kLinSwiGLU) YOCO_LIN(float, kLinSwiGLU);
    else YOCO_LIN(float, kLinResidual);
  }
#undef YOCO_LIN
  return hipGetLastError();
}

}  // namespace yoco
