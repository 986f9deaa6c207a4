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
//  * bf16 without a norm gain, when the features fill 256-row tiles and the
//    grid still covers the chip: 256 features x 128 tokens per 8-wave
//    workgroup, one workgroup per CU, a ring of three LDS stages with both
//    operands loaded global -> LDS two stages ahead, so that a stage's load
//    latency is covered by two stages of matrix work.  The row sums of
//    squares come from the X fragments each wave reads for the matrix core
//    (summed in the same order as the staging form's, so both forms give
//    identical bits).
#include "common.hpp"
#include "launch.hpp"
#include "index_map.hpp"

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

// (swz8, the XOR swizzle of 128-byte tile rows, is defined in index_map.hpp)

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
  // Workgroup -> (token tile, feature tile).  Workgroups are dealt to the 8
  // XCDs round-robin; each XCD takes one block of a 2 x 4 partition of the
  // (feature tile, token tile) grid -- half of the features, a quarter of
  // the tokens -- so that X is fetched by 2 XCDs and W by 4 (dealing only the
  // feature tiles made every XCD fetch all of X).  Workgroups of the padded
  // partition that fall outside the grid have no work.
  const int nft = F / C::BM;
  const int ntt = (M + C::BN - 1) / C::BN;
  int tt, ft;
  if (!proj_tile(blockIdx.x, nft, ntt, ft, tt)) return;
  const int t0 = tt * C::BN;
  const int f0 = ft * C::BM;

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
  // A wave's 64 features lie in one head of one of K and V (f0 is a multiple
  // of 128 and Hkv*d, d of 64).
  float amax = 0.f;   // largest |value| this lane stores (amax_bits mode)
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
                 ((size_t)(bb * a.Hkv + hh) * a.n_cap + a.row0 + n) * a.d + c;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][jj][4 * qd + e] * rs;
        if (a.rope_log2_theta != 0.0 && !which) {   // keys only, at their cache position
          const long long p = a.pos0 + n;
          rope_pair(v[0], v[1], (double)p * rope_inv_freq(c >> 1, a.d, a.rope_log2_theta));
          rope_pair(v[2], v[3], (double)p * rope_inv_freq((c >> 1) + 1, a.d, a.rope_log2_theta));
        }
        // the values as stored in the activation dtype
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (float)(bf16)v[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(v[e]));
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)v[e];   // exact: already bf16 values
          *reinterpret_cast<bf16x4*>(dst) = v4;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
  if (a.amax_bits != nullptr) {
    // per-head maxima for a following 8-bit encode: one atomic per wave
    // (integer max on the bit patterns of non-negative floats orders them
    // like their values)
    amax = row16_max(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int f = f0 + wf * 64;
    const int which = f >= HD;
    const int hh = (which ? f - HD : f) / a.d;
    if (l == 0 && amax > 0.f) atomicMax(a.amax_bits + which * a.Hkv + hh, __float_as_uint(amax));
  }
}


// ---------------------------------------------------------------------------
// Three-stage ring form (bf16, no norm gain).  Eight waves: wave w computes
// features f0 + (w >> 1) * 64 .. + 63 for tokens t0 + (w & 1) * 64 .. + 63.
// Every load is an LDS DMA issued in inline assembly, so the compiler sees
// no memory operation in flight in the k loop and adds no waits of its own;
// the loop waits for exactly the stage it needs (vmcnt) before each barrier.
// ---------------------------------------------------------------------------
struct ProjRing {
  static constexpr int BM = 256, BN = 128, NW = 8, NT = 512;
  static constexpr int BKK = 64;                   // bf16 elements per stage (128-byte rows)
  static constexpr int W_PER_T = BM * 8 / NT;      // W chunks per thread per stage (4)
  static constexpr int X_PER_T = BN * 8 / NT;      // X chunks per thread per stage (2)
  static constexpr int LOADS = W_PER_T + X_PER_T;  // loads per thread per stage
  static constexpr int W_BYTES = BM * 128, X_BYTES = BN * 128;
  static constexpr int NKS = BKK / 16;
};

// one 16-byte global -> LDS load; m0 = the wave's LDS destination.  m0 is a
// reserved register the compiler cannot be told about; it is safe here
// because nothing else in kv_proj_ring_kernel reads m0 (no LDS-DMA builtin,
// no m0-indexed instruction; the cross-lane exchanges are ds_bpermute).
__device__ __forceinline__ void proj_dma16(const char* src, unsigned lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_dst) : "memory");
}
// wait until at most N loads are in flight, then a workgroup barrier
// (the scheduling barriers keep the instruction scheduler from moving LDS
// reads of either stage across it)
template <int N>
__device__ __forceinline__ void proj_stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(512, 2) void kv_proj_ring_kernel(ProjArgs a) {
  using C = ProjRing;
  __shared__ __attribute__((aligned(16))) char wb0[C::W_BYTES], xb0[C::X_BYTES];
  __shared__ __attribute__((aligned(16))) char wb1[C::W_BYTES], xb1[C::X_BYTES];
  __shared__ __attribute__((aligned(16))) char wb2[C::W_BYTES], xb2[C::X_BYTES];
  char* const wbuf[3] = {wb0, wb1, wb2};
  char* const xbuf[3] = {xb0, xb1, xb2};

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 5, r32 = l & 31;
  const int wf = w >> 1, wt = w & 1;
  const int HD = a.Hkv * a.d;
  const int F = 2 * HD;
  const int M = a.B * a.N;
  // the same 2 x 4 XCD partition of the (feature tile, token tile) grid as
  // the staging form
  const int nft = F / C::BM;
  const int ntt = (M + C::BN - 1) / C::BN;
  int tt, ft;
  if (!proj_tile(blockIdx.x, nft, ntt, ft, tt)) return;
  const int t0 = tt * C::BN;
  const int f0 = ft * C::BM;

  // slot P = NT r + tid of a tile holds row P / 8 at physical chunk P % 8,
  // fetched from logical chunk (P % 8) ^ swizzle(row); each wave
  // instruction fills 64 consecutive slots.  Token rows past the end read
  // the last row (finite data; never written).
  const char* wsrc[C::W_PER_T];
  const char* xsrc[C::X_PER_T];
#pragma unroll
  for (int r = 0; r < C::W_PER_T; ++r) {
    const int slot = C::NT * r + tid, row = slot >> 3, pch = slot & 7;
    const int frow = f0 + row;
    const void* wmat = frow < HD ? a.w_k : a.w_v;
    const int fr = frow < HD ? frow : frow - HD;
    wsrc[r] = static_cast<const char*>(wmat) + (size_t)fr * a.D * 2 + ((pch ^ swz8(row)) << 4);
  }
#pragma unroll
  for (int r = 0; r < C::X_PER_T; ++r) {
    const int slot = C::NT * r + tid, row = slot >> 3, pch = slot & 7;
    const int trow = min(t0 + row, M - 1);
    xsrc[r] = static_cast<const char*>(a.x) + (size_t)trow * a.D * 2 + ((pch ^ swz8(row)) << 4);
  }
  // (m0 takes the LDS byte offset: the low 32 bits of a generic pointer to
  // LDS, whose aperture base is 4 GiB-aligned)
  auto issue = [&](int ks, int buf) __attribute__((always_inline)) {
    const size_t koff = (size_t)ks * C::BKK * 2;
    const unsigned wd = (unsigned)(size_t)wbuf[buf] + 64 * 16 * w;
    const unsigned xd = (unsigned)(size_t)xbuf[buf] + 64 * 16 * w;
#pragma unroll
    for (int r = 0; r < C::W_PER_T; ++r) proj_dma16(wsrc[r] + koff, __builtin_amdgcn_readfirstlane(wd + C::NT * 16 * r));
#pragma unroll
    for (int r = 0; r < C::X_PER_T; ++r) proj_dma16(xsrc[r] + koff, __builtin_amdgcn_readfirstlane(xd + C::NT * 16 * r));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x16{};
  // sums of squares of this lane's X rows (tokens wt*64 + jj*32 + r32) at
  // the 16-byte chunk position 2 wf + g of every stage: the four waves that
  // read the same rows take one k step each
  float ssc[2] = {0.f, 0.f};

  const int nks = a.D / C::BKK;
  // stage work from buffer buf; the loads of stage ks_next into buffer nbuf
  // are issued once the first k steps' fragments are requested
  auto compute = [&](int buf, int ks_next, int nbuf) __attribute__((always_inline)) {
    const char* wt_tile = wbuf[buf];
    const char* xt_tile = xbuf[buf];
    // every fragment of the stage requested ahead of its matrix steps
    bf16x8 af[C::NKS][2], bfr[C::NKS][2];
#pragma unroll
    for (int kc = 0; kc < C::NKS; ++kc) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[kc][i] = lds_frag_row<bf16>(wt_tile, wf * 64 + i * 32 + r32, kc, g);
        bfr[kc][i] = lds_frag_row<bf16>(xt_tile, wt * 64 + i * 32 + r32, kc, g);
      }
      if (kc == 1) issue(ks_next, nbuf);
    }
    // this wave's share of the row sums: its rows' chunk 2 wf + g, read again
    const bf16x8 xs0 = lds_frag_row<bf16>(xt_tile, wt * 64 + r32, wf, g);
    const bf16x8 xs1 = lds_frag_row<bf16>(xt_tile, wt * 64 + 32 + r32, wf, g);
#pragma unroll
    for (int kc = 0; kc < C::NKS; ++kc) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mma32(af[kc][i], bfr[kc][jj], acc[i][jj]);
    }
    ssc[0] += chunk_sumsq<bf16>(__builtin_bit_cast(u32x4, xs0));
    ssc[1] += chunk_sumsq<bf16>(__builtin_bit_cast(u32x4, xs1));
    // issue order: the reads of two k steps, then each k step's 4 matrix
    // steps followed by the reads two steps ahead (masks: 0x100 LDS read,
    // 0x008 MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // prologue: stages 0 and 1 in flight, wait for stage 0
  issue(0, 0);
  issue(min(1, nks - 1), 1);
  proj_stage_barrier<C::LOADS>();
  // stage ks: compute from stage ks's buffer, issuing stage ks + 2 on the
  // way (the last stage again past the end: its buffer is never read again
  // and the count in flight stays fixed), then wait for stage ks + 1 and
  // barrier.  Buffer indices rotate by three, so the loop is unrolled by
  // three.
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    compute(0, min(ks + 2, nks - 1), 2); proj_stage_barrier<C::LOADS>();
    compute(1, min(ks + 3, nks - 1), 0); proj_stage_barrier<C::LOADS>();
    compute(2, min(ks + 4, nks - 1), 1); proj_stage_barrier<C::LOADS>();
  }
  if (ks < nks) { compute(0, min(ks + 2, nks - 1), 2); proj_stage_barrier<C::LOADS>(); }
  if (ks + 1 < nks) { compute(1, min(ks + 3, nks - 1), 0); proj_stage_barrier<C::LOADS>(); }
  // drain the loads still in flight (the LDS is reused below and released)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Row factors: the chunk sums of the 128 rows meet in LDS (row-major, 8
  // per row), and each row's sum is formed as
  // ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)).
  float* const csum = reinterpret_cast<float*>(xb0);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) csum[(wt * 64 + jj * 32 + r32) * 8 + 2 * wf + g] = ssc[jj];
  __syncthreads();
  float rs[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(csum + (wt * 64 + jj * 32 + r32) * 8);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(csum + (wt * 64 + jj * 32 + r32) * 8 + 4);
    const float s = ((lo[0] + lo[1]) + (lo[2] + lo[3])) + ((hi[0] + hi[1]) + (hi[2] + hi[3]));
    rs[jj] = 1.0f / sqrtf(s / (float)a.D + a.eps);
  }

  // Epilogue: acc[i][jj][e] = C^T[feature f0 + wf*64 + i*32 + 8*(e/4) + 4g + e%4][token t0 + wt*64 + jj*32 + r32]
  // A wave's 64 features lie in one head of one of K and V (f0 is a multiple
  // of 128 and Hkv*d, d of 64).
  float amax = 0.f;   // largest |value| this lane stores (amax_bits mode)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tl = wt * 64 + jj * 32 + r32;
    const int tok = t0 + tl;
    if (tok >= M) continue;
    const float rsj = rs[jj];
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
        bf16* dst = static_cast<bf16*>(which ? a.v_out : a.k_out) +
                 ((size_t)(bb * a.Hkv + hh) * a.n_cap + a.row0 + n) * a.d + c;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][jj][4 * qd + e] * rsj;
        if (a.rope_log2_theta != 0.0 && !which) {   // keys only, at their cache position
          const long long p = a.pos0 + n;
          rope_pair(v[0], v[1], (double)p * rope_inv_freq(c >> 1, a.d, a.rope_log2_theta));
          rope_pair(v[2], v[3], (double)p * rope_inv_freq((c >> 1) + 1, a.d, a.rope_log2_theta));
        }
        // the values as stored
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)(bf16)v[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(v[e]));
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)v[e];   // exact: already bf16 values
        *reinterpret_cast<bf16x4*>(dst) = v4;
      }
    }
  }
  if (a.amax_bits != nullptr) {
    // per-head maxima for a following 8-bit encode: one atomic per wave
    // (integer max on the bit patterns of non-negative floats orders them
    // like their values)
    amax = row16_max(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int f = f0 + wf * 64;
    const int which = f >= HD;
    const int hh = (which ? f - HD : f) / a.d;
    if (l == 0 && amax > 0.f) atomicMax(a.amax_bits + which * a.Hkv + hh, __float_as_uint(amax));
  }
}

hipError_t launch_kv_proj(const ProjArgs& a, bool is_bf16, hipStream_t stream) {
  const int F = 2 * a.Hkv * a.d;
  const int M = a.B * a.N;
  const long long ntt = (M + 127) / 128, nft = F / 128;
  // the ring form when its grid (one workgroup per CU) still covers the 256 CUs
  if (proj_ring_form((long long)M, F, is_bf16, a.norm_w != nullptr)) {
    hipLaunchKernelGGL(kv_proj_ring_kernel, dim3((unsigned)proj_workgroups(F / 256, (int)ntt)), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  // the 2 x 4 XCD partition pads the token tiles to a multiple of 4
  const long long nwg = proj_workgroups((int)nft, (int)ntt);
  dim3 grid((unsigned)nwg);
  if (is_bf16)
    hipLaunchKernelGGL((kv_proj_kernel<bf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((kv_proj_kernel<float>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace yoco
