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
// order (only B*H workgroups), the prefill runs three launches that are each
// parallel over chunks:
//  1. state:  per chunk (8 waves), the log2 decay prefix sums and the
//             chunk's total decay, then dR^T = (V scaled by e^{L_last - L_m})^T K
//             on the matrix cores (both operands read transposed from LDS),
//             stored [dv][dk];
//  2. scan:   per (head, 32 x 32 block of the state), R_c = e^{L_last}
//             R_{c-1} + dR_c in float32 with the chunks' dR loaded in
//             groups ahead of use, storing the state entering every chunk
//             as bf16 R^T [dv][dk], the operand layout of 3;
//  3. output: per (chunk, 128 query rows), the cross-chunk term R^T Q^T
//             (R^T staged in LDS), then an attention-like tile loop with
//             decay weights e^{L_n - L_m} (formed per pair from the
//             difference, so a strong gate can never overflow) instead of a
//             softmax, with direct global -> LDS double-buffered 32-key K/V
//             tiles (three workgroups per CU), on the same accumulator.  The
//             heavier second halves of the chunks (twice the key tiles) are
//             dispatched first.
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
// 1+2. per chunk: log2-decay prefix sums (written out for the output kernel)
//      and the state contribution, stored transposed:
//      dR^T[dv][dk] = sum_m V[m][dv] w_m K[m][dk],  w_m = 2^{L_last - L_m}
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) void gret_state_kernel(GretArgs a) {
  using C = GretCfg<D>;
  __shared__ __attribute__((aligned(16))) char kt[C::TILE], vt[C::TILE];
  __shared__ float lgc[256];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int l = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c0 = c * a.chunk, clen = min(a.chunk, a.N - c0);

  const bf16* kb = static_cast<const bf16*>(a.k) + ((size_t)bh * a.N + c0) * D;
  const bf16* vb = static_cast<const bf16*>(a.v) + ((size_t)bh * a.N + c0) * D;
  constexpr int TILES = C::NDB * C::NDB, TPW = TILES / 8 > 0 ? TILES / 8 : 1;
  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
  const bool active = w * TPW < TILES;

  // Each thread owns the same PER_T chunk slots of every tile; the raw chunks
  // of tile r0 + BK are loaded into registers while tile r0 is multiplied.
  constexpr int PER_T = C::BK * C::CH / 512;
  u32x4 kraw[PER_T], vraw[PER_T];
  auto fetch = [&](int r0) {
    const int rows = min(C::BK, clen - r0);
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      const int slot = 512 * r + t, row = slot / C::CH, pch = slot % C::CH;
      const int lch = pch ^ swz_v<C::CH>(row);
      const size_t off = (size_t)(r0 + min(row, rows - 1)) * D + lch * 8;
      kraw[r] = *reinterpret_cast<const u32x4*>(kb + off);
      vraw[r] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  float l_last = 0.f;   // set once the prefix sums are in LDS
  auto put = [&](int r0) {   // rows past the chunk become zero; V rows scaled by 2^{L_last - L_m}
    const int rows = min(C::BK, clen - r0);
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      const int slot = 512 * r + t, row = slot / C::CH;
      u32x4 kw{0, 0, 0, 0}, vw{0, 0, 0, 0};
      if (row < rows) {
        kw = kraw[r];
        const float f = __builtin_amdgcn_exp2f(l_last - lgc[r0 + row]);
        bf16x8 v = __builtin_bit_cast(bf16x8, vraw[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * f);
        vw = __builtin_bit_cast(u32x4, v);
      }
      *reinterpret_cast<u32x4*>(kt + slot * 16) = kw;
      *reinterpret_cast<u32x4*>(vt + slot * 16) = vw;
    }
  };
  // the first K/V tile is requested before the decay prefix sums, which do
  // not need it, so that both memory round trips overlap
  fetch(0);
  // inclusive prefix sum of the chunk's log2 decays (positions past the end add 0)
  {
    const bool scan_t = t < 256;
    float x = t < clen ? gate_log2(a.gate[(size_t)bh * a.N + c0 + t], a.inv_tau) : 0.f;
    if (scan_t) lgc[t] = x;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const float y = scan_t && t >= off ? lgc[t - off] : 0.f;
      __syncthreads();
      x += y;
      if (scan_t) lgc[t] = x;
      __syncthreads();
    }
    if (t < clen) a.lg2[(size_t)bh * a.N + c0 + t] = x;
    if (t == clen - 1) a.lam[(size_t)bh * a.nc + c] = __builtin_amdgcn_exp2f(x);
  }
  l_last = lgc[clen - 1];
  for (int r0 = 0; r0 < clen; r0 += C::BK) {
    put(r0);
    if (r0 + C::BK < clen) fetch(r0 + C::BK);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tt = w * TPW + i, dkb = tt / C::NDB, dvb = tt % C::NDB;
#pragma unroll
        for (int s = 0; s < C::BK / 16; ++s)
          acc[i] = mma32(lds_frag_vt<bf16, C::CH>(vt, s, dvb, l), lds_frag_vt<bf16, C::CH>(kt, s, dkb, l), acc[i]);
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
        const int dv = dvb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
        dst[dv * D + dkb * 32 + (l & 31)] = acc[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. scan over chunks on 32 x 32 blocks of the state: R_c = lam_c R_{c-1} + dR_c
//    in float32, all in the transposed [dv][dk] layout (lanes along dk); the
//    state entering chunk c is stored in bf16 (rinT[c][dv][dk], the operand
//    layout of the output kernel's R^T Q^T).  No barriers: the loads of the
//    next group of chunks stay in flight while the current one is summed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gret_scan_kernel(GretArgs a) {
  constexpr int PF = 4;                      // chunks per prefetch group
  const int bh = blockIdx.y;
  const int nb = a.d / 32;
  const int dv0 = (blockIdx.x / nb) * 32, dk0 = (blockIdx.x % nb) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // dk0 + tx, dv0 + ty + 8u
  const size_t DD = (size_t)a.d * a.d;
  float R[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)   // the state is [dk][dv] at the interface
    R[u] = a.state_in ? a.state_in[bh * DD + (size_t)(dk0 + tx) * a.d + dv0 + ty + 8 * u] : 0.f;
  const float* dRb = a.dR + (size_t)bh * a.nc * DD;
  bf16* rinb = static_cast<bf16*>(a.rin) + (size_t)bh * a.nc * DD;
  const float* lamb = a.lam + (size_t)bh * a.nc;
  auto load = [&](int cb, float (&x)[PF][4]) {
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (cb + j < a.nc)
#pragma unroll
        for (int u = 0; u < 4; ++u) x[j][u] = dRb[(size_t)(cb + j) * DD + (size_t)(dv0 + ty + 8 * u) * a.d + dk0 + tx];
  };
  auto step = [&](int cb, const float (&x)[PF][4]) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int c = cb + j;
      if (c < a.nc) {
        const float lam = lamb[c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          rinb[(size_t)c * DD + (size_t)(dv0 + ty + 8 * u) * a.d + dk0 + tx] = (bf16)R[u];
          R[u] = fmaf(lam, R[u], x[j][u]);
        }
      }
    }
  };
  float xa[PF][4], xb[PF][4];
  load(0, xa);
  for (int cb = 0; cb < a.nc; cb += 2 * PF) {
    load(cb + PF, xb);
    step(cb, xa);
    load(cb + 2 * PF, xa);
    step(cb + PF, xb);
  }
  if (a.state_out) {
#pragma unroll
    for (int u = 0; u < 4; ++u) a.state_out[bh * DD + (size_t)(dk0 + tx) * a.d + dv0 + ty + 8 * u] = R[u];
  }
}

// ---------------------------------------------------------------------------
// 4. outputs of 128 query rows of one chunk; K/V tiles (and the keys' log2
//    decays) are staged global -> LDS directly and double-buffered
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 3) void gret_out_kernel(GretArgs a) {
  using C = GretCfg<D>;
  // 32-key tiles: with at most 168 VGPRs and 48 KB of LDS, three workgroups
  // share a CU (the 3B shape's 768 workgroups are then one round, not 1.5)
  constexpr int BK = 32;                         // key rows per LDS tile
  constexpr int TB = BK * D * 2;                 // bytes of one K or V tile
  constexpr int PER_T = BK * C::CH / 256;        // 16-byte chunks per thread per tile
  static_assert(2 * TB <= D * D * 2, "the second tile set fits in the R^T region");
  // set 0 as its own LDS objects; the chunk's R^T (D rows, K-tile layout)
  // first, and once it has been used, set 1, in a region of its own -- so the
  // loads into one set are never taken for writes to the other
  __shared__ __attribute__((aligned(16))) char kt0[TB], vt0[TB];
  __shared__ __attribute__((aligned(16))) char rset[D * D * 2];
  char* const kt1 = rset;
  char* const vt1 = rset + TB;
  __shared__ __attribute__((aligned(16))) float lg0[64], lg1[64];   // one log-decay per lane of wave 0
  const int nrb = a.chunk / 128;
  // linear block index -> (row block, descending: the later rows see more keys; head; chunk)
  const int nblk_bh = a.nc * a.B * a.H;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int rb = nrb - 1 - lin / nblk_bh, rem = lin % nblk_bh;
  const int bh = rem / a.nc, c = rem % a.nc;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 5, r32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = c * a.chunk;
  const int q0 = c0 + rb * 128;                 // first query row of the workgroup
  if (q0 >= a.N) return;                        // whole workgroup past the end (uniform)
  const int wq0 = q0 + 32 * w;                  // first row of this wave
  const int n = wq0 + r32;                      // this lane's query row
  const bool row_ok = n < a.N;
  const bool wave_live = wq0 < a.N;
  const size_t hrow = (size_t)bh * a.N;
  const int k_end = min(q0 + 127, a.N - 1);     // last key any row here can see
  const int pw1 = min(wq0 + 31, a.N - 1);       // last row of this wave
  const int ntiles = (k_end - c0) / BK + 1;

  // ---- tile staging by DMA: slot P = 256 r + tid of a tile holds row P / CH
  // at physical chunk P % CH; rows past k_end re-read row k_end (finite data,
  // always masked: their keys lie after every row of the workgroup)
  const char* kbase = static_cast<const char*>(a.k) + hrow * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + hrow * D * 2;
  unsigned koff[PER_T], voff[PER_T];
  int srow[PER_T];
#pragma unroll
  for (int r = 0; r < PER_T; ++r) {
    const int slot = 256 * r + 64 * w + l;
    const int row = slot / C::CH, pch = slot % C::CH;
    srow[r] = row;
    koff[r] = (unsigned)(row * D * 2 + ((pch ^ swz_k<C::CH>(row)) << 4));
    voff[r] = (unsigned)(row * D * 2 + ((pch ^ swz_v<C::CH>(row)) << 4));
  }
  auto load_tile = [&](int t, char* kd, char* vd, float* lgd) {
    const int k0 = c0 + t * BK;
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      const int over = k0 + srow[r] - k_end;
      const unsigned back = over > 0 ? (unsigned)(over * D * 2) : 0u;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(kbase + (size_t)k0 * D * 2 + koff[r] - back),
                                       (__attribute__((address_space(3))) void*)(kd + (256 * r + 64 * w) * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(vbase + (size_t)k0 * D * 2 + voff[r] - back),
                                       (__attribute__((address_space(3))) void*)(vd + (256 * r + 64 * w) * 16), 16, 0, 0);
    }
    if (w == 0) {
      const int key = min(k0 + l, k_end);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(a.lg2 + hrow + key),
                                       (__attribute__((address_space(3))) void*)lgd, 4, 0, 0);
    }
  };
  load_tile(0, kt0, vt0, lg0);
  // R^T of the chunk (D rows) into its region, K-tile layout, BK rows per tile
  {
    const char* rbase = static_cast<const char*>(a.rin) + ((size_t)bh * a.nc + c) * D * D * 2;
#pragma unroll
    for (int h = 0; h < D / BK; ++h)
#pragma unroll
      for (int r = 0; r < PER_T; ++r)
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(rbase + h * TB + koff[r]),
                                         (__attribute__((address_space(3))) void*)(rset + h * TB + (256 * r + 64 * w) * 16),
                                         16, 0, 0);
  }

  // query fragments (as for attention: row n, dims 16c + 8g + j)
  bf16x8 qf[C::NC];
  {
    const bf16* qrow = static_cast<const bf16*>(a.q) + (hrow + (row_ok ? n : q0)) * D;
#pragma unroll
    for (int cc = 0; cc < C::NC; ++cc)
      qf[cc] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * g) : bf16x8{};
  }
  const float l_n = row_ok ? a.lg2[hrow + n] : 0.f;

  // cross-chunk term O^T = R^T Q^T (R^T from LDS), then column n scaled by 2^{L_n}
  f32x16 acc[C::NDB];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const char* rt = rset + db * TB;   // R^T rows db*32 .. db*32 + 31
      bf16x8 rf[C::NC];
#pragma unroll
      for (int cc = 0; cc < C::NC; ++cc) rf[cc] = lds_frag_k<bf16, C::CH>(rt, r32, cc, g);
      acc[db] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NC; ++cc) acc[db] = mma32(rf[cc], qf[cc], acc[db]);
    }
    const float f = __builtin_amdgcn_exp2f(l_n);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] *= f;
  }

  // one key tile: compute from (kt, vt, lgt) while tile t+1 streams into the other set
  auto tile_step = [&](int t, const char* kt, const char* vt, const float* lgt, char* kn, char* vn, float* lgn)
      __attribute__((always_inline)) {
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(t + 1, kn, vn, lgn);
    const int k0 = c0 + t * BK;
    if (wave_live && k0 <= pw1) {
      // S^T = K Q^T; element i <-> key k0 + 16*(i/8) + 8g + i%8
      f32x16 s = f32x16{};
      const int krow = sigma(r32);
#pragma unroll
      for (int cc = 0; cc < C::NC; ++cc) s = mma32(lds_frag_k<bf16, C::CH>(kt, krow, cc, g), qf[cc], s);
      // decay weights, masked by m <= n (a select: 2^{L_n - L_m} may
      // overflow above the diagonal)
      bf16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 16 * (i >> 3) + 8 * g + (i & 7);
        const float wgt = s[i] * __builtin_amdgcn_exp2f(l_n - lgt[off]);
        pf[i >> 3][i & 7] = (bf16)((k0 + off <= n) ? wgt : 0.f);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) acc[db] = mma32(lds_frag_vt<bf16, C::CH>(vt, cc, db, l), pf[cc], acc[db]);
      }
    }
    if (has_next) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  __syncthreads();   // R^T reads done before tile 1 overwrites it
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(t, kt0, vt0, lg0, kt1, vt1, lg1);
    if (t + 1 < ntiles) tile_step(t + 1, kt1, vt1, lg1, kt0, vt0, lg0);
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
// recurrent step: S <- gamma S + k^T v; o = q S   (state float32 [dk][dv]).
// A workgroup serves 64 dv columns of one head; its 4 waves take a quarter of
// the dk rows each and meet in LDS for o.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void gret_decode_kernel(GretDecodeArgs a) {
  __shared__ float red[4][64];
  constexpr int RPW = D / 4;                      // rows per wave
  const int bh = blockIdx.y, l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x * 64 + l;              // this lane's dv column
  const T* q = static_cast<const T*>(a.q) + (size_t)bh * D;
  const T* k = static_cast<const T*>(a.k) + (size_t)bh * D;
  const T* v = static_cast<const T*>(a.v) + (size_t)bh * D;
  const float gam = __builtin_amdgcn_exp2f(gate_log2(a.gate[bh], a.inv_tau));
  const float vj = to_f32(v[j]);
  float* S = a.state + (size_t)bh * D * D + (size_t)(w * RPW) * D + j;
  float sv[RPW];
#pragma unroll
  // the state is streamed once per step (read, then written back):
  // non-temporal loads and stores (10.2 vs 12.2 us at B16 x 24 heads)
  for (int i = 0; i < RPW; ++i) sv[i] = __builtin_nontemporal_load(S + (size_t)i * D);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = w * RPW + i;
    const float sn = fmaf(gam, sv[i], to_f32(k[row]) * vj);
    __builtin_nontemporal_store(sn, S + (size_t)i * D);
    acc[i & 3] = fmaf(to_f32(q[row]), sn, acc[i & 3]);
  }
  red[w][l] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (w == 0)
    static_cast<T*>(a.o)[(size_t)bh * D + j] = from_f32<T>((red[0][l] + red[1][l]) + (red[2][l] + red[3][l]));
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
  const dim3 heads(a.B * a.H);
  if (a.d == 128) hipLaunchKernelGGL(gret_state_kernel<128>, dim3(a.nc, a.B * a.H), dim3(512), 0, stream, a);
  else hipLaunchKernelGGL(gret_state_kernel<64>, dim3(a.nc, a.B * a.H), dim3(512), 0, stream, a);
  hipLaunchKernelGGL(gret_scan_kernel, dim3((a.d / 32) * (a.d / 32), a.B * a.H), dim3(256), 0, stream, a);
  const int nblk = a.nc * (a.chunk / 128);
  if (a.d == 128) hipLaunchKernelGGL(gret_out_kernel<128>, dim3(nblk, a.B * a.H), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gret_out_kernel<64>, dim3(nblk, a.B * a.H), dim3(256), 0, stream, a);
  (void)heads;
  return hipGetLastError();
}

hipError_t launch_gret_decode(const GretDecodeArgs& a, bool is_bf16, hipStream_t stream) {
  const dim3 grid(a.d / 64, a.B * a.H);
  if (a.d == 128) {
    if (is_bf16) hipLaunchKernelGGL((gret_decode_kernel<bf16, 128>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gret_decode_kernel<float, 128>), grid, dim3(256), 0, stream, a);
  } else {
    if (is_bf16) hipLaunchKernelGGL((gret_decode_kernel<bf16, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gret_decode_kernel<float, 64>), grid, dim3(256), 0, stream, a);
  }
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
