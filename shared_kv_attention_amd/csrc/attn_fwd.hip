// Tiled flash-attention forward for gfx950: causal cross-attention over the
// shared global cache, and the self-decoder's sliding-window attention.
//
// What is computed (paperlayer.ai summary of "You Only Cache Once", sections
// 2-3; YOCO podcast transcript, segment 12): for query position p of head h,
//   O = sum_{s in A(p)} softmax_s(scale * q . k_s) v_s,   kv head = h / (Hq/Hkv),
// with A(p) = {s <= p} (causal) or {p - W < s <= p} (sliding window W).
//
// Design (MI355X-first):
//  * One workgroup = 4 waves = 128 query rows of one (batch, head); keys are
//    streamed in tiles of BK rows (64 for the causal bf16 form, 32 for the
//    sliding window and for float32) staged through LDS with
//    double buffering: the next tile's global loads are in flight while the
//    current tile is multiplied.
//  * Scores are formed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA so
//    that every lane owns one query row (lane l -> row l%32 of its wave):
//    softmax statistics need only one cross-lane exchange (lane l ^ 32).
//    K rows are fed to the matrix core in a bit-permuted order (bits 2 and 3
//    of the row index swapped), which makes each lane's 16 probabilities
//    exactly the B operand of O^T = V^T P^T -- no shuffle of P at all.
//  * V stays row-major in LDS; its transposed operand is read with the gfx950
//    LDS transpose load (ds_read_b64_tr_b16), two per fragment.
//  * Online softmax in the exp2 domain with the log2(e) folded into the
//    scale; a row's running maximum is only raised (and its O rescaled) when
//    a tile exceeds it by more than 2^8 -- rare, and decided per row so that
//    no row's arithmetic depends on another row's data.
//  * Masking is a select to -inf on tiles that straddle a boundary; tiles
//    entirely outside a wave's rows are skipped.  Keys past the valid rows
//    are never loaded (zero-filled), so stale cache memory cannot leak in.
//  * Grid order: heaviest query tiles first (causal; natural order for the
//    sliding window, whose tiles all cost the same), and within each round
//    the heads of one KV head are placed on one XCD (workgroups go to the 8
//    XCDs round-robin), so each XCD's L2 holds one KV head's K/V.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile_lds.hpp"

namespace yoco {

template <typename T, int D, bool SWA>
struct AttnCfg {
  static constexpr int E = Elem<T>::bytes;
  // 4 waves x 32 query rows.  (Two 32-row blocks per wave halve the LDS
  // traffic per MFMA but need one wave per SIMD; measured slower.)
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int BQ = NW * 32;            // query rows per workgroup (128)
  // bf16 sliding window: 32-key tiles (32 KB of LDS per workgroup) and at most
  // 168 VGPRs, so that three workgroups share a CU.  Its query tiles all cost
  // about the same, and at the 3B shape (4096 rows x 24 heads = 768 tiles)
  // two per CU is one and a half rounds; three per CU is one.  The causal
  // kernel keeps 64-key tiles and two workgroups per CU: its tiles range from
  // 1 to 64 key tiles and run heaviest first.
  static constexpr bool THREE = SWA && E == 2;
  static constexpr int BK = (E == 2 && !THREE) ? 64 : 32;
  static constexpr int CH = D * E / 16;         // 16-byte chunks per K/V row
  static constexpr int PER_T = BK * CH / NT;    // chunks per thread per tensor
  static constexpr int NKB = BK / 32;           // 32-key score blocks per tile
  static constexpr int NC = D / 16;             // 16-deep k steps over d
  static constexpr int NDB = D / 32;            // 32-wide dim blocks of O
  static constexpr int NPC = BK / 16;           // 16-key steps of P V
  static constexpr int TILE_BYTES = BK * D * E;
  // bf16 matrix steps read their LDS fragments this many MFMA slots ahead
  static constexpr int FRAG_AHEAD = THREE ? 2 : 3;
  static_assert(PER_T >= 1 && BK * CH % NT == 0, "tile must split over the workgroup");
  static constexpr int MIN_WAVES_PER_EU = THREE ? 3 : 2;
};

// Scheduler hints for a run of NS matrix-core slots whose LDS operand (R
// reads each) is fetched PD slots ahead: the reads of the first PD slots,
// then per slot one MFMA followed by the reads of slot n + PD.  Without them
// the compiler reads one or two fragments ahead and every step waits for
// the LDS round trip.
template <int R, int PD, int n>
__device__ __forceinline__ void pipe_sched_prologue() {
  if constexpr (n < PD) {
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);   // DS reads
    pipe_sched_prologue<R, PD, n + 1>();
  }
}
template <int R, int NS, int PD, int n>
__device__ __forceinline__ void pipe_sched_steps() {
  if constexpr (n < NS) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    if constexpr (n + PD < NS) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    pipe_sched_steps<R, NS, PD, n + 1>();
  }
}

// Key tiles [lo, hi] that query tile qt (bq rows) needs.
__device__ __forceinline__ void key_span(const AttnArgs& a, bool swa, int bq, int bk, int qt, int& lo, int& hi) {
  attn_key_span(a.Nq, a.n_kv, a.q_offset, a.window, swa, bq, bk, qt, lo, hi);
}

// One wave's 32 query rows of one (batch, head): Q operands, running
// softmax state and unnormalised O, and the per-tile step.
template <typename T, int D, bool SWA>
struct AttnWave {
  using C = AttnCfg<T, D, SWA>;
  using frag = typename Elem<T>::frag;
  frag qf[C::NC];
  f32x16 acc[C::NDB];
  float m_run, l_run;        // running max (log2 domain) and this lane's partial denominator
  int qi, lo_key, hi_key;    // this lane's query row and its allowed keys
  int pw0, pw1;              // first and last query position of the wave
  bool live;                 // the wave holds at least one valid row

  // rows wq0 .. wq0 + 31 (lane l -> row wq0 + l % 32) of the head at qbase
  __device__ __forceinline__ void init(const AttnArgs& a, const T* qbase, int wq0, int l) {
    const int g = l >> 5;
    qi = wq0 + (l & 31);
    const int pos = a.q_offset + qi;
    lo_key = SWA ? max(0, pos - a.window + 1) : 0;
    hi_key = min(pos, a.n_kv - 1);
    if (qi < a.Nq) {
      const T* qrow = qbase + (size_t)qi * D;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) qf[c] = load_frag_global<T>(qrow + 16 * c + 8 * g);
    } else {
#pragma unroll
      for (int c = 0; c < C::NC; ++c) qf[c] = frag{};
    }
    // wave-uniform: kept in scalar registers so that tile decisions are scalar branches
    live = __builtin_amdgcn_readfirstlane(wq0 < a.Nq) != 0;
    pw0 = __builtin_amdgcn_readfirstlane(a.q_offset + wq0);
    pw1 = __builtin_amdgcn_readfirstlane(a.q_offset + min(wq0 + 31, a.Nq - 1));
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // key tile t from (ktile, vtile) in LDS
  __device__ __forceinline__ void tile(const AttnArgs& a, int t, const char* ktile, const char* vtile, int l) {
    const int g = l >> 5, r32 = l & 31;
    const int k0 = t * C::BK, k1 = k0 + C::BK - 1;
    const bool skip = !live || k0 > pw1 || (SWA && k1 <= pw0 - a.window);
    if (skip) return;
    const bool need_mask = k1 > pw0 || k1 >= a.n_kv || (SWA && k0 <= pw1 - a.window);

    // S^T = K Q^T
    f32x16 s[C::NKB];
    if constexpr (sizeof(T) == 2) {
      // slot n = (k step c = n / NKB, key block kb = n % NKB): the two key
      // blocks alternate, so consecutive MFMAs are independent; fragments
      // are read FRAG_AHEAD slots ahead through a small ring
      constexpr int NS = C::NC * C::NKB, PD = C::FRAG_AHEAD;
      const int krow = sigma(r32);
      frag ring[PD + 1];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int n = 0; n < PD; ++n) ring[n] = lds_frag_k<T, C::CH>(ktile, (n % C::NKB) * 32 + krow, n / C::NKB, g);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + PD < NS) {
          const int m = n + PD;
          ring[m % (PD + 1)] = lds_frag_k<T, C::CH>(ktile, (m % C::NKB) * 32 + krow, m / C::NKB, g);
        }
        s[n % C::NKB] = mma32(ring[n % (PD + 1)], qf[n / C::NKB], s[n % C::NKB]);
      }
      pipe_sched_prologue<1, PD, 0>();
      pipe_sched_steps<1, NS, PD, 0>();
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        s[kb] = f32x16{};
        const int krow = kb * 32 + sigma(r32);
#pragma unroll
        for (int c = 0; c < C::NC; ++c) s[kb] = mma32(lds_frag_k<T, C::CH>(ktile, krow, c, g), qf[c], s[kb]);
      }
    }

    // element i of block kb <-> key k0 + kb*32 + 16*(i/8) + 8*g + i%8.
    // Masked scores become -inf (a select, never an additive mask).
    float mraw = -INFINITY;
    if (need_mask) {
      // allowed keys of this lane's row: [lo_key, hi_key], i.e. element
      // offsets off (key = k0 + 8g + off) in [lim_lo, lim_hi].  The lower
      // bound can only bite on a tile that reaches below some row's window.
      const int lim_hi = hi_key - (k0 + 8 * g), lim_lo = lo_key - (k0 + 8 * g);
      auto mask_tile = [&](auto both) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = kb * 32 + 16 * (i >> 3) + (i & 7);
            // both bounds: one unsigned range test; upper bound only: one signed test
            const bool ok = decltype(both)::value ? (unsigned)(off - lim_lo) <= (unsigned)(lim_hi - lim_lo)
                                                  : off <= lim_hi;
            const float x = ok ? s[kb][i] : -INFINITY;
            s[kb][i] = x;
            mraw = fmaxf(mraw, x);
          }
        }
      };
      if (SWA && k0 <= pw1 - a.window) mask_tile(std::true_type{});
      else mask_tile(std::false_type{});
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[kb][i]);
      }
    }
    mraw = pair32_max(mraw);
    const float mloc = mraw * a.scale_log2;   // scale > 0: max commutes with it
    // Each row decides from its own scores only (rows never influence each
    // other, so results are bitwise causal).
    const bool up = mloc > m_run + 8.0f;
    if (__any(up)) {
      const float alpha = !up ? 1.f : (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mloc));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) acc[db] *= alpha;
      m_run = up ? mloc : m_run;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, neg_m));
    }
    // P^T fragments: step c covers keys 16c .. 16c+15 of the tile
    frag pf[C::NPC];
#pragma unroll
    for (int c = 0; c < C::NPC; ++c) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pf[c][jj] = from_f32<T>(s[c >> 1][8 * (c & 1) + jj]);
    }
    // float32 row sum (4 independent partial sums for instruction-level parallelism)
    float ls[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int i = (kb == 0 ? 4 : 0); i < 16; ++i) ls[i & 3] += s[kb][i];
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      // slot n = (key step c = n / NDB, dim block db = n % NDB): the dim
      // blocks alternate; each fragment is two transposed reads, issued
      // FRAG_AHEAD slots ahead
      constexpr int NS = C::NPC * C::NDB, PD = C::FRAG_AHEAD;
      frag ring[PD + 1];
#pragma unroll
      for (int n = 0; n < PD; ++n) ring[n] = lds_frag_vt<T, C::CH>(vtile, n / C::NDB, n % C::NDB, l);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + PD < NS) {
          const int m = n + PD;
          ring[m % (PD + 1)] = lds_frag_vt<T, C::CH>(vtile, m / C::NDB, m % C::NDB, l);
        }
        acc[n % C::NDB] = mma32(ring[n % (PD + 1)], pf[n / C::NDB], acc[n % C::NDB]);
      }
      pipe_sched_prologue<2, PD, 0>();
      pipe_sched_steps<2, NS, PD, 0>();
    } else {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int c = 0; c < C::NPC; ++c) acc[db] = mma32(lds_frag_vt<T, C::CH>(vtile, c, db, l), pf[c], acc[db]);
      }
    }
  }

  // normalise and write this lane's row of O (and its log-sum-exp)
  __device__ __forceinline__ void write(const AttnArgs& a, size_t bh, int l) const {
    const int g = l >> 5;
    const float l_tot = pair32_sum(l_run);
    if (qi >= a.Nq) return;
    const float inv = 1.f / l_tot;
    T* orow = static_cast<T*>(a.o) + (bh * a.Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int dim = db * 32 + 8 * qd + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][4 * qd + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + dim) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[db][4 * qd + e] * inv;
          *reinterpret_cast<f32x4*>(orow + dim) = v4;
        }
      }
    }
    if (a.lse != nullptr && g == 0) {
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      a.lse[bh * a.Nq + qi] = (mref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
};

// Cooperative staging of K/V tiles (global -> LDS directly, no registers) by
// the 4 waves (256 threads) that share the tiles.  Each wave instruction
// fills 64 consecutive 16-byte LDS slots (lane i -> slot base + i).  Slot P of
// a tile holds row P / CH at physical chunk P % CH, i.e. logical chunk
// (P % CH) ^ swizzle(row); so each lane fetches the global chunk that belongs
// in its slot.  The loads are buffer loads through a per-tile resource whose
// base is the tile and whose size ends at row n_kv: the lane offsets are
// loop-invariant registers (no per-load address arithmetic), and rows at or
// past n_kv are never read -- they load as zeros (always masked out).
template <typename T, int D, bool SWA>
struct TileStager {
  using C = AttnCfg<T, D, SWA>;
  static constexpr int ROWB = D * C::E;   // bytes per K/V row
  unsigned koff[C::PER_T], voff[C::PER_T];
  const char* kbase;
  const char* vbase;
  int n_kv, wslot;

  __device__ __forceinline__ void init(const char* kb, const char* vb, int n_kv_, int wi, int l) {
    // the bases are uniform: keep them scalar so the buffer resources are built in SGPRs
    kbase = uniform_ptr(kb);
    vbase = uniform_ptr(vb);
    n_kv = __builtin_amdgcn_readfirstlane(n_kv_);
    wslot = __builtin_amdgcn_readfirstlane(64 * wi);
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int slot = C::NT * r + wslot + l;
      koff[r] = stage_offset<C::CH, true>(slot, ROWB);
      voff[r] = stage_offset<C::CH, false>(slot, ROWB);
    }
  }
  // Every buffer starts zeroed, so a slot that an out-of-range load leaves
  // untouched still holds finite data; this lane's zeros land before its loads.
  __device__ __forceinline__ void zero(char* k0, char* v0, char* k1, char* v1, int l) const {
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int o = (C::NT * r + wslot + l) * 16;
      *reinterpret_cast<u32x4*>(k0 + o) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(v0 + o) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(k1 + o) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(v1 + o) = u32x4{0, 0, 0, 0};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  __device__ __forceinline__ void load(int t, char* kdst_tile, char* vdst_tile) const {
    const size_t tb = (size_t)t * C::BK * ROWB;   // uniform tile base
    // bytes of rows < n_kv (uniform; read back as a scalar so the resource
    // stays in SGPRs).  The row count is clamped to one tile before it is
    // scaled to bytes, so the product stays small for any cache length.
    const int valid = __builtin_amdgcn_readfirstlane(tile_valid_bytes(n_kv, t, C::BK, ROWB));
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + tb), (short)0, valid, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + tb), (short)0, valid, kBufferFlags);
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      char* kdst = kdst_tile + (C::NT * r + wslot) * 16;
      char* vdst = vdst_tile + (C::NT * r + wslot) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)kdst, 16, (int)koff[r], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)vdst, 16, (int)voff[r], 0, 0, 0);
    }
  }
};

// the tile loads' LDS writes land asynchronously: wait for this wave's before
// the barrier that hands the buffer to the other waves
__device__ __forceinline__ void tile_landed() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// One 4-wave workgroup per query tile.
// ---------------------------------------------------------------------------
template <typename T, int D, bool SWA>
__global__ __launch_bounds__((AttnCfg<T, D, SWA>::NT), (AttnCfg<T, D, SWA>::MIN_WAVES_PER_EU)) void attn_fwd_kernel(AttnArgs a) {
  using C = AttnCfg<T, D, SWA>;
  // Two buffer sets as distinct LDS objects, used in a statically alternating
  // order (the tile loop is unrolled by two): the compiler can then see that
  // the asynchronous loads into one set never alias reads of the other, and
  // does not wait for them before the current tile's LDS reads.
  __shared__ __attribute__((aligned(16))) char kbuf0[C::TILE_BYTES], vbuf0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char kbuf1[C::TILE_BYTES], vbuf1[C::TILE_BYTES];

  const int tid = threadIdx.x;
  // wave index as a scalar: every wave-level decision below is a scalar branch
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;

  // ---- workgroup -> (batch, head, query tile) ----
  // causal: heaviest (latest) query tiles first; sliding window: all tiles
  // cost the same, and the natural order lets neighbouring windows share L2;
  // the heads of one KV head on one XCD
  const int nqt = (a.Nq + C::BQ - 1) / C::BQ;
  const AttnTile tile = attn_tile(blockIdx.x, a.B, a.Hq, nqt, SWA);
  const int qt = tile.qt, b = tile.b, h = tile.h;
  const int kvh = h / (a.Hq / a.Hkv);

  const T* qbase = static_cast<const T*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq) * D;
  const char* kbase = static_cast<const char*>(a.k) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;
  const char* vbase = static_cast<const char*>(a.v) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;

  AttnWave<T, D, SWA> wv;
  wv.init(a, qbase, qt * C::BQ + w * 32, l);
  int t_lo, t_hi;
  key_span(a, SWA, C::BQ, C::BK, qt, t_lo, t_hi);

  TileStager<T, D, SWA> st;
  st.init(kbase, vbase, a.n_kv, w, l);
  st.zero(kbuf0, vbuf0, kbuf1, vbuf1, l);

  // one tile: compute from (ktile, vtile) while tile t+1 streams into (knext, vnext)
  auto tile_step = [&](int t, const char* ktile, const char* vtile, char* knext, char* vnext)
      __attribute__((always_inline)) {
    const bool has_next = t < t_hi;
    if (has_next) st.load(t + 1, knext, vnext);   // this set was released by the last barrier
    wv.tile(a, t, ktile, vtile, l);
    if (has_next) tile_landed();
    __syncthreads();
  };

  st.load(t_lo, kbuf0, vbuf0);
  tile_landed();
  __syncthreads();
  for (int t = t_lo; t <= t_hi; t += 2) {
    tile_step(t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 <= t_hi) tile_step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }
  wv.write(a, (size_t)(b * a.Hq + h), l);
}

template <typename T, int D, bool SWA>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  using C = AttnCfg<T, D, SWA>;
  const int nqt = (a.Nq + C::BQ - 1) / C::BQ;
  const long long nblocks = (long long)nqt * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, SWA>), dim3((unsigned)nblocks), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, bool is_bf16, int d, bool swa, hipStream_t stream) {
  if (is_bf16) {
    if (d == 128) return swa ? launch_attn_t<bf16, 128, true>(a, stream) : launch_attn_t<bf16, 128, false>(a, stream);
    return swa ? launch_attn_t<bf16, 64, true>(a, stream) : launch_attn_t<bf16, 64, false>(a, stream);
  }
  if (d == 128) return swa ? launch_attn_t<float, 128, true>(a, stream) : launch_attn_t<float, 128, false>(a, stream);
  return swa ? launch_attn_t<float, 64, true>(a, stream) : launch_attn_t<float, 64, false>(a, stream);
}

}  // namespace yoco
