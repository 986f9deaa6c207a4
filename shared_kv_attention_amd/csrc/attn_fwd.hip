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
//    streamed in tiles of BK rows (64 for bf16) staged through LDS with
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
#include "common.hpp"
#include "launch.hpp"
#include "tile_lds.hpp"

namespace yoco {

template <typename T, int D>
struct AttnCfg {
  static constexpr int E = Elem<T>::bytes;
  // 4 waves x 32 query rows.  (Two 32-row blocks per wave halve the LDS
  // traffic per MFMA but need one wave per SIMD; measured slower.)
  static constexpr int RB = 1;                  // 32-row blocks per wave
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int BQ = NW * 32 * RB;       // query rows per workgroup (128)
  static constexpr int BK = (E == 2) ? 64 : 32;
  static constexpr int CH = D * E / 16;         // 16-byte chunks per K/V row
  static constexpr int PER_T = BK * CH / NT;    // chunks per thread per tensor
  static constexpr int NKB = BK / 32;           // 32-key score blocks per tile
  static constexpr int NC = D / 16;             // 16-deep k steps over d
  static constexpr int NDB = D / 32;            // 32-wide dim blocks of O
  static constexpr int NPC = BK / 16;           // 16-key steps of P V
  static constexpr int TILE_BYTES = BK * D * E;
  // bf16 matrix steps read their LDS fragments this many MFMA slots ahead
  static constexpr int FRAG_AHEAD = 3;
  static_assert(PER_T >= 1 && BK * CH % NT == 0, "tile must split over the workgroup");
  static constexpr int MIN_WAVES_PER_EU = (RB == 2) ? 1 : 2;
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

template <typename T, int D, bool SWA>
__global__ __launch_bounds__((AttnCfg<T, D>::NT), (AttnCfg<T, D>::MIN_WAVES_PER_EU)) void attn_fwd_kernel(AttnArgs a) {
  using C = AttnCfg<T, D>;
  using frag = typename Elem<T>::frag;
  constexpr int RB = C::RB;
  // Two buffer sets as distinct LDS objects, used in a statically alternating
  // order (the tile loop is unrolled by two): the compiler can then see that
  // the asynchronous loads into one set never alias reads of the other, and
  // does not wait for them before the current tile's LDS reads.
  __shared__ __attribute__((aligned(16))) char kbuf0[C::TILE_BYTES], vbuf0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char kbuf1[C::TILE_BYTES], vbuf1[C::TILE_BYTES];

  const int tid = threadIdx.x;
  // wave index as a scalar: every wave-level decision below is a scalar branch
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, r32 = l & 31;

  // ---- workgroup -> (batch, head, query tile) ----
  const int BH = a.B * a.Hq;
  const int nqt = (a.Nq + C::BQ - 1) / C::BQ;
  const int id = blockIdx.x;
  // causal: heaviest (latest) query tiles first; sliding window: all tiles
  // cost the same, and the natural order lets neighbouring windows share L2
  const int qt = SWA ? id / BH : nqt - 1 - id / BH;
  int j = id % BH;
  if ((BH & 7) == 0) j = (j & 7) * (BH >> 3) + (j >> 3);   // same KV head -> same XCD
  const int b = j / a.Hq, h = j % a.Hq;
  const int kvh = h / (a.Hq / a.Hkv);

  const T* qbase = static_cast<const T*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq) * D;
  const char* kbase = static_cast<const char*>(a.k) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;
  const char* vbase = static_cast<const char*>(a.v) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;

  // ---- this lane's query rows (one per 32-row block) ----
  const int q_first = qt * C::BQ;
  const int wq0 = q_first + w * 32 * RB;
  int qi[RB], lo_key[RB], hi_key[RB];
  frag qf[RB][C::NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qi[rb] = wq0 + rb * 32 + r32;
    const int pos = a.q_offset + qi[rb];
    lo_key[rb] = SWA ? max(0, pos - a.window + 1) : 0;   // allowed keys of this row
    hi_key[rb] = min(pos, a.n_kv - 1);
    if (qi[rb] < a.Nq) {
      const T* qrow = qbase + (size_t)qi[rb] * D;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) qf[rb][c] = load_frag_global<T>(qrow + 16 * c + 8 * g);
    } else {
#pragma unroll
      for (int c = 0; c < C::NC; ++c) qf[rb][c] = frag{};
    }
  }

  // ---- key-tile range of the workgroup and of this wave ----
  const int q_last = min(q_first + C::BQ, a.Nq) - 1;
  const int P0 = a.q_offset + q_first, P1 = a.q_offset + q_last;
  const int t_lo = SWA ? max(0, P0 - a.window + 1) / C::BK : 0;
  const int t_hi = min(P1, a.n_kv - 1) / C::BK;
  const bool wave_live = wq0 < a.Nq;
  const int pw0 = a.q_offset + wq0;
  const int pw1 = a.q_offset + min(wq0 + 32 * RB - 1, a.Nq - 1);

  // ---- cooperative tile staging: global -> LDS directly (no registers) ----
  // Each wave instruction fills 64 consecutive 16-byte LDS slots (lane i ->
  // slot base + i).  Slot P of a tile holds row P / CH at physical chunk
  // P % CH, i.e. logical chunk (P % CH) ^ swizzle(row); so each lane fetches
  // the global chunk that belongs in its slot.  Rows at or past n_kv are
  // clamped to the last valid row (finite data, always masked out).
  constexpr int ROWB = D * C::E;   // bytes per K/V row
  unsigned koff[C::PER_T], voff[C::PER_T];   // loop-invariant byte offsets of this lane's slots
  int srow[C::PER_T];
#pragma unroll
  for (int r = 0; r < C::PER_T; ++r) {
    const int slot = C::NT * r + 64 * w + l;
    const int row = slot / C::CH, pch = slot % C::CH;
    srow[r] = row;
    koff[r] = (unsigned)(row * ROWB + ((pch ^ swz_k<C::CH>(row)) << 4));
    voff[r] = (unsigned)(row * ROWB + ((pch ^ swz_v<C::CH>(row)) << 4));
  }
  auto load_tile = [&](int t, char* kdst_tile, char* vdst_tile) {
    const char* kt = kbase + (size_t)t * C::BK * ROWB;   // uniform tile base
    const char* vt = vbase + (size_t)t * C::BK * ROWB;
    const bool tail = (t + 1) * C::BK > a.n_kv;         // tile crosses the last valid row
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      unsigned ko = koff[r], vo = voff[r];
      if (tail) {
        const int over = t * C::BK + srow[r] - (a.n_kv - 1);   // rows past n_kv-1 re-read row n_kv-1
        if (over > 0) {
          ko -= (unsigned)(over * ROWB);
          vo -= (unsigned)(over * ROWB);
        }
      }
      char* kdst = kdst_tile + (C::NT * r + 64 * w) * 16;
      char* vdst = vdst_tile + (C::NT * r + 64 * w) * 16;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(kt + ko),
                                       (__attribute__((address_space(3))) void*)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(vt + vo),
                                       (__attribute__((address_space(3))) void*)vdst, 16, 0, 0);
    }
  };
  // the tile's LDS writes land asynchronously: wait for them before the
  // barrier that hands the buffer to the other waves
  auto tile_landed = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 acc_o[RB][C::NDB];
  float m_run[RB], l_run[RB];   // running max (log2 domain) and this lane's partial denominator
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc_o[rb][db] = f32x16{};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  // one tile: compute from (ktile, vtile) while tile t+1 streams into (knext, vnext)
  auto tile_step = [&](int t, const char* ktile, const char* vtile, char* knext, char* vnext)
      __attribute__((always_inline)) {
    const bool has_next = t < t_hi;
    if (has_next) load_tile(t + 1, knext, vnext);   // this set was released by the last barrier
    const int k0 = t * C::BK, k1 = k0 + C::BK - 1;
    const bool skip = !wave_live || k0 > pw1 || (SWA && k1 <= pw0 - a.window);
    if (!skip) {
      const bool need_mask = k1 > pw0 || k1 >= a.n_kv || (SWA && k0 <= pw1 - a.window);

      // S^T = K Q^T: each K fragment serves every row block of the wave
      f32x16 s[RB][C::NKB];
      if constexpr (sizeof(T) == 2 && RB == 1) {
        // slot n = (k step c = n / NKB, key block kb = n % NKB): the two key
        // blocks alternate, so consecutive MFMAs are independent; fragments
        // are read FRAG_AHEAD slots ahead through a small ring
        constexpr int NS = C::NC * C::NKB, PD = C::FRAG_AHEAD;
        const int krow = sigma(r32);
        frag ring[PD + 1];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s[0][kb] = f32x16{};
#pragma unroll
        for (int n = 0; n < PD; ++n) ring[n] = lds_frag_k<T, C::CH>(ktile, (n % C::NKB) * 32 + krow, n / C::NKB, g);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (n + PD < NS) {
            const int m = n + PD;
            ring[m % (PD + 1)] = lds_frag_k<T, C::CH>(ktile, (m % C::NKB) * 32 + krow, m / C::NKB, g);
          }
          s[0][n % C::NKB] = mma32(ring[n % (PD + 1)], qf[0][n / C::NKB], s[0][n % C::NKB]);
        }
        pipe_sched_prologue<1, PD, 0>();
        pipe_sched_steps<1, NS, PD, 0>();
      } else {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[rb][kb] = f32x16{};
          const int krow = kb * 32 + sigma(r32);
#pragma unroll
          for (int c = 0; c < C::NC; ++c) {
            const frag kf = lds_frag_k<T, C::CH>(ktile, krow, c, g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mma32(kf, qf[rb][c], s[rb][kb]);
          }
        }
      }

      frag pf[RB][C::NPC];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // element i of block kb <-> key k0 + kb*32 + 16*(i/8) + 8*g + i%8.
        // Masked scores become -inf (a select, never an additive mask).
        float mraw = -INFINITY;
        if (need_mask) {
          // allowed keys of this lane's row: [lo_key, hi_key]; one unsigned range test per score
          const unsigned span = (unsigned)(hi_key[rb] - lo_key[rb]);
          const int base = k0 + 8 * g - lo_key[rb];
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int off = kb * 32 + 16 * (i >> 3) + (i & 7);
              const float x = ((unsigned)(base + off) <= span) ? s[rb][kb][i] : -INFINITY;
              s[rb][kb][i] = x;
              mraw = fmaxf(mraw, x);
            }
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[rb][kb][i]);
          }
        }
        mraw = fmaxf(mraw, xor32(mraw));
        const float mloc = mraw * a.scale_log2;   // scale > 0: max commutes with it
        // Each row decides from its own scores only (rows never influence
        // each other, so results are bitwise causal).
        const bool up = mloc > m_run[rb] + 8.0f;
        if (__any(up)) {
          const float alpha = !up ? 1.f : (m_run[rb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - mloc));
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) acc_o[rb][db] *= alpha;
          m_run[rb] = up ? mloc : m_run[rb];
        }
        const float neg_m = (m_run[rb] == -INFINITY) ? 0.f : -m_run[rb];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[rb][kb][i] = __builtin_amdgcn_exp2f(fmaf(s[rb][kb][i], a.scale_log2, neg_m));
        }
        // P^T fragments: step c covers keys 16c .. 16c+15 of the tile
#pragma unroll
        for (int c = 0; c < C::NPC; ++c) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) pf[rb][c][jj] = from_f32<T>(s[rb][c >> 1][8 * (c & 1) + jj]);
        }
        // float32 row sum (4 independent partial sums for instruction-level parallelism)
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) ls[i & 3] += s[rb][kb][i];
        }
        const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        l_run[rb] += lsum;
      }
      // O^T += V^T P^T: each V^T fragment serves every row block of the wave
      if constexpr (sizeof(T) == 2 && RB == 1) {
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
          acc_o[0][n % C::NDB] = mma32(ring[n % (PD + 1)], pf[0][n / C::NDB], acc_o[0][n % C::NDB]);
        }
        pipe_sched_prologue<2, PD, 0>();
        pipe_sched_steps<2, NS, PD, 0>();
      } else {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
          for (int c = 0; c < C::NPC; ++c) {
            const frag vf = lds_frag_vt<T, C::CH>(vtile, c, db, l);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc_o[rb][db] = mma32(vf, pf[rb][c], acc_o[rb][db]);
          }
        }
      }
    }

    if (has_next) tile_landed();
    __syncthreads();
  };

  load_tile(t_lo, kbuf0, vbuf0);
  tile_landed();
  __syncthreads();
  for (int t = t_lo; t <= t_hi; t += 2) {
    tile_step(t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 <= t_hi) tile_step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }

  // ---- normalise and write ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + xor32(l_run[rb]);
    if (qi[rb] < a.Nq) {
      const float inv = 1.f / l_tot;
      T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.Hq + h) * a.Nq + qi[rb]) * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int dim = db * 32 + 8 * qd + 4 * g;
          if constexpr (sizeof(T) == 2) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc_o[rb][db][4 * qd + e] * inv);
            *reinterpret_cast<bf16x4*>(orow + dim) = v4;
          } else {
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = acc_o[rb][db][4 * qd + e] * inv;
            *reinterpret_cast<f32x4*>(orow + dim) = v4;
          }
        }
      }
      if (a.lse != nullptr && g == 0) {
        const float mref = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
        a.lse[(size_t)(b * a.Hq + h) * a.Nq + qi[rb]] = (mref + __builtin_amdgcn_logf(l_tot)) * kLn2;
      }
    }
  }
}

template <typename T, int D, bool SWA>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int nqt = (a.Nq + AttnCfg<T, D>::BQ - 1) / AttnCfg<T, D>::BQ;
  const long long nblocks = (long long)nqt * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, SWA>), dim3((unsigned)nblocks), dim3(AttnCfg<T, D>::NT), 0, stream, a);
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
