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
//  * Grid order: heaviest query tiles first (causal), and within each round
//    the heads of one KV head are placed on one XCD (workgroups go to the 8
//    XCDs round-robin), so each XCD's L2 holds one KV head's K/V.
#include "common.hpp"
#include "launch.hpp"

namespace yoco {

template <typename T, int D>
struct AttnCfg {
  static constexpr int E = Elem<T>::bytes;
  static constexpr int BQ = 128;
  static constexpr int BK = (E == 2) ? 64 : 32;
  static constexpr int CH = D * E / 16;         // 16-byte chunks per K/V row
  static constexpr int PER_T = BK * CH / 256;   // chunks per thread per tensor
  static constexpr int NKB = BK / 32;           // 32-key score blocks per tile
  static constexpr int NC = D / 16;             // 16-deep k steps over d
  static constexpr int NDB = D / 32;            // 32-wide dim blocks of O
  static constexpr int NPC = BK / 16;           // 16-key steps of P V
  static constexpr int TILE_BYTES = BK * D * E;
  static_assert(PER_T >= 1 && BK * CH % 256 == 0, "tile must split over 256 threads");
};

// Swizzle of the 16-byte chunk index within a row of the K tile: the 32 rows a
// wave reads at once (bit-permuted order) land on distinct chunk columns.
template <int CH>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (CH >= 16) return row & 15;
  else return (row & 3) | ((row >> 1) & 4);
}
// V tile: the transpose loads read 4 consecutive rows x 32 bytes per 16 lanes.
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & 3); }

// Row index permutation: swap bits 2 and 3.
__device__ __forceinline__ int sigma(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag load_frag_global(const T* p) {
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    f = *reinterpret_cast<const bf16x8*>(p);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// K fragment: elements [16c + 8g, 16c + 8g + 8) of LDS row `row`.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_k(const char* tile, int row, int c, int g) {
  using C = AttnCfg<T, D>;
  const char* rowp = tile + row * C::CH * 16;
  const int sw = swz_k<C::CH>(row);
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    const int ch = 2 * c + g;
    f = *reinterpret_cast<const bf16x8*>(rowp + ((ch ^ sw) << 4));
  } else {
    const int ch = 4 * c + 2 * g;
    f32x4 a = *reinterpret_cast<const f32x4*>(rowp + ((ch ^ sw) << 4));
    f32x4 b = *reinterpret_cast<const f32x4*>(rowp + (((ch + 1) ^ sw) << 4));
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// V^T fragment for the O^T = V^T P^T step: lane l (row = l%32 -> dim
// db*32 + l%32; k = 8*(l/32) + j -> key 16c + 8*(l/32) + j).
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_vt(const char* tile, int c, int db, int l) {
  using C = AttnCfg<T, D>;
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    // ds_read_b64_tr_b16 works on groups of 16 lanes: lane i supplies the
    // address of 4 consecutive 16-bit elements (row i/4, columns 4*(i%4)..+3
    // of a 4x16 block); lane j receives column j of that block, i.e. the 4
    // elements of rows 0..3 at column j.
    const int G = l >> 4, j16 = l & 15;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 16 * c + 8 * (G >> 1) + 4 * hh + (j16 >> 2);
      const int col = db * 32 + 16 * (G & 1) + 4 * (j16 & 3);
      const int ch = col >> 3;
      const char* p = tile + row * C::CH * 16 + ((ch ^ swz_v(row)) << 4) + ((col & 7) << 1);
      i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p));
      bf16x4 rb = __builtin_bit_cast(bf16x4, r);
      f[4 * hh + 0] = rb[0];
      f[4 * hh + 1] = rb[1];
      f[4 * hh + 2] = rb[2];
      f[4 * hh + 3] = rb[3];
    }
  } else {
    const int g = l >> 5, col = db * 32 + (l & 31);
    const int ch = col >> 2, off = (col & 3) << 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 16 * c + 8 * g + j;
      f[j] = *reinterpret_cast<const float*>(tile + row * C::CH * 16 + ((ch ^ swz_v(row)) << 4) + off);
    }
  }
  return f;
}

template <typename T, int D, bool SWA>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  using C = AttnCfg<T, D>;
  using frag = typename Elem<T>::frag;
  __shared__ __attribute__((aligned(16))) char smem[2][2][C::TILE_BYTES];  // [buf][K|V]

  const int tid = threadIdx.x;
  // wave index as a scalar: every wave-level decision below is a scalar branch
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, r32 = l & 31;

  // ---- workgroup -> (batch, head, query tile) ----
  const int BH = a.B * a.Hq;
  const int nqt = (a.Nq + C::BQ - 1) / C::BQ;
  const int id = blockIdx.x;
  const int qt = nqt - 1 - id / BH;          // heaviest (latest) tiles first
  int j = id % BH;
  if ((BH & 7) == 0) j = (j & 7) * (BH >> 3) + (j >> 3);   // same KV head -> same XCD
  const int b = j / a.Hq, h = j % a.Hq;
  const int kvh = h / (a.Hq / a.Hkv);

  const T* qbase = static_cast<const T*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq) * D;
  const char* kbase = static_cast<const char*>(a.k) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;
  const char* vbase = static_cast<const char*>(a.v) + ((size_t)(b * a.Hkv + kvh) * a.kv_rows) * D * C::E;

  // ---- this lane's query row ----
  const int q_first = qt * C::BQ;
  const int qi = q_first + w * 32 + r32;
  const int pos = a.q_offset + qi;
  const int lo_key = SWA ? max(0, pos - a.window + 1) : 0;   // allowed keys of this row
  const int hi_key = min(pos, a.n_kv - 1);
  frag qf[C::NC];
  if (qi < a.Nq) {
    const T* qrow = qbase + (size_t)qi * D;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) qf[c] = load_frag_global<T>(qrow + 16 * c + 8 * g);
  } else {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) qf[c] = frag{};
  }

  // ---- key-tile range of the workgroup and of this wave ----
  const int q_last = min(q_first + C::BQ, a.Nq) - 1;
  const int P0 = a.q_offset + q_first, P1 = a.q_offset + q_last;
  const int t_lo = SWA ? max(0, P0 - a.window + 1) / C::BK : 0;
  const int t_hi = min(P1, a.n_kv - 1) / C::BK;
  const int wq0 = q_first + w * 32;
  const bool wave_live = wq0 < a.Nq;
  const int pw0 = a.q_offset + wq0;
  const int pw1 = a.q_offset + min(wq0 + 31, a.Nq - 1);

  // ---- cooperative tile staging ----
  u32x4 kr[C::PER_T], vr[C::PER_T];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int cid = tid + 256 * r;
      const int row = cid / C::CH, ch = cid % C::CH;
      const int key = t * C::BK + row;
      if (key < a.n_kv) {
        const size_t off = (size_t)key * (D * C::E) + ch * 16;
        kr[r] = *reinterpret_cast<const u32x4*>(kbase + off);
        vr[r] = *reinterpret_cast<const u32x4*>(vbase + off);
      } else {
        kr[r] = u32x4{0, 0, 0, 0};
        vr[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::PER_T; ++r) {
      const int cid = tid + 256 * r;
      const int row = cid / C::CH, ch = cid % C::CH;
      *reinterpret_cast<u32x4*>(&smem[buf][0][row * C::CH * 16 + ((ch ^ swz_k<C::CH>(row)) << 4)]) = kr[r];
      *reinterpret_cast<u32x4*>(&smem[buf][1][row * C::CH * 16 + ((ch ^ swz_v(row)) << 4)]) = vr[r];
    }
  };

  f32x16 acc_o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY;   // running max (log2 domain) of this lane's row
  float l_run = 0.f;         // this lane's partial softmax denominator

  load_tile(t_lo);
  store_tile(0);
  __syncthreads();

  for (int t = t_lo; t <= t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const bool has_next = t < t_hi;
    if (has_next) load_tile(t + 1);

    const int k0 = t * C::BK, k1 = k0 + C::BK - 1;
    const bool skip = !wave_live || k0 > pw1 || (SWA && k1 <= pw0 - a.window);
    if (!skip) {
      const bool need_mask = k1 > pw0 || k1 >= a.n_kv || (SWA && k0 <= pw1 - a.window);
      const char* ktile = smem[buf][0];
      const char* vtile = smem[buf][1];

      // S^T = K Q^T for NKB blocks of 32 keys
      f32x16 s[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        s[kb] = f32x16{};
        const int krow = kb * 32 + sigma(r32);
#pragma unroll
        for (int c = 0; c < C::NC; ++c) s[kb] = mma32(lds_frag_k<T, D>(ktile, krow, c, g), qf[c], s[kb]);
      }
      // element i of block kb <-> key k0 + kb*32 + 16*(i/8) + 8*g + i%8.
      // Masked scores become -inf (a select, never an additive mask).
      float mraw = -INFINITY;
      if (need_mask) {
        // allowed keys of this lane's row: [lo_key, hi_key]; one unsigned range test per score
        const unsigned span = (unsigned)(hi_key - lo_key);
        const int base = k0 + 8 * g - lo_key;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = kb * 32 + 16 * (i >> 3) + (i & 7);
            const float x = ((unsigned)(base + off) <= span) ? s[kb][i] : -INFINITY;
            s[kb][i] = x;
            mraw = fmaxf(mraw, x);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[kb][i]);
        }
      }
      mraw = fmaxf(mraw, xor32(mraw));
      const float mloc = mraw * a.scale_log2;   // scale > 0: max commutes with it
      // Each row decides from its own scores only (rows of a wave never
      // influence each other, so results are bitwise causal).
      const bool up = mloc > m_run + 8.0f;
      if (__any(up)) {
        const float alpha = !up ? 1.f : (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mloc));
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) acc_o[db] *= alpha;
        m_run = up ? mloc : m_run;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, neg_m));
          s[kb][i] = p;
          lsum += p;
        }
      }
      l_run += lsum;

      // P^T fragments: step c covers keys 16c .. 16c+15 of the tile
      frag pf[C::NPC];
#pragma unroll
      for (int c = 0; c < C::NPC; ++c) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pf[c][jj] = from_f32<T>(s[c >> 1][8 * (c & 1) + jj]);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int c = 0; c < C::NPC; ++c) acc_o[db] = mma32(lds_frag_vt<T, D>(vtile, c, db, l), pf[c], acc_o[db]);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write ----
  if (qi < a.Nq) {
    const float l_tot = l_run + xor32(l_run);
    const float inv = 1.f / l_tot;
    T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.Hq + h) * a.Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int dim = db * 32 + 8 * qd + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc_o[db][4 * qd + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + dim) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc_o[db][4 * qd + e] * inv;
          *reinterpret_cast<f32x4*>(orow + dim) = v4;
        }
      }
    }
    if (a.lse != nullptr && g == 0) {
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      a.lse[(size_t)(b * a.Hq + h) * a.Nq + qi] = (mref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

template <typename T, int D, bool SWA>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int nqt = (a.Nq + AttnCfg<T, D>::BQ - 1) / AttnCfg<T, D>::BQ;
  const long long nblocks = (long long)nqt * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, SWA>), dim3((unsigned)nblocks), dim3(256), 0, stream, a);
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
