// Split-K decode attention over the shared global cache (one query token per
// sequence), and the combine pass that merges the splits.
//
// What is computed (YOCO podcast transcript, segments 4, 14 and 26;
// paperlayer.ai summary of "You Only Cache Once", section 2): for sequence b
// and query head h, o = softmax(scale * q K^T) V over cache rows 0..ctx_b-1 of
// KV head h / (Hq/Hkv).  Every cross-decoder layer streams the whole cache at
// every step, so the kernel is bound by HBM bandwidth.
//
// Design (MI355X-first):
//  * Grid (split, kv-head x head-group, batch); one wave per workgroup.  A
//    workgroup reads its slice of K and V exactly once and serves all (up to
//    4) query heads of its KV head.  Splits give thousands of workgroups even
//    for one sequence, so all 256 CUs stream concurrently.
//  * Keys are processed 16 at a time.  For q . k, lane l holds key l%16 and
//    dims {32c + 8*(l/16) + j}, the operand layout of the 16x16x32 matrix
//    core, so K needs no LDS staging.  fp8 and float32 caches load that
//    layout directly (one 8- or 32-byte row piece per lane and step), and so
//    do bf16 caches with short splits.  With long splits bf16 caches load
//    whole 128-byte lines instead -- each instruction 8 keys x one line,
//    non-temporal -- and a row rotate by 8 within 16-lane rows
//    (DPP, written into half of the lanes) rearranges two such loads into
//    the fragments of two matrix steps.  The A operand is the query block
//    replicated 4 times (row r -> head r%4), so every lane receives all 4
//    heads' scores of its own key.
//  * For P V each lane owns D/64 output dims across all keys: one V row is
//    read by one load instruction (fully contiguous), and the per-lane
//    accumulator is only 4 heads x D/64 floats -- no cross-lane reduction of
//    O is ever needed and occupancy stays high.  Probabilities reach the
//    lanes as wave-uniform scalars (readlane); for bf16 / fp8 caches two keys
//    are handled per v_dot2_f32_bf16 (probabilities rounded to bf16, as in
//    any bf16 attention; float32 accumulation), for float32 caches by exact
//    float32 FMAs.
//  * Online softmax in the exp2 domain; the running max per head is raised
//    only when a block exceeds it by 2^8 (wave-uniform branch).
//  * Loads run ahead of use: V one block; K one block (fp8, float32), two
//    for the bf16 instruction that first touches a line, three in the
//    whole-line form.  The whole-line form takes 3 waves per SIMD instead of
//    4 and pays only on long splits (>= 1024 keys: the 32K x B16 and 1M
//    decodes, +3 %); shorter splits keep the operand-layout form.
//  * fp8-e4m3 caches: codes are decoded in registers (exactly, to bf16 for
//    the matrix core and to f32 for P V); the per-head scales factor out of
//    both products: the K scale is folded into the softmax scale and the V
//    scale multiplies the split's partial output once.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "index_map.hpp"

namespace yoco {

template <typename KVT> struct KvTraits;
template <> struct KvTraits<bf16> { static constexpr int bytes = 2; using mma_t = bf16; };
template <> struct KvTraits<float> { static constexpr int bytes = 4; using mma_t = float; };
template <> struct KvTraits<uint8_t> { static constexpr int bytes = 1; using mma_t = bf16; };

// Raw per-lane storage for 8 consecutive elements of one K row.
template <typename KVT> struct Raw8;
template <> struct Raw8<bf16> { u32x4 w; };
template <> struct Raw8<float> { u32x4 lo, hi; };
template <> struct Raw8<uint8_t> { u32x2 w; };

// The same 8 elements through a buffer resource: `off` bytes from its base.
// Bytes at or past the resource's size read as zeros.
template <typename KVT>
__device__ __forceinline__ Raw8<KVT> buf_raw8(__amdgpu_buffer_rsrc_t r, int off) {
  Raw8<KVT> x;
  if constexpr (sizeof(KVT) == 2) {
    x.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else if constexpr (sizeof(KVT) == 4) {
    x.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    x.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  } else {
    x.w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
  return x;
}

// The same 8 elements from a plain pointer.
template <typename KVT>
__device__ __forceinline__ Raw8<KVT> raw8_at(const char* p) {
  Raw8<KVT> x;
  if constexpr (sizeof(KVT) == 2) {
    x.w = *reinterpret_cast<const u32x4*>(p);
  } else if constexpr (sizeof(KVT) == 4) {
    x.lo = *reinterpret_cast<const u32x4*>(p);
    x.hi = *reinterpret_cast<const u32x4*>(p + 16);
  } else {
    x.w = *reinterpret_cast<const u32x2*>(p);
  }
  return x;
}

// Cache-policy bits of a buffer load: streaming (non-temporal).
constexpr int kLoadNT = 2;

// Raw K elements -> matrix-core operand fragment.
template <typename KVT>
__device__ __forceinline__ typename Elem<typename KvTraits<KVT>::mma_t>::frag to_frag(const Raw8<KVT>& r) {
  if constexpr (sizeof(KVT) == 2) {
    return __builtin_bit_cast(bf16x8, r.w);
  } else if constexpr (sizeof(KVT) == 4) {
    f32x4 a = __builtin_bit_cast(f32x4, r.lo), b = __builtin_bit_cast(f32x4, r.hi);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    // two codes per instruction, straight to bf16 (exact: every e4m3 value
    // is a bf16 value; the scale operand is 1)
    bf16x8 f;
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w[wd], 1.0f, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w[wd], 1.0f, true);
      f[4 * wd + 0] = lo[0];
      f[4 * wd + 1] = lo[1];
      f[4 * wd + 2] = hi[0];
      f[4 * wd + 3] = hi[1];
    }
    return f;
  }
}

// One lane's V slice of one row through a buffer resource (streaming load).
template <typename W>
__device__ __forceinline__ W buf_vword(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (sizeof(W) == 1) return (W)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kLoadNT);
  else if constexpr (sizeof(W) == 2) return (W)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kLoadNT);
  else if constexpr (sizeof(W) == 4) return (W)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadNT);
  else return __builtin_bit_cast(W, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadNT));
}

// The V slice one lane owns in one key row: DPL = D/64 consecutive elements.
template <typename KVT, int DPL> struct VSlice {
  static constexpr int bytes = DPL * (int)sizeof(KVT);
  using type = typename std::conditional<bytes == 1, uint8_t,
               typename std::conditional<bytes == 2, uint16_t,
               typename std::conditional<bytes == 4, uint32_t, u32x2>::type>::type>::type;
};

template <typename KVT, int DPL>
__device__ __forceinline__ void vslice_to_f32(typename VSlice<KVT, DPL>::type w, float* out) {
  if constexpr (sizeof(KVT) == 1) {
    const f32x2 v = fp8x2_to_f32((uint32_t)w, false);
    out[0] = v[0];
    if constexpr (DPL == 2) out[1] = v[1];
  } else if constexpr (sizeof(KVT) == 2) {
    if constexpr (DPL == 1) {
      out[0] = __uint_as_float((uint32_t)w << 16);
    } else {
      out[0] = __uint_as_float((uint32_t)w << 16);
      out[1] = __uint_as_float((uint32_t)w & 0xFFFF0000u);
    }
  } else {
    if constexpr (DPL == 1) {
      out[0] = __uint_as_float((uint32_t)w);
    } else {
      out[0] = __uint_as_float(w[0]);
      out[1] = __uint_as_float(w[1]);
    }
  }
}

template <typename QT>
__device__ __forceinline__ typename Elem<QT>::frag load_q_frag(const QT* p) {
  if constexpr (sizeof(QT) == 2) {
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

__device__ __forceinline__ int decode_ctx(const DecodeArgs& a, int b) {
  if (a.ctx_lens == nullptr) return a.ctx;
  return min(max((int)a.ctx_lens[b], 1), a.ctx);
}

template <typename QT, typename KVT, int D, bool KF, bool RING = false>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using MT = typename KvTraits<KVT>::mma_t;
  static_assert(sizeof(MT) == sizeof(QT), "query dtype must match the matrix-core dtype");
  using frag = typename Elem<MT>::frag;
  constexpr int NC = D / 32;     // 32-dim matrix-core steps of q . k
  constexpr int DPL = D / 64;    // output dims owned by each lane in P V
  using vword = typename VSlice<KVT, DPL>::type;

  const int l = threadIdx.x, r16 = l & 15, G = l >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / a.n_hg, hg = blockIdx.y % a.n_hg;
  const int b = blockIdx.z;
  const int grp = a.Hq / a.Hkv;
  const int h0 = kvh * grp + 4 * hg;
  const int nh = min(4, grp - 4 * hg);

  const int ctx_b = decode_ctx(a, b);
  const int key_begin = decode_key_begin(split, a.chunk);
  if (key_begin >= ctx_b) return;
  const int key_end = decode_key_end(split, a.chunk, ctx_b);

  // Query operand: row r -> head (r & 3) of this group (zero beyond nh).
  frag qa[NC];
  {
    const int hh = r16 & 3;
    if (hh < nh) {
      const QT* qrow = static_cast<const QT*>(a.q) + (size_t)(b * a.Hq + h0 + hh) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qa[c] = load_q_frag<QT>(qrow + 32 * c + 8 * G);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qa[c] = frag{};
    }
  }
  float sc = a.scale_log2;
  if constexpr (sizeof(KVT) == 1) sc *= a.k_scale[kvh];

  // Loads go through buffer resources built per 16-key block: base = the
  // block's first row, size = its rows below key_end.  Lane offsets are then
  // loop-invariant (no per-load address arithmetic) and rows at or past
  // key_end -- the tail of the last block -- read as zeros (masked out).
  constexpr int RB = D * (int)sizeof(KVT);                                       // bytes per cache row
  const size_t head_off = (size_t)(b * a.Hkv + kvh) * a.n_cap;
  const char* kh = uniform_ptr(static_cast<const char*>(a.k) + head_off * RB);
  const char* vh = uniform_ptr(static_cast<const char*>(a.v) + head_off * RB);
  const int kend = __builtin_amdgcn_readfirstlane(key_end);
  auto block_rsrc = [&](const char* hb, int key0) {
    const int rows = __builtin_amdgcn_readfirstlane(decode_block_rows(kend, key0));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(hb + (size_t)key0 * RB), (short)0, rows * RB, kBufferFlags);
  };
  const int koff = decode_k_offset(l, RB, (int)sizeof(KVT));     // K, operand layout: key r16, elements 8G ..
  const int voff = decode_v_offset(l, DPL, (int)sizeof(KVT));    // V: this lane's dims

  // The current token of a ring cache (the append folded in): its row lies
  // in this split's range for one split only; that split reads it from
  // k_new / v_new (below), and its first head group writes it into the
  // ring.  No other workgroup of this launch reads that ring row.
  const int ns = RING ? a.new_slot : -1;
  const bool patch = RING && ns >= key_begin && ns < key_end;
  const char* knew_row = static_cast<const char*>(a.k_new) + (size_t)(b * a.Hkv + kvh) * RB;
  const char* vnew_row = static_cast<const char*>(a.v_new) + (size_t)(b * a.Hkv + kvh) * RB;
  if (RING && patch && hg == 0) {
    char* kd = const_cast<char*>(kh) + (size_t)ns * RB;
    char* vd = const_cast<char*>(vh) + (size_t)ns * RB;
    for (int i = l; i < RB / 4; i += 64) {
      reinterpret_cast<uint32_t*>(kd)[i] = reinterpret_cast<const uint32_t*>(knew_row)[i];
      reinterpret_cast<uint32_t*>(vd)[i] = reinterpret_cast<const uint32_t*>(vnew_row)[i];
    }
  }

  float m_run[4], l_run[4];
  float acc[4][DPL];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[i][e] = 0.f;
  }

  // Operand-layout K loads (fp8, float32, and bf16 with short splits): lane
  // (G, r16) loads key r16's elements 32c + 8G .. +7 for each step c.  One
  // instruction covers 16 rows x 32 dims, half of a 128-byte line of each
  // bf16 row; for bf16 the instruction that touches a line first ("lead") is
  // issued two blocks ahead and the other one block ahead, so the line's fill
  // is under way when the second arrives (+3 % on the 32K decode; fp8 measured
  // slower with it and keeps one block).
  constexpr bool KFULL = KF && sizeof(KVT) == 2;
  // fp8 caches: every K and V load is issued two blocks ahead (a block is
  // only 4 KB there, half of a bf16 block)
  constexpr bool AHEAD2 = sizeof(KVT) == 1;
  auto is_lead = [](int c) { return AHEAD2 || (!KFULL && sizeof(KVT) == 2 && (c & 1) == 0); };
  Raw8<KVT> kc[NC], kn[NC], k2[NC];
  auto load_k = [&](int key0, Raw8<KVT>* kr, bool lead) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kh, key0);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (is_lead(c) == lead) kr[c] = buf_raw8<KVT>(rk, koff + 32 * c * (int)sizeof(KVT));
  };
  // Whole-line K loads (bf16, long splits): instruction (line L, half h)
  // gives lane (G, k) the 16 bytes of key 8h + (k & 7) at element
  // 64L + 32(k >> 3) + 8G: 8 keys x one full line per instruction, so it
  // streams non-temporally (the operand-layout loads above touch each line
  // with two instructions and must stay cached).  A row rotate by 8 within
  // each 16-lane row, written into half of the lanes (bank mask), turns the
  // two halves of line L into the fragments of steps 2L and 2L + 1 (lane
  // (G, k): key k, elements 32c + 8G .. +7).  Three blocks in flight.
  constexpr int NL = D / 64;
  const int kfoff = decode_kf_offset(l, RB, (int)sizeof(KVT));
  auto load_kf = [&](int key0, u32x4 (&raw)[NL][2]) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kh, key0);
#pragma unroll
    for (int L = 0; L < NL; ++L)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        raw[L][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            rk, kfoff + 8 * h * RB + 64 * L * (int)sizeof(KVT), 0, kLoadNT));
  };
  auto kf_frags = [&](const u32x4 (&raw)[NL][2], Raw8<KVT>* kr) {
    if constexpr (KFULL) {
#pragma unroll
      for (int L = 0; L < NL; ++L)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // row_ror:8 (0x128); banks 2-3 (lanes k >= 8) take the other half's keys
          kr[2 * L].w[w] = (uint32_t)__builtin_amdgcn_update_dpp((int)raw[L][0][w], (int)raw[L][1][w], 0x128, 0xF, 0xC, false);
          kr[2 * L + 1].w[w] = (uint32_t)__builtin_amdgcn_update_dpp((int)raw[L][1][w], (int)raw[L][0][w], 0x128, 0xF, 0x3, false);
        }
    }
  };
  u32x4 kf0[NL][2], kf1[NL][2], kf2[NL][2], kf3[NL][2];
  vword vc[16], vn[16], v2[16];
  auto load_v = [&](int key0, vword* vr) {
    // each V row is consumed whole by these loads: stream it non-temporally
    // (+8 % on the 32K decode over cached loads)
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vh, key0);
#pragma unroll
    for (int j = 0; j < 16; ++j) vr[j] = buf_vword<vword>(rv, voff + j * RB);
  };

  if constexpr (KFULL) {
    load_kf(key_begin, kf0);
    if (key_begin + 16 < key_end) load_kf(key_begin + 16, kf1);
    if (key_begin + 32 < key_end) load_kf(key_begin + 32, kf2);
  } else {
    load_k(key_begin, kc, true);
    load_k(key_begin, kc, false);
  }
  load_v(key_begin, vc);
  if (!KFULL && key_begin + 16 < key_end) load_k(key_begin + 16, kn, true);
  if (AHEAD2 && key_begin + 16 < key_end) load_v(key_begin + 16, vn);
  for (int key0 = key_begin; key0 < key_end; key0 += 16) {
    const bool has_next = key0 + 16 < key_end;
    if (has_next) {
      if constexpr (!KFULL) load_k(key0 + 16, kn, false);
      if constexpr (!AHEAD2) load_v(key0 + 16, vn);
    }
    if (!KFULL && key0 + 32 < key_end) load_k(key0 + 32, k2, true);
    if (AHEAD2 && key0 + 32 < key_end) load_v(key0 + 32, v2);
    if constexpr (KFULL) {
      if (key0 + 48 < key_end) load_kf(key0 + 48, kf3);
      kf_frags(kf0, kc);
    }

    if (RING && patch && key0 <= ns && ns < key0 + 16) {
      // the current token's row: K for the lanes of its key, V for every lane
      const int rel = ns - key0;
      if (r16 == rel) {
#pragma unroll
        for (int c = 0; c < NC; ++c) kc[c] = raw8_at<KVT>(knew_row + (32 * c + 8 * G) * (int)sizeof(KVT));
      }
      const vword nv = *reinterpret_cast<const vword*>(vnew_row + voff);
#pragma unroll
      for (int j = 0; j < 16; ++j) vc[j] = j == rel ? nv : vc[j];
    }

    // scores: lane (G, r16) receives head i's score of key key0 + r16 in s[i]
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = mma16(qa[c], to_frag<KVT>(kc[c]), s);
    const bool valid = key0 + r16 < key_end;
    float x[4];
    bool up = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = valid ? s[i] * sc : -INFINITY;
      up |= x[i] > m_run[i] + 8.0f;
    }
    if (__any(up)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m_new = fmaxf(m_run[i], row16_max(x[i]));
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
        l_run[i] *= alpha;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[i][e] *= alpha;
        m_run[i] = m_new;
      }
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mref = (m_run[i] == -INFINITY) ? 0.f : m_run[i];
      p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
      l_run[i] += p[i];
    }
    if constexpr (sizeof(KVT) == 4) {
      // float32 cache: exact float32 products; key j's probabilities are
      // read from lane j as wave-uniform scalars
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float vf[DPL];
        vslice_to_f32<KVT, DPL>(vc[j], vf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pjf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[i]), j));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[i][e] = fmaf(pjf, vf[e], acc[i][e]);
        }
      }
    } else {
      // bf16 / fp8 cache: two keys per instruction with v_dot2_f32_bf16.
      // Lane 2m packs (p_2m, p_2m+1) as bf16x2 (neighbour via DPP); the pair
      // is read as a wave-uniform scalar.  The V values of keys 2m, 2m+1 at
      // the same dim are paired with a byte permute (fp8 codes are decoded
      // exactly to bf16 first).  Accumulation stays float32.
      uint32_t pp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float nb = dpp_f32<kDppQuadSwap1>(p[i]);
        pp[i] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)p[i], (bf16)nb});
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        bf16x2 ps[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ps[i] = __builtin_bit_cast(bf16x2, (uint32_t)__builtin_amdgcn_readlane((int)pp[i], 2 * m));
        bf16x2 vp[DPL];
        if constexpr (sizeof(KVT) == 2) {
          if constexpr (DPL == 2) {
            vp[0] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm((uint32_t)vc[2 * m + 1], (uint32_t)vc[2 * m], 0x05040100u));
            vp[1] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm((uint32_t)vc[2 * m + 1], (uint32_t)vc[2 * m], 0x07060302u));
          } else {
            vp[0] = __builtin_bit_cast(bf16x2, (uint32_t)vc[2 * m] | ((uint32_t)vc[2 * m + 1] << 16));
          }
        } else {
          // codes of keys 2m (a) and 2m + 1 (b), interleaved by dim, then two
          // codes per instruction to bf16 (exact)
          if constexpr (DPL == 2) {
            const uint32_t x = __builtin_amdgcn_perm((uint32_t)vc[2 * m + 1], (uint32_t)vc[2 * m], 0x05010400u);  // a0 b0 a1 b1
            vp[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
            vp[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
          } else {
            const uint32_t w = (uint32_t)vc[2 * m] | ((uint32_t)vc[2 * m + 1] << 8);   // a0 b0
            vp[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[i][e] = __builtin_amdgcn_fdot2_f32_bf16(ps[i], vp[e], acc[i][e], false);
        }
      }
    }
    if (has_next) {
      if constexpr (KFULL) {
#pragma unroll
        for (int L = 0; L < NL; ++L)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            kf0[L][h] = kf1[L][h];
            kf1[L][h] = kf2[L][h];
            kf2[L][h] = kf3[L][h];
          }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          kc[c] = kn[c];
          if (is_lead(c)) kn[c] = k2[c];
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        vc[j] = vn[j];
        if constexpr (AHEAD2) vn[j] = v2[j];
      }
    }
  }

  // l: sum of the 16 key-lanes (the 4 rows hold identical copies)
  float vscale = 1.f;
  if constexpr (sizeof(KVT) == 1) vscale = a.v_scale[kvh];
  const size_t S = gridDim.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lt = row16_sum(l_run[i]);
    if (i < nh) {
      const size_t row = (size_t)(b * a.Hq + h0 + i) * S + split;
      float* dst = a.part_o + row * D + DPL * l;
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[e] = acc[i][e] * vscale;
      if (l == 0) {
        a.part_m[row] = m_run[i];
        a.part_l[row] = lt;
      }
    }
  }
}

// Merge of the split partials.  The maximum, the weights 2^(m_s - M) and the
// denominator are reduced over splits in parallel; then 8 thread groups sum
// strided subsets of the splits' partial numerators (coalesced 128-byte rows,
// four independent chains each) and meet in LDS.
constexpr int kMaxSplits = kDecodeMaxSplits;

__device__ __forceinline__ float block256_reduce(float x, bool is_max, float* red4) {
  x = is_max ? row16_max(x) : row16_sum(x);
  const float y16 = __shfl_xor(x, 16);
  x = is_max ? fmaxf(x, y16) : x + y16;
  const float y32 = __shfl_xor(x, 32);
  x = is_max ? fmaxf(x, y32) : x + y32;
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = is_max ? fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]))
                         : (red4[0] + red4[1]) + (red4[2] + red4[3]);
  __syncthreads();
  return r;
}

template <typename OT, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  // grid (query head, batch, D / 32): each workgroup owns 32 output dims;
  // its 256 threads are 8 split groups x 32 dims.
  constexpr int NG = 8;
  __shared__ float wgt[kMaxSplits];
  __shared__ float red4[4];
  __shared__ float part[NG][32];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int S = a.n_splits;
  const int ctx_b = decode_ctx(a, b);
  const int ns = (ctx_b + a.chunk - 1) / a.chunk;
  const size_t base = (size_t)(b * a.Hq + h) * S;

  const int dl = tid & 31, grp = tid >> 5;
  const int dim = blockIdx.z * 32 + dl;
  // this thread's first PF partial outputs (splits grp, grp + NG, ...) are
  // requested with the maxima, so that the three phases below share one
  // round trip to memory for the common split counts (ns <= NG * PF)
  constexpr int PF = 8;
  float ov[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int sk = grp + k * NG;
    ov[k] = sk < ns ? a.part_o[(base + sk) * D + dim] : 0.f;
  }

  float m = -INFINITY;
  for (int s = tid; s < ns; s += 256) m = fmaxf(m, a.part_m[base + s]);
  const float M = block256_reduce(m, true, red4);
  float lsum = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float w = __builtin_amdgcn_exp2f(a.part_m[base + s] - M);
    wgt[s] = w;
    lsum = fmaf(w, a.part_l[base + s], lsum);
  }
  const float L = block256_reduce(lsum, false, red4);   // its barriers also publish wgt[]

  // split k of this thread (s = grp + k NG, k < K) goes to chain k % 4 while
  // a whole group of four remains (k < K4), the rest to chain 0, in order
  float acc[4] = {0.f, 0.f, 0.f, 0.f};   // independent chains
  const int K = grp < ns ? (ns - grp + NG - 1) / NG : 0;
  const int K4 = K & ~3;
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    if (k < K) {
      const float wk = wgt[grp + k * NG];
      if (k < K4) acc[k & 3] = fmaf(wk, ov[k], acc[k & 3]);
      else acc[0] = fmaf(wk, ov[k], acc[0]);
    }
  }
  int k = PF;
  for (; k < K4; k += 4) {   // PF and K4 are multiples of 4
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int su = grp + (k + u) * NG;
      acc[u] = fmaf(wgt[su], a.part_o[(base + su) * D + dim], acc[u]);
    }
  }
  for (; k < K; ++k) {
    const int sk = grp + k * NG;
    acc[0] = fmaf(wgt[sk], a.part_o[(base + sk) * D + dim], acc[0]);
  }
  part[grp][dl] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (grp == 0) {
    float tot = part[0][dl];
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) tot += part[g2][dl];
    OT* o = static_cast<OT*>(a.o) + (size_t)(b * a.Hq + h) * D;
    o[dim] = from_f32<OT>(tot / L);
    if (a.lse != nullptr && dim == 0) a.lse[b * a.Hq + h] = (M + __builtin_amdgcn_logf(L)) * kLn2;
  }
}

template <typename QT, typename KVT, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.Hkv * a.n_hg, a.B);
  // ring caches with a token to append take the RING instantiations (the
  // plain decode kernels carry none of that code)
  const bool ring = sizeof(KVT) != 1 && a.k_new != nullptr;
  bool launched = false;
  if constexpr (sizeof(KVT) == 2 && D == 128) {
    if (a.full_lines) {
      if (ring) hipLaunchKernelGGL((decode_split_kernel<QT, KVT, D, true, true>), grid, dim3(64), 0, stream, a);
      else hipLaunchKernelGGL((decode_split_kernel<QT, KVT, D, true>), grid, dim3(64), 0, stream, a);
      launched = true;
    }
  }
  if constexpr (sizeof(KVT) != 1) {
    if (!launched && ring) {
      hipLaunchKernelGGL((decode_split_kernel<QT, KVT, D, false, true>), grid, dim3(64), 0, stream, a);
      launched = true;
    }
  }
  if (!launched) hipLaunchKernelGGL((decode_split_kernel<QT, KVT, D, false>), grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<QT, D>), dim3(a.Hq, a.B, D / 32), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of per-shard attention results (a cache split across devices, each
// shard decoded with its log-sum-exp): o = sum_s exp(lse_s - L) o_s with
// L = log sum_s exp(lse_s).  One workgroup per row, one thread per channel.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void attn_merge_kernel(MergeArgs a) {
  const int row = blockIdx.x, c = threadIdx.x;
  const size_t stride = (size_t)a.rows;   // between shards, in rows
  float m = -INFINITY;
  for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.lse_parts[s * stride + row]);
  float tot = 0.f, acc = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const float w = __expf(a.lse_parts[s * stride + row] - m);
    tot += w;
    acc = fmaf(w, to_f32(static_cast<const T*>(a.o_parts)[(s * stride + row) * a.d + c]), acc);
  }
  static_cast<T*>(a.o)[(size_t)row * a.d + c] = from_f32<T>(acc / tot);
  if (a.lse != nullptr && c == 0) a.lse[row] = m + __logf(tot);
}

hipError_t launch_attn_merge(const MergeArgs& a, bool is_bf16, hipStream_t stream) {
  if (is_bf16) hipLaunchKernelGGL(attn_merge_kernel<bf16>, dim3((unsigned)a.rows), dim3(a.d), 0, stream, a);
  else hipLaunchKernelGGL(attn_merge_kernel<float>, dim3((unsigned)a.rows), dim3(a.d), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int q_kind, int kv_kind, int d, hipStream_t stream) {
  // kinds: 0 = f32, 1 = bf16, 2 = fp8-e4m3 codes
  if (q_kind == 0) return d == 128 ? launch_decode_t<float, float, 128>(a, stream) : launch_decode_t<float, float, 64>(a, stream);
  if (kv_kind == 1) return d == 128 ? launch_decode_t<bf16, bf16, 128>(a, stream) : launch_decode_t<bf16, bf16, 64>(a, stream);
  return d == 128 ? launch_decode_t<bf16, uint8_t, 128>(a, stream) : launch_decode_t<bf16, uint8_t, 64>(a, stream);
}

}  // namespace yoco
