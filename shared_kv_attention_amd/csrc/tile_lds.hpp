// LDS tile layout and matrix-core fragment readers shared by the attention
// and gated-retention kernels of libyoco (gfx950).
//
// A tile holds rows of CH 16-byte chunks (CH = row bytes / 16).  Chunks are
// XOR-swizzled per row so that the reads of one wave instruction spread over
// all LDS banks; the swizzles depend on how the rows are read:
//  * "K" tiles are read as the A operand of S^T = K Q^T, 32 rows at once in
//    the permuted order sigma(r);
//  * "V" tiles are read transposed (8 consecutive rows of one column per
//    lane) with the LDS transpose load, as the A operand of O^T = V^T P^T or
//    of any product that contracts over the tile's rows.
#pragma once

#include "common.hpp"
#include "index_map.hpp"

namespace yoco {

// (sigma, swz_k and swz_v are defined in index_map.hpp)

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
template <typename T, int CH>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_k(const char* tile, int row, int c, int g) {
  const char* rowp = tile + row * CH * 16;
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    f = *reinterpret_cast<const bf16x8*>(rowp + chunk_in_row<CH, true>(row, 2 * c + g));
  } else {
    const int ch = 4 * c + 2 * g;
    f32x4 a = *reinterpret_cast<const f32x4*>(rowp + chunk_in_row<CH, true>(row, ch));
    f32x4 b = *reinterpret_cast<const f32x4*>(rowp + chunk_in_row<CH, true>(row, ch + 1));
    f = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return f;
}

// Transposed fragment of a V tile: lane l gets tile column db*32 + l%32 at
// rows 16c + 8*(l/32) + j, j = 0..7 (for O^T = V^T P^T: dim db*32 + l%32,
// keys 16c + 8*(l/32) + j).
template <typename T, int CH>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_vt(const char* tile, int c, int db, int l) {
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    // ds_read_b64_tr_b16 works on groups of 16 lanes: lane i supplies the
    // address of 4 consecutive 16-bit elements (row i/4, columns 4*(i%4)..+3
    // of a 4x16 block); lane j receives column j of that block, i.e. the 4
    // elements of rows 0..3 at column j.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = vt_frag_row(c, l, hh), col = vt_frag_col(db, l);
      const char* p = tile + row * CH * 16 + chunk_in_row<CH, false>(row, col >> 3) + ((col & 7) << 1);
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
      f[j] = *reinterpret_cast<const float*>(tile + row * CH * 16 + chunk_in_row<CH, false>(row, ch) + off);
    }
  }
  return f;
}

}  // namespace yoco
