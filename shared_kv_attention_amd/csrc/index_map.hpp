// Index arithmetic of the libyoco kernels that decides which memory a lane
// touches: workgroup -> work-item maps, key-tile spans, LDS swizzles, tile
// staging slots and fragment offsets, decode split ranges and per-block
// row counts.  Everything here is plain integer arithmetic compiled for the
// device and for the host, so that a host program can enumerate every
// workgroup, lane and slot of a launch and check coverage and bounds.
// Built with YOCO_CHECK_BOUNDS on the host, the functions also assert their
// preconditions (the device build never checks: the same arithmetic, no
// extra instructions).
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#include <hip/hip_runtime.h>
#define YOCO_HD __host__ __device__ __forceinline__
#else
#define YOCO_HD inline
#endif

#if defined(YOCO_CHECK_BOUNDS) && !defined(__HIP_DEVICE_COMPILE__)
#include <cstdio>
#include <cstdlib>
#define YOCO_ASSERT(c)                                                                     \
  do {                                                                                     \
    if (!(c)) {                                                                            \
      std::fprintf(stderr, "index check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::abort();                                                                        \
    }                                                                                      \
  } while (0)
#else
#define YOCO_ASSERT(c) ((void)0)
#endif

namespace yoco {

YOCO_HD int imin(int a, int b) { return a < b ? a : b; }
YOCO_HD int imax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// LDS row swizzles (XOR of the 16-byte chunk index within a tile row)
// ---------------------------------------------------------------------------
// Row index permutation: swap bits 2 and 3.
YOCO_HD int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// K tile (CH chunks per row): a wave reads 32 rows at once in the permuted
// order sigma(r); rows sigma(0..7) and sigma(0..15) map to distinct chunk
// columns, whether the LDS serves 8 or 16 lanes of 16-byte accesses per cycle.
template <int CH>
YOCO_HD int swz_k(int row) {
  if constexpr (CH >= 16) return sigma(row) & 15;
  else return (row & 3) | ((row >> 1) & 4);
}
// V tile: the transpose loads of 16 lanes read 4 consecutive rows x 32 bytes;
// 32 lanes read the same 4 rows x 64 bytes.
template <int CH>
YOCO_HD int swz_v(int row) {
  if constexpr (CH >= 16) return 4 * (row & 3) + 2 * ((row >> 1) & 1);
  else return 2 * (row & 3);
}
// 128-byte rows (8 chunks) read 32 rows at once: the projection's W and X tiles.
YOCO_HD int swz8(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

// ---------------------------------------------------------------------------
// Attention (flash form): workgroup -> (query tile, batch, head), key span
// ---------------------------------------------------------------------------
struct AttnTile {
  int qt, b, h;
};
// Causal: heaviest (latest) query tiles first; sliding window: natural
// order.  Within a round the heads of one KV head go to one XCD (workgroups
// are dealt to the 8 XCDs round-robin) when B*Hq is a multiple of 8.
YOCO_HD AttnTile attn_tile(int id, int B, int Hq, int nqt, bool swa) {
  const int BH = B * Hq;
  YOCO_ASSERT(id >= 0 && id < nqt * BH);
  const int qt = swa ? id / BH : nqt - 1 - id / BH;
  int j = id % BH;
  if ((BH & 7) == 0) j = (j & 7) * (BH >> 3) + (j >> 3);
  return AttnTile{qt, j / Hq, j % Hq};
}

// Key tiles [lo, hi] that query tile qt (bq rows) needs: keys up to the last
// row's position (and below n_kv), from the first row's window start.
YOCO_HD void attn_key_span(int Nq, int n_kv, int q_offset, int window, bool swa, int bq, int bk, int qt, int& lo,
                           int& hi) {
  YOCO_ASSERT(qt >= 0 && qt * bq < Nq && q_offset + Nq <= n_kv);
  const int q_first = qt * bq, q_last = imin(q_first + bq, Nq) - 1;
  const int P0 = q_offset + q_first, P1 = q_offset + q_last;
  lo = swa ? imax(0, P0 - window + 1) / bk : 0;
  hi = imin(P1, n_kv - 1) / bk;
}

// Tile staging: slot P of a tile (16-byte units, filled by consecutive
// lanes) holds row P / ch at physical chunk P % ch, i.e. logical chunk
// (P % ch) ^ swz(row); the lane that fills slot P reads that logical chunk
// of the row: this is its byte offset within the tile's rows in memory.
template <int CH, bool K>
YOCO_HD unsigned stage_offset(int slot, int row_bytes) {
  YOCO_ASSERT(row_bytes == CH * 16 && slot >= 0);
  const int row = slot / CH, pch = slot % CH;
  const int lch = pch ^ (K ? swz_k<CH>(row) : swz_v<CH>(row));
  YOCO_ASSERT(lch >= 0 && lch < CH);
  return (unsigned)(row * row_bytes + (lch << 4));
}
// Bytes of tile t (bk rows) below row n_kv (the buffer resource's size).
YOCO_HD int tile_valid_bytes(int n_kv, int t, int bk, int row_bytes) {
  return imax(0, imin(bk, n_kv - t * bk)) * row_bytes;
}

// Byte offset, within its row, of the 16-byte chunk holding logical chunk
// lch of row `row`; the row itself starts at row * CH * 16.
template <int CH, bool K>
YOCO_HD int chunk_in_row(int row, int lch) {
  YOCO_ASSERT(lch >= 0 && lch < CH && row >= 0);
  return (lch ^ (K ? swz_k<CH>(row) : swz_v<CH>(row))) << 4;
}
template <int CH, bool K>
YOCO_HD int lds_chunk_offset(int row, int lch) { return row * CH * 16 + chunk_in_row<CH, K>(row, lch); }
// Transposed V fragment (bf16, d = 8 * CH): lane l's half hh reads 4
// elements (8 bytes) at tile row 16c + 8*(G/2) + 4hh + j16/4, column
// db*32 + 16*(G%2) + 4*(j16%4), G = l / 16, j16 = l % 16.
YOCO_HD int vt_frag_row(int c, int l, int hh) { return 16 * c + 8 * ((l >> 4) >> 1) + 4 * hh + ((l & 15) >> 2); }
YOCO_HD int vt_frag_col(int db, int l) { return db * 32 + 16 * ((l >> 4) & 1) + 4 * ((l & 15) & 3); }
template <int CH>
YOCO_HD int vt_frag_offset(int c, int db, int l, int hh) {
  const int row = vt_frag_row(c, l, hh), col = vt_frag_col(db, l);
  return lds_chunk_offset<CH, false>(row, col >> 3) + ((col & 7) << 1);
}

// ---------------------------------------------------------------------------
// Global KV projection: workgroup -> (feature tile, token tile)
// ---------------------------------------------------------------------------
// With an even number of feature tiles, each XCD takes one block of a 2 x 4
// partition (half of the feature tiles, a quarter of the token tiles, the
// token tiles padded to a multiple of 4); padded workgroups have no work.
// The projection's three-stage ring form: bf16 without a norm gain, the
// features in 256-row tiles, and at least one such tile per CU (256).
YOCO_HD bool proj_ring_form(long long M, int F, bool is_bf16, bool has_gain) {
  return is_bf16 && !has_gain && F % 256 == 0 && ((M + 127) / 128) * (F / 256) >= 256;
}
YOCO_HD int proj_workgroups(int nft, int ntt) { return nft % 2 == 0 ? 8 * (nft / 2) * ((ntt + 3) / 4) : ntt * nft; }
YOCO_HD bool proj_tile(int id, int nft, int ntt, int& ft, int& tt) {
  YOCO_ASSERT(id >= 0 && id < proj_workgroups(nft, ntt));
  if (nft % 2 == 0) {
    const int xcd = id & 7, sl = id >> 3;
    const int fpx = nft / 2, tpx = (ntt + 3) / 4;
    ft = (xcd & 1) * fpx + sl % fpx;
    tt = (xcd >> 1) * tpx + sl / fpx;
    return tt < ntt;
  }
  ft = id % nft;
  tt = id / nft;
  return true;
}

// ---------------------------------------------------------------------------
// Decode: a split's key range and the rows of one 16-key block
// ---------------------------------------------------------------------------
YOCO_HD int decode_key_begin(int split, int chunk) { return split * chunk; }
YOCO_HD int decode_key_end(int split, int chunk, int ctx_b) { return imin(split * chunk + chunk, ctx_b); }
// rows of the 16-key block at key0 below key_end (its buffer resource's rows)
YOCO_HD int decode_block_rows(int key_end, int key0) { return imax(0, imin(16, key_end - key0)); }
// lane byte offsets within a block (rb bytes per row, esz bytes per element):
// K in operand layout (key r16, elements 8G.. of each 32-element step),
// V slices (the lane's dpl dims of a row), whole-line K (key r16 % 8 of
// half (r16 / 8), elements 32 (r16 / 8) + 8G..)
YOCO_HD int decode_k_offset(int l, int rb, int esz) { return (l & 15) * rb + 8 * (l >> 4) * esz; }
YOCO_HD int decode_v_offset(int l, int dpl, int esz) { return dpl * l * esz; }
YOCO_HD int decode_kf_offset(int l, int rb, int esz) {
  const int r16 = l & 15, G = l >> 4;
  return (r16 & 7) * rb + (32 * (r16 >> 3) + 8 * G) * esz;
}

}  // namespace yoco
