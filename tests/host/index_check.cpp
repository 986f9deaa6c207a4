// Host enumeration of the kernels' index arithmetic (index_map.hpp, built
// with YOCO_CHECK_BOUNDS so that every helper also asserts its
// preconditions), under AddressSanitizer and UndefinedBehaviorSanitizer:
//  * LDS swizzles are permutations of a row's chunks;
//  * tile staging and fragment reads agree: the slot a lane fills with
//    logical chunk (row, c) is the slot every reader of (row, c) addresses,
//    and a wave's K fragment reads (transposed V reads) cover the tile once;
//  * attention workgroups cover every (query tile, batch, head) once, and a
//    query tile's key span holds every key its rows may see;
//  * the projection's XCD partition covers every (feature, token) tile once;
//  * decode splits partition the context, block rows stay within 16, and
//    every lane offset stays inside a 16-key block.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <vector>

#include "index_map.hpp"
#include "launch.hpp"

#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "CHECK failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::abort();                                                              \
    }                                                                            \
  } while (0)

using namespace yoco;

template <int CH>
static void check_swizzles() {
  for (int row = 0; row < 256; ++row) {
    for (int K = 0; K < 2; ++K) {
      std::set<int> seen;
      for (int lch = 0; lch < CH; ++lch) {
        const int off = K ? chunk_in_row<CH, true>(row, lch) : chunk_in_row<CH, false>(row, lch);
        CHECK(off % 16 == 0 && off / 16 < CH);
        seen.insert(off / 16);
      }
      CHECK((int)seen.size() == CH);
    }
  }
}

// staging of a BK-row tile by NT threads (wave w fills 64 consecutive slots
// per instruction), then the readers' offsets
template <int CH, int BK, int NT>
static void check_tile(bool bf16) {
  constexpr int ROWB = CH * 16, TILE = BK * ROWB;
  constexpr int PER_T = BK * CH / NT;
  static_assert(PER_T >= 1 && BK * CH % NT == 0, "tile split");
  for (int K = 0; K < 2; ++K) {
    std::vector<int> filled(BK * CH, 0);
    for (int w = 0; w < NT / 64; ++w)
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < PER_T; ++r) {
          const int slot = NT * r + 64 * w + l;
          CHECK(slot < BK * CH);
          const unsigned src = K ? stage_offset<CH, true>(slot, ROWB) : stage_offset<CH, false>(slot, ROWB);
          CHECK(src % 16 == 0 && src < (unsigned)TILE);
          const int row = (int)src / ROWB, lch = (int)(src % ROWB) / 16;
          // the reader of (row, lch) addresses exactly this slot
          const int dst = K ? lds_chunk_offset<CH, true>(row, lch) : lds_chunk_offset<CH, false>(row, lch);
          CHECK(dst == slot * 16);
          ++filled[slot];
        }
    for (int s : filled) CHECK(s == 1);
  }
  if (!bf16) return;
  // K fragments of one wave: rows kb*32 + sigma(l % 32), chunk 2c + l / 32
  {
    std::vector<int> hits(BK * CH, 0);
    for (int kb = 0; kb < BK / 32; ++kb)
      for (int c = 0; c < CH / 2; ++c)
        for (int l = 0; l < 64; ++l) {
          const int row = kb * 32 + sigma(l & 31);
          const int off = row * ROWB + chunk_in_row<CH, true>(row, 2 * c + (l >> 5));
          CHECK(off >= 0 && off + 16 <= TILE && off % 16 == 0);
          ++hits[off / 16];
        }
    for (int h : hits) CHECK(h == 1);
  }
  // transposed V fragments of one wave: 4 elements per (lane, half)
  {
    constexpr int D = CH * 8;
    std::vector<int> hits(BK * D / 4, 0);
    for (int c = 0; c < BK / 16; ++c)
      for (int db = 0; db < D / 32; ++db)
        for (int l = 0; l < 64; ++l)
          for (int hh = 0; hh < 2; ++hh) {
            const int off = vt_frag_offset<CH>(c, db, l, hh);
            CHECK(off >= 0 && off + 8 <= TILE && off % 8 == 0);
            ++hits[off / 8];
            // the four elements are column vt_frag_col .. +3 of row vt_frag_row
            const int row = vt_frag_row(c, l, hh), col = vt_frag_col(db, l);
            CHECK(row < BK && col + 3 < D && (col & 3) == 0);
          }
    for (int h : hits) CHECK(h == 1);
  }
}

static void check_attention_maps() {
  struct Case { int B, Hq, Nq, n_kv, q_offset, window, bq, bk; bool swa; };
  const Case cases[] = {
      {1, 24, 4096, 4096, 0, 1024, 128, 64, false}, {1, 24, 4096, 4096, 0, 1024, 128, 32, true},
      {2, 6, 190, 190, 0, 0, 128, 64, false},       {1, 8, 70, 300, 230, 0, 128, 64, false},
      {2, 4, 1, 257, 256, 0, 128, 64, false},       {1, 3, 130, 130, 0, 1000, 128, 32, true},
      {2, 6, 300, 300, 0, 70, 128, 32, true},       {1, 8, 200, 200, 0, 1, 128, 32, true},
      {3, 8, 517, 517, 0, 256, 128, 64, true},      {1, 32, 1000, 3000, 2000, 64, 128, 64, true}};
  for (const Case& c : cases) {
    const int nqt = (c.Nq + c.bq - 1) / c.bq, total = nqt * c.B * c.Hq;
    std::set<std::tuple<int, int, int>> seen;
    for (int id = 0; id < total; ++id) {
      const AttnTile t = attn_tile(id, c.B, c.Hq, nqt, c.swa);
      CHECK(t.qt >= 0 && t.qt < nqt && t.b >= 0 && t.b < c.B && t.h >= 0 && t.h < c.Hq);
      seen.insert({t.qt, t.b, t.h});
    }
    CHECK((int)seen.size() == total);
    for (int qt = 0; qt < nqt; ++qt) {
      int lo, hi;
      attn_key_span(c.Nq, c.n_kv, c.q_offset, c.window, c.swa, c.bq, c.bk, qt, lo, hi);
      CHECK(0 <= lo && lo <= hi && hi <= (c.n_kv - 1) / c.bk);
      for (int i = qt * c.bq; i < std::min((qt + 1) * c.bq, c.Nq); ++i) {
        const int pos = c.q_offset + i;
        const int k_lo = c.swa ? std::max(0, pos - c.window + 1) : 0, k_hi = std::min(pos, c.n_kv - 1);
        CHECK(k_lo >= lo * c.bk && k_hi < (hi + 1) * c.bk);
      }
      for (int t = lo; t <= hi; ++t) {
        const int bytes = tile_valid_bytes(c.n_kv, t, c.bk, 256);
        CHECK(bytes >= 0 && bytes <= c.bk * 256 && t * c.bk + bytes / 256 <= c.n_kv);
      }
    }
  }
}

static void check_projection_maps() {
  for (int nft = 1; nft <= 34; ++nft)
    for (int ntt = 1; ntt <= 70; ntt += (ntt < 20 ? 1 : 7)) {
      std::set<std::pair<int, int>> seen;
      const int n = proj_workgroups(nft, ntt);
      for (int id = 0; id < n; ++id) {
        int ft, tt;
        if (!proj_tile(id, nft, ntt, ft, tt)) continue;
        CHECK(ft >= 0 && ft < nft && tt >= 0 && tt < ntt);
        CHECK(seen.insert({ft, tt}).second);
      }
      CHECK((int)seen.size() == nft * ntt);
    }
}

static void check_decode_maps() {
  struct Case { int B, Hq, Hkv, ctx; };
  const Case cases[] = {{16, 32, 8, 32768}, {8, 32, 8, 1 << 19}, {1, 24, 8, 1 << 20}, {2, 8, 2, 100},
                        {3, 6, 2, 1}, {1, 32, 8, 1000}, {32, 32, 8, 16384}, {5, 12, 4, 77777}};
  for (const Case& c : cases)
    for (int target : {256 * 12, kDecodeMaxWorkgroups}) {
      int n_splits, chunk, n_hg;
      decode_plan(c.B, c.Hq, c.Hkv, c.ctx, target, &n_splits, &chunk, &n_hg);
      for (int ctx_b : {c.ctx, (c.ctx + 1) / 2, 1}) {
        int covered = 0;
        for (int s = 0; s < n_splits; ++s) {
          const int kb = decode_key_begin(s, chunk);
          if (kb >= ctx_b) continue;
          const int ke = decode_key_end(s, chunk, ctx_b);
          CHECK(kb == covered && ke > kb && ke <= ctx_b);
          covered = ke;
          for (int key0 = kb; key0 < ke; key0 += 16) {
            const int rows = decode_block_rows(ke, key0);
            CHECK(rows >= 1 && rows <= 16 && key0 + rows <= ke);
          }
        }
        CHECK(covered == ctx_b);
      }
    }
  // lane offsets inside a 16-key block (d in {64, 128}; 1, 2 and 4-byte elements)
  for (int d : {64, 128})
    for (int esz : {1, 2, 4}) {
      const int RB = d * esz, NC = d / 32, DPL = d / 64, NL = d / 64;
      for (int l = 0; l < 64; ++l) {
        for (int c = 0; c < NC; ++c) {
          const int o = decode_k_offset(l, RB, esz) + 32 * c * esz;
          CHECK(o >= 0 && o + 8 * esz <= 16 * RB);
        }
        for (int j = 0; j < 16; ++j) {
          const int o = decode_v_offset(l, DPL, esz) + j * RB;
          CHECK(o >= 0 && o + DPL * esz <= 16 * RB);
        }
        if (esz == 2)
          for (int L = 0; L < NL; ++L)
            for (int h = 0; h < 2; ++h) {
              const int o = decode_kf_offset(l, RB, esz) + 8 * h * RB + 64 * L * esz;
              CHECK(o >= 0 && o + 16 <= 16 * RB);
            }
      }
    }
}

int main() {
  check_swizzles<8>();
  check_swizzles<16>();
  check_swizzles<32>();
  // attention tiles: bf16 d = 128 / 64 with 64- and 32-key tiles, float32 d = 64 / 128
  check_tile<16, 64, 256>(true);
  check_tile<16, 32, 256>(true);
  check_tile<8, 64, 256>(true);
  check_tile<8, 32, 256>(true);
  check_tile<16, 32, 256>(false);
  check_tile<32, 32, 256>(false);
  check_attention_maps();
  check_projection_maps();
  check_decode_maps();
  std::printf("all index checks passed\n");
  return 0;
}
