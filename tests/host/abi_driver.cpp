// Drives every entry point of the C ABI on the host with stub launchers:
// valid argument sets must reach the launcher with the expected argument
// block, invalid ones must return their status without launching, and the
// decode workspace layout must fit in exactly the bytes the query returns.
#include <array>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../include/yoco.h"
#include "../../shared_kv_attention_amd/csrc/launch.hpp"

namespace yoco {
extern int g_launches;
extern AttnArgs g_attn;
extern DecodeArgs g_decode;
extern ProjArgs g_proj;
extern QuantArgs g_quant;
extern GretArgs g_gret;
extern LinArgs g_lin;
extern MergeArgs g_merge;
extern int g_lin_mode;
extern int g_decode_kinds[3];
extern uint32_t* g_clear_ptr;
extern int g_clear_n;
extern QuantArgs g_encode[2];
extern int g_encodes;
extern int g_amax_passes;
}  // namespace yoco

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);    \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

alignas(256) static unsigned char arena[1 << 16];

int main() {
  void* P = arena;
  void* M = arena + 4;   // misaligned
  int n;

  // ---- global KV projection
  n = yoco::g_launches;
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 100, 128, 2, 64, 132, 3, 1e-6f, 0.f, YOCO_BF16, YOCO_BF16, nullptr, 0, nullptr) == YOCO_OK);
  CHECK(yoco::g_launches == n + 1);
  CHECK(yoco::g_proj.B == 2 && yoco::g_proj.N == 100 && yoco::g_proj.pos0 == 3 && yoco::g_proj.n_cap == 132);
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 10, 128, 2, 64, 12, 3, 1e-6f, 0.f, YOCO_BF16, YOCO_BF16, nullptr, 0, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco_global_kv_proj(P, M, P, P, P, P, nullptr, nullptr, 2, 10, 128, 2, 64, 32, 3, 1e-6f, 0.f, YOCO_F32, YOCO_F32, nullptr, 0, nullptr) == YOCO_ERR_ALIGN);
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 10, 100, 2, 64, 32, 3, 1e-6f, 0.f, YOCO_F32, YOCO_F32, nullptr, 0, nullptr) == YOCO_ERR_UNSUPPORTED);
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 10, 128, 2, 64, 32, 3, NAN, 0.f, YOCO_F32, YOCO_F32, nullptr, 0, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco::g_launches == n + 1);
  // bf16 with 16384 tokens or more goes to the block-layer GEMM's Q/K/V form with no query heads
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 9000, 128, 2, 64, 9100, 7, 1e-6f, 0.f, YOCO_BF16, YOCO_BF16, nullptr, 0, nullptr) == YOCO_OK);
  CHECK(yoco::g_lin_mode == yoco::kLinQKV && yoco::g_lin.F == 256 && yoco::g_lin.f1 == 0 && yoco::g_lin.f2 == 128);
  CHECK(yoco::g_lin.h1 == 2 && yoco::g_lin.kv_rows == 9100 && yoco::g_lin.kv_pos0 == 7 && yoco::g_lin.norm == 1);
  CHECK(yoco::g_lin.w0 == nullptr && yoco::g_lin.y0 == nullptr && yoco::g_launches == n + 2);
  CHECK(yoco::g_lin.rope_log2_theta == 0.0);
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 2, 9000, 128, 2, 64, 9100, 7, 1e-6f, 1024.f, YOCO_BF16, YOCO_BF16, nullptr, 0, nullptr) ==
        YOCO_OK);
  CHECK(yoco::g_lin.rope_log2_theta == 10.0 && yoco::g_lin.rope_pos0 == 7);
  n = yoco::g_launches;
  // and so does a one-token append (the form for a few tokens)
  CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, nullptr, 16, 1, 128, 2, 64, 40, 39, 1e-6f, 0.f, YOCO_BF16, YOCO_BF16, nullptr, 0, nullptr) == YOCO_OK);
  CHECK(yoco::g_lin_mode == yoco::kLinQKV && yoco::g_lin.kv_pos0 == 39 && yoco::g_lin.B == 16 && yoco::g_launches == n + 1);

  // ---- global KV projection into an 8-bit cache
  {
    float* ks = reinterpret_cast<float*>(arena + 1024);
    float* vs = reinterpret_cast<float*>(arena + 1056);
    const int B = 2, N = 40, Hkv = 2, d = 64, n_cap = 64;   // B * N > 64: the 128 x 128 kernel
    const size_t need = yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, YOCO_BF16, YOCO_FP8_E4M3);
    CHECK(need == 16 + 2 * (size_t)B * Hkv * N * d * 2);
    CHECK(yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, YOCO_F32, YOCO_FP8_E4M3) == 16 + 2 * (size_t)B * Hkv * N * d * 4);
    CHECK(yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, YOCO_BF16, YOCO_BF16) == 0);
    CHECK(yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, YOCO_FP8_E4M3, YOCO_FP8_E4M3) == 0);
    CHECK(yoco_global_kv_proj_workspace_bytes(B, N, Hkv, 96, YOCO_BF16, YOCO_FP8_E4M3) == 0);
    unsigned char* big = static_cast<unsigned char*>(std::aligned_alloc(256, 1 << 20));
    unsigned char* ws = big;
    n = yoco::g_launches;
    yoco::g_encodes = 0;
    // scales from these rows: clear, projection into the staging (the 128 x 128
    // kernel collects the maxima), two encodes
    yoco::g_amax_passes = 0;
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws, need, nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 4 && yoco::g_encodes == 2 && yoco::g_amax_passes == 0);
    CHECK(yoco::g_clear_ptr == reinterpret_cast<uint32_t*>(ws) && yoco::g_clear_n == 2 * Hkv);
    CHECK(yoco::g_proj.amax_bits == reinterpret_cast<uint32_t*>(ws));
    CHECK(yoco::g_proj.n_cap == N && yoco::g_proj.pos0 == 0 && yoco::g_proj.row0 == 0);
    CHECK(yoco::g_proj.k_out == ws + 16 && yoco::g_proj.v_out == ws + 16 + (size_t)B * Hkv * N * d * 2);
    CHECK(static_cast<const unsigned char*>(yoco::g_proj.v_out) + (size_t)B * Hkv * N * d * 2 == ws + need);
    CHECK(yoco::g_encode[0].kv == yoco::g_proj.k_out && yoco::g_encode[0].codes == P && yoco::g_encode[0].scale == ks);
    CHECK(yoco::g_encode[1].kv == yoco::g_proj.v_out && yoco::g_encode[1].scale == vs);
    CHECK(yoco::g_encode[0].amax_bits == reinterpret_cast<uint32_t*>(ws));
    CHECK(yoco::g_encode[1].amax_bits == reinterpret_cast<uint32_t*>(ws) + Hkv);
    CHECK(yoco::g_encode[0].slab == (long long)N * d && yoco::g_encode[0].dst_slab == (long long)n_cap * d &&
          yoco::g_encode[0].dst_off == 0 && yoco::g_encode[0].scale_given == 0);
    // a few tokens (the block-layer GEMM's form): a separate pass collects the maxima
    n = yoco::g_launches;
    const size_t need1 = yoco_global_kv_proj_workspace_bytes(B, 1, Hkv, d, YOCO_BF16, YOCO_FP8_E4M3);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, 1, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws, need1, nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 6 && yoco::g_amax_passes == 2 && yoco::g_lin.kv_rows == 1 && yoco::g_lin.kv_pos0 == 0);
    // appended rows: staged, then encoded with the given scales at row pos0
    n = yoco::g_launches;
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, 1, 128, Hkv, d, n_cap, 30, 1e-6f, 1e4f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws, need1, nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 3 && yoco::g_amax_passes == 2);
    CHECK(yoco::g_lin.kv_rows == 1 && yoco::g_lin.kv_pos0 == 0 && yoco::g_lin.rope_pos0 == 30);
    CHECK(yoco::g_encode[0].scale_given == 1 && yoco::g_encode[0].dst_off == 30LL * d && yoco::g_encode[0].scale == ks);
    CHECK(yoco::g_encode[1].scale_given == 1 && yoco::g_encode[1].scale == vs);
    n = yoco::g_launches;
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 16, 1e-6f, 0.f, YOCO_F32,
                              YOCO_FP8_E4M3, ws, 1 << 20, nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 3 && yoco::g_proj.pos0 == 16 && yoco::g_proj.row0 == 0 &&
          yoco::g_proj.amax_bits == nullptr && yoco::g_proj.n_cap == N);
    // errors, none of which launches
    n = yoco::g_launches;
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, nullptr, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws, need, nullptr) == YOCO_ERR_NULL);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws, need - 1, nullptr) == YOCO_ERR_WORKSPACE);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, nullptr, 0, nullptr) == YOCO_ERR_WORKSPACE);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_FP8_E4M3, ws + 4, need, nullptr) == YOCO_ERR_ALIGN);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_FP8_E4M3,
                              YOCO_FP8_E4M3, ws, need, nullptr) == YOCO_ERR_DTYPE);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, ks, vs, B, N, 128, Hkv, d, n_cap, 0, 1e-6f, 0.f, YOCO_BF16,
                              YOCO_F32, ws, need, nullptr) == YOCO_ERR_DTYPE);
    CHECK(yoco_global_kv_proj(P, nullptr, P, P, P, P, reinterpret_cast<float*>(arena + 1025), vs, B, N, 128, Hkv, d,
                              n_cap, 0, 1e-6f, 0.f, YOCO_BF16, YOCO_FP8_E4M3, ws, need, nullptr) == YOCO_ERR_ALIGN);
    CHECK(yoco::g_launches == n);
    std::free(big);
  }

  // ---- sliding window and cross prefill
  n = yoco::g_launches;
  CHECK(yoco_swa_attn(P, P, P, P, nullptr, 1, 8, 2, 300, 128, 64, 0.f, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(std::fabs(yoco::g_attn.scale_log2 - 1.4426950408889634f / std::sqrt(128.f)) < 1e-6f);
  CHECK(yoco::g_attn.window == 64 && yoco::g_attn.n_kv == 300 && yoco::g_attn.kv_rows == 300);
  CHECK(yoco_cross_attn_prefill(P, P, P, P, (float*)P, 2, 6, 3, 17, 40, 64, 23, 64, 0.5f, YOCO_F32, nullptr) == YOCO_OK);
  CHECK(yoco::g_attn.window == 0 && yoco::g_attn.q_offset == 23 && yoco::g_attn.kv_rows == 64);
  CHECK(std::fabs(yoco::g_attn.scale_log2 - 0.5f * 1.4426950408889634f) < 1e-6f);
  CHECK(yoco_cross_attn_prefill(P, P, P, P, nullptr, 2, 6, 3, 18, 40, 64, 23, 64, 0.f, YOCO_F32, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco_swa_attn(P, P, P, P, (float*)(arena + 2), 1, 8, 2, 300, 128, 64, 0.f, YOCO_BF16, nullptr) == YOCO_ERR_ALIGN);
  CHECK(yoco::g_launches == n + 2);

  // ---- decode: the workspace layout fits in exactly the queried size
  const int shapes[][5] = {{16, 32, 8, 32768, 128}, {1, 32, 8, 1 << 20, 128}, {3, 8, 2, 1000, 64}, {2, 12, 2, 300, 128},
                           {1, 4, 4, 1, 64}, {8, 32, 8, 1 << 19, 128}, {1, 1, 1, 2000000000, 64}};
  for (const auto& s : shapes) {
    const int B = s[0], Hq = s[1], Hkv = s[2], ctx = s[3], d = s[4];
    const size_t need = yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d);
    CHECK(need > 0 && need % 16 == 0);
    unsigned char* ws = (unsigned char*)std::malloc(need);
    n = yoco::g_launches;
    const yoco_status st = yoco_cross_attn_decode(P, P, P, nullptr, nullptr, nullptr, ctx, P, nullptr, B, Hq, Hkv, ctx, d,
                                                  0.f, YOCO_BF16, YOCO_BF16, ws, need, nullptr);
    if ((long long)B * Hkv * ctx > 2147483647LL) {
      CHECK(st == YOCO_ERR_SHAPE);
    } else {
      CHECK(st == YOCO_OK && yoco::g_launches == n + 1);
      const yoco::DecodeArgs& a = yoco::g_decode;
      CHECK(a.n_splits >= 1 && a.n_splits <= yoco::kDecodeMaxSplits);
      CHECK((long long)a.n_splits * a.chunk >= ctx && (long long)(a.n_splits - 1) * a.chunk < ctx);
      CHECK(a.chunk % 64 == 0);
      const size_t rows = (size_t)B * Hq * a.n_splits;
      CHECK((unsigned char*)a.part_o == ws);
      CHECK((unsigned char*)(a.part_o + rows * d) <= (unsigned char*)a.part_m);
      CHECK((unsigned char*)(a.part_m + rows) <= (unsigned char*)a.part_l);
      CHECK((unsigned char*)(a.part_l + rows) <= ws + need);
      CHECK(yoco_cross_attn_decode(P, P, P, nullptr, nullptr, nullptr, ctx, P, nullptr, B, Hq, Hkv, ctx, d, 0.f, YOCO_BF16,
                                   YOCO_BF16, ws, need - 1, nullptr) == YOCO_ERR_WORKSPACE);
      // every kernel form plans within the same (dtype-independent) workspace;
      // the bf16 form's smaller workgroup target never gives more splits
      const int bf16_splits = a.n_splits;
      const yoco_dtype forms[][2] = {{YOCO_F32, YOCO_F32}, {YOCO_BF16, YOCO_FP8_E4M3}};
      for (const auto& f : forms) {
        CHECK(yoco_cross_attn_decode(P, P, P, (float*)P, (float*)P, nullptr, ctx, P, nullptr, B, Hq, Hkv, ctx, d, 0.f,
                                     f[0], f[1], ws, need, nullptr) == YOCO_OK);
        const yoco::DecodeArgs& b = yoco::g_decode;
        CHECK(b.n_splits >= bf16_splits && b.n_splits <= yoco::kDecodeMaxSplits);
        CHECK((long long)b.n_splits * b.chunk >= ctx && b.chunk % 64 == 0);
        CHECK((unsigned char*)(b.part_l + (size_t)B * Hq * b.n_splits) <= ws + need);
      }
    }
    std::free(ws);
  }
  {
    // long bf16 d = 128 splits take the whole-line K form (12-wave-per-CU
    // plan); short splits, fp8 and float32 caches do not.  Long fp8 d = 128
    // splits get the 12-wave-per-CU plan too.
    struct Case { int B, Hq, Hkv, ctx, d; yoco_dtype kv; int full, twelve; };
    const Case cases[] = {{16, 32, 8, 32768, 128, YOCO_BF16, 1, 1}, {1, 24, 8, 1 << 20, 128, YOCO_BF16, 1, 1},
                          {32, 32, 8, 16384, 128, YOCO_BF16, 1, 1}, {1, 24, 8, 131072, 128, YOCO_BF16, 0, 0},
                          {16, 32, 8, 32768, 64, YOCO_BF16, 0, 0}, {16, 32, 8, 32768, 128, YOCO_FP8_E4M3, 0, 1},
                          {8, 32, 8, 1 << 19, 128, YOCO_FP8_E4M3, 0, 1}, {1, 24, 8, 131072, 128, YOCO_FP8_E4M3, 0, 0},
                          {16, 32, 8, 32768, 128, YOCO_F32, 0, 0}};
    for (const Case& c : cases) {
      const size_t need = yoco_cross_attn_decode_workspace_bytes(c.B, c.Hq, c.Hkv, c.ctx, c.d);
      unsigned char* ws = (unsigned char*)std::malloc(need);
      const yoco_dtype qd = c.kv == YOCO_F32 ? YOCO_F32 : YOCO_BF16;
      CHECK(yoco_cross_attn_decode(P, P, P, (float*)P, (float*)P, nullptr, c.ctx, P, nullptr, c.B, c.Hq, c.Hkv, c.ctx,
                                   c.d, 0.f, qd, c.kv, ws, need, nullptr) == YOCO_OK);
      const yoco::DecodeArgs& a = yoco::g_decode;
      CHECK(a.full_lines == c.full);
      const long long wgs = (long long)a.n_splits * c.B * c.Hkv * a.n_hg;
      if (c.twelve) CHECK(a.chunk >= yoco::kDecodeFullLineMinChunk && wgs <= 256 * 12 && wgs > 256 * 8);
      else CHECK(wgs > 256 * 12 || a.chunk < yoco::kDecodeFullLineMinChunk || c.d != 128);
      CHECK((unsigned char*)(a.part_l + (size_t)c.B * c.Hq * a.n_splits) <= ws + need);
      std::free(ws);
    }
  }
  {
    const size_t need = yoco_cross_attn_decode_workspace_bytes(2, 8, 2, 100, 128);
    n = yoco::g_launches;
    CHECK(yoco_cross_attn_decode(P, P, P, (float*)P, (float*)P, (const int32_t*)P, 100, P, nullptr, 2, 8, 2, 128, 128, 0.f,
                                 YOCO_BF16, YOCO_FP8_E4M3, arena, need, nullptr) == YOCO_OK);
    CHECK(yoco::g_decode_kinds[0] == 1 && yoco::g_decode_kinds[1] == 2 && yoco::g_decode_kinds[2] == 128);
    CHECK(yoco_cross_attn_decode(P, P, P, nullptr, (float*)P, nullptr, 100, P, nullptr, 2, 8, 2, 128, 128, 0.f, YOCO_BF16,
                                 YOCO_FP8_E4M3, arena, need, nullptr) == YOCO_ERR_NULL);
    CHECK(yoco_cross_attn_decode(P, P, P, nullptr, nullptr, nullptr, 129, P, nullptr, 2, 8, 2, 128, 128, 0.f, YOCO_BF16,
                                 YOCO_BF16, arena, need, nullptr) == YOCO_ERR_SHAPE);
    CHECK(yoco::g_launches == n + 1);
  }

  // ---- self-decoder ring decode: one launch (the append folded into the decode), workspace bound over all positions
  {
    const int B = 3, Hq = 8, Hkv = 2, W = 1024, d = 128;
    const size_t need = yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d);
    CHECK(need > 0 && need % 16 == 0);
    unsigned char* ws = (unsigned char*)std::malloc(need);
    for (int pos : {0, 1, 255, 256, 1022, 1023, 1024, 5000, 1 << 20}) {
      n = yoco::g_launches;
      CHECK(yoco_swa_decode(P, P, P, P, P, pos, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_BF16, ws, need, nullptr) == YOCO_OK);
      CHECK(yoco::g_launches == n + 1);
      const yoco::DecodeArgs& a = yoco::g_decode;
      CHECK(a.k_new == P && a.v_new == P && a.new_slot == pos % W && a.new_slot < a.ctx);
      CHECK(a.ctx == (pos + 1 < W ? pos + 1 : W) && a.n_cap == W && a.ctx_lens == nullptr);
      const size_t rows = (size_t)B * Hq * a.n_splits;
      CHECK((unsigned char*)(a.part_l + rows) <= ws + need);
      CHECK((long long)a.n_splits * a.chunk >= a.ctx);
    }
    n = yoco::g_launches;
    CHECK(yoco_swa_decode(P, nullptr, nullptr, P, P, 7, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_F32, ws, need, nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 1 && yoco::g_decode.k_new == nullptr);   // no append without new K/V
    CHECK(yoco_swa_decode(P, P, nullptr, P, P, 7, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_F32, ws, need, nullptr) == YOCO_ERR_NULL);
    CHECK(yoco_swa_decode(P, P, P, P, P, -1, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_F32, ws, need, nullptr) == YOCO_ERR_SHAPE);
    CHECK(yoco_swa_decode(P, P, P, P, P, 7, P, nullptr, B, Hq, Hkv, 0, d, 0.f, YOCO_F32, ws, need, nullptr) == YOCO_ERR_SHAPE);
    CHECK(yoco_swa_decode(P, P, P, P, P, 7, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_FP8_E4M3, ws, need, nullptr) == YOCO_ERR_DTYPE);
    CHECK(yoco_swa_decode(P, P, P, P, P, 7000, P, nullptr, B, Hq, Hkv, W, d, 0.f, YOCO_F32, ws, 16, nullptr) == YOCO_ERR_WORKSPACE);
    CHECK(yoco::g_launches == n + 1);
    std::free(ws);
  }

  // ---- gated retention: the prefill workspace holds every region it is split into
  for (const auto& s : {std::array<int, 5>{1, 24, 4096, 128, 256}, std::array<int, 5>{3, 2, 77, 64, 128},
                        std::array<int, 5>{2, 4, 1, 128, 256}, std::array<int, 5>{1, 1, 300, 64, 256}}) {
    const int B = s[0], H = s[1], N = s[2], d = s[3], chunk = s[4];
    const size_t need = yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk);
    CHECK(need > 0 && need % 16 == 0);
    unsigned char* ws = (unsigned char*)std::malloc(need);
    n = yoco::g_launches;
    CHECK(yoco_gret_prefill(P, P, P, (const float*)P, 4.f, nullptr, P, nullptr, B, H, N, d, chunk, YOCO_BF16, ws, need,
                            nullptr) == YOCO_OK);
    CHECK(yoco::g_launches == n + 1);
    const yoco::GretArgs& a = yoco::g_gret;
    const size_t bh = (size_t)B * H, nc = (size_t)(N + chunk - 1) / chunk;
    CHECK(a.nc == (int)nc && a.inv_tau == 0.25f);
    CHECK((unsigned char*)a.lg2 == ws);
    CHECK((unsigned char*)(a.lg2 + bh * N) <= (unsigned char*)a.lam);
    CHECK((unsigned char*)(a.lam + bh * nc) <= (unsigned char*)a.dR);
    CHECK((unsigned char*)(a.dR + bh * nc * d * d) <= (unsigned char*)a.rin);
    CHECK((unsigned char*)a.rin + bh * nc * d * d * 2 <= ws + need);
    CHECK(yoco_gret_prefill(P, P, P, (const float*)P, 4.f, nullptr, P, nullptr, B, H, N, d, chunk, YOCO_BF16, ws,
                            need - 1, nullptr) == YOCO_ERR_WORKSPACE);
    std::free(ws);
  }
  CHECK(yoco_gret_prefill_workspace_bytes(1, 1, 10, 96, 256) == 0);
  CHECK(yoco_gret_prefill_workspace_bytes(1, 1, 10, 64, 192) == 0);

  // ---- block layer glue: the argument block each form reaches its kernel with
  n = yoco::g_launches;
  CHECK(yoco_qkv_proj(P, nullptr, P, P, P, P, P, P, 2, 9, 256, 4, 1, 64, 1e-6f, 0.f, 0, YOCO_F32, nullptr) == YOCO_OK);
  CHECK(yoco::g_lin_mode == yoco::kLinQKV && yoco::g_lin.F == 384 && yoco::g_lin.f1 == 256 && yoco::g_lin.f2 == 320);
  CHECK(yoco::g_lin.h0 == 4 && yoco::g_lin.h1 == 1 && yoco::g_lin.norm == 1 && yoco::g_lin.K == 256);
  CHECK(yoco_qkv_proj(P, nullptr, P, nullptr, nullptr, P, nullptr, nullptr, 1, 5, 128, 3, 0, 128, 1e-6f, 0.f, 0, YOCO_BF16,
                      nullptr) == YOCO_OK);
  CHECK(yoco::g_lin.F == 384 && yoco::g_lin.f1 == 384 && yoco::g_lin.f2 == 384 && yoco::g_lin.w1 == nullptr);
  CHECK(yoco_qkv_proj(P, nullptr, P, nullptr, P, P, P, P, 1, 5, 128, 3, 1, 128, 1e-6f, 0.f, 0, YOCO_BF16, nullptr) ==
        YOCO_ERR_NULL);
  CHECK(yoco_swiglu(P, nullptr, P, P, P, 1, 7, 192, 344, 1e-6f, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(yoco::g_lin_mode == yoco::kLinSwiGLU && yoco::g_lin.F == 344 && yoco::g_lin.K == 192 && yoco::g_lin.norm == 1);
  CHECK(yoco_linear_residual(P, 4, P, P, 2, 3, 512, 256, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(yoco::g_lin_mode == yoco::kLinResidual && yoco::g_lin.x_heads == 4 && yoco::g_lin.norm == 0);
  CHECK(yoco_linear_residual(P, 3, P, P, 2, 3, 512, 256, YOCO_BF16, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco_linear_residual(P, 0, P, M, 2, 3, 512, 256, YOCO_BF16, nullptr) == YOCO_ERR_ALIGN);
  CHECK(yoco::g_launches == n + 4);

  // ---- one shard of a split sequence: window attention with a halo, merge of decode shards
  n = yoco::g_launches;
  CHECK(yoco_swa_attn_halo(P, P, P, P, nullptr, 1, 8, 2, 300, 1323, 128, 1024, 0.f, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(yoco::g_attn.q_offset == 1023 && yoco::g_attn.n_kv == 1323 && yoco::g_attn.kv_rows == 1323 &&
        yoco::g_attn.Nq == 300 && yoco::g_attn.window == 1024);
  CHECK(yoco_swa_attn_halo(P, P, P, P, nullptr, 1, 8, 2, 301, 300, 128, 1024, 0.f, YOCO_BF16, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco_attn_merge(P, (const float*)P, P, (float*)P, 8, 512, 128, YOCO_BF16, nullptr) == YOCO_OK);
  CHECK(yoco::g_merge.S == 8 && yoco::g_merge.rows == 512 && yoco::g_merge.d == 128);
  CHECK(yoco_attn_merge(P, (const float*)P, P, nullptr, 0, 512, 128, YOCO_BF16, nullptr) == YOCO_ERR_SHAPE);
  CHECK(yoco_attn_merge(M, (const float*)P, P, nullptr, 2, 512, 128, YOCO_BF16, nullptr) == YOCO_ERR_ALIGN);
  CHECK(yoco::g_launches == n + 2);

  // ---- fp8 quantiser
  n = yoco::g_launches;
  CHECK(yoco_kv_quantize_fp8(P, YOCO_F32, P, (float*)P, 2, 3, 17, 64, arena, yoco_kv_quantize_fp8_workspace_bytes(3), nullptr) ==
        YOCO_OK);
  CHECK(yoco::g_quant.slab == 17LL * 64 && yoco::g_quant.Hkv == 3);
  CHECK(yoco_kv_quantize_fp8(P, YOCO_F32, P, (float*)P, 2, 3, 17, 64, arena, 8, nullptr) == YOCO_ERR_WORKSPACE);
  CHECK(yoco::g_launches == n + 1);

  // ---- strings
  for (int s = -1; s < 10; ++s) CHECK(yoco_status_string((yoco_status)s) != nullptr);
  CHECK(yoco_version() == 100);

  if (failures) return 1;
  std::printf("abi host driver: all checks passed\n");
  return 0;
}
