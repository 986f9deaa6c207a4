// Test-only library (not part of libyoco): runs the decode kernels of
// decode.hip over an explicit split plan with either K-load form -- the
// operand-layout loads or the whole-line loads with the row rotate -- so that
// a test can check that the two forms give bitwise equal outputs over the
// same plan.  libyoco itself picks the form from the plan and has no switch.
#include "../../shared_kv_attention_amd/csrc/launch.hpp"

extern "C" int yoco_test_decode_form(const void* q, const void* k, const void* v, const int32_t* ctx_lens, int ctx,
                                     void* o, float* lse, float* ws, int B, int Hq, int Hkv, int n_cap, int n_splits,
                                     int chunk, int full_lines, float scale_log2, void* stream) {
  yoco::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.ctx_lens = ctx_lens;
  a.ctx = ctx;
  const size_t rows = (size_t)B * Hq * n_splits;
  a.part_o = ws;
  a.part_m = ws + rows * 128;
  a.part_l = ws + rows * 129;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_cap = n_cap;
  a.n_splits = n_splits;
  a.chunk = chunk;
  a.n_hg = (Hq / Hkv + 3) / 4;
  a.scale_log2 = scale_log2;
  a.full_lines = full_lines;
  // bf16 queries and cache, head dim 128: the only case with two forms
  return yoco::launch_decode(a, 1, 1, 128, static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 7;
}
