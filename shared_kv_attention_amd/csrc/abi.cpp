// C ABI of libyoco: argument validation, workspace layout and dispatch to the
// gfx950 kernels.  Validation runs before any HIP call, so every argument
// error is reported synchronously and leaves the outputs untouched.
// Check order for every call: null pointers, dtypes, sizes, unsupported
// sizes, alignment, workspace.
#include "../../include/yoco.h"

#include <math.h>

#include "launch.hpp"
#include "index_map.hpp"

namespace {

constexpr int kVersion = 100;   // 0.1.0
constexpr long long kIntMax = 2147483647LL;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_act(yoco_dtype t) { return t == YOCO_F32 || t == YOCO_BF16; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
size_t align16(size_t n) { return (n + 15) / 16 * 16; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

float resolve_scale(float s, int d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

yoco_status launched(hipError_t e) { return e == hipSuccess ? YOCO_OK : YOCO_ERR_HIP; }

// log2 of a rotary base (0 = no rotation).  A base of exactly 1 would turn
// nothing either, but is kept distinct from "off" by a tiny non-zero value.
double rope_log2(float theta) {
  if (!(theta > 0.f)) return 0.0;
  const double l = log2((double)theta);
  return l != 0.0 ? l : 1e-300;
}

struct DecodeLayout {
  int n_splits, chunk, n_hg, full_lines;
  size_t o_bytes, ml_bytes, total;
};

// The workspace holds the partials of the plan for kDecodeMaxWorkgroups
// (what the size queries return, whatever the dtype).  A bf16 d = 128 cache
// whose splits are long enough is read by the whole-line K form, and an fp8
// d = 128 cache with splits that long by the 8-bit form; both are planned for
// their own workgroup target (never more splits).
DecodeLayout decode_layout(int B, int Hq, int Hkv, int ctx, int d, int kv_kind = 1) {
  DecodeLayout L{};
  yoco::decode_plan(B, Hq, Hkv, ctx, yoco::kDecodeMaxWorkgroups, &L.n_splits, &L.chunk, &L.n_hg);
  const int cap_splits = L.n_splits;
  const bool long_splits = d == 128 && L.chunk >= yoco::kDecodeFullLineMinChunk;
  L.full_lines = kv_kind == 1 && long_splits;
  if (long_splits && (kv_kind == 1 || kv_kind == 2))
    yoco::decode_plan(B, Hq, Hkv, ctx, yoco::decode_workgroup_target(kv_kind, d), &L.n_splits, &L.chunk, &L.n_hg);
  const size_t rows = (size_t)B * Hq * cap_splits;
  L.o_bytes = align16(rows * d * sizeof(float));
  L.ml_bytes = align16(rows * sizeof(float));
  L.total = L.o_bytes + 2 * L.ml_bytes;
  return L;
}

// Workspace of an 8-bit global projection that sets the scales: the
// per-head maxima of K and V (2 Hkv words), then K and V staged in the
// activation dtype as [B, Hkv, N, d].
struct ProjFp8Layout {
  size_t amax, k_stage, v_stage, total;
};
ProjFp8Layout proj_fp8_layout(int B, int N, int Hkv, int d, yoco_dtype act) {
  ProjFp8Layout L{};
  const size_t stage = align16((size_t)B * Hkv * N * d * (act == YOCO_F32 ? 4 : 2));
  L.amax = 0;
  L.k_stage = align16((size_t)2 * Hkv * sizeof(uint32_t));
  L.v_stage = L.k_stage + stage;
  L.total = L.v_stage + stage;
  return L;
}

// The projection GEMM into a [B, Hkv, n_cap, d] activation-dtype cache,
// token t at position pos0 + t written to row row0 + t.  amax (non-null) asks
// for the per-head maxima of the written values; *fused_amax tells whether
// the chosen kernel form collected them.
hipError_t proj_gemm(const void* x, const void* norm_w, const void* w_k, const void* w_v, void* k_out, void* v_out,
                     int B, int N, int D, int Hkv, int d, int n_cap, int pos0, int row0, float eps,
                     float rope_theta, bool is_bf16, uint32_t* amax, hipStream_t st, bool* fused_amax = nullptr) {
  if (fused_amax) *fused_amax = false;
  // bf16 without a norm gain whose 256-feature tiles cover the 256 CUs: the
  // projection's own three-stage ring form at every length (2^20 tokens:
  // 16.4 ms against 19.3 for the wide form below; 4096 tokens: 55 us)
  const long long M = (long long)B * N;
  const bool ring = yoco::proj_ring_form(M, 2 * Hkv * d, is_bf16, norm_w != nullptr);
  if (is_bf16 && !ring && (M >= 16384 || M <= 64)) {
    // the block-layer GEMM in its Q/K/V form with no query heads: for long
    // prompts with a norm gain its wide bf16 tiles (measured 18.7 vs 22.9 ms
    // at 2^20 tokens against the 128 x 128 kernel), for a few tokens (the
    // one-token append of generation) its form that spreads K over many
    // waves.  In between, the 128 x 128 kernel below, two workgroups per CU,
    // hides latency better (72 vs 80 us at 4096 tokens); it also serves
    // float32.
    yoco::LinArgs la{};
    la.x = x;
    la.norm_w = norm_w;
    la.w1 = w_k;
    la.w2 = w_v;
    la.y1 = k_out;
    la.y2 = v_out;
    la.B = B; la.N = N; la.K = D; la.F = 2 * Hkv * d;
    la.f1 = 0; la.f2 = Hkv * d;
    la.h0 = 0; la.h1 = Hkv; la.d = d;
    la.kv_rows = n_cap; la.kv_pos0 = row0;
    la.norm = 1;
    la.eps = eps;
    la.rope_log2_theta = rope_log2(rope_theta);
    la.rope_pos0 = pos0;
    return yoco::launch_linear(la, yoco::kLinQKV, true, st);
  }
  yoco::ProjArgs a{x, norm_w, w_k, w_v, k_out, v_out, B, N, D, Hkv, d, n_cap, pos0, row0, eps, rope_log2(rope_theta),
                   amax};
  if (fused_amax) *fused_amax = amax != nullptr;
  return yoco::launch_kv_proj(a, is_bf16, st);
}

bool decode_sizes_ok(int B, int Hq, int Hkv, int ctx, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || ctx < 1 || Hq % Hkv != 0) return false;
  if (!head_dim_ok(d)) return false;
  if ((long long)B * Hq > 65535LL * 64 || (long long)B > 65535) return false;
  return true;
}

}  // namespace

extern "C" {

const char* yoco_status_string(yoco_status s) {
  switch (s) {
    case YOCO_OK: return "ok";
    case YOCO_ERR_NULL: return "a required pointer is NULL";
    case YOCO_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case YOCO_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case YOCO_ERR_UNSUPPORTED: return "valid but unsupported size (head_dim must be 64 or 128; D a multiple of 64)";
    case YOCO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case YOCO_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case YOCO_ERR_HIP: return "a HIP launch failed";
  }
  return "unknown status";
}

int yoco_version(void) { return kVersion; }

size_t yoco_global_kv_proj_workspace_bytes(int B, int N, int Hkv, int d, yoco_dtype act_dtype, yoco_dtype kv_dtype) {
  if (B < 1 || N < 1 || Hkv < 1 || !head_dim_ok(d) || !is_act(act_dtype)) return 0;
  if (kv_dtype != YOCO_FP8_E4M3) return 0;   // no workspace (or an invalid dtype)
  if ((long long)B * N > kIntMax || (long long)B * Hkv * N > kIntMax) return 0;
  return proj_fp8_layout(B, N, Hkv, d, act_dtype).total;
}

yoco_status yoco_global_kv_proj(const void* x, const void* norm_w, const void* w_k, const void* w_v,
                                void* k_out, void* v_out, float* k_scale, float* v_scale, int B, int N, int D,
                                int Hkv, int d, int n_cap, int pos0, float eps, float rope_theta,
                                yoco_dtype act_dtype, yoco_dtype kv_dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const bool fp8 = kv_dtype == YOCO_FP8_E4M3;
  if (!x || !w_k || !w_v || !k_out || !v_out) return YOCO_ERR_NULL;
  if (fp8 && (!k_scale || !v_scale)) return YOCO_ERR_NULL;
  if (!is_act(act_dtype) || (kv_dtype != act_dtype && !fp8)) return YOCO_ERR_DTYPE;
  if (B < 1 || N < 1 || D < 1 || Hkv < 1 || n_cap < 1 || pos0 < 0 || (long long)pos0 + N > n_cap)
    return YOCO_ERR_SHAPE;
  if (!(eps >= 0.f) || isinf(eps) || !(rope_theta >= 0.f) || isinf(rope_theta)) return YOCO_ERR_SHAPE;
  if ((long long)B * N > kIntMax || (long long)2 * Hkv * d > kIntMax || (long long)B * Hkv * n_cap > kIntMax)
    return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d) || D % 64 != 0 || D > 65536) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) ||
      (norm_w && !aligned(norm_w, 16)) || (k_scale && fp8 && !aligned(k_scale, 4)) ||
      (v_scale && fp8 && !aligned(v_scale, 4)))
    return YOCO_ERR_ALIGN;
  const bool is_bf16 = act_dtype == YOCO_BF16;
  hipStream_t st = as_stream(stream);
  if (!fp8) return launched(proj_gemm(x, norm_w, w_k, w_v, k_out, v_out, B, N, D, Hkv, d, n_cap, pos0, pos0, eps,
                                      rope_theta, is_bf16, nullptr, st));
  // 8-bit cache: the rows are projected exactly as into an act_dtype cache, but
  // into a staging buffer in the workspace; then each tensor is encoded into
  // the cache rows [pos0, pos0 + N) -- with scales set from the staged rows'
  // per-head maxima (pos0 == 0), or with the given scales (pos0 > 0).
  const ProjFp8Layout L = proj_fp8_layout(B, N, Hkv, d, act_dtype);
  if (!workspace || workspace_bytes < L.total) return YOCO_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return YOCO_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  uint32_t* amax = reinterpret_cast<uint32_t*>(ws + L.amax);
  const bool set_scales = pos0 == 0;
  yoco_status s = YOCO_OK;
  if (set_scales && (s = launched(yoco::launch_quant_clear(amax, 2 * Hkv, st))) != YOCO_OK) return s;
  // the 128 x 128 projection kernel collects the maxima in its epilogue; the
  // block-layer GEMM forms (long prompts, a few tokens) are followed by a pass
  // over the staged rows
  bool fused_amax = false;
  s = launched(proj_gemm(x, norm_w, w_k, w_v, ws + L.k_stage, ws + L.v_stage, B, N, D, Hkv, d, N, pos0, 0, eps,
                         rope_theta, is_bf16, set_scales ? amax : nullptr, st, &fused_amax));
  if (s != YOCO_OK) return s;
  const long long slab = (long long)N * d;
  yoco::QuantArgs qk{ws + L.k_stage, static_cast<uint8_t*>(k_out), k_scale, amax, B, Hkv, slab,
                     (long long)n_cap * d, (long long)pos0 * d, set_scales ? 0 : 1};
  yoco::QuantArgs qv{ws + L.v_stage, static_cast<uint8_t*>(v_out), v_scale, amax + Hkv, B, Hkv, slab,
                     (long long)n_cap * d, (long long)pos0 * d, set_scales ? 0 : 1};
  if (set_scales && !fused_amax) {
    if ((s = launched(yoco::launch_quant_amax(qk, is_bf16, st))) != YOCO_OK) return s;
    if ((s = launched(yoco::launch_quant_amax(qv, is_bf16, st))) != YOCO_OK) return s;
  }
  if ((s = launched(yoco::launch_quant_encode(qk, is_bf16, st))) != YOCO_OK) return s;
  return launched(yoco::launch_quant_encode(qv, is_bf16, st));
}

static bool lin_sizes_ok(int B, int N, int K, int F, int fpt) {
  if (B < 1 || N < 1 || K < 1 || F < 1) return false;
  const long long M = (long long)B * N;
  if (M > kIntMax) return false;
  return ((M + 127) / 128) * (((long long)F + fpt - 1) / fpt) <= kIntMax;
}

yoco_status yoco_qkv_proj(const void* x, const void* norm_w, const void* w_q, const void* w_k, const void* w_v,
                          void* q_out, void* k_out, void* v_out, int B, int N, int D, int Hq, int Hkv, int d,
                          float eps, float rope_theta, int rope_pos0, yoco_dtype dtype, void* stream) {
  if (!x || !w_q || !q_out) return YOCO_ERR_NULL;
  if (Hkv > 0 && (!w_k || !w_v || !k_out || !v_out)) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (Hq < 1 || Hkv < 0 || !(eps >= 0.f) || isinf(eps)) return YOCO_ERR_SHAPE;
  if (!(rope_theta >= 0.f) || isinf(rope_theta) || rope_pos0 < 0 || (long long)rope_pos0 + N > kIntMax)
    return YOCO_ERR_SHAPE;
  if ((long long)(Hq + 2LL * Hkv) * d > kIntMax) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  const int F = (Hq + 2 * Hkv) * d;
  if (!lin_sizes_ok(B, N, D, F, 128)) return YOCO_ERR_SHAPE;
  if (D % 64 != 0 || D > 65536) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(q_out, 16) || (norm_w && !aligned(norm_w, 16)) ||
      (Hkv > 0 && (!aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))))
    return YOCO_ERR_ALIGN;
  yoco::LinArgs a{};
  a.x = x;
  a.norm_w = norm_w;
  a.w0 = w_q;
  a.w1 = Hkv > 0 ? w_k : nullptr;
  a.w2 = Hkv > 0 ? w_v : nullptr;
  a.y0 = q_out;
  a.y1 = Hkv > 0 ? k_out : nullptr;
  a.y2 = Hkv > 0 ? v_out : nullptr;
  a.B = B; a.N = N; a.K = D; a.F = F;
  a.x_heads = 0;
  a.f1 = Hkv > 0 ? Hq * d : F;
  a.f2 = Hkv > 0 ? (Hq + Hkv) * d : F;
  a.h0 = Hq; a.h1 = Hkv; a.d = d;
  a.kv_rows = N; a.kv_pos0 = 0;
  a.norm = 1;
  a.eps = eps;
  a.rope_log2_theta = rope_log2(rope_theta);
  a.rope_pos0 = rope_pos0;
  return launched(yoco::launch_linear(a, yoco::kLinQKV, dtype == YOCO_BF16, as_stream(stream)));
}

yoco_status yoco_swiglu(const void* x, const void* norm_w, const void* w_gate, const void* w_up, void* h, int B,
                        int N, int D, int F, float eps, yoco_dtype dtype, void* stream) {
  if (!x || !w_gate || !w_up || !h) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (!(eps >= 0.f) || isinf(eps)) return YOCO_ERR_SHAPE;
  if (!lin_sizes_ok(B, N, D, F, 64) || F % 4 != 0) return YOCO_ERR_SHAPE;
  if (D % 64 != 0 || D > 65536) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(h, 16) ||
      (norm_w && !aligned(norm_w, 16)))
    return YOCO_ERR_ALIGN;
  yoco::LinArgs a{};
  a.x = x;
  a.norm_w = norm_w;
  a.w0 = w_gate;
  a.w1 = w_up;
  a.y0 = h;
  a.B = B; a.N = N; a.K = D; a.F = F;
  a.norm = 1;
  a.eps = eps;
  return launched(yoco::launch_linear(a, yoco::kLinSwiGLU, dtype == YOCO_BF16, as_stream(stream)));
}

yoco_status yoco_linear_residual(const void* x, int a_heads, const void* w, void* y, int B, int N, int K, int F,
                                 yoco_dtype dtype, void* stream) {
  if (!x || !w || !y) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (a_heads < 0 || !lin_sizes_ok(B, N, K, F, 128) || F % 4 != 0) return YOCO_ERR_SHAPE;
  if (a_heads > 0 && K % a_heads != 0) return YOCO_ERR_SHAPE;
  if (K % 64 != 0 || K > 65536 || (a_heads > 0 && (K / a_heads) % 64 != 0)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return YOCO_ERR_ALIGN;
  yoco::LinArgs a{};
  a.x = x;
  a.w0 = w;
  a.y0 = y;
  a.B = B; a.N = N; a.K = K; a.F = F;
  a.x_heads = a_heads;
  return launched(yoco::launch_linear(a, yoco::kLinResidual, dtype == YOCO_BF16, as_stream(stream)));
}

static yoco_status attn_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int Nq, int n_kv, int kv_rows, int q_offset, int d, int window,
                               bool swa, float softmax_scale, yoco_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || n_kv < 1 || Hq % Hkv != 0) return YOCO_ERR_SHAPE;
  if (q_offset < 0 || (long long)q_offset + Nq > n_kv || n_kv > kv_rows) return YOCO_ERR_SHAPE;
  if (swa && window < 1) return YOCO_ERR_SHAPE;
  if (isnan(softmax_scale) || isinf(softmax_scale)) return YOCO_ERR_SHAPE;
  const long long nqt = (Nq + 127) / 128;
  if (nqt * B * Hq > kIntMax || (long long)kv_rows > kIntMax / 2) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
    return YOCO_ERR_ALIGN;
  const float scale = resolve_scale(softmax_scale, d);
  yoco::AttnArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, n_kv, kv_rows, q_offset, swa ? window : 0,
                   scale * 1.4426950408889634f};
  return launched(yoco::launch_attn(a, dtype == YOCO_BF16, d, swa, as_stream(stream)));
}

yoco_status yoco_swa_attn(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int N, int d, int window, float softmax_scale, yoco_dtype dtype, void* stream) {
  return attn_common(q, k, v, o, lse, B, Hq, Hkv, N, N, N, 0, d, window, true, softmax_scale, dtype, stream);
}

yoco_status yoco_swa_attn_halo(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int Nq, int Nkv, int d, int window, float softmax_scale, yoco_dtype dtype,
                               void* stream) {
  if (Nq > Nkv) return YOCO_ERR_SHAPE;
  return attn_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, Nkv, Nkv - Nq, d, window, true, softmax_scale, dtype,
                     stream);
}

yoco_status yoco_attn_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int S, int rows, int d,
                            yoco_dtype dtype, void* stream) {
  if (!o_parts || !lse_parts || !o) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (S < 1 || rows < 1 || (long long)S * rows > kIntMax) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || (lse && !aligned(lse, 4)))
    return YOCO_ERR_ALIGN;
  yoco::MergeArgs a{o_parts, lse_parts, o, lse, S, rows, d};
  return launched(yoco::launch_attn_merge(a, dtype == YOCO_BF16, as_stream(stream)));
}

yoco_status yoco_peak_hbm_read(const void* buf, size_t bytes, uint32_t* partial, int blocks, void* stream) {
  if (!buf || !partial) return YOCO_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > 65536) return YOCO_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(partial, 4)) return YOCO_ERR_ALIGN;
  return launched(yoco::launch_peak_read(buf, (long long)bytes, partial, blocks, as_stream(stream)));
}

yoco_status yoco_peak_mfma_bf16(int iters, float* out, int blocks, void* stream) {
  if (!out) return YOCO_ERR_NULL;
  if (iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536) return YOCO_ERR_SHAPE;
  if (!aligned(out, 4)) return YOCO_ERR_ALIGN;
  return launched(yoco::launch_peak_mfma(iters, out, blocks, as_stream(stream)));
}

yoco_status yoco_peak_mfma_bf16_toggling(int iters, float* out, int blocks, void* stream) {
  if (!out) return YOCO_ERR_NULL;
  if (iters < 8 || iters % 8 != 0 || iters > (1 << 20) || blocks < 1 || blocks > 65536) return YOCO_ERR_SHAPE;
  if (!aligned(out, 4)) return YOCO_ERR_ALIGN;
  return launched(yoco::launch_peak_mfma_toggle(iters, out, blocks, as_stream(stream)));
}

yoco_status yoco_cross_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                    int Hq, int Hkv, int Nq, int n_kv, int n_cap, int q_offset, int d,
                                    float softmax_scale, yoco_dtype dtype, void* stream) {
  return attn_common(q, k, v, o, lse, B, Hq, Hkv, Nq, n_kv, n_cap, q_offset, d, 0, false, softmax_scale, dtype,
                     stream);
}

size_t yoco_cross_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int ctx, int d) {
  if (!decode_sizes_ok(B, Hq, Hkv, ctx, d)) return 0;
  return decode_layout(B, Hq, Hkv, ctx, d).total;
}

yoco_status yoco_cross_attn_decode(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* ctx_lens, int ctx, void* o, float* lse,
                                   int B, int Hq, int Hkv, int n_cap, int d, float softmax_scale,
                                   yoco_dtype q_dtype, yoco_dtype kv_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const bool fp8 = kv_dtype == YOCO_FP8_E4M3;
  if (!q || !k_cache || !v_cache || !o) return YOCO_ERR_NULL;
  if (fp8 && (!k_scale || !v_scale)) return YOCO_ERR_NULL;
  const bool combo_ok = (q_dtype == YOCO_F32 && kv_dtype == YOCO_F32) ||
                        (q_dtype == YOCO_BF16 && kv_dtype == YOCO_BF16) ||
                        (q_dtype == YOCO_BF16 && kv_dtype == YOCO_FP8_E4M3);
  if (!combo_ok) return YOCO_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || n_cap < 1 || ctx < 1 || ctx > n_cap || Hq % Hkv != 0) return YOCO_ERR_SHAPE;
  if (B > 65535 || (long long)B * Hkv * n_cap > kIntMax || (long long)Hkv * ((Hq / Hkv + 3) / 4) > 65535)
    return YOCO_ERR_SHAPE;
  if (isnan(softmax_scale) || isinf(softmax_scale)) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)) || (ctx_lens && !aligned(ctx_lens, 4)) || (k_scale && !aligned(k_scale, 4)) ||
      (v_scale && !aligned(v_scale, 4)))
    return YOCO_ERR_ALIGN;
  const int kk = kv_dtype == YOCO_F32 ? 0 : (kv_dtype == YOCO_BF16 ? 1 : 2);
  const DecodeLayout L = decode_layout(B, Hq, Hkv, ctx, d, kk);
  if (!workspace || workspace_bytes < L.total) return YOCO_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return YOCO_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  yoco::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.ctx_lens = ctx_lens;
  a.ctx = ctx;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + L.o_bytes);
  a.part_l = reinterpret_cast<float*>(ws + L.o_bytes + L.ml_bytes);
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_cap = n_cap;
  a.n_splits = L.n_splits;
  a.chunk = L.chunk;
  a.n_hg = L.n_hg;
  a.full_lines = L.full_lines;
  a.scale_log2 = resolve_scale(softmax_scale, d) * 1.4426950408889634f;
  const int qk = q_dtype == YOCO_F32 ? 0 : 1;
  return launched(yoco::launch_decode(a, qk, kk, d, as_stream(stream)));
}

size_t yoco_swa_decode_workspace_bytes(int B, int Hq, int Hkv, int W, int d) {
  if (!decode_sizes_ok(B, Hq, Hkv, W, d)) return 0;
  // a call at position pos plans ctx = min(pos + 1, W) <= W, whose split count
  // is at most decode_split_bound(.., W)
  const size_t rows = (size_t)B * Hq * yoco::decode_split_bound(B, Hq, Hkv, W);
  return align16(rows * d * sizeof(float)) + 2 * align16(rows * sizeof(float));
}

yoco_status yoco_swa_decode(const void* q, const void* k_new, const void* v_new, void* k_ring, void* v_ring,
                            int pos, void* o, float* lse, int B, int Hq, int Hkv, int W, int d,
                            float softmax_scale, yoco_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!q || !k_ring || !v_ring || !o) return YOCO_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || W < 1 || pos < 0 || Hq % Hkv != 0) return YOCO_ERR_SHAPE;
  if (B > 65535 || (long long)B * Hkv * W > kIntMax || (long long)Hkv * ((Hq / Hkv + 3) / 4) > 65535)
    return YOCO_ERR_SHAPE;
  if (isnan(softmax_scale) || isinf(softmax_scale)) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_ring, 16) || !aligned(v_ring, 16) || !aligned(o, 16) ||
      (k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)) || (lse && !aligned(lse, 4)))
    return YOCO_ERR_ALIGN;
  const int ctx = pos + 1 < W ? pos + 1 : W;   // slots 0 .. ctx-1 hold the window
  const DecodeLayout L = decode_layout(B, Hq, Hkv, ctx, d, dtype == YOCO_F32 ? 0 : 1);
  if (!workspace || workspace_bytes < L.total) return YOCO_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return YOCO_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  yoco::DecodeArgs a{};
  a.q = q;
  a.k = k_ring;
  a.v = v_ring;
  a.ctx_lens = nullptr;
  a.ctx = ctx;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + L.o_bytes);
  a.part_l = reinterpret_cast<float*>(ws + L.o_bytes + L.ml_bytes);
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_cap = W;
  a.n_splits = L.n_splits;
  a.chunk = L.chunk;
  a.n_hg = L.n_hg;
  a.full_lines = L.full_lines;
  a.scale_log2 = resolve_scale(softmax_scale, d) * 1.4426950408889634f;
  // the token's K/V go into slot pos % W inside the decode launch
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slot = pos % W;
  const int kind = dtype == YOCO_F32 ? 0 : 1;
  return launched(yoco::launch_decode(a, kind, kind, d, as_stream(stream)));
}

}  // extern "C"

namespace {

struct GretLayout {
  size_t lg2, lam, dR, rin, total;
};

bool gret_sizes_ok(int B, int H, int N, int d, int chunk) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || (chunk != 128 && chunk != 256)) return false;
  const long long nc = (N + chunk - 1) / chunk;
  return (long long)B * H <= 65535 && (long long)B * H * N <= kIntMax && nc * (chunk / 128) <= 65535;
}

GretLayout gret_layout(int B, int H, int N, int d, int chunk) {
  GretLayout L{};
  const size_t bh = (size_t)B * H, nc = (size_t)(N + chunk - 1) / chunk;
  L.lg2 = 0;
  L.lam = align16(bh * N * sizeof(float));
  L.dR = L.lam + align16(bh * nc * sizeof(float));
  L.rin = L.dR + align16(bh * nc * d * d * sizeof(float));
  L.total = L.rin + align16(bh * nc * d * d * 2);
  return L;
}

}  // namespace

extern "C" {

size_t yoco_gret_prefill_workspace_bytes(int B, int H, int N, int d, int chunk) {
  if (!gret_sizes_ok(B, H, N, d, chunk)) return 0;
  return gret_layout(B, H, N, d, chunk).total;
}

yoco_status yoco_gret_prefill(const void* q, const void* k, const void* v, const float* gate_logit, float tau,
                              const float* state_in, void* o, float* state_out, int B, int H, int N, int d,
                              int chunk, yoco_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !gate_logit || !o) return YOCO_ERR_NULL;
  if (dtype != YOCO_BF16) return YOCO_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1 || !(tau > 0.f)) return YOCO_ERR_SHAPE;
  if (d != 64 && d != 128) return YOCO_ERR_UNSUPPORTED;
  if (chunk != 128 && chunk != 256) return YOCO_ERR_UNSUPPORTED;
  if (!gret_sizes_ok(B, H, N, d, chunk)) return YOCO_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(gate_logit, 4) ||
      (state_in && !aligned(state_in, 4)) || (state_out && !aligned(state_out, 4)))
    return YOCO_ERR_ALIGN;
  const GretLayout L = gret_layout(B, H, N, d, chunk);
  if (!workspace || workspace_bytes < L.total) return YOCO_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return YOCO_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  yoco::GretArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate_logit;
  a.inv_tau = 1.f / tau;
  a.state_in = state_in;
  a.o = o;
  a.state_out = state_out;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.chunk = chunk;
  a.nc = (N + chunk - 1) / chunk;
  a.lg2 = reinterpret_cast<float*>(ws + L.lg2);
  a.lam = reinterpret_cast<float*>(ws + L.lam);
  a.dR = reinterpret_cast<float*>(ws + L.dR);
  a.rin = ws + L.rin;
  return launched(yoco::launch_gret_prefill(a, as_stream(stream)));
}

yoco_status yoco_gret_decode(const void* q, const void* k, const void* v, const float* gate_logit, float tau,
                             float* state, void* o, int B, int H, int d, yoco_dtype dtype, void* stream) {
  if (!q || !k || !v || !gate_logit || !state || !o) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (B < 1 || H < 1 || (long long)B * H > 65535 || !(tau > 0.f)) return YOCO_ERR_SHAPE;
  if (d != 64 && d != 128) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(o, 4) || !aligned(gate_logit, 4) ||
      !aligned(state, 4))
    return YOCO_ERR_ALIGN;
  yoco::GretDecodeArgs a{q, k, v, gate_logit, 1.f / tau, state, o, B, H, d};
  return launched(yoco::launch_gret_decode(a, dtype == YOCO_BF16, as_stream(stream)));
}

yoco_status yoco_gret_group_norm_swish(const void* y, const void* g, void* out, int B, int H, int N, int d,
                                       float eps, yoco_dtype dtype, void* stream) {
  if (!y || !g || !out) return YOCO_ERR_NULL;
  if (!is_act(dtype)) return YOCO_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1 || !(eps >= 0.f) || isinf(eps)) return YOCO_ERR_SHAPE;
  if (((long long)B * N * H + 3) / 4 > kIntMax) return YOCO_ERR_SHAPE;
  if (d != 64 && d != 128) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(y, 4) || !aligned(g, 4) || !aligned(out, 4)) return YOCO_ERR_ALIGN;
  yoco::GretNormArgs a{y, g, out, B, H, N, d, eps};
  return launched(yoco::launch_gret_norm(a, dtype == YOCO_BF16, as_stream(stream)));
}

size_t yoco_kv_quantize_fp8_workspace_bytes(int Hkv) {
  if (Hkv < 1) return 0;
  return align16((size_t)Hkv * sizeof(uint32_t));
}

yoco_status yoco_kv_quantize_fp8(const void* kv, yoco_dtype in_dtype, void* codes, float* scale, int B, int Hkv,
                                 int n, int d, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv || !codes || !scale) return YOCO_ERR_NULL;
  if (!is_act(in_dtype)) return YOCO_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || n < 1 || B > 65535 || Hkv > 65535) return YOCO_ERR_SHAPE;
  if (!head_dim_ok(d)) return YOCO_ERR_UNSUPPORTED;
  if (!aligned(kv, 16) || !aligned(codes, 16) || !aligned(scale, 4)) return YOCO_ERR_ALIGN;
  if (!workspace || workspace_bytes < yoco_kv_quantize_fp8_workspace_bytes(Hkv)) return YOCO_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return YOCO_ERR_ALIGN;
  yoco::QuantArgs a{kv, static_cast<uint8_t*>(codes), scale, static_cast<uint32_t*>(workspace), B, Hkv,
                    (long long)n * d, (long long)n * d, 0};
  return launched(yoco::launch_quant_fp8(a, in_dtype == YOCO_BF16, as_stream(stream)));
}

}  // extern "C"
