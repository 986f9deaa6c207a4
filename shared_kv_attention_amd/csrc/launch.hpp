// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
// Argument blocks are passed to kernels by value; every pointer is a device
// pointer that abi.cpp has already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace yoco {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  int B, Hq, Hkv, Nq;
  int n_kv;            // valid key rows (keys >= n_kv are never read)
  int kv_rows;         // rows per head in the k/v buffers
  int q_offset;        // absolute position of query row 0
  int window;          // sliding window (only read by the window variant)
  float scale_log2;    // softmax scale * log2(e)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;    // fp8 caches only
  const float* v_scale;
  const int32_t* ctx_lens; // may be null
  int ctx;
  float* part_o;           // [B, Hq, n_splits, d]
  float* part_m;           // [B, Hq, n_splits]  (log2 domain)
  float* part_l;           // [B, Hq, n_splits]
  void* o;
  float* lse;              // may be null
  int B, Hq, Hkv, n_cap;
  int n_splits, chunk, n_hg;
  float scale_log2;
  int full_lines;          // bf16 K read in whole lines, three blocks ahead (long splits)
  // Ring append folded into the decode (self-decoder window): when k_new is
  // set, key row new_slot of every (sequence, KV head) is read from
  // k_new / v_new [B, Hkv, d] instead of k / v, and written into k / v
  const void* k_new;
  const void* v_new;
  int new_slot;
};

struct ProjArgs {
  const void* x;
  const void* norm_w;  // may be null
  const void* w_k;
  const void* w_v;
  void* k_out;
  void* v_out;
  int B, N, D, Hkv, d, n_cap;
  int pos0;                // position of token 0 (rotary embedding)
  int row0;                // cache row written for token 0 (pos0, or 0 into a staging buffer)
  float eps;
  double rope_log2_theta;  // rotary embedding of K at position pos0 + n (0: none)
  // amax_bits (non-null, for an 8-bit cache that follows): also raise
  // amax_bits[head] (K) and amax_bits[Hkv + head] (V) to the bit pattern of
  // the largest |value| written, each value as stored in the activation dtype
  uint32_t* amax_bits;
};

// Position-wise block layers (linear.hip).  Weight matrices are [rows, K]
// ("out x in"); x rows are [K] (row-major [B*N, K]) or, with x_heads > 0,
// gathered from a head-major [B, x_heads, N, K / x_heads] tensor.
enum { kLinQKV = 0, kLinSwiGLU = 1, kLinResidual = 2 };
struct LinArgs {
  const void* x;
  const void* norm_w;  // [K] gain or null (QKV / SwiGLU with norm)
  const void* w0;      // QKV: W_q; SwiGLU: W_gate; residual: W
  const void* w1;      // QKV: W_k (or null); SwiGLU: W_up
  const void* w2;      // QKV: W_v (or null)
  void* y0;            // QKV: q [B, h0, N, d]; SwiGLU: h [B*N, F]; residual: y [B*N, F] (+=)
  void* y1;            // QKV: k [B, h1, kv_rows, d], rows [kv_pos0, kv_pos0 + N)
  void* y2;            // QKV: v [B, h1, kv_rows, d], likewise
  int B, N, K, F;      // F: output features (QKV: (h0 + 2 h1) d; SwiGLU: hidden size)
  int x_heads;         // 0 or the head count of a head-major x
  int f1, f2;          // QKV: first k feature, first v feature (F when absent)
  int h0, h1, d;       // QKV: q heads, k/v heads, head dim
  int kv_rows, kv_pos0;  // QKV: rows per head of the k/v buffers, first row written
  int norm;            // fused RMSNorm of the x rows (QKV, SwiGLU)
  float eps;
  double rope_log2_theta;  // QKV: rotary embedding of q and k, log2 of its base (0: none)
  int rope_pos0;           // QKV: position of token row n is rope_pos0 + n
};

struct MergeArgs {
  const void* o_parts;     // [S, rows, d] activation dtype
  const float* lse_parts;  // [S, rows]
  void* o;                 // [rows, d]
  float* lse;              // [rows] or null
  int S, rows, d;
};

struct GretArgs {
  const void* q;           // [B, H, N, d] bf16
  const void* k;
  const void* v;
  const float* gate;       // [B, H, N] gate logits z
  float inv_tau;           // 1 / temperature
  const float* state_in;   // [B, H, d, d] or null (zero state)
  void* o;                 // [B, H, N, d] bf16
  float* state_out;        // [B, H, d, d] or null
  int B, H, N, d, chunk, nc;
  float* lg2;              // workspace: [B, H, N] log2 decay, prefix sums within each chunk
  float* lam;              // workspace: [B, H, nc] total decay of each chunk
  float* dR;               // workspace: [B, H, nc, d, d] per-chunk state contributions
  void* rin;               // workspace: [B, H, nc, d, d] bf16 state entering each chunk
};

struct GretDecodeArgs {
  const void* q;           // [B, H, d]
  const void* k;
  const void* v;
  const float* gate;       // [B, H] gate logits
  float inv_tau;
  float* state;            // [B, H, d, d] float32, updated in place
  void* o;                 // [B, H, d]
  int B, H, d;
};

struct GretNormArgs {
  const void* y;           // [B, H, N, d]
  const void* g;           // [B, N, H*d]
  void* out;               // [B, N, H*d]
  int B, H, N, d;
  float eps;
};

struct QuantArgs {
  const void* kv;
  uint8_t* codes;
  float* scale;
  uint32_t* amax_bits;  // workspace [Hkv]
  int B, Hkv;
  long long slab;       // n * d elements per (batch, head) of kv
  long long dst_slab;   // elements per (batch, head) of codes (n_cap * d)
  long long dst_off;    // first element written in each codes slab (pos0 * d)
  int scale_given;      // encode with scale[] as given instead of setting it from amax_bits
};

hipError_t launch_attn(const AttnArgs& a, bool is_bf16, int d, bool swa, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int q_kind, int kv_kind, int d, hipStream_t stream);
hipError_t launch_kv_proj(const ProjArgs& a, bool is_bf16, hipStream_t stream);
hipError_t launch_linear(const LinArgs& a, int mode, bool is_bf16, hipStream_t stream);
hipError_t launch_quant_fp8(const QuantArgs& a, bool is_bf16, hipStream_t stream);
// The steps of launch_quant_fp8 one by one (clear n maxima, raise them over a
// tensor, encode), for an 8-bit cache filled from a staged projection.
hipError_t launch_quant_clear(uint32_t* amax_bits, int n, hipStream_t stream);
hipError_t launch_quant_amax(const QuantArgs& a, bool is_bf16, hipStream_t stream);
hipError_t launch_quant_encode(const QuantArgs& a, bool is_bf16, hipStream_t stream);
hipError_t launch_attn_merge(const MergeArgs& a, bool is_bf16, hipStream_t stream);
hipError_t launch_peak_read(const void* src, long long bytes, uint32_t* partial, int blocks, hipStream_t stream);
hipError_t launch_peak_mfma(int iters, float* out, int blocks, hipStream_t stream);
hipError_t launch_peak_mfma_toggle(int iters, float* out, int blocks, hipStream_t stream);
hipError_t launch_gret_prefill(const GretArgs& a, hipStream_t stream);
hipError_t launch_gret_decode(const GretDecodeArgs& a, bool is_bf16, hipStream_t stream);
hipError_t launch_gret_norm(const GretNormArgs& a, bool is_bf16, hipStream_t stream);

// Split plan of the decode kernel (host code, plan.cpp); the workspace size
// follows from it.  At most kDecodeMaxSplits splits (the combine pass keeps one
// weight per split in LDS).
constexpr int kDecodeMaxSplits = 4096;
// Workgroup targets: at most kDecodeMaxWorkgroups (the workspace is sized for
// it); decode_workgroup_target gives the one for a kernel form (kv_kind:
// 0 float32, 1 bf16, 2 fp8).
constexpr int kDecodeMaxWorkgroups = 4096;
// bf16 d = 128 splits of at least this many keys use the whole-line K form
// (three blocks in flight, 3 waves per SIMD) and its own workgroup target;
// fp8 d = 128 splits that long are planned for 3 waves per SIMD as well.
constexpr int kDecodeFullLineMinChunk = 1024;
int decode_workgroup_target(int kv_kind, int d);
void decode_plan(int B, int Hq, int Hkv, int ctx, int target, int* n_splits, int* chunk, int* n_hg);
// An upper bound on decode_plan's n_splits for every context length <= ctx
// and every target <= kDecodeMaxWorkgroups.
int decode_split_bound(int B, int Hq, int Hkv, int ctx);

}  // namespace yoco
