/*
 * yoco.h -- C ABI of libyoco.so, the MI355X (gfx950) hot path of YOCO
 * ("You Only Cache Once") decoder-decoder attention.
 *
 * The method (pages cited by title and section/segment):
 *   - paperlayer.ai summary of "You Only Cache Once: Decoder-Decoder
 *     Architectures for Language Models" (arXiv 2405.05254v2), sections 1-3;
 *   - podcast transcript "YOCO: caching once for decoder-decoder long-context
 *     language models" (2026-09-25), segments 4, 8, 12, 14, 26.
 * A self-decoder of sliding-window attention layers produces a hidden state;
 * that state is normalised once and projected by one pair of matrices into a
 * single global key/value cache; every cross-decoder layer has its own
 * queries and attends causally, with grouped-query heads, to that one cache.
 * Prefill may skip the cross-decoder for every prompt token but the last.
 *
 * Conventions shared by every call
 *   Layouts     Q, O       [B, H, N, d]      d innermost, head-major
 *               K, V       [B, Hkv, rows, d] head-major; for the global cache
 *                          rows = n_cap (capacity), rows [0, n_kv) valid
 *               X          [B, N, D]
 *               W_K, W_V   [Hkv*d, D]        "out x in": K = norm(X) @ W_K^T
 *               LSE        [B, H, N] float32, natural log of the softmax
 *                          denominator, scale included
 *   Heads       query head h reads KV head h / (Hq / Hkv) (contiguous groups)
 *   dtypes      YOCO_F32 and YOCO_BF16 for activations, caches and outputs;
 *               YOCO_FP8_E4M3 (OCP e4m3fn codes, uint8) only for the global
 *               cache (written by yoco_global_kv_proj or
 *               yoco_kv_quantize_fp8, read by yoco_cross_attn_decode).  All
 *               arithmetic accumulates in float32.
 *   head_dim    d must be 64 or 128.
 *   Pointers    device pointers (HIP), 16-byte aligned, owned by the caller.
 *               Outputs must not overlap inputs.
 *   Stream      `stream` is a hipStream_t passed as void* (NULL = the default
 *               stream).  Every call is stream-ordered and asynchronous:
 *               it enqueues kernels and returns; it never synchronises,
 *               never allocates and keeps no mutable global state, so calls
 *               on different streams may run concurrently (the one
 *               exception, yoco_cross_attn_decode_noalloc, uses a fixed
 *               device array of the library and says so below).
 *   Errors      argument errors are detected before any HIP call and leave
 *               every output untouched; YOCO_ERR_HIP reports a failed launch
 *               (hipGetLastError).  Faults inside a kernel surface
 *               asynchronously at the caller's next synchronisation.
 *               No C++ exception crosses this interface.
 */
#ifndef YOCO_H
#define YOCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  YOCO_OK = 0,
  YOCO_ERR_NULL = 1,        /* a required pointer is NULL                         */
  YOCO_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent  */
  YOCO_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination             */
  YOCO_ERR_UNSUPPORTED = 4, /* valid but not implemented (head_dim, D alignment)  */
  YOCO_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                   */
  YOCO_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required         */
  YOCO_ERR_HIP = 7          /* a HIP launch failed                                */
} yoco_status;

typedef enum { YOCO_F32 = 0, YOCO_BF16 = 1, YOCO_FP8_E4M3 = 2 } yoco_dtype;

/*
 * Global KV projection ("cache once").
 * Source: podcast segment 12 (the self-decoder output is normalised once and
 * projected by a single pair of matrices into the shared keys and values);
 * paperlayer.ai summary section 2 (one global cache reused by every
 * cross-decoder layer).  Normalisation read as RMSNorm:
 *   n_t = x_t / sqrt(mean_j x_tj^2 + eps) * gamma,
 *   K[b,h,pos0+t,c] = sum_j n_bt,j W_K[h*d+c, j]   (V likewise with W_V).
 *   x       [B, N, D] act_dtype (F32 or BF16)
 *   norm_w  [D] act_dtype (gamma), or NULL for gamma = 1
 *   w_k,w_v [Hkv*d, D] act_dtype
 *   k_out,v_out [B, Hkv, n_cap, d] kv_dtype; rows [pos0, pos0+N) written,
 *           other rows untouched (so prompt chunks can be appended)
 * Requires 1 <= N, 0 <= pos0, pos0 + N <= n_cap, D % 64 == 0, D <= 65536.
 * Numerics: float32 accumulation; with gamma given and act_dtype bf16, x*gamma
 * is rounded to bf16 before the product (the row scale is applied in float32).
 * rope_theta > 0 rotates every key (not the values) at its cache position
 * pos0 + t by the rotary embedding of base rope_theta (paperlayer.ai summary
 * appendix E and podcast segment 20: RoPE with a per-stage base, 640K, 5M,
 * 80M): channel pair (2i, 2i+1) turns by (pos0 + t) * rope_theta^(-2i/d), the
 * angle reduced in double precision.  0 = no rotation; NaN, inf or < 0 is
 * YOCO_ERR_SHAPE.
 *
 * kv_dtype is act_dtype (k_scale, v_scale and the workspace are then unused
 * and may be NULL), or YOCO_FP8_E4M3: the cache is written as 8-bit codes
 * (podcast segments 1 and 24: an 8-bit KV cache is the deployed form; the
 * shared cache is written once, segment 12), in the format of
 * yoco_kv_quantize_fp8.  Each value is first rounded to act_dtype, exactly as
 * the act_dtype cache would hold it, and then encoded:
 *   pos0 == 0  the call sets the scales from its own rows: k_scale[h] =
 *              max |K[:, h, 0:N, :]| / 448 (1 if that is 0), v_scale likewise,
 *              both written ([Hkv] float32 each).  The codes equal
 *              yoco_kv_quantize_fp8 applied to the act_dtype projection of the
 *              same rows, bit for bit.
 *   pos0 > 0   rows appended to a cache whose scales are set: k_scale and
 *              v_scale are read, not written, and each value is encoded with
 *              them as yoco_kv_quantize_fp8 encodes (saturating at +-448).
 *   The rows are staged in act_dtype in the workspace: >=
 *   yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, act_dtype, kv_dtype)
 *   bytes, 16-byte aligned, not shared by concurrent calls.
 */
yoco_status yoco_global_kv_proj(const void* x, const void* norm_w,
                                const void* w_k, const void* w_v,
                                void* k_out, void* v_out,
                                float* k_scale, float* v_scale,
                                int B, int N, int D, int Hkv, int d,
                                int n_cap, int pos0, float eps, float rope_theta,
                                yoco_dtype act_dtype, yoco_dtype kv_dtype,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* Workspace of yoco_global_kv_proj for these sizes: 0 unless kv_dtype is
 * YOCO_FP8_E4M3 (and 0 on invalid sizes). */
size_t yoco_global_kv_proj_workspace_bytes(int B, int N, int Hkv, int d,
                                           yoco_dtype act_dtype, yoco_dtype kv_dtype);

/*
 * Self-decoder sliding-window attention.
 * Source: paperlayer.ai summary section 3, "Sliding-Window Attention" (each
 * query restricted to a fixed window, constant-size cache); podcast
 * segments 8 and 15.  Window read as W keys including the query itself:
 *   O[b,h,t] = sum_{t-W < s <= t} softmax_s(scale * q_t . k_s) v_s.
 *   q, o  [B, Hq, N, d];  k, v [B, Hkv, N, d];  lse [B, Hq, N] or NULL.
 * window >= N is ordinary causal attention.  softmax_scale <= 0 selects
 * 1/sqrt(d).
 */
yoco_status yoco_swa_attn(const void* q, const void* k, const void* v,
                          void* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, int window,
                          float softmax_scale, yoco_dtype dtype, void* stream);

/*
 * One sequence shard's sliding-window attention (a long sequence split across
 * devices; the pages' chunk parallelism: paperlayer.ai summary appendix A,
 * podcast segment 14 -- the self-decoder exchanges only with its neighbour).
 * k, v hold the shard's Nkv rows preceded by a halo of the previous shard's
 * last rows: [B, Hkv, Nkv, d]; q, o are the shard's own Nq rows, the last Nq
 * rows of that buffer: [B, Hq, Nq, d]; lse [B, Hq, Nq] or NULL.  Row i sits
 * at buffer position Nkv - Nq + i and sees the window of W keys ending there,
 * so a halo of at least W - 1 rows gives exactly those rows of the full
 * sequence's sliding-window attention (bitwise when the halo starts at a
 * multiple of 64 sequence positions: the key tiles then coincide).
 * Requires 1 <= Nq <= Nkv; otherwise as yoco_swa_attn.
 */
yoco_status yoco_swa_attn_halo(const void* q, const void* k, const void* v,
                               void* o, float* lse,
                               int B, int Hq, int Hkv, int Nq, int Nkv, int d, int window,
                               float softmax_scale, yoco_dtype dtype, void* stream);

/*
 * Merge of attention results over disjoint key sets (the shards of a cache
 * split across devices, each decoded with yoco_cross_attn_decode and its
 * log-sum-exp): o = sum_s exp(lse_s - L) o_s, L = log sum_s exp(lse_s).
 *   o_parts [S, rows, d] (F32 or BF16), lse_parts [S, rows] float32,
 *   o [rows, d], lse [rows] float32 or NULL; rows = B * Hq of the decode.
 * Requires S >= 1, d in {64, 128}.  Float32 arithmetic.
 */
yoco_status yoco_attn_merge(const void* o_parts, const float* lse_parts, void* o, float* lse,
                            int S, int rows, int d, yoco_dtype dtype, void* stream);

/*
 * Cross-decoder causal attention over the shared cache, many queries
 * (full prefill of one cross-decoder layer, or a chunk of it).
 * Source: podcast segment 12 (each cross layer has its own queries and
 * attends causally to the one shared pair, grouped-query heads); paperlayer.ai
 * summary sections 1-2 (causal masking; one cache reused across layers).
 * Every cross layer passes the SAME k/v pointers: the call only reads them.
 *   q, o  [B, Hq, Nq, d]: query i sits at absolute position q_offset + i and
 *         sees cache rows 0 .. q_offset + i.
 *   k, v  [B, Hkv, n_cap, d], rows [0, n_kv) valid.   lse [B, Hq, Nq] or NULL.
 * Requires 0 <= q_offset, q_offset + Nq <= n_kv <= n_cap.
 */
yoco_status yoco_cross_attn_prefill(const void* q, const void* k, const void* v,
                                    void* o, float* lse,
                                    int B, int Hq, int Hkv, int Nq, int n_kv,
                                    int n_cap, int q_offset, int d,
                                    float softmax_scale, yoco_dtype dtype,
                                    void* stream);

/*
 * Cross-decoder attention for one new token per sequence (decode step, and
 * the last prompt position of an early-exit prefill).
 * Source: podcast segment 4 and 26 (every decode step streams the whole
 * cache, bandwidth bound), segment 14 and its Figure 3 (only the final prompt
 * position goes through the cross-decoder; output unchanged).
 * The cache already holds the current token: sequence b attends to rows
 * 0 .. ctx_b - 1.  Split-K over the context with a combine pass.
 *   q, o       [B, Hq, d] q_dtype (o in q_dtype)
 *   k_cache, v_cache [B, Hkv, n_cap, d] kv_dtype
 *   k_scale, v_scale [Hkv] float32, required iff kv_dtype == YOCO_FP8_E4M3:
 *              a code c stands for scale[h] * decode_e4m3fn(c)
 *   ctx_lens   [B] int32 on the device, or NULL: then every ctx_b = ctx.
 *              When given, every ctx_lens[b] must lie in [1, ctx]
 *              (checked by the kernel only by clamping: rows >= ctx are
 *              never read).
 *   ctx        1 <= ctx <= n_cap (context length, or its upper bound)
 *   lse        [B, Hq] float32 or NULL
 *   workspace  >= yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d)
 *              bytes of device memory, 16-byte aligned; contents need not
 *              be initialised; must not be shared by calls running
 *              concurrently.
 * Supported (q, kv) dtypes: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 */
yoco_status yoco_cross_attn_decode(const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* ctx_lens,
                                   int ctx, void* o, float* lse,
                                   int B, int Hq, int Hkv, int n_cap, int d,
                                   float softmax_scale, yoco_dtype q_dtype,
                                   yoco_dtype kv_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace of yoco_cross_attn_decode for these sizes (0 on invalid sizes). */
size_t yoco_cross_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int ctx, int d);

/*
 * yoco_cross_attn_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP stream capture, tight serving
 * loops, harnesses that forbid allocation.  The split partials live in a
 * fixed device array of the library (one copy per GPU, held until the process
 * ends); the call allocates nothing and runs the same kernels, so its output
 * equals yoco_cross_attn_decode's bit for bit.
 *   Arguments, layouts and checks as yoco_cross_attn_decode.
 *   Limit: the workspace yoco_cross_attn_decode_workspace_bytes would return
 *   for these sizes must not exceed yoco_cross_attn_decode_noalloc_max_bytes()
 *   (16 MiB: 32768 partial rows of d = 128 floats, which covers every call
 *   with up to 512 sequences of 32 query heads at d = 128, whatever the
 *   context length); larger sizes return YOCO_ERR_WORKSPACE before any
 *   launch.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or different host threads) race and must
 *   be serialised by the caller.  Nothing in the array needs clearing between
 *   calls.  The first call on each device looks up that device's copy (one
 *   hipGetSymbolAddress, no allocation); a failure there is YOCO_ERR_HIP.
 */
yoco_status yoco_cross_attn_decode_noalloc(const void* q, const void* k_cache,
                                           const void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* ctx_lens,
                                           int ctx, void* o, float* lse,
                                           int B, int Hq, int Hkv, int n_cap, int d,
                                           float softmax_scale, yoco_dtype q_dtype,
                                           yoco_dtype kv_dtype, void* stream);

/* Bytes of the fixed device array behind yoco_cross_attn_decode_noalloc. */
size_t yoco_cross_attn_decode_noalloc_max_bytes(void);

/*
 * Self-decoder sliding-window attention for one new token per sequence (a
 * generation step), over the layer's ring cache of W slots.
 * Source: paperlayer.ai summary section 3 (each query sees a fixed window of
 * recent positions, so the self-decoder's cache stays window-sized however
 * long the sequence) and section 2; podcast segment 4 (one token per decoding
 * step).
 * Ring layout: k_ring, v_ring [B, Hkv, W, d]; position t lives in slot t mod W.
 * If k_new and v_new ([B, Hkv, d]) are given, they are first written to slot
 * pos mod W (the current token's K/V; both or neither may be NULL).  The query
 * at position pos then attends to positions max(0, pos - W + 1) .. pos, i.e.
 * ring slots 0 .. min(pos + 1, W) - 1; the caller must have written every
 * earlier position of that window.  All sequences are at the same pos.
 *   q, o  [B, Hq, d]      lse [B, Hq] float32 or NULL      pos >= 0, W >= 1
 *   workspace >= yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d) bytes of
 *   device memory, 16-byte aligned, not shared by concurrent calls.
 * Supported dtypes: F32, BF16 (q, rings, new K/V and o in that dtype).
 */
yoco_status yoco_swa_decode(const void* q, const void* k_new, const void* v_new,
                            void* k_ring, void* v_ring, int pos, void* o, float* lse,
                            int B, int Hq, int Hkv, int W, int d, float softmax_scale,
                            yoco_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace of yoco_swa_decode for any pos with this window (0 on invalid sizes). */
size_t yoco_swa_decode_workspace_bytes(int B, int Hq, int Hkv, int W, int d);

/*
 * Gated retention, the self-decoder's other choice (prefill, chunkwise form).
 * Source: paperlayer.ai summary section 3 Gated Retention and appendix B;
 * podcast segment 16 (retention with a data-dependent, head-wise scalar
 * decay gate sigmoid(z)^(1/tau); recurrent, parallel and chunkwise forms give
 * equal results; chunk size 256).  Per head (state S is d x d, [dk][dv]):
 *     S_n = gamma_n S_{n-1} + k_n^T v_n,   o_n = q_n S_n,
 *     gamma_n = sigmoid(gate_logit_n)^(1/tau)
 * computed chunkwise over chunks of `chunk` positions.  No scale on q . k
 * and no rotation (the per-head GroupNorm that follows cancels a scale).
 *   q, k, v, o   [B, H, N, d] BF16          gate_logit [B, H, N] float32
 *   state_in     [B, H, d, d] float32, or NULL for a zero state
 *   state_out    [B, H, d, d] float32, or NULL: the state after position N-1
 *                (feed it to yoco_gret_decode to continue)
 *   tau > 0; d in {64, 128}; chunk in {128, 256}
 *   workspace >= yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk) bytes,
 *   16-byte aligned, not shared by concurrent calls.
 */
yoco_status yoco_gret_prefill(const void* q, const void* k, const void* v, const float* gate_logit,
                              float tau, const float* state_in, void* o, float* state_out,
                              int B, int H, int N, int d, int chunk, yoco_dtype dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of yoco_gret_prefill for these sizes (0 on invalid sizes). */
size_t yoco_gret_prefill_workspace_bytes(int B, int H, int N, int d, int chunk);

/*
 * Gated retention, one decode step (recurrent form): for every (b, h),
 *     S <- gamma S + k^T v,  o = q S,  gamma = sigmoid(gate_logit)^(1/tau).
 * Source: podcast segment 16 (recurrent form for decoding, one d x d state
 * per head, constant memory); paperlayer.ai summary section 3.
 *   q, k, v, o [B, H, d] (F32 or BF16)   gate_logit [B, H] float32
 *   state      [B, H, d, d] float32, read and updated in place
 *   tau > 0; d in {64, 128}
 */
yoco_status yoco_gret_decode(const void* q, const void* k, const void* v, const float* gate_logit,
                             float tau, float* state, void* o, int B, int H, int d,
                             yoco_dtype dtype, void* stream);

/*
 * Multi-head gated retention's output combination: each head's output is
 * normalised over its d channels (GroupNorm with one group per head, unit
 * gain, zero bias) and multiplied by a swish gate.
 * Source: paperlayer.ai summary section 3 Gated Retention (heads combined
 * with GroupNorm, plus a swish gate).
 *   out[b, n, h*d + j] = swish(g[b, n, h*d + j]) * (y[b,h,n,j] - mean) / sqrt(var + eps)
 *   y [B, H, N, d]; g, out [B, N, H*d]; F32 or BF16; d in {64, 128}; eps >= 0
 */
yoco_status yoco_gret_group_norm_swish(const void* y, const void* g, void* out, int B, int H, int N,
                                       int d, float eps, yoco_dtype dtype, void* stream);

/*
 * Block layer glue: pre-norm Q/K/V projection of one attention layer.
 * Source: podcast segment 12 (a self-decoder layer runs its attention on the
 * normalised input, plus a residual; a cross-decoder layer keeps only its own
 * query projection).  Normalisation read as RMSNorm, as for the global
 * projection:
 *   n_t = x_t / sqrt(mean_j x_tj^2 + eps) * gamma,
 *   q[b,h,t,c] = sum_j n_bt,j W_q[h*d+c, j]       (k, v likewise)
 *   x          [B, N, D];  norm_w [D] or NULL (gamma = 1)
 *   w_q        [Hq*d, D];  q_out [B, Hq, N, d]
 *   w_k, w_v   [Hkv*d, D]; k_out, v_out [B, Hkv, N, d]; Hkv = 0 (all four
 *              NULL) projects q only, as a cross-decoder layer does
 * rope_theta > 0 rotates q and k (not v) of token t at position rope_pos0 + t
 * exactly as yoco_global_kv_proj rotates its keys; 0 = no rotation.
 * Requires D % 64 == 0, D <= 65536, d in {64, 128}, rope_pos0 >= 0; one dtype
 * (F32 or BF16) for every tensor.  Numerics as yoco_global_kv_proj.
 */
yoco_status yoco_qkv_proj(const void* x, const void* norm_w, const void* w_q, const void* w_k,
                          const void* w_v, void* q_out, void* k_out, void* v_out, int B, int N,
                          int D, int Hq, int Hkv, int d, float eps, float rope_theta, int rope_pos0,
                          yoco_dtype dtype, void* stream);

/*
 * Block layer glue: the SwiGLU feed-forward's gated hidden activations.
 * Source: podcast segment 12 (each layer's attention is followed by a SwiGLU
 * feed-forward; the sizes are the caller's, the pages give none).
 *   h[b,t,j] = silu(n_bt . W_gate[j]) * (n_bt . W_up[j]),  silu(z) = z / (1 + e^-z),
 *   n = RMSNorm(x) * gamma as above.
 *   x [B, N, D]; norm_w [D] or NULL; w_gate, w_up [F, D]; h [B, N, F]
 * Requires D % 64 == 0, D <= 65536, F % 4 == 0.  h is rounded to the dtype
 * (it feeds yoco_linear_residual with W_down).
 */
yoco_status yoco_swiglu(const void* x, const void* norm_w, const void* w_gate, const void* w_up,
                        void* h, int B, int N, int D, int F, float eps, yoco_dtype dtype,
                        void* stream);

/*
 * Block layer glue: a residual product, y += a W^T, row by row.
 * Source: podcast segment 12 (every sub-layer adds its result to the
 * residual stream): the attention output projection W_o and the
 * feed-forward's W_down.
 *   a_heads == 0: a [B, N, K], row (b, n) is a[b, n, :]
 *   a_heads  > 0: a [B, a_heads, N, K / a_heads] head-major (an attention
 *                 output); row (b, n) is the concatenation over heads h of
 *                 a[b, h, n, :]
 *   w [F, K];  y [B, N, F] read and updated in place (the residual stream);
 *   y must not overlap a or w.
 * Requires K % 64 == 0 (and (K / a_heads) % 64 == 0), K <= 65536, F % 4 == 0.
 * With BF16, y + a W^T is formed in float32 and rounded once.
 */
yoco_status yoco_linear_residual(const void* a, int a_heads, const void* w, void* y, int B, int N,
                                 int K, int F, yoco_dtype dtype, void* stream);

/*
 * Quantise a K or V tensor to an 8-bit cache.
 * Source: podcast segments 1 and 24 (8-bit KV cache as the deployed form);
 * the format is fixed here: OCP e4m3fn, one float32 scale per KV head over
 * all (b, n, d), s_h = amax_h / 448 (1 if the head is all zero),
 * code = RNE-saturating e4m3fn(x / s_h) with x / s_h one IEEE float32
 * division.
 *   kv     [B, Hkv, n, d] in_dtype (F32 or BF16), finite values
 *   codes  [B, Hkv, n, d] uint8 (written)
 *   scale  [Hkv] float32 (written)
 *   workspace >= yoco_kv_quantize_fp8_workspace_bytes(Hkv) bytes.
 */
yoco_status yoco_kv_quantize_fp8(const void* kv, yoco_dtype in_dtype, void* codes,
                                 float* scale, int B, int Hkv, int n, int d,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

size_t yoco_kv_quantize_fp8_workspace_bytes(int Hkv);

/*
 * Achievable-peak microbenchmarks (diagnostics, not part of the method): what
 * this chip reaches at its clock under load, beside the spec peaks.
 * yoco_peak_hbm_read streams `bytes` (a multiple of 16) of `buf` once with
 * `blocks` workgroups of 256 threads, each reading one contiguous 1/blocks of
 * the buffer, and writes one wrapping 32-bit sum of the words each workgroup
 * read to partial[blocks] (their sum, modulo 2^32, is the sum of every 32-bit
 * word of the buffer).
 * yoco_peak_mfma_bf16 runs `blocks` workgroups of 4 waves, each wave `iters`
 * rounds of 8 independent 32x32x16 bf16 MFMAs (2^18 flops per round) on
 * operands of ones, and writes out[4 * blocks] = 128 * iters per wave
 * (exact for iters <= 2^20).
 * yoco_peak_mfma_bf16_toggling runs the same count of MFMAs (iters a
 * multiple of 8) on operands that change every instruction, as real data's
 * do: per-lane integers in [-127, 127] whose products cancel over every 8
 * rounds, so out[4 * blocks] = 0 exactly per wave.
 */
yoco_status yoco_peak_hbm_read(const void* buf, size_t bytes, uint32_t* partial, int blocks, void* stream);
yoco_status yoco_peak_mfma_bf16(int iters, float* out, int blocks, void* stream);
yoco_status yoco_peak_mfma_bf16_toggling(int iters, float* out, int blocks, void* stream);

/* Static description of a status code (never NULL). */
const char* yoco_status_string(yoco_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int yoco_version(void);

#ifdef __cplusplus
}
#endif

#endif /* YOCO_H */
