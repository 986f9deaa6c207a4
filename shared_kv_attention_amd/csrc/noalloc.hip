// The allocation-free form of the one-token cross-decoder decode: the split
// partials live in a fixed device array of this library instead of a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  It runs exactly the kernels of yoco_cross_attn_decode.
//
// The array is a file-scope __device__ object; each GPU holds its own copy at
// its own address until the process ends.  Host code never passes the
// array's name to a kernel (on the host that name is only a stand-in): the
// first call on a device, with that device current, looks the copy's address
// up with hipGetSymbolAddress and keeps it per device; every later use goes
// through that address.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/yoco.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_addr[kMaxDevices];

// Address of the current device's copy of `scratch` (looked up once per
// device; concurrent first calls look up the same address).
yoco_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return YOCO_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return YOCO_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return YOCO_OK;
}

}  // namespace

extern "C" {

size_t yoco_cross_attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

yoco_status yoco_cross_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                           const float* k_scale, const float* v_scale, const int32_t* ctx_lens,
                                           int ctx, void* o, float* lse, int B, int Hq, int Hkv, int n_cap, int d,
                                           float softmax_scale, yoco_dtype q_dtype, yoco_dtype kv_dtype,
                                           void* stream) {
  // Every argument check of the workspace form, without launching anything:
  // with no workspace a valid call stops at YOCO_ERR_WORKSPACE.
  const yoco_status dry = yoco_cross_attn_decode(q, k_cache, v_cache, k_scale, v_scale, ctx_lens, ctx, o, lse, B, Hq,
                                                 Hkv, n_cap, d, softmax_scale, q_dtype, kv_dtype, nullptr, 0, stream);
  if (dry != YOCO_ERR_WORKSPACE) return dry;
  const size_t need = yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d);
  if (need == 0 || need > kScratchBytes) return YOCO_ERR_WORKSPACE;
  void* ws = nullptr;
  const yoco_status st = device_scratch(&ws);
  if (st != YOCO_OK) return st;
  return yoco_cross_attn_decode(q, k_cache, v_cache, k_scale, v_scale, ctx_lens, ctx, o, lse, B, Hq, Hkv, n_cap, d,
                                softmax_scale, q_dtype, kv_dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
