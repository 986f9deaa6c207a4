// Host-side launch planning shared by the C ABI and the decode launcher.
#include "launch.hpp"

namespace yoco {

// The split count before the chunk is rounded up: it never decreases with
// ctx, and the final count ceil(ctx / chunk) never exceeds it.
static long long split_target(int B, int Hq, int Hkv, int ctx, int target) {
  const long long units = (long long)B * Hkv * ((Hq / Hkv + 3) / 4);
  long long s = (target + units - 1) / units;          // target: workgroups (one wave each)
  const long long max_s = (ctx + 63) / 64;             // at least 64 keys per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return s;
}

int decode_split_bound(int B, int Hq, int Hkv, int ctx) {
  return (int)split_target(B, Hq, Hkv, ctx, kDecodeMaxWorkgroups);
}

// One resident round of the whole-line K form (bf16, d = 128): three K
// blocks in flight take 152 VGPRs, 3 waves per SIMD, 12 per CU.  The fp8
// d = 128 form (116 VGPRs) could hold 4 waves per SIMD, but with long splits
// 3 per SIMD stream faster (512K-key x 8 decode: 6.30 against 6.16 TB/s).
int decode_workgroup_target(int kv_kind, int d) {
  return (kv_kind == 1 || kv_kind == 2) && d == 128 ? 256 * 12 : kDecodeMaxWorkgroups;
}

// Split-K plan of the decode kernel: about `target` one-wave workgroups (one
// resident round on the 256 CUs), at least 64 keys per split, the chunk a
// multiple of 64 keys, and never more than kDecodeMaxSplits splits.  The
// split count never exceeds the plan for a larger target.
void decode_plan(int B, int Hq, int Hkv, int ctx, int target, int* n_splits, int* chunk, int* n_hg) {
  *n_hg = (Hq / Hkv + 3) / 4;
  const long long s = split_target(B, Hq, Hkv, ctx, target);
  long long c = (ctx + s - 1) / s;
  c = (c + 63) / 64 * 64;
  if ((ctx + c - 1) / c > kDecodeMaxSplits) c = ((ctx + kDecodeMaxSplits - 1) / kDecodeMaxSplits + 63) / 64 * 64;
  *chunk = (int)c;
  *n_splits = (int)((ctx + c - 1) / c);
}

}  // namespace yoco
