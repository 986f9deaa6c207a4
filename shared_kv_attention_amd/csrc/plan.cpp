// Host-side launch planning shared by the C ABI and the decode launcher.
#include "launch.hpp"

namespace yoco {

// The split count before the chunk is rounded up: it never decreases with
// ctx, and the final count ceil(ctx / chunk) never exceeds it.
static long long split_target(int B, int Hq, int Hkv, int ctx) {
  const long long units = (long long)B * Hkv * ((Hq / Hkv + 3) / 4);
  const long long target = 4096;                       // workgroups (one wave each)
  long long s = (target + units - 1) / units;
  const long long max_s = (ctx + 63) / 64;             // at least 64 keys per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return s;
}

int decode_split_bound(int B, int Hq, int Hkv, int ctx) { return (int)split_target(B, Hq, Hkv, ctx); }

// Split-K plan of the decode kernel: enough one-wave workgroups to keep all
// 256 CUs streaming (about 4096), at least 64 keys per split, the chunk a
// multiple of 64 keys, and never more than kDecodeMaxSplits splits.
void decode_plan(int B, int Hq, int Hkv, int ctx, int* n_splits, int* chunk, int* n_hg) {
  *n_hg = (Hq / Hkv + 3) / 4;
  const long long s = split_target(B, Hq, Hkv, ctx);
  long long c = (ctx + s - 1) / s;
  c = (c + 63) / 64 * 64;
  if ((ctx + c - 1) / c > kDecodeMaxSplits) c = ((ctx + kDecodeMaxSplits - 1) / kDecodeMaxSplits + 63) / 64 * 64;
  *chunk = (int)c;
  *n_splits = (int)((ctx + c - 1) / c);
}

}  // namespace yoco
