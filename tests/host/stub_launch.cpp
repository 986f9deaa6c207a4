// Host-only stand-ins for the kernel launchers of libyoco, so that the C ABI
// (argument validation, workspace layout, dispatch) can be built with the
// host compiler under AddressSanitizer / UndefinedBehaviorSanitizer.  Each
// stub records the argument block it received and reports success.
#include "../../shared_kv_attention_amd/csrc/launch.hpp"

namespace yoco {
int g_launches = 0;
AttnArgs g_attn;
DecodeArgs g_decode;
ProjArgs g_proj;
QuantArgs g_quant;
GretArgs g_gret;
GretDecodeArgs g_gret_dec;
GretNormArgs g_gret_norm;
LinArgs g_lin;
MergeArgs g_merge;
int g_lin_mode = -1;
int g_decode_kinds[3];

hipError_t launch_attn(const AttnArgs& a, bool, int, bool, hipStream_t) { ++g_launches; g_attn = a; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs& a, int qk, int kk, int d, hipStream_t) {
  ++g_launches; g_decode = a; g_decode_kinds[0] = qk; g_decode_kinds[1] = kk; g_decode_kinds[2] = d; return hipSuccess;
}
hipError_t launch_kv_proj(const ProjArgs& a, bool, hipStream_t) { ++g_launches; g_proj = a; return hipSuccess; }
hipError_t launch_quant_fp8(const QuantArgs& a, bool, hipStream_t) { ++g_launches; g_quant = a; return hipSuccess; }
uint32_t* g_clear_ptr = nullptr;
int g_clear_n = 0;
QuantArgs g_encode[2];
int g_encodes = 0;
hipError_t launch_quant_clear(uint32_t* p, int n, hipStream_t) {
  ++g_launches; g_clear_ptr = p; g_clear_n = n; return hipSuccess;
}
int g_amax_passes = 0;
hipError_t launch_quant_amax(const QuantArgs&, bool, hipStream_t) { ++g_launches; ++g_amax_passes; return hipSuccess; }
hipError_t launch_quant_encode(const QuantArgs& a, bool, hipStream_t) {
  ++g_launches; g_encode[g_encodes++ & 1] = a; return hipSuccess;
}
hipError_t launch_gret_prefill(const GretArgs& a, hipStream_t) { ++g_launches; g_gret = a; return hipSuccess; }
hipError_t launch_gret_decode(const GretDecodeArgs& a, bool, hipStream_t) { ++g_launches; g_gret_dec = a; return hipSuccess; }
hipError_t launch_gret_norm(const GretNormArgs& a, bool, hipStream_t) { ++g_launches; g_gret_norm = a; return hipSuccess; }
hipError_t launch_attn_merge(const MergeArgs& a, bool, hipStream_t) { ++g_launches; g_merge = a; return hipSuccess; }
hipError_t launch_peak_read(const void*, long long, uint32_t*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_peak_mfma(int, float*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_peak_mfma_toggle(int, float*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_linear(const LinArgs& a, int mode, bool, hipStream_t) {
  ++g_launches; g_lin = a; g_lin_mode = mode; return hipSuccess;
}
}  // namespace yoco
