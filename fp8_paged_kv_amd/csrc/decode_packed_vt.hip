// The packed-heads decode kernels for V pools in a token-major layout (page
// "fp8 paged attention for MoE serving", section "Supported scope": pack_heads
// with the "heads" and "tokens" payload orders): one workgroup per (sequence,
// group of KV heads), one KV head per wave, each wave staging its V position
// rows in its own LDS stage and reading them back transposed.  Default kernel
// shapes, compiled apart from the d-major packed kernels.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_packed_vt(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                   hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false, true, false, true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
