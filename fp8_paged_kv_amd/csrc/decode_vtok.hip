// The decode kernels for V pools in a token-major layout: the page's own
// "heads" ([Hkv][P][D]) and "tokens" ([P][Hkv][D]) payload orders (page "fp8
// paged attention for MoE serving", section "Supported scope").  V position
// rows are staged per wave in LDS and read back transposed; the default kernel
// shape of each head dim, compiled apart from the plain kernels.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_vtok(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                              hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false, true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
