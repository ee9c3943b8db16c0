// The decode kernels for V pools in a token-major layout: the page's own
// "heads" ([Hkv][P][D]) and "tokens" ([P][Hkv][D]) payload orders (page "fp8
// paged attention for MoE serving", section "Supported scope").  V position
// rows are staged per wave in LDS and read back transposed; the default kernel
// shape of each head dim, compiled apart from the plain kernels.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_vtok(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                              hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  auto l = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() {
    return launch_d<DD, NS, PF, OCC, KNT, NW, false, true>(a, scale_kind, W, lds, st, e0, e1);
  };
  return k_whole_lines ? default_shape<true>(D, l) : default_shape<false>(D, l);
}

size_t decode_vstage_bytes(int D) {
  auto l = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() -> size_t {
    return (size_t)NW * 32 * NS * VStage<DD>::RS + 16;   // + slack to align the stages to 16 bytes
  };
  return default_shape<false>(D, l);
}

}  // namespace fp8pa
