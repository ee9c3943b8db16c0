// The packed-heads decode kernels with splits: a unit is (sequence, group of
// KV heads read by one workgroup together, one head per wave), and long spans
// are cut into balanced shares and merged like the split kernel's units
// (page "fp8 paged attention for MoE serving", pack_heads; the split grid of
// section "Why it happens").  Default kernel shapes.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_pksplit(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                 hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false, false, false, false, true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
