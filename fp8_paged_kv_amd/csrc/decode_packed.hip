// The packed-heads decode kernels (page "fp8 paged attention for MoE
// serving", sections "Two compute paths" and "Supported scope": a program
// that packs the KV heads of a block, for short or windowed calls): one
// workgroup per (sequence, group of KV heads), one KV head per wave, no
// splits and no merge.  Default kernel shapes.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_packed(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false, false, false, true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
