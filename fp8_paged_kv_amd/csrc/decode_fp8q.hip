// The decode kernels of the fp8 compute mode (page "fp8 paged attention for
// MoE serving", section "Two compute paths": an fp8 tensor-core dot that
// rounds q to E4M3): QK^T on the gfx950 fp8 MFMA with the K codes as they are
// stored, PV in bf16 as in the default mode.  Default kernel shapes, per-page
// and per-token fp32 scales.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_fp8q(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                              hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (scale_kind == 2 && D % 128) return hipErrorNotSupported;
  return launch_family<false, false, true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
