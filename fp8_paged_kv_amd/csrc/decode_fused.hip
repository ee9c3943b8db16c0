// The decode kernels that also append each sequence's new token (page
// "Lecture 8 — Inference Path: KV Cache, Decode, RoPE, GQA, Paged KV" of the
// FlashAttention course, section "In-kernel KV cache update"): the default
// kernel shape of each head dim, compiled apart from the plain kernels.
#include "decode_kernel.h"

namespace fp8pa {

hipError_t launch_decode_fused(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                               hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<true>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
