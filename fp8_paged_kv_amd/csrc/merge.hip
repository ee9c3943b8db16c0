// Standalone log-sum-exp merge of split partials (see merge_common.h for the
// formula).  One workgroup per (sequence, group of query heads).
#include "fp8pa_internal.h"
#include "merge_common.h"

namespace fp8pa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  extern __shared__ float s_w[];
  __shared__ float s_inv[16];
  const int grp = blockIdx.x, b = blockIdx.y;
  merge_heads<D, false>(a.part_o, a.part_lse, a.sinks, a.out, b, a.Hq, a.S, grp * a.G, a.G, a.S, s_w, s_inv);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t st) {
  dim3 grid(a.Hq / a.G, B), block(256);
  const size_t lds = (size_t)a.G * (a.S > 0 ? a.S : 1) * sizeof(float);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, block, lds, st, a); break;
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, block, lds, st, a); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL(merge_kernel<512>, grid, block, lds, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace fp8pa
