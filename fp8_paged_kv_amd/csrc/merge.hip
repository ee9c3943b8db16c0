// Log-sum-exp merge of split partials for gfx950.
//
// The method splits each sequence across workgroups so the whole chip is busy
// (page "fp8 paged attention for MoE serving", section "Why it happens"); the
// pages do not print how the partial results are combined.  The reading taken
// is the standard one: split s carries o_s (normalised) and lse_s (natural-log
// sum of exp of its scores); with M = max(max_s lse_s, sink),
//   o = sum_s e^(lse_s - M) o_s / (sum_s e^(lse_s - M) + e^(sink - M)).
// One wave64 per (sequence, query head); each lane owns D/64 dims.
#include "device_common.h"
#include "fp8pa_internal.h"

namespace fp8pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  int ns = a.S;
  if (a.seq_lens) {
    // Same split count as the decode kernel; at most one split means the
    // decode kernel wrote the final output itself.
    const int L = a.seq_lens[b];
    const int start = (a.window > 0 && L > a.window) ? L - a.window : 0;
    const int tbeg = start & ~(a.tile_tokens - 1);
    const int need = (L > start) ? (L - tbeg + a.split_tokens - 1) / a.split_tokens : 0;
    ns = need < a.S ? need : a.S;
    if (ns <= 1) return;
  }
  const size_t base = ((size_t)b * a.Hq + h) * a.S;
  float M = a.sinks ? a.sinks[h] : kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_lse[base + s]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * D;
  if (M == kNegInf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) orow[lane + 64 * i] = 0;
    return;
  }
  float den = a.sinks ? __builtin_expf(a.sinks[h] - M) : 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float lse = a.part_lse[base + s];
    if (lse == kNegInf) continue;            // empty split: its o_s is never read
    const float w = __builtin_expf(lse - M);
    den += w;
    const float* o = a.part_o + (base + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += w * o[lane + 64 * i];
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[lane + 64 * i] = f32_to_bf16_bits(acc[i] * inv);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t st) {
  dim3 grid(a.Hq, B), block(64);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, st, a); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(merge_kernel<512>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace fp8pa
