// The log-sum-exp merge of split partials (standalone merge kernel).
//
// The pages split each sequence so the whole chip is busy (page "fp8 paged
// attention for MoE serving", section "Why it happens") but do not print how
// the partial results are combined; the reading taken is the standard one:
// split s carries o_s (normalised) and lse_s (natural-log sum of exp of its
// scores); with M = max(max_s lse_s, sink),
//   o = sum_s e^(lse_s - M) o_s / (sum_s e^(lse_s - M) + e^(sink - M)).
// An lse of -inf marks an empty split, whose o_s is never used.
#pragma once

#include "device_common.h"

namespace fp8pa {

template <bool COHERENT>
__device__ __forceinline__ float ld_part(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Merges the nsplit partials of query heads [h0, h0 + G) of sequence b and
// writes their bf16 outputs.  Called by every thread of the block; s_w holds
// G * nsplit floats and s_inv G floats of LDS.  COHERENT loads are coherent
// across the per-XCD L2 caches (partials written by other workgroups of the
// same launch).
template <int D, bool COHERENT>
__device__ void merge_heads(const float* part_o, const float* part_lse, const float* sinks, uint16_t* out,
                            int b, int Hq, int S, int h0, int G, int nsplit, float* s_w, float* s_inv) {
  constexpr float kNegInf = -__builtin_inff();
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < G * nsplit; i += nt) {
    const int h = i / nsplit, s = i - h * nsplit;
    s_w[i] = ld_part<COHERENT>(part_lse + ((size_t)b * Hq + h0 + h) * S + s);
  }
  __syncthreads();
  for (int h = tid; h < G; h += nt) {
    const float sink = sinks ? sinks[h0 + h] : kNegInf;
    float M = sink;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, s_w[h * nsplit + s]);
    float den = (sinks && M != kNegInf) ? __builtin_expf(sink - M) : 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float lse = s_w[h * nsplit + s];
      const float w = (lse == kNegInf || M == kNegInf) ? 0.0f : __builtin_expf(lse - M);
      s_w[h * nsplit + s] = w;
      den += w;
    }
    s_inv[h] = (M == kNegInf || !(den > 0.0f)) ? 0.0f : 1.0f / den;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += nt) {
    const int h = idx / D, d = idx - h * D;
    const float* o = part_o + ((size_t)b * Hq + h0 + h) * S * D + d;
    const float* w = s_w + h * nsplit;
    float num = 0.0f;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      const float o0 = ld_part<COHERENT>(o + (size_t)s * D), o1 = ld_part<COHERENT>(o + (size_t)(s + 1) * D);
      const float o2 = ld_part<COHERENT>(o + (size_t)(s + 2) * D), o3 = ld_part<COHERENT>(o + (size_t)(s + 3) * D);
      num += (w[s] > 0.0f ? w[s] * o0 : 0.0f) + (w[s + 1] > 0.0f ? w[s + 1] * o1 : 0.0f);
      num += (w[s + 2] > 0.0f ? w[s + 2] * o2 : 0.0f) + (w[s + 3] > 0.0f ? w[s + 3] * o3 : 0.0f);
    }
    for (; s < nsplit; ++s) {
      const float os = ld_part<COHERENT>(o + (size_t)s * D);
      num += w[s] > 0.0f ? w[s] * os : 0.0f;
    }
    out[((size_t)b * Hq + h0 + h) * D + d] = f32_to_bf16_bits(num * s_inv[h]);
  }
}

}  // namespace fp8pa
