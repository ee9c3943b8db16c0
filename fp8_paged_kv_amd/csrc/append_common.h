// Quantizing append of new K or V tokens into one page of one KV head (page
// "fp8 paged attention for MoE serving", section "Supported scope":
// per-token-per-head E4M3 with an fp32 scale or sub-row groups, and a
// one-launch append).  Shared by the append kernel (append_page: a whole
// workgroup per page and head) and the fused append + decode path
// (append_token_wave: one wave per token).
//
// Encoding of a value x with scale s: y = fp32(x / s) (IEEE division), clamped
// to +-448, rounded to the nearest E4M3 with ties to even.
// Scales:
//  * fp32 per (token, head):  s = fp32(amax / 448), 1 if amax = 0.
//  * fp32 per (token, head, S dims): each group of S dims as a per-token row.
//  * E8M0 per 32 dims:        the smallest 2**k with amax <= 448 * 2**k,
//                             stored as k + 127 clamped to [0, 254].
//  * fp32 per (page, head):   the page scale only grows.  s_old counts as 0
//    when the append writes the page's first slot; s_new = max(s_old,
//    fp32(amax_new / 448)), 1 if that is 0.  When s_new > s_old > 0 the earlier
//    tokens of the page are re-encoded from their fp32 values code x s_old.
#pragma once

#include "device_common.h"
#include "fp8pa_internal.h"

namespace fp8pa {

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }

__device__ __forceinline__ int64_t code_at(const PoolGeom& g, int t, int d) {
  return (int64_t)(t / g.tblk) * g.tblk_stride + (int64_t)(t % g.tblk) * g.tok_stride +
         (int64_t)(d >> 6) * g.dchunk_stride + (int64_t)(d & 63) * g.d_stride;
}

// Maximum over the workgroup (NW waves); red holds NW floats.
template <int NW>
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  v = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) v = fmaxf(v, red[i]);
  __syncthreads();
  return v;
}

// E8M0 code of the smallest power of two 2**k with amax <= 448 * 2**k.
__device__ __forceinline__ uint32_t e8m0_code(float amax) {
  if (amax == 0.0f) return 127u;
  int e;
  const float f = frexpf(amax, &e);          // amax = f * 2**e, f in [0.5, 1)
  int k = (f <= 0.875f) ? e - 9 : e - 8;     // 448 * 2**(e-9) = 0.875 * 2**e
  k += 127;
  return (uint32_t)(k < 0 ? 0 : (k > 254 ? 254 : k));
}

// One wave writes the token at in-page slot `slot` of KV head h in row `row`
// (x: its D bf16 values).  For page scales this is the whole append of a
// single token; for token and E8M0 scales it is one token of any append.
__device__ inline void append_token_wave(uint8_t* pool, const PoolGeom& gm, int kind, int32_t row, int h, int D,
                                         int slot, const uint16_t* x) {
  const int lane = threadIdx.x & 63;
  const RowBases rbase = row_bases(gm, row);
  uint8_t* rowp = pool + rbase.code + (int64_t)h * gm.head_stride;
  uint8_t* foot = pool + rbase.scale + (int64_t)h * gm.sc_head_stride;
  if (kind == 0) {
    float am = 0.0f;
    for (int d = lane; d < D; d += 64) am = fmaxf(am, fabsf(bf16_to_f32(x[d])));
    am = wave_max(am);
    const float s_old = slot > 0 ? *reinterpret_cast<const float*>(foot) : 0.0f;
    const float cand = am > 0.0f ? am / 448.0f : 0.0f;
    float s_new = fmaxf(s_old, cand);
    if (s_new == 0.0f) s_new = 1.0f;
    if (slot > 0 && s_old > 0.0f && s_new > s_old) {
      for (int e = lane; e < slot * D; e += 64) {
        const int t = e / D, d = e % D;
        uint8_t* c = rowp + code_at(gm, t, d);
        const float v = e4m3_to_f32(*c) * s_old;
        *c = (uint8_t)f32_to_e4m3(v / s_new);
      }
    }
    for (int d = lane; d < D; d += 64) rowp[code_at(gm, slot, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[d]) / s_new);
    if (lane == 0) *reinterpret_cast<float*>(foot) = s_new;
  } else if (kind == 1) {
    float am = 0.0f;
    for (int d = lane; d < D; d += 64) am = fmaxf(am, fabsf(bf16_to_f32(x[d])));
    am = wave_max(am);
    const float s = am > 0.0f ? am / 448.0f : 1.0f;
    for (int d = lane; d < D; d += 64) rowp[code_at(gm, slot, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[d]) / s);
    if (lane == 0) *reinterpret_cast<float*>(foot + (int64_t)slot * gm.sc_tok_stride) = s;
  } else if (kind >= 3) {
    const int S = 1 << gm.sc_gshift;
    for (int g0 = 0; g0 < D; g0 += S) {
      float am = 0.0f;
      for (int d = g0 + lane; d < g0 + S; d += 64) am = fmaxf(am, fabsf(bf16_to_f32(x[d])));
      am = wave_max(am);
      const float s = am > 0.0f ? am / 448.0f : 1.0f;
      for (int d = g0 + lane; d < g0 + S; d += 64)
        rowp[code_at(gm, slot, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[d]) / s);
      if (lane == 0)
        *reinterpret_cast<float*>(foot + (int64_t)slot * gm.sc_tok_stride + 4 * (g0 >> gm.sc_gshift)) = s;
    }
  } else {
    // lanes 0-31 / 32-63 form the 32-dim groups
    for (int d0 = 0; d0 < D; d0 += 64) {
      const int d = d0 + lane;
      const float v = bf16_to_f32(x[d]);
      float am = fabsf(v);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
      const uint32_t u = e8m0_code(am);
      const float s = __builtin_bit_cast(float, u << 23);   // 2**(u-127) for u in 1..254
      const float sv = (u == 0u) ? __builtin_ldexpf(1.0f, -127) : s;
      rowp[code_at(gm, slot, d)] = (uint8_t)f32_to_e4m3(v / sv);
      if ((lane & 31) == 0) foot[(int64_t)slot * gm.sc_tok_stride + d / 32] = (uint8_t)u;
    }
  }
}

// Write tokens lo..lo+nn-1 (all in page `page`, row `row`) of KV head h.
// x points at the first token's D bf16 values; token i is at x + i*xtok.
// kind is the pool's FP8PA_SCALE_*.  Uniform arguments across the workgroup.
template <int NW>
__device__ void append_page(uint8_t* pool, const PoolGeom& gm, int kind, int32_t row, int h, int P, int D, int lo,
                            int nn, const uint16_t* x, int64_t xtok, float* red) {
  constexpr int NT = 64 * NW;
  const int slot0 = lo % P;
  const RowBases rbase = row_bases(gm, row);
  uint8_t* rowp = pool + rbase.code + (int64_t)h * gm.head_stride;
  uint8_t* foot = pool + rbase.scale + (int64_t)h * gm.sc_head_stride;
  if (kind == 0) {
    // ---- fp32 scale per (page, head).
    float am = 0.0f;
    for (int e = threadIdx.x; e < nn * D; e += NT) am = fmaxf(am, fabsf(bf16_to_f32(x[(e / D) * xtok + (e % D)])));
    am = block_max<NW>(am, red);
    const float s_old = slot0 > 0 ? *reinterpret_cast<const float*>(foot) : 0.0f;
    const float cand = am > 0.0f ? am / 448.0f : 0.0f;
    float s_new = fmaxf(s_old, cand);
    if (s_new == 0.0f) s_new = 1.0f;
    if (slot0 > 0 && s_old > 0.0f && s_new > s_old) {
      for (int e = threadIdx.x; e < slot0 * D; e += NT) {
        const int t = e / D, d = e % D;
        uint8_t* c = rowp + code_at(gm, t, d);
        const float v = e4m3_to_f32(*c) * s_old;
        *c = (uint8_t)f32_to_e4m3(v / s_new);
      }
    }
    for (int e = threadIdx.x; e < nn * D; e += NT) {
      const int i = e / D, d = e % D;
      rowp[code_at(gm, slot0 + i, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[i * xtok + d]) / s_new);
    }
    if (threadIdx.x == 0) *reinterpret_cast<float*>(foot) = s_new;
  } else {
    // ---- per-token scales (fp32 or E8M0): one wave per token.
    for (int i = threadIdx.x >> 6; i < nn; i += NW)
      append_token_wave(pool, gm, kind, row, h, D, slot0 + i, x + i * xtok);
  }
}

}  // namespace fp8pa
