// KV append: quantize new bf16 K/V tokens to E4M3 and write them into the
// paged pools, one launch for K and V together (page "fp8 paged attention for
// MoE serving", section "Supported scope": per-token-per-head E4M3 with an fp32
// scale or sub-row groups, and a one-launch append).
//
// Encoding of a value x with scale s: y = fp32(x / s) (IEEE division), clamped
// to +-448, rounded to the nearest E4M3 with ties to even.
// Scales:
//  * fp32 per (token, head):  s = fp32(amax / 448), 1 if amax = 0.
//  * E8M0 per 32 dims:        the smallest 2**k with amax <= 448 * 2**k,
//                             stored as k + 127 clamped to [0, 254].
//  * fp32 per (page, head):   the page scale only grows.  s_old counts as 0
//    when this call writes the page's first slot; s_new = max(s_old,
//    fp32(amax_new / 448)), 1 if that is 0.  When s_new > s_old > 0 the earlier
//    tokens of the page are re-encoded from their fp32 values code x s_old.
//
// Grid: (page of the append span, KV head, 2*sequence + {K, V}); 256 threads.
#include "device_common.h"
#include "fp8pa_internal.h"

namespace fp8pa {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }

__device__ __forceinline__ int64_t code_at(const PoolGeom& g, int t, int d) {
  return (int64_t)(t / g.tblk) * g.tblk_stride + (int64_t)(t % g.tblk) * g.tok_stride +
         (int64_t)(d >> 6) * g.dchunk_stride + (int64_t)(d & 63) * g.d_stride;
}

__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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

__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  __shared__ float red[4];
  const int pi = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const uint16_t* xin = which ? a.v_new : a.k_new;
  uint8_t* pool = which ? a.vp : a.kp;
  const PoolGeom gm = which ? a.vg : a.kg;
  const int kind = which ? a.v_kind : a.k_kind;
  const int P = a.P, D = a.D, H = a.Hkv;

  int nb = a.counts ? a.counts[b] : a.T;
  nb = nb < 0 ? 0 : (nb > a.T ? a.T : nb);
  if (nb == 0) return;
  const int pos0 = a.positions[b];
  const int page = pos0 / P + pi;
  if (page > (pos0 + nb - 1) / P) return;
  const int lo = max(pos0, page * P), hi = min(pos0 + nb, (page + 1) * P);
  const int slot0 = lo - page * P, nn = hi - lo;
  const int32_t row = a.bt[(int64_t)b * a.bt_stride + page];
  const RowBases rbase = row_bases(gm, row);
  uint8_t* rowp = pool + rbase.code + (int64_t)h * gm.head_stride;
  uint8_t* foot = pool + rbase.scale + (int64_t)h * gm.sc_head_stride;
  const uint16_t* x = xin + (((size_t)b * a.T + (lo - pos0)) * H + h) * D;   // token i at x + i*H*D
  const int64_t xtok = (int64_t)H * D;

  if (kind == 0) {
    // ---- fp32 scale per (page, head).
    float am = 0.0f;
    for (int e = threadIdx.x; e < nn * D; e += blockDim.x)
      am = fmaxf(am, fabsf(bf16_to_f32(x[(e / D) * xtok + (e % D)])));
    am = block_max(am, red);
    const float s_old = slot0 > 0 ? *reinterpret_cast<const float*>(foot) : 0.0f;
    const float cand = am > 0.0f ? am / 448.0f : 0.0f;
    float s_new = fmaxf(s_old, cand);
    if (s_new == 0.0f) s_new = 1.0f;
    if (slot0 > 0 && s_old > 0.0f && s_new > s_old) {
      for (int e = threadIdx.x; e < slot0 * D; e += blockDim.x) {
        const int t = e / D, d = e % D;
        uint8_t* c = rowp + code_at(gm, t, d);
        const float v = e4m3_to_f32(*c) * s_old;
        *c = (uint8_t)f32_to_e4m3(v / s_new);
      }
    }
    for (int e = threadIdx.x; e < nn * D; e += blockDim.x) {
      const int i = e / D, d = e % D;
      rowp[code_at(gm, slot0 + i, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[i * xtok + d]) / s_new);
    }
    if (threadIdx.x == 0) *reinterpret_cast<float*>(foot) = s_new;
  } else if (kind == 1) {
    // ---- fp32 scale per (token, head): one wave per token.
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = w; i < nn; i += 4) {
      float am = 0.0f;
      for (int d = lane; d < D; d += 64) am = fmaxf(am, fabsf(bf16_to_f32(x[i * xtok + d])));
      am = wave_max(am);
      const float s = am > 0.0f ? am / 448.0f : 1.0f;
      for (int d = lane; d < D; d += 64)
        rowp[code_at(gm, slot0 + i, d)] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[i * xtok + d]) / s);
      if (lane == 0) *reinterpret_cast<float*>(foot + (int64_t)(slot0 + i) * gm.sc_tok_stride) = s;
    }
  } else {
    // ---- E8M0 per 32 dims: one wave per token; lanes 0-31 / 32-63 form groups.
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = w; i < nn; i += 4) {
      for (int d0 = 0; d0 < D; d0 += 64) {
        const int d = d0 + lane;
        const float v = bf16_to_f32(x[i * xtok + d]);
        float am = fabsf(v);
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
        const uint32_t u = e8m0_code(am);
        const float s = __builtin_bit_cast(float, u << 23);   // 2**(u-127) for u in 1..254
        const float sv = (u == 0u) ? __builtin_ldexpf(1.0f, -127) : s;
        rowp[code_at(gm, slot0 + i, d)] = (uint8_t)f32_to_e4m3(v / sv);
        if ((lane & 31) == 0) foot[(int64_t)(slot0 + i) * gm.sc_tok_stride + d / 32] = (uint8_t)u;
      }
    }
  }
}

__global__ void debug_dequant_kernel(const uint8_t* codes, const void* scales, int kind, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t c = codes[i];
  if (kind == 2) {
    // The decode path's K conversion with an E8M0 scale.
    const uint32_t u = reinterpret_cast<const uint8_t*>(scales)[i];
    out[i] = __builtin_bit_cast(float, e4m3x2_to_bf16x2<false>(c, e8m0_as_scale_operand(u)) << 16);
  } else {
    // The decode path's conversion, then the fp32 scale.
    const float v = __builtin_bit_cast(float, e4m3x2_to_bf16x2<false>(c, 1.0f) << 16);
    out[i] = v * reinterpret_cast<const float*>(scales)[i];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int B, int max_pages, hipStream_t st) {
  dim3 grid(max_pages, a.Hkv, 2 * B), block(256);
  hipLaunchKernelGGL(append_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_debug_dequant(const uint8_t* codes, const void* scales, int kind, int n, float* out,
                                hipStream_t st) {
  dim3 grid((n + 255) / 256), block(256);
  hipLaunchKernelGGL(debug_dequant_kernel, grid, block, 0, st, codes, scales, kind, n, out);
  return hipGetLastError();
}

}  // namespace fp8pa
