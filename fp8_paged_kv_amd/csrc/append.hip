// KV append: quantize new bf16 K/V tokens to E4M3 and write them into the
// paged pools, one launch for K and V together (page "fp8 paged attention for
// MoE serving", section "Supported scope").  The encoding and the scale rules
// are in append_common.h.
//
// Grid: (page of the append span, KV head, 2*sequence + {K, V}); 256 threads.
#include "append_common.h"

namespace fp8pa {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  __shared__ float red[4];
  const int pi = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const uint16_t* xin = which ? a.v_new : a.k_new;
  uint8_t* pool = which ? a.vp : a.kp;
  const PoolGeom gm = which ? a.vg : a.kg;
  const int kind = which ? a.v_kind : a.k_kind;
  const int P = a.P, D = a.D, H = a.Hkv;

  int nb, pos0;
  if (a.positions) {
    nb = a.counts ? a.counts[b] : a.T;
    nb = nb < 0 ? 0 : (nb > a.T ? a.T : nb);
    pos0 = nb > 0 ? a.positions[b] : 0;
  } else {
    // One token per sequence at seq_lens[b] - 1 (the append + decode call).
    const int L = a.seq_lens[b];
    nb = L > 0 ? 1 : 0;
    pos0 = L - 1;
  }
  if (nb == 0) return;
  // Debug checks: positions outside the table's pages, or rows outside the
  // pools, skip the write and set an error word.
  if (a.dbg && (pos0 < 0 || (int64_t)(pos0 + nb - 1) / P >= a.bt_stride)) {
    if (threadIdx.x == 0) __hip_atomic_store(a.dbg + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int page = pos0 / P + pi;
  if (page > (pos0 + nb - 1) / P) return;
  const int lo = max(pos0, page * P), hi = min(pos0 + nb, (page + 1) * P);
  const int32_t row = a.bt[(int64_t)b * a.bt_stride + page];
  if (a.dbg && (uint32_t)row >= (uint32_t)a.dbg_rows) {
    if (threadIdx.x == 0) __hip_atomic_store(a.dbg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const uint16_t* x = xin + (((size_t)b * a.T + (lo - pos0)) * H + h) * D;   // token i at x + i*H*D
  append_page<4>(pool, gm, kind, row, h, P, D, lo, hi - lo, x, (int64_t)H * D, red);
}

__global__ void debug_dequant_kernel(const uint8_t* codes, const void* scales, int kind, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t c = codes[i];
  if (kind == 2) {
    // The decode path's K conversion with an E8M0 scale.
    const uint32_t u = reinterpret_cast<const uint8_t*>(scales)[i];
    out[i] = __builtin_bit_cast(float, e4m3x2_to_bf16x2<false>(c, e8m0_as_scale_operand(u)) << 16);
  } else if (kind >= 3) {
    // The sub-row key path's conversion: fp32(code x scale), formed before
    // the hi/lo split into bf16 operands.
    float v[8];
    scaled_e4m3x8(c, 0u, reinterpret_cast<const float*>(scales)[i], v);
    out[i] = v[0];
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
