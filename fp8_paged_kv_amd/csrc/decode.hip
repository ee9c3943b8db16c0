// Paged flash-decode over an E4M3 KV cache for gfx950.
//
// Operation (page "fp8 paged attention for MoE serving", "Smallest correct
// example" and "Expected result"): for sequence b, KV head g and the G query
// heads that share it, attend over the positions [start, L) of the sequence
// through its block table, with E4M3 K/V dequantized as code x scale, a custom
// sm_scale, and an optional per-head sink logit in the denominator.
//
// Work decomposition.  The grid runs over (split, KV head, sequence) so the
// GQA group shares every K/V read (page section "Why it happens").  A
// workgroup is four wave64s; each wave walks its own tiles of the split with
// an independent online softmax, and the four partial states are combined in
// LDS at the end.  A split with more than one split per sequence writes a
// normalised partial and its log-sum-exp for the merge kernel.
//
// Tile = 32*NS positions = four groups of 8*NS consecutive positions; a group
// never crosses a page (P >= 16 and tiles are aligned to their size).
//
// QK^T on MFMA 16x16x32 bf16: A = 16 K rows (positions), B = Q^T (the G query
// heads in columns, zero-padded to 16), K-dim = head dims.  Lane l of the A
// operand holds position row l%16 and eight dims; the dims a lane holds are
// chosen so that it reads 16 contiguous bytes of its position's row per 64
// dims (the dot product does not care which dims share an MFMA as long as Q
// uses the same assignment).  The rows are assigned to positions so that the
// C layout (lane holds rows 4*(l/16)..+3 of column l%16) leaves each lane with
// exactly the probabilities it must supply to the PV MFMA.
//
// PV on MFMA 16x16x32 bf16: O^T = V^T P^T with A = V^T (16 head dims x 32
// positions) and B = P^T.  V is stored d-major per (page, head), so lane
// (dim l%16, quad l/16) loads the 8*NS positions it needs as one 16-byte (or
// 8-byte) load straight from HBM; no LDS transpose is needed.
//
// Scales.  fp32 per (page, head) or per (token, head): the K scale multiplies
// the score after the dot product and the V scale multiplies the probability
// before the PV product (both are exact reassociations of code x scale).
// E8M0 per 32 dims: the K scale is applied inside the E4M3 -> bf16 conversion
// (a power of two, exact); the V scale varies along the dims, so the PV B
// operand is built once per 32-dim group with p x 2**(e - 127).
//
// Masked positions (outside [start, L): the tail of the last page, positions
// before the window) get a score of -inf by selection and their V bytes are
// zeroed, so NaN codes or scales there never reach the output.  Pages with no
// attended position are never looked up in the block table.
#include "device_common.h"
#include "fp8pa_internal.h"

namespace fp8pa {
namespace {

constexpr int kWaves = 4;
constexpr float kNegInf = -__builtin_inff();

template <int NS>
struct VRaw;
template <>
struct VRaw<1> { typedef u32x2 type; };
template <>
struct VRaw<2> { typedef u32x4 type; };

// Split bookkeeping shared with the merge kernel: the first tile-aligned
// position, the number of splits that hold attended positions.
__device__ __forceinline__ void split_range(int L, int window, int tile, int split_tokens, int S,
                                            int& start, int& tbeg, int& nsplit) {
  start = (window > 0 && L > window) ? L - window : 0;
  tbeg = start & ~(tile - 1);
  int need = (L > start) ? (L - tbeg + split_tokens - 1) / split_tokens : 0;
  nsplit = need < S ? need : S;
}

template <int D, int NS, int SK>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int TT = 32 * NS;   // positions per tile
  constexpr int GT = 8 * NS;    // positions per group
  constexpr int NM = D / 64;    // 16-byte K pieces per position row per lane
  constexpr int NQ = D / 32;    // QK MFMAs per 16 positions
  constexpr int NC = D / 16;    // PV MFMAs per subtile (16 dims each)
  constexpr int NG = D / 32;    // E8M0 groups along D
  typedef typename VRaw<NS>::type vraw_t;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;      // MFMA column: query head of the group
  const int quad = lane >> 4;   // MFMA k/row quad
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, P = a.P;

  const int L = a.seq_lens[b];
  int start, tbeg, nsplit;
  split_range(L, a.window, TT, a.split_tokens, a.S, start, tbeg, nsplit);
  if (split >= (nsplit > 1 ? nsplit : 1)) return;
  const int r0 = tbeg + split * a.split_tokens;
  const int r1 = (split == nsplit - 1 || nsplit <= 1) ? L : min(L, r0 + a.split_tokens);
  const int ntiles = (r1 > r0) ? (r1 - r0 + TT - 1) / TT : 0;

  // ---- Q operand (B of QK): lane (head n, quad) holds dims 64m + 16quad + 8h2 + i.
  bf16x8 qop[NQ];
  {
    const bool has = n < G;
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)g * G + (has ? n : 0)) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 v = has ? ld_global<u32x4>(qrow + 64 * m + 16 * quad + 8 * h2) : u32x4{0, 0, 0, 0};
        qop[2 * m + h2] = __builtin_bit_cast(bf16x8, v);
      }
  }

  const int32_t* btr = a.bt + (int64_t)b * a.bt_stride;
  const uint8_t* kpool = a.kp + (int64_t)g * a.kg.head_stride;
  const uint8_t* vpool = a.vp + (int64_t)g * a.vg.head_stride;
  const int kgrp = n >> 2;      // group of this lane's K row
  const int kslot = n & 3;

  float m_run = kNegInf;        // running max (log2 units) of this lane's head column
  float l_run = 0.0f;           // this lane's share of the running sum
  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = wave; it < ntiles; it += kWaves) {
    const int T0 = r0 + it * TT;
    const bool interior = (T0 >= start) && (T0 + TT <= L);

    // Rows of the four groups (wave-uniform); a group with no attended
    // position is not looked up.
    int32_t row[4];
    bool gval[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int t0 = T0 + gi * GT;
      gval[gi] = (t0 + GT > start) && (t0 < L);
      row[gi] = gval[gi] ? btr[t0 >> a.log2P] : 0;
    }
    const int32_t row_k = kgrp == 0 ? row[0] : kgrp == 1 ? row[1] : kgrp == 2 ? row[2] : row[3];
    const bool val_k = kgrp == 0 ? gval[0] : kgrp == 1 ? gval[1] : kgrp == 2 ? gval[2] : gval[3];
    const int32_t row_q = quad == 0 ? row[0] : quad == 1 ? row[1] : quad == 2 ? row[2] : row[3];
    const bool val_q = quad == 0 ? gval[0] : quad == 1 ? gval[1] : quad == 2 ? gval[2] : gval[3];

    // ---- K loads: lane row = position GT*kgrp + 8s + 4aa + kslot of the tile.
    u32x4 kraw[NS][2][NM];
    const uint8_t* krow = kpool + (int64_t)row_k * a.kg.row_bytes + 16 * quad;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        const int tp = (T0 + GT * kgrp + 8 * s + 4 * aa + kslot) & (P - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m)
          kraw[s][aa][m] = val_k ? ld_global<u32x4>(krow + tp * a.kg.tok_stride + 64 * m) : u32x4{0, 0, 0, 0};
      }

    // ---- V loads: lane (dim n of chunk c, quad) holds positions GT*quad + [0, GT).
    vraw_t vraw[NC];
    {
      const int tp = (T0 + GT * quad) & (P - 1);
      const uint8_t* vrow = vpool + (int64_t)row_q * a.vg.row_bytes + (int64_t)n * a.vg.d_stride + tp;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        vraw_t z = {};
        vraw[c] = val_q ? ld_global<vraw_t>(vrow + (int64_t)16 * c * a.vg.d_stride) : z;
      }
    }

    // ---- scales for this lane's score positions (group `quad`).
    const uint8_t* ksc = a.kp + (int64_t)row_q * a.kg.row_bytes + a.kg.sc_off + g * a.kg.sc_head_stride;
    const uint8_t* vsc = a.vp + (int64_t)row_q * a.vg.row_bytes + a.vg.sc_off + g * a.vg.sc_head_stride;
    const int tq = (T0 + GT * quad) & (P - 1);   // in-page slot of the group's first position
    float kscale[NS][2][4];
    float vscale[NS][8];
    if constexpr (SK == 0) {
      const float ks = val_q ? ld_global<float>(ksc) : 0.0f;
      const float vs = val_q ? ld_global<float>(vsc) : 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { kscale[s][0][i] = ks; kscale[s][1][i] = ks; }
#pragma unroll
        for (int i = 0; i < 8; ++i) vscale[s][i] = vs;
      }
    } else if constexpr (SK == 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = tq + 8 * s + i;
          kscale[s][i >> 2][i & 3] = val_q ? ld_global<float>(ksc + t * a.kg.sc_tok_stride) : 0.0f;
          vscale[s][i] = val_q ? ld_global<float>(vsc + t * a.vg.sc_tok_stride) : 0.0f;
        }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) { kscale[s][i >> 2][i & 3] = 1.0f; vscale[s][i] = 1.0f; }
    }

    // ---- S = K Q^T for the 16 position rows of each (subtile s, half aa).
    float sc[NS][2][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        float cvt[NM];
        if constexpr (SK == 2) {
          // E8M0 scale of this lane's K row for the 32-dim group 2m + quad/2.
          const int tp = (T0 + GT * kgrp + 8 * s + 4 * aa + kslot) & (P - 1);
          const uint8_t* kfoot = a.kp + (int64_t)row_k * a.kg.row_bytes + a.kg.sc_off +
                                 g * a.kg.sc_head_stride + tp * a.kg.sc_tok_stride;
#pragma unroll
          for (int m = 0; m < NM; ++m)
            cvt[m] = e8m0_as_scale_operand(val_k ? (uint32_t)kfoot[2 * m + (quad >> 1)] : 127u);
        } else {
#pragma unroll
          for (int m = 0; m < NM; ++m) cvt[m] = 1.0f;
        }
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const u32x4 w = kraw[s][aa][m];
          s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[0], w[1], cvt[m]), qop[2 * m], s4);
          s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[2], w[3], cvt[m]), qop[2 * m + 1], s4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[s][aa][j] = s4[j] * (kscale[s][aa][j] * a.qk_scale);
      }

    // ---- mask positions outside [start, L) (boundary tiles only).
    if (!interior) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int pos = T0 + GT * quad + 8 * s + 4 * aa + j;
            if (pos < start || pos >= L) sc[s][aa][j] = kNegInf;
          }
    }

    // ---- online softmax (log2 domain) for this lane's head column.
    float tmax = kNegInf;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, sc[s][aa][j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    m_run = m_new;
    float psum = 0.0f;
    float p[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(sc[s][i >> 2][i & 3] - m_ref);
        psum += e;
        p[s][i] = e;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= alpha;

    // ---- V bytes of masked positions are zeroed (boundary tiles only).
    if (!interior) {
      const int base = T0 + GT * quad;
      const int lo = start - base, hi = L - base;   // keep bytes in [lo, hi)
      uint32_t keep[GT / 4];
#pragma unroll
      for (int k = 0; k < GT / 4; ++k) {
        uint32_t mk = 0;
#pragma unroll
        for (int byte = 0; byte < 4; ++byte) {
          const int bi = 4 * k + byte;
          if (bi >= lo && bi < hi) mk |= 0xffu << (8 * byte);
        }
        keep[k] = mk;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < GT / 4; ++k) vraw[c][k] &= keep[k];
    }

    // ---- O^T += V^T P^T.
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (SK == 2) {
        // V scale per (position, 32-dim group): one B operand per group.
        const uint8_t* vfoot = a.vp + (int64_t)row_q * a.vg.row_bytes + a.vg.sc_off + g * a.vg.sc_head_stride;
        const int t8 = tq + 8 * s;
        constexpr int NE = (8 * NG) / 16;
        u32x4 e8[NE];      // byte i*NG + gq: position t8 + i, 32-dim group gq
        {
          const uint8_t* src = vfoot + t8 * a.vg.sc_tok_stride;
#pragma unroll
          for (int k = 0; k < NE; ++k) e8[k] = val_q ? ld_global<u32x4>(src + 16 * k) : u32x4{0, 0, 0, 0};
        }
        bf16x8 pop[NG];
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) {
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int bi = i * NG + gq;
            const int ex = (int)((e8[bi >> 4][(bi >> 2) & 3] >> (8 * (bi & 3))) & 0xffu) - 127;
            const float x = __builtin_amdgcn_ldexpf(p[s][i], ex);
            pv[i] = (p[s][i] == 0.0f) ? 0.0f : x;
          }
          u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                      pack_bf16x2(pv[6], pv[7])};
          pop[gq] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(vraw[c][2 * s], vraw[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop[c >> 1], acc[c]);
        }
      } else {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = (p[s][i] == 0.0f) ? 0.0f : p[s][i] * vscale[s][i];
        u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                    pack_bf16x2(pv[6], pv[7])};
        const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(vraw[c][2 * s], vraw[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop, acc[c]);
        }
      }
    }
  }

  // ---- combine the four waves' states in LDS.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  extern __shared__ float s_o[];   // [2][G][D + 4]
  constexpr int OS = D + 4;
  if (quad == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_run;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][n]);
  const float M_ref = (M == kNegInf) ? 0.0f : M;
  float Ltot = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Ltot += s_l[w][n] * __builtin_amdgcn_exp2f(s_m[w][n] - M_ref);
  {
    const float f = __builtin_amdgcn_exp2f(m_run - M_ref);
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= f;
  }
  const bool col = n < G;
  if (wave >= 2 && col) {
    float* dst = s_o + ((wave - 2) * G + n) * OS + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c) = acc[c];
  }
  __syncthreads();
  if (wave < 2 && col) {
    const float* src = s_o + (wave * G + n) * OS + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] += *reinterpret_cast<const f32x4*>(src + 16 * c);
  }
  __syncthreads();
  if (wave == 1 && col) {
    float* dst = s_o + n * OS + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c) = acc[c];
  }
  __syncthreads();
  if (wave != 0 || !col) return;
  {
    const float* src = s_o + n * OS + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] += *reinterpret_cast<const f32x4*>(src + 16 * c);
  }

  const int h = g * G + n;
  if (nsplit <= 1) {
    // Final output: o = acc / (sum + e^(sink - max)), sink in log2 units.
    float den = Ltot;
    if (a.sinks) den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - M_ref);
    const float inv = (M == kNegInf || !(den > 0.0f)) ? 0.0f : 1.0f / den;
    uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * D + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x2 pk = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv), pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * c) = pk;
    }
  } else {
    const size_t ph = ((size_t)b * a.Hq + h) * a.S + split;
    const float inv = (Ltot > 0.0f) ? 1.0f / Ltot : 0.0f;
    float* orow = a.part_o + ph * D + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(orow + 16 * c) = acc[c] * inv;
    if (quad == 0)
      a.part_lse[ph] = (M == kNegInf || !(Ltot > 0.0f)) ? kNegInf : (M + __builtin_amdgcn_logf(Ltot)) * kLn2;
  }
}

template <int D, int NS>
hipError_t launch_d(const DecodeArgs& a, int sk, int B, hipStream_t st) {
  dim3 grid(a.S, a.Hkv, B), block(256);
  const size_t lds = (size_t)2 * a.G * (D + 4) * sizeof(float);
  switch (sk) {
    case 0: hipLaunchKernelGGL((decode_kernel<D, NS, 0>), grid, block, lds, st, a); break;
    case 1: hipLaunchKernelGGL((decode_kernel<D, NS, 1>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((decode_kernel<D, NS, 2>), grid, block, lds, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, int B, hipStream_t st) {
  switch (D) {
    case 64: return launch_d<64, 2>(a, scale_kind, B, st);
    case 128: return launch_d<128, 2>(a, scale_kind, B, st);
    case 256: return launch_d<256, 1>(a, scale_kind, B, st);
    default: return launch_d<512, 1>(a, scale_kind, B, st);
  }
}

}  // namespace fp8pa
