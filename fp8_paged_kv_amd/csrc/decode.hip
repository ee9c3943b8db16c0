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
// workgroup is four wave64s; each wave walks every fourth tile of the split
// with an independent online softmax, and the four partial states are combined
// in LDS at the end.  The block-table entries of the split are staged in LDS
// once, and each wave double-buffers its tiles in registers: the loads of its
// next tile are in flight while it computes the current one.
//
// Splits.  When a sequence spans more than one split, each split writes a
// normalised partial and its log-sum-exp to the workspace, and the last split
// of a (sequence, KV head) to arrive merges them and writes the output (the
// standard log-sum-exp combination; the sink enters once).  Arrival counters
// carry the call's epoch in their upper half, so a workspace needs no
// initialisation, and the last arriver resets the count so a replayed graph
// (same epoch) starts from zero again.
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
#include <hip/hip_ext.h>

#include "device_common.h"
#include "fp8pa_internal.h"
#include "merge_common.h"

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

// The D/32 E8M0 bytes of one position (one 32-dim group each), zero-extended
// into a u32x4.
template <int NG>
__device__ __forceinline__ u32x4 load_e8_row(const uint8_t* p) {
  if constexpr (NG == 2) return u32x4{(uint32_t)ld_global<uint16_t>(p), 0, 0, 0};
  else if constexpr (NG == 4) return u32x4{ld_global<uint32_t>(p), 0, 0, 0};
  else if constexpr (NG == 8) { const u32x2 v = ld_global<u32x2>(p); return u32x4{v[0], v[1], 0, 0}; }
  else return ld_global<u32x4>(p);
}

__device__ __forceinline__ uint32_t byte_of(const u32x4& v, int i) { return (v[i >> 2] >> (8 * (i & 3))) & 0xffu; }

// Registers of one tile for one lane.
template <int D, int NS, int SK>
struct Tile {
  static constexpr int NM = D / 64, NC = D / 16, NG = D / 32, NE = (8 * NG) / 16;
  typedef typename VRaw<NS>::type vraw_t;
  u32x4 k[NS][2][NM];   // K codes of the lane's position rows
  vraw_t v[NC];         // V codes of the lane's dims, GT positions each
  float ks, vs;         // per-(page, head) scales of the lane's score group
  float kst[NS][8];     // per-(token, head) scales of the lane's score positions
  float vst[NS][8];
  u32x4 ke8[NS][2];     // E8M0 bytes of the lane's K rows
  u32x4 ve8[NS][NE];    // E8M0 bytes of the lane's 8 score positions, all groups
};

template <int D, int NS, int SK, bool PF, int OCC, bool KNT>
__global__ __launch_bounds__(256, OCC) void decode_kernel(const DecodeArgs a) {
  constexpr int TT = 32 * NS;   // positions per tile
  constexpr int GT = 8 * NS;    // positions per group
  constexpr int NM = D / 64;    // 16-byte K pieces per position row per lane
  constexpr int NQ = D / 32;    // QK MFMAs per 16 positions
  constexpr int NC = D / 16;    // PV MFMAs per subtile (16 dims each)
  constexpr int NG = D / 32;    // E8M0 groups along D
  typedef Tile<D, NS, SK> TileT;

  extern __shared__ float s_dyn[];   // staged block table, later the wave-combine buffer
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;      // MFMA column: query head of the group
  const int quad = lane >> 4;   // MFMA k/row quad
  // Workgroup -> (KV head, sequence, split), KV head fastest and split
  // slowest.  Workgroups are dispatched to the eight XCDs round-robin by id,
  // so every XCD receives the same share of every sequence (grouping a
  // sequence's heads on one XCD to share scale-footer lines in its L2 was
  // measured slower: per-XCD work then follows a few sequence lengths), and
  // the short last splits of long sequences are dispatched last.
  const int id = blockIdx.x;
  const int g = id % a.Hkv;
  const int unit = id / a.Hkv;
  const int split = unit / a.B, b = unit - split * a.B;
  const int G = a.G, P = a.P, log2P = a.log2P;

  const int L = a.seq_lens[b];
  int start, tbeg, nsplit;
  split_range(L, a.window, TT, a.split_tokens, a.S, start, tbeg, nsplit);
  if (split >= (nsplit > 1 ? nsplit : 1)) return;
  const int r0 = tbeg + split * a.split_tokens;
  const int r1 = (split == nsplit - 1 || nsplit <= 1) ? L : min(L, r0 + a.split_tokens);
  const int ntiles = (r1 > r0) ? (r1 - r0 + TT - 1) / TT : 0;

  // ---- stage the block-table rows of the split's attended pages in LDS.
  const int32_t* btr = a.bt + (int64_t)b * a.bt_stride;
  int* s_tab = reinterpret_cast<int*>(s_dyn);
  const int p_first = (r0 > start ? r0 : start) >> log2P;
  const int n_pages = ntiles > 0 ? ((r1 - 1) >> log2P) - p_first + 1 : 0;
  const int nstaged = n_pages;   // the host sizes the stage for the longest split
  for (int i = threadIdx.x; i < nstaged; i += 256) s_tab[i] = btr[p_first + i];

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
  __syncthreads();

  const uint8_t* kpool = a.kp + (int64_t)g * a.kg.head_stride;
  const uint8_t* vpool = a.vp + (int64_t)g * a.vg.head_stride;
  const int kgrp = n >> 2;      // group of this lane's K row
  const int kslot = n & 3;

  // Row of a page of this split.  A group with no attended position reads a
  // clamped (attended) page instead: its scores are masked to -inf and its V
  // bytes zeroed, so every lane issues the same loads and the compiler can
  // count outstanding loads exactly across the prefetch.
  auto row_of = [&](int page) -> int32_t {
    int i = page - p_first;
    i = i < 0 ? 0 : (i >= nstaged ? nstaged - 1 : i);
    return s_tab[i];
  };

  // ---- issue the loads of one tile: scales first, then the K and V codes, so
  // that the large code loads are the most recent ones in flight (a later
  // wait for a scale, or for the reuse of a scale's register, then leaves
  // them outstanding).
  auto load_tile = [&](TileT& t, int T0) {
    const int tk = T0 + GT * kgrp;   // first position of the lane's K group
    const int tq = T0 + GT * quad;   // first position of the lane's score/V group
    const int32_t row_k = row_of(tk >> log2P);
    const int32_t row_q = row_of(tq >> log2P);
    const int tpq = tq & (P - 1);
    const uint8_t* ksc = a.kp + (int64_t)row_q * a.kg.row_bytes + a.kg.sc_off + g * a.kg.sc_head_stride;
    const uint8_t* vsc = a.vp + (int64_t)row_q * a.vg.row_bytes + a.vg.sc_off + g * a.vg.sc_head_stride;
    if constexpr (SK == 0) {
      t.ks = ld_global<float>(ksc);
      t.vs = ld_global<float>(vsc);
    } else if constexpr (SK == 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tt = tpq + 8 * s + i;
          t.kst[s][i] = ld_global<float>(ksc + tt * a.kg.sc_tok_stride);
          t.vst[s][i] = ld_global<float>(vsc + tt * a.vg.sc_tok_stride);
        }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint8_t* src = vsc + (tpq + 8 * s) * a.vg.sc_tok_stride;
#pragma unroll
        for (int k = 0; k < TileT::NE; ++k) t.ve8[s][k] = ld_global<u32x4>(src + 16 * k);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const int tp = (tk + 8 * s + 4 * aa + kslot) & (P - 1);
          const uint8_t* kf = a.kp + (int64_t)row_k * a.kg.row_bytes + a.kg.sc_off + g * a.kg.sc_head_stride +
                              tp * a.kg.sc_tok_stride;
          t.ke8[s][aa] = load_e8_row<NG>(kf);
        }
    }
    const uint8_t* krow = kpool + (int64_t)row_k * a.kg.row_bytes + 16 * quad;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        const int tp = (tk + 8 * s + 4 * aa + kslot) & (P - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const uint8_t* src = krow + tp * a.kg.tok_stride + m * a.kg.dchunk_stride;
          t.k[s][aa][m] = KNT ? ld_stream<u32x4>(src) : ld_global<u32x4>(src);
        }
      }
    // The lane's GT positions lie in one token block of the d-major V layout.
    const uint8_t* vrow = vpool + (int64_t)row_q * a.vg.row_bytes + (int64_t)(tpq / a.vg.tblk) * a.vg.tblk_stride +
                          (tpq % a.vg.tblk);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d = 16 * c + n;
      t.v[c] = ld_stream<typename TileT::vraw_t>(vrow + (int64_t)(d >> 6) * a.vg.dchunk_stride +
                                                 (int64_t)(d & 63) * a.vg.d_stride);
    }
  };

  float m_run = kNegInf;        // running max (log2 units) of this lane's head column
  float l_run = 0.0f;           // this lane's share of the running sum
  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- online-softmax update with one tile.
  auto compute_tile = [&](TileT& t, int T0) {
    const bool interior = (T0 >= start) && (T0 + TT <= L);
    float sc[NS][2][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          float cvt = 1.0f;
          if constexpr (SK == 2) {
            const uint32_t e = byte_of(t.ke8[s][aa], 2 * m + (quad >> 1));
            cvt = e8m0_as_scale_operand(e);
          }
          const u32x4 w = t.k[s][aa][m];
          s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[0], w[1], cvt), qop[2 * m], s4);
          s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[2], w[3], cvt), qop[2 * m + 1], s4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float f = a.qk_scale;
          if constexpr (SK == 0) f *= t.ks;
          if constexpr (SK == 1) f *= t.kst[s][4 * aa + j];
          sc[s][aa][j] = s4[j] * f;
        }
      }
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
    if (!interior) {
      const int base = T0 + GT * quad;
      const int lo = start - base, hi = L - base;   // keep bytes in [lo, hi)
#pragma unroll
      for (int k = 0; k < GT / 4; ++k) {
        uint32_t mk = 0;
#pragma unroll
        for (int byte = 0; byte < 4; ++byte) {
          const int bi = 4 * k + byte;
          if (bi >= lo && bi < hi) mk |= 0xffu << (8 * byte);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) t.v[c][k] &= mk;
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (SK == 2) {
        bf16x8 pop[NG];
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) {
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int bi = i * NG + gq;
            const int ex = (int)byte_of(t.ve8[s][bi >> 4], bi & 15) - 127;
            const float x = __builtin_amdgcn_ldexpf(p[s][i], ex);
            pv[i] = (p[s][i] == 0.0f) ? 0.0f : x;
          }
          u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                      pack_bf16x2(pv[6], pv[7])};
          pop[gq] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(t.v[c][2 * s], t.v[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop[c >> 1], acc[c]);
        }
      } else {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float vsc = 1.0f;
          if constexpr (SK == 0) vsc = t.vs;
          if constexpr (SK == 1) vsc = t.vst[s][i];
          pv[i] = (p[s][i] == 0.0f) ? 0.0f : p[s][i] * vsc;
        }
        u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                    pack_bf16x2(pv[6], pv[7])};
        const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(t.v[c][2 * s], t.v[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop, acc[c]);
        }
      }
    }
  };

  // ---- tile loop: wave w takes tiles w, w+4, ...
  {
    const int nmine = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
    auto tile_pos = [&](int k) { return r0 + (wave + kWaves * k) * TT; };
    if constexpr (PF) {
      // Loads run one tile ahead, ping-ponging two register buffers.  The trip
      // count is fixed and loads are unconditional (a prefetch past the last
      // tile re-reads a cache-hot tile), so the waits before each compute
      // cover only that tile's loads.
      TileT A, B;
      if (nmine > 0) load_tile(A, tile_pos(0));
      const int npairs = nmine / 2;
      for (int k = 0; k < npairs; ++k) {
        load_tile(B, tile_pos(2 * k + 1));
        compute_tile(A, tile_pos(2 * k));
        load_tile(A, tile_pos(2 * k + 2 < nmine ? 2 * k + 2 : 2 * k + 1));
        compute_tile(B, tile_pos(2 * k + 1));
      }
      if (nmine & 1) compute_tile(A, tile_pos(nmine - 1));
    } else {
      TileT A;
      for (int k = 0; k < nmine; ++k) {
        load_tile(A, tile_pos(k));
        compute_tile(A, tile_pos(k));
      }
    }
  }

  // ---- combine the four waves' states in LDS.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* s_o = s_dyn;   // [2][G][D + 4]; the staged table is no longer read after the barrier
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
  if (wave == 0 && col) {
    const float* src = s_o + n * OS + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] += *reinterpret_cast<const f32x4*>(src + 16 * c);
  }

  const int h = g * G + n;
  if (nsplit <= 1) {
    if (wave != 0 || !col) return;
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
    return;
  }

  // ---- partial of this split, then arrival; the last split merges.
  // Partials are written and read with agent-scope atomic accesses, which on
  // this multi-XCD part are coherent across the per-XCD L2 caches without a
  // cache write-back or invalidate; the barrier waits for the stores to
  // complete before the arrival is counted.
  if (wave == 0 && col) {
    const size_t ph = ((size_t)b * a.Hq + h) * a.S + split;
    const float inv = (Ltot > 0.0f) ? 1.0f / Ltot : 0.0f;
    float* orow = a.part_o + ph * D + 4 * quad;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __hip_atomic_store(orow + 16 * c + j, acc[c][j] * inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (quad == 0)
      __hip_atomic_store(a.part_lse + ph,
                         (M == kNegInf || !(Ltot > 0.0f)) ? kNegInf : (M + __builtin_amdgcn_logf(Ltot)) * kLn2,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!a.fused_merge) return;   // a separate merge kernel combines the partials
  if (threadIdx.x == 0) {
    // Wave 0 wrote the partials; wait until its stores have completed at the
    // coherence point before counting this split as arrived.
    __builtin_amdgcn_s_waitcnt(0);
    unsigned long long* cnt = a.counters + ((size_t)b * a.Hkv + g);
    const unsigned long long tag = (unsigned long long)a.epoch << 32;
    unsigned long long old = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned int arrived;
    while (true) {
      arrived = ((old >> 32) == a.epoch) ? (unsigned int)(old & 0xffffffffu) : 0u;
      unsigned long long want = tag | (unsigned long long)(arrived + 1);
      if (__hip_atomic_compare_exchange_strong(cnt, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        break;
    }
    const bool last = (int)(arrived + 1) == nsplit;
    if (last) __hip_atomic_store(cnt, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __shared__ float s_inv[16];
  merge_heads<D, true>(a.part_o, a.part_lse, a.sinks, a.out, b, a.Hq, a.S, g * G, G, nsplit, s_dyn, s_inv);
}

template <int D, int NS, bool PF, int OCC, bool KNT>
hipError_t launch_d(const DecodeArgs& a, int sk, int B, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  dim3 grid(a.S * B * a.Hkv), block(256);
  size_t lds = (size_t)2 * a.G * (D + 4) * sizeof(float);                                     // wave combine
  lds = lds > (size_t)a.max_staged * sizeof(int) ? lds : (size_t)a.max_staged * sizeof(int);   // table
  lds = lds > (size_t)a.G * a.S * sizeof(float) ? lds : (size_t)a.G * a.S * sizeof(float);     // merge
  switch (sk) {
    case 0: hipExtLaunchKernelGGL((decode_kernel<D, NS, 0, PF, OCC, KNT>), grid, block, lds, st, e0, e1, 0, a); break;
    case 1: hipExtLaunchKernelGGL((decode_kernel<D, NS, 1, PF, OCC, KNT>), grid, block, lds, st, e0, e1, 0, a); break;
    default: hipExtLaunchKernelGGL((decode_kernel<D, NS, 2, PF, OCC, KNT>), grid, block, lds, st, e0, e1, 0, a); break;
  }
  return hipGetLastError();
}

template <bool KNT>
hipError_t launch_k(const DecodeArgs& a, int D, int sk, int B, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  // tile_variant (tuning): 0 default, 1 prefetch at one wave per SIMD,
  // 2 prefetch with 32-position tiles (D = 128), 3 no prefetch, 4 prefetch.
  const int v = a.tile_variant;
  switch (D) {
    case 64:
      return v == 4 ? launch_d<64, 2, true, 2, KNT>(a, sk, B, st, e0, e1)
                    : launch_d<64, 2, false, 2, KNT>(a, sk, B, st, e0, e1);
    case 128:
      switch (v) {
        case 1: return launch_d<128, 2, true, 1, KNT>(a, sk, B, st, e0, e1);
        case 2: return launch_d<128, 1, true, 2, KNT>(a, sk, B, st, e0, e1);
        case 4: return launch_d<128, 2, true, 2, KNT>(a, sk, B, st, e0, e1);
        default: return launch_d<128, 2, false, 2, KNT>(a, sk, B, st, e0, e1);
      }
    case 256:
      return v == 4 ? launch_d<256, 1, true, 1, KNT>(a, sk, B, st, e0, e1)
                    : launch_d<256, 1, false, 1, KNT>(a, sk, B, st, e0, e1);
    default: return launch_d<512, 1, false, 1, KNT>(a, sk, B, st, e0, e1);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int B, hipStream_t st,
                         hipEvent_t e0, hipEvent_t e1) {
  return k_whole_lines ? launch_k<true>(a, D, scale_kind, B, st, e0, e1)
                       : launch_k<false>(a, D, scale_kind, B, st, e0, e1);
}

}  // namespace fp8pa
