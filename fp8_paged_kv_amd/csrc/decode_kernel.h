// Paged flash-decode kernel template and its shape dispatch (internal).
// The plain and the fused-append instantiations are compiled in separate
// translation units (decode.hip, decode_fused.hip) that include this file.
#pragma once

// Paged flash-decode over an E4M3 KV cache for gfx950.
//
// Operation (page "fp8 paged attention for MoE serving", "Smallest correct
// example" and "Expected result"): for sequence b, KV head g and the G query
// heads that share it, attend over the positions [start, L) of the sequence
// through its block table, with E4M3 K/V dequantized as code x scale, a custom
// sm_scale, and an optional per-head sink logit in the denominator.
//
// Work decomposition.  A unit is one (sequence, KV head): the G query heads
// of the unit share every K/V read (page section "Why it happens": the grid
// runs over sequence, KV head and split).  A unit's attended positions form a
// run of tiles; the tiles of all units, sequence by sequence (or KV head by
// KV head, so that the heads' shares of the same pages run side by side on
// one XCD), make one global list, and workgroup w of W takes an equal share
// of it, so every
// workgroup streams the same number of bytes however uneven the sequence
// lengths are, and W is chosen so that all workgroups are resident at once.
// A call with few tiles uses only as many workgroups as give each at least
// one tile per wave (counting the units' fixed costs, or, for a call with few
// units, on average), so the shares stay worth a launch; a share that falls
// inside a unit's fixed cost is empty and simply ends.
// Every workgroup builds the list itself from seq_lens (a prefix sum in LDS),
// so the grid depends on host values only.  A workgroup's share cuts units
// into segments; a workgroup is NW wave64s (four by default), each wave walks
// every NW-th tile of a segment with its own online softmax, and the states
// are combined in LDS.  The block-table rows of a segment are staged in LDS.
// How many workgroups a CU runs is part of the kernel shape: at head dim 128
// one four-wave workgroup per CU streams as fast as two and halves the
// number of cut units.
//
// Merging.  A segment that covers a whole unit writes the output.  Otherwise
// it writes a normalised partial and its base-2 log-sum-exp (only a
// workgroup's first and last segments can be partial: two slots per
// workgroup) and then a flag holding the call's epoch.  The workgroup holding a unit's last piece (its
// first segment) merges the unit's partials at the end of its own share, when
// the other holders, all of lower index, are finishing too: it waits for
// their flags, combines (the standard log-sum-exp combination; the sink
// enters once) and clears the flags, so a replayed graph (same epoch) starts
// clean.  Flags need no initialisation: stale ones hold another call's
// epoch.  No read-modify-write atomics are involved.
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
// positions) and B = P^T, the probabilities as a hi/lo pair of bf16 operands
// in two MFMAs (split_bf16x8).  V stored d-major per (page, head) lets lane
// (dim l%16, quad l/16) load the 8*NS positions it needs as one 16-byte (or
// 8-byte) load straight from HBM.  V stored token-major (the page's "heads"
// and "tokens" orders, VT) is loaded as whole 16-byte pieces of position rows,
// written to a per-wave LDS stage and read back with gfx950's 8-bit transpose
// read (ds_read_b64_tr_b8), which hands each lane 8 positions of one dim.
//
// Scales.  fp32 per (page, head) or per (token, head): the K scale multiplies
// the score after the dot product and the V scale multiplies the probability
// before the PV product (both are exact reassociations of code x scale).
// E8M0 per 32 dims: the K scale is applied inside the E4M3 -> bf16 conversion
// (a power of two, exact); the V scale varies along the dims, so the PV B
// operand is built once per 32-dim group with p x 2**(e - 127).
// fp32 per (token, head, S dims) for K (sub-row key scales, SK = 3): each
// lane's 8-code MFMA piece lies in one position row and one group, so the
// lane scales its codes in fp32 and feeds the product as a hi/lo pair of bf16
// operands (two MFMAs); V then takes per-(token, head) scales.
//
// Masked positions (outside [start, L): the tail of the last page, positions
// before the window) get a score of -inf by selection and their V bytes are
// zeroed, so NaN codes or scales there never reach the output.  Pages with no
// attended position are never looked up in the block table.
#include <hip/hip_ext.h>

#include "append_common.h"
#include "device_common.h"
#include "fp8pa_internal.h"
#include "merge_common.h"

namespace fp8pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int NS>
struct VRaw;
template <>
struct VRaw<1> { typedef u32x2 type; };
template <>
struct VRaw<2> { typedef u32x4 type; };

// The probabilities of a PV operand as two bf16 octets, hi = bf16(v) and
// lo = bf16(v - hi), so that the product carries v to about 16 significant
// bits: a single bf16 rounding of p (relative error up to 2^-8) can move an
// output whose terms cancel by more than 4e-3.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    const float h0 = __builtin_bit_cast(float, h[j] << 16), h1 = __builtin_bit_cast(float, h[j] & 0xffff0000u);
    l[j] = pack_bf16x2(v[2 * j] - h0, v[2 * j + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Eight E4M3 codes (element i from byte i of w0:w1) times an fp32 scale, as
// a hi/lo pair of bf16 operands: x = fp32(code * s) (scaled_e4m3x8), hi =
// bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void scaled_e4m3x8_hilo(uint32_t w0, uint32_t w1, float s, bf16x8& hi, bf16x8& lo) {
  float v[8];
  scaled_e4m3x8(w0, w1, s, v);
  split_bf16x8(v, hi, lo);
}

// The D/32 E8M0 bytes of one position (one 32-dim group each), zero-extended
// into a u32x4.
template <int NG>
__device__ __forceinline__ u32x4 load_e8_row(const uint8_t* p) {
  if constexpr (NG == 2) return u32x4{(uint32_t)ld_global<uint16_t>(p), 0, 0, 0};
  else if constexpr (NG == 4) return u32x4{ld_global<uint32_t>(p), 0, 0, 0};
  else if constexpr (NG == 8) { const u32x2 v = ld_global<u32x2>(p); return u32x4{v[0], v[1], 0, 0}; }
  else return ld_global<u32x4>(p);
}

// floor(a / b) for 0 <= a < 2^53, 0 < b: 32-bit division when both fit,
// else a double-precision quotient corrected by one step either way (much
// shorter than 64-bit integer division).
__device__ __forceinline__ int64_t floordiv(int64_t a, int64_t b) {
  if ((((uint64_t)a | (uint64_t)b) >> 32) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  int64_t q = (int64_t)((double)a / (double)b);
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}

// A 64-bit value of lane l (l uniform).
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t byte_of(const u32x4& v, int i) { return (v[i >> 2] >> (8 * (i & 3))) & 0xffu; }

// V token-major (VT): a lane loads NIV = NS*D/32 16-byte pieces, dims
// 16*(l % (D/16)).. +15 of NIV consecutive positions (one page), staged per
// wave in LDS (VStage<D>).

// Registers of one tile for one lane.
template <int D, int NS, int SK, bool VT>
struct Tile {
  static constexpr int NM = D / 64, NC = D / 16, NG = D / 32, NE = (8 * NG) / 16;
  static constexpr int NIV = NS * D / 32;
  typedef typename VRaw<NS>::type vraw_t;
  u32x4 k[NS][2][NM];   // K codes of the lane's position rows
  vraw_t v[NC];         // V codes of the lane's dims, GT positions each
  u32x4 vt[VT ? NIV : 1];   // VT: the lane's pieces of V position rows, as loaded
  float ks, vs;         // per-(page, head) scales of the lane's score group
  float kst[NS][8];     // per-(token, head) scales of the lane's score positions
  float vst[NS][8];
  u32x4 ke8[NS][2];     // E8M0 bytes of the lane's K rows
  u32x4 ve8[NS][NE];    // E8M0 bytes of the lane's 8 score positions, all groups
  // fp32 sub-row K scales of the lane's 16-dim K pieces (SK >= 5: of their
  // two 8-dim halves)
  float kgs[NS][2][NM][SK >= 5 ? 2 : 1];
  float vgs[SK == 4 || SK == 6 ? 8 * NS : 1];   // V in groups: the lane's share of the tile's V scales
};

// FUSED: also append each sequence's new token (DecodeArgs::k_new / v_new)
// before reading it.
// VT: V in a token-major layout (HEADS or TOKENS), staged through LDS.
// F8: fp8 compute mode for QK^T: each query row is rounded to E4M3 with one
// fp32 scale (amax / 448), and the K codes enter an fp8 MFMA unconverted; the
// PV product stays bf16.
// PK: packed heads (low latency, no splits): workgroup w holds sequence
// w / ceil(Hkv/NW) and NW consecutive KV heads, one per wave, each wave
// streaming every tile of its head; the waves read the same page rows
// together and nothing is merged.
// PS: packed heads with splits: a unit is (sequence, NW consecutive KV heads),
// its NW*G query heads merged as one; wave v of a workgroup streams every
// tile of its segment for KV head NW*g + v (the NW waves read the same page
// rows together), so no wave combine is needed; shares, partials and merges
// are those of the split kernel over these wider units.
template <int D, int SK, bool KNT, bool FUSED, bool VT, bool F8 = false, bool PK = false, bool PS = false>
__global__ __launch_bounds__(64 * Shape<D>::NW, Shape<D>::OCC) void decode_kernel(const DecodeArgs a) {
  static_assert(!(PS && (FUSED || PK)), "packed splits: plain kernels");
  // Scale classes: 0 page, 1 token, 2 E8M0 (K and V alike); fp32 sub-row K
  // groups with V per (token, head) (3: groups of 16 dims or more, 5: of 8)
  // or V in groups too (4, 6).
  constexpr bool KG = SK >= 3;                // K in fp32 sub-row groups
  constexpr bool VG = SK == 4 || SK == 6;     // V in fp32 sub-row groups
  constexpr bool K8 = SK >= 5;                // K groups of 8 dims: two scales per 16-dim piece
  static_assert(!(F8 && KG), "sub-row fp32 K scales vary inside one fp8 MFMA");
  static_assert(!(F8 && SK == 2 && D % 128), "the MX-scaled fp8 MFMA contracts 128 dims at a time");
  // MX: the fp8 mode over E8M0 pools: QK^T on the MX-scaled fp8 MFMA, which
  // applies the keys' E8M0 scales and the query's own (MXFP8) scales itself.
  constexpr bool MX = F8 && SK == 2;
  static_assert(!(KG && (FUSED || PK || PS)), "sub-row scales: split kernels without the fused append");
  static_assert(!(PK && (FUSED || F8)), "packed heads: plain bf16 kernels");
  constexpr int NS = Shape<D>::NS;
  constexpr int NW = Shape<D>::NW;
  constexpr int NT = 64 * NW;   // threads (NW wave64s)
  constexpr int TT = 32 * NS;   // positions per tile
  constexpr int GT = 8 * NS;    // positions per group
  constexpr int NM = D / 64;    // 16-byte K pieces per position row per lane
  constexpr int NQ = D / 32;    // QK MFMAs per 16 positions
  constexpr int NC = D / 16;    // PV MFMAs per subtile (16 dims each)
  constexpr int NG = D / 32;    // E8M0 groups along D
  typedef Tile<D, NS, SK, VT> TileT;

  extern __shared__ int s_dyn[];   // tile prefix, non-empty prefix, lengths, then the page-row stage / wave-combine buffer
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];
  __shared__ float s_M[16], s_den[16], s_sc[16];
  __shared__ int s_wsum[NW], s_wsum_ne[NW];
  __shared__ int s_timeout;
  __shared__ int s_app;   // fused append: number of the last segment whose new token is written
  __shared__ int64_t s_bnd[2];
  __shared__ int s_first[3];   // capped W and the first segment's (b, g), from wave 0

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (FUSED && threadIdx.x == 0) s_app = 0;   // ordered by the set-up barriers below
  const int n = lane & 15;      // MFMA column: query head of the group
  const int quad = lane >> 4;   // MFMA k/row quad
  // PS: G and Hkv count the query heads and units of a packed unit.
  const int G = PS ? a.G * NW : a.G, P = a.P, log2P = a.log2P, B = a.B, Hkv = PS ? a.Hkv / NW : a.Hkv;
  int W = gridDim.x;
  const int w = blockIdx.x;
  // XCD-blocked shares.  The dispatcher hands workgroups to the eight XCDs in
  // turn (workgroup w runs on XCD w mod 8), and each XCD has its own L2.
  // Workgroup w takes share sw = (w mod 8) * G8 + w / 8 (G8 = W / 8), so each
  // XCD works through one contiguous block of the share list: whole runs of
  // units, i.e. the KV heads of the same page rows.  The scale footer lines
  // and the lines at head boundaries that neighbouring heads' shares touch
  // are then fetched once into one L2 instead of into several.  A launch
  // whose grid is not a multiple of 8 keeps sw = w.
  //
  // Head-major order.  When the grid is not capped and W is a multiple of
  // 8 * Hkv, units are ordered KV head first (all sequences of head 0, then
  // of head 1, ...).  Every head's run then costs Ct / Hkv, a whole number of
  // shares, so shares j, W/Hkv + j, 2W/Hkv + j, ... cover the same positions
  // of the same sequences, one KV head each.  Those Hkv shares go to Hkv
  // consecutive workgroups of one XCD (its k-th workgroup takes head k mod
  // Hkv of share group x * G8h + k / Hkv, G8h = W / (8 Hkv)), which start
  // together and walk the same page rows in step: the scale-footer lines and
  // the lines that straddle two heads' payloads are fetched into that L2 once
  // for all the heads.  A share then lies inside one head's run, so its
  // head and its place in the run are known without a division (Hkv a power
  // of two).  Otherwise units are ordered sequence first.  (Head dims 128
  // and 512 keep the sequence-first order: the extra set-up state made them
  // spill.)
  constexpr bool HMK = D == 64 || D == 256;
  const int G8 = (gridDim.x % 8 == 0 && gridDim.x >= 16) ? (int)gridDim.x / 8 : 0;
  int sw = 0;         // this workgroup's share
  bool hm = false;    // head-major unit order
  int G8m = 0;        // shares per XCD block (of one head's run in head-major order)
  int hgh = 0, hj = 0, hlog = 0;   // head-major: the share's head, its share in that head's run, log2 Hkv
  // Every value is assigned from uniform ones (W, w, Hkv), whatever ran
  // before, so that they stay in scalar registers.
  auto set_order = [&]() {
    hm = HMK && G8 && W == (int)gridDim.x && (Hkv & (Hkv - 1)) == 0 && W % (8 * Hkv) == 0;
    hlog = hm ? __builtin_ctz((unsigned)Hkv) : 0;
    G8m = hm ? W >> (3 + hlog) : G8;
    hgh = hm ? (w >> 3) & (Hkv - 1) : 0;
    hj = hm ? (w & 7) * G8m + (w >> (3 + hlog)) : 0;
    sw = hm ? hgh * (W >> hlog) + hj : (G8 ? (w % 8) * G8 + w / 8 : w);
  };
  const bool col = n < (PS ? a.G : G);

  // Debug checks (a.dbg set): a length outside [0, dbg_max_len] counts as 0
  // and a table entry outside [0, dbg_rows) as row 0, so nothing is read
  // outside the pools; the caller gathers the verdicts and sets the error word
  // once after its loads (a store among them would order the loads behind it).
  auto chk_len = [&](int len, bool& bad) -> int {
    const bool b = a.dbg && (len < 0 || len > a.dbg_max_len);
    bad |= b;
    return b ? 0 : len;
  };
  auto chk_row = [&](int32_t r, bool& bad) -> int32_t {
    const bool b = a.dbg && (uint32_t)r >= (uint32_t)a.dbg_rows;
    bad |= b;
    return b ? 0 : r;
  };
  auto flag = [&](bool bad, int word) {
    if (bad) __hip_atomic_store(a.dbg + word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- tiles per sequence and their prefix sums.
  auto tiles_of = [&](int L) {
    const int st = (a.window > 0 && L > a.window) ? L - a.window : 0;
    const int tb = st & ~(TT - 1);
    return L > st ? (L - tb + TT - 1) / TT : 0;
  };
  int* s_pre = s_dyn;                       // [B + 1] tiles before sequence b
  int* s_nep = s_dyn + ((B + 4) & ~3);      // [B + 1] non-empty sequences before b
  int* s_len = s_nep + ((B + 4) & ~3);      // [B] seq_lens, read from global memory once
  int* s_work_i = s_len + ((B + 4) & ~3);
  float* s_work = reinterpret_cast<float*>(s_work_i);
  // Shares are balanced in cost: a tile costs TC = 4 and every (non-empty)
  // unit a fixed SC more (its setup, wave combine and partial), laid out
  // before its tiles.  Workgroup w takes the tiles whose cost start lies in
  // [floor(w*Ct/W), floor((w+1)*Ct/W)).  Any cost window of SC + TC holds a
  // tile start, so capping W at Ct / (SC + TC*min_tiles) keeps every share
  // non-empty (at least min_tiles tiles' worth).  When units average at most
  // one tile per wave, a split would only add merges: tiles then cost 0 and a
  // unit 1, so shares are whole units (unit-aligned mode).
  int64_t T = 0, U = 0, TC = 0, SC = 0, Ct = 0, T1 = 0, Ct1 = 0;
  auto set_costs = [&](int tiles, int nonempty) {
    T = (int64_t)tiles * Hkv;
    U = (int64_t)nonempty * Hkv;
    const bool unit_mode = T <= (int64_t)(PS ? 1 : NW) * U;
    TC = unit_mode ? 0 : 4;
    SC = unit_mode ? 1 : a.seg_cost;
    Ct = SC * U + TC * T;
    T1 = tiles;                           // tiles of one KV head's run (head-major order)
    Ct1 = SC * nonempty + TC * T1;        // and its cost: Ct = Hkv * Ct1
  };
  // A call with few units (single long sequences) may also take up to one
  // share per NW tiles (min_tiles = NW outside packed splits), ignoring the
  // units' fixed costs: every share then costs at least 4 * NW, so it holds a
  // tile of any unit whose tiles it overlaps; a share that holds only part of
  // a unit's fixed cost is empty, holds no unit and merges nothing.
  auto cap_W = [&]() {
    int64_t want = floordiv(Ct, SC + TC * a.min_tiles);
    if (!PS && TC > 0 && T / NW > want) want = T / NW;
    if (want < 1) want = 1;
    if (T == 0) want = 0;
    if (want < W) W = (int)want;
  };
  // A share bound as a global tile index: the first tile whose cost start is
  // >= c, for c inside the cost range of sequence bb (which starts at lo,
  // after pre tiles, and has nbb tiles per unit, hk units); past a unit's
  // last tile that is the next unit's first.  In head-major order the range
  // is one head's (hk = 1) and the caller adds the head run's offset.
  auto bound_in = [&](int64_t c, int64_t lo, int pre, int nbb, int hk) -> int64_t {
    const int64_t span = SC + TC * nbb;
    int64_t gg = floordiv(c - lo, span);
    const int64_t r = c - lo - gg * span;
    int64_t t = r <= SC ? 0 : (TC > 0 ? (r - SC + 3) >> 2 : nbb);
    if (t >= nbb) {
      t = 0;
      ++gg;
    }
    return (int64_t)hk * pre + gg * nbb + t;
  };
  // Page rows of the chunk [ca, cb) of the current segment's tiles.
  int b = 0, g = 0, L = 0, start = 0, tbeg = 0, p_first = 0, nstaged = 1;
  auto chunk_rows = [&](int ca, int cb) {
    const int pos0 = tbeg + ca * TT > start ? tbeg + ca * TT : start;
    const int pos1 = tbeg + cb * TT < L ? tbeg + cb * TT : L;
    p_first = pos0 >> log2P;
    nstaged = ((pos1 - 1) >> log2P) - p_first + 1;
  };
  constexpr int CH = kMaxSplitTokens / TT;   // tiles whose page rows are staged at once
  int* s_tab = s_work_i;

  // Up to 64 sequences, wave 0 alone computes the prefix sums, the share
  // bounds and the first segment's unit in registers, and stages that
  // segment's first page rows, so the workgroup passes a single barrier
  // before its first tile loads.  Larger batches use all four waves.
  const bool fast = !PK && B <= 64;
  if constexpr (PK) {
  } else if (fast) {
    if (wave == 0) {
      bool bad_len = false;
      const int len = lane < B ? chk_len(a.seq_lens[lane], bad_len) : 0;
      flag(bad_len, 1);
      const int nt = tiles_of(len), ne = nt > 0 ? 1 : 0;
      const int incl = wave_incl_sum(nt), incl_ne = wave_incl_sum(ne);
      const int pre = incl - nt, nep = incl_ne - ne;
      if (lane < B) {
        s_len[lane] = len;
        s_pre[lane] = pre;
        s_nep[lane] = nep;
      }
      const int tot = __builtin_amdgcn_readlane(incl, 63), tot_ne = __builtin_amdgcn_readlane(incl_ne, 63);
      if (lane == 0) {
        s_pre[B] = tot;
        s_nep[B] = tot_ne;
      }
      set_costs(tot, tot_ne);
      cap_W();
      set_order();
      if (sw < W) {
        const int hk = hm ? 1 : Hkv;   // units of a sequence inside one cost range
        const int64_t lo = SC * hk * nep + TC * (int64_t)hk * pre;
        const int64_t hiw = lo + (int64_t)hk * (SC * ne + TC * nt);
        const int64_t gofs = hm ? (int64_t)hgh * T1 : 0;   // head-major: first tile of the share's head run
        int64_t bnd[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // head-major: the bound inside the head's run (cost Ct1, W >> hlog shares)
          const int64_t c = hm ? floordiv((int64_t)(hj + e) * Ct1, W >> hlog) : floordiv((int64_t)(sw + e) * Ct, W);
          const bool hit = lane < B && c >= lo && c < hiw;
          const int64_t v = hit ? gofs + bound_in(c, lo, pre, nt, hk) : 0;
          const uint64_t mask = __ballot(hit);
          bnd[e] = mask ? readlane64(v, (int)__builtin_ctzll(mask)) : (hm ? gofs + T1 : T);
        }
        if (bnd[0] < bnd[1]) {
          // The first segment's unit: b is the last sequence whose tiles start
          // at or before bnd[0] (a non-empty one, as bnd[0] < T), within the
          // share's head run in head-major order.
          const int64_t r0 = bnd[0] - gofs;
          const int bl = 63 - (int)__builtin_clzll(__ballot(lane < B && (int64_t)hk * pre <= r0));
          b = bl;
          const int nb = __builtin_amdgcn_readlane(nt, bl);
          const int64_t ubase = gofs + (int64_t)hk * __builtin_amdgcn_readlane(pre, bl);
          g = hm ? hgh : (int)floordiv(bnd[0] - ubase, nb);
          const int64_t ustart = hm ? ubase : ubase + (int64_t)g * nb;
          const int ta = (int)(bnd[0] - ustart);
          const int tc = (int)((bnd[1] < ustart + nb ? bnd[1] : ustart + nb) - ustart);
          L = __builtin_amdgcn_readlane(len, bl);
          start = (a.window > 0 && L > a.window) ? L - a.window : 0;
          tbeg = start & ~(TT - 1);
          chunk_rows(ta, tc < ta + CH ? tc : ta + CH);
          const int32_t* btr0 = a.bt + (int64_t)b * a.bt_stride;
          bool bad = false;
          for (int i = lane; i < nstaged; i += 64) s_tab[i] = chk_row(btr0[p_first + i], bad);
          flag(bad, 0);
        }
        if (lane == 0) {
          s_bnd[0] = bnd[0];
          s_bnd[1] = bnd[1];
          s_first[1] = b;
          s_first[2] = g;
        }
      }
      if (lane == 0) s_first[0] = W;
    }
    __syncthreads();
    W = s_first[0];
    set_costs(s_pre[B], s_nep[B]);
    set_order();
  } else {
    const int per = (B + NT - 1) / NT;
    const int bb0 = threadIdx.x * per;
    int local = 0, lne = 0;
    bool bad_len = false;
    for (int i = 0; i < per; ++i)
      if (bb0 + i < B) {
        const int len = chk_len(a.seq_lens[bb0 + i], bad_len);
        s_len[bb0 + i] = len;
        const int nt = tiles_of(len);
        local += nt;
        lne += nt > 0;
      }
    flag(bad_len, 1);
    const int incl = wave_incl_sum(local), incl_ne = wave_incl_sum(lne);
    if (lane == 63) {
      s_wsum[wave] = incl;
      s_wsum_ne[wave] = incl_ne;
    }
    __syncthreads();
    int excl = incl - local, excl_ne = incl_ne - lne;
    for (int i = 0; i < wave; ++i) {
      excl += s_wsum[i];
      excl_ne += s_wsum_ne[i];
    }
    for (int i = 0; i < per; ++i)
      if (bb0 + i < B) {
        const int nt = tiles_of(s_len[bb0 + i]);
        s_pre[bb0 + i] = excl;
        s_nep[bb0 + i] = excl_ne;
        excl += nt;
        excl_ne += nt > 0;
      }
    if (threadIdx.x == 0) {
      int t = 0, tn = 0;
      for (int i = 0; i < NW; ++i) {
        t += s_wsum[i];
        tn += s_wsum_ne[i];
      }
      s_pre[B] = t;
      s_nep[B] = tn;
    }
    __syncthreads();
    set_costs(s_pre[B], s_nep[B]);
    cap_W();
    set_order();
  }

  // Sequences with nothing to attend get a zero output (packed heads: each
  // wave writes its own head's, and the tile prefix is not built).
  if constexpr (!PK) {
    for (int bb = w; bb < B; bb += (int)gridDim.x) {
      if (s_pre[bb + 1] != s_pre[bb]) continue;
      uint16_t* o = a.out + (size_t)bb * a.Hq * D;
      for (int i = threadIdx.x; i < a.Hq * D; i += NT) o[i] = 0;
    }
    if (sw >= W) return;
  }
  // Cost start of sequence bb's units (of one head's run in head-major order).
  auto cpre = [&](int bb) -> int64_t {
    const int hk = hm ? 1 : Hkv;
    return SC * hk * s_nep[bb] + TC * (int64_t)hk * s_pre[bb];
  };
  // Cost start of tile i of unit (bb, gg).
  auto tile_cost = [&](int bb, int gg, int i) -> int64_t {
    const int nbb = s_pre[bb + 1] - s_pre[bb];
    return hm ? (int64_t)gg * Ct1 + cpre(bb) + SC + TC * i : cpre(bb) + (int64_t)gg * (SC + TC * nbb) + SC + TC * i;
  };
  // Share holding a tile of cost start c: the largest sh with floor(sh*Ct/W) <= c.
  auto share_of_cost = [&](int64_t c) -> int { return (int)(floordiv((c + 1) * W + Ct - 1, Ct) - 1); };
  // The holder of a cut unit's pieces (shares sa..sb) that merges them: the
  // one with the highest workgroup index, so that it waits only on workgroups
  // dispatched before it.  Within an XCD block the workgroup index grows with
  // the share; the last share of a block outranks every share of the next
  // blocks but that block's own last one.  So: sb, unless the unit crosses
  // into sb's block from an earlier one and sb does not end its block, in
  // which case the end of the block before sb's.
  // (In head-major order a unit's pieces lie in one head's run, whose XCD
  // blocks are G8m shares long, and the same holds.)
  auto merger_share = [&](int sa, int sb) -> int {
    if (!G8m || sb % G8m == G8m - 1) return sb;
    const int e = (sb / G8m) * G8m - 1;
    return e >= sa ? e : sb;
  };
  if (!fast) {
    // The share's first and end tiles: the first tile whose cost start is >=
    // floor(w*Ct/W), resp. floor((w+1)*Ct/W), found by the thread whose
    // sequence's cost range holds that point (T past the end).
    // (head-major: inside the share's head run, of cost Ct1 and W >> hlog shares)
    const int64_t gofs = hm ? (int64_t)hgh * T1 : 0;
    const int64_t cb[2] = {hm ? floordiv((int64_t)hj * Ct1, W >> hlog) : floordiv((int64_t)sw * Ct, W),
                           hm ? floordiv((int64_t)(hj + 1) * Ct1, W >> hlog) : floordiv((int64_t)(sw + 1) * Ct, W)};
    if (threadIdx.x < 2) s_bnd[threadIdx.x] = hm ? gofs + T1 : T;
    __syncthreads();
    const int per = (B + NT - 1) / NT;
    const int hk = hm ? 1 : Hkv;
    for (int i = 0; i < per; ++i) {
      const int bb = threadIdx.x * per + i;
      if (bb >= B) break;
      const int64_t lo = cpre(bb), hiw = cpre(bb + 1);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t c = cb[e];
        if (c >= lo && c < hiw) s_bnd[e] = gofs + bound_in(c, lo, s_pre[bb], s_pre[bb + 1] - s_pre[bb], hk);
      }
    }
    __syncthreads();
  }

  // Per-segment state (captured by the tile helpers below).
  const int32_t* btr = a.bt;
  const uint8_t* kpool = a.kp;
  const uint8_t* vpool = a.vp;
  const int kgrp = n >> 2;      // group of this lane's K row
  const int kslot = n & 3;
  bf16x8 qop[NQ];
  uint64_t qop8[NQ];   // F8: E4M3 codes of the same dims
  float qsc = 1.0f;    // F8: scale of the lane's query row
  // MX: the 16x16x128 MFMA takes, from lane (quad, n), bytes 0-15 as
  // contraction elements 16quad.. and bytes 16-31 as 64 + 16quad.., and the
  // lane's scale byte for elements 32quad .. 32quad + 31.  With element k =
  // dim 128x + k, a lane's K bytes are exactly the two 16-byte pieces the
  // bf16 path loads (t.k[s][aa][2x], [2x + 1]) and its key scale is the E8M0
  // byte of dims 128x + 32quad .. +31 of its row.
  constexpr int NX = D / 128;   // MX: MFMAs of 128 dims per 16 positions
  v8i32 qmx[MX ? NX : 1];       // MX: E4M3 codes of the lane's query head, same dims as its K bytes
  uint32_t qmxs[MX ? NX : 1];   // MX: E8M0 scale of dims 128x + 32quad .. +31 of that head

  // Row of a page of the current chunk.  A group with no attended position
  // reads a clamped (attended) page instead: its scores are masked to -inf and
  // its V bytes zeroed, so every lane issues the same loads and the compiler
  // can count outstanding loads exactly across the prefetch.
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
    const RowBases rk = row_bases(a.kg, row_k), rqk = row_bases(a.kg, row_q), rqv = row_bases(a.vg, row_q);
    const int kvh = PS ? g * NW + wave : g;   // the lane's KV head
    const uint8_t* ksc = a.kp + rqk.scale + kvh * a.kg.sc_head_stride;
    const uint8_t* vsc = a.vp + rqv.scale + kvh * a.vg.sc_head_stride;
    if constexpr (SK == 0) {
      t.ks = ld_global<float>(ksc);
      t.vs = ld_global<float>(vsc);
    } else if constexpr (SK == 1 && !VT) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tt = tpq + 8 * s + i;
          t.kst[s][i] = ld_global<float>(ksc + tt * a.kg.sc_tok_stride);
          t.vst[s][i] = ld_global<float>(vsc + tt * a.vg.sc_tok_stride);
        }
    } else if constexpr (SK == 1) {
      // VT: the 8 scales of a group as two 16-byte loads where consecutive
      // positions' scales are adjacent (every layout but TOKENS), else one
      // load per position.  (Measured: 72.6 -> 68.1 us on the Llama-shaped
      // call with both pools in HEADS; the same runtime choice in the
      // d-major-V kernels cost them 4-16 us, so those keep one load per
      // position.)
      auto scales8 = [&](float (&dst)[8], const uint8_t* base, int tt0, int stride) {
        if (stride == 4) {
          const f32x4 lo = ld_global<f32x4>(base + 4 * tt0), hi = ld_global<f32x4>(base + 4 * tt0 + 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[i] = lo[i];
            dst[4 + i] = hi[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[i] = ld_global<float>(base + (tt0 + i) * stride);
        }
      };
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        scales8(t.kst[s], ksc, tpq + 8 * s, a.kg.sc_tok_stride);
        scales8(t.vst[s], vsc, tpq + 8 * s, a.vg.sc_tok_stride);
      }
    } else if constexpr (KG) {
      // K: the scale of each of the lane's 16-dim pieces (position row tk +
      // 8s + 4aa + kslot, dims 64m + 16*quad..: one group, as groups span 16
      // dims or more), or of its two 8-dim halves (K8).
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const int tp = (tk + 8 * s + 4 * aa + kslot) & (P - 1);
          const uint8_t* kf = a.kp + rk.scale + kvh * a.kg.sc_head_stride + tp * a.kg.sc_tok_stride;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            t.kgs[s][aa][m][0] = ld_global<float>(kf + 4 * ((64 * m + 16 * quad) >> a.kg.sc_gshift));
            if constexpr (K8) t.kgs[s][aa][m][K8 ? 1 : 0] = ld_global<float>(kf + 4 * ((64 * m + 16 * quad + 8) >> 3));
          }
        }
      if constexpr (!VG) {
        // V: per (token, head), as for SK = 1.
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) t.vst[s][i] = ld_global<float>(vsc + (tpq + 8 * s + i) * a.vg.sc_tok_stride);
      } else {
        // V in sub-row groups: lane l loads the groups gh, gh + LP, ... of
        // tile position l % TT (gh = l / TT, LP = 64 / TT lanes per position).
        constexpr int LP = 64 / TT;
        const int pos = T0 + lane % TT, gh = lane / TT, ngv = D >> a.vg.sc_gshift;
        const RowBases rvg = row_bases(a.vg, row_of(pos >> log2P));
        const uint8_t* vf = a.vp + rvg.scale + kvh * a.vg.sc_head_stride + (pos & (P - 1)) * a.vg.sc_tok_stride;
#pragma unroll
        for (int i = 0; i < 8 * NS; ++i) {
          // (Unconditional loads, clamped into the head's groups.)
          const int gg = gh + LP * i;
          const float v = ld_global<float>(vf + 4 * (gg < ngv ? gg : ngv - 1));
          t.vgs[i] = gg < ngv ? v : 0.0f;
        }
      }
    } else {
      if constexpr (VT) {
        // One position's NG bytes at a time: in the TOKENS layout consecutive
        // positions' scale bytes are Hkv*NG apart.
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint8_t* src = vsc + (tpq + 8 * s + i) * a.vg.sc_tok_stride;
            if constexpr (NG == 16) {
              t.ve8[s][i] = ld_global<u32x4>(src);
            } else if constexpr (NG == 8) {
              const u32x2 v2 = ld_global<u32x2>(src);
              t.ve8[s][i >> 1][2 * (i & 1)] = v2[0];
              t.ve8[s][i >> 1][2 * (i & 1) + 1] = v2[1];
            } else if constexpr (NG == 4) {
              t.ve8[s][i >> 2][i & 3] = ld_global<uint32_t>(src);
            } else {
              const uint32_t h16 = ld_global<uint16_t>(src);
              if (i & 1) t.ve8[s][0][i >> 1] |= h16 << 16;
              else t.ve8[s][0][i >> 1] = h16;
            }
          }
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint8_t* src = vsc + (tpq + 8 * s) * a.vg.sc_tok_stride;
#pragma unroll
          for (int k = 0; k < TileT::NE; ++k) t.ve8[s][k] = ld_global<u32x4>(src + 16 * k);
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const int tp = (tk + 8 * s + 4 * aa + kslot) & (P - 1);
          const uint8_t* kf = a.kp + rk.scale + kvh * a.kg.sc_head_stride +
                              tp * a.kg.sc_tok_stride;
          t.ke8[s][aa] = load_e8_row<NG>(kf);
        }
    }
    {
      const uint8_t* krow = kpool + rk.code + 16 * quad;
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
    }
    if constexpr (VT) {
      // Whole 16-byte pieces of NIV consecutive position rows (NIV <= 16
      // divides P, so they share a page).
      constexpr int LPP = D / 16, NIV = TileT::NIV;
      const int tv0 = T0 + (lane / LPP) * NIV;
      const RowBases rv = row_bases(a.vg, row_of(tv0 >> log2P));
      const uint8_t* src = vpool + rv.code + (int64_t)(tv0 & (P - 1)) * a.vg.tok_stride + 16 * (lane % LPP);
#pragma unroll
      for (int j = 0; j < NIV; ++j) t.vt[j] = ld_stream<u32x4>(src + (int64_t)j * a.vg.tok_stride);
    } else {
      // The lane's GT positions lie in one token block of the d-major V layout.
      const uint8_t* vrow = vpool + rqv.code + (int64_t)(tpq / a.vg.tblk) * a.vg.tblk_stride +
                            (tpq % a.vg.tblk);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d = 16 * c + n;
        t.v[c] = ld_stream<typename TileT::vraw_t>(vrow + (int64_t)(d >> 6) * a.vg.dchunk_stride +
                                                   (int64_t)(d & 63) * a.vg.d_stride);
      }
    }
  };

  // VT: turn the loaded position-row pieces into the PV operand layout (lane
  // (dim n, quad) gets the GT positions of its group for every 16-dim chunk).
  // A transpose read takes, in each 16-lane group, eight 8-byte row pieces
  // (lane i reads half i&1 of the 16 dims of row i>>1) and gives lane m the
  // byte m&7 of the pieces of lanes m>>3, 2+(m>>3), ..., 14+(m>>3): dim m of
  // the eight rows.  The stage is private to the wave, whose LDS operations
  // complete in order.
  // (vstage_off leaves 16 bytes of slack to round the stage up to 16 bytes.)
  uint8_t* const vstage = reinterpret_cast<uint8_t*>(s_dyn) + a.vstage_off +
                          ((0u - (uint32_t)reinterpret_cast<uintptr_t>(s_dyn)) & 15u) + wave * (TT * VStage<D>::RS);
  // SK = 4: the wave's stage of the tile's V group scales, [group][position].
  float* const vgstage = reinterpret_cast<float*>(
      reinterpret_cast<uint8_t*>(s_dyn) + a.vgstage_off + ((0u - (uint32_t)reinterpret_cast<uintptr_t>(s_dyn)) & 15u) +
      wave * (TT * (D >> a.vg.sc_gshift) * 4));
  auto stage_v = [&](TileT& t) {
    constexpr int VH = VStage<D>::VH, RS = VStage<D>::RS, NIV = TileT::NIV, LPP = D / 16, CPP = VH / 16;
    const int prow = (lane / LPP) * NIV, pc = lane % LPP;
#pragma unroll
    for (int h = 0; h < D / VH; ++h) {
      if (pc / CPP == h) {
#pragma unroll
        for (int j = 0; j < NIV; ++j)
          *reinterpret_cast<u32x4*>(vstage + (prow + j) * RS + 16 * (pc % CPP)) = t.vt[j];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int cc = 0; cc < CPP; ++cc)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint8_t* src = vstage + (GT * quad + 8 * s + (n >> 1)) * RS + 16 * cc + 8 * (n & 1);
          const v2i32 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i32*)(src));
          t.v[h * CPP + cc][2 * s] = (uint32_t)r[0];
          t.v[h * CPP + cc][2 * s + 1] = (uint32_t)r[1];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  float m_run = kNegInf;        // running max (log2 units) of this lane's head column
  float l_run = 0.0f;           // this lane's share of the running sum
  f32x4 acc[NC];

  // ---- online-softmax update with one tile.
  auto compute_tile = [&](TileT& t, int T0) {
    const bool interior = (T0 >= start) && (T0 + TT <= L);
    float sc[NS][2][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (MX) {
#pragma unroll
          for (int x = 0; x < NX; ++x) {
            const u32x4 lo = t.k[s][aa][2 * x], hi = t.k[s][aa][2 * x + 1];
            const v8i32 kx = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            // Formats 0, 0: E4M3 for both operands; scale bytes in bits 0-7.
            s4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                kx, qmx[x], s4, 0, 0, 0, (int)byte_of(t.ke8[s][aa], 4 * x + quad), 0, (int)qmxs[x]);
          }
        }
#pragma unroll
        for (int m = 0; m < (MX ? 0 : NM); ++m) {
          float cvt = 1.0f;
          if constexpr (SK == 2) {
            const uint32_t e = byte_of(t.ke8[s][aa], 2 * m + (quad >> 1));
            cvt = e8m0_as_scale_operand(e);
          }
          const u32x4 w = t.k[s][aa][m];
          if constexpr (F8) {
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)(((uint64_t)w[1] << 32) | w[0]), (long)qop8[2 * m],
                                                            s4, 0, 0, 0);
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)(((uint64_t)w[3] << 32) | w[2]),
                                                            (long)qop8[2 * m + 1], s4, 0, 0, 0);
          } else if constexpr (KG) {
            bf16x8 hi, lo;
            scaled_e4m3x8_hilo(w[0], w[1], t.kgs[s][aa][m][0], hi, lo);
            s4 = mfma_16x16x32_bf16(hi, qop[2 * m], s4);
            s4 = mfma_16x16x32_bf16(lo, qop[2 * m], s4);
            scaled_e4m3x8_hilo(w[2], w[3], t.kgs[s][aa][m][K8 ? 1 : 0], hi, lo);
            s4 = mfma_16x16x32_bf16(hi, qop[2 * m + 1], s4);
            s4 = mfma_16x16x32_bf16(lo, qop[2 * m + 1], s4);
          } else {
            s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[0], w[1], cvt), qop[2 * m], s4);
            s4 = mfma_16x16x32_bf16(e4m3x8_to_bf16x8(w[2], w[3], cvt), qop[2 * m + 1], s4);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float f = a.qk_scale;
          if constexpr (F8 && !MX) f *= qsc;
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
    tmax = pair_max32(pair_max16(tmax));
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
    // Once the running maxima settle, alpha is 1 in every lane: skip the
    // rescale then (multiplying by 1 changes nothing).
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] *= alpha;
    }
    if constexpr (VT) stage_v(t);
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
    if constexpr (VG) {
      // The lane's V group scales to the wave's stage, [group][tile position].
      constexpr int LP = 64 / TT;
      const int ngv = D >> a.vg.sc_gshift;
#pragma unroll
      for (int i = 0; i < 8 * NS; ++i) {
        const int gg = lane / TT + LP * i;
        if (gg < ngv) vgstage[gg * TT + lane % TT] = t.vgs[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (VG) {
        // One probability operand (hi/lo pair) per V group: p x the group
        // scale of each of the lane's 8 positions; a 16-dim chunk lies in one
        // group, so chunk c uses group 16c / S.
        int gprev = -1;
        bf16x8 pop, pol;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int gg = (16 * c) >> a.vg.sc_gshift;
          if (gg != gprev) {
            const float* sp = vgstage + gg * TT + GT * quad + 8 * s;
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(sp), s1 = *reinterpret_cast<const f32x4*>(sp + 4);
            float pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float sv = i < 4 ? s0[i] : s1[i - 4];
              pv[i] = (p[s][i] == 0.0f) ? 0.0f : p[s][i] * sv;
            }
            split_bf16x8(pv, pop, pol);
            gprev = gg;
          }
          const bf16x8 vop = e4m3x8_to_bf16x8(t.v[c][2 * s], t.v[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop, acc[c]);
          acc[c] = mfma_16x16x32_bf16(vop, pol, acc[c]);
        }
      } else if constexpr (SK == 2) {
        bf16x8 pop[NG], pol[NG];
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
          split_bf16x8(pv, pop[gq], pol[gq]);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(t.v[c][2 * s], t.v[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop[c >> 1], acc[c]);
          acc[c] = mfma_16x16x32_bf16(vop, pol[c >> 1], acc[c]);
        }
      } else {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // A page scale belongs to an attended page (groups outside [start,
          // L) read a clamped attended one), so p * scale is 0 where p is;
          // a token scale of a masked position may be anything.
          if constexpr (SK == 0) pv[i] = p[s][i] * t.vs;
          if constexpr (SK == 1 || (KG && !VG)) pv[i] = (p[s][i] == 0.0f) ? 0.0f : p[s][i] * t.vst[s][i];
        }
        bf16x8 pop, pol;
        split_bf16x8(pv, pop, pol);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 vop = e4m3x8_to_bf16x8(t.v[c][2 * s], t.v[c][2 * s + 1], 1.0f);
          acc[c] = mfma_16x16x32_bf16(vop, pop, acc[c]);
          acc[c] = mfma_16x16x32_bf16(vop, pol, acc[c]);
        }
      }
    }
    if constexpr (VG) {
      // The next tile rewrites the stage only after these reads.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  if constexpr (PK) {
    const int hpg = (Hkv + NW - 1) / NW;
    b = w / hpg;
    g = (w - b * hpg) * NW + wave;
    const bool active = g < Hkv;
    if (!active) g = Hkv - 1;   // an idle wave: in-range pointers, no tiles, no output
    bool bad_len = false;
    L = chk_len(a.seq_lens[b], bad_len);
    flag(bad_len, 1);
    start = (a.window > 0 && L > a.window) ? L - a.window : 0;
    tbeg = start & ~(TT - 1);
    btr = a.bt + (int64_t)b * a.bt_stride;
    kpool = a.kp + (int64_t)g * a.kg.head_stride;
    vpool = a.vp + (int64_t)g * a.vg.head_stride;
    {
      const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)g * G + (col ? n : 0)) * D;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 v = col ? ld_global<u32x4>(qrow + 64 * m + 16 * quad + 8 * h2) : u32x4{0, 0, 0, 0};
          qop[2 * m + h2] = __builtin_bit_cast(bf16x8, v);
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nb = tiles_of(L);
    for (int ca = 0; ca < nb; ca += CH) {
      const int cb = nb < ca + CH ? nb : ca + CH;
      chunk_rows(ca, cb);
      __syncthreads();   // earlier readers of the stage are done
      bool bad = false;
      for (int i = threadIdx.x; i < nstaged; i += NT) s_tab[i] = chk_row(btr[p_first + i], bad);
      flag(bad, 0);
      __syncthreads();
      if (active) {
        TileT A;
        for (int k = ca; k < cb; ++k) {
          load_tile(A, tbeg + k * TT);
          compute_tile(A, tbeg + k * TT);
        }
      }
    }
    // The wave's head is complete: o = acc / (sum + e^(sink - max)).
    float lsum = l_run;
    lsum = pair_sum32(pair_sum16(lsum));
    if (active && col) {
      const int h = g * G + n;
      const float m_ref = (m_run == kNegInf) ? 0.0f : m_run;
      float den = lsum;
      if (a.sinks) den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - m_ref);
      const float inv = (m_run == kNegInf || !(den > 0.0f)) ? 0.0f : __builtin_amdgcn_rcpf(den);
      uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * D + 4 * quad;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x2 pk = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv), pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * c) = pk;
      }
    }
    return;
  }

  int64_t cur = s_bnd[0];
  const int64_t hi = s_bnd[1];
  int slot = 0;
  // Units to merge at the end of the share (uniform across the workgroup):
  // at most two, the share's first and last segments.
  int npend = 0;
  int pend_b[2] = {0, 0}, pend_g[2] = {0, 0}, pend_sa[2] = {0, 0}, pend_sb[2] = {0, 0}, pend_fsa[2] = {0, 0};
  // Wave 0 located the first segment and staged its first page rows.
  bool staged = fast;
  int seg_no = 0;
  while (cur < hi) {
    ++seg_no;
    // ---- the segment: unit (b, g), tiles [ta, tc) of the unit.
    if (staged) {
      b = s_first[1];
      g = s_first[2];
    } else if (hm) {
      g = hgh;   // the share's head run, then the sequence inside it
      const int64_t r = cur - (int64_t)g * T1;
      int lo_b = 0, hi_b = B - 1;   // largest b with s_pre[b] <= r (a non-empty sequence)
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if ((int64_t)s_pre[mid] <= r) lo_b = mid;
        else hi_b = mid - 1;
      }
      b = lo_b;
    } else {
      int lo_b = 0, hi_b = B - 1;   // largest b with s_pre[b] * Hkv <= cur (a non-empty sequence)
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if ((int64_t)s_pre[mid] * Hkv <= cur) lo_b = mid;
        else hi_b = mid - 1;
      }
      b = lo_b;
      g = (int)floordiv(cur - (int64_t)s_pre[b] * Hkv, s_pre[b + 1] - s_pre[b]);
    }
    const int nb = s_pre[b + 1] - s_pre[b];
    const int64_t ustart = hm ? (int64_t)g * T1 + s_pre[b] : (int64_t)s_pre[b] * Hkv + (int64_t)g * nb;
    const int64_t uend = ustart + nb;
    const int64_t send = hi < uend ? hi : uend;
    const int ta = (int)(cur - ustart), tc = (int)(send - ustart);
    L = s_len[b];
    start = (a.window > 0 && L > a.window) ? L - a.window : 0;
    tbeg = start & ~(TT - 1);
    btr = a.bt + (int64_t)b * a.bt_stride;
    const int kvh = PS ? g * NW + wave : g;   // this wave's KV head
    kpool = a.kp + (int64_t)kvh * a.kg.head_stride;
    vpool = a.vp + (int64_t)kvh * a.vg.head_stride;
    {
      // Q operand (B of QK): lane (head n, quad) holds dims 64m + 16quad + 8h2 + i.
      const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)kvh * a.G + (col ? n : 0)) * D;
      if constexpr (MX) {
        // MXFP8 query: each 32-dim group of the head gets the E8M0 scale 2^k
        // of the KV quantizer (the smallest with amax <= 448 * 2^k) and codes
        // e4m3(q * 2^-k) (an exact scaling).  The lane holds dims 128x +
        // 16quad .. +15 (bytes 0-15) and 128x + 64 + 16quad .. +15 (bytes
        // 16-31): halves of groups 4x + quad/2 and 4x + 2 + quad/2, whose
        // other halves sit in the lane 16 apart (quad ^ 1).  Its scale operand
        // is group 4x + quad's, found in lane n + 32 * (quad & 1).
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          uint32_t wv[16];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const u32x4 v =
                  col ? ld_global<u32x4>(qrow + 128 * x + 64 * h + 16 * quad + 8 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
              for (int j = 0; j < 4; ++j) wv[8 * h + 4 * c + j] = v[j];
            }
          float am[2] = {0.0f, 0.0f};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              am[h] = fmaxf(am[h], fmaxf(fabsf(bf16_to_f32((uint16_t)wv[8 * h + j])),
                                         fabsf(bf16_to_f32((uint16_t)(wv[8 * h + j] >> 16)))));
            am[h] = pair_max16(am[h]);
          }
          const uint32_t u0 = e8m0_code(am[0]), u1 = e8m0_code(am[1]);
          v8i32 codes;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int sh = 127 - (int)(h ? u1 : u0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t w0 = wv[8 * h + 2 * j], w1 = wv[8 * h + 2 * j + 1];
              const uint32_t c0 = f32_to_e4m3(__builtin_amdgcn_ldexpf(bf16_to_f32((uint16_t)w0), sh));
              const uint32_t c1 = f32_to_e4m3(__builtin_amdgcn_ldexpf(bf16_to_f32((uint16_t)(w0 >> 16)), sh));
              const uint32_t c2 = f32_to_e4m3(__builtin_amdgcn_ldexpf(bf16_to_f32((uint16_t)w1), sh));
              const uint32_t c3 = f32_to_e4m3(__builtin_amdgcn_ldexpf(bf16_to_f32((uint16_t)(w1 >> 16)), sh));
              codes[4 * h + j] = (int)(c0 | (c1 << 8) | (c2 << 16) | (c3 << 24));
            }
          }
          qmx[x] = codes;
          const int src = n + 32 * (quad & 1);
          const uint32_t g0 = (uint32_t)__shfl((int)u0, src), g1 = (uint32_t)__shfl((int)u1, src);
          qmxs[x] = quad >= 2 ? g1 : g0;
        }
      } else {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            u32x4 v = col ? ld_global<u32x4>(qrow + 64 * m + 16 * quad + 8 * h2) : u32x4{0, 0, 0, 0};
            qop[2 * m + h2] = __builtin_bit_cast(bf16x8, v);
          }
      }
      if constexpr (F8 && !MX) {
        // The row's amax (the four quads of a head column hold its dims),
        // its scale fp32(amax / 448) (1 for a zero row), and the codes
        // e4m3(fp32(q / scale)) with the IEEE-rounded quotient (the rule of
        // the KV quantizer), byte i of a dword pair = dim i of the operand.
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const u32x4 v = __builtin_bit_cast(u32x4, qop[i]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            am = fmaxf(am, fmaxf(fabsf(bf16_to_f32((uint16_t)v[j])), fabsf(bf16_to_f32((uint16_t)(v[j] >> 16)))));
        }
        am = pair_max32(pair_max16(am));
        qsc = am > 0.0f ? am / 448.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const u32x4 v = __builtin_bit_cast(u32x4, qop[i]);
          uint64_t c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            c |= (uint64_t)f32_to_e4m3(bf16_to_f32((uint16_t)v[j]) / qsc) << (16 * j);
            c |= (uint64_t)f32_to_e4m3(bf16_to_f32((uint16_t)(v[j] >> 16)) / qsc) << (16 * j + 8);
          }
          qop8[i] = c;
        }
      }
    }
    m_run = kNegInf;
    l_run = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ca = ta; ca < tc; ca += CH) {
      const int cb = tc < ca + CH ? tc : ca + CH;
      chunk_rows(ca, cb);
      if (!staged) {
        __syncthreads();   // earlier readers of the stage are done
        bool bad = false;
        for (int i = threadIdx.x; i < nstaged; i += NT) s_tab[i] = chk_row(btr[p_first + i], bad);
        flag(bad, 0);
        __syncthreads();
      }
      staged = false;
      // ---- tile loop: wave w takes tiles ca + w, ca + w + 4, ...
      // (PS: every wave takes every tile, for its own KV head.)
      const int nmine = PS ? cb - ca : (cb - ca > wave ? (cb - ca - wave + NW - 1) / NW : 0);
      auto tile_pos = [&](int k) { return PS ? tbeg + (ca + k) * TT : tbeg + (ca + wave + NW * k) * TT; };
      // Fused append: a segment that holds its unit's last tile holds the
      // only tile that reads the new token's page (position L - 1; groups
      // past L read a clamped page of that tile).  The last wave, which has
      // the fewest tiles, quantizes the token into K and V while the others
      // stream, then publishes the segment number; the wave that reads the
      // last tile waits for it before loading that tile.
      const bool app = FUSED && tc == nb;
      if (app && ca == ta && wave == NW - 1) {
        const int pos = L - 1;
        const int32_t row = btr[pos >> log2P];
        const size_t xo = ((size_t)b * Hkv + g) * D;
        append_token_wave(a.kw, a.kg, SK, row, g, D, pos & (P - 1), a.k_new + xo);
        append_token_wave(a.vw, a.vg, SK, row, g, D, pos & (P - 1), a.v_new + xo);
        __hip_atomic_store(&s_app, seg_no, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      auto await_append = [&](int k) {
        if (app && ca + wave + NW * k == tc - 1)
          while (__hip_atomic_load(&s_app, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != seg_no)
            __builtin_amdgcn_s_sleep(1);
      };
      {
        TileT A;
        for (int k = 0; k < nmine; ++k) {
          if constexpr (FUSED) await_append(k);
          load_tile(A, tile_pos(k));
          compute_tile(A, tile_pos(k));
        }
      }
    }

    // ---- combine the waves' states in LDS.
    float lsum = l_run;
    lsum = pair_sum32(pair_sum16(lsum));
    // Wave combine, in the order ((w0 + w2) + (w1 + w3)).  The combine
    // buffer s_o may overlap the page-row and V stages, all read for the last
    // time before the barrier below.
    //  - Sliced (head dim 64, and 128 with page or E8M0 scales): the waves'
    //    rescaled accumulators go to LDS ([NW][NC][G][16]) and each wave sums
    //    its NC/4 16-dim chunks over the four waves, then stores those chunks
    //    of the output or partial.
    //  - Otherwise a pairwise tree ([NW/2][G][D+4]): waves 2, 3 hand their
    //    accumulators to waves 0, 1, then wave 1 to wave 0, which stores
    //    everything (the sliced form spills registers in those kernels).
    float* s_o = s_work;
    constexpr bool SLICED = D == 64 || (D == 128 && (SK == 0 || SK == 2));
    constexpr int CPW = NC / NW;   // chunks each wave sums (sliced)
    static_assert(NW == 4 && CPW >= 1, "four-wave combine");
    auto owned = [&](int c) { return SLICED ? c / CPW == wave : wave == 0; };
    if (quad == 0) {
      s_m[wave][n] = m_run;
      s_l[wave][n] = lsum;
    }
    __syncthreads();   // also: every wave is past its last read of the page-row stage
    // (PS: each wave's state is already its KV head's whole segment.)
    float M = kNegInf;
    if constexpr (PS) {
      M = m_run;
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) M = fmaxf(M, s_m[i][n]);
    }
    const float M_ref = (M == kNegInf) ? 0.0f : M;
    float Ltot = 0.0f;
    if constexpr (PS) {
      Ltot = lsum;
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) Ltot += s_l[i][n] * __builtin_amdgcn_exp2f(s_m[i][n] - M_ref);
      {
        const float f = __builtin_amdgcn_exp2f(m_run - M_ref);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] *= f;
      }
      if constexpr (SLICED) {
        if (col) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            *reinterpret_cast<f32x4*>(s_o + ((wave * NC + c) * G + n) * 16 + 4 * quad) = acc[c];
        }
        __syncthreads();
        if (col) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if (!owned(c)) continue;
            const float* src = s_o + (c * G + n) * 16 + 4 * quad;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + NC * G * 16);
            const f32x4 v2 = *reinterpret_cast<const f32x4*>(src + 2 * NC * G * 16);
            const f32x4 v3 = *reinterpret_cast<const f32x4*>(src + 3 * NC * G * 16);
            acc[c] = (v0 + v2) + (v1 + v3);
          }
        }
      } else {
        constexpr int OS = D + 4;
#pragma unroll
        for (int half = NW / 2; half >= 1; half >>= 1) {
          if (wave >= half && wave < 2 * half && col) {
            float* dst = s_o + ((wave - half) * G + n) * OS + 4 * quad;
#pragma unroll
            for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(dst + 16 * c) = acc[c];
          }
          __syncthreads();
          if (wave < half && col) {
            // Reads in groups of eight, each group one LDS round trip (read
            // one at a time, the adds waited on every read).
            const float* src = s_o + (wave * G + n) * OS + 4 * quad;
            static_assert(NC % 8 == 0, "whole groups of chunks");
#pragma unroll
            for (int c0 = 0; c0 < NC; c0 += 8) {
              f32x4 t[8];
#pragma unroll
              for (int c = 0; c < 8; ++c) t[c] = *reinterpret_cast<const f32x4*>(src + 16 * (c0 + c));
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[c0 + c] += t[c];
            }
          }
          if (half > 1) __syncthreads();
        }
      }
    }

    const int h = PS ? kvh * a.G + n : g * G + n;   // the lane's query head
    const int prow = PS ? wave * a.G + n : n;         // its row among the unit's G
    if (ta == 0 && tc == nb) {
      // The segment is the whole unit: o = acc / (sum + e^(sink - max)),
      // each wave its own chunks (packed splits: each wave its own rows).
      if (col) {
        float den = Ltot;
        if (a.sinks) den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - M_ref);
        const float inv = (M == kNegInf || !(den > 0.0f)) ? 0.0f : __builtin_amdgcn_rcpf(den);
        uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * D + 4 * quad;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (!PS && !owned(c)) continue;
          u32x2 pk = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv), pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
          *reinterpret_cast<u32x2*>(orow + 16 * c) = pk;
        }
      }
    } else {
      // ---- partial of this segment, then its flag (or, for the unit's last
      // piece, a merge at the end of the share).  Partials are written and
      // read with sc1 (agent-coherent) accesses, which on this multi-XCD part
      // are coherent across the per-XCD L2 caches without a cache write-back
      // or invalidate.
      const size_t pbase = ((size_t)sw * 2 + slot) * G;
      const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(a.part_o, (uint32_t)((size_t)gridDim.x * 2 * G * D * 4));
      if (col) {
        // Lane (head n, quad) holds dims 16c + 4quad .. +3: one 16-byte store
        // per c, each wave its own chunks (packed splits: its own rows).
        const float inv = (Ltot > 0.0f) ? __builtin_amdgcn_rcpf(Ltot) : 0.0f;
        const uint32_t row = (uint32_t)((pbase + prow) * D * 4) + 16 * quad;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (PS || owned(c)) st_coherent4(prs, row + 64 * c, acc[c] * inv);
        if (quad == 0 && (PS || wave == 0))
          __hip_atomic_store(a.part_lse + pbase + prow,
                             (M == kNegInf || !(Ltot > 0.0f)) ? kNegInf : M + __builtin_amdgcn_logf(Ltot),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const int s_a = share_of_cost(tile_cost(b, g, 0)), s_b = share_of_cost(tile_cost(b, g, nb - 1));
      if (sw == merger_share(s_a, s_b)) {
        // This share merges the unit, at its end.
        pend_b[npend] = b;
        pend_g[npend] = g;
        pend_sa[npend] = s_a;
        pend_sb[npend] = s_b;
        // s_a's share holds an earlier segment (so this unit sits in its
        // last slot) iff it starts at or before the previous unit's last
        // tile, whose cost start is SC + TC below this unit's first.
        pend_fsa[npend] = floordiv((int64_t)s_a * Ct, W) <= tile_cost(b, g, 0) - SC - TC ? 1 : 0;
        ++npend;
      } else {
        // Every wave wrote part of the partial: once all its stores have
        // completed at the coherence point, the slot is published.  (A merger
        // waits for its own stores when its merge begins.)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
          __hip_atomic_store(a.flags + 2 * sw + slot, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();   // LDS is reused by the next segment
    cur = send;
    slot = 1;
  }

  for (int pi = 0; pi < npend; ++pi) {
    // ---- merge a unit whose pieces are held by shares w_a..s_b (this share
    // among them); w_a holds it in its last slot when its share began before
    // the unit, every other one in its first slot.
    const int w_a = pend_sa[pi];
    const int nseg = pend_sb[pi] - w_a + 1;
    const int first_slot_a = pend_fsa[pi];
    auto slot_of = [&](int wi) -> int { return wi == w_a ? first_slot_a : 0; };
    auto part_row = [&](int wi) -> uint32_t { return (uint32_t)(((size_t)wi * 2 + slot_of(wi)) * G); };
    __builtin_amdgcn_s_waitcnt(0);   // every wave's part of this workgroup's own partial is complete
    if (threadIdx.x == 0) s_timeout = 0;
    __syncthreads();
    // Wait for the other holders' flags.  Their workgroups have lower
    // indices, so they were dispatched first and never wait on this
    // workgroup; the wait is bounded all the same: a merge that gives up
    // writes NaN outputs and counts itself in the device status word.
    for (int i = threadIdx.x; i < nseg; i += NT) {
      if (w_a + i == sw) continue;
      const uint32_t* f = a.flags + 2 * (w_a + i) + slot_of(w_a + i);
      int spins = 0;
      while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.wait_epoch) {
        if (++spins > a.spin_limit) {
          s_timeout = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_timeout)
      __hip_atomic_fetch_add(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int bq = pend_b[pi], gq = pend_g[pi];
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(a.part_o, (uint32_t)((size_t)gridDim.x * 2 * G * D * 4));
    // Merged 64 partials at a time with a running maximum per head (the sink
    // is the initial maximum, with weight 1): per chunk the weights go to LDS
    // and every thread accumulates float4 groups of the G x D outputs in
    // registers.
    constexpr int CHS = 64;   // partials per chunk
    constexpr int NJ = D >= 512 ? 4 : (D >= 256 ? 2 : 1);   // float4 groups per thread per pass
    constexpr int KB = 8;     // partials whose loads are in flight together
    const int ngrp = G * D / 4;
    float* s_wt = s_work;     // [G][CHS]
    constexpr int KF = NJ == 1 ? 32 : 4;   // most partials merged in registers
    if (NJ <= 2 && nseg <= KF && ngrp <= NT * NJ) {
      // Few partials, one pass, head dim <= 256: every thread issues the lse
      // values and the float4 groups of its heads together (one round trip)
      // and merges them in registers, in the same order and arithmetic as the
      // chunked path.  (At head dim 512 the chunked path measured faster.)
      // KFv loads per group are issued whatever nseg is, so up to 16 partials
      // take the shorter form.
      auto reg_merge = [&]<int KFv>() {
        constexpr uint32_t kNone = 0xFFFFFFF0u;   // past the buffer: reads zero
        int hhj[NJ];
        bool okj[NJ];
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gi = threadIdx.x + NT * j;
          okj[j] = gi < ngrp;
          hhj[j] = okj[j] ? (4 * gi) / D : 0;
        }
        f32x4 ov[NJ][KFv];
        float lv[NJ][KFv];
  #pragma unroll
        for (int k = 0; k < KFv; ++k) {
          const bool ok = k < nseg;
          const uint32_t row = ok ? part_row(w_a + k) : 0u;
  #pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t gi = threadIdx.x + (uint32_t)NT * j;
            ov[j][k] = ld_coherent4(prs, (ok && okj[j]) ? row * (uint32_t)D * 4u + 16u * gi : kNone);
            lv[j][k] = ok ? __hip_atomic_load(a.part_lse + row + hhj[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : kNegInf;
          }
        }
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (!okj[j]) continue;
          const int gi = threadIdx.x + NT * j;
          const int hh = hhj[j], d = 4 * gi - hh * D;
          const float sk = a.sinks ? a.sinks[gq * G + hh] * kLog2e : kNegInf;
          float M = sk;
  #pragma unroll
          for (int k = 0; k < KFv; ++k) M = fmaxf(M, lv[j][k]);
          float den = (sk != kNegInf) ? __builtin_amdgcn_exp2f(sk - M) : 0.0f;
          f32x4 num = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int k = 0; k < KFv; ++k) {
            const float wv = (lv[j][k] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(lv[j][k] - M);
            den += wv;
            num += ov[j][k] * wv;
          }
          const float inv = (M == kNegInf || !(den > 0.0f)) ? 0.0f : __builtin_amdgcn_rcpf(den);
          const f32x4 o = num * inv;
          u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          if (s_timeout) pk = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
          *reinterpret_cast<u32x2*>(a.out + ((size_t)bq * a.Hq + gq * G + hh) * D + d) = pk;
        }
      };
      if constexpr (NJ == 1) {
        if (nseg <= 16)
          reg_merge.template operator()<16>();
        else
          reg_merge.template operator()<KF>();
      } else {
        // The same steps written out at KF = 4 (head dim 256): called through
        // the lambda, that kernel's main loop compiled to slower code.
        constexpr uint32_t kNone = 0xFFFFFFF0u;   // past the buffer: reads zero
        int hhj[NJ];
        bool okj[NJ];
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gi = threadIdx.x + NT * j;
          okj[j] = gi < ngrp;
          hhj[j] = okj[j] ? (4 * gi) / D : 0;
        }
        f32x4 ov[NJ][KF];
        float lv[NJ][KF];
  #pragma unroll
        for (int k = 0; k < KF; ++k) {
          const bool ok = k < nseg;
          const uint32_t row = ok ? part_row(w_a + k) : 0u;
  #pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t gi = threadIdx.x + (uint32_t)NT * j;
            ov[j][k] = ld_coherent4(prs, (ok && okj[j]) ? row * (uint32_t)D * 4u + 16u * gi : kNone);
            lv[j][k] = ok ? __hip_atomic_load(a.part_lse + row + hhj[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : kNegInf;
          }
        }
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (!okj[j]) continue;
          const int gi = threadIdx.x + NT * j;
          const int hh = hhj[j], d = 4 * gi - hh * D;
          const float sk = a.sinks ? a.sinks[gq * G + hh] * kLog2e : kNegInf;
          float M = sk;
  #pragma unroll
          for (int k = 0; k < KF; ++k) M = fmaxf(M, lv[j][k]);
          float den = (sk != kNegInf) ? __builtin_amdgcn_exp2f(sk - M) : 0.0f;
          f32x4 num = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int k = 0; k < KF; ++k) {
            const float wv = (lv[j][k] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(lv[j][k] - M);
            den += wv;
            num += ov[j][k] * wv;
          }
          const float inv = (M == kNegInf || !(den > 0.0f)) ? 0.0f : __builtin_amdgcn_rcpf(den);
          const f32x4 o = num * inv;
          u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          if (s_timeout) pk = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
          *reinterpret_cast<u32x2*>(a.out + ((size_t)bq * a.Hq + gq * G + hh) * D + d) = pk;
        }
      }
    } else {
      for (int pass0 = 0; pass0 < ngrp; pass0 += NT * NJ) {
        f32x4 num[NJ];
  #pragma unroll
        for (int j = 0; j < NJ; ++j) num[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (threadIdx.x < G) {
          const float sk = a.sinks ? a.sinks[gq * G + threadIdx.x] * kLog2e : kNegInf;
          s_M[threadIdx.x] = sk;
          s_den[threadIdx.x] = (sk != kNegInf) ? 1.0f : 0.0f;
        }
        // Loads of KB partials x NJ groups are issued together; absent ones
        // use an offset past the buffer's range, which reads zero.
        constexpr uint32_t kNone = 0xFFFFFFF0u;
        int hhj[NJ];
        uint32_t offj[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gi = pass0 + threadIdx.x + NT * j;
          hhj[j] = gi < ngrp ? (4 * gi) / D : 0;
          offj[j] = gi < ngrp ? (uint32_t)(16 * gi) : kNone;
        }
        f32x4 ov[NJ][KB];
        auto issue = [&](int c0, int k0, int nc) {
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const bool ok = k0 + kk < nc;
            const uint32_t rb = ok ? part_row(w_a + c0 + k0 + kk) * (uint32_t)D * 4u : 0u;
#pragma unroll
            for (int j = 0; j < NJ; ++j) ov[j][kk] = ld_coherent4(prs, (ok && offj[j] != kNone) ? rb + offj[j] : kNone);
          }
        };
        for (int c0 = 0; c0 < nseg; c0 += CHS) {
          const int nc = nseg - c0 < CHS ? nseg - c0 : CHS;
          issue(c0, 0, nc);   // the first partials' loads overlap the round trip of the weights
          for (int i = threadIdx.x; i < G * CHS; i += NT) {
            const int hh = i / CHS, k = i - hh * CHS;
            s_wt[i] = k < nc ? __hip_atomic_load(a.part_lse + part_row(w_a + c0 + k) + hh, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : kNegInf;
          }
          __syncthreads();
          if (threadIdx.x < G) {
            const int hh = threadIdx.x;
            const float Mo = s_M[hh];
            float Mn = Mo;
            for (int k = 0; k < nc; ++k) Mn = fmaxf(Mn, s_wt[hh * CHS + k]);
            const float sc = (Mo == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(Mo - Mn);
            float den = s_den[hh] * sc;
            for (int k = 0; k < nc; ++k) {
              const float l = s_wt[hh * CHS + k];
              const float wv = (l == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(l - Mn);
              s_wt[hh * CHS + k] = wv;
              den += wv;
            }
            s_M[hh] = Mn;
            s_den[hh] = den;
            s_sc[hh] = sc;
          }
          __syncthreads();
          {
  #pragma unroll
            for (int j = 0; j < NJ; ++j) num[j] *= s_sc[hhj[j]];
            for (int k0 = 0; k0 < nc; k0 += KB) {
              if (k0 > 0) issue(c0, k0, nc);
  #pragma unroll
              for (int kk = 0; kk < KB; ++kk) {
                const int kx = k0 + kk < CHS ? k0 + kk : CHS - 1;
  #pragma unroll
                for (int j = 0; j < NJ; ++j) {
                  const float wv = (k0 + kk < nc) ? s_wt[hhj[j] * CHS + kx] : 0.0f;
                  num[j] += ov[j][kk] * wv;
                }
              }
            }
          }
          __syncthreads();   // s_wt, s_M, s_den are rewritten next
        }
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gi = pass0 + threadIdx.x + NT * j;
          if (gi < ngrp) {
            const int hh = (4 * gi) / D, d = 4 * gi - hh * D;
            const float den = s_den[hh];
            const float inv = (s_M[hh] == kNegInf || !(den > 0.0f)) ? 0.0f : __builtin_amdgcn_rcpf(den);
            const f32x4 o = num[j] * inv;
            u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            if (s_timeout) pk = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
            *reinterpret_cast<u32x2*>(a.out + ((size_t)bq * a.Hq + gq * G + hh) * D + d) = pk;
          }
        }
        __syncthreads();   // every thread has read s_M / s_den before the next pass resets them
      }
    }
    // Clear the consumed flags (a replayed graph reuses the epoch).
    for (int i = threadIdx.x; i < nseg; i += NT)
      if (w_a + i != sw)
        __hip_atomic_store(a.flags + 2 * (w_a + i) + slot_of(w_a + i), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();   // s_timeout and the LDS weights are reused by the next merge
  }
}

template <int D, bool KNT, bool FUSED, bool VT = false, bool F8 = false, bool PK = false, bool PS = false>
hipError_t launch_d(const DecodeArgs& a, int sk, int W, size_t lds, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  dim3 grid(W), block(64 * Shape<D>::NW);
  switch (sk) {
    case 0:
      hipExtLaunchKernelGGL((decode_kernel<D, 0, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    case 1:
      hipExtLaunchKernelGGL((decode_kernel<D, 1, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    case 2:
      if constexpr (F8 && D % 128) return hipErrorNotSupported;
      else hipExtLaunchKernelGGL((decode_kernel<D, 2, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    case 3:    // fp32 sub-row K scales (groups of 16 dims or more), V per (token, head)
      if constexpr (F8 || FUSED || PK || PS) return hipErrorNotSupported;
      else hipExtLaunchKernelGGL((decode_kernel<D, 3, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    case 4:    // fp32 sub-row K and V scales
      if constexpr (F8 || FUSED || PK || PS) return hipErrorNotSupported;
      else hipExtLaunchKernelGGL((decode_kernel<D, 4, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    case 5:    // K groups of 8 dims, V per (token, head)
      if constexpr (F8 || FUSED || PK || PS) return hipErrorNotSupported;
      else hipExtLaunchKernelGGL((decode_kernel<D, 5, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
    default:   // K groups of 8 dims, V in groups
      if constexpr (F8 || FUSED || PK || PS) return hipErrorNotSupported;
      else hipExtLaunchKernelGGL((decode_kernel<D, 6, KNT, FUSED, VT, F8, PK, PS>), grid, block, lds, st, e0, e1, 0, a);
      break;
  }
  return hipGetLastError();
}

// Launch of one kernel family (FUSED, VT, F8, PK, PS) at the head dim and K
// line coverage of the call.
template <bool FUSED, bool VT = false, bool F8 = false, bool PK = false, bool PS = false>
hipError_t launch_family(const DecodeArgs& a, int D, int sk, bool k_whole_lines, int W, size_t lds, hipStream_t st,
                         hipEvent_t e0, hipEvent_t e1) {
  return with_head_dim(D, [&]<int DD>() {
    return k_whole_lines ? launch_d<DD, true, FUSED, VT, F8, PK, PS>(a, sk, W, lds, st, e0, e1)
                         : launch_d<DD, false, FUSED, VT, F8, PK, PS>(a, sk, W, lds, st, e0, e1);
  });
}

template <int D, bool KNT>
int occupancy_d(int sk, size_t lds) {
  int nb = 0;
  hipError_t e;
  constexpr int NT = 64 * Shape<D>::NW;
  switch (sk) {
    case 0: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 0, KNT, false, false>, NT, lds); break;
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 1, KNT, false, false>, NT, lds); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 2, KNT, false, false>, NT, lds); break;
    case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 3, KNT, false, false>, NT, lds); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 4, KNT, false, false>, NT, lds); break;
    case 5: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 5, KNT, false, false>, NT, lds); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel<D, 6, KNT, false, false>, NT, lds); break;
  }
  return e == hipSuccess ? nb : -1;
}

}  // namespace
}  // namespace fp8pa
