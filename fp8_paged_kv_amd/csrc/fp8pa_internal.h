// Internal interface between the C-ABI host layer (api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/fp8pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8pa {

// Byte geometry of one pool, resolved on the host from fp8pa_pool_desc.
// Code of (KV head h, in-page token t, dim d) sits at
//   h*head_stride + (t / tblk)*tblk_stride + (t % tblk)*tok_stride
//     + (d / 64)*dchunk_stride + (d % 64)*d_stride
struct PoolGeom {
  int64_t row_bytes;
  int32_t head_stride;     // payload bytes between KV heads of a row
  int32_t tblk;            // tokens per token block (a power of two; P if unblocked)
  int32_t tblk_stride;     // bytes between token blocks
  int32_t tok_stride;      // bytes between tokens inside a block
  int32_t dchunk_stride;   // bytes between 64-dim chunks
  int32_t d_stride;        // bytes between dims inside a chunk
  int32_t sc_off;          // scale footer offset in the row
  int32_t sc_head_stride;  // footer bytes between heads
  int32_t sc_tok_stride;   // footer bytes between tokens (0 for per-page scales)
  int32_t align64;         // rows placed by FP8PA_POOL_ALIGN64
  int32_t payload_bytes;   // P * Hkv * D
  int32_t scale_bytes;     // bytes of a row's scale block
  int32_t sc_gshift;       // fp32 sub-row scales: log2 of the dims per scale (else 0)
};

// Byte offsets, from the pool base, of row r's payload and scale block
// (0 <= r < 2^31 and row_bytes < 2^31: one 32 x 32 -> 64-bit multiply).
struct RowBases {
  int64_t code, scale;
};
__host__ __device__ inline RowBases row_bases(const PoolGeom& g, int64_t r) {
  const int64_t base = (int64_t)((uint64_t)(uint32_t)r * (uint64_t)(uint32_t)g.row_bytes);
  if (!g.align64) return {base, base + g.sc_off};
  const int64_t sh = (-base) & 63;
  return {base + sh, sh >= g.scale_bytes ? base : base + sh + g.payload_bytes};
}

struct DecodeArgs {
  const uint16_t* q;       // bf16 [B, Hq, D]
  uint16_t* out;           // bf16 [B, Hq, D]
  const uint8_t* kp;
  const uint8_t* vp;
  const int32_t* bt;       // [B, bt_stride]
  int64_t bt_stride;
  const int32_t* seq_lens;
  const float* sinks;      // [Hq] or null
  const uint16_t* k_new;   // fused append: bf16 [B, Hkv, D], the token at position seq_lens[b] - 1; or null
  const uint16_t* v_new;
  uint8_t* kw;             // the pools, writable (fused append only)
  uint8_t* vw;
  float* part_o;           // [W][2][G][D] partial outputs (first / last segment of a workgroup)
  float* part_lse;         // [W][2][G] base-2 log-sum-exp of each partial
  uint32_t* flags;         // [W][2] a slot's flag holds the call's epoch once its partial is complete
  uint32_t epoch;          // distinct per call, never 0 (cleared flags hold 0)
  uint32_t wait_epoch;     // the flag value a merger waits for (= epoch)
  int32_t spin_limit;      // sleeps after which a merger's wait for a flag gives up
  uint32_t* status;        // device status words: [0] counts merges whose wait gave up
  int32_t min_tiles;       // fewest tiles per active workgroup (>= 1)
  int32_t seg_cost;        // fixed cost of a unit in the share balance, in quarter tiles (>= 0)
  PoolGeom kg, vg;
  int32_t P, log2P, B, Hq, Hkv, G, window;
  float qk_scale;          // sm_scale * log2(e)
  int32_t vstage_off;      // V token-major: byte offset of the per-wave V stages in dynamic LDS
  int32_t vgstage_off;     // V sub-row scales: byte offset of the per-wave scale stages in dynamic LDS
  uint32_t* dbg;           // debug checks: error words [2] (table, lengths), or null (no checks)
  int32_t dbg_rows;        // rows of the smaller pool (debug checks)
  int32_t dbg_max_len;     // largest valid seq_lens[b] (debug checks)
};

struct MergeArgs {
  const float* part_o;     // [B, Hq, S, D]
  const float* part_lse;   // [B, Hq, S]
  const float* sinks;
  uint16_t* out;
  int32_t Hq, S, D;
  int32_t G;               // query heads merged per workgroup (divides Hq, <= 16)
};

struct AppendArgs {
  const uint16_t* k_new;   // bf16 [B, T, Hkv, D]
  const uint16_t* v_new;
  uint8_t* kp;
  uint8_t* vp;
  PoolGeom kg, vg;
  int32_t k_kind, v_kind;  // FP8PA_SCALE_*
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* positions; // or null: one token per sequence, at seq_lens[b] - 1
  const int32_t* counts;   // or null
  const int32_t* seq_lens; // with positions null
  int32_t T, P, Hkv, D;
  uint32_t* dbg;           // as in DecodeArgs
  int32_t dbg_rows;
};

// Kernel shape of each head dim: NS (a tile is 32*NS positions), the
// occupancy the kernel is compiled for (OCC waves per SIMD), waves per
// workgroup (NW), workgroups launched per CU (WPC), and a unit's fixed cost in
// the share balance, in quarter tiles (SC).  At head dim 128 one four-wave
// workgroup per CU streams as fast as two and cuts half as many units.
template <int D>
struct Shape;
template <>
struct Shape<64> { static constexpr int NS = 2, OCC = 2, NW = 4, WPC = 2, SC = 24; };
template <>
struct Shape<128> { static constexpr int NS = 2, OCC = 2, NW = 4, WPC = 1, SC = 48; };
template <>
struct Shape<256> { static constexpr int NS = 1, OCC = 1, NW = 4, WPC = 1, SC = 24; };
template <>
struct Shape<512> { static constexpr int NS = 1, OCC = 1, NW = 4, WPC = 1, SC = 24; };

// f.template operator()<D>() for a supported head dim D (64, 128, 256, 512).
template <typename F>
auto with_head_dim(int D, F&& f) {
  switch (D) {
    case 64: return f.template operator()<64>();
    case 128: return f.template operator()<128>();
    case 256: return f.template operator()<256>();
    default: return f.template operator()<512>();
  }
}

// Tokens per decode tile (one tile = one MFMA round of one wave), wave64s per
// decode workgroup, and a unit's default fixed cost in the share balance.
inline int decode_tile_tokens(int D) {
  return with_head_dim(D, []<int DD>() { return 32 * Shape<DD>::NS; });
}
inline int decode_waves(int D) {
  return with_head_dim(D, []<int DD>() { return Shape<DD>::NW; });
}
inline int decode_seg_cost(int D) {
  return with_head_dim(D, []<int DD>() { return Shape<DD>::SC; });
}
inline int decode_wg_per_cu(int D) {
  return with_head_dim(D, []<int DD>() { return Shape<DD>::WPC; });
}

// Positions whose page rows a workgroup stages in LDS at once.
constexpr int kMaxSplitTokens = 16384;

// V token-major (VT): the stage of a wave holds a tile's positions as rows of
// VH dims, RS bytes apart (16 bytes of padding spread the 8 rows of a
// transpose read over distinct banks); D > VH takes D/VH passes.
template <int D>
struct VStage {
  static constexpr int VH = D < 128 ? D : 128;   // dims per pass
  static constexpr int RS = VH + 16;             // stage row stride, bytes
};

// Dynamic LDS of a decode launch: the tile and non-empty prefixes and the
// lengths (3 words per sequence), then the page-row stage (decode_stage_end),
// after which the token-major V and V-scale stages go; the wave-combine
// buffer starts after the prefixes too and may overlap all three stages (they
// are dead while the waves combine), so the launch needs at least
// decode_lds_bytes.  The combine holds the four waves' accumulators of G
// rows up to head dim 128, and two waves' rows of D + 4 floats above.
inline size_t decode_prefix_bytes(int64_t B) { return (size_t)3 * ((B + 4) & ~int64_t(3)) * 4; }
inline size_t decode_stage_end(int D, int64_t B, int P) {
  const int TT = decode_tile_tokens(D);
  return decode_prefix_bytes(B) + (size_t)(kMaxSplitTokens / TT * TT / P + 2) * 4;
}
inline size_t decode_combine_bytes(int D, int G) {
  return D <= 128 ? (size_t)decode_waves(D) * G * D * 4 : (size_t)(decode_waves(D) / 2) * G * (D + 4) * 4;
}
inline size_t decode_lds_bytes(int D, int B, int G, int P) {
  const size_t st = decode_stage_end(D, B, P), cb = decode_prefix_bytes(B) + decode_combine_bytes(D, G);
  return st > cb ? st : cb;
}

// The per-wave V stages a token-major V pool adds (+ slack to align them to
// 16 bytes).
inline size_t decode_vstage_bytes(int D) {
  return with_head_dim(D, []<int DD>() -> size_t {
    return (size_t)Shape<DD>::NW * 32 * Shape<DD>::NS * VStage<DD>::RS + 16;
  });
}

// Dynamic LDS of a decode launch, resident workgroups per CU, and the launch
// itself (start/stop: optional events that time the decode kernel alone;
// k_whole_lines: the K layout lets every 16-byte K load of a wave cover whole
// 128-byte lines, so non-temporal loads are used).
int decode_blocks_per_cu(int D, int scale_kind, bool k_whole_lines, size_t lds);
// Device address of the current device's status words (see DecodeArgs::status),
// or null if it cannot be resolved.
uint32_t* device_status_words();
// Device address of the current device's copy of the allocation-free decode's
// scratch (FP8PA_NOALLOC_SCRATCH_BYTES, 256-byte aligned), or null if it
// cannot be resolved.
uint8_t* device_scratch();
hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                         hipStream_t st, hipEvent_t start, hipEvent_t stop);
// The same with the new tokens appended in-kernel (a.k_new, a.v_new).
hipError_t launch_decode_fused(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                               hipStream_t st, hipEvent_t start, hipEvent_t stop);
// V in a token-major layout (HEADS or TOKENS), staged through LDS.
hipError_t launch_decode_vtok(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                              hipStream_t st, hipEvent_t start, hipEvent_t stop);
// The fp8 compute mode (fp8 MFMA for QK^T over E4M3-rounded queries), default
// kernel shapes, fp32 scales only.
hipError_t launch_decode_fp8q(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                              hipStream_t st, hipEvent_t start, hipEvent_t stop);
// Packed heads: grid B * ceil(Hkv / decode_waves(D, 0)), no splits, default
// kernel shapes.
hipError_t launch_decode_packed(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                hipStream_t st, hipEvent_t start, hipEvent_t stop);
// Packed heads with V in a token-major layout (a.vstage_off set).
hipError_t launch_decode_packed_vt(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                   hipStream_t st, hipEvent_t start, hipEvent_t stop);
// Packed heads with splits: units of decode_waves(D, 0) KV heads (a.G and
// a.Hkv are the per-KV-head values), default kernel shapes.
hipError_t launch_decode_pksplit(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                                 hipStream_t st, hipEvent_t start, hipEvent_t stop);
hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int B, int max_pages, hipStream_t st);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_debug_dequant(const uint8_t* codes, const void* scales, int kind, int n,
                                float* out, hipStream_t st);

}  // namespace fp8pa
