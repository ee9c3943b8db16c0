// Host side of the paged decode: shape policy, LDS sizing, occupancy and the
// launch of the plain (no append) kernels.  The kernel is in decode_kernel.h.
#include <unordered_map>

#include "decode_kernel.h"

namespace fp8pa {

int decode_waves(int D, int tile_variant) {
  auto q = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() { return NW; };
  return by_shape<true>(D, tile_variant, q);
}

int decode_seg_cost(int D, int tile_variant) {
  auto q = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() { return SCD; };
  return by_shape<true>(D, tile_variant, q);
}

size_t decode_lds_bytes(int D, int tile_variant, int B, int G, int P) {
  const int TT = decode_tile_tokens(D, tile_variant);
  const size_t pre = (size_t)3 * ((B + 4) & ~3) * 4;
  const size_t stage = (size_t)(kMaxSplitTokens / TT * TT / P + 2) * 4;
  const size_t combine = (size_t)(decode_waves(D, tile_variant) / 2) * G * (D + 4) * 4;
  return pre + (stage > combine ? stage : combine);
}

int decode_blocks_per_cu(int D, int scale_kind, bool k_whole_lines, int tile_variant, size_t lds) {
  // Workgroups launched per CU: the shape's count, if that many fit.  The
  // occupancy query is a host call; its answers are remembered per thread
  // (they depend only on the kernel and its LDS, the same on every device
  // of this architecture).
  thread_local std::unordered_map<uint64_t, int> memo;
  const uint64_t key = (uint64_t)D | ((uint64_t)scale_kind << 12) | ((uint64_t)k_whole_lines << 14) |
                       ((uint64_t)tile_variant << 16) | ((uint64_t)lds << 24);
  const auto it = memo.find(key);
  if (it != memo.end()) return it->second;
  auto q = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() {
    const int nb = occupancy_d<DD, NS, PF, OCC, KNT, NW>(scale_kind, lds);
    return nb < WPC ? nb : WPC;
  };
  const int r = k_whole_lines ? by_shape<true>(D, tile_variant, q) : by_shape<false>(D, tile_variant, q);
  if (r > 0) memo.emplace(key, r);
  return r;
}

hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                         hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  auto l = [&]<int DD, int NS, bool PF, int OCC, bool KNT, int NW, int WPC, int SCD>() {
    return launch_d<DD, NS, PF, OCC, KNT, NW, false>(a, scale_kind, W, lds, st, e0, e1);
  };
  return k_whole_lines ? by_shape<true>(D, a.tile_variant, l) : by_shape<false>(D, a.tile_variant, l);
}

}  // namespace fp8pa
