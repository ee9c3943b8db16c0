// Host side of the paged decode: LDS sizing, occupancy, the device status
// words and the launch of the plain (no append) kernels.  The kernel is in
// decode_kernel.h.
#include <mutex>
#include <unordered_map>

#include "decode_kernel.h"

namespace fp8pa {

int decode_blocks_per_cu(int D, int scale_kind, bool k_whole_lines, size_t lds) {
  // Workgroups launched per CU: the shape's count, if that many fit.  The
  // occupancy query is a host call; its answers are remembered per thread
  // (they depend only on the kernel and its LDS, the same on every device
  // of this architecture).
  thread_local std::unordered_map<uint64_t, int> memo;
  const uint64_t key = (uint64_t)D | ((uint64_t)scale_kind << 12) | ((uint64_t)k_whole_lines << 14) |
                       ((uint64_t)lds << 24);
  const auto it = memo.find(key);
  if (it != memo.end()) return it->second;
  const int r = with_head_dim(D, [&]<int DD>() {
    const int nb = k_whole_lines ? occupancy_d<DD, true>(scale_kind, lds) : occupancy_d<DD, false>(scale_kind, lds);
    return nb < Shape<DD>::WPC ? nb : Shape<DD>::WPC;
  });
  if (r > 0) memo.emplace(key, r);
  return r;
}

namespace {
// Status words of each device (DecodeArgs::status): one copy per device,
// which holds it until the process ends.
__device__ __align__(16) uint32_t status_words[4];
}  // namespace

uint32_t* device_status_words() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(status_words)) != hipSuccess) return nullptr;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  return addr[dev];
}

hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                         hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
