// Host side of the paged decode: LDS sizing, occupancy, the device status
// words and the launch of the plain (no append) kernels.  The kernel is in
// decode_kernel.h.
#include <mutex>
#include <unordered_map>

#include "decode_kernel.h"
#include "fp8pa.h"

namespace fp8pa {

int decode_blocks_per_cu(int D, int scale_kind, bool k_whole_lines, size_t lds) {
  // Workgroups launched per CU: the shape's count, if that many fit.  The
  // occupancy query is a host call; its answers are remembered per thread
  // (they depend only on the kernel and its LDS, the same on every device
  // of this architecture).
  thread_local std::unordered_map<uint64_t, int> memo;
  const uint64_t key = (uint64_t)D | ((uint64_t)scale_kind << 12) | ((uint64_t)k_whole_lines << 16) |
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
// Status words of each device (DecodeArgs::status), and the scratch of the
// allocation-free decode (fp8pa_decode_noalloc: its split partials, their
// log-sum-exp and flags).  Each device holds its own copy of both until the
// process ends.  In host code these names are host-side stand-ins, not device
// addresses: the addresses come from hipGetSymbolAddress, once per device.
__device__ __align__(16) uint32_t status_words[4];
__device__ __align__(256) uint8_t scratch[FP8PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The current device's address of a device symbol, resolved on the first
// call per device (with that device current) and remembered.
template <typename T>
T* symbol_address(const void* symbol, T* (&cache)[kMaxDevices], std::mutex& mu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, symbol) != hipSuccess || !p) return nullptr;
    cache[dev] = static_cast<T*>(p);
  }
  return cache[dev];
}
}  // namespace

uint32_t* device_status_words() {
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  return symbol_address(HIP_SYMBOL(status_words), addr, mu);
}

uint8_t* device_scratch() {
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  return symbol_address(HIP_SYMBOL(scratch), addr, mu);
}

hipError_t launch_decode(const DecodeArgs& a, int D, int scale_kind, bool k_whole_lines, int W, size_t lds,
                         hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_family<false>(a, D, scale_kind, k_whole_lines, W, lds, st, e0, e1);
}

}  // namespace fp8pa
