// Host-only test of the C ABI (built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_abi.py; no GPU, no HIP
// runtime).  The library's host layer (api.cpp) is compiled into this program
// with stub kernel launchers that record what would be launched, and stub
// HIP runtime calls.  Checked: every refusal returns its status, sets a
// message and launches nothing; accepted calls launch exactly once with
// arguments that stay inside the buffers the caller passed; the plan agrees
// with the call; the epoch generator never hands out 0; random arguments
// never trip the sanitizers.
#include "../../fp8_paged_kv_amd/csrc/api.cpp"

#include <cstdio>
#include <random>
#include <vector>

// ---- stub HIP runtime (host only: no device is present)
static int g_memcpy_fail = 0;
extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  if (g_memcpy_fail) return hipErrorInvalidValue;
  std::memcpy(dst, src, n);
  return hipSuccess;
}
}

// ---- stub launchers: record the launch
struct Launch {
  int kind;   // 0 decode, 1 fused, 2 vtok, 3 fp8, 4 packed, 5 psplit, 6 merge, 7 append, 8 read, 9 dequant,
             // 10 packed with token-major V
  fp8pa::DecodeArgs a;
  int W;
  size_t lds;
  int sk;     // the kernel scale class the launcher was given
};
static std::vector<Launch> g_launches;
static int g_last_sk = -1;   // scale class of the last launch expect_launch made
static uint32_t g_status_stub[4];
alignas(256) static uint8_t g_scratch_stub[FP8PA_NOALLOC_SCRATCH_BYTES];
uint8_t* fp8pa::device_scratch() { return g_scratch_stub; }

namespace fp8pa {
int decode_blocks_per_cu(int D, int, bool, size_t lds) { return lds <= 65536 ? decode_wg_per_cu(D) : 0; }
uint32_t* device_status_words() { return g_status_stub; }
uint8_t* device_scratch();
#define STUB_DECODE(name, k)                                                                                      \
  hipError_t name(const DecodeArgs& a, int, int sk, bool, int W, size_t lds, hipStream_t, hipEvent_t, hipEvent_t) { \
    g_launches.push_back({k, a, W, lds, sk});                                                                     \
    return hipSuccess;                                                                                            \
  }
STUB_DECODE(launch_decode, 0)
STUB_DECODE(launch_decode_fused, 1)
STUB_DECODE(launch_decode_vtok, 2)
STUB_DECODE(launch_decode_fp8q, 3)
STUB_DECODE(launch_decode_packed, 4)
STUB_DECODE(launch_decode_pksplit, 5)
STUB_DECODE(launch_decode_packed_vt, 10)
hipError_t launch_merge(const MergeArgs&, int, hipStream_t) {
  g_launches.push_back({6, {}, 0, 0});
  return hipSuccess;
}
hipError_t launch_append(const AppendArgs&, int, int, hipStream_t) {
  g_launches.push_back({7, {}, 0, 0});
  return hipSuccess;
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) {
  g_launches.push_back({8, {}, 0, 0});
  return hipSuccess;
}
hipError_t launch_debug_dequant(const uint8_t*, const void*, int, int, float*, hipStream_t) {
  g_launches.push_back({9, {}, 0, 0});
  return hipSuccess;
}
}  // namespace fp8pa

// ---- checks
static int g_fail = 0;
#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      std::printf("FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #c, fp8pa_last_error()); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// Fake device addresses: validation never dereferences them.
static uint8_t* fake(uintptr_t a) { return reinterpret_cast<uint8_t*>(a); }
static const uintptr_t F = 0x100000;

static fp8pa_pool_desc desc(int H, int D, int P, int layout, int kind, int64_t rb, int64_t rows = 100) {
  fp8pa_pool_desc d{};
  d.num_kv_heads = H;
  d.head_dim = D;
  d.page_size = P;
  d.layout = layout;
  d.scale_kind = kind;
  d.flags = 0;
  d.row_bytes = rb;
  d.scale_offset = -1;
  d.num_rows = rows;
  return d;
}

struct Call {
  fp8pa_pool_desc kd = desc(8, 128, 16, FP8PA_LAYOUT_HEADS_D64, FP8PA_SCALE_F32_PAGE_HEAD, 16416);
  fp8pa_pool_desc vd = desc(8, 128, 16, FP8PA_LAYOUT_HEADS_DMAJOR, FP8PA_SCALE_F32_PAGE_HEAD, 16416);
  uintptr_t q = F, out = F, kp = F, vp = F, bt = F, sl = F, sinks = 0, ws = 0;
  int64_t bt_stride = 512;
  int B = 4, Hq = 32, window = 0, msl = 8192, workgroups = 0, variant = 0;
  float sm_scale = 0.08f;
  size_t ws_bytes = 0;
  int run() const {
    return fp8pa_decode(fake(q), fake(out), fake(kp), fake(vp), &kd, &vd, reinterpret_cast<const int32_t*>(bt),
                        bt_stride, reinterpret_cast<const int32_t*>(sl), B, Hq, window,
                        reinterpret_cast<const float*>(sinks), sm_scale, msl, workgroups, variant, fake(ws), ws_bytes,
                        nullptr);
  }
  int plan(fp8pa_plan* p) const { return fp8pa_decode_plan(B, Hq, &kd, &vd, msl, window, workgroups, variant, p); }
};

// A refusal: the status, a message, no launch, one more error counted.
static void expect_refusal(const Call& c, int code, int line) {
  g_launches.clear();
  fp8pa_counters before{}, after{};
  fp8pa_get_counters(&before);
  const int rc = c.run();
  fp8pa_get_counters(&after);
  if (rc != code || g_launches.size() != 0 || fp8pa_last_error()[0] == 0 || after.errors != before.errors + 1) {
    std::printf("FAIL line %d: rc %d (want %d), %zu launches, msg '%s'\n", line, rc, code, g_launches.size(),
                fp8pa_last_error());
    ++g_fail;
  }
}
#define REFUSE(c, code) expect_refusal(c, code, __LINE__)

// An accepted call with a workspace of exactly the plan's size: one launch,
// its split buffers inside the workspace, a nonzero epoch.
static void expect_launch(Call c, int line) {
  fp8pa_plan p{};
  int rc = c.plan(&p);
  if (rc != 0) {
    std::printf("FAIL line %d: plan refused (%s)\n", line, fp8pa_last_error());
    ++g_fail;
    return;
  }
  std::vector<uint8_t> ws((size_t)p.workspace_bytes + 256);
  const uintptr_t base = (reinterpret_cast<uintptr_t>(ws.data()) + 255) & ~uintptr_t(255);
  c.ws = p.workspace_bytes > 0 ? base : 0;
  c.ws_bytes = (size_t)p.workspace_bytes;
  g_launches.clear();
  rc = c.run();
  if (rc != 0 || g_launches.size() != 1) {
    std::printf("FAIL line %d: rc %d, %zu launches (%s)\n", line, rc, g_launches.size(), fp8pa_last_error());
    ++g_fail;
    return;
  }
  const Launch& l = g_launches[0];
  g_last_sk = l.sk;
  CHECK(l.W == p.workgroups);
  CHECK(l.lds <= 65536);
  {
    // The wave-combine buffer (which may overlap the stages) fits the launch's LDS.
    const int Gu = c.Hq / c.kd.num_kv_heads * (p.variant == FP8PA_VARIANT_PACKED_SPLIT ? 4 : 1);
    CHECK(l.lds >= fp8pa::decode_lds_bytes(c.kd.head_dim, c.B, Gu, c.kd.page_size));
  }
  CHECK(l.a.epoch != 0 && l.a.wait_epoch == l.a.epoch && l.a.status != nullptr);
  const int kinds[] = {0, 0, 4, 5};   // what each plan variant launches (bf16 may be plain, fused or vtok)
  (void)kinds;
  const bool vt = c.vd.layout == FP8PA_LAYOUT_HEADS || c.vd.layout == FP8PA_LAYOUT_TOKENS;
  if (p.variant == FP8PA_VARIANT_PACKED_HEADS) CHECK(l.kind == (vt ? 10 : 4));
  if (vt) CHECK(l.kind == 2 || l.kind == 10);
  if (vt) CHECK(l.a.vstage_off > 0 && l.lds >= (size_t)l.a.vstage_off + fp8pa::decode_vstage_bytes(c.kd.head_dim));
  // Every kernel but packed heads cuts units when W > 1 and then stores
  // partials and flags: they must point into the workspace.
  if (l.kind != 4 && l.kind != 10 && l.W > 1) CHECK(l.a.part_o && l.a.part_lse && l.a.flags);
  if (l.kind == 4 || l.kind == 10) CHECK(p.workspace_bytes == 0 && l.W == c.B * ((c.kd.num_kv_heads + 3) / 4));
  if (p.variant == FP8PA_VARIANT_PACKED_SPLIT) CHECK(l.kind == 5);
  if (p.variant == FP8PA_VARIANT_MFMA_FP8) CHECK(l.kind == 3);
  if (p.workspace_bytes > 0) {
    const uintptr_t lo = c.ws, hi = c.ws + c.ws_bytes;
    const int64_t G = c.Hq / c.kd.num_kv_heads * (p.variant == FP8PA_VARIANT_PACKED_SPLIT ? 4 : 1);
    const uintptr_t po = reinterpret_cast<uintptr_t>(l.a.part_o), pl = reinterpret_cast<uintptr_t>(l.a.part_lse),
                    pf = reinterpret_cast<uintptr_t>(l.a.flags);
    CHECK(po >= lo && po + (uintptr_t)l.W * 2 * G * c.kd.head_dim * 4 <= hi);
    CHECK(pl >= lo && pl + (uintptr_t)l.W * 2 * G * 4 <= hi);
    CHECK(pf >= lo && pf + (uintptr_t)l.W * 2 * 4 <= hi);
    CHECK(po % 256 == 0 && pl % 256 == 0 && pf % 256 == 0);
    // one byte less is refused
    Call d = c;
    d.ws_bytes -= 1;
    REFUSE(d, FP8PA_EWORKSPACE);
  } else {
    CHECK(l.a.part_o == nullptr);
  }
  CHECK(fp8pa_decode_workspace_bytes(c.B, c.Hq, &c.kd, &c.vd, c.msl, c.window, c.workgroups, c.variant) ==
        p.workspace_bytes);
}
#define LAUNCH(c) expect_launch(c, __LINE__)

int main() {
  // ---- the epoch generator never hands out 0 (mergers clear flags to 0)
  {
    std::atomic<uint32_t> ctr{0xFFFFFFFEu};
    CHECK(next_epoch(ctr) == 0xFFFFFFFFu);
    CHECK(next_epoch(ctr) == 1u);
    CHECK(next_epoch(ctr) == 2u);
    std::atomic<uint32_t> z{0};
    CHECK(next_epoch(z) == 1u);
    g_epoch.store(0xFFFFFFFFu);
    Call c;
    c.workgroups = 1;
    g_launches.clear();
    CHECK(c.run() == 0 && g_launches.size() == 1 && g_launches[0].a.epoch == 1u);
  }

  // ---- refusals of fp8pa_decode
  {
    Call c;
    c.q = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.out = F + 8; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kp = F + 4; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.bt = F + 2; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.sl = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.sinks = F + 2; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.bt_stride = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.bt_stride = 511; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.B = -1; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.Hq = 30; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.Hq = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.Hq = 8 * 17; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.msl = -1; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.workgroups = -1; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.variant = 9; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = -1; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.sm_scale = NAN; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.sm_scale = INFINITY; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.workgroups = 4; REFUSE(c, FP8PA_EWORKSPACE);
    c = Call(); c.workgroups = 4; c.ws = F + 16; c.ws_bytes = 1 << 30; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.head_dim = 96; c.vd.head_dim = 96; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.page_size = 24; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.page_size = 8; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.page_size = 2048; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.row_bytes = 16400; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.row_bytes = 16424; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.row_bytes = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.row_bytes = -16; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.row_bytes = int64_t(1) << 31; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.row_bytes = INT64_MAX - 15; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.num_rows = INT64_MAX; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.num_rows = -1; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.scale_offset = 16392; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.scale_offset = 16000; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.scale_offset = INT64_MAX - 15; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.layout = 7; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.layout = FP8PA_LAYOUT_HEADS_DMAJOR; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.vd.layout = FP8PA_LAYOUT_HEADS_D64; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.scale_kind = 9; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.scale_kind = -1; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.flags = 2; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.num_kv_heads = 0; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.vd.num_kv_heads = 4; c.vd.row_bytes = 8208; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.vd.scale_kind = FP8PA_SCALE_F32_TOKEN_HEAD; c.vd.row_bytes = 16384 + 512; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.B = 20000; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.vd.layout = FP8PA_LAYOUT_TOKENS; c.B = 2100; REFUSE(c, FP8PA_EUNSUPPORTED);
    // fp8 mode
    c = Call(); c.variant = FP8PA_VARIANT_MFMA_FP8; c.sm_scale = 0.09f; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = FP8PA_VARIANT_MFMA_FP8; c.vd.layout = FP8PA_LAYOUT_TOKENS; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = FP8PA_VARIANT_MFMA_FP8; c.kd.scale_kind = c.vd.scale_kind = FP8PA_SCALE_E8M0_G32;
    c.kd.head_dim = c.vd.head_dim = 64; c.kd.row_bytes = c.vd.row_bytes = 8192 + 4096; c.sm_scale = 0.125f;
    REFUSE(c, FP8PA_EUNSUPPORTED);   // the MX-scaled MFMA contracts 128 dims
    // packed variants
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_HEADS; c.workgroups = 3; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_SPLIT; c.vd.layout = FP8PA_LAYOUT_HEADS; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_HEADS; c.kd.scale_kind = c.vd.scale_kind = FP8PA_SCALE_F32_G32;
    c.kd.row_bytes = c.vd.row_bytes = 16 * 1024 + 8 * 16 * 4 * 4; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_SPLIT; c.Hq = 64; REFUSE(c, FP8PA_EUNSUPPORTED);
    // sub-row K scales
    c = Call(); c.kd.scale_kind = FP8PA_SCALE_F32_G32; c.kd.row_bytes = 16384 + 2048; REFUSE(c, FP8PA_EUNSUPPORTED);
    c = Call(); c.kd.scale_kind = FP8PA_SCALE_F32_G256; c.kd.row_bytes = 16384 + 512;
    c.vd.scale_kind = FP8PA_SCALE_F32_TOKEN_HEAD; c.vd.row_bytes = 16384 + 512; REFUSE(c, FP8PA_EINVAL);
    // aligned rows
    c = Call(); c.kd.flags = FP8PA_POOL_ALIGN64; c.kd.scale_offset = 16384; REFUSE(c, FP8PA_EINVAL);
    c = Call(); c.kd.flags = FP8PA_POOL_ALIGN64; c.kp = F + 16; REFUSE(c, FP8PA_EINVAL);
  }

  // ---- accepted calls: one launch each, buffers inside the workspace
  {
    Call c;
    LAUNCH(c);
    c.workgroups = 1; LAUNCH(c);
    c.workgroups = 7; LAUNCH(c);
    c = Call(); c.kd.head_dim = c.vd.head_dim = 64; c.kd.row_bytes = c.vd.row_bytes = 8224; c.window = 128;
    c.sinks = F; LAUNCH(c);
    c = Call(); c.vd.layout = FP8PA_LAYOUT_TOKENS; c.workgroups = 5; LAUNCH(c);
    c = Call(); c.variant = FP8PA_VARIANT_MFMA_FP8; LAUNCH(c);
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_HEADS; LAUNCH(c);
    // Packed heads with V token-major: the packed kernel with its V stage,
    // the packed grid and no workspace (not the split kernel for token-major
    // V, which would cut units with no partials to store into), e.g. head dim
    // 256, P 16, 3 sequences x 4 KV heads.
    for (int lay : {FP8PA_LAYOUT_HEADS, FP8PA_LAYOUT_TOKENS})
      for (int D : {64, 128, 256, 512}) {
        c = Call(); c.variant = FP8PA_VARIANT_PACKED_HEADS; c.B = 3; c.Hq = 16; c.msl = 300;
        c.kd = desc(4, D, 16, FP8PA_LAYOUT_HEADS_D64, FP8PA_SCALE_F32_PAGE_HEAD, (int64_t)4 * 16 * D + 16);
        c.vd = desc(4, D, 16, lay, FP8PA_SCALE_F32_PAGE_HEAD, (int64_t)4 * 16 * D + 16);
        LAUNCH(c);
        CHECK(g_launches.size() == 1 && g_launches[0].kind == 10 && g_launches[0].W == 3 &&
              g_launches[0].a.part_o == nullptr);
      }
    c = Call(); c.variant = FP8PA_VARIANT_MFMA_FP8; c.kd.scale_kind = c.vd.scale_kind = FP8PA_SCALE_E8M0_G32;
    c.kd.row_bytes = c.vd.row_bytes = 16384 + 4096;
    {
      fp8pa_counters c0{}, c1{};
      fp8pa_get_counters(&c0);
      LAUNCH(c);   // MX-scaled fp8 MFMA
      fp8pa_get_counters(&c1);
      CHECK(c1.decode_mfma_fp8 == c0.decode_mfma_fp8 + 1 && c1.decode_mfma_mxfp8 == c0.decode_mfma_mxfp8 + 1 &&
            c1.decode_mfma_bf16 == c0.decode_mfma_bf16);
    }
    c = Call(); c.variant = FP8PA_VARIANT_PACKED_SPLIT; c.workgroups = 9; LAUNCH(c);
    {
      // Automatic grids of small calls stop at the shares the kernel can
      // form: 2 units of 4 tiles are 2 shares (whole units); 8 units of 30
      // tiles give 60 (one tile per wave), rounded up to 64 (a multiple of 8);
      // 8 units of 256 tiles give 512 shares, so a full grid; a large call
      // keeps one workgroup per CU (256 stub CUs).
      fp8pa_plan p{};
      c = Call(); c.B = 1; c.Hq = 8; c.msl = 256;
      c.kd = desc(2, 64, 16, FP8PA_LAYOUT_HEADS_D64, FP8PA_SCALE_F32_PAGE_HEAD, 2064);
      c.vd = desc(2, 64, 16, FP8PA_LAYOUT_HEADS_DMAJOR, FP8PA_SCALE_F32_PAGE_HEAD, 2064);
      CHECK(c.plan(&p) == 0 && p.workgroups == 2);
      LAUNCH(c);
      c = Call(); c.B = 1; c.msl = 1900;
      CHECK(c.plan(&p) == 0 && p.workgroups == 64);
      LAUNCH(c);
      c = Call(); c.B = 1; c.msl = 16384; c.bt_stride = 1024;
      CHECK(c.plan(&p) == 0 && p.workgroups == 256);
      LAUNCH(c);
      c = Call(); c.B = 32; c.msl = 8192;
      CHECK(c.plan(&p) == 0 && p.workgroups == 256);
    }
    c = Call(); c.kd.scale_kind = FP8PA_SCALE_F32_G32; c.kd.row_bytes = 16384 + 2048;
    c.vd.scale_kind = FP8PA_SCALE_F32_TOKEN_HEAD; c.vd.row_bytes = 16384 + 2048; c.workgroups = 3; LAUNCH(c);
    CHECK(g_last_sk == 3);   // K groups of 16+ dims, V per token
    c.kd.scale_kind = FP8PA_SCALE_F32_G8; c.kd.row_bytes = c.vd.row_bytes = 16384 + 8192; LAUNCH(c);
    CHECK(g_last_sk == 5);   // K groups of 8 dims, V per token
    c = Call(); c.kd.scale_kind = c.vd.scale_kind = FP8PA_SCALE_F32_G32; c.kd.row_bytes = c.vd.row_bytes = 16384 + 2048;
    c.workgroups = 3; LAUNCH(c);
    CHECK(g_last_sk == 4);   // K and V groups of 16+ dims
    c = Call(); c.kd.scale_kind = FP8PA_SCALE_F32_G8; c.vd.scale_kind = FP8PA_SCALE_F32_G16;   // K and V groups
    c.kd.row_bytes = c.vd.row_bytes = 16384 + 8192; c.workgroups = 3; LAUNCH(c);
    CHECK(g_last_sk == 6);   // K groups of 8 dims, V groups
    c.workgroups = 1;
    g_launches.clear();
    CHECK(c.run() == 0 && g_launches.size() == 1 && g_launches[0].lds > (size_t)4 * 64 * 8 * 4 &&
          g_launches[0].a.vgstage_off > 0);   // a stage of 8 V groups x 64 positions per wave
    c = Call(); c.kd.head_dim = c.vd.head_dim = 512; c.kd.num_kv_heads = c.vd.num_kv_heads = 2; c.Hq = 16;
    c.kd.page_size = c.vd.page_size = 32; c.kd.row_bytes = c.vd.row_bytes = 65568; c.sm_scale = 1.0f; LAUNCH(c);
    c = Call(); c.kd.flags = c.vd.flags = FP8PA_POOL_ALIGN64; c.kd.row_bytes = c.vd.row_bytes = 16448; LAUNCH(c);
    // automatic packed heads when the units fill the device (256 stub CUs)
    c = Call(); c.B = 300; c.kd.head_dim = c.vd.head_dim = 128;
    fp8pa_plan p{};
    CHECK(c.plan(&p) == 0 && p.variant == FP8PA_VARIANT_PACKED_HEADS && p.workspace_bytes == 0);
    LAUNCH(c);
    // empty batch: nothing launched
    c = Call(); c.B = 0; c.q = c.out = 0; g_launches.clear(); CHECK(c.run() == 0 && g_launches.empty());
  }

  // ---- the allocation-free decode: its partials inside the scratch, or a refusal
  {
    Call c;
    c.workgroups = 7;
    fp8pa_plan p{};
    CHECK(c.plan(&p) == 0 && p.workspace_bytes > 0);
    g_launches.clear();
    auto noalloc = [](const Call& c) {
      return fp8pa_decode_noalloc(fake(c.q), fake(c.out), fake(c.kp), fake(c.vp), &c.kd, &c.vd,
                                  reinterpret_cast<const int32_t*>(c.bt), c.bt_stride,
                                  reinterpret_cast<const int32_t*>(c.sl), c.B, c.Hq, c.window,
                                  reinterpret_cast<const float*>(c.sinks), c.sm_scale, c.msl, c.workgroups,
                                  c.variant, nullptr);
    };
    CHECK(noalloc(c) == 0 && g_launches.size() == 1);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(g_scratch_stub), end = lo + sizeof(g_scratch_stub);
    const uintptr_t po = reinterpret_cast<uintptr_t>(g_launches[0].a.part_o),
                    pf = reinterpret_cast<uintptr_t>(g_launches[0].a.flags);
    CHECK(po == lo && pf > po && pf + 7 * 2 * 4 <= end);
    Call d;                                    // 600 x 2 x 8 x 512 x 4 bytes of partials > 16 MiB
    d.kd = d.vd = desc(2, 512, 32, FP8PA_LAYOUT_HEADS, FP8PA_SCALE_F32_PAGE_HEAD, 65568);
    d.vd.layout = FP8PA_LAYOUT_HEADS_DMAJOR;
    d.Hq = 16; d.workgroups = 600; d.sm_scale = 1.0f;
    g_launches.clear();
    CHECK(noalloc(d) == FP8PA_EWORKSPACE && g_launches.empty() && fp8pa_last_error()[0]);
    d.workgroups = 1;                          // no split: no scratch needed
    CHECK(noalloc(d) == 0 && g_launches.size() == 1 && g_launches[0].a.part_o == nullptr);
    Call e;
    e.Hq = 30;
    g_launches.clear();
    CHECK(noalloc(e) == FP8PA_EINVAL && g_launches.empty());
  }

  // ---- forced merge timeout: the merger waits for a value no holder writes
  {
    fp8pa_debug_force_merge_timeout(1);
    Call c;
    c.workgroups = 1;
    g_launches.clear();
    CHECK(c.run() == 0 && g_launches.size() == 1);
    CHECK(g_launches[0].a.wait_epoch != g_launches[0].a.epoch && g_launches[0].a.spin_limit < (1 << 22));
    fp8pa_debug_force_merge_timeout(0);
    g_launches.clear();
    CHECK(c.run() == 0 && g_launches[0].a.wait_epoch == g_launches[0].a.epoch);
  }

  // ---- device status query
  {
    fp8pa_device_status st{};
    g_status_stub[0] = 5;
    CHECK(fp8pa_get_device_status(&st, 1) == 0 && st.merge_timeouts == 5 && g_status_stub[0] == 0);
    CHECK(fp8pa_get_device_status(nullptr, 0) == FP8PA_EINVAL);
    g_memcpy_fail = 1;
    CHECK(fp8pa_get_device_status(&st, 0) == FP8PA_EHIP);
    g_memcpy_fail = 0;
  }

  // ---- the other entry points refuse before launching
  {
    fp8pa_pool_desc kd = desc(8, 128, 16, FP8PA_LAYOUT_HEADS, FP8PA_SCALE_F32_PAGE_HEAD, 16416);
    fp8pa_pool_desc vd = kd;
    const int32_t* I = reinterpret_cast<const int32_t*>(F);
    g_launches.clear();
    CHECK(fp8pa_append_quant(nullptr, fake(F), fake(F), fake(F), &kd, &vd, I, 8, I, nullptr, 2, 1, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_append_quant(fake(F), fake(F), fake(F), fake(F), &kd, &vd, I, 0, I, nullptr, 2, 1, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_append_quant(fake(F), fake(F), fake(F), fake(F), &kd, &vd, I, 8, I, nullptr, -1, 1, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_append_quant(fake(F + 1), fake(F), fake(F), fake(F), &kd, &vd, I, 8, I, nullptr, 2, 1, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_append_quant(fake(F), fake(F), fake(F), fake(F), nullptr, &vd, I, 8, I, nullptr, 2, 1, nullptr) == FP8PA_EINVAL);
    const float* Ff = reinterpret_cast<const float*>(F);
    CHECK(fp8pa_merge_splits(Ff, Ff, nullptr, fake(F), 2, 8, 4, 80, nullptr) == FP8PA_EUNSUPPORTED);
    CHECK(fp8pa_merge_splits(nullptr, Ff, nullptr, fake(F), 2, 8, 4, 64, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_merge_splits(Ff, Ff, nullptr, fake(F), 2, 0, 4, 64, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_debug_dequant(fake(F), Ff, 9, 16, reinterpret_cast<float*>(F), nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_debug_dequant(fake(F), Ff, 0, -1, reinterpret_cast<float*>(F), nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_stream_read(fake(F + 4), 64, reinterpret_cast<uint32_t*>(F), nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_stream_read(fake(F), 60, reinterpret_cast<uint32_t*>(F), nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_decode_plan(4, 32, &kd, &vd, 8192, 0, 0, 0, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_decode_plan(4, 32, &kd, nullptr, 8192, 0, 0, 0, nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_set_decode_events(reinterpret_cast<void*>(F), nullptr) == FP8PA_EINVAL);
    CHECK(fp8pa_set_debug_checks(reinterpret_cast<uint32_t*>(F + 2)) == FP8PA_EINVAL);
    CHECK(g_launches.empty());
  }

  // ---- plan and call agree over a grid of shapes and variants
  {
    const int dims[] = {64, 128, 256, 512};
    const int pages[] = {16, 32, 128};
    const int kinds[] = {FP8PA_SCALE_F32_PAGE_HEAD, FP8PA_SCALE_F32_TOKEN_HEAD, FP8PA_SCALE_E8M0_G32};
    const int vlayouts[] = {FP8PA_LAYOUT_HEADS_DMAJOR, FP8PA_LAYOUT_HEADS, FP8PA_LAYOUT_TOKENS};
    int n = 0;
    for (int D : dims)
      for (int P : pages)
        for (int kind : kinds)
          for (int vl : vlayouts)
            for (int variant = 0; variant <= 4; ++variant)
              for (int wg : {0, 1, 6}) {
                Call c;
                const int H = 4;
                const int64_t pay = (int64_t)P * H * D;
                const int64_t sc = kind == 0 ? 4 * H : kind == 1 ? 4 * H * P : H * P * D / 32;
                c.kd = desc(H, D, P, FP8PA_LAYOUT_HEADS, kind, (pay + sc + 15) / 16 * 16);
                c.vd = desc(H, D, P, vl, kind, (pay + sc + 15) / 16 * 16);
                c.Hq = 16;
                c.B = 3;
                c.workgroups = wg;
                c.variant = variant;
                c.sm_scale = (float)(1.0 / std::sqrt((double)D));
                c.msl = 4096;
                c.bt_stride = 4096 / P;
                fp8pa_plan p{};
                const int prc = c.plan(&p);
                g_launches.clear();
                const int rc = c.run();
                if (prc != 0) {
                  CHECK(rc == prc && g_launches.empty());
                  continue;
                }
                if (p.workspace_bytes > 0) CHECK(rc == FP8PA_EWORKSPACE);
                else CHECK(rc == 0 && g_launches.size() == 1);
                expect_launch(c, __LINE__);
                ++n;
              }
    CHECK(n > 100);
  }

  // ---- random arguments: no sanitizer report; a refusal launches nothing
  {
    std::mt19937_64 rng(12345);
    auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
    for (int it = 0; it < 20000; ++it) {
      Call c;
      for (fp8pa_pool_desc* d : {&c.kd, &c.vd}) {
        d->num_kv_heads = (int)pick({-1, 0, 1, 2, 3, 4, 8, 64, INT32_MAX});
        d->head_dim = (int)pick({0, 32, 64, 96, 128, 256, 512, 1024, -64});
        d->page_size = (int)pick({0, 1, 8, 16, 24, 32, 128, 1024, 4096, -16});
        d->layout = (int)pick({-1, 0, 1, 2, 3, 4});
        d->scale_kind = (int)pick({-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9});
        d->flags = (int)pick({0, 0, 1, 2});
        d->row_bytes = pick({0, 16, 2064, 8224, 16416, 65568, 135168, int64_t(1) << 31, INT64_MAX, -16, 16448});
        d->scale_offset = pick({-1, -1, 0, 16384, 65536, INT64_MAX});
        d->num_rows = pick({0, 1, 100, INT64_MAX, -3});
      }
      c.B = (int)pick({-1, 0, 1, 3, 64, 65, 300, 20000, INT32_MAX});
      c.Hq = (int)pick({0, 1, 8, 16, 32, 64, 128, INT32_MAX});
      c.window = (int)pick({-5, 0, 1, 128, INT32_MAX});
      c.msl = (int)pick({-1, 0, 1, 8192, INT32_MAX});
      c.workgroups = (int)pick({-1, 0, 1, 7, 100000});
      c.variant = (int)pick({-1, 0, 1, 2, 3, 4, 5});
      c.bt_stride = pick({-1, 0, 1, 512, INT64_MAX});
      c.sm_scale = (float)pick({0, 1, 2}) * 0.05f;
      c.ws = pick({0, 0, (int64_t)F});
      c.ws_bytes = (size_t)pick({0, 1024, int64_t(1) << 40});
      g_launches.clear();
      const int rc = c.run();
      CHECK(rc == 0 || rc == FP8PA_EINVAL || rc == FP8PA_EUNSUPPORTED || rc == FP8PA_EWORKSPACE);
      if (rc != 0) CHECK(g_launches.empty());
      else CHECK(g_launches.size() == (c.B > 0 ? 1u : 0u));
      fp8pa_plan p{};
      (void)c.plan(&p);
      (void)fp8pa_decode_workspace_bytes(c.B, c.Hq, &c.kd, &c.vd, c.msl, c.window, c.workgroups, c.variant);
    }
  }

  // ---- huge sizes are refused, never wrapped
  {
    Call c;
    c.B = INT32_MAX; REFUSE(c, FP8PA_EUNSUPPORTED);
    // packed heads: 5000 sequences x ceil(1.9M / 4) head groups > 2^31 workgroups
    c = Call(); c.kd.num_kv_heads = c.vd.num_kv_heads = 1900000; c.kd.head_dim = c.vd.head_dim = 64;
    c.kd.row_bytes = c.vd.row_bytes = (int64_t)16 * 1900000 * 64 + (int64_t)4 * 1900000;
    c.Hq = 1900000; c.B = 5000; c.variant = FP8PA_VARIANT_PACKED_HEADS; c.bt_stride = 512;
    REFUSE(c, FP8PA_EUNSUPPORTED);
    c.B = 4000; c.kd.num_kv_heads = c.vd.num_kv_heads = 1000; c.Hq = 1000;   // 4000 x 250 fits
    c.kd.row_bytes = c.vd.row_bytes = (int64_t)16 * 1000 * 64 + 4000;
    fp8pa_plan pp{};
    CHECK(c.plan(&pp) == 0 && pp.workgroups == 4000 * 250);
    fp8pa_pool_desc kd = desc(8, 128, 16, FP8PA_LAYOUT_HEADS, FP8PA_SCALE_F32_PAGE_HEAD, 16416);
    const int32_t* I = reinterpret_cast<const int32_t*>(F);
    g_launches.clear();
    CHECK(fp8pa_append_quant(fake(F), fake(F), fake(F), fake(F), &kd, &kd, I, 8, I, nullptr, INT32_MAX, 1, nullptr) ==
          FP8PA_EUNSUPPORTED);
    CHECK(fp8pa_append_quant(fake(F), fake(F), fake(F), fake(F), &kd, &kd, I, 8, I, nullptr, 2, INT32_MAX, nullptr) ==
          FP8PA_EUNSUPPORTED);
    const float* Ff = reinterpret_cast<const float*>(F);
    CHECK(fp8pa_merge_splits(Ff, Ff, nullptr, fake(F), 2, 8, INT32_MAX, 64, nullptr) == FP8PA_EUNSUPPORTED);
    CHECK(fp8pa_merge_splits(Ff, Ff, nullptr, fake(F), INT32_MAX, 8, 4, 64, nullptr) == FP8PA_EUNSUPPORTED);
    CHECK(g_launches.empty());
  }

  // ---- random arguments to the other entry points
  {
    std::mt19937_64 rng(777);
    auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
    for (int it = 0; it < 20000; ++it) {
      fp8pa_pool_desc d[2];
      for (auto& x : d) {
        x = desc((int)pick({-1, 1, 2, 8, 1 << 20, INT32_MAX}), (int)pick({64, 96, 128, 512}),
                 (int)pick({8, 16, 128, 2048}), (int)pick({-1, 0, 1, 2, 3, 4}), (int)pick({-1, 0, 1, 2, 3, 6, 7}),
                 pick({16, 2064, 16416, 135168, INT64_MAX - 15, -16}), pick({0, 100, INT64_MAX}));
        x.flags = (int)pick({0, 1});
      }
      const int B = (int)pick({-1, 0, 1, 5, 70000, INT32_MAX}), T = (int)pick({-1, 0, 1, 33, INT32_MAX});
      const int32_t* I = reinterpret_cast<const int32_t*>(pick({0, (int64_t)F, (int64_t)F + 2}));
      g_launches.clear();
      int rc = fp8pa_append_quant(fake(pick({0, (int64_t)F, (int64_t)F + 1})), fake(F), fake(F), fake(F), &d[0],
                                  &d[1], I, pick({-1, 0, 8, INT64_MAX}), I, nullptr, B, T, nullptr);
      CHECK(rc <= 0 && (rc == 0 || g_launches.empty()));
      g_launches.clear();
      const float* Ff = reinterpret_cast<const float*>(pick({0, (int64_t)F, (int64_t)F + 2}));
      rc = fp8pa_merge_splits(Ff, Ff, nullptr, fake(F), B, (int)pick({-1, 0, 8, INT32_MAX}),
                              (int)pick({-1, 0, 4, INT32_MAX}), (int)pick({64, 80, 512}), nullptr);
      CHECK(rc <= 0 && (rc == 0 || g_launches.empty()));
      g_launches.clear();
      rc = fp8pa_append_decode(fake(F), fake(F), fake(F), fake(F), fake(F), fake(F), &d[0], &d[1], I,
                               pick({-1, 1, 512, INT64_MAX}), I, B, (int)pick({1, 8, 32, INT32_MAX}),
                               (int)pick({0, 128}), nullptr, 0.05f, (int)pick({0, 1024, 8192, INT32_MAX}),
                               (int)pick({0, 1, 7}), (int)pick({0, 2, 3, 9}), nullptr, 0, nullptr);
      CHECK(rc <= 0 && (rc == 0 || g_launches.empty()));
    }
  }

  if (g_fail) {
    std::printf("%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
