// C-ABI of libfp8pa: argument validation, split planning, workspace carving,
// launch counters and error reporting.  Every check runs on the host before
// anything is enqueued; an invalid call launches nothing (the page's
// convention: an explicit request is honoured or refused, never silently
// replaced, and what ran is recorded).
#include <algorithm>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fp8pa.h"
#include "fp8pa_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
thread_local uint32_t* g_dbg = nullptr;   // debug checks: device error words [2], or null
thread_local bool g_force_timeout = false;   // test hook: merges give up waiting

struct Counters {
  std::atomic<int64_t> decode_calls{0}, decode_mfma{0}, decode_split{0}, merge{0}, append{0}, debug{0}, fused_append{0},
      decode_vtok{0}, decode_fp8{0}, decode_mx{0}, decode_packed{0}, decode_psplit{0}, errors{0};
};
Counters g_cnt;
std::atomic<uint32_t> g_epoch{0};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  g_cnt.errors.fetch_add(1);
  return code;
}

void ok() { g_err[0] = 0; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

// Dims per scale of the fp32 sub-row kinds (FP8PA_SCALE_F32_G8..G256).
bool grouped(int kind) { return kind >= FP8PA_SCALE_F32_G32 && kind <= FP8PA_SCALE_F32_G16; }
int group_dims(int kind) {
  return kind == FP8PA_SCALE_F32_G8 ? 8 : kind == FP8PA_SCALE_F32_G16 ? 16 : 32 << (kind - FP8PA_SCALE_F32_G32);
}

int64_t scale_bytes(const fp8pa_pool_desc& d) {
  const int64_t H = d.num_kv_heads, P = d.page_size, D = d.head_dim;
  switch (d.scale_kind) {
    case FP8PA_SCALE_F32_PAGE_HEAD: return 4 * H;
    case FP8PA_SCALE_F32_TOKEN_HEAD: return 4 * H * P;
    case FP8PA_SCALE_E8M0_G32: return H * P * D / 32;
    default: return 4 * H * P * (D / group_dims(d.scale_kind));
  }
}

int64_t footer_offset(const fp8pa_pool_desc& d) {
  return d.scale_offset < 0 ? (int64_t)d.page_size * d.num_kv_heads * d.head_dim : d.scale_offset;
}

// Checks one pool descriptor; returns 0 or an error code (message set).
int check_desc(const fp8pa_pool_desc* d, const char* name) {
  if (!d) return fail(FP8PA_EINVAL, "%s: descriptor is NULL", name);
  if (d->flags != 0 && d->flags != FP8PA_POOL_ALIGN64) return fail(FP8PA_EINVAL, "%s: unknown flags %d", name, d->flags);
  if (d->num_kv_heads < 1) return fail(FP8PA_EINVAL, "%s: num_kv_heads must be >= 1", name);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256 && d->head_dim != 512)
    return fail(FP8PA_EUNSUPPORTED, "%s: head_dim %d not in {64,128,256,512}", name, d->head_dim);
  if (!pow2(d->page_size) || d->page_size < 16 || d->page_size > 1024)
    return fail(FP8PA_EUNSUPPORTED, "%s: page_size %d is not a power of two in [16,1024]", name, d->page_size);
  if (d->layout < FP8PA_LAYOUT_HEADS || d->layout > FP8PA_LAYOUT_HEADS_D64)
    return fail(FP8PA_EINVAL, "%s: unknown layout %d", name, d->layout);
  if (d->scale_kind < FP8PA_SCALE_F32_PAGE_HEAD || d->scale_kind > FP8PA_SCALE_F32_G16)
    return fail(FP8PA_EINVAL, "%s: unknown scale_kind %d", name, d->scale_kind);
  if (grouped(d->scale_kind) && group_dims(d->scale_kind) > d->head_dim)
    return fail(FP8PA_EINVAL, "%s: %d dims per scale exceed head_dim %d", name, group_dims(d->scale_kind),
                d->head_dim);
  // (head counts up to 2^31, pages up to 2^10 and head dims up to 2^9 keep
  // the payload and scale sizes below 2^52.)
  const int64_t payload = (int64_t)d->page_size * d->num_kv_heads * d->head_dim;
  const int64_t foot = footer_offset(*d);
  if (d->row_bytes <= 0 || d->row_bytes % 16)
    return fail(FP8PA_EINVAL, "%s: row_bytes %lld must be a positive multiple of 16", name, (long long)d->row_bytes);
  if (foot < payload || foot % 16)
    return fail(FP8PA_EINVAL, "%s: scale_offset %lld must be a multiple of 16 and >= the payload (%lld)", name,
                (long long)foot, (long long)payload);
  if (foot > d->row_bytes || scale_bytes(*d) > d->row_bytes - foot)
    return fail(FP8PA_EINVAL, "%s: payload + scales exceed row_bytes %lld", name, (long long)d->row_bytes);
  if (d->row_bytes > INT32_MAX) return fail(FP8PA_EUNSUPPORTED, "%s: row_bytes %lld >= 2^31", name, (long long)d->row_bytes);
  if (d->flags & FP8PA_POOL_ALIGN64) {
    if (d->scale_offset >= 0) return fail(FP8PA_EINVAL, "%s: aligned rows need the default scale_offset", name);
    // Every payload shift the rows take must leave room for payload and scales.
    for (int64_t r = 0; r < 64; ++r) {
      const int64_t sh = (-(r * d->row_bytes)) & 63;
      const int64_t end = sh >= scale_bytes(*d) ? sh + payload : sh + payload + scale_bytes(*d);
      if (end > d->row_bytes)
        return fail(FP8PA_EINVAL, "%s: row_bytes %lld leave no room for a payload shifted by %lld bytes", name,
                    (long long)d->row_bytes, (long long)sh);
    }
  }
  if (d->num_rows < 0) return fail(FP8PA_EINVAL, "%s: num_rows must be >= 0", name);
  if (d->row_bytes > INT64_MAX / (d->num_rows > 0 ? d->num_rows : 1))
    return fail(FP8PA_EINVAL, "%s: pool size overflows", name);
  return 0;
}

fp8pa::PoolGeom geometry(const fp8pa_pool_desc& d) {
  fp8pa::PoolGeom g{};
  const int H = d.num_kv_heads, P = d.page_size, D = d.head_dim;
  g.row_bytes = d.row_bytes;
  g.sc_off = (int32_t)footer_offset(d);
  g.align64 = (d.flags & FP8PA_POOL_ALIGN64) ? 1 : 0;
  g.payload_bytes = P * H * D;
  g.scale_bytes = (int32_t)scale_bytes(d);
  const bool tok = d.layout == FP8PA_LAYOUT_TOKENS;
  g.tblk = P;
  g.tblk_stride = 0;
  g.d_stride = 1;
  g.dchunk_stride = 64;
  switch (d.layout) {
    case FP8PA_LAYOUT_HEADS: g.head_stride = P * D; g.tok_stride = D; break;
    case FP8PA_LAYOUT_TOKENS: g.head_stride = D; g.tok_stride = H * D; break;
    case FP8PA_LAYOUT_HEADS_D64: g.head_stride = P * D; g.tok_stride = 64; g.dchunk_stride = 64 * P; break;
    default: {
      const int W = P < 64 ? P : 64;
      g.head_stride = P * D;
      g.tblk = W;
      g.tblk_stride = D * W;
      g.tok_stride = 1;
      g.dchunk_stride = 64 * W;
      g.d_stride = W;
      break;
    }
  }
  switch (d.scale_kind) {
    case FP8PA_SCALE_F32_PAGE_HEAD: g.sc_head_stride = 4; g.sc_tok_stride = 0; break;
    case FP8PA_SCALE_F32_TOKEN_HEAD:
      g.sc_head_stride = tok ? 4 : 4 * P;
      g.sc_tok_stride = tok ? 4 * H : 4;
      break;
    case FP8PA_SCALE_E8M0_G32:
      g.sc_head_stride = tok ? D / 32 : P * (D / 32);
      g.sc_tok_stride = tok ? H * (D / 32) : D / 32;
      break;
    default: {
      const int ng = D / group_dims(d.scale_kind);
      g.sc_head_stride = tok ? 4 * ng : 4 * P * ng;
      g.sc_tok_stride = tok ? 4 * H * ng : 4 * ng;
      g.sc_gshift = ilog2(group_dims(d.scale_kind));
      break;
    }
  }
  return g;
}

// Compute units of the current device (0 when no device can be queried),
// remembered per thread for the last device asked about.
int device_cus() {
  thread_local int last_dev = -1, last_n = 0;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == last_dev) return last_n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  last_dev = dev;
  last_n = n;
  return n;
}

// Whether an automatic call takes packed heads: when the (sequence, group of
// four KV heads) units alone fill every resident workgroup slot, reading all
// heads of the page rows together streams faster than cutting units into
// balanced shares (measured at D = 128: B 256 x L 1024 4.8 -> 6.1 TB/s,
// B 1024 x L 256 2.9 -> 5.4 TB/s; below one unit per slot it is slower).
// No side effects; false for any invalid argument.
bool auto_packs(int B, int Hq, const fp8pa_pool_desc* kd, int workgroups, int variant) {
  if (variant != FP8PA_VARIANT_AUTO || workgroups != 0 || !kd || B <= 0 || kd->num_kv_heads < 1 ||
      kd->num_kv_heads > (1 << 24) || Hq < 1 || Hq % kd->num_kv_heads || Hq / kd->num_kv_heads > 16 ||
      kd->page_size < 1)
    return false;
  const int D = kd->head_dim;
  if (D != 64 && D != 128) return false;   // the head dims where the gain was measured
  const int cus = device_cus();
  if (cus <= 0) return false;
  const size_t lds = fp8pa::decode_lds_bytes(D, B, Hq / kd->num_kv_heads, kd->page_size);
  const bool k_whole = kd->layout == FP8PA_LAYOUT_HEADS_D64 || (D == 64 && kd->layout == FP8PA_LAYOUT_HEADS);
  const int per_cu = fp8pa::decode_blocks_per_cu(D, kd->scale_kind, k_whole, lds);
  const int nw = fp8pa::decode_waves(D);
  return per_cu > 0 && (int64_t)B * ((kd->num_kv_heads + nw - 1) / nw) >= (int64_t)cus * per_cu;
}

// Everything a decode call launches, decided on the host from host values
// only (the grid and the workspace never depend on device data, so a call can
// be captured in a graph).  The plan and the call use the same resolution.
struct Resolved {
  int variant;             // FP8PA_VARIANT_* that runs
  bool vt, f8, packed, psplit, kgroups, k_whole;
  int W;                   // workgroups launched
  int Gu;                  // query heads per unit (packed splits: NW * G)
  size_t lds;              // dynamic LDS bytes
  size_t vstage_off;       // V token-major: offset of the per-wave V stages
  size_t vgstage_off;      // V sub-row scales: offset of the per-wave scale stages
  int sk;                  // kernel scale class: the K kind 0-2; K groups of 16+ dims with V per token (3)
                           // or V groups (4); K groups of 8 dims with V per token (5) or V groups (6)
  int64_t part_o_bytes, part_lse_bytes, flag_bytes;   // workspace pieces, 256-byte aligned
  int64_t workspace_bytes; // 0 when nothing is split
};

int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

// Validates a decode request (everything but pointers and scalars of the
// call) and resolves what it launches.  fused: the one-launch append.
// An upper bound on the shares the split kernel keeps for a call whose
// lengths are at most max_seq_len: its own cap, the larger of floor(cost /
// (unit cost + one tile per wave)) and floor(tiles / waves), at the most tiles
// a unit can have (a window only lowers it).  Workgroups beyond it would
// start, find no share and exit.
int64_t share_bound(int B, int Hkv, int D, int max_seq_len) {
  const int TT = fp8pa::decode_tile_tokens(D), NW = fp8pa::decode_waves(D);
  const int64_t nt = ((int64_t)max_seq_len + TT - 1) / TT;
  const int64_t U = (int64_t)B * Hkv, T = U * nt;
  if (T == 0) return 1;
  const bool unit_mode = T <= (int64_t)NW * U;
  const int64_t TC = unit_mode ? 0 : 4, SC = unit_mode ? 1 : fp8pa::decode_seg_cost(D);
  const int64_t by_cost = (SC * U + TC * T) / (SC + TC * NW), by_tiles = unit_mode ? 0 : T / NW;
  return std::max<int64_t>(1, std::max(by_cost, by_tiles));
}

int resolve(int B, int Hq, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd, int max_seq_len, int workgroups,
            int variant, bool fused, Resolved* r) {
  if (int rc = check_desc(kd, "kd")) return rc;
  if (B < 0) return fail(FP8PA_EINVAL, "B must be >= 0");
  if (Hq < 1 || Hq % kd->num_kv_heads) return fail(FP8PA_EINVAL, "Hq must be a positive multiple of num_kv_heads");
  const int G = Hq / kd->num_kv_heads;
  if (G > 16) return fail(FP8PA_EUNSUPPORTED, "query heads per KV head G=%d > 16", G);
  if (max_seq_len < 0) return fail(FP8PA_EINVAL, "max_seq_len must be >= 0");
  if (workgroups < 0) return fail(FP8PA_EINVAL, "workgroups must be >= 0");
  if (variant != FP8PA_VARIANT_AUTO && variant != FP8PA_VARIANT_MFMA_BF16 && variant != FP8PA_VARIANT_MFMA_FP8 &&
      variant != FP8PA_VARIANT_PACKED_HEADS && variant != FP8PA_VARIANT_PACKED_SPLIT)
    return fail(FP8PA_EUNSUPPORTED, "variant %d is not available", variant);
  const bool packed_req = variant == FP8PA_VARIANT_PACKED_HEADS;
  if (packed_req && workgroups != 0)
    return fail(FP8PA_EUNSUPPORTED, "packed heads fix the grid: workgroups must be 0");
  const int D = kd->head_dim;
  const int nw = fp8pa::decode_waves(D);
  // Packed splits: units of nw KV heads, nw * G query heads merged together.
  const bool psplit = variant == FP8PA_VARIANT_PACKED_SPLIT;
  if (psplit && (kd->num_kv_heads % nw || G * nw > 16))
    return fail(FP8PA_EUNSUPPORTED, "packed splits need Hkv %% %d == 0 and G <= %d", nw, 16 / nw);
  const int Gu = psplit ? G * nw : G;
  // The stages end at decode_stage_end; the combine buffer may overlap them,
  // so the launch takes the larger of the stages' end and decode_lds_bytes.
  const size_t lds_min = fp8pa::decode_lds_bytes(D, B, Gu, kd->page_size);
  size_t lds = fp8pa::decode_stage_end(D, B, kd->page_size);
  if (lds_min > 65536)
    return fail(FP8PA_EUNSUPPORTED, "B=%d, G=%d, head_dim %d need %zu bytes of LDS (> 64 KiB)", B, G, D, lds_min);
  if (int rc = check_desc(vd, "vd")) return rc;
  if (kd->layout == FP8PA_LAYOUT_HEADS_DMAJOR)
    return fail(FP8PA_EUNSUPPORTED, "kd: decode reads K in the HEADS_D64, HEADS or TOKENS layout");
  // fp32 sub-row V scales: with K in sub-row groups too; one PV MFMA covers 16
  // dims, so V groups span at least 16; the per-wave stage holds 16 groups.
  const bool vgroups = grouped(vd->scale_kind);
  if (vgroups && (!grouped(kd->scale_kind) || group_dims(vd->scale_kind) < 16 ||
                  vd->head_dim / group_dims(vd->scale_kind) > 16))
    return fail(FP8PA_EUNSUPPORTED,
                "vd: decode reads fp32 sub-row V scales with K in sub-row scales, groups of 16 to head_dim dims and "
                "at most 16 groups per head");
  if (g_dbg && (kd->num_rows < 1 || vd->num_rows < 1))
    return fail(FP8PA_EINVAL, "debug checks need num_rows >= 1 in both descriptors");
  if (vd->layout == FP8PA_LAYOUT_HEADS_D64)
    return fail(FP8PA_EUNSUPPORTED, "vd: decode reads V in the HEADS_DMAJOR, HEADS or TOKENS layout");
  // V in a token-major layout is staged through LDS.
  const bool vt = vd->layout == FP8PA_LAYOUT_HEADS || vd->layout == FP8PA_LAYOUT_TOKENS;
  if (vt && fused) return fail(FP8PA_EUNSUPPORTED, "the one-launch append reads V in the HEADS_DMAJOR layout");
  const bool f8 = variant == FP8PA_VARIANT_MFMA_FP8;
  if (f8 && (grouped(kd->scale_kind) || vt || fused))
    return fail(FP8PA_EUNSUPPORTED,
                "the fp8 compute mode takes page, token or E8M0 scales, V in HEADS_DMAJOR and no fused append");
  // With E8M0 pools the fp8 mode runs the MX-scaled fp8 MFMA, 128 dims each.
  if (f8 && kd->scale_kind == FP8PA_SCALE_E8M0_G32 && kd->head_dim % 128)
    return fail(FP8PA_EUNSUPPORTED, "the fp8 mode over E8M0 pools needs a head_dim multiple of 128 (got %d)",
                kd->head_dim);
  // fp32 sub-row K scales: K pieces are scaled before the MFMA (plain,
  // token-major-V and split kernels only).
  const bool kgroups = grouped(kd->scale_kind);
  if (kgroups && (fused || packed_req || psplit))
    return fail(FP8PA_EUNSUPPORTED, "sub-row K scales take the split kernels and no fused append");
  if ((packed_req || psplit) && fused) return fail(FP8PA_EUNSUPPORTED, "packed heads take no fused append");
  if (psplit && vt) return fail(FP8PA_EUNSUPPORTED, "packed splits read V in HEADS_DMAJOR");
  size_t vstage_off = 0;
  if (vt) {
    vstage_off = (lds + 15) / 16 * 16;
    lds = vstage_off + fp8pa::decode_vstage_bytes(D);
    if (lds > 65536)
      return fail(FP8PA_EUNSUPPORTED, "B=%d, head_dim %d with V staged through LDS need %zu bytes of LDS (> 64 KiB)",
                  B, D, lds);
  }
  if (vd->num_kv_heads != kd->num_kv_heads || vd->head_dim != kd->head_dim || vd->page_size != kd->page_size ||
      (vd->scale_kind != kd->scale_kind &&
       !(kgroups && (vd->scale_kind == FP8PA_SCALE_F32_TOKEN_HEAD || vgroups))))
    return fail(FP8PA_EUNSUPPORTED,
                "K and V pools must share num_kv_heads, head_dim, page_size and scale_kind (or K in fp32 "
                "sub-row scales with V in F32_TOKEN_HEAD or fp32 sub-row scales)");
  // V sub-row scales: a per-wave LDS stage of the tile's (position, group) scales.
  size_t vgstage_off = 0;
  if (vgroups) {
    vgstage_off = (lds + 15) / 16 * 16;
    lds = vgstage_off + (size_t)nw * fp8pa::decode_tile_tokens(D) * (D / group_dims(vd->scale_kind)) * 4 + 16;
    if (lds > 65536)
      return fail(FP8PA_EUNSUPPORTED, "B=%d, head_dim %d with V sub-row scales need %zu bytes of LDS (> 64 KiB)", B,
                  D, lds);
  }
  if (lds < lds_min) lds = lds_min;   // the wave-combine buffer
  // Packed heads: requested, or taken automatically when the units fill the
  // device (V d-major, no fused append).
  const bool packed = packed_req || (!vt && !fused && !kgroups && auto_packs(B, Hq, kd, workgroups, variant));
  const bool k_whole = kd->layout == FP8PA_LAYOUT_HEADS_D64 || (D == 64 && kd->layout == FP8PA_LAYOUT_HEADS);
  const int sk = !kgroups ? kd->scale_kind
                 : group_dims(kd->scale_kind) == 8 ? (vgroups ? 6 : 5)
                                                   : (vgroups ? 4 : 3);
  int W = workgroups;
  if (packed) {
    const int64_t Wp = (int64_t)B * ((kd->num_kv_heads + nw - 1) / nw);
    if (Wp > INT32_MAX) return fail(FP8PA_EUNSUPPORTED, "packed heads: %lld workgroups exceed the grid", (long long)Wp);
    W = Wp < 1 ? 1 : (int)Wp;
  } else if (W == 0) {
    // One resident generation: every workgroup gets an equal share of the
    // tiles and all of them run at once.
    const int cus = device_cus();
    const int per_cu = cus > 0 ? fp8pa::decode_blocks_per_cu(D, sk, k_whole, lds) : 0;
    W = (cus > 0 && per_cu > 0) ? cus * per_cu : 1024;
    // Small calls: about as many workgroups as the kernel can give shares
    // to (rounded up to a multiple of 8 from 16 on, so that the shares form
    // one block per XCD), instead of a full grid whose first XCD blocks take
    // all the shares (workgroup w runs on XCD w mod 8).
    if (!psplit) {
      int64_t cap = share_bound(B, kd->num_kv_heads, D, max_seq_len);
      if (cap >= 16) cap = (cap + 7) / 8 * 8;
      if (cap < W) W = (int)cap;
    }
  }
  r->variant = f8 ? FP8PA_VARIANT_MFMA_FP8
               : packed ? FP8PA_VARIANT_PACKED_HEADS
               : psplit ? FP8PA_VARIANT_PACKED_SPLIT
                        : FP8PA_VARIANT_MFMA_BF16;
  r->vt = vt;
  r->f8 = f8;
  r->packed = packed;
  r->psplit = psplit;
  r->kgroups = kgroups;
  r->k_whole = k_whole;
  r->W = W;
  r->Gu = Gu;
  r->lds = lds;
  r->vstage_off = vstage_off;
  r->vgstage_off = vgstage_off;
  r->sk = sk;
  if (W > 1 && !packed) {
    r->part_o_bytes = round256((int64_t)W * 2 * Gu * D * 4);
    r->part_lse_bytes = round256((int64_t)W * 2 * Gu * 4);
    r->flag_bytes = round256((int64_t)W * 2 * 4);
  } else {
    r->part_o_bytes = r->part_lse_bytes = r->flag_bytes = 0;
  }
  r->workspace_bytes = r->part_o_bytes + r->part_lse_bytes + r->flag_bytes;
  return 0;
}

// Epochs tag published split partials; a merger clears consumed flags to 0,
// so 0 is never handed out (the counter skips it when it wraps).
uint32_t next_epoch(std::atomic<uint32_t>& counter) {
  uint32_t e = counter.fetch_add(1) + 1;
  while (e == 0) e = counter.fetch_add(1) + 1;
  return e;
}

}  // namespace

extern "C" {

const char* fp8pa_version(void) { return "fp8pa 0.1.0 gfx950"; }

const char* fp8pa_last_error(void) { return g_err; }

int fp8pa_decode_plan(int B, int Hq, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd, int max_seq_len,
                      int window, int workgroups, int variant, fp8pa_plan* out) {
  if (!out) return fail(FP8PA_EINVAL, "plan output is NULL");
  Resolved r{};
  if (int rc = resolve(B, Hq, kd, vd, max_seq_len, workgroups, variant, false, &r)) return rc;
  (void)window;   // the grid never depends on the window (nor on the lengths)
  out->workgroups = r.W;
  out->tile_tokens = fp8pa::decode_tile_tokens(kd->head_dim);
  out->variant = r.variant;
  out->reserved = 0;
  out->workspace_bytes = r.workspace_bytes;
  ok();
  return FP8PA_OK;
}

int64_t fp8pa_decode_workspace_bytes(int B, int Hq, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                                     int max_seq_len, int window, int workgroups, int variant) {
  fp8pa_plan p{};
  if (int rc = fp8pa_decode_plan(B, Hq, kd, vd, max_seq_len, window, workgroups, variant, &p)) return rc;
  return p.workspace_bytes;
}

namespace {

// fp8pa_decode, and the fused fp8pa_append_decode when k_new / v_new are
// given.  dry_run: validate everything, launch nothing.
int decode_impl(const void* k_new, const void* v_new, const void* q, void* out, const uint8_t* k_pool,
                const uint8_t* v_pool, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int B, int Hq, int window,
                const float* sinks, float sm_scale, int max_seq_len, int workgroups, int variant, void* workspace,
                size_t workspace_bytes, void* stream, bool dry_run = false) {
  const bool fused = k_new != nullptr || v_new != nullptr;
  Resolved r{};
  if (int rc = resolve(B, Hq, kd, vd, max_seq_len, workgroups, variant, fused, &r)) return rc;
  const bool vt = r.vt, f8 = r.f8, packed = r.packed, psplit = r.psplit;
  // The fp8 mode's E4M3 query moves each logit by up to 2^-4 of sm_scale *
  // sum |q_d k_d|: within the page's fp8 tolerance class at the default score
  // scale D^-0.5, not at larger ones (sm_scale = 1 with D = 256 spreads the
  // logits over tens of units).  Larger scales are refused.
  if (f8 && std::fabs((double)sm_scale) * std::sqrt((double)kd->head_dim) > 1.0 + 1e-6)
    return fail(FP8PA_EUNSUPPORTED, "the fp8 compute mode serves |sm_scale| <= head_dim^-0.5 only (got %g at head_dim %d)",
                (double)sm_scale, kd->head_dim);
  if (B == 0) {
    if (!dry_run) {
      ok();
      g_cnt.decode_calls.fetch_add(1);
    }
    return FP8PA_OK;
  }
  if (!q || !out || !k_pool || !v_pool || !block_table || !seq_lens || (fused && (!k_new || !v_new)))
    return fail(FP8PA_EINVAL, "a required device pointer is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(FP8PA_EINVAL, "q and out must be 16-byte aligned");
  if (fused && (!aligned(k_new, 2) || !aligned(v_new, 2))) return fail(FP8PA_EINVAL, "k_new/v_new misaligned");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return fail(FP8PA_EINVAL, "pools must be 16-byte aligned");
  if (((kd->flags & FP8PA_POOL_ALIGN64) && !aligned(k_pool, 64)) || ((vd->flags & FP8PA_POOL_ALIGN64) && !aligned(v_pool, 64)))
    return fail(FP8PA_EINVAL, "pools with aligned rows must be 64-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4)) return fail(FP8PA_EINVAL, "block_table/seq_lens misaligned");
  if (sinks && !aligned(sinks, 4)) return fail(FP8PA_EINVAL, "sinks misaligned");
  if (bt_stride < 1) return fail(FP8PA_EINVAL, "bt_stride must be >= 1");
  if (max_seq_len > 0 && bt_stride < (max_seq_len + kd->page_size - 1) / kd->page_size)
    return fail(FP8PA_EINVAL, "bt_stride %lld is smaller than the pages of max_seq_len", (long long)bt_stride);
  if (!std::isfinite(sm_scale)) return fail(FP8PA_EINVAL, "sm_scale must be finite");
  if (r.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < (size_t)r.workspace_bytes)
      return fail(FP8PA_EWORKSPACE, "workspace of %lld bytes required (%zu given)", (long long)r.workspace_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(FP8PA_EINVAL, "workspace must be 256-byte aligned");
  }
  if (dry_run) return FP8PA_OK;
  uint32_t* status = fp8pa::device_status_words();
  if (!status) return fail(FP8PA_EHIP, "the device status words cannot be resolved on this device");
  const int D = kd->head_dim;
  const int G = Hq / kd->num_kv_heads;
  const int W = r.W;
  fp8pa::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.kp = k_pool;
  a.vp = v_pool;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.sinks = sinks;
  if (fused) {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.kw = const_cast<uint8_t*>(k_pool);
    a.vw = const_cast<uint8_t*>(v_pool);
  }
  a.kg = geometry(*kd);
  a.vg = geometry(*vd);
  a.P = kd->page_size;
  a.log2P = ilog2(kd->page_size);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = kd->num_kv_heads;
  a.G = G;
  a.window = window > 0 ? window : 0;
  a.qk_scale = (float)((double)sm_scale * 1.4426950408889634);
  a.vstage_off = (int32_t)r.vstage_off;
  a.vgstage_off = (int32_t)r.vgstage_off;
  a.dbg = g_dbg;
  a.dbg_rows = (int32_t)std::min<int64_t>(std::min(kd->num_rows, vd->num_rows), INT32_MAX);
  a.dbg_max_len = max_seq_len;
  // Packed splits: every wave reads every tile of a segment, so one tile per
  // share suffices, and a tile carries NW heads, so a unit's fixed cost is
  // NW times smaller in tiles.
  const int nw = fp8pa::decode_waves(D);
  a.min_tiles = psplit ? 1 : nw;
  a.seg_cost = psplit ? fp8pa::decode_seg_cost(D) / nw : fp8pa::decode_seg_cost(D);
  a.epoch = next_epoch(g_epoch);
  // A forced timeout (test hook) waits for a flag value no holder writes.
  a.wait_epoch = g_force_timeout ? a.epoch ^ 0x80000000u : a.epoch;
  a.spin_limit = g_force_timeout ? (1 << 10) : (1 << 22);
  a.status = status;
  if (W > 1 && !packed) {
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + r.part_o_bytes);
    a.flags = reinterpret_cast<uint32_t*>(ws + r.part_o_bytes + r.part_lse_bytes);
  }
  const size_t lds = r.lds;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // A wave's 16-byte K loads cover 64 bytes of each of 16 tokens: whole lines
  // when the 64-byte pieces of consecutive tokens are adjacent.
  const bool k_whole = r.k_whole;
  // The kernel family: packed heads (which take no workspace) first, then the
  // split kernels, which must have their partials and flags.
  if (!packed && W > 1 && (!a.part_o || !a.part_lse || !a.flags))
    return fail(FP8PA_EWORKSPACE, "internal: a split launch without its workspace");
  hipError_t e = packed ? (vt ? fp8pa::launch_decode_packed_vt(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop)
                              : fp8pa::launch_decode_packed(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop))
                 : psplit ? fp8pa::launch_decode_pksplit(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop)
                 : fused  ? fp8pa::launch_decode_fused(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop)
                 : vt     ? fp8pa::launch_decode_vtok(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop)
                 : f8     ? fp8pa::launch_decode_fp8q(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop)
                          : fp8pa::launch_decode(a, D, r.sk, k_whole, W, lds, st, g_ev_start, g_ev_stop);
  if (e != hipSuccess) return fail(FP8PA_EHIP, "decode launch: %s", hipGetErrorString(e));
  if (f8) g_cnt.decode_fp8.fetch_add(1);
  else g_cnt.decode_mfma.fetch_add(1);
  if (f8 && kd->scale_kind == FP8PA_SCALE_E8M0_G32) g_cnt.decode_mx.fetch_add(1);
  if (W > 1 && !packed) g_cnt.decode_split.fetch_add(1);
  if (packed) g_cnt.decode_packed.fetch_add(1);
  if (psplit) g_cnt.decode_psplit.fetch_add(1);
  if (fused) g_cnt.fused_append.fetch_add(1);
  if (vt) g_cnt.decode_vtok.fetch_add(1);
  g_cnt.decode_calls.fetch_add(1);
  ok();
  return FP8PA_OK;
}

}  // namespace

int fp8pa_decode(const void* q, void* out, const uint8_t* k_pool, const uint8_t* v_pool,
                 const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd, const int32_t* block_table,
                 int64_t bt_stride, const int32_t* seq_lens, int B, int Hq, int window, const float* sinks,
                 float sm_scale, int max_seq_len, int workgroups, int variant, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return decode_impl(nullptr, nullptr, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens, B, Hq,
                     window, sinks, sm_scale, max_seq_len, workgroups, variant, workspace, workspace_bytes, stream);
}

int fp8pa_decode_noalloc(const void* q, void* out, const uint8_t* k_pool, const uint8_t* v_pool,
                         const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd, const int32_t* block_table,
                         int64_t bt_stride, const int32_t* seq_lens, int B, int Hq, int window, const float* sinks,
                         float sm_scale, int max_seq_len, int workgroups, int variant, void* stream) {
  Resolved r{};
  if (int rc = resolve(B, Hq, kd, vd, max_seq_len, workgroups, variant, false, &r)) return rc;
  if (r.workspace_bytes > FP8PA_NOALLOC_SCRATCH_BYTES)
    return fail(FP8PA_EWORKSPACE,
                "this call needs %lld bytes of split scratch, more than the %d the allocation-free decode holds "
                "(use fp8pa_decode with a workspace, or fewer workgroups)",
                (long long)r.workspace_bytes, (int)FP8PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (r.workspace_bytes > 0 && B > 0) {
    ws = fp8pa::device_scratch();
    if (!ws) return fail(FP8PA_EHIP, "the scratch of the allocation-free decode cannot be resolved on this device");
  }
  return decode_impl(nullptr, nullptr, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens, B, Hq,
                     window, sinks, sm_scale, max_seq_len, workgroups, variant, ws,
                     ws ? (size_t)FP8PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

// Longest attended span (max_seq_len, or the window) for which
// fp8pa_append_decode appends inside the decode kernel.
constexpr int kFusedMaxSpan = 2048;

int fp8pa_append_decode(const void* k_new, const void* v_new, const void* q, void* out, uint8_t* k_pool,
                        uint8_t* v_pool, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                        const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int B, int Hq,
                        int window, const float* sinks, float sm_scale, int max_seq_len, int workgroups, int variant,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return fail(FP8PA_EINVAL, "k_new and v_new are required");
  if (B > 0 && (!aligned(k_new, 2) || !aligned(v_new, 2))) return fail(FP8PA_EINVAL, "k_new/v_new misaligned");
  // In-kernel appends sit on the critical path of the workgroup that reads
  // each new token.  Short attended spans are launch-bound, and there the one
  // launch wins (about 24 -> 13.5 us on the tiny and window-128 calls);
  // longer ones run the append kernel and then the plain decode.
  // V in a token-major layout and the fp8 compute mode take the two launches
  // as well.
  const int span = (window > 0 && window < max_seq_len) ? window : max_seq_len;
  // So do calls whose automatic plan takes packed heads (then the output
  // equals the append followed by the same decode).
  if (span <= kFusedMaxSpan && vd && vd->layout == FP8PA_LAYOUT_HEADS_DMAJOR && variant != FP8PA_VARIANT_MFMA_FP8 &&
      !(kd && grouped(kd->scale_kind)) && !g_dbg &&
      variant != FP8PA_VARIANT_PACKED_HEADS && variant != FP8PA_VARIANT_PACKED_SPLIT &&
      !auto_packs(B, Hq, kd, workgroups, variant))
    return decode_impl(k_new, v_new, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens, B, Hq,
                       window, sinks, sm_scale, max_seq_len, workgroups, variant, workspace, workspace_bytes, stream);
  // Every check of the call runs before the append launches.
  if (int rc = decode_impl(nullptr, nullptr, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens, B,
                           Hq, window, sinks, sm_scale, max_seq_len, workgroups, variant, workspace, workspace_bytes,
                           stream, true))
    return rc;
  if (B == 0) return decode_impl(nullptr, nullptr, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens,
                                 B, Hq, window, sinks, sm_scale, max_seq_len, workgroups, variant, workspace,
                                 workspace_bytes, stream);
  fp8pa::AppendArgs ap{};
  ap.k_new = static_cast<const uint16_t*>(k_new);
  ap.v_new = static_cast<const uint16_t*>(v_new);
  ap.kp = k_pool;
  ap.vp = v_pool;
  ap.kg = geometry(*kd);
  ap.vg = geometry(*vd);
  ap.k_kind = kd->scale_kind;
  ap.v_kind = vd->scale_kind;
  ap.dbg = g_dbg;
  ap.dbg_rows = (int32_t)std::min<int64_t>(std::min(kd->num_rows, vd->num_rows), INT32_MAX);
  ap.bt = block_table;
  ap.bt_stride = bt_stride;
  ap.seq_lens = seq_lens;
  ap.T = 1;
  ap.P = kd->page_size;
  ap.Hkv = kd->num_kv_heads;
  ap.D = kd->head_dim;
  hipError_t e = fp8pa::launch_append(ap, B, 1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8PA_EHIP, "append launch: %s", hipGetErrorString(e));
  g_cnt.append.fetch_add(1);
  return decode_impl(nullptr, nullptr, q, out, k_pool, v_pool, kd, vd, block_table, bt_stride, seq_lens, B, Hq,
                     window, sinks, sm_scale, max_seq_len, workgroups, variant, workspace, workspace_bytes, stream);
}

int fp8pa_merge_splits(const float* part_o, const float* part_lse, const float* sinks, void* out, int B, int Hq,
                       int S, int D, void* stream) {
  if (B < 0 || Hq < 1 || S < 0) return fail(FP8PA_EINVAL, "bad B/Hq/S");
  if (D != 64 && D != 128 && D != 256 && D != 512) return fail(FP8PA_EUNSUPPORTED, "D %d not in {64,128,256,512}", D);
  // Grid (Hq, B); the S lse weights of a head are staged in LDS.
  if (S > 16384 || B > 65535 || Hq > (1 << 24))
    return fail(FP8PA_EUNSUPPORTED, "merge of B %d, Hq %d, S %d exceeds the grid or LDS", B, Hq, S);
  if (B == 0) {
    ok();
    return FP8PA_OK;
  }
  if (!out || (S > 0 && (!part_o || !part_lse))) return fail(FP8PA_EINVAL, "a required device pointer is NULL");
  if (!aligned(out, 4) || (part_o && !aligned(part_o, 4)) || (part_lse && !aligned(part_lse, 4)) ||
      (sinks && !aligned(sinks, 4)))
    return fail(FP8PA_EINVAL, "misaligned pointer");
  fp8pa::MergeArgs m{};
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.sinks = sinks;
  m.out = static_cast<uint16_t*>(out);
  m.Hq = Hq;
  m.S = S;
  m.D = D;
  m.G = 1;
  hipError_t e = fp8pa::launch_merge(m, B, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8PA_EHIP, "merge launch: %s", hipGetErrorString(e));
  g_cnt.merge.fetch_add(1);
  ok();
  return FP8PA_OK;
}

int fp8pa_append_quant(const void* k_new, const void* v_new, uint8_t* k_pool, uint8_t* v_pool,
                       const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd, const int32_t* block_table,
                       int64_t bt_stride, const int32_t* positions, const int32_t* counts, int B, int T,
                       void* stream) {
  if (int rc = check_desc(kd, "kd")) return rc;
  if (int rc = check_desc(vd, "vd")) return rc;
  if (vd->num_kv_heads != kd->num_kv_heads || vd->head_dim != kd->head_dim || vd->page_size != kd->page_size)
    return fail(FP8PA_EUNSUPPORTED, "K and V pools must share num_kv_heads, head_dim and page_size");
  if (B < 0 || T < 0) return fail(FP8PA_EINVAL, "B and T must be >= 0");
  if (B == 0 || T == 0) {
    ok();
    return FP8PA_OK;
  }
  // Grid: (pages of the span, KV heads, 2 B) workgroups of 256 threads.
  const int64_t max_pages = ((int64_t)T + kd->page_size - 1) / kd->page_size + 1;
  if (B > (1 << 24) || max_pages > (1 << 23) || kd->num_kv_heads > 65535)
    return fail(FP8PA_EUNSUPPORTED, "append grid too large (B %d, T %d, Hkv %d)", B, T, kd->num_kv_heads);
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !positions)
    return fail(FP8PA_EINVAL, "a required device pointer is NULL");
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_table, 4) || !aligned(positions, 4) || (counts && !aligned(counts, 4)))
    return fail(FP8PA_EINVAL, "misaligned pointer");
  if (((kd->flags & FP8PA_POOL_ALIGN64) && !aligned(k_pool, 64)) || ((vd->flags & FP8PA_POOL_ALIGN64) && !aligned(v_pool, 64)))
    return fail(FP8PA_EINVAL, "pools with aligned rows must be 64-byte aligned");
  if (bt_stride < 1) return fail(FP8PA_EINVAL, "bt_stride must be >= 1");
  if (g_dbg && (kd->num_rows < 1 || vd->num_rows < 1))
    return fail(FP8PA_EINVAL, "debug checks need num_rows >= 1 in both descriptors");
  fp8pa::AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.kp = k_pool;
  a.vp = v_pool;
  a.kg = geometry(*kd);
  a.vg = geometry(*vd);
  a.k_kind = kd->scale_kind;
  a.v_kind = vd->scale_kind;
  a.dbg = g_dbg;
  a.dbg_rows = (int32_t)std::min<int64_t>(std::min(kd->num_rows, vd->num_rows), INT32_MAX);
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.positions = positions;
  a.counts = counts;
  a.T = T;
  a.P = kd->page_size;
  a.Hkv = kd->num_kv_heads;
  a.D = kd->head_dim;
  hipError_t e = fp8pa::launch_append(a, B, (int)max_pages, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8PA_EHIP, "append launch: %s", hipGetErrorString(e));
  g_cnt.append.fetch_add(1);
  ok();
  return FP8PA_OK;
}

int fp8pa_debug_dequant(const uint8_t* codes, const void* scales, int scale_kind, int n, float* out,
                        void* stream) {
  if (n < 0) return fail(FP8PA_EINVAL, "n must be >= 0");
  if (scale_kind < FP8PA_SCALE_F32_PAGE_HEAD || scale_kind > FP8PA_SCALE_F32_G16)
    return fail(FP8PA_EINVAL, "unknown scale_kind %d", scale_kind);
  if (n == 0) {
    ok();
    return FP8PA_OK;
  }
  if (!codes || !scales || !out) return fail(FP8PA_EINVAL, "a required device pointer is NULL");
  if (!aligned(out, 4) || (scale_kind != FP8PA_SCALE_E8M0_G32 && !aligned(scales, 4)))
    return fail(FP8PA_EINVAL, "misaligned pointer");
  hipError_t e = fp8pa::launch_debug_dequant(codes, scales, scale_kind, n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8PA_EHIP, "debug launch: %s", hipGetErrorString(e));
  g_cnt.debug.fetch_add(1);
  ok();
  return FP8PA_OK;
}

int fp8pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(FP8PA_EINVAL, "a required device pointer is NULL");
  if (bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4)) return fail(FP8PA_EINVAL, "misaligned buffer or size");
  if (bytes == 0) {
    ok();
    return FP8PA_OK;
  }
  hipError_t e = fp8pa::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8PA_EHIP, "probe launch: %s", hipGetErrorString(e));
  ok();
  return FP8PA_OK;
}

int fp8pa_get_counters(fp8pa_counters* c) {
  if (!c) return fail(FP8PA_EINVAL, "counters output is NULL");
  c->decode_calls = g_cnt.decode_calls.load();
  c->decode_mfma_bf16 = g_cnt.decode_mfma.load();
  c->decode_split = g_cnt.decode_split.load();
  c->merge_launches = g_cnt.merge.load();
  c->append_launches = g_cnt.append.load();
  c->debug_launches = g_cnt.debug.load();
  c->errors = g_cnt.errors.load();
  c->fused_appends = g_cnt.fused_append.load();
  c->decode_v_token_major = g_cnt.decode_vtok.load();
  c->decode_mfma_fp8 = g_cnt.decode_fp8.load();
  c->decode_packed_heads = g_cnt.decode_packed.load();
  c->decode_packed_split = g_cnt.decode_psplit.load();
  c->decode_mfma_mxfp8 = g_cnt.decode_mx.load();
  return FP8PA_OK;
}

int fp8pa_set_decode_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(FP8PA_EINVAL, "set both events or neither");
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  ok();
  return FP8PA_OK;
}

int fp8pa_set_debug_checks(uint32_t* err) {
  if (err && !aligned(err, 4)) return fail(FP8PA_EINVAL, "err must be 4-byte aligned");
  g_dbg = err;
  ok();
  return FP8PA_OK;
}

int fp8pa_get_device_status(fp8pa_device_status* out, int reset) {
  if (!out) return fail(FP8PA_EINVAL, "status output is NULL");
  uint32_t* w = fp8pa::device_status_words();
  if (!w) return fail(FP8PA_EHIP, "the device status words cannot be resolved on this device");
  hipError_t e = hipDeviceSynchronize();
  uint32_t words[4] = {0, 0, 0, 0};
  if (e == hipSuccess) e = hipMemcpy(words, w, sizeof(words), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) {
    const uint32_t zero[4] = {0, 0, 0, 0};
    e = hipMemcpy(w, zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return fail(FP8PA_EHIP, "device status: %s", hipGetErrorString(e));
  out->merge_timeouts = words[0];
  for (int i = 0; i < 3; ++i) out->reserved[i] = 0;
  ok();
  return FP8PA_OK;
}

int fp8pa_debug_force_merge_timeout(int on) {
  g_force_timeout = on != 0;
  ok();
  return FP8PA_OK;
}

int fp8pa_reset_counters(void) {
  g_cnt.decode_calls = 0;
  g_cnt.decode_mfma = 0;
  g_cnt.decode_split = 0;
  g_cnt.merge = 0;
  g_cnt.append = 0;
  g_cnt.debug = 0;
  g_cnt.errors = 0;
  g_cnt.fused_append = 0;
  g_cnt.decode_vtok = 0;
  g_cnt.decode_fp8 = 0;
  g_cnt.decode_packed = 0;
  g_cnt.decode_psplit = 0;
  g_cnt.decode_mx = 0;
  return FP8PA_OK;
}

}  // extern "C"
