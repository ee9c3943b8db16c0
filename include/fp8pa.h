/*
 * fp8pa -- paged flash-decode attention over an FP8 (E4M3) KV cache, for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "fp8 paged attention for MoE serving", sections
 * "Smallest correct example", "Expected result" and "Supported scope"): one
 * decode query token per sequence attends, through a per-sequence block
 * table, to E4M3 keys and values stored in flat byte pools of packed rows;
 * values are dequantized as code x scale; query head h reads KV head h / G
 * (G = Hq / Hkv); an optional window keeps only the last W keys; an optional
 * per-query-head sink adds one logit to the softmax denominator with no value;
 * sm_scale replaces head_dim ** -0.5.
 *
 * Conventions shared by every entry point:
 *  - Pointers named "device" are HIP device pointers; the caller owns every
 *    buffer (including the workspace).  The library allocates no device
 *    memory, never synchronizes, and enqueues all work on `stream` (a
 *    hipStream_t; NULL is the default stream).  Calls are asynchronous.
 *  - Every entry point validates its host-visible arguments first.  On any
 *    error it returns a negative status, records a message readable with
 *    fp8pa_last_error(), and launches nothing.
 *  - Values that live in device memory (seq_lens, block_table) are trusted:
 *    they must describe rows inside the pools.  Table entries are read only
 *    for pages that hold attended (or appended) positions; other entries may
 *    hold anything, e.g. -1.
 */
#ifndef FP8PA_H
#define FP8PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  FP8PA_OK = 0,
  FP8PA_EINVAL = -1,        /* a bad argument (null, misaligned, out of range) */
  FP8PA_EUNSUPPORTED = -2,  /* valid request this library does not implement   */
  FP8PA_EWORKSPACE = -3,    /* workspace missing or smaller than required      */
  FP8PA_EHIP = -4           /* a HIP launch reported an error                  */
};

/* ---- pool row payload layouts (byte offset of the code of KV head h,
 *      in-page token t, dim d inside a row) --------------------------------
 * The page names two orders, "tokens" and "heads" ("Supported scope").  The
 * other two are this library's own, chosen so that one wave-wide 16-byte load
 * of the decode kernel covers whole 128-byte lines: HEADS_D64 for keys (the
 * 64-byte pieces of consecutive tokens side by side), HEADS_DMAJOR for values
 * (token-contiguous per dim, which the value operand of the MFMA that
 * contracts over tokens needs).  The decode kernel reads K in HEADS, TOKENS or
 * HEADS_D64 (fastest) and V in HEADS_DMAJOR (fastest), HEADS or TOKENS (the
 * last two through a transposing stage in LDS). */
enum {
  FP8PA_LAYOUT_HEADS = 0,         /* [Hkv][P][D]: (h*P + t)*D + d */
  FP8PA_LAYOUT_TOKENS = 1,        /* [P][Hkv][D]: (t*Hkv + h)*D + d */
  FP8PA_LAYOUT_HEADS_DMAJOR = 2,  /* [Hkv][P/W][D][W], W = min(P, 64):
                                     h*P*D + (t/W)*D*W + d*W + t%W
                                     (for P <= 64: [Hkv][D][P]) */
  FP8PA_LAYOUT_HEADS_D64 = 3      /* [Hkv][D/64][P][64]:
                                     ((h*(D/64) + d/64)*P + t)*64 + d%64 */
};

/* ---- scale kinds.  The scale footer starts at scale_offset inside the row
 *      (the page's "fp8 payload + fp32 scales per block"); byte offsets from
 *      there, with slot = t*Hkv + h for the TOKENS layout, else h*P + t:
 *   F32_PAGE_HEAD   fp32 per (page, head):          4*h
 *   F32_TOKEN_HEAD  fp32 per (token, head):         4*slot
 *   E8M0_G32        E8M0 per (token, head, 32 dims along D), the MXFP8 scale
 *                   of page "Attention MXFP8 TKG Kernel API Reference":
 *                   slot*(D/32) + d/32.  Value 2**(u-127).
 *   F32_G<S>        fp32 per (token, head, S dims along D), S = 8, 16, 32, 64,
 *                   128 or 256 dividing D: the sub-row scales of page "fp8 paged
 *                   attention for MoE serving" ("Supported scope", k_groups or
 *                   v_groups = D/S): 4*(slot*(D/S) + d/S).  Written by
 *                   fp8pa_append_quant for K or V.  fp8pa_decode reads them for
 *                   K with V in F32_TOKEN_HEAD, or for K and V together (V
 *                   groups of at least 16 dims and at most 16 groups per head);
 *                   other pairings are refused with FP8PA_EUNSUPPORTED.     */
enum {
  FP8PA_SCALE_F32_PAGE_HEAD = 0,
  FP8PA_SCALE_F32_TOKEN_HEAD = 1,
  FP8PA_SCALE_E8M0_G32 = 2,
  FP8PA_SCALE_F32_G32 = 3,
  FP8PA_SCALE_F32_G64 = 4,
  FP8PA_SCALE_F32_G128 = 5,
  FP8PA_SCALE_F32_G256 = 6,
  FP8PA_SCALE_F32_G8 = 7,
  FP8PA_SCALE_F32_G16 = 8
};

/* ---- decode variants.  An explicit request is honoured or refused with
 *      FP8PA_EUNSUPPORTED, never replaced by another variant. */
enum {
  FP8PA_VARIANT_AUTO = 0,
  FP8PA_VARIANT_MFMA_BF16 = 1,  /* E4M3 -> bf16 exactly, bf16 MFMA, fp32 accumulate */
  FP8PA_VARIANT_MFMA_FP8 = 2,   /* fp8 compute mode (page "fp8 paged attention for MoE
                                   serving", "Two compute paths": the fp8 dot rounds q to
                                   E4M3): each query row (sequence, query head) is
                                   quantized with one fp32 scale fp32(amax/448) (1 for a
                                   zero row) and codes e4m3(fp32(q/scale)) with the IEEE
                                   quotient (the KV quantizer's rule); QK^T takes the K
                                   codes unconverted on the fp8 MFMA; PV and the softmax as
                                   in MFMA_BF16.  With E8M0 pools (head_dim a multiple of
                                   128) q is rounded to the keys' own MXFP8 format instead:
                                   one E8M0 scale per 32 dims (the KV quantizer's rule) and
                                   codes e4m3(q / scale); QK^T then runs on the MX-scaled
                                   fp8 MFMA, which applies both operands' E8M0 scales
                                   itself (counted in decode_mfma_mxfp8).  Only on explicit
                                   request; V in HEADS_DMAJOR, |sm_scale| <= D^-0.5 (the
                                   page's fp8 tolerance class, rtol = atol = 1.5e-1, holds
                                   at the default score scale; larger scales spread the
                                   logits so that q's rounding exceeds it), not with the
                                   fused append (else FP8PA_EUNSUPPORTED);
                                   fp8pa_append_decode runs it after the append kernel. */
  FP8PA_VARIANT_PACKED_HEADS = 3  /* packed heads (page "fp8 paged attention for MoE
                                   serving", pack_heads): one workgroup per (sequence,
                                   group of KV heads), one KV head per wave, no split and
                                   no merge; arithmetic as MFMA_BF16.  For short or
                                   windowed calls and for large batches.  The grid is fixed
                                   (workgroups must be 0; the plan reports B * ceil(Hkv / 4),
                                   no workspace); no fused append (fp8pa_append_decode runs
                                   it after the append kernel); V in HEADS_DMAJOR, HEADS or
                                   TOKENS (each wave stages its V rows in LDS, as the split
                                   kernel does); no sub-row fp32 scales (else
                                   FP8PA_EUNSUPPORTED).  With AUTO and workgroups 0,
                                   fp8pa_decode runs it instead of the split kernel when V
                                   is in HEADS_DMAJOR, D <= 128 and the B * ceil(Hkv / 4) units alone
                                   fill every resident workgroup slot of the device (the
                                   plan, given the same pools, reports it). */,
  FP8PA_VARIANT_PACKED_SPLIT = 4  /* packed heads with splits: a unit is (sequence, 4
                                   consecutive KV heads), one KV head per wave, so a
                                   workgroup reads whole groups of heads of each page row
                                   together; long spans are split over workgroups and
                                   merged as in MFMA_BF16 (same arithmetic, another
                                   summation order).  Needs Hkv % 4 == 0 and G <= 4; V in
                                   HEADS_DMAJOR; no fused append (else
                                   FP8PA_EUNSUPPORTED); fp8pa_append_decode runs it
                                   after the append kernel. */
};

/* ---- row placement flags (fp8pa_pool_desc.flags).
 *   FP8PA_POOL_ALIGN64  the payload of row r starts at the row's first 64-byte
 *       boundary, r*row_bytes + ((-r*row_bytes) mod 64) bytes from the pool
 *       base (which must then be 64-byte aligned), and the scale block sits
 *       in the gap before the payload when it fits there, else right after
 *       the payload.  For rows whose width is not a multiple of 64 bytes
 *       (a 32-byte scale footer, say), this keeps every 64-byte memory unit
 *       of the payload inside one wave-wide load.  Needs the default
 *       scale_offset and a row wide enough for every shift its rows take. */
enum { FP8PA_POOL_ALIGN64 = 1 };

/* One pool (K or V) of one layer.  K and V pools may differ in layout and
 * stride; several layers may share a pool through row_bytes. */
typedef struct fp8pa_pool_desc {
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D: 64, 128, 256 or 512 */
  int32_t page_size;     /* P tokens per row: a power of two in [16, 1024] */
  int32_t layout;        /* FP8PA_LAYOUT_* */
  int32_t scale_kind;    /* FP8PA_SCALE_* */
  int32_t flags;         /* 0 or FP8PA_POOL_ALIGN64 */
  int64_t row_bytes;     /* stride between rows; multiple of 16, >= natural row, < 2^31 */
  int64_t scale_offset;  /* footer offset in the row; multiple of 16, >= P*Hkv*D;
                            -1 selects the default P*Hkv*D */
  int64_t num_rows;      /* rows in the pool (host-side sanity only) */
} fp8pa_pool_desc;

/* Plan of one decode call (computed on the host from host values only, so a
 * call can be captured in a HIP graph).  The attended positions of every
 * (sequence, KV head) are cut into tiles; the tiles of all of them form one
 * list, and each of `workgroups` workgroups takes an equal share, so the work
 * is balanced however uneven the sequence lengths are.  Units cut between
 * workgroups are merged by log-sum-exp inside the same launch. */
typedef struct fp8pa_plan {
  int32_t workgroups;       /* W launched (auto: all resident at once on this device) */
  int32_t tile_tokens;      /* positions per tile */
  int32_t variant;          /* FP8PA_VARIANT_* that fp8pa_decode runs with these arguments */
  int32_t reserved;
  int64_t workspace_bytes;  /* needed by fp8pa_decode (0 when nothing is split) */
} fp8pa_plan;

/* Library version string; never NULL. */
const char* fp8pa_version(void);

/* Message of the last error on the calling thread ("" if none).  Every
 * refusal is reported, as the page "fp8 paged attention for MoE serving"
 * ("Two compute paths") asks of an explicit request that cannot be served:
 * it is refused with a reason, never silently replaced. */
const char* fp8pa_last_error(void);

/* Plan a decode call (the split grid of page "fp8 paged attention for MoE
 * serving", section "Why it happens": the grid runs over sequence, KV head
 * and split, and an unsplit grid leaves most of the device idle).  B
 * sequences, Hq query heads, pools `kd` and `vd` as they will be passed to
 * fp8pa_decode; every seq_lens[b] must be <= max_seq_len; window <= 0 means
 * none (the grid does not depend on it); workgroups 0 lets the library
 * choose, else it is used as given (>= 1).  Validates the geometry exactly as
 * fp8pa_decode does (same refusals) and reports the variant, grid and
 * workspace that call launches.  Refuses (FP8PA_EUNSUPPORTED) shapes whose
 * LDS needs exceed 64 KiB: 12 bytes per sequence plus the larger of the
 * page-row stage and the wave combine, i.e. B above about 4700 (head dim 128,
 * G = 4) or 2700 (head dim 512 with G = 8). */
int fp8pa_decode_plan(int B, int Hq, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                      int max_seq_len, int window, int workgroups, int variant, fp8pa_plan* out);

/* Workspace bytes fp8pa_decode needs for these arguments (plan.workspace_bytes):
 * >= 0, or a negative status (and fp8pa_last_error) when fp8pa_decode_plan
 * would refuse.  The workspace holds the split partials [W][2][G][D] fp32,
 * their log-sum-exp [W][2][G] and a flag per partial [W][2], each piece
 * 256-byte aligned. */
int64_t fp8pa_decode_workspace_bytes(int B, int Hq, const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                                     int max_seq_len, int window, int workgroups, int variant);

/*
 * Decode attention (the hot path).
 *   q           device bf16 [B, Hq, D], contiguous, 16-byte aligned.
 *   out         device bf16 [B, Hq, D], contiguous, 16-byte aligned; written.
 *   k_pool,
 *   v_pool      device uint8 pools, 16-byte aligned, described by kd / vd.
 *               kd: layout HEADS_D64, HEADS or TOKENS; vd: layout
 *               HEADS_DMAJOR, HEADS or TOKENS.  Both: same Hkv, D, P and
 *               scale kind, except that K in F32_G<S> takes V in
 *               F32_TOKEN_HEAD (V in F32_G<S> is refused; K in F32_G<S>
 *               runs the MFMA_BF16 split kernels only, without the fused
 *               append).  With V in HEADS or TOKENS the launch needs
 *               more LDS (B up to about 2000 at D = 128; FP8PA_EUNSUPPORTED
 *               beyond).
 *   block_table device int32 [B, bt_stride]: logical page -> row.
 *   seq_lens    device int32 [B]: valid positions of each sequence, the token
 *               being decoded included (append first, then decode); each
 *               <= max_seq_len.
 *   window      > 0: attend positions [L - window, L) only; <= 0: all.
 *   sinks       device fp32 [Hq] sink logits (already in scaled-score units)
 *               or NULL for none.
 *   sm_scale    finite score scale (D ** -0.5 is the usual value).
 *   max_seq_len, workgroups, variant: as for fp8pa_decode_plan.
 *   workspace   device buffer of >= plan.workspace_bytes (256-byte aligned),
 *               or NULL when that is 0.  Its contents need no initialisation
 *               (split partials are published with flags tagged by a per-call
 *               epoch, and cleared once merged, so a replayed graph starts
 *               clean).  Calls that share a workspace must not overlap: issue
 *               them on one stream.
 * Output rows are bf16 (round to nearest even) of the fp32 result.
 */
int fp8pa_decode(const void* q, void* out, const uint8_t* k_pool, const uint8_t* v_pool,
                 const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                 const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                 int B, int Hq, int window, const float* sinks, float sm_scale,
                 int max_seq_len, int workgroups, int variant,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fp8pa_decode without the workspace arguments.  The split
 * partials, their log-sum-exp and flags go to a scratch array the library
 * holds per device, FP8PA_NOALLOC_SCRATCH_BYTES long, resolved on the first
 * call on each device (with that device current) and held until the process
 * ends.  The call allocates nothing.  Calls whose plan needs more workspace
 * than that (plan.workspace_bytes) are refused with FP8PA_EWORKSPACE before
 * anything is launched; every other argument, check and result is exactly
 * fp8pa_decode's (same kernels, same plan, bit-identical output).  The
 * scratch needs no clearing: flags carry the call's epoch.  Every call on one
 * device shares that device's scratch: calls that overlap in time on one
 * device (different streams, or threads) race and must not be issued.
 */
#define FP8PA_NOALLOC_SCRATCH_BYTES (16 << 20)
int fp8pa_decode_noalloc(const void* q, void* out, const uint8_t* k_pool, const uint8_t* v_pool,
                         const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                         int B, int Hq, int window, const float* sinks, float sm_scale,
                         int max_seq_len, int workgroups, int variant, void* stream);

/*
 * Append + decode (page "Lecture 8 — Inference Path: KV Cache, Decode, RoPE,
 * GQA, Paged KV" of the FlashAttention course, section "In-kernel KV cache
 * update": the attention kernel itself writes the new token's K and V,
 * saving the separate append launch).  When the attended span (window if set and smaller, else
 * max_seq_len) is at most 2048 positions, which makes the call launch-bound,
 * the decode kernel performs the appends (one launch); otherwise the append
 * kernel runs first and then the decode (two launches on `stream`), since an
 * in-kernel append delays the workgroups that read the new tokens by more
 * than a launch costs.  V pools in the HEADS or TOKENS layout and the fp8
 * compute mode always take the two launches.  Same contract as fp8pa_decode, plus:
 *   k_new, v_new  device bf16 [B, Hkv, D], 2-byte aligned: sequence b's new
 *               token, written at position seq_lens[b] - 1 (seq_lens counts it)
 *               and attended in the same call.  Sequences with seq_lens[b] = 0
 *               get no append.
 *   k_pool, v_pool  are written: exactly as fp8pa_append_quant(k_new, v_new,
 *               ..., positions = seq_lens - 1, counts = NULL, T = 1) would, and
 *               the output equals that append followed by fp8pa_decode.
 * In the one-launch form, the workgroup holding a unit's last tile performs
 * the unit's append before it reads that tile; no other workgroup reads the
 * new token's page.  Every check runs before anything is launched.
 */
int fp8pa_append_decode(const void* k_new, const void* v_new, const void* q, void* out,
                        uint8_t* k_pool, uint8_t* v_pool,
                        const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                        const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                        int B, int Hq, int window, const float* sinks, float sm_scale,
                        int max_seq_len, int workgroups, int variant,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Log-sum-exp merge of split partials (page section "Why it happens": the
 * grid splits each sequence; the partial results are combined afterwards).
 *   part_o    device fp32 [B, Hq, S, D]: each split's normalised output.
 *   part_lse  device fp32 [B, Hq, S]: each split's natural-log sum of
 *             exp(score); -inf marks an empty split (its part_o is ignored).
 *   sinks     device fp32 [Hq] or NULL; the sink enters the denominator once.
 *   out       device bf16 [B, Hq, D].
 *   D         64, 128, 256 or 512.
 */
int fp8pa_merge_splits(const float* part_o, const float* part_lse, const float* sinks,
                       void* out, int B, int Hq, int S, int D, void* stream);

/*
 * Quantize and write new K and V tokens into the pools (page section
 * "Supported scope": per-token-per-head E4M3 with an fp32 scale or sub-row
 * groups, and a one-launch append).  Sequence b receives tokens
 * k_new[b, 0:n_b] at positions positions[b] + t, n_b = counts ? counts[b] : T.
 *   k_new, v_new  device bf16 [B, T, Hkv, D], contiguous.
 *   kd, vd        any layout; same Hkv, D, P as each other.
 *   positions     device int32 [B]; counts device int32 [B] or NULL.
 * Encoding: y = fp32(x / s) correctly rounded, clamped to +-448, rounded to
 * the nearest E4M3 (ties to even).  Scales:
 *   F32_TOKEN_HEAD: s = fp32(amax / 448) per (token, head), 1 when amax = 0.
 *   E8M0_G32: the smallest 2**k with amax <= 448 * 2**k per 32 dims.
 *   F32_PAGE_HEAD: the page scale only grows: s = max(s_old, fp32(amax_new /
 *     448)) (1 if that is 0), where s_old is 0 when the call writes the page's
 *     first slot; if it grows, the page's earlier tokens are re-encoded from
 *     their fp32 values.  Appends to one page must be ordered in time.
 * Pages written must be distinct between sequences of one call.
 */
int fp8pa_append_quant(const void* k_new, const void* v_new, uint8_t* k_pool, uint8_t* v_pool,
                       const fp8pa_pool_desc* kd, const fp8pa_pool_desc* vd,
                       const int32_t* block_table, int64_t bt_stride,
                       const int32_t* positions, const int32_t* counts,
                       int B, int T, void* stream);

/*
 * Test hook: dequantize n codes with the device conversion the decode kernel
 * uses, so that it can be compared bit for bit with code x scale (page "fp8
 * paged attention for MoE serving", "Smallest correct example": the reference
 * dequantizes with the code and its scale).  scales: device fp32 [n] (F32
 * kinds) or uint8 E8M0 [n] (E8M0_G32).  out: device fp32 [n]:
 *   F32_PAGE_HEAD, F32_TOKEN_HEAD: the E4M3 -> bf16 operand conversion, then
 *     the product with the scale (the decode applies fp32 scales to the score
 *     or the probability, the same product up to association);
 *   E8M0_G32: the scaled conversion, exact for all finite codes (E8M0 codes
 *     10..245);
 *   F32_G<S>: fp32(code x scale) as the sub-row key path forms it before
 *     splitting it into a hi/lo pair of bf16 operands.
 */
int fp8pa_debug_dequant(const uint8_t* codes, const void* scales, int scale_kind, int n,
                        float* out, void* stream);

/* Measurement helper: reads `bytes` (a multiple of 16) of device memory at
 * `buf` (16-byte aligned) once with a plain streaming kernel and nothing
 * else, so that its rate gives this machine's HBM read ceiling.  `sink` is a
 * device uint32 that the kernel may write. */
int fp8pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Launch counters: what actually ran, not what was requested (the page "fp8
 * paged attention for MoE serving", "Two compute paths", reports which path
 * served a call through compute_counts(); these are this library's). */
typedef struct fp8pa_counters {
  int64_t decode_calls;     /* successful fp8pa_decode calls */
  int64_t decode_mfma_bf16; /* decode kernels launched, MFMA bf16 variant */
  int64_t decode_split;     /* calls run with more than one workgroup */
  int64_t merge_launches;   /* fp8pa_merge_splits kernels launched */
  int64_t append_launches;
  int64_t debug_launches;
  int64_t errors;           /* calls refused or failed */
  int64_t fused_appends;    /* decode launches that also appended (fp8pa_append_decode) */
  int64_t decode_v_token_major; /* decode launches reading V in the HEADS or TOKENS layout */
  int64_t decode_mfma_fp8;  /* decode kernels launched, fp8 compute mode */
  int64_t decode_packed_heads; /* decode kernels launched, packed heads */
  int64_t decode_packed_split;  /* decode kernels launched, packed heads with splits */
  int64_t decode_mfma_mxfp8;  /* of decode_mfma_fp8: over E8M0 pools, on the MX-scaled fp8 MFMA */
} fp8pa_counters;

int fp8pa_get_counters(fp8pa_counters* out);

/* Debug checks of the device-resident arguments (off by default; the
 * boundary otherwise trusts them).  With err (device uint32 [2], 4-byte
 * aligned, cleared by the caller) set, later calls on this thread check in
 * the kernels every block-table entry they read against [0, num_rows) of the
 * smaller pool and, in decode, every seq_lens[b] against [0, max_seq_len]
 * (append: the written pages against bt_stride).  A bad entry reads row 0 (in
 * append: nothing is written) and sets err[0] = 1; a bad length counts as 0
 * (that sequence's output is zeros) and sets err[1] = 1.  So a bad value
 * never leads to an access outside the pools, and the output of a call that
 * sets an error word is not meaningful.  fp8pa_append_decode runs the append
 * kernel then the decode while the checks are on.  Both descriptors need
 * num_rows >= 1 (else FP8PA_EINVAL).  err NULL turns the checks off. */
int fp8pa_set_debug_checks(uint32_t* err);
int fp8pa_reset_counters(void);

/* Device status of the current device.  merge_timeouts counts the split
 * merges whose bounded wait for another workgroup's partial gave up since the
 * library was loaded or last reset (a unit whose merge gave up has NaN
 * outputs; the wait only gives up if a workgroup that holds an earlier piece
 * never publishes it).  After a timeout the workspace's flags are in an
 * unknown state: clear the workspace (zeros) before replaying a captured
 * graph with it.  This query synchronizes the device (hipDeviceSynchronize)
 * and is not for use under graph capture; reset != 0 clears the words. */
typedef struct fp8pa_device_status {
  uint64_t merge_timeouts;
  uint64_t reserved[3];
} fp8pa_device_status;
int fp8pa_get_device_status(fp8pa_device_status* out, int reset);

/* Test hook (calling thread only): while on, decode merges wait for a flag
 * value that no workgroup writes, with a short bound, so every cut unit's
 * merge gives up (NaN outputs, counted in merge_timeouts) and every kernel
 * still ends.  For testing the timeout report; off by default. */
int fp8pa_debug_force_merge_timeout(int on);

/* Profiling hook (calling thread only): while set, every fp8pa_decode records
 * `start` on its stream just before the decode kernel and `stop` just after
 * it, before any merge kernel, so the pair times the decode kernel alone.
 * Both are hipEvent_t created by the caller; pass NULL, NULL to clear. */
int fp8pa_set_decode_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif
#endif /* FP8PA_H */
