"""Thin Python binding of libfp8pa (ctypes).  Argument marshalling only: every
step of the computation runs in the HIP library; torch supplies device memory
and the current stream.  A missing library raises; there is no fallback."""
import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8pa.so")

LAYOUTS = {"heads": 0, "tokens": 1, "heads_dmajor": 2, "heads_d64": 3}
SCALE_KINDS = {"page_head": 0, "token_head": 1, "e8m0_32": 2, "f32_g32": 3, "f32_g64": 4, "f32_g128": 5, "f32_g256": 6,
               "f32_g8": 7, "f32_g16": 8}
VARIANTS = {"auto": 0, "mfma_bf16": 1, "mfma_fp8": 2, "packed_heads": 3, "packed_split": 4}

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4


class Fp8paError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"fp8pa error {code}: {msg}")
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("scale_kind", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("scale_offset", ctypes.c_int64), ("num_rows", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_int32), ("tile_tokens", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]


class Counters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("decode_calls", "decode_mfma_bf16", "decode_split", "merge_launches",
                                              "append_launches", "debug_launches", "errors", "fused_appends",
                                              "decode_v_token_major", "decode_mfma_fp8",
                                              "decode_packed_heads",
                                              "decode_packed_split", "decode_mfma_mxfp8")]


class DeviceStatus(ctypes.Structure):
    _fields_ = [("merge_timeouts", ctypes.c_uint64), ("reserved", ctypes.c_uint64 * 3)]


_lib = None
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "fp8pa_version": ([], ctypes.c_char_p),
    "fp8pa_last_error": ([], ctypes.c_char_p),
    "fp8pa_decode_plan": ([_I, _I, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _I, _I, _I, _I,
                           ctypes.POINTER(Plan)], _I),
    "fp8pa_decode_workspace_bytes": ([_I, _I, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _I, _I, _I, _I],
                                     _I64),
    "fp8pa_decode": ([_P, _P, _P, _P, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _P, _I64, _P, _I, _I, _I,
                      _P, _F, _I, _I, _I, _P, _SZ, _P], _I),
    "fp8pa_decode_noalloc": ([_P, _P, _P, _P, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _P, _I64, _P, _I,
                              _I, _I, _P, _F, _I, _I, _I, _P], _I),
    "fp8pa_append_decode": ([_P, _P, _P, _P, _P, _P, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _P, _I64,
                             _P, _I, _I, _I, _P, _F, _I, _I, _I, _P, _SZ, _P], _I),
    "fp8pa_merge_splits": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "fp8pa_append_quant": ([_P, _P, _P, _P, ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _P, _I64, _P, _P,
                            _I, _I, _P], _I),
    "fp8pa_debug_dequant": ([_P, _P, _I, _I, _P, _P], _I),
    "fp8pa_get_counters": ([ctypes.POINTER(Counters)], _I),
    "fp8pa_reset_counters": ([], _I),
    "fp8pa_set_debug_checks": ([_P], _I),
    "fp8pa_set_decode_events": ([_P, _P], _I),
    "fp8pa_stream_read": ([_P, _SZ, _P, _P], _I),
    "fp8pa_get_device_status": ([ctypes.POINTER(DeviceStatus), _I], _I),
    "fp8pa_debug_force_merge_timeout": ([_I], _I),
}


def lib():
    """The loaded library (built by fp8_paged_kv_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m fp8_paged_kv_amd.build`")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def last_error():
    return lib().fp8pa_last_error().decode()


def _check(rc):
    if rc != OK:
        raise Fp8paError(rc, last_error())


POOL_ALIGN64 = 1


def pool_desc(num_kv_heads, head_dim, page_size, layout, scale_kind, row_bytes, num_rows, scale_offset=-1,
              align64=False):
    return PoolDesc(num_kv_heads, head_dim, page_size, LAYOUTS.get(layout, layout),
                    SCALE_KINDS.get(scale_kind, scale_kind), POOL_ALIGN64 if align64 else 0, row_bytes,
                    scale_offset, num_rows)


def _ptr(t):
    # (ctypes turns a Python int into the c_void_p argument itself.)
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:   # the current stream's handle without building a Stream object
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype=None, device=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def decode_plan(B, Hq, kd, vd, max_seq_len, window=0, workgroups=0, variant="auto"):
    """The variant, grid and workspace an fp8pa_decode call with these
    arguments launches (raises what that call would)."""
    p = Plan()
    _check(lib().fp8pa_decode_plan(B, Hq, ctypes.byref(kd), ctypes.byref(vd), max_seq_len, window, workgroups,
                                   VARIANTS.get(variant, variant), ctypes.byref(p)))
    return p


def decode_workspace_bytes(B, Hq, kd, vd, max_seq_len, window=0, workgroups=0, variant="auto"):
    n = lib().fp8pa_decode_workspace_bytes(B, Hq, ctypes.byref(kd), ctypes.byref(vd), max_seq_len, window,
                                           workgroups, VARIANTS.get(variant, variant))
    if n < 0:
        raise Fp8paError(n, last_error())
    return n


def decode(q, k_pool, v_pool, kd, vd, block_table, seq_lens, max_seq_len, window=0, sinks=None, sm_scale=None,
           workgroups=0, variant="auto", out=None, workspace=None, stream=None):
    """Decode attention.  q bf16 [B, Hq, D]; returns bf16 [B, Hq, D].

    variant: "auto" or "mfma_bf16" (the default bf16 MFMA path), "mfma_fp8"
    (the fp8 compute mode: query rows rounded to E4M3) or "packed_heads" (one
    workgroup per sequence and group of KV heads, no split; workgroups must be
    0).  A variant the call cannot run raises; none is replaced by another."""
    _need(q, "q", torch.bfloat16)
    _need(k_pool, "k_pool", torch.uint8)
    _need(v_pool, "v_pool", torch.uint8)
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16)
    scale = D ** -0.5 if sm_scale is None else float(sm_scale)
    if workspace is None:   # (a given workspace is checked by the library)
        plan = decode_plan(B, Hq, kd, vd, max_seq_len, window, workgroups, variant)
        if plan.workspace_bytes > 0:
            workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8pa_decode(_ptr(q), _ptr(out), _ptr(k_pool), _ptr(v_pool), ctypes.byref(kd), ctypes.byref(vd),
                              _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, Hq, window, _ptr(sinks),
                              scale, max_seq_len, workgroups, VARIANTS.get(variant, variant), _ptr(workspace),
                              ws_bytes, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc(q, k_pool, v_pool, kd, vd, block_table, seq_lens, max_seq_len, window=0, sinks=None,
                   sm_scale=None, workgroups=0, variant="auto", out=None, stream=None):
    """decode() through the allocation-free entry point: the library's
    per-device scratch holds the split partials (no workspace; calls that
    overlap on one device race).  `out` is allocated here only when not given."""
    _need(q, "q", torch.bfloat16)
    _need(k_pool, "k_pool", torch.uint8)
    _need(v_pool, "v_pool", torch.uint8)
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16)
    scale = D ** -0.5 if sm_scale is None else float(sm_scale)
    _check(lib().fp8pa_decode_noalloc(_ptr(q), _ptr(out), _ptr(k_pool), _ptr(v_pool), ctypes.byref(kd),
                                      ctypes.byref(vd), _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, Hq,
                                      window, _ptr(sinks), scale, max_seq_len, workgroups,
                                      VARIANTS.get(variant, variant), _stream(stream)))
    return out


def append_decode(q, k_new, v_new, k_pool, v_pool, kd, vd, block_table, seq_lens, max_seq_len, window=0, sinks=None,
                  sm_scale=None, workgroups=0, variant="auto", out=None, workspace=None, stream=None):
    """Append each sequence's new token (bf16 [B, Hkv, D] k_new / v_new, at
    position seq_lens[b] - 1) into the pools and decode: in one launch for
    attended spans up to 2048 positions with V in "heads_dmajor" and the
    default variant, else the append kernel and then the decode."""
    _need(q, "q", torch.bfloat16)
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    _need(k_pool, "k_pool", torch.uint8)
    _need(v_pool, "v_pool", torch.uint8)
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32)
    B, Hq, D = q.shape
    if tuple(k_new.shape) != (B, kd.num_kv_heads, D) or tuple(v_new.shape) != (B, kd.num_kv_heads, D):
        raise ValueError("k_new / v_new must be [B, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16)
    scale = D ** -0.5 if sm_scale is None else float(sm_scale)
    if workspace is None:   # (a given workspace is checked by the library)
        plan = decode_plan(B, Hq, kd, vd, max_seq_len, window, workgroups, variant)
        if plan.workspace_bytes > 0:
            workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8pa_append_decode(_ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), _ptr(k_pool), _ptr(v_pool),
                                     ctypes.byref(kd), ctypes.byref(vd), _ptr(block_table), block_table.shape[1],
                                     _ptr(seq_lens), B, Hq, window, _ptr(sinks), scale, max_seq_len, workgroups,
                                     VARIANTS.get(variant, variant), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def merge_splits(part_o, part_lse, sinks=None, out=None, stream=None):
    """part_o fp32 [B, Hq, S, D], part_lse fp32 [B, Hq, S] -> bf16 [B, Hq, D]."""
    _need(part_o, "part_o", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    B, Hq, S, D = part_o.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=part_o.device)
    _check(lib().fp8pa_merge_splits(_ptr(part_o), _ptr(part_lse), _ptr(sinks), _ptr(out), B, Hq, S, D,
                                    _stream(stream)))
    return out


def append_quant(k_new, v_new, k_pool, v_pool, kd, vd, block_table, positions, counts=None, stream=None):
    """Quantize bf16 [B, T, Hkv, D] tokens into the pools in place."""
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    _need(positions, "positions", torch.int32)
    _need(block_table, "block_table", torch.int32)
    B, T = k_new.shape[:2]
    _check(lib().fp8pa_append_quant(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), ctypes.byref(kd),
                                    ctypes.byref(vd), _ptr(block_table), block_table.shape[1], _ptr(positions),
                                    _ptr(counts), B, T, _stream(stream)))


def debug_dequant(codes, scales, scale_kind, stream=None):
    _need(codes, "codes", torch.uint8)
    out = torch.empty(codes.numel(), dtype=torch.float32, device=codes.device)
    _check(lib().fp8pa_debug_dequant(_ptr(codes), _ptr(scales), SCALE_KINDS.get(scale_kind, scale_kind),
                                     codes.numel(), _ptr(out), _stream(stream)))
    return out


def counters():
    c = Counters()
    _check(lib().fp8pa_get_counters(ctypes.byref(c)))
    return {n: getattr(c, n) for n, _ in Counters._fields_}


def reset_counters():
    lib().fp8pa_reset_counters()


def set_debug_checks(err=None):
    """Turn the in-kernel checks of block-table entries and sequence lengths
    on (``err``: a device uint32 tensor of 2 words, zeroed by the caller; word
    0 flags a table entry outside the pools, word 1 a bad length) or off
    (None), for later calls on this thread."""
    if err is not None:
        assert err.dtype == torch.uint32 or err.dtype == torch.int32, "err: 32-bit words"
        assert err.numel() >= 2 and err.is_cuda
    _check(lib().fp8pa_set_debug_checks(None if err is None else _ptr(err)))


def stream_read(buf, sink, stream=None):
    """Measurement helper: one streaming read of the whole of `buf`."""
    _check(lib().fp8pa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def device_status(reset=False):
    """The current device's status words (synchronizes the device):
    {"merge_timeouts": n}; reset clears them."""
    st = DeviceStatus()
    _check(lib().fp8pa_get_device_status(ctypes.byref(st), 1 if reset else 0))
    return {"merge_timeouts": int(st.merge_timeouts)}


def force_merge_timeout(on):
    """Test hook: while on (this thread), split merges give up waiting."""
    _check(lib().fp8pa_debug_force_merge_timeout(1 if on else 0))


def set_decode_events(start, stop):
    """Raw hipEvent_t handles (ints) that bracket the next decode kernels; None clears."""
    _check(lib().fp8pa_set_decode_events(None if start is None else ctypes.c_void_p(start),
                                         None if stop is None else ctypes.c_void_p(stop)))
