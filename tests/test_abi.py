"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8pa.h declares, and refuses bad arguments before launching anything
(the counters do not move).  Fake device addresses are used: validation never
dereferences them and every case here fails before a launch."""
import ctypes
import os
import re

import pytest

from fp8_paged_kv_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ops.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ops.SIGNATURES), "binding and header disagree"


def test_version_and_struct_sizes():
    assert b"gfx950" in ops.lib().fp8pa_version()
    assert ctypes.sizeof(ops.PoolDesc) == 48
    assert ctypes.sizeof(ops.Plan) == 24
    assert ctypes.sizeof(ops.Counters) == 104


def kd(**kw):
    a = dict(num_kv_heads=8, head_dim=128, page_size=16, layout="heads", scale_kind="page_head",
             row_bytes=16416, num_rows=100)
    a.update(kw)
    return ops.pool_desc(**a)


def vd(**kw):
    kw.setdefault("layout", "heads_dmajor")
    return kd(**kw)


F = 0x10000     # fake 16-byte aligned device address


def call_decode(k=None, v=None, **kw):
    a = dict(q=F, out=F, k_pool=F, v_pool=F, bt=F, bt_stride=512, seq_lens=F, B=2, Hq=32, window=0, sinks=None,
             sm_scale=0.1, max_seq_len=8192, workgroups=1, variant=0, ws=None, ws_bytes=0)
    a.update(kw)
    k = kd() if k is None else k
    v = vd() if v is None else v
    P = ctypes.c_void_p
    return ops.lib().fp8pa_decode(P(a["q"]), P(a["out"]), P(a["k_pool"]), P(a["v_pool"]), ctypes.byref(k),
                                  ctypes.byref(v), P(a["bt"]), a["bt_stride"], P(a["seq_lens"]), a["B"], a["Hq"],
                                  a["window"], P(a["sinks"]) if a["sinks"] else None, a["sm_scale"],
                                  a["max_seq_len"], a["workgroups"], a["variant"],
                                  P(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("case,code", [
    (dict(k=kd(head_dim=96), v=vd(head_dim=96)), ops.EUNSUPPORTED),
    (dict(k=kd(page_size=24)), ops.EUNSUPPORTED),
    (dict(k=kd(page_size=8)), ops.EUNSUPPORTED),
    (dict(k=kd(row_bytes=16400)), ops.EINVAL),                  # payload + scales do not fit
    (dict(k=kd(row_bytes=16424)), ops.EINVAL),                  # not a multiple of 16
    (dict(k=kd(scale_offset=16392)), ops.EINVAL),               # footer not 16-aligned
    (dict(k=kd(row_bytes=1 << 31)), ops.EUNSUPPORTED),          # rows of 2 GiB or more
    (dict(k=kd(scale_offset=16000)), ops.EINVAL),               # footer inside the payload
    (dict(k=kd(layout="heads_dmajor")), ops.EUNSUPPORTED),      # K must be token-major
    (dict(v=vd(layout="heads_d64")), ops.EUNSUPPORTED),         # V in HEADS_D64 is not read
    (dict(v=vd(layout="tokens"), B=2100), ops.EUNSUPPORTED),    # tile prefix + V stage exceed 64 KiB of LDS
    (dict(v=vd(num_kv_heads=4, row_bytes=8208)), ops.EUNSUPPORTED),
    (dict(v=vd(scale_kind="token_head", row_bytes=16384 + 512)), ops.EUNSUPPORTED),
    (dict(Hq=30), ops.EINVAL),
    (dict(Hq=8 * 32), ops.EUNSUPPORTED),                        # G = 32
    (dict(q=0), ops.EINVAL),
    (dict(seq_lens=0), ops.EINVAL),
    (dict(q=F + 8), ops.EINVAL),
    (dict(k_pool=F + 4), ops.EINVAL),
    (dict(bt_stride=0), ops.EINVAL),
    (dict(bt_stride=100), ops.EINVAL),                          # fewer than ceil(8192 / 16) entries
    (dict(sm_scale=float("nan")), ops.EINVAL),
    (dict(sm_scale=float("inf")), ops.EINVAL),
    (dict(variant=7), ops.EUNSUPPORTED),
    (dict(variant=2, k=kd(scale_kind="e8m0_32", head_dim=64, row_bytes=8192 + 4096),
          v=vd(scale_kind="e8m0_32", head_dim=64, row_bytes=8192 + 4096)), ops.EUNSUPPORTED),  # MX fp8: D % 128
    (dict(variant=2, v=vd(layout="tokens")), ops.EUNSUPPORTED),                    # fp8 mode: V d-major only
    (dict(variant=2, sm_scale=0.09), ops.EUNSUPPORTED),                             # fp8 mode: sm_scale > D^-0.5
    (dict(variant=2, sm_scale=-1.0), ops.EUNSUPPORTED),
    (dict(variant=3, workgroups=4, ws=F, ws_bytes=1 << 20), ops.EUNSUPPORTED),      # packed heads fix the grid
    (dict(variant=4, workgroups=0, v=vd(layout="heads")), ops.EUNSUPPORTED),        # packed splits: V d-major only
    (dict(variant=4, workgroups=0, Hq=64), ops.EUNSUPPORTED),                       # packed splits: G <= 4
    (dict(k=kd(scale_kind="f32_g32", row_bytes=16384 + 8192),
          v=vd(scale_kind="f32_g8", row_bytes=16384 + 8192)), ops.EUNSUPPORTED),    # V groups under 16 dims
    (dict(k=kd(scale_kind="token_head", row_bytes=16384 + 2048),
          v=vd(scale_kind="f32_g32", row_bytes=16384 + 2048)), ops.EUNSUPPORTED),   # V groups need K groups
    (dict(k=kd(scale_kind="f32_g32", row_bytes=16384 + 2048)), ops.EUNSUPPORTED),   # K groups with V page scales
    (dict(k=kd(scale_kind="f32_g32", row_bytes=16384 + 1024)), ops.EINVAL),         # group scales do not fit
    (dict(k=kd(scale_kind="f32_g256", row_bytes=16384 + 512),
          v=vd(scale_kind="token_head", row_bytes=16384 + 512)), ops.EINVAL),       # group wider than the head
    (dict(variant=2, k=kd(scale_kind="f32_g32", row_bytes=16384 + 2048),
          v=vd(scale_kind="token_head", row_bytes=16384 + 512)), ops.EUNSUPPORTED),  # fp8 mode: no sub-row scales
    (dict(variant=3, workgroups=0, k=kd(scale_kind="f32_g64", row_bytes=16384 + 1024),
          v=vd(scale_kind="token_head", row_bytes=16384 + 512)), ops.EUNSUPPORTED),  # packed heads: none either
    (dict(variant=4, workgroups=0, k=kd(scale_kind="f32_g64", row_bytes=16384 + 1024),
          v=vd(scale_kind="token_head", row_bytes=16384 + 512)), ops.EUNSUPPORTED),
    (dict(k=kd(scale_kind=9)), ops.EINVAL),
    (dict(max_seq_len=-1), ops.EINVAL),
    (dict(workgroups=-2), ops.EINVAL),
    (dict(workgroups=4), ops.EWORKSPACE),                       # cut units need a workspace
    (dict(workgroups=4, ws=F, ws_bytes=1024), ops.EWORKSPACE),
    (dict(workgroups=4, ws=F + 16, ws_bytes=1 << 30), ops.EINVAL),   # workspace must be 256-aligned
    (dict(B=20000), ops.EUNSUPPORTED),                          # the tile prefix would not fit in LDS
])
def test_decode_refuses_before_launch(case, code):
    ops.reset_counters()
    case = dict(case)
    rc = call_decode(**case)
    assert rc == code, ops.last_error()
    assert ops.last_error()
    c = ops.counters()
    assert c["decode_calls"] == 0 and c["decode_mfma_bf16"] == 0 and c["merge_launches"] == 0
    assert c["errors"] == 1


def test_unknown_flags_are_refused():
    k = kd()
    k.flags = 2
    assert call_decode(k=k) == ops.EINVAL


@pytest.mark.parametrize("case", [
    dict(k=kd(align64=True, scale_offset=16384)),               # aligned rows need the default footer
    dict(k=kd(head_dim=64, num_kv_heads=2, row_bytes=2048 + 128 + 48 - 64, scale_kind="token_head",
              align64=True),
         v=vd(head_dim=64, num_kv_heads=2, row_bytes=2048 + 128 + 48 - 64, scale_kind="token_head"),
         Hq=8, bt_stride=600),                                    # no room for a 48-byte shift
    dict(k=kd(align64=True), k_pool=F + 16),                     # aligned rows need a 64-byte aligned pool
])
def test_aligned_rows_are_checked(case):
    ops.reset_counters()
    assert call_decode(**case) == ops.EINVAL, ops.last_error()
    assert ops.counters()["decode_calls"] == 0


def call_append_decode(k_new=F, v_new=F, **kw):
    a = dict(q=F, out=F, k_pool=F, v_pool=F, bt=F, bt_stride=512, seq_lens=F, B=2, Hq=32, window=0, sinks=None,
             sm_scale=0.1, max_seq_len=8192, workgroups=1, variant=0, ws=None, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return ops.lib().fp8pa_append_decode(P(k_new) if k_new else None, P(v_new) if v_new else None, P(a["q"]),
                                         P(a["out"]), P(a["k_pool"]), P(a["v_pool"]), ctypes.byref(kd()),
                                         ctypes.byref(vd()), P(a["bt"]), a["bt_stride"], P(a["seq_lens"]), a["B"],
                                         a["Hq"], a["window"], None, a["sm_scale"], a["max_seq_len"],
                                         a["workgroups"], a["variant"], None, 0, None)


@pytest.mark.parametrize("case,code", [
    (dict(k_new=0), ops.EINVAL),
    (dict(v_new=0), ops.EINVAL),
    (dict(k_new=F + 1), ops.EINVAL),          # bf16 tokens must be 2-byte aligned
    (dict(k_new=F + 1, max_seq_len=1024), ops.EINVAL),   # the same on the one-launch path
    (dict(v_new=0, max_seq_len=1024), ops.EINVAL),
    (dict(Hq=30), ops.EINVAL),                # every decode check applies
])
def test_append_decode_refuses_before_launch(case, code):
    ops.reset_counters()
    assert call_append_decode(**case) == code, ops.last_error()
    c = ops.counters()
    assert c["decode_calls"] == 0 and c["fused_appends"] == 0 and c["errors"] == 1


def test_empty_batch_is_a_no_op():
    ops.reset_counters()
    assert call_decode(B=0, q=0, out=0) == ops.OK
    assert ops.counters()["decode_mfma_bf16"] == 0


def test_plan_is_host_only_and_sane():
    k = kd()
    p = ops.decode_plan(32, 32, k, vd(), 8192)
    assert p.workgroups >= 1 and p.tile_tokens == 64
    G, D = 4, 128
    if p.workgroups > 1:
        assert p.workspace_bytes >= p.workgroups * 2 * G * (D + 1) * 4 + 32 * 8 * 8
    # explicit workgroup counts are honoured
    p1 = ops.decode_plan(32, 32, k, vd(), 8192, workgroups=1)
    assert p1.workgroups == 1 and p1.workspace_bytes == 0
    p7 = ops.decode_plan(4, 32, k, vd(), 8192, workgroups=7)
    assert p7.workgroups == 7 and p7.workspace_bytes >= 7 * 2 * G * (D + 1) * 4
    # the plan depends on host values only: same answer twice, any seq_lens
    assert ops.decode_plan(32, 32, k, vd(), 8192).workgroups == p.workgroups
    # head dims 256 and 512 use 32-position tiles
    assert ops.decode_plan(16, 16, kd(head_dim=512, num_kv_heads=2, page_size=32, row_bytes=65568),
                           vd(head_dim=512, num_kv_heads=2, page_size=32, row_bytes=65568), 16384).tile_tokens == 32
    with pytest.raises(ops.Fp8paError):
        ops.decode_plan(1, 8, kd(head_dim=80), vd(head_dim=80), 100)


def call_append(**kw):
    a = dict(k_new=F, v_new=F, k_pool=F, v_pool=F, bt=F, bt_stride=8, positions=F, counts=None, B=2, T=1)
    a.update(kw)
    k, v = kw.get("k", kd()), kw.get("v", vd())
    P = ctypes.c_void_p
    return ops.lib().fp8pa_append_quant(P(a["k_new"]), P(a["v_new"]), P(a["k_pool"]), P(a["v_pool"]),
                                        ctypes.byref(k), ctypes.byref(v), P(a["bt"]), a["bt_stride"],
                                        P(a["positions"]), P(a["counts"]) if a["counts"] else None, a["B"], a["T"],
                                        None)


@pytest.mark.parametrize("case,code", [
    (dict(k_new=0), ops.EINVAL), (dict(positions=0), ops.EINVAL), (dict(k_new=F + 1), ops.EINVAL),
    (dict(bt_stride=0), ops.EINVAL), (dict(B=-1), ops.EINVAL),
    (dict(v=vd(page_size=32, row_bytes=32800)), ops.EUNSUPPORTED),
    (dict(k=kd(head_dim=48)), ops.EUNSUPPORTED),
])
def test_append_refuses_before_launch(case, code):
    ops.reset_counters()
    assert call_append(**case) == code
    assert ops.counters()["append_launches"] == 0


def test_merge_and_debug_refuse_before_launch():
    P = ctypes.c_void_p
    ops.reset_counters()
    assert ops.lib().fp8pa_merge_splits(P(F), P(F), None, P(F), 2, 8, 4, 80, None) == ops.EUNSUPPORTED
    assert ops.lib().fp8pa_merge_splits(None, P(F), None, P(F), 2, 8, 4, 64, None) == ops.EINVAL
    assert ops.lib().fp8pa_merge_splits(P(F), P(F), None, P(F), 2, 0, 4, 64, None) == ops.EINVAL
    assert ops.lib().fp8pa_debug_dequant(P(F), P(F), 9, 16, P(F), None) == ops.EINVAL
    assert ops.lib().fp8pa_debug_dequant(None, P(F), 0, 16, P(F), None) == ops.EINVAL
    c = ops.counters()
    assert c["merge_launches"] == 0 and c["debug_launches"] == 0 and c["errors"] == 5


def test_plan_of_the_variants():
    """Host-only plans: packed heads fix the grid at B * ceil(Hkv / 4) with no
    workspace; packed splits need partials for 4 * G query heads per unit;
    the fp8 mode plans like the default; the plan reports the variant."""
    k = kd()                                   # Hkv 8, D 128
    pk = ops.decode_plan(5, 32, k, vd(), 8192, variant="packed_heads")
    assert pk.workgroups == 10 and pk.workspace_bytes == 0 and pk.variant == ops.VARIANTS["packed_heads"]
    k6 = kd(num_kv_heads=6, row_bytes=12320)
    assert ops.decode_plan(3, 24, k6, vd(num_kv_heads=6, row_bytes=12320), 8192, variant="packed_heads").workgroups == 6
    ps = ops.decode_plan(4, 32, k, vd(), 8192, workgroups=7, variant="packed_split")
    df = ops.decode_plan(4, 32, k, vd(), 8192, workgroups=7)
    assert ps.variant == ops.VARIANTS["packed_split"] and ps.workgroups == 7
    assert ps.workspace_bytes >= 7 * 2 * 16 * (128 + 1) * 4 > df.workspace_bytes
    f8 = ops.decode_plan(4, 32, k, vd(), 8192, workgroups=7, variant="mfma_fp8")
    assert f8.variant == ops.VARIANTS["mfma_fp8"] and f8.workspace_bytes == df.workspace_bytes
    assert df.variant == ops.VARIANTS["mfma_bf16"]


def test_debug_checks_setting():
    """fp8pa_set_debug_checks: a misaligned word is refused; with checks on, a
    descriptor without a row count is refused before launch; NULL turns them off."""
    P = ctypes.c_void_p
    assert ops.lib().fp8pa_set_debug_checks(P(F + 2)) == ops.EINVAL
    assert ops.lib().fp8pa_set_debug_checks(P(F)) == ops.OK
    try:
        ops.reset_counters()
        assert call_decode(k=kd(num_rows=0)) == ops.EINVAL, ops.last_error()
        assert ops.counters()["decode_calls"] == 0
    finally:
        assert ops.lib().fp8pa_set_debug_checks(None) == ops.OK
    assert call_decode(k=kd(num_rows=0), workgroups=4) == ops.EWORKSPACE   # checks off: the next check applies


def test_plan_validates_like_decode_and_sizes_the_workspace():
    """The plan refuses what fp8pa_decode refuses for the pools (V in
    HEADS_D64, K/V geometry mismatch, V sub-row groups), and
    fp8pa_decode_workspace_bytes equals plan.workspace_bytes or returns the
    refusal's status."""
    for v in (vd(layout="heads_d64"), vd(num_kv_heads=4, row_bytes=8208),
              vd(scale_kind="f32_g32", row_bytes=16384 + 2048)):
        with pytest.raises(ops.Fp8paError) as e:
            ops.decode_plan(4, 32, kd(), v, 8192, workgroups=7)
        assert e.value.code == ops.EUNSUPPORTED
        with pytest.raises(ops.Fp8paError):
            ops.decode_workspace_bytes(4, 32, kd(), v, 8192, workgroups=7)
        assert ops.lib().fp8pa_decode_workspace_bytes(4, 32, ctypes.byref(kd()), ctypes.byref(v), 8192, 0, 7, 0) \
            == ops.EUNSUPPORTED
    for wg in (1, 7, 300):
        p = ops.decode_plan(4, 32, kd(), vd(), 8192, workgroups=wg)
        assert ops.decode_workspace_bytes(4, 32, kd(), vd(), 8192, workgroups=wg) == p.workspace_bytes
    # V token-major: the same grid, more LDS; the split kernel's workspace
    assert ops.decode_plan(4, 32, kd(), vd(layout="tokens"), 8192, workgroups=7).workspace_bytes == \
        ops.decode_plan(4, 32, kd(), vd(), 8192, workgroups=7).workspace_bytes
    # a call with fewer bytes than the plan's is refused; exactly the plan's is accepted by validation
    n = ops.decode_workspace_bytes(2, 32, kd(), vd(), 8192, workgroups=4)
    assert call_decode(workgroups=4, ws=F, ws_bytes=n - 1) == ops.EWORKSPACE
