"""CPU-side checks of libhogwild_attn: it loads, exports every declared call, and
rejects bad arguments on the host before touching the GPU.  No compute calls."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# The descriptors below carry made-up device pointers: every call must be rejected on
# the host.  Where a GPU is visible a call that slipped through would launch on them, so
# these checks run only where none is.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host-only checks with made-up device pointers")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hw.LIB_PATH):
        from decode_attention_shared_hw_amd import build
        build.build()
    return hw.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hogwild_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(hw_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(hw.EXPORTED)


def test_header_constants_match_binding():
    """Every #define of the header that the binding mirrors has the same value."""
    src = open(os.path.join(ROOT, "include", "hogwild_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    defs = dict(re.findall(r"^#define\s+(HW_\w+)\s+(.+?)\s*$", src, flags=re.M))
    value = lambda v: eval(re.sub(r"(\d)u\b", r"\1", v), {})  # noqa: E731
    checked = [n for n in defs if hasattr(hw, n)]
    for n in checked:
        assert getattr(hw, n) == value(defs[n]), n
    assert {"HW_DEV_SPIN_LIMIT", "HW_DEV_WORKSPACE", "HW_MAX_ROWS", "HW_TILE_TOKENS"} <= set(checked)
    assert hw.NOALLOC_SCRATCH_BYTES == value(defs["HW_NOALLOC_SCRATCH_BYTES"])


def test_abi_version_and_status_text(lib):
    assert hw.hw_abi_version() == 3
    assert hw.hw_status_str(hw.HW_OK) == "ok"
    assert "workspace" in hw.hw_status_str(hw.HW_EWORKSPACE)


def test_struct_layout_matches_header(lib):
    assert ctypes.sizeof(hw.hw_entry) == 8
    # 6 int32 + int64 + 8 pointers
    assert ctypes.sizeof(hw.hw_pool) == 6 * 4 + 8 + 8 * 8
    assert hw.hw_pool.num_slots.offset == 24 and hw.hw_pool.k.offset == 32
    assert hw.hw_pool.k_scale.offset == 80 and hw.hw_pool.v_scale.offset == 88


class FakePool:
    """A pool descriptor whose device pointers are never dereferenced (host checks only)."""

    def __init__(self, dtype=hw.HW_BF16, D=128, caps=(64, 32, 32), starts=None, Hkv=2, layers=1,
                 slots=None, k_scale=None, v_scale=None):
        starts = starts if starts is not None else list(np.cumsum([0] + list(caps[:-1])))
        self._s = (ctypes.c_int64 * len(caps))(*starts)
        self._c = (ctypes.c_int32 * len(caps))(*caps)
        slots = slots if slots is not None else int(sum(caps))
        self._ks = (ctypes.c_float * len(k_scale))(*k_scale) if k_scale is not None else None
        self._vs = (ctypes.c_float * len(v_scale))(*v_scale) if v_scale is not None else None
        self.desc = hw.hw_pool(dtype, layers, Hkv, D, len(caps), 0, slots, 0x1000, 0x2000,
                               0x3000, 0x4000, ctypes.cast(self._s, ctypes.c_void_p),
                               ctypes.cast(self._c, ctypes.c_void_p),
                               ctypes.cast(self._ks, ctypes.c_void_p) if self._ks else None,
                               ctypes.cast(self._vs, ctypes.c_void_p) if self._vs else None)


def decode_rc(lib, pool, layer=0, W=2, Hq=4, E=3, theta=1e4, ws_bytes=1 << 30, ptr=0x5000):
    p = ctypes.c_void_p(ptr)
    return lib.hw_attn_decode(ctypes.byref(pool.desc), layer, p, W, Hq, p, E, p, theta, p, p,
                              ws_bytes, None)


def test_decode_host_validation(lib):
    ok = FakePool()
    assert decode_rc(lib, FakePool(D=96)) == hw.HW_EUNSUPPORTED
    assert decode_rc(lib, FakePool(dtype=7)) == hw.HW_EUNSUPPORTED
    assert decode_rc(lib, ok, Hq=3) == hw.HW_EINVAL              # Hq % Hkv
    assert decode_rc(lib, ok, layer=1) == hw.HW_EINVAL           # layer out of range
    assert decode_rc(lib, ok, W=0) == hw.HW_ERANGE
    assert decode_rc(lib, ok, W=33) == hw.HW_ERANGE
    assert decode_rc(lib, ok, W=32, Hq=8) == hw.HW_ERANGE        # rows 128 > 80
    assert decode_rc(lib, ok, W=21, Hq=8) == hw.HW_ERANGE        # rows 84 > 80
    assert decode_rc(lib, ok, E=0) == hw.HW_ERANGE
    assert decode_rc(lib, ok, theta=-1.0) == hw.HW_EINVAL
    assert decode_rc(lib, ok, theta=float("nan")) == hw.HW_EINVAL
    assert decode_rc(lib, ok, ws_bytes=16) == hw.HW_EWORKSPACE
    assert decode_rc(lib, ok, ptr=0) == hw.HW_EINVAL             # null q/tables/out
    assert decode_rc(lib, FakePool(caps=(64, 33, 32))) == hw.HW_EINVAL       # cap % 32
    assert decode_rc(lib, FakePool(caps=(64, 32), starts=[0, 32])) == hw.HW_EINVAL  # overlap
    assert decode_rc(lib, FakePool(caps=(64,), slots=32)) == hw.HW_EINVAL    # beyond slots
    assert decode_rc(lib, FakePool(caps=tuple([32] * 65))) == hw.HW_ERANGE   # too many blocks
    # kv heads x split units must stay below 2^16 workgroups (units are lowered to what the
    # device holds at once, so only 2^16 kv heads at one unit each reach the bound)
    hw.hw_set_tuning(hw.PATH_AUTO, 256)
    try:
        big = FakePool(caps=(256 * 32,), Hkv=65536)
        assert decode_rc(lib, big, Hq=65536) == hw.HW_ERANGE
    finally:
        hw.hw_set_tuning(hw.PATH_AUTO, 0)


def test_noalloc_host_validation(lib):
    p = ctypes.c_void_p(0x5000)

    def rc(pool, W, Hq):
        return lib.hw_attn_decode_noalloc(ctypes.byref(pool.desc), 0, p, W, Hq, p, 3, p, 1e4, p,
                                          None)
    ok = FakePool()
    assert rc(ok, 0, 4) == hw.HW_ERANGE
    assert rc(ok, 2, 3) == hw.HW_EINVAL  # Hq % Hkv
    assert rc(FakePool(D=96), 2, 4) == hw.HW_EUNSUPPORTED
    # 1024 kv heads at one unit each and 80 stacked rows: ~42 MB of workspace,
    # more than the static scratch; rejected before any device call
    big = FakePool(Hkv=1024, caps=(32,))
    assert lib.hw_attn_workspace_bytes(ctypes.byref(big.desc), 16, 5120) > hw.NOALLOC_SCRATCH_BYTES
    assert rc(big, 16, 5120) == hw.HW_ERANGE


def test_workspace_bytes(lib):
    pool = FakePool(caps=(4096, 32, 32))
    n = lib.hw_attn_workspace_bytes(ctypes.byref(pool.desc), 2, 4)
    # merge counters (16 KB), a plan, then (m, l) + accumulators for Hkv=2 heads, rows 4,
    # D=128 and at least 2 units per head (the device's resident workgroups / Hkv)
    assert n >= 16384 + 2 * 2 * 4 * (128 + 2) * 4
    assert lib.hw_attn_workspace_bytes(ctypes.byref(pool.desc), 2, 3) == 0
    hw.hw_set_tuning(hw.PATH_AUTO, 2)
    try:
        assert lib.hw_attn_workspace_bytes(ctypes.byref(pool.desc), 2, 4) < n
    finally:
        hw.hw_set_tuning(hw.PATH_AUTO, 0)
    # at most one unit per tile the blocks can hold: counters, plan, partials,
    # tile counts and the fused kernel's first-tile hints (8 waves per unit),
    # each region 256-byte aligned
    small = FakePool(caps=(64, 32, 32))
    assert lib.hw_attn_workspace_bytes(ctypes.byref(small.desc), 2, 4) <= \
        16384 + 4 * (600 + 3 * 2) + 2 * 4 * 4 * (128 + 2) * 4 + 2 * 4 * 4 + 2 * 4 * 8 * 4 + 4 * 256
    # plans: 600 header words + one row end per (block, query row)
    assert lib.hw_attn_plan_bytes(ctypes.byref(pool.desc), 2, 1, 4) == 4 * (600 + 3 * 2)
    assert lib.hw_attn_plan_bytes(ctypes.byref(pool.desc), 2, 5, 4) == 4 * (600 + 3 * 10)
    assert lib.hw_attn_plan_bytes(ctypes.byref(pool.desc), 2, 1, 3) == 0


def test_plan_and_run_host_validation(lib):
    pool = FakePool()
    P = ctypes.byref(pool.desc)
    p = ctypes.c_void_p(0x5000)
    nb = lib.hw_attn_plan_bytes(P, 2, 1, 4)
    plan = lambda W=2, n=1, Hq=4, E=3, ptr=p, pb=nb: lib.hw_attn_plan(
        P, W, n, Hq, ptr, E, ptr, ptr, pb, None)
    assert plan(W=0) == hw.HW_ERANGE
    assert plan(n=0) == hw.HW_ERANGE
    assert plan(Hq=3) == hw.HW_EINVAL
    assert plan(E=0) == hw.HW_ERANGE
    assert plan(E=65) == hw.HW_ERANGE
    assert plan(ptr=None) == hw.HW_EINVAL
    assert plan(pb=nb - 4) == hw.HW_EWORKSPACE
    assert plan(W=21, Hq=8) == hw.HW_ERANGE     # 84 rows
    run = lambda layer=0, W=2, n=1, Hq=4, ptr=p, pb=nb, theta=1e4, ws=1 << 30: lib.hw_attn_run(
        P, layer, ptr, W, n, Hq, ptr, pb, theta, ptr, ptr, ws, None)
    assert run(layer=1) == hw.HW_EINVAL
    assert run(Hq=3) == hw.HW_EINVAL
    assert run(W=33) == hw.HW_ERANGE
    assert run(ptr=None) == hw.HW_EINVAL
    assert run(pb=nb - 4) == hw.HW_EWORKSPACE
    assert run(ws=16) == hw.HW_EWORKSPACE
    assert run(theta=0.0) == hw.HW_EINVAL
    assert run(theta=float("inf")) == hw.HW_EINVAL
    assert run(n=2) == hw.HW_EWORKSPACE         # the plan is for one query token
    # fp32 pools: the VALU kernel only, up to 64 rows
    f32 = FakePool(dtype=hw.HW_F32, Hkv=1)
    assert lib.hw_attn_plan(ctypes.byref(f32.desc), 1, 65, 1, p, 3, p, p, 1 << 20,
                            None) == hw.HW_ERANGE
    try:
        hw.hw_set_tuning(hw.PATH_MFMA, 0)
        assert lib.hw_attn_plan(ctypes.byref(f32.desc), 1, 1, 1, p, 3, p, p, 1 << 20,
                                None) == hw.HW_EUNSUPPORTED
    finally:
        hw.hw_set_tuning(hw.PATH_AUTO, 0)


def test_tuning_validation(lib):
    assert lib.hw_set_tuning(3, 0, 1) == hw.HW_EINVAL
    assert lib.hw_set_tuning(0, -1, 1) == hw.HW_EINVAL
    assert lib.hw_set_tuning(0, 257, 1) == hw.HW_EINVAL
    assert lib.hw_set_tuning(0, 0, 2) == hw.HW_EINVAL
    assert lib.hw_set_tuning(0, 0, -1) == hw.HW_EINVAL
    assert lib.hw_set_tuning(0, 0, 0) == hw.HW_OK
    assert lib.hw_set_tuning(0, 0, 1) == hw.HW_OK


def test_append_reset_tables_host_validation(lib):
    pool = FakePool()
    P = ctypes.byref(pool.desc)
    assert lib.hw_block_append(P, 1, 1, 1e4, None) == hw.HW_EINVAL
    assert lib.hw_block_append(P, 1, 3, 1e4, None) == hw.HW_EINVAL
    assert lib.hw_block_append(P, -1, 0, 1e4, None) == hw.HW_EINVAL
    assert lib.hw_block_append(P, 1, 0, 0.0, None) == hw.HW_EINVAL
    assert lib.hw_block_reset(P, 5, None) == hw.HW_EINVAL
    wb = (ctypes.c_int32 * 2)(1, 1)
    p = ctypes.c_void_p(0x5000)
    assert lib.hw_build_combined_tables(P, 2, 0, ctypes.cast(wb, ctypes.c_void_p), p, p,
                                        None) == hw.HW_EINVAL
    wb = (ctypes.c_int32 * 2)(0, 1)
    assert lib.hw_build_combined_tables(P, 2, 0, ctypes.cast(wb, ctypes.c_void_p), p, p,
                                        None) == hw.HW_EINVAL
    assert lib.hw_build_combined_tables(P, 0, 0, ctypes.cast(wb, ctypes.c_void_p), p, p,
                                        None) == hw.HW_ERANGE
    assert lib.hw_pool_status(None, None, 0, None) == hw.HW_EINVAL


def test_layout_positions_follow_the_documented_formula():
    for D in (64, 128):
        S = 64
        x = torch.arange(S * D, dtype=torch.float64).reshape(S, D)   # value = logical index
        pk = layout.pack_keys(x).reshape(-1)
        pv = layout.pack_values(x).reshape(-1)
        for slot in (0, 1, 15, 16, 17, 31, 32, 47, 63):
            for d in (0, 1, 7, 8, 63, D - 1):
                T, t = slot // 32, slot % 32
                ko = T * 32 * D + (t // 16) * 16 * D + (d // 8) * 128 + (t % 16) * 8 + d % 8
                vo = T * 32 * D + ((t % 16) // 4) * 8 * D + d * 8 + (t // 16) * 4 + t % 4
                assert pk[ko] == slot * D + d
                assert pv[vo] == slot * D + d
        assert torch.equal(layout.unpack_keys(layout.pack_keys(x)), x)
        assert torch.equal(layout.unpack_values(layout.pack_values(x)), x)


def test_token_write_host_validation(lib):
    pool = FakePool()
    P = ctypes.byref(pool.desc)
    p = ctypes.c_void_p(0x5000)
    ok = (ctypes.c_int32 * 2)(1, 2)
    dup = (ctypes.c_int32 * 2)(1, 1)
    bad = (ctypes.c_int32 * 2)(1, 3)
    cast = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert lib.hw_block_advance(P, 2, cast(dup), None) == hw.HW_EINVAL
    assert lib.hw_block_advance(P, 2, cast(bad), None) == hw.HW_EINVAL
    assert lib.hw_block_advance(P, 0, cast(ok), None) == hw.HW_ERANGE
    assert lib.hw_block_advance(P, 33, cast(ok), None) == hw.HW_ERANGE
    assert lib.hw_block_advance(P, 2, None, None) == hw.HW_EINVAL
    assert lib.hw_block_write(P, 0, 2, cast(dup), p, p, 1e4, None) == hw.HW_EINVAL
    assert lib.hw_block_write(P, 1, 2, cast(ok), p, p, 1e4, None) == hw.HW_EINVAL   # layer
    assert lib.hw_block_write(P, 0, 2, cast(ok), None, p, 1e4, None) == hw.HW_EINVAL
    assert lib.hw_block_write(P, 0, 2, cast(ok), p, p, 0.0, None) == hw.HW_EINVAL
    assert lib.hw_block_write(P, 0, 0, cast(ok), p, p, 1e4, None) == hw.HW_ERANGE


def test_view_tables_host_validation(lib):
    pool = FakePool()
    P = ctypes.byref(pool.desc)
    p = ctypes.c_void_p(0x5000)
    wb = (ctypes.c_int32 * 2)(1, 2)
    cast = ctypes.cast(wb, ctypes.c_void_p)
    assert lib.hw_build_view_tables(P, 3, 2, 0, cast, p, p, None) == hw.HW_EINVAL
    assert lib.hw_build_view_tables(P, -1, 2, 0, cast, p, p, None) == hw.HW_EINVAL


def test_chunk_host_validation(lib):
    pool = FakePool()
    P = ctypes.byref(pool.desc)
    p = ctypes.c_void_p(0x5000)
    call = lambda W, n, Hq: lib.hw_attn_chunk(P, 0, p, W, n, Hq, p, 3, p, 1e4, p, p, 1 << 30, None)
    assert call(2, 0, 4) == hw.HW_ERANGE          # chunk < 1
    assert call(2, 21, 4) == hw.HW_ERANGE         # 2 * 21 * 2 rows > 80
    assert call(2, 16, 3) == hw.HW_EINVAL         # Hq % Hkv
    assert lib.hw_attn_workspace_bytes(P, 80, 2) > 0      # 80 stacked rows (chunk of 80, G = 1)
    assert lib.hw_attn_workspace_bytes(P, 81, 2) == 0


def test_fp8_pool_host_validation(lib):
    """FP8 pools need positive finite scales for the layer's kv heads, at most
    HW_MAX_FP8_KV_HEADS kv heads, and run on the MFMA kernel only (<= 80 rows)."""
    good = [0.5, 0.25]
    assert decode_rc(lib, FakePool(dtype=hw.HW_FP8)) == hw.HW_EINVAL                # no scales
    assert decode_rc(lib, FakePool(dtype=hw.HW_FP8, k_scale=good)) == hw.HW_EINVAL  # no v scales
    for bad in ([0.5, 0.0], [0.5, -1.0], [float("nan"), 1.0], [float("inf"), 1.0]):
        assert decode_rc(lib, FakePool(dtype=hw.HW_FP8, k_scale=bad, v_scale=good)) == hw.HW_EINVAL
        assert decode_rc(lib, FakePool(dtype=hw.HW_FP8, k_scale=good, v_scale=bad)) == hw.HW_EINVAL
    many = [1.0] * 65
    assert decode_rc(lib, FakePool(dtype=hw.HW_FP8, Hkv=65, k_scale=many, v_scale=many),
                     Hq=65) == hw.HW_ERANGE
    fp8 = FakePool(dtype=hw.HW_FP8, k_scale=good, v_scale=good)
    assert decode_rc(lib, fp8, W=21, Hq=8) == hw.HW_ERANGE   # 84 rows > 80
    try:
        hw.hw_set_tuning(hw.PATH_VALU, 0)
        assert decode_rc(lib, fp8) == hw.HW_EUNSUPPORTED
    finally:
        hw.hw_set_tuning(hw.PATH_AUTO, 0)
    assert lib.hw_attn_workspace_bytes(ctypes.byref(fp8.desc), 2, 4) > 0
