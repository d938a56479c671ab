"""The Python binding rejects tensors the C ABI could misread: wrong dtype,
shape, device or layout raise ValueError before any library call.  Host only:
every call below fails validation, so nothing reaches a kernel (and the file
is skipped where a GPU is visible, since its tensors live on the host)."""
import ctypes
import types

import pytest
import torch

from decode_attention_shared_hw_amd import hogwild_attn as hw

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host tensors stand in for device buffers")

W, HQ, HKV, D = 2, 4, 2, 64


def _pool(dtype=torch.bfloat16):
    """A stand-in with the attributes the binding validates against."""
    return types.SimpleNamespace(k=torch.zeros(1, dtype=dtype), dtype=dtype, head_dim=D,
                                 num_kv_heads=HKV, num_layers=1, desc=None)


def _good(dtype=torch.bfloat16):
    qd = hw.query_dtype(dtype)
    return dict(q=torch.zeros(W, HQ, D, dtype=qd), out=torch.zeros(W, HQ, D),
                tables=torch.zeros(W, 3, 2, dtype=torch.int32),
                ne=torch.zeros(W, dtype=torch.int32))


def _decode(pool, a, noalloc=False):
    if noalloc:
        return hw.hw_attn_decode_noalloc(pool, 0, a["q"], a["tables"], a["ne"], 1e4, a["out"])
    return hw.hw_attn_decode(pool, 0, a["q"], a["tables"], a["ne"], 1e4, a["out"],
                             torch.zeros(16, dtype=torch.uint8))


MISMATCHES = [
    ("q dtype", "q", lambda t: t.float()),
    ("q shape", "q", lambda t: t[:, :HQ - 1].contiguous()),
    ("q head_dim", "q", lambda t: torch.zeros(W, HQ, D + 1, dtype=t.dtype)),
    ("q strided", "q", lambda t: torch.zeros(W, HQ, 2 * D, dtype=t.dtype)[..., ::2]),
    ("q device", "q", lambda t: torch.empty(t.shape, dtype=t.dtype, device="meta")),
    ("out dtype", "out", lambda t: t.bfloat16()),
    ("out shape", "out", lambda t: torch.zeros(W + 1, HQ, D)),
    ("out strided", "out", lambda t: torch.zeros(W, HQ, D, 2)[..., 0]),
    ("tables dtype", "tables", lambda t: t.long()),
    ("tables shape", "tables", lambda t: torch.zeros(W, 3, 3, dtype=torch.int32)),
    ("tables workers", "tables", lambda t: torch.zeros(W + 1, 3, 2, dtype=torch.int32)),
    ("num_entries dtype", "ne", lambda t: t.long()),
    ("num_entries shape", "ne", lambda t: torch.zeros(W + 1, dtype=torch.int32)),
]


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("what,key,bad", MISMATCHES, ids=[m[0] for m in MISMATCHES])
def test_decode_rejects_mismatched_tensors(what, key, bad, noalloc):
    a = _good()
    a[key] = bad(a[key])
    with pytest.raises(ValueError):
        _decode(_pool(), a, noalloc)


def test_fp32_pool_wants_fp32_queries():
    a = _good(torch.float32)
    a["q"] = a["q"].bfloat16()
    with pytest.raises(ValueError):
        _decode(_pool(torch.float32), a)


def test_chunk_rejects_mismatched_tensors():
    pool = _pool()
    q = torch.zeros(W, 3, HQ, D, dtype=torch.bfloat16)
    out = torch.zeros(W, 3, HQ, D)
    tables = torch.zeros(W, 3, 2, dtype=torch.int32)
    ne = torch.zeros(W, dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    for bad_q, bad_out in ((q.float(), out), (q, out[:, :2].contiguous()),
                           (q[:, :, :, :D - 1].contiguous(), out), (q, out.bfloat16())):
        with pytest.raises(ValueError):
            hw.hw_attn_chunk(pool, 0, bad_q, tables, ne, 1e4, bad_out, ws)


def test_run_rejects_mismatched_tensors():
    pool = _pool()
    a = _good()
    plan = torch.zeros(4, dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        hw.hw_attn_run(pool, 0, a["q"].float(), plan, 1e4, a["out"], ws)
    with pytest.raises(ValueError):
        hw.hw_attn_run(pool, 0, a["q"], plan, 1e4, a["out"].bfloat16(), ws)
    with pytest.raises(ValueError):
        hw.hw_attn_run(pool, 0, a["q"][None], plan, 1e4, a["out"], ws)


def test_token_write_rejects_mismatched_tensors():
    pool = _pool()
    good = torch.zeros(1, HKV, D)
    for k, v in ((good.bfloat16(), good), (good, torch.zeros(1, HKV, D + 1)),
                 (torch.zeros(2, HKV, D), good), (torch.zeros(1, HKV, 2 * D)[..., ::2], good)):
        with pytest.raises(ValueError):
            hw.hw_block_write(pool, 0, [1], k, v, 1e4)


def test_workspace_too_small_is_rejected():
    """The workspace check asks the library for the call's size (a host-only query)."""
    caps = (ctypes.c_int32 * 2)(64, 32)
    starts = (ctypes.c_int64 * 2)(0, 64)
    pool = _pool()
    pool.desc = hw.hw_pool(hw.HW_BF16, 1, HKV, D, 2, 0, 96, 0x1000, 0x2000, 0x3000, 0x4000,
                           ctypes.cast(starts, ctypes.c_void_p), ctypes.cast(caps, ctypes.c_void_p),
                           None, None)
    a = _good()
    need = hw.hw_attn_workspace_bytes(pool, W, HQ)
    assert need > 0
    with pytest.raises(ValueError):
        hw.hw_attn_decode(pool, 0, a["q"], a["tables"], a["ne"], 1e4, a["out"],
                          torch.zeros(need - 1, dtype=torch.uint8))
