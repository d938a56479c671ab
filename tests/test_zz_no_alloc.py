"""hw_attn_decode_noalloc (the library's static per-GPU scratch as workspace)
against hw_attn_decode with a caller workspace, through the C ABI: two calls in
a row on one GPU, the second with a smaller input, so the second call finds the
scratch holding the first call's partials, plan and hints.  Both entry points
run the same kernels with the same fixed tile ranges: the outputs must be
bitwise equal, and within the bf16 bar (5e-3 max-abs, 1e-2 relative L2) of
the oracle."""
import sys

import numpy as np
import pytest
import torch

from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import workloads
from hw_harness import Setup, assert_close

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _wl(W, lens, seed):
    caps = [workloads.round_up(max(x, 1)) for x in lens]
    return workloads.Workload(f"noalloc_W{W}", W, 40, 8, 128, 1e6, torch.bfloat16, 1, list(lens),
                              caps, 0.5, seed)


def _noalloc(s):
    wl = s.wl
    out = torch.full((wl.W, wl.Hq, wl.D), float("nan"), device="cuda")
    hw.hw_attn_decode_noalloc(s.pool, 0, s.q[0].cuda(), s.tables, s.num_entries, wl.theta, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    hw.hw_set_tuning(hw.PATH_AUTO, 0, 0)
    # call 1: 8 workers x 5 q-heads per kv head = 40 stacked rows (plan + run kernels)
    # call 2: smaller, 2 workers = 10 rows (the kernel that plans in-launch)
    for case, wl in (("40 rows", _wl(8, [6000] + [37, 300, 0, 129, 64, 1, 500, 250], 11)),
                     ("10 rows", _wl(2, [1500, 90, 333], 12))):
        _say(f"[noalloc] {case}")
        s = Setup(wl, poison_unused=True)
        hw.hw_pool_status(s.pool, clear=True)
        got = _noalloc(s)
        ref = s.decode(api="decode")
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref), f"{case}: max diff {np.abs(got - ref).max():.3e}"
        want, rc = s.oracle_decode()
        assert rc == 0
        assert_close(got, want, torch.bfloat16, f"noalloc {case}")
        assert hw.hw_pool_status(s.pool) == 0


def test_noalloc_rejects_a_call_beyond_the_scratch():
    # 1024 kv heads (one unit each), 80 stacked rows: ~42 MB of workspace
    wl = workloads.Workload("noalloc_big", 16, 5120, 1024, 128, 1e6, torch.bfloat16, 1, [32],
                            [32], 0.5, 13)
    pool = hw.Pool(1, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    assert hw.hw_attn_workspace_bytes(pool, wl.W, wl.Hq) > hw.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(wl.W, wl.Hq, wl.D, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(wl.W, wl.Hq, wl.D, device="cuda")
    tables = torch.zeros(wl.W, 1, 2, dtype=torch.int32, device="cuda")
    ne = torch.ones(wl.W, dtype=torch.int32, device="cuda")
    with pytest.raises(hw.HWError) as e:
        hw.hw_attn_decode_noalloc(pool, 0, q, tables, ne, wl.theta, out)
    assert e.value.code == hw.HW_ERANGE
