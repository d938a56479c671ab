"""GPU parity: libhogwild_attn (through its C ABI) against the CPU oracle.

Attention outputs: bf16 inputs within 5e-3 max-abs and 1e-2 relative L2 of the
fp64 oracle; fp32 inputs within 1e-5 (normwise).  Tables, lengths and append
indexing: bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import workloads
import hw_harness
from hw_harness import Setup, assert_close, errors

pytestmark = pytest.mark.gpu

# The MFMA path through both entry points: hw_attn_decode (the kernel with the
# in-kernel plan, up to 32 rows) and hw_attn_plan + hw_attn_run (MFMA_RUN).
MFMA_RUN = "mfma_plan_run"
PATHS = [hw.PATH_VALU, hw.PATH_MFMA, MFMA_RUN]


def _tune(path, units=0, balance=0):
    hw_harness.API = "plan_run" if path == MFMA_RUN else "decode"
    hw.hw_set_tuning(hw.PATH_MFMA if path == MFMA_RUN else path, units, balance)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _tuning(request):
    _say(f"[case] {request.node.name}")
    yield
    hw_harness.API = "decode"
    hw.hw_set_tuning(hw.PATH_AUTO, 0)


def _custom(W, Hq, Hkv, D, lens, dtype=torch.bfloat16, theta=1e6, caps=None, sigma=0.5, seed=7):
    caps = caps or [workloads.round_up(max(x, 1)) for x in lens]
    return workloads.Workload(f"custom_W{W}_G{Hq // Hkv}_D{D}", W, Hq, Hkv, D, theta, dtype, 1,
                              list(lens), list(caps), sigma, seed)


# ---------------------------------------------------------------- tables (a1)
@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_device_tables_match_oracle(W):
    rng = np.random.default_rng(W)
    for trial in range(5):
        lens = [int(x) for x in rng.integers(0, 300, size=W + 1)]
        wl = _custom(W, 8 * W, 8, 64, lens)
        pool = hw.Pool(1, 1, 64, wl.caps, dtype=torch.bfloat16)
        pool.set_lengths(lens)
        t = torch.zeros(W, W + 1, 2, dtype=torch.int32, device="cuda")
        ne = torch.zeros(W, dtype=torch.int32, device="cuda")
        hw.hw_build_combined_tables(pool, W, 0, list(range(1, W + 1)), t, ne)
        tb, to, one = oracle.build_combined_tables(0, list(range(1, W + 1)), lens)
        t = t.cpu().numpy()
        assert (t[..., 0] == tb).all() and (t[..., 1] == to).all()
        assert (ne.cpu().numpy() == one).all()


# --------------------------------------------------------- decode, configs
def test_tiny_fp32_matches_oracle_definition_form():
    s = Setup(workloads.tiny())
    ref, rc = s.oracle_decode(form=oracle.FORM_DEFINITION)
    assert rc == 0
    got = s.decode()
    assert_close(got, ref, torch.float32, "tiny fp32")


@pytest.mark.parametrize("path", PATHS)
def test_qwq_layer_bf16_matches_oracle(path):
    _tune(path, 0)
    s = Setup(workloads.qwq_layer())
    ref, rc = s.oracle_decode()
    assert rc == 0
    got = s.decode()
    ma, rl = assert_close(got, ref, torch.bfloat16, f"qwq layer path {path}")
    _say(f"  path {path}: max_abs {ma:.2e} rel_l2 {rl:.2e}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", [
    # (W, Hq, Hkv, D, lens)  ragged tails, empty blocks, one-token blocks, GQA 1..8
    (1, 8, 8, 128, [37, 0]),
    (1, 1, 1, 64, [1, 0]),
    (1, 2, 1, 128, [0, 1]),
    (2, 4, 2, 64, [256, 64, 64]),
    (2, 16, 2, 128, [70, 0, 33]),
    (3, 6, 2, 64, [1, 1, 1, 1]),
    (4, 40, 8, 128, [1000, 257, 31, 0, 64]),
    (8, 8, 2, 64, [300] + [5, 17, 0, 33, 64, 1, 2, 40]),
    (4, 32, 8, 128, [2048, 100, 200, 300, 400]),
    (16, 16, 4, 64, [129] + [3] * 16),
])
def test_ragged_shapes_match_oracle(path, case):
    W, Hq, Hkv, D, lens = case
    _tune(path, 0)
    wl = _custom(W, Hq, Hkv, D, lens)
    s = Setup(wl, poison_unused=True)
    ref, rc = s.oracle_decode()
    assert rc == 0
    got = s.decode()
    assert np.isfinite(got).all()
    assert_close(got, ref, torch.bfloat16, f"{case} path {path}")


@pytest.mark.parametrize("path", PATHS)
def test_fp32_ragged_matches_oracle(path):
    if path != hw.PATH_VALU:
        wl = _custom(2, 4, 2, 64, [40, 3, 9], dtype=torch.float32, theta=1e4, sigma=0.0)
        s = Setup(wl)
        _tune(path, 0)
        assert hw.hw_attn_workspace_bytes(s.pool, 2, 4) == 0
        q = s.q[0].cuda()
        out = torch.zeros(2, 4, 64, device="cuda")
        with pytest.raises(hw.HWError) as e:
            hw.hw_attn_decode(s.pool, 0, q, s.tables, s.num_entries, wl.theta, out, s.ws)
        assert e.value.code == hw.HW_EUNSUPPORTED
        return
    wl = _custom(3, 6, 3, 128, [200, 31, 0, 65], dtype=torch.float32, theta=1e4, sigma=0.0)
    s = Setup(wl, poison_unused=True)
    ref, rc = s.oracle_decode(form=oracle.FORM_DEFINITION)
    assert rc == 0
    assert_close(s.decode(), ref, torch.float32, "fp32 ragged")


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("path", PATHS)
def test_single_visible_token_returns_value_exactly(path):
    _tune(path, 0)
    wl = _custom(2, 4, 2, 128, [1, 0, 0], seed=3)
    s = Setup(wl, poison_unused=True)
    got = s.decode()
    V = s.V[0].float().numpy()
    for w in range(2):
        for h in range(4):
            assert (got[w, h] == V[h // 2, 0]).all()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("units", [1, 2])
def test_unit_spanning_many_blocks(path, units):
    # one or two work units cover 8-17 visible blocks (16 workers, 32 rows):
    # the rotated queries are built for several groups of blocks in turn
    # inside one workgroup
    wl = _custom(16, 2, 1, 128, [40] + [3] * 12 + [0, 33, 1, 64])
    _tune(path, units)
    s = Setup(wl, poison_unused=True)
    ref, rc = s.oracle_decode()
    assert rc == 0
    got = s.decode()
    assert np.isfinite(got).all()
    assert_close(got, ref, torch.bfloat16, f"many blocks units {units} path {path}")


@pytest.mark.parametrize("path", PATHS)
def test_unit_count_does_not_change_the_result(path):
    wl = _custom(4, 40, 8, 128, [3000, 100, 31, 250, 7])
    s = Setup(wl)
    outs = []
    for units in (1, 3, 16, 64):
        _tune(path, units)
        s.ws = hw.alloc_workspace(s.pool, wl.W, wl.Hq)
        outs.append(s.decode())
    ref, _ = s.oracle_decode()
    for o in outs:
        assert_close(o, ref, torch.bfloat16, f"units path {path}")
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 2e-3


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_across_runs(path):
    """Static tile ranges (balance 0): bitwise the same result on every run; balanced
    tile order: the same result within rounding, and both match the oracle."""
    _tune(path, 0, 0)
    s = Setup(workloads.qwq_layer())
    a = s.decode()
    b = s.decode()
    assert np.array_equal(a, b)
    _tune(path, 0, 1)
    c = s.decode()
    d = s.decode()
    assert np.abs(c - a).max() < 1e-4 and np.abs(d - a).max() < 1e-4
    ref, _ = s.oracle_decode()
    assert_close(c, ref, torch.bfloat16, "balanced")
    assert hw.hw_pool_status(s.pool) == 0


@pytest.mark.parametrize("path", PATHS)
def test_batched_workers_equal_single_worker_calls(path):
    _tune(path, 0)
    wl = _custom(4, 16, 4, 128, [500, 40, 90, 3, 77])
    s = Setup(wl)
    full = s.decode()
    tb = s.tables.cpu()
    ne = s.num_entries.cpu()
    for w in range(wl.W):
        one = s.decode(q=s.q[0][w:w + 1], tables=tb[w:w + 1].contiguous().cuda(),
                       num_entries=ne[w:w + 1].contiguous().cuda())
        assert np.abs(one[0] - full[w]).max() < 1e-6


@pytest.mark.parametrize("path", PATHS)
def test_partial_visibility_and_entry_order(path):
    _tune(path, 0)
    wl = _custom(3, 6, 2, 64, [120, 50, 60, 70])
    s = Setup(wl)
    # worker 0: only common and its own block; worker 1: reversed order of entries;
    # worker 2: common only, shifted offsets
    tables = np.zeros((3, 4, 2), np.int32)
    ne = np.array([2, 4, 1], np.int32)
    tables[0, :2] = [(0, 0), (1, 120)]
    tables[1, :4] = [(2, 240), (3, 170), (1, 120), (0, 0)]
    tables[2, :1] = [(0, 1000)]
    got = s.decode(tables=torch.from_numpy(tables).cuda(), num_entries=torch.from_numpy(ne).cuda())
    ref, rc = s.oracle_decode(tables=(tables[..., 0].copy(), tables[..., 1].copy(), ne))
    assert rc == 0
    assert_close(got, ref, torch.bfloat16, "partial visibility")


# ------------------------------------------------------- device error paths
def test_spin_limit_ends_the_launch_and_reports(monkeypatch):
    """The waits between the waves of a work unit are bounded.  Forced from the host
    (HW_SPIN_LIMIT=0 polls: a wait not satisfied at its first poll gives up), every
    launch still ends; a call either matches the oracle (all its waits happened to
    be satisfied at once) or reports HW_DEV_SPIN_LIMIT.  At the default limit the
    result is exact again and no bit is set."""
    s = Setup(workloads.qwq_layer())
    ref, rc = s.oracle_decode()
    assert rc == 0
    hw.hw_pool_status(s.pool, clear=True)
    monkeypatch.setenv("HW_SPIN_LIMIT", "0")
    hits = 0
    for _ in range(5):
        got = s.decode(api="decode")
        flags = hw.hw_pool_status(s.pool, clear=True)
        assert not np.isnan(got).any()
        if flags & hw.HW_DEV_SPIN_LIMIT:
            hits += 1
        else:
            assert_close(got, ref, torch.bfloat16, "zero spin limit, no wait gave up")
    monkeypatch.delenv("HW_SPIN_LIMIT")
    assert_close(s.decode(api="decode"), ref, torch.bfloat16, "default spin limit")
    assert hw.hw_pool_status(s.pool) == 0
    _say(f"  {hits} of 5 calls at a zero limit reported HW_DEV_SPIN_LIMIT")


@pytest.mark.parametrize("api", ["decode", "plan_run"])
def test_bad_table_entry_sets_status_and_zeroes_that_worker(api):
    wl = _custom(2, 4, 2, 64, [64, 32, 32])
    s = Setup(wl)
    hw.hw_pool_status(s.pool, clear=True)
    tables = s.tables.clone()
    tables[1, 1, 0] = 99  # block id out of range for worker 1
    got = s.decode(tables=tables, api=api)
    flags = hw.hw_pool_status(s.pool, clear=True)
    assert flags & hw.HW_DEV_BAD_ENTRY
    assert (got[1] == 0).all()
    ref, _ = s.oracle_decode()
    assert_close(got[0], ref[0], torch.bfloat16, "healthy worker")


@pytest.mark.parametrize("api", ["decode", "plan_run"])
def test_length_beyond_capacity_sets_status(api):
    wl = _custom(1, 2, 2, 64, [64, 32])
    s = Setup(wl)
    hw.hw_pool_status(s.pool, clear=True)
    s.pool.set_lengths([64, 33])  # capacity of block 1 is 32
    s.decode(api=api)
    assert hw.hw_pool_status(s.pool, clear=True) & hw.HW_DEV_BAD_LENGTH


@pytest.mark.parametrize("api", ["decode", "plan_run"])
def test_worker_without_tokens_gets_zeros_and_status(api):
    wl = _custom(2, 4, 2, 64, [0, 0, 0])
    s = Setup(wl)
    hw.hw_pool_status(s.pool, clear=True)
    got = s.decode(api=api)
    assert (got == 0).all()
    assert hw.hw_pool_status(s.pool, clear=True) & hw.HW_DEV_NO_TOKENS


# ---------------------------------------------------------------- append (a5)
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_matches_oracle_bit_exact(dtype, D):
    theta = 1e6 if dtype == torch.bfloat16 else 1e4
    lens = [1000, 333, 17, 64]
    wl = workloads.Workload("append", 3, 6, 2, D, theta, dtype, 2, lens,
                            [2048, 352, 32, 64], 0.5, 11)
    s = Setup(wl, n_layers=2)
    src, dst = 1, 0
    K0 = np.stack([k.double().numpy() for k in s.K])
    V0 = np.stack([v.double().numpy() for v in s.V])
    Ko, Vo = K0.copy(), V0.copy()
    lo = np.array(lens, np.int32)
    rc = oracle.block_append(Ko, Vo, s.pool.block_start, s.pool.block_cap, lo, src, dst, theta,
                             oracle.HWO_BF16 if dtype == torch.bfloat16 else oracle.HWO_F32)
    assert rc == 0
    hw.hw_block_append(s.pool, src, dst, theta)
    torch.cuda.synchronize()
    assert s.pool.block_len.cpu().tolist() == lo.tolist()
    for layer in range(2):
        Kg, Vg = s.pool.load_layer(layer)
        Kg = Kg.cpu().double().numpy()
        Vg = Vg.cpu().double().numpy()
        assert np.array_equal(Vg, Vo[layer])
        if dtype == torch.bfloat16:
            assert np.array_equal(Kg, Ko[layer])
        else:
            diff = Kg != Ko[layer]
            if diff.any():  # at most one ulp of fp32, and rarely
                ulp = np.spacing(np.abs(Ko[layer][diff]).astype(np.float32)).astype(np.float64)
                assert (np.abs(Kg[diff] - Ko[layer][diff]) <= ulp).all()
                assert diff.sum() <= 4


def test_append_then_review_attention_is_unchanged():
    """src right after common in worker 0's view: attention before == after the append."""
    wl = _custom(2, 8, 2, 128, [700, 45, 300], caps=[1024, 64, 320])
    s = Setup(wl)
    before = s.decode()
    hw.hw_block_append(s.pool, 2, 0, wl.theta)  # worker 1's block follows common for worker 0
    hw.hw_build_combined_tables(s.pool, wl.W, 0, wl.worker_block, s.tables, s.num_entries)
    after = s.decode()
    assert s.pool.block_len.cpu().tolist() == [1000, 45, 0]
    assert np.abs(after[0] - before[0]).max() < 5e-3


def test_append_overflow_moves_nothing():
    wl = _custom(1, 2, 2, 64, [30, 20], caps=[32, 32])
    s = Setup(wl)
    hw.hw_pool_status(s.pool, clear=True)
    k0, v0 = s.pool.k.clone(), s.pool.v.clone()
    hw.hw_block_append(s.pool, 1, 0, wl.theta)
    assert hw.hw_pool_status(s.pool, clear=True) & hw.HW_DEV_APPEND_OVERFLOW
    assert s.pool.block_len.cpu().tolist() == [30, 20]
    assert torch.equal(s.pool.k, k0) and torch.equal(s.pool.v, v0)


def test_reset_block():
    wl = _custom(1, 2, 2, 64, [30, 20], caps=[32, 32])
    s = Setup(wl)
    hw.hw_block_reset(s.pool, 1)
    assert s.pool.block_len.cpu().tolist() == [30, 0]


# ------------------------------------------- full-size step (sampled outputs)
# ------------------------------------------------------ cache layouts (NEXT-2)
@pytest.mark.parametrize("layout", [hw.HW_LAYOUT_COMBINED, hw.HW_LAYOUT_INTERLEAVED,
                                    hw.HW_LAYOUT_CONTIGUOUS])
@pytest.mark.parametrize("W", [1, 2, 4])
def test_view_tables_match_oracle(layout, W):
    lens = [700] + [37 * (w + 1) for w in range(W)]
    wl = _custom(W, 2 * W, W, 64, lens)
    s = Setup(wl)
    hw.hw_build_view_tables(s.pool, layout, W, 0, wl.worker_block, s.tables, s.num_entries)
    torch.cuda.synchronize()
    build = (oracle.build_interleaved_tables if layout == hw.HW_LAYOUT_INTERLEAVED
             else oracle.build_combined_tables)
    tb, to, ne = build(0, wl.worker_block, np.array(lens, np.int32))
    t = s.tables.cpu().numpy()
    assert s.num_entries.cpu().tolist() == ne.tolist()
    assert np.array_equal(t[:, :, 0], tb) and np.array_equal(t[:, :, 1], to)


@pytest.mark.parametrize("path", PATHS)
def test_interleaved_layout_attention_matches_oracle(path):
    _tune(path, 0)
    wl = _custom(4, 40, 8, 128, [3000, 500, 77, 300, 129])
    s = Setup(wl, poison_unused=True)
    hw.hw_build_view_tables(s.pool, hw.HW_LAYOUT_INTERLEAVED, wl.W, 0, wl.worker_block, s.tables,
                            s.num_entries)
    got = s.decode()
    lens = np.array(wl.lens, np.int32)
    ref, rc = s.oracle_decode(tables=oracle.build_interleaved_tables(0, wl.worker_block, lens))
    assert rc == 0
    assert_close(got, ref, torch.bfloat16, f"interleaved path {path}")


# --------------------------------------------- multi-token query chunks (NEXT-3)
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", [
    # (W, n, Hq, Hkv, D, lens): rows = W * n * Hq / Hkv
    (2, 4, 4, 2, 128, [900, 70, 45]),
    (4, 8, 8, 8, 64, [300, 9, 33, 64, 1]),        # chunk longer than some own blocks
    (1, 16, 16, 4, 128, [2048, 100]),            # 64 rows
    (2, 3, 40, 8, 128, [4000, 333, 517]),        # QwQ heads, 30 rows
    (4, 4, 40, 8, 128, [3000, 200, 5, 64, 77]),  # four 4-token block headers at G = 5: 80 rows
    (1, 12, 40, 8, 128, [5000, 900]),            # a 12-token prompt of one worker: 60 rows
    (3, 3, 40, 8, 64, [700, 40, 41, 3]),         # 45 rows, D = 64
    (3, 3, 40, 8, 128, [1500, 70, 9, 300]),      # 45 rows, D = 128: row groups of 2 + 1 row tiles
    (2, 7, 40, 8, 128, [2500, 130, 7]),          # 70 rows: the second group's last row tile partly used
    (4, 4, 40, 8, 64, [900, 60, 5, 64, 33]),     # 80 rows, D = 64: row groups of 3 + 2 row tiles
    (1, 16, 32, 8, 64, [1300, 200]),             # 64 rows, D = 64: row groups of 2 + 2 row tiles
])
def test_chunk_matches_oracle(path, case):
    W, n, Hq, Hkv, D, lens = case
    _tune(path, 0)
    wl = _custom(W, Hq, Hkv, D, lens)
    if path == hw.PATH_VALU and W * n * (Hq // Hkv) > 64:
        pytest.skip("the VALU kernel holds at most 64 rows")
    s = Setup(wl, poison_unused=True)
    g = torch.Generator().manual_seed(9)
    q = torch.randn(W, n, Hq, D, generator=g).to(wl.dtype)
    out = torch.full((W, n, Hq, D), float("nan"), device="cuda")
    ws = hw.alloc_workspace(s.pool, W * n, Hq)
    if path == MFMA_RUN:
        plan = hw.alloc_plan(s.pool, W, Hq, chunk=n)
        hw.hw_attn_plan(s.pool, s.tables, s.num_entries, plan, Hq, chunk=n)
        hw.hw_attn_run(s.pool, 0, q.cuda(), plan, wl.theta, out, ws)
    else:
        hw.hw_attn_chunk(s.pool, 0, q.cuda(), s.tables, s.num_entries, wl.theta, out, ws)
    torch.cuda.synchronize()
    tb, to, ne = s.oracle_tables()
    ref, rc = oracle.attn_chunk(oracle.FORM_METHOD, q.double().numpy(), s.K[0].double().numpy(),
                                s.V[0].double().numpy(), tb, to, ne, np.array(lens, np.int32),
                                np.asarray(s.pool.block_start, np.int64), wl.theta)
    assert rc == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, torch.bfloat16, f"chunk {case} path {path}")
    assert hw.hw_pool_status(s.pool) == 0


@pytest.mark.parametrize("path", [hw.PATH_MFMA, MFMA_RUN])
@pytest.mark.parametrize("n", [3, 4])
def test_chunk_partial_visibility_and_entry_order(path, n):
    """Chunks over views that leave blocks out, list entries out of order and
    shift offsets: 4 workers x n tokens x G = 5 (60 or 80 rows, the row-group
    kernel).  Worker 0 sees the common block and its own; worker 1 three
    blocks in reversed order; worker 2 only the common block, shifted (its
    chunk is then the common block's last n tokens); worker 3 every block, its
    own one first at a far offset."""
    _tune(path, 0)
    lens = [900, 60, 5, 64, 33]
    wl = _custom(4, 40, 8, 128, lens)
    s = Setup(wl, poison_unused=True)
    tables = np.zeros((4, 5, 2), np.int32)
    ne = np.array([2, 3, 1, 5], np.int32)
    tables[0, :2] = [(0, 0), (1, 900)]
    tables[1, :3] = [(3, 965), (2, 1029), (0, 0)]
    tables[2, :1] = [(0, 500)]
    tables[3, :5] = [(4, 2000), (1, 900), (0, 0), (2, 960), (3, 965)]
    g = torch.Generator().manual_seed(11)
    q = torch.randn(4, n, 40, 128, generator=g).to(wl.dtype)
    out = torch.full((4, n, 40, 128), float("nan"), device="cuda")
    ws = hw.alloc_workspace(s.pool, 4 * n, 40)
    tb_dev, ne_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(ne).cuda()
    if path == MFMA_RUN:
        plan = hw.alloc_plan(s.pool, 4, 40, chunk=n)
        hw.hw_attn_plan(s.pool, tb_dev, ne_dev, plan, 40, chunk=n)
        hw.hw_attn_run(s.pool, 0, q.cuda(), plan, wl.theta, out, ws)
    else:
        hw.hw_attn_chunk(s.pool, 0, q.cuda(), tb_dev, ne_dev, wl.theta, out, ws)
    torch.cuda.synchronize()
    ref, rc = oracle.attn_chunk(oracle.FORM_METHOD, q.double().numpy(), s.K[0].double().numpy(),
                                s.V[0].double().numpy(), tables[..., 0].copy(),
                                tables[..., 1].copy(), ne, np.array(lens, np.int32),
                                np.asarray(s.pool.block_start, np.int64), wl.theta)
    assert rc == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, torch.bfloat16, f"chunk partial visibility n={n} path {path}")
    assert hw.hw_pool_status(s.pool) == 0


def test_chunk_of_one_equals_decode():
    wl = _custom(4, 40, 8, 128, [2000, 300, 31, 64, 5])
    s = Setup(wl)
    dec = s.decode()
    out = torch.zeros(wl.W, 1, wl.Hq, wl.D, device="cuda")
    hw.hw_attn_chunk(s.pool, 0, s.q[0][:, None].contiguous().cuda(), s.tables, s.num_entries,
                     wl.theta, out, s.ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy()[:, 0], dec)


# ------------------------------------------------------- token write (NEXT-1)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_token_write_matches_oracle_bit_exact(dtype):
    theta = 1e6 if dtype == torch.bfloat16 else 1e4
    lens = [300, 31, 64, 0]
    wl = workloads.Workload("write", 3, 6, 2, 128, theta, dtype, 2, lens, [512, 64, 96, 32], 0.5, 13)
    s = Setup(wl, n_layers=2)
    blocks = [1, 2, 3]
    g = torch.Generator().manual_seed(5)
    kn = [torch.randn(3, wl.Hkv, wl.D, generator=g) for _ in range(2)]
    vn = [torch.randn(3, wl.Hkv, wl.D, generator=g) for _ in range(2)]
    hw.hw_block_advance(s.pool, blocks)
    for layer in range(2):
        hw.hw_block_write(s.pool, layer, blocks, kn[layer].cuda(), vn[layer].cuda(), theta)
    torch.cuda.synchronize()
    lo = np.array(lens, np.int32)
    lo[blocks] += 1
    assert s.pool.block_len.cpu().tolist() == lo.tolist()
    assert hw.hw_pool_status(s.pool) == 0
    dt = oracle.HWO_BF16 if dtype == torch.bfloat16 else oracle.HWO_F32
    for layer in range(2):
        Ko = s.K[layer].double().numpy().copy()
        Vo = s.V[layer].double().numpy().copy()
        rc = oracle.block_write(Ko, Vo, s.pool.block_start, lo, blocks, kn[layer].double().numpy(),
                                vn[layer].double().numpy(), theta, dt)
        assert rc == 0
        Kg, Vg = s.pool.load_layer(layer)
        Kg, Vg = Kg.cpu().double().numpy(), Vg.cpu().double().numpy()
        assert np.array_equal(Vg, Vo)
        if dtype == torch.bfloat16:
            assert np.array_equal(Kg, Ko)
        else:
            diff = Kg != Ko
            if diff.any():  # at most one ulp of fp32, and rarely
                ulp = np.spacing(np.abs(Ko[diff]).astype(np.float32)).astype(np.float64)
                assert (np.abs(Kg[diff] - Ko[diff]) <= ulp).all() and diff.sum() <= 4


def test_token_write_overflow_and_empty_block():
    wl = _custom(1, 2, 2, 64, [32, 0], caps=[32, 32])
    s = Setup(wl)
    K0, _ = s.pool.load_layer(0)
    hw.hw_block_advance(s.pool, [0])          # block 0 is full: nothing reserved
    one = torch.ones(1, wl.Hkv, wl.D, device="cuda")
    hw.hw_block_write(s.pool, 0, [1], one, one, wl.theta)   # block 1 is empty: nothing written
    torch.cuda.synchronize()
    assert s.pool.block_len.cpu().tolist() == [32, 0]
    assert hw.hw_pool_status(s.pool, clear=True) == hw.HW_DEV_WRITE_OVERFLOW
    K1, _ = s.pool.load_layer(0)
    assert torch.equal(K0, K1)


def test_loop_checkpoint_resume_is_bit_exact():
    """Checkpoint and resume: the pool, its lengths and the tables are caller-owned
    tensors, so a checkpoint is a host copy of them.  A shortened config-5 loop run
    straight through, and the same loop saved to host memory after step 99 (one
    append done), restored into a freshly created pool and continued, give
    bit-identical outputs at every later step and a bit-identical pool at the end
    (the merge runs in a fixed order, so a call's result depends on its inputs only)."""
    steps, L, cut = 160, 2, 100
    wl = workloads.qwen3_loop(layers=L, common0=2048, steps=steps)
    sched = workloads.loop_appends(wl, steps)
    assert any(st < cut for st in sched) and any(st >= cut for st in sched)
    gk = torch.Generator().manual_seed(23)
    kn = [torch.randn(wl.W, wl.Hkv, wl.D, generator=gk).cuda() for _ in range(L)]
    vn = [torch.randn(wl.W, wl.Hkv, wl.D, generator=gk).cuda() for _ in range(L)]

    def run(s, lo, hi, outs):
        out = torch.zeros(L, wl.W, wl.Hq, wl.D, device="cuda")
        for step in range(lo, hi):
            hw.hw_block_advance(s.pool, wl.worker_block)
            hw.hw_build_combined_tables(s.pool, wl.W, wl.common_block, wl.worker_block, s.tables,
                                        s.num_entries)
            for layer in range(L):
                hw.hw_block_write(s.pool, layer, wl.worker_block, kn[layer], vn[layer], wl.theta)
                hw.hw_attn_decode(s.pool, layer, s.q[layer].cuda(), s.tables, s.num_entries,
                                  wl.theta, out[layer], s.ws)
            outs[step] = out.cpu()
            if step in sched:
                b = wl.worker_block[sched[step]]
                hw.hw_block_append(s.pool, b, wl.common_block, wl.theta)
                hw.hw_block_reset(s.pool, b)
        torch.cuda.synchronize()

    _say("  straight run")
    a = Setup(wl, n_layers=L)
    outs_a = {}
    run(a, 0, steps, outs_a)
    _say("  run to the checkpoint, save, restore into a new pool, continue")
    b = Setup(wl, n_layers=L)
    outs_b = {}
    run(b, 0, cut, outs_b)
    ck = {"k": b.pool.k.cpu(), "v": b.pool.v.cpu(), "len": b.pool.block_len.cpu()}
    del b
    torch.cuda.empty_cache()
    c = Setup(wl, n_layers=L)
    c.pool.k.copy_(ck["k"])
    c.pool.v.copy_(ck["v"])
    c.pool.block_len.copy_(ck["len"])
    run(c, cut, steps, outs_b)
    for step in range(steps):
        assert torch.equal(outs_a[step], outs_b[step]), f"step {step}"
    assert torch.equal(a.pool.block_len.cpu(), c.pool.block_len.cpu())
    assert torch.equal(a.pool.k.cpu(), c.pool.k.cpu()) and torch.equal(a.pool.v.cpu(), c.pool.v.cpu())
    assert hw.hw_pool_status(a.pool) == 0 and hw.hw_pool_status(c.pool) == 0


# ------------------------------------------------- generation loop (config 5)
def test_generation_loop_matches_oracle():
    """A shortened config-5 loop (Qwen3-8B heads, 4 workers): every step each
    worker's block reserves a slot for its new token (hw_block_advance), the
    tables are rebuilt on the device, and every layer writes the new tokens'
    K/V (hw_block_write) and decodes; every 64 steps one worker's block is
    appended into the common block and reset.  The oracle replays the writes
    and appends on its own fp64 copy of the pool; attention is checked at
    several steps and the whole pool bit-exactly at the end."""
    steps, L = 256, 2
    wl = workloads.qwen3_loop(layers=L, common0=2048, steps=steps)
    sched = workloads.loop_appends(wl, steps)
    s = Setup(wl, n_layers=L)
    Kh = np.stack([k.double().numpy() for k in s.K])
    Vh = np.stack([v.double().numpy() for v in s.V])
    lens = np.array(wl.lens, np.int32)
    starts = np.asarray(s.pool.block_start, np.int64)
    out = torch.zeros(L, wl.W, wl.Hq, wl.D, device="cuda")
    checks = {0, 63, 64, 130, 255}
    worst = 0.0
    gk = torch.Generator().manual_seed(17)
    kn = [torch.randn(wl.W, wl.Hkv, wl.D, generator=gk) for _ in range(L)]
    vn = [torch.randn(wl.W, wl.Hkv, wl.D, generator=gk) for _ in range(L)]
    kn_d = [k.cuda() for k in kn]
    vn_d = [v.cuda() for v in vn]
    for step in range(steps):
        lens[1:] += 1
        hw.hw_block_advance(s.pool, wl.worker_block)
        hw.hw_build_combined_tables(s.pool, wl.W, wl.common_block, wl.worker_block, s.tables,
                                    s.num_entries)
        for layer in range(L):
            hw.hw_block_write(s.pool, layer, wl.worker_block, kn_d[layer], vn_d[layer], wl.theta)
            rc = oracle.block_write(Kh[layer], Vh[layer], starts, lens, wl.worker_block,
                                    kn[layer].double().numpy(), vn[layer].double().numpy(),
                                    wl.theta, oracle.HWO_BF16)
            assert rc == 0
            hw.hw_attn_decode(s.pool, layer, s.q[layer].cuda(), s.tables, s.num_entries, wl.theta,
                              out[layer], s.ws)
        if step in checks:
            got = out.cpu().numpy()
            tb, to, ne = oracle.build_combined_tables(wl.common_block, wl.worker_block, lens)
            for layer in range(L):
                ref, rc = oracle.attn_decode(oracle.FORM_METHOD, s.q[layer].double().numpy(),
                                             Kh[layer], Vh[layer], tb, to, ne, lens, starts,
                                             wl.theta)
                assert rc == 0
                ma, _ = assert_close(got[layer], ref, torch.bfloat16, f"loop step {step} layer {layer}")
                worst = max(worst, ma)
        if step in sched:
            b = wl.worker_block[sched[step]]
            hw.hw_block_append(s.pool, b, wl.common_block, wl.theta)
            hw.hw_block_reset(s.pool, b)
            rc = oracle.block_append(Kh, Vh, starts, s.pool.block_cap, lens, b, wl.common_block,
                                     wl.theta, oracle.HWO_BF16)
            assert rc == 0
    torch.cuda.synchronize()
    assert s.pool.block_len.cpu().tolist() == lens.tolist()
    assert hw.hw_pool_status(s.pool) == 0
    for layer in range(L):
        Kg, Vg = s.pool.load_layer(layer)
        assert np.array_equal(Kg.cpu().double().numpy(), Kh[layer])
        assert np.array_equal(Vg.cpu().double().numpy(), Vh[layer])
    _say(f"  loop: {len(sched)} appends, common {lens[0]} tokens, worst max_abs {worst:.2e}")
