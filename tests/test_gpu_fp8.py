"""GPU parity of FP8 E4M3 pools (the mixed-precision item of news 1114328 sec. 6)
against the CPU oracle, through the C ABI.

Attention: the oracle attends over the stored values (code * scale, exact in
fp64) with the same bf16 queries; the GPU must stay within the bf16 bar
(5e-3 max-abs, 1e-2 relative L2).  Append and token write: the stored codes
are bit-exact against the oracle's nearest-even E4M3 rounding.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import workloads
from hw_harness import Setup, assert_close, errors

pytestmark = pytest.mark.gpu

FP8 = torch.float8_e4m3fn
# hw_attn_decode (in-kernel plan up to 32 rows) and hw_attn_plan + hw_attn_run
APIS = ["decode", "plan_run"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _tuning(request):
    _say(f"[case] {request.node.name}")
    yield
    hw.hw_set_tuning(hw.PATH_AUTO, 0)


def _custom(W, Hq, Hkv, D, lens, theta=1e6, caps=None, sigma=0.5, seed=7, layers=1):
    caps = caps or [workloads.round_up(max(x, 1)) for x in lens]
    return workloads.Workload(f"custom_fp8_W{W}_G{Hq // Hkv}_D{D}", W, Hq, Hkv, D, theta, FP8,
                              layers, list(lens), list(caps), sigma, seed)


@pytest.mark.parametrize("api", APIS)
def test_fp8_qwq_layer_matches_oracle(api):
    s = Setup(workloads.with_fp8(workloads.qwq_layer()))
    ref, rc = s.oracle_decode()
    assert rc == 0
    got = s.decode(api=api)
    ma, rl = assert_close(got, ref, FP8, f"qwq layer fp8 {api}")
    # informational: the distance to attention over the unquantized bf16 pool
    sb = Setup(workloads.qwq_layer())
    refb, _ = sb.oracle_decode()
    qa, ql = errors(got, refb)
    _say(f"  fp8 vs oracle: max_abs {ma:.2e} rel_l2 {rl:.2e}; vs bf16 pool: {qa:.2e} / {ql:.2e}")


@pytest.mark.parametrize("case", [
    # (W, Hq, Hkv, D, lens)
    (1, 1, 1, 64, [1, 0]),
    (1, 8, 1, 128, [31, 0, 5]),
    (3, 6, 2, 64, [100, 1, 0, 45]),
    (2, 16, 2, 128, [300, 7, 33]),       # 16 rows
    (8, 32, 8, 128, [5000] + [17] * 8),  # 32 rows
    (4, 40, 8, 128, [2047, 511, 2, 64, 96]),
    (12, 48, 8, 64, [900] + [33] * 12),  # 72 rows
    (16, 40, 8, 128, [700] + [9] * 16),  # 80 rows
])
@pytest.mark.parametrize("api", APIS)
def test_fp8_ragged_shapes_match_oracle(case, api):
    W, Hq, Hkv, D, lens = case
    s = Setup(_custom(W, Hq, Hkv, D, lens), poison_unused=True)
    ref, rc = s.oracle_decode()
    assert rc == 0
    got = s.decode(api=api)
    assert np.isfinite(got).all()
    assert_close(got, ref, FP8, f"fp8 {case} {api}")
    assert hw.hw_pool_status(s.pool) == 0


@pytest.mark.parametrize("api", APIS)
def test_fp8_single_visible_token_returns_its_value(api):
    s = Setup(_custom(2, 4, 2, 128, [1, 0, 0]))
    got = s.decode(api=api)
    V = s.V[0]
    for w in range(2):
        for h in range(4):
            # one visible token: its value (code * scale) up to the fp32 scale product
            np.testing.assert_allclose(got[w, h], V[h // 2, 0].numpy(), rtol=1e-6, atol=0)


@pytest.mark.parametrize("case", [
    # (W, n, Hq, Hkv, D, lens): rows = W * n * Hq / Hkv
    (2, 3, 40, 8, 128, [4000, 333, 517]),        # 30 rows: one row group
    (3, 3, 40, 8, 64, [700, 40, 41, 3]),         # 45 rows, D = 64: two row groups of 2 + 1 row tiles
    (1, 12, 40, 8, 128, [5000, 900]),            # 60 rows
    (4, 4, 40, 8, 128, [3000, 200, 5, 64, 77]),  # 80 rows: row groups of 3 + 2 row tiles
    (2, 7, 40, 8, 128, [2500, 130, 7]),          # 70 rows
    (4, 4, 40, 8, 64, [900, 60, 5, 64, 33]),     # 80 rows, D = 64
])
def test_fp8_chunk_matches_oracle(case):
    W, n, Hq, Hkv, D, lens = case
    wl = _custom(W, Hq, Hkv, D, lens)
    s = Setup(wl, poison_unused=True)
    g = torch.Generator().manual_seed(9)
    q = torch.randn(W, n, Hq, D, generator=g).to(torch.bfloat16)
    out = torch.full((W, n, Hq, D), float("nan"), device="cuda")
    ws = hw.alloc_workspace(s.pool, W * n, Hq)
    hw.hw_attn_chunk(s.pool, 0, q.cuda(), s.tables, s.num_entries, wl.theta, out, ws)
    torch.cuda.synchronize()
    tb, to, ne = s.oracle_tables()
    ref, rc = oracle.attn_chunk(oracle.FORM_METHOD, q.double().numpy(), s.K[0].numpy(),
                                s.V[0].numpy(), tb, to, ne, np.array(lens, np.int32),
                                np.asarray(s.pool.block_start, np.int64), wl.theta)
    assert rc == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, FP8, f"fp8 chunk {case}")
    assert hw.hw_pool_status(s.pool) == 0


@pytest.mark.parametrize("api", APIS)
def test_fp8_unit_count_does_not_change_the_result(api):
    s = Setup(_custom(4, 40, 8, 128, [3000, 100, 200, 64, 5]))
    ref, _ = s.oracle_decode()
    for units in (1, 3, 16, 64):
        hw.hw_set_tuning(hw.PATH_AUTO, units)
        s.ws = hw.alloc_workspace(s.pool, 4, 40)
        got = s.decode(api=api)
        assert_close(got, ref, FP8, f"units {units} {api}")


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_append_matches_oracle_bit_exact(D):
    theta = 1e6
    lens = [1000, 333, 17, 64]
    wl = workloads.Workload("append_fp8", 3, 6, 2, D, theta, FP8, 2, lens,
                            [2048, 352, 32, 64], 0.5, 11)
    s = Setup(wl, n_layers=2)
    src, dst = 1, 0
    Ko = np.stack([k.numpy() for k in s.K])
    Vo = np.stack([v.numpy() for v in s.V])
    lo = np.array(lens, np.int32)
    rc = oracle.block_append(Ko, Vo, s.pool.block_start, s.pool.block_cap, lo, src, dst, theta,
                             oracle.HWO_FP8, k_scale=s.k_scale.double().numpy())
    assert rc == 0
    hw.hw_block_append(s.pool, src, dst, theta)
    torch.cuda.synchronize()
    assert s.pool.block_len.cpu().tolist() == lo.tolist()
    for layer in range(2):
        K8, V8 = s.pool.load_layer(layer)
        Kg = K8.cpu().double().numpy() * s.k_scale[layer].double().numpy()[:, None, None]
        Vg = V8.cpu().double().numpy() * s.v_scale[layer].double().numpy()[:, None, None]
        assert np.array_equal(Vg, Vo[layer])
        assert np.array_equal(Kg, Ko[layer]), int((Kg != Ko[layer]).sum())


def test_fp8_append_then_review_attention_is_nearly_unchanged():
    """src right after common in worker 0's view: the append re-rounds keys to the
    E4M3 grid, so attention moves by no more than that rounding allows."""
    wl = _custom(2, 8, 2, 128, [700, 45, 300], caps=[1024, 64, 320])
    s = Setup(wl)
    before = s.decode()
    hw.hw_block_append(s.pool, 2, 0, wl.theta)
    hw.hw_build_combined_tables(s.pool, wl.W, 0, wl.worker_block, s.tables, s.num_entries)
    after = s.decode()
    assert s.pool.block_len.cpu().tolist() == [1000, 45, 0]
    assert np.abs(after[0] - before[0]).max() < 3e-2


def test_fp8_token_write_matches_oracle_bit_exact():
    theta = 1e6
    lens = [300, 31, 64, 0]
    wl = workloads.Workload("write_fp8", 3, 6, 2, 128, theta, FP8, 2, lens, [512, 64, 96, 32], 0.5,
                            13)
    s = Setup(wl, n_layers=2)
    blocks = [1, 2, 3]
    g = torch.Generator().manual_seed(5)
    kn = [torch.randn(3, wl.Hkv, wl.D, generator=g) * 3.0 for _ in range(2)]
    vn = [torch.randn(3, wl.Hkv, wl.D, generator=g) for _ in range(2)]
    hw.hw_block_advance(s.pool, blocks)
    for layer in range(2):
        hw.hw_block_write(s.pool, layer, blocks, kn[layer].cuda(), vn[layer].cuda(), theta)
    torch.cuda.synchronize()
    lo = np.array(lens, np.int32)
    lo[blocks] += 1
    assert s.pool.block_len.cpu().tolist() == lo.tolist()
    assert hw.hw_pool_status(s.pool) == 0
    for layer in range(2):
        ks = s.k_scale[layer].double().numpy()
        vs = s.v_scale[layer].double().numpy()
        Ko, Vo = s.K[layer].numpy().copy(), s.V[layer].numpy().copy()
        rc = oracle.block_write(Ko, Vo, s.pool.block_start, lo, blocks, kn[layer].double().numpy(),
                                vn[layer].double().numpy(), theta, oracle.HWO_FP8, k_scale=ks,
                                v_scale=vs)
        assert rc == 0
        K8, V8 = s.pool.load_layer(layer)
        Kg = K8.cpu().double().numpy() * ks[:, None, None]
        Vg = V8.cpu().double().numpy() * vs[:, None, None]
        assert np.array_equal(Vg, Vo) and np.array_equal(Kg, Ko)
