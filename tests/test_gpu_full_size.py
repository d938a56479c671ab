"""Full-size parity: every output row at the shapes the benchmark times, against
the fp64 oracle (run on the host's threads: its C calls release the GIL).

  * the 64-layer QwQ-32B-shaped step (4 workers, 40 q / 8 kv heads, D 128,
    16K shared history): all 160 rows of layers 0 and 63, bf16 and FP8 pools,
    through hw_attn_decode and through hw_attn_plan + hw_attn_run;
  * one cell per worker count of the workers x context grid (1/2/4 workers at
    16K/8K/1K tokens): all rows;
  * the 36-layer generation loop (Qwen3-8B heads, 4 workers, 32K shared
    history, a token written per worker and layer every step, one block append)
    at its stated size: the oracle replays every write and the append layer by
    layer; all rows of three layers before and after the append, and every
    layer's K/V bit-exact at the end.

Bar: bf16 inputs within 5e-3 max-abs and 1e-2 relative L2 of the oracle
(FP8 pools: of attention over code * scale)."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import workloads
from hw_harness import assert_close

pytestmark = pytest.mark.gpu

FP8 = torch.float8_e4m3fn
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
APIS = ["decode", "plan_run"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _tuning(request):
    _say(f"[case] {request.node.name}")
    hw.hw_set_tuning(hw.PATH_AUTO, 0, 0)
    yield
    hw.hw_set_tuning(hw.PATH_AUTO, 0)


def oracle_layer(q, K, V, tb, to, lens, starts, theta, G, pairs=None):
    """Rows (worker, q-head) of one layer with the fp64 oracle on THREADS threads.
    q [W][Hq][D]; K, V float64 [Hkv][num_slots][D]; tables from the oracle."""
    qd = q.double().numpy() if isinstance(q, torch.Tensor) else np.asarray(q, np.float64)
    qd = np.ascontiguousarray(qd)
    W, Hq, D = qd.shape
    out = np.full((W, Hq, D), np.nan)
    lens = np.ascontiguousarray(lens, np.int32)
    starts = np.ascontiguousarray(starts, np.int64)
    pairs = pairs if pairs is not None else [(w, h) for w in range(W) for h in range(Hq)]

    def one(p):
        w, h = p
        r, rc = oracle.attn_one(oracle.FORM_METHOD, qd[w, h], K[h // G], V[h // G], tb[w], to[w],
                                lens, starts, theta)
        assert rc == 0
        out[w, h] = r

    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(one, pairs))
    return out


class Attend:
    """One pool's attention calls through either entry point."""

    def __init__(self, pool, wl):
        self.pool, self.wl = pool, wl
        self.tables = torch.zeros(wl.W, wl.W + 1, 2, dtype=torch.int32, device="cuda")
        self.ne = torch.zeros(wl.W, dtype=torch.int32, device="cuda")
        hw.hw_build_combined_tables(pool, wl.W, wl.common_block, wl.worker_block, self.tables,
                                    self.ne)
        self.ws = hw.alloc_workspace(pool, wl.W, wl.Hq)
        self.plan = hw.alloc_plan(pool, wl.W, wl.Hq)

    def __call__(self, layer, q, api):
        wl = self.wl
        out = torch.full((wl.W, wl.Hq, wl.D), float("nan"), device="cuda")
        if api == "plan_run":
            hw.hw_attn_plan(self.pool, self.tables, self.ne, self.plan, wl.Hq)
            hw.hw_attn_run(self.pool, layer, q.cuda(), self.plan, wl.theta, out, self.ws)
        else:
            hw.hw_attn_decode(self.pool, layer, q.cuda(), self.tables, self.ne, wl.theta, out,
                              self.ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def _step_pool(wl, keep_layers):
    """The step's pool, drawn on the GPU; host float64 K/V (FP8: code * scale) and q
    of `keep_layers`."""
    slots = sum(wl.caps)
    starts = list(np.cumsum([0] + list(wl.caps[:-1])))
    draws, host, ks_all, vs_all = [], {}, [], []
    for layer in range(wl.layers):
        if wl.fp8:
            K, V, ks, vs = workloads.make_kv_fp8(wl, layer, slots, device="cuda",
                                                 block_start=starts)
            ks_all.append(ks)
            vs_all.append(vs)
        else:
            K, V = workloads.make_kv(wl, layer, slots, device="cuda")
        if layer in keep_layers:
            Kd, Vd = K.cpu().double(), V.cpu().double()
            if wl.fp8:
                Kd *= ks.double()[:, None, None]
                Vd *= vs.double()[:, None, None]
            host[layer] = (Kd.numpy(), Vd.numpy(), workloads.make_q(wl, layer, device="cuda").cpu())
        draws.append((K, V))
    pool = hw.Pool(wl.layers, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype,
                   k_scale=torch.stack(ks_all) if wl.fp8 else None,
                   v_scale=torch.stack(vs_all) if wl.fp8 else None)
    assert pool.block_start == starts
    pool.set_lengths(wl.lens)
    for layer, (K, V) in enumerate(draws):
        pool.store_layer(layer, K, V)
    del draws
    torch.cuda.synchronize()
    return pool, host


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_qwq_step_every_row(fp8):
    wl = workloads.qwq_step()
    if fp8:
        wl = workloads.with_fp8(wl)
    full, sampled = (0, 63), 31
    pool, host = _step_pool(wl, full + (sampled,))
    att = Attend(pool, wl)
    tb, to, _ = oracle.build_combined_tables(wl.common_block, wl.worker_block, wl.lens)
    bar = FP8 if fp8 else torch.bfloat16
    for layer in full:
        K, V, q = host[layer]
        ref = oracle_layer(q, K, V, tb, to, wl.lens, pool.block_start, wl.theta, wl.G)
        for api in APIS:
            got = att(layer, q, api)
            ma, rl = assert_close(got, ref, bar, f"layer {layer} {api}")
            _say(f"  layer {layer} {api}: all {wl.W * wl.Hq} rows, max_abs {ma:.2e} "
                 f"rel_l2 {rl:.2e}")
    K, V, q = host[sampled]
    rng = np.random.default_rng(0)
    pairs = [(int(rng.integers(wl.W)), int(rng.integers(wl.Hq))) for _ in range(8)]
    ref = oracle_layer(q, K, V, tb, to, wl.lens, pool.block_start, wl.theta, wl.G, pairs)
    got = att(sampled, q, "decode")
    for w, h in pairs:
        assert_close(got[w, h], ref[w, h], bar, f"layer {sampled} row ({w}, {h})")
    assert hw.hw_pool_status(pool) == 0


@pytest.mark.parametrize("C,W", [(16384, 1), (8192, 2), (1024, 4)])
def test_grid_cell_every_row(C, W):
    wl = workloads.sweep(C, W)
    pool, host = _step_pool(wl, (0,))
    att = Attend(pool, wl)
    tb, to, _ = oracle.build_combined_tables(wl.common_block, wl.worker_block, wl.lens)
    K, V, q = host[0]
    ref = oracle_layer(q, K, V, tb, to, wl.lens, pool.block_start, wl.theta, wl.G)
    for api in APIS:
        ma, rl = assert_close(att(0, q, api), ref, torch.bfloat16, f"C {C} W {W} {api}")
        _say(f"  C={C} W={W} {api}: max_abs {ma:.2e} rel_l2 {rl:.2e}")
    assert hw.hw_pool_status(pool) == 0


def test_generation_loop_at_stated_size():
    steps, L = 72, 36
    wl = workloads.qwen3_loop(layers=L, steps=steps)
    assert wl.lens[0] >= 32768
    sched = workloads.loop_appends(wl, steps)
    assert len(sched) >= 1
    W, G = wl.W, wl.G
    pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    S = pool.num_slots
    starts = np.asarray(pool.block_start, np.int64)
    pool.set_lengths(wl.lens)
    for layer in range(L):
        K, V = workloads.make_kv(wl, layer, S, device="cuda")
        pool.store_layer(layer, K, V)
        del K, V
    q = [workloads.make_q(wl, layer, device="cuda") for layer in range(L)]
    gk = torch.Generator().manual_seed(17)
    kn = [torch.randn(W, wl.Hkv, wl.D, generator=gk) for _ in range(L)]
    vn = [torch.randn(W, wl.Hkv, wl.D, generator=gk) for _ in range(L)]
    kn_d = [k.cuda() for k in kn]
    vn_d = [v.cuda() for v in vn]
    tables = torch.zeros(W, W + 1, 2, dtype=torch.int32, device="cuda")
    ne = torch.zeros(W, dtype=torch.int32, device="cuda")
    ws = hw.alloc_workspace(pool, W, wl.Hq)
    out = torch.zeros(L, W, wl.Hq, wl.D, device="cuda")
    first_append = min(sched)
    check_steps = (first_append - 1, steps - 1)   # before the append, and the last step
    check_layers = (0, 17, 35)
    saved = {}
    lens = np.array(wl.lens, np.int32)
    for step in range(steps):
        lens[1:] += 1
        hw.hw_block_advance(pool, wl.worker_block)
        hw.hw_build_combined_tables(pool, W, wl.common_block, wl.worker_block, tables, ne)
        for layer in range(L):
            hw.hw_block_write(pool, layer, wl.worker_block, kn_d[layer], vn_d[layer], wl.theta)
            hw.hw_attn_decode(pool, layer, q[layer], tables, ne, wl.theta, out[layer], ws)
        if step in check_steps:
            saved[step] = out[list(check_layers)].cpu().numpy()
        if step in sched:
            b = wl.worker_block[sched[step]]
            hw.hw_block_append(pool, b, wl.common_block, wl.theta)
            hw.hw_block_reset(pool, b)
            lens[0] += lens[b]
            lens[b] = 0
    torch.cuda.synchronize()
    assert pool.block_len.cpu().tolist() == lens.tolist()
    assert hw.hw_pool_status(pool) == 0
    _say(f"  loop: {steps} steps x {L} layers, {len(sched)} append(s), common "
         f"{wl.lens[0]} -> {lens[0]} tokens")

    # the oracle replays the loop one layer at a time from the same initial draws
    worst = 0.0
    for layer in range(L):
        K, V = workloads.make_kv(wl, layer, S, device="cuda")
        Kh = K.cpu().double().numpy()
        Vh = V.cpu().double().numpy()
        del K, V
        lr = np.array(wl.lens, np.int32)
        for step in range(steps):
            lr[1:] += 1
            rc = oracle.block_write(Kh, Vh, starts, lr, wl.worker_block, kn[layer].double().numpy(),
                                    vn[layer].double().numpy(), wl.theta, oracle.HWO_BF16)
            assert rc == 0
            if layer in check_layers and step in check_steps:
                tb, to, _ = oracle.build_combined_tables(wl.common_block, wl.worker_block, lr)
                ref = oracle_layer(q[layer].cpu(), Kh, Vh, tb, to, lr, starts, wl.theta, G)
                got = saved[step][check_layers.index(layer)]
                ma, _ = assert_close(got, ref, torch.bfloat16, f"loop step {step} layer {layer}")
                worst = max(worst, ma)
            if step in sched:
                rc = oracle.block_append(Kh[None], Vh[None], starts, pool.block_cap, lr,
                                         wl.worker_block[sched[step]], wl.common_block, wl.theta,
                                         oracle.HWO_BF16)
                assert rc == 0
        assert lr.tolist() == lens.tolist()
        Kg, Vg = pool.load_layer(layer)
        assert np.array_equal(Kg.cpu().double().numpy(), Kh), f"layer {layer} K"
        assert np.array_equal(Vg.cpu().double().numpy(), Vh), f"layer {layer} V"
    _say(f"  loop: all {L} layers' K/V bit-exact; rows of layers {check_layers} at steps "
         f"{check_steps}: worst max_abs {worst:.2e}")
