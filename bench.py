#!/usr/bin/env python3
"""Benchmark: Hogwild! concurrent-attention decode step on one MI355X.

Workload (synthetic, seeded): QwQ-32B-shaped full decode step — 64 layers,
4 workers, 40 query / 8 KV heads, head_dim 128, bf16 KV pool, RoPE theta 1e6,
common cache 16384 tokens, one in-progress block per worker of U[256, 1024]
tokens (drawn once from the seed).  K, V ~ N(0,1) + a per-channel offset
N(0, 0.5); q ~ N(0,1).

One step = one pass of the whole path over the resident inputs:
  build the combined-layout tables on the device from the block lengths,
  64 x concurrent-attention decode (rotation prologue, split-K loop, merge),
  append one worker's finished block into the common history (round robin),
then the harness restores the block lengths so every step sees the same
workload (the appended tokens sit past the restored common length).
The step is captured once in a HIP graph and replayed.

Metric: worker-tokens/s per layer = W * layers / step time.  The roofline
object reports the decode call's algorithmic HBM bytes divided by its average
duration (HIP events on the launch stream around the 64 back-to-back calls of
a step, eager replay) against MI355X's 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_qwq32b_step_hbm_traffic.md")


# the sources a decode call's kernels and launch geometry come from (the
# traffic summary stays valid while these are unchanged)
DECODE_SOURCES = ("hw_api.hip", "hw_decode.hip", "hw_fused.hip", "hw_internal.h", "hw_kernels.h",
                  "hw_plan.hip")


def kernel_source_sha256() -> str:
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_attention_shared_hw_amd", "csrc", "*"))):
        if os.path.basename(f) in DECODE_SOURCES:
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when the kernel sources changed since the counters were taken."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as fh:
            for line in fh:
                if ":" in line:
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_sha256") != kernel_source_sha256():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--path", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--units", type=int, default=0, help="split-K units per kv head (0 = auto)")
    ap.add_argument("--balance", action="store_true",
                    help="balanced tile order (tiles after each wave's first from a per-head "
                         "counter) instead of fixed tile ranges per work unit")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=48,
                    help="(worker, q-head) pairs of one layer timed on one CPU thread")
    ap.add_argument("--kernel-timing-steps", type=int, default=10)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--config", choices=["step", "sweep", "loop", "cell", "chunk"],
                    default="step",
                    help="step: the headline 64-layer step (default); sweep: context x workers "
                         "grid, per-layer time on both paths; loop: 36-layer generation loop "
                         "with appends; cell: one grid point (--context, --workers); chunk: "
                         "one 80-row chunk call")
    ap.add_argument("--context", type=int, default=16384, help="cell: visible context tokens")
    ap.add_argument("--workers", type=int, default=4, help="cell: workers")
    ap.add_argument("--loop-steps", type=int, default=2048)
    ap.add_argument("--api", choices=["decode", "plan_run"], default="decode",
                    help="decode: hw_attn_decode per layer (plan built in-kernel, the default); "
                         "plan_run: hw_attn_plan once per step + hw_attn_run per layer")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline step only: no plan_run A/B, sweep, loop or chunk objects")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 E4M3 pool variant of the step (reported as fp8_step)")
    return ap.parse_args()


def _graph_layers_us(hw, torch, pool, wl, q, reps=20, api="decode", chunk=1):
    """Per-layer time of one decode (or chunk) call over every layer of `pool`, in
    graph replay."""
    W, L = wl.W, pool.num_layers
    out = torch.zeros(L, W, wl.Hq, wl.D, device="cuda")
    tables = torch.zeros(W, W + 1, 2, dtype=torch.int32, device="cuda")
    ne = torch.zeros(W, dtype=torch.int32, device="cuda")
    ws = hw.alloc_workspace(pool, W * chunk, wl.Hq)
    plan = hw.alloc_plan(pool, W, wl.Hq, chunk=chunk)
    if chunk > 1:
        out = torch.zeros(L, W, chunk, wl.Hq, wl.D, device="cuda")
    # the inputs were written on the default stream: complete them before the
    # side stream reads them, and build the tables on the side stream itself
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    hw.hw_build_combined_tables(pool, W, wl.common_block, wl.worker_block, tables, ne, st)

    def body():
        if api == "plan_run":
            hw.hw_attn_plan(pool, tables, ne, plan, wl.Hq, chunk=chunk, stream=st)
            for layer in range(L):
                hw.hw_attn_run(pool, layer, q[layer], plan, wl.theta, out[layer], ws, st)
        elif chunk > 1:
            for layer in range(L):
                hw.hw_attn_chunk(pool, layer, q[layer], tables, ne, wl.theta, out[layer], ws, st)
        else:
            for layer in range(L):
                hw.hw_attn_decode(pool, layer, q[layer], tables, ne, wl.theta, out[layer], ws, st)

    with torch.cuda.stream(st):
        body()
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            body()
        g.replay()
        st.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        st.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * L)


def run_sweep(args, paths=("mfma", "valu"), reps=20):
    """Context x workers grid (40 q / 8 kv heads, D 128, bf16): per-layer time of
    one decode call.  The K/V bytes do not depend on W, so with the reads shared
    by all workers the time stays flat in W.  Each point cycles through enough
    layers (distinct K/V) that the 256 MB Infinity Cache cannot hold them."""
    import torch

    from decode_attention_shared_hw_amd import hogwild_attn as hw
    from decode_attention_shared_hw_amd import workloads

    points = []
    for path_name, path in (("mfma", hw.PATH_MFMA), ("valu", hw.PATH_VALU)):
        if path_name not in paths:
            continue
        hw.hw_set_tuning(path, args.units)
        for C in (1024, 8192, 16384):
            for W in (1, 2, 4):
                wl = workloads.sweep(C, W)
                L = min(256, max(8, -(-2 * 256 * 2**20 // wl.kv_bytes_per_layer())))
                wl.layers = L
                pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
                pool.set_lengths(wl.lens)
                for layer in range(L):
                    K, V = workloads.make_kv(wl, layer, pool.num_slots, device="cuda")
                    pool.store_layer(layer, K, V)
                    del K, V
                q = torch.stack([workloads.make_q(wl, layer, device="cuda") for layer in range(L)])
                us = _graph_layers_us(hw, torch, pool, wl, q, reps=reps)
                b = wl.algorithmic_bytes_per_layer()
                points.append({"path": path_name, "context": C, "workers": W, "layers_cycled": L,
                               "us_per_layer": us, "worker_tokens_per_s_per_layer": W / (us * 1e-6),
                               "algorithmic_bytes": b, "achieved_gbs": b / (us * 1e-6) / 1e9,
                               "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               "status": hw.hw_pool_status(pool)})
                print(f"# {path_name} C={C} W={W}: {us:.2f} us/layer", file=sys.stderr, flush=True)
                del pool, q
                torch.cuda.empty_cache()
    hw.hw_set_tuning(hw.PATH_AUTO, 0)
    return {"config": "sweep", "unit": "us per layer (graph replay, hw_attn_decode)",
            "data": "synthetic, seeded", "points": points}


def calibrate_copy(torch, mib):
    """One plain device copy of `mib` MiB (bytes read = bytes written = mib MiB):
    its HBM counters scale the decode kernels' counters in the same run."""
    if mib <= 0:
        return
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def gpu_clocks(torch):
    """The GPU's DPM clock levels from sysfs (read-only files; no tool is run),
    matched to device 0 by its PCI address: {"pci", "sclk", "mclk"}, each
    clock a list of levels with the current one marked '*', or None."""
    import glob

    try:
        p = torch.cuda.get_device_properties(0)
        slot = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        for dev in glob.glob("/sys/class/drm/card*/device"):
            with open(os.path.join(dev, "uevent")) as f:
                if f"PCI_SLOT_NAME={slot}" not in f.read().split():
                    continue
            res = {"pci": slot}
            for k in ("sclk", "mclk"):
                with open(os.path.join(dev, f"pp_dpm_{k}")) as f:
                    res[k] = [ln.strip() for ln in f if ln.strip()]
            return res
    except Exception:  # metadata only: a host without these files reports None
        pass
    return None


def copy_bandwidth(torch, mib=1024, reps=20):
    """Device-to-device copy rate of this GPU in the same run (read + written
    bytes per second, GB/s): a practical ceiling next to the 8 TB/s peak.  One
    `mib` MiB buffer copied `reps` times between HIP events on one stream."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for _ in range(3):
            dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(st)
        st.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / sec / 1e9


def run_cell(args, reps=10):
    """One point of the workers x context grid (40 q / 8 kv heads, D 128, bf16):
    per-layer time of hw_attn_decode in graph replay, cycling layers of distinct K/V."""
    import torch

    from decode_attention_shared_hw_amd import hogwild_attn as hw
    from decode_attention_shared_hw_amd import workloads

    wl = workloads.sweep(args.context, args.workers)
    L = min(256, max(8, -(-2 * 256 * 2**20 // wl.kv_bytes_per_layer())))
    wl.layers = L
    pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    pool.set_lengths(wl.lens)
    for layer in range(L):
        K, V = workloads.make_kv(wl, layer, pool.num_slots, device="cuda")
        pool.store_layer(layer, K, V)
        del K, V
    q = torch.stack([workloads.make_q(wl, layer, device="cuda") for layer in range(L)])
    us = _graph_layers_us(hw, torch, pool, wl, q, reps=reps)
    b = wl.algorithmic_bytes_per_layer()
    res = {"config": "cell", "workload": wl.name, "context": args.context,
           "workers": args.workers, "layers_cycled": L, "us_per_layer": us,
           "algorithmic_bytes": b, "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "status": hw.hw_pool_status(pool)}
    del pool, q
    torch.cuda.empty_cache()
    return res


def run_chunk(args, chunk=4, reps=10):
    """One chunk call (chunked prefill: each worker's last `chunk` tokens as
    queries, causal inside the chunk) at the QwQ heads, 4 workers, 16K context:
    4 * chunk * 5 = 80 stacked rows per kv head on the MFMA path.  Per-layer time
    in graph replay, cycling layers of distinct K/V."""
    import torch

    from decode_attention_shared_hw_amd import hogwild_attn as hw
    from decode_attention_shared_hw_amd import workloads

    wl = workloads.sweep(16384, 4)
    L = max(8, -(-2 * 256 * 2**20 // wl.kv_bytes_per_layer()))
    wl.layers = L
    pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    pool.set_lengths(wl.lens)
    for layer in range(L):
        K, V = workloads.make_kv(wl, layer, pool.num_slots, device="cuda")
        pool.store_layer(layer, K, V)
        del K, V
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 21)
    q = torch.randn(L, wl.W, chunk, wl.Hq, wl.D, generator=gen, device="cuda").to(wl.q_dtype)
    # the plan once per step (every layer's call has the same views), then one
    # run per layer
    us = _graph_layers_us(hw, torch, pool, wl, q, reps=reps, api="plan_run", chunk=chunk)
    b = wl.kv_bytes_per_layer() + wl.W * chunk * wl.Hq * wl.D * (q.element_size() + 4)
    res = {"workload": f"chunk_16384_4w_x{chunk}", "rows_per_kv_head": wl.W * chunk * wl.G,
           "api": "hw_attn_plan once + hw_attn_run per layer",
           "kernel": "run_mfma<128,5,bf16> + merge_kernel<128>", "us_per_layer": us,
           "algorithmic_bytes": b, "achieved_gbs": b / (us * 1e-6) / 1e9,
           "frac_of_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "status": hw.hw_pool_status(pool)}
    del pool, q
    torch.cuda.empty_cache()
    return res


def run_loop(args):
    """Generation loop (Qwen3-8B heads: 36 layers, 32 q / 8 kv heads, D 128, bf16,
    4 workers, common cache from 32768 tokens), device-resident end to end.
    One step: every worker's block reserves a slot for the new token
    (hw_block_advance), the tables are rebuilt on the device, and each layer
    writes the new tokens' K/V (hw_block_write; synthetic, seeded) and decodes.
    The step is captured once as a HIP graph and replayed; every 64 steps one
    worker's block is appended into the common block and reset (shuffled round
    robin), launched between replays.  Timed end to end with HIP events."""
    import numpy as np
    import torch

    from decode_attention_shared_hw_amd import hogwild_attn as hw
    from decode_attention_shared_hw_amd import workloads

    steps = args.loop_steps
    wl = workloads.qwen3_loop(steps=steps)
    sched = workloads.loop_appends(wl, steps)
    L, W = wl.layers, wl.W
    pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    pool.set_lengths(wl.lens)
    for layer in range(L):
        K, V = workloads.make_kv(wl, layer, pool.num_slots, device="cuda")
        pool.store_layer(layer, K, V)
        del K, V
    q = torch.stack([workloads.make_q(wl, layer, device="cuda") for layer in range(L)])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 11)
    k_new = torch.randn(L, W, wl.Hkv, wl.D, generator=gen, device="cuda")
    v_new = torch.randn(L, W, wl.Hkv, wl.D, generator=gen, device="cuda")
    out = torch.zeros(L, W, wl.Hq, wl.D, device="cuda")
    tables = torch.zeros(W, W + 1, 2, dtype=torch.int32, device="cuda")
    ne = torch.zeros(W, dtype=torch.int32, device="cuda")
    ws = hw.alloc_workspace(pool, W, wl.Hq)
    st = torch.cuda.Stream()

    def step_body():
        hw.hw_block_advance(pool, wl.worker_block, st)
        hw.hw_build_combined_tables(pool, W, wl.common_block, wl.worker_block, tables, ne, st)
        for layer in range(L):
            hw.hw_block_write(pool, layer, wl.worker_block, k_new[layer], v_new[layer], wl.theta, st)
            hw.hw_attn_decode(pool, layer, q[layer], tables, ne, wl.theta, out[layer], ws, st)

    lens = np.array(wl.lens, np.int64)
    dec_bytes = 0
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            step_body()
        st.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for step in range(steps):
            graph.replay()
            lens[1:] += 1
            dec_bytes += L * (int(lens.sum()) * wl.Hkv * wl.D * 2 * 2 + W * wl.Hq * wl.D * 6)
            if step in sched:
                b = wl.worker_block[sched[step]]
                hw.hw_block_append(pool, b, wl.common_block, wl.theta, st)
                hw.hw_block_reset(pool, b, st)
                lens[0] += lens[b]
                lens[b] = 0
        e1.record(st)
        st.synchronize()
    ms = e0.elapsed_time(e1)
    step_us = ms * 1e3 / steps
    res = {"config": "loop", "workload": wl.name, "steps": steps, "layers": L, "workers": W,
           "appends": len(sched), "common_tokens": [int(wl.lens[0]), int(lens[0])],
           "step": "advance + tables + 36 x (token write + decode), HIP graph; appends between",
           "us_per_step": step_us, "us_per_layer": step_us / L,
           "worker_tokens_per_s_per_layer": W * L / (step_us * 1e-6),
           "decode_achieved_gbs": dec_bytes / (ms * 1e-3) / 1e9,
           "status": hw.hw_pool_status(pool),
           "final_lengths": pool.block_len.cpu().tolist(), "expected_lengths": lens.tolist()}
    res["lengths_ok"] = res["final_lengths"] == res["expected_lengths"]
    del pool, q, k_new, v_new, out, ws
    torch.cuda.empty_cache()
    return res


def host_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_threads() -> int:
    """Threads of the CPU baseline: the host CPUs this process may use, at most 16
    (the host share of one GPU on the machines this runs on)."""
    return max(1, min(host_cpus(), 16))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_layer_seconds(wl, K, V, q, starts, threads):
    """Wall time of every (worker, q-head) row of one layer with the fp64 oracle
    (definition form) on `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    tb, to, _ = oracle.build_combined_tables(wl.common_block, wl.worker_block, wl.lens)
    lens = np.asarray(wl.lens, np.int32)
    starts = np.asarray(starts, np.int64)
    Kd, Vd, qd = K.double().numpy(), V.double().numpy(), q.double().numpy()

    def one(pair):
        w, h = pair
        _, rc = oracle.attn_one(oracle.FORM_DEFINITION, qd[w, h], Kd[h // wl.G], Vd[h // wl.G],
                                tb[w], to[w], lens, starts, wl.theta)
        assert rc == 0

    pairs = [(w, h) for w in range(wl.W) for h in range(wl.Hq)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, pairs))
    return time.perf_counter() - t0


def cpu_breadth(threads):
    """The oracle on one layer of every other configuration (all rows): the tiny
    fp32 layer, the QwQ single layer, the workers x context grid and a layer of
    the generation loop at its initial 32K history."""
    import numpy as np

    from decode_attention_shared_hw_amd import workloads

    cases = [("tiny_fp32_2w", workloads.tiny()), ("qwq32b_layer_bf16_2w", workloads.qwq_layer())]
    cases += [(f"sweep_{C}_{W}w", workloads.sweep(C, W)) for C in (1024, 8192, 16384)
              for W in (1, 2, 4)]
    cases += [("qwen3_8b_loop_bf16_4w (layer 0, first step)", workloads.qwen3_loop())]
    out = []
    for name, wl in cases:
        slots = max(sum(wl.caps), 32)
        starts = np.cumsum([0] + list(wl.caps[:-1]))
        K, V = workloads.make_kv(wl, 0, slots)
        q = workloads.make_q(wl, 0)
        sec = _oracle_layer_seconds(wl, K, V, q, starts, threads)
        b = wl.algorithmic_bytes_per_layer()
        out.append({"workload": name, "rows": wl.W * wl.Hq, "tokens": wl.tokens,
                    "seconds_per_layer": sec, "worker_tokens_per_s_per_layer": wl.W / sec,
                    "equivalent_gbs": b / sec / 1e9})
    return out


def cpu_baseline(wl, pool_block_start, K, V, q, pairs):
    """Time the fp64 oracle (definition form) on layer 0: every (worker, q-head)
    pair on all host threads (the oracle's C calls release the GIL), and a
    sample of `pairs` pairs on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    tb, to, ne = oracle.build_combined_tables(wl.common_block, wl.worker_block, wl.lens)
    lens = np.asarray(wl.lens, np.int32)
    starts = np.asarray(pool_block_start, np.int64)
    Kd = K.double().numpy()
    Vd = V.double().numpy()
    qd = q.double().numpy()

    def one(pair):
        w, h = pair
        g = h // wl.G
        _, rc = oracle.attn_one(oracle.FORM_DEFINITION, qd[w, h], Kd[g], Vd[g], tb[w], to[w],
                                lens, starts, wl.theta)
        assert rc == 0

    all_pairs = [(w, h) for w in range(wl.W) for h in range(wl.Hq)]
    step = max(1, len(all_pairs) // pairs)
    sample = all_pairs[::step][:pairs]
    t0 = time.perf_counter()
    for pair in sample:
        one(pair)
    dt1 = time.perf_counter() - t0
    layer_s1 = dt1 / len(sample) * len(all_pairs)
    n = cpu_threads()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, all_pairs))
    layer_s = time.perf_counter() - t0
    b = wl.algorithmic_bytes_per_layer()
    return {
        "value": wl.W / layer_s, "unit": "worker-tokens/s per layer", "cores": n,
        "kind": "oracle",
        "sample": f"fp64 definition form, all {len(all_pairs)} (worker, q-head) pairs of layer 0 "
                  f"({wl.tokens} tokens each) on {n} threads in {layer_s:.1f} s; single thread: "
                  f"{len(sample)} pairs in {dt1:.1f} s, scaled to the layer",
        "seconds_per_layer": layer_s,
        "seconds_per_step": layer_s * wl.layers,
        "equivalent_gbs": b / layer_s / 1e9,
        "value_1_thread": wl.W / layer_s1,
        "cpu_model": cpu_model(), "host_cpus": host_cpus(),
        "threads_note": "at most 16 threads: the host share of one GPU",
        "other_configs": cpu_breadth(n),
    }


def make_step_pool(hw, torch, workloads, wl, keep_layer0):
    """Device pool of every layer of `wl` (bf16 or FP8 codes with scales), its
    queries, output and tables; the host copy of layer 0 when asked."""
    import numpy as np

    L = wl.layers
    host_layer0 = None
    draws, ks_all, vs_all = [], [], []
    slots = sum(wl.caps)
    starts = [int(x) for x in np.cumsum([0] + list(wl.caps[:-1]))]
    pool = None
    if not wl.fp8:
        pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype)
    for layer in range(L):
        if wl.fp8:
            K, V, ks, vs = workloads.make_kv_fp8(wl, layer, slots, device="cuda", block_start=starts)
            draws.append((K, V))
            ks_all.append(ks)
            vs_all.append(vs)
        else:
            K, V = workloads.make_kv(wl, layer, pool.num_slots, device="cuda")
            pool.store_layer(layer, K, V)
            if layer == 0 and keep_layer0:
                host_layer0 = (K.cpu(), V.cpu())
            del K, V
    if wl.fp8:
        pool = hw.Pool(L, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype, k_scale=torch.stack(ks_all),
                       v_scale=torch.stack(vs_all))
        for layer, (K, V) in enumerate(draws):
            pool.store_layer(layer, K, V)
        del draws
    pool.set_lengths(wl.lens)
    q = torch.stack([workloads.make_q(wl, layer, device="cuda") for layer in range(L)])
    return pool, q, host_layer0


def time_step(args, hw, torch, np, wl, pool, q, api="decode"):
    """Graph (or eager) replay of the step, then per-launch HIP-event durations of
    the decode calls and the append in an eager replay behind a GPU spin."""
    L, W = wl.layers, wl.W
    saved_lens = pool.block_len.clone()
    out = torch.zeros(L, W, wl.Hq, wl.D, dtype=torch.float32, device="cuda")
    tables = torch.zeros(W, W + 1, 2, dtype=torch.int32, device="cuda")
    ne = torch.zeros(W, dtype=torch.int32, device="cuda")
    ws = hw.alloc_workspace(pool, W, wl.Hq)
    plan = hw.alloc_plan(pool, W, wl.Hq)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    counter = [0]

    def step(events=None):
        k = counter[0]
        counter[0] += 1
        hw.hw_build_combined_tables(pool, W, wl.common_block, wl.worker_block, tables, ne, stream)
        if api == "plan_run":
            hw.hw_attn_plan(pool, tables, ne, plan, wl.Hq, stream=stream)
        if events is not None:
            events["dec"][0].record(stream)
        for layer in range(L):
            if api == "plan_run":
                hw.hw_attn_run(pool, layer, q[layer], plan, wl.theta, out[layer], ws, stream)
            else:
                hw.hw_attn_decode(pool, layer, q[layer], tables, ne, wl.theta, out[layer], ws,
                                  stream)
        if events is not None:
            events["dec"][1].record(stream)
        src = wl.worker_block[k % W]
        if events is not None:
            events["app"][0].record(stream)
        hw.hw_block_append(pool, src, wl.common_block, wl.theta, stream)
        if events is not None:
            events["app"][1].record(stream)
        # harness: restore the lengths (an elementwise kernel, graph-safe)
        torch.add(saved_lens, 0, out=pool.block_len)

    use_graph = not args.no_graph
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        graph = None
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step()
            for _ in range(2):
                graph.replay()
            stream.synchronize()

        # ---- timed region: K steps
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            if use_graph:
                graph.replay()
            else:
                step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)

        # ---- per-launch durations: HIP events on the launch stream around the
        # step's L back-to-back decode calls (per call: the span / L, so the
        # events do not sit between the launches they time) and around the
        # append; a GPU spin first lets the host enqueue ahead
        dec_us, app_us = [], []
        for _ in range(args.kernel_timing_steps):
            evs = {"dec": (torch.cuda.Event(enable_timing=True),
                           torch.cuda.Event(enable_timing=True)),
                   "app": (torch.cuda.Event(enable_timing=True),
                           torch.cuda.Event(enable_timing=True))}
            torch.cuda._sleep(20_000_000)
            step(evs)
            stream.synchronize()
            dec_us.append(evs["dec"][0].elapsed_time(evs["dec"][1]) * 1e3 / L)
            app_us.append(evs["app"][0].elapsed_time(evs["app"][1]) * 1e3)
    torch.cuda.synchronize()
    return {"ms_per_step": gpu_ms / args.steps, "dec_us": dec_us, "app_us": app_us, "wall": wall,
            "flags": hw.hw_pool_status(pool), "graph": use_graph}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the decode path runs on one GPU; --gpus must be 1 "
              "(sharding the kv heads over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decode_attention_shared_hw_amd import hogwild_attn as hw
    from decode_attention_shared_hw_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hw.lib()  # fail loudly if the library is missing
    if args.config == "sweep":
        print(json.dumps(run_sweep(args)), flush=True)
        return
    if args.config == "loop":
        print(json.dumps(run_loop(args)), flush=True)
        return
    if args.config == "cell":
        res = run_cell(args)
        calibrate_copy(torch, args.calibrate_copy)
        print(json.dumps(res), flush=True)
        return
    if args.config == "chunk":
        print(json.dumps(run_chunk(args)), flush=True)
        return
    path = {"auto": hw.PATH_AUTO, "valu": hw.PATH_VALU, "mfma": hw.PATH_MFMA}[args.path]
    hw.hw_set_tuning(path, args.units, 1 if args.balance else 0)

    wl = workloads.qwq_step(layers=args.layers)
    L, W = wl.layers, wl.W
    pool, q, host_layer0 = make_step_pool(hw, torch, workloads, wl, not args.no_cpu_baseline)
    t = time_step(args, hw, torch, np, wl, pool, q, api=args.api)
    calibrate_copy(torch, args.calibrate_copy)
    copy_gbs = copy_bandwidth(torch)

    ms_per_step = t["ms_per_step"]
    step_s = ms_per_step / 1e3
    value = W * L / step_s  # worker-tokens/s per layer
    dec_us = t["dec_us"]
    dec_avg = float(np.mean(dec_us))
    bytes_per_launch = wl.algorithmic_bytes_per_layer()
    achieved = bytes_per_launch / (dec_avg * 1e-6) / 1e9
    use_graph = t["graph"]
    result = {
        "metric": "worker-tokens/s per layer + achieved HBM GB/s (% of peak), 4 workers, 16K",
        "value": value,
        "unit": "worker-tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q; K,V N(0,1) + per-channel N(0,0.5) offset)",
        "config": {**workloads.summary(wl), "parallelism": "single GPU", "api": args.api,
                   "step": ("tables + " + ("plan + " if args.api == "plan_run" else "")
                            + "64 x decode + 1 block append ("
                            + ("graph replay)" if use_graph else "eager)"))},
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic() if path != hw.PATH_VALU else None,
            "kernel": ("decode call = run_valu<bf16,128,10> + merge_kernel<128>"
                       if path == hw.PATH_VALU else
                       "decode call = run_mfma<128,2,bf16> + merge_kernel<128>"
                       if args.api == "plan_run" else
                       "decode call = decode_mfma<128,2,bf16> (fused plan) + merge_kernel<128>"),
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": dec_avg,
            "p10_us": float(np.percentile(dec_us, 10)),
            "p90_us": float(np.percentile(dec_us, 90)),
            "copy_gbs": copy_gbs,
            "frac_of_copy": achieved / copy_gbs,
            "copy_note": "1 GiB device-to-device copy in the same run, read + written bytes",
        },
        "us_per_layer": ms_per_step * 1e3 / L,
        "append_us": float(np.mean(t["app_us"])),
        "wall_s": t["wall"],
        "gpu_clocks": gpu_clocks(torch),
        "device_status": t["flags"],
    }
    if not args.no_extras and path != hw.PATH_VALU:
        # A/B: the same step with the plan computed once per step (hw_attn_plan)
        # and read by every layer's call (hw_attn_run)
        other = "plan_run" if args.api == "decode" else "decode"
        ta = time_step(args, hw, torch, np, wl, pool, q, api=other)
        da = float(np.mean(ta["dec_us"]))
        result["ab_api"] = {"api": other, "us_per_layer": ta["ms_per_step"] * 1e3 / L,
                            "avg_launch_us": da, "frac": bytes_per_launch / (da * 1e-6) / 1e9
                            / HBM_PEAK_GBS, "device_status": ta["flags"]}
    if not args.no_cpu_baseline:
        K0, V0 = host_layer0
        result["cpu_baseline"] = cpu_baseline(wl, pool.block_start, K0, V0, q[0].cpu(),
                                              args.cpu_pairs)
    if not args.no_fp8 and path != hw.PATH_VALU:
        # the same step over an FP8 E4M3 pool (half the K/V bytes; a separate
        # numerics contract: bf16 queries, codes widened exactly)
        del pool, q
        torch.cuda.empty_cache()
        wl8 = workloads.with_fp8(wl)
        pool8, q8, _ = make_step_pool(hw, torch, workloads, wl8, False)
        t8 = time_step(args, hw, torch, np, wl8, pool8, q8, api=args.api)
        d8 = float(np.mean(t8["dec_us"]))
        b8 = wl8.algorithmic_bytes_per_layer()
        result["fp8_step"] = {
            "workload": wl8.name, "kv_dtype": "fp8_e4m3 (per-(layer, kv head) scales)",
            "value": W * L / (t8["ms_per_step"] / 1e3), "unit": "worker-tokens/s per layer",
            "ms_per_step": t8["ms_per_step"], "us_per_layer": t8["ms_per_step"] * 1e3 / L,
            "decode_avg_launch_us": d8, "bytes_per_launch": b8,
            "achieved_gbs": b8 / (d8 * 1e-6) / 1e9,
            "frac_of_peak": b8 / (d8 * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "append_us": float(np.mean(t8["app_us"])), "device_status": t8["flags"],
        }
        del pool8, q8
    if not args.no_extras and path != hw.PATH_VALU:
        pool = q = None  # (the FP8 variant may have released them already)
        torch.cuda.empty_cache()
        hw.hw_set_tuning(hw.PATH_AUTO, args.units)
        result["chunk"] = run_chunk(args)
        sw = run_sweep(args, paths=("mfma",), reps=10)
        result["sweep"] = [{k: p[k] for k in ("context", "workers", "us_per_layer",
                                               "frac_of_peak", "status")} for p in sw["points"]]
        result["loop"] = run_loop(args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
