"""Seeded synthetic workloads shaped like the pages' runs (no method arithmetic here).

Every input is drawn from torch generators seeded per (seed, layer, tensor), so
a workload can be regenerated on the CPU (for the oracle) or on the GPU (for
speed) — the same draw is then copied to the other side, never regenerated.

Shapes (QwQ-32B / Qwen3-8B attention shapes; the pages' throughput table uses
1, 2, 4 workers at 1024 / 8192 / 16384 tokens):
  tiny      2 workers, 4q/2kv heads, D=64, fp32, theta 1e4; common 256, blocks 64+64
  qwq_layer 2 workers, 40q/8kv, D=128, bf16, theta 1e6; common 8192, blocks 512+512
  qwq_step  64 layers, 4 workers, common 16384, worker blocks U[256,1024]
  sweep     4/2/1 workers, total view 1024/8192/16384 (85% common)
  qwen3_loop 36 layers, 32q/8kv, 4 workers, common from 32768, appends every 64 steps
  *_fp8     the same shapes with an FP8 E4M3 K/V pool (bf16 queries)
Values: q ~ N(0,1); K, V ~ N(0,1) + a fixed per-(layer, kv head, channel)
offset ~ N(0, 0.5) for the bf16 shapes (separate offsets for K and V).  FP8
pools hold the same draws as codes of x / scale, with one scale per (layer,
kv head) for K and one for V, amax / 448 over the head's plane (a
calibration choice of the input generator; the pages give none).
"""
from __future__ import annotations

import dataclasses
import numpy as np
import torch

TILE = 32


def round_up(x: int, m: int = TILE) -> int:
    return (int(x) + m - 1) // m * m


@dataclasses.dataclass
class Workload:
    name: str
    W: int
    Hq: int
    Hkv: int
    D: int
    theta: float
    dtype: torch.dtype
    layers: int
    lens: list            # [common, worker 0, ..., worker W-1]
    caps: list            # capacities, multiples of 32
    offset_sigma: float   # std of the per-channel K/V mean offset (0: none)
    seed: int

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def rows(self):
        return self.W * self.G

    @property
    def common_block(self):
        return 0

    @property
    def worker_block(self):
        return list(range(1, self.W + 1))

    @property
    def tokens(self):
        """Unique visible tokens per layer (every worker sees every block)."""
        return int(sum(self.lens))

    @property
    def q_dtype(self):
        """fp32 queries for fp32 pools, bf16 for bf16 and FP8 pools."""
        return torch.float32 if self.dtype == torch.float32 else torch.bfloat16

    @property
    def fp8(self):
        return self.dtype == torch.float8_e4m3fn

    def kv_bytes_per_layer(self):
        return self.tokens * self.Hkv * self.D * 2 * self.dtype.itemsize

    def algorithmic_bytes_per_layer(self):
        """Each visible K/V token read once + q read + out (fp32) written."""
        return self.kv_bytes_per_layer() + self.W * self.Hq * self.D * (self.q_dtype.itemsize + 4)


def tiny(seed: int = 1001) -> Workload:
    lens = [256, 64, 64]
    return Workload("tiny_fp32_2w", 2, 4, 2, 64, 1e4, torch.float32, 1, lens,
                    [round_up(x) for x in lens], 0.0, seed)


def qwq_layer(seed: int = 1002) -> Workload:
    lens = [8192, 512, 512]
    return Workload("qwq32b_layer_bf16_2w", 2, 40, 8, 128, 1e6, torch.bfloat16, 1, lens,
                    [round_up(x) for x in lens], 0.5, seed)


def qwq_step(seed: int = 1003, layers: int = 64, append_room: int = 1024) -> Workload:
    rng = np.random.default_rng(seed)
    workers = [int(x) for x in rng.integers(256, 1025, size=4)]
    lens = [16384] + workers
    caps = [round_up(16384 + append_room)] + [1024] * 4
    return Workload("qwq32b_step_bf16_4w_16k", 4, 40, 8, 128, 1e6, torch.bfloat16, layers, lens,
                    caps, 0.5, seed)


def sweep(C: int, W: int, seed: int = 1004) -> Workload:
    common = 85 * C // 100
    rest = C - common
    per = [rest // W + (1 if i < rest % W else 0) for i in range(W)]
    lens = [common] + per
    return Workload(f"sweep_{C}_{W}w", W, 40, 8, 128, 1e6, torch.bfloat16, 1, lens,
                    [round_up(x) for x in lens], 0.5, seed)


def qwen3_loop(seed: int = 1005, layers: int = 36, common0: int = 32768, steps: int = 2048,
               private_cap: int = 512) -> Workload:
    rng = np.random.default_rng(seed)
    lens = [common0] + [int(x) for x in rng.integers(0, 64, size=4)]
    common_cap = round_up(common0 + steps * 4 + 4 * private_cap)
    return Workload("qwen3_8b_loop_bf16_4w", 4, 32, 8, 128, 1e6, torch.bfloat16, layers, lens,
                    [common_cap] + [private_cap] * 4, 0.5, seed)


def loop_appends(wl: Workload, steps: int, every: int = 64) -> dict:
    """Generation-loop schedule: {step: worker} for the steps after which one
    worker's block is appended into the common block and reset.

    Every `every` steps exactly one worker is picked, by a shuffled round
    robin: a fresh seeded permutation of the W workers for every W * every
    steps, so the gap between two appends of one worker is 1 to 2W - 1
    windows and a private block never holds more than (2W - 1) * every plus
    its initial length of tokens.
    """
    rng = np.random.default_rng(wl.seed + 7)
    out = {}
    order = []
    for k, s in enumerate(range(every - 1, steps, every)):
        if not order:
            order = [int(x) for x in rng.permutation(wl.W)]
        out[s] = order.pop(0)
    return out


def _gen(seed: int, layer: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 97 + tag) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def with_fp8(wl: Workload) -> Workload:
    """The same workload over an FP8 E4M3 pool (same draws, same seed)."""
    return dataclasses.replace(wl, name=wl.name.replace("bf16", "fp8"), dtype=torch.float8_e4m3fn)


def make_q(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    """q [W][Hq][D] in the query dtype of the pool, N(0,1)."""
    g = _gen(wl.seed, layer, 1, device)
    q = torch.randn(wl.W, wl.Hq, wl.D, generator=g, device=device, dtype=torch.float32)
    return q.to(wl.q_dtype)


def make_kv(wl: Workload, layer: int, num_slots: int, device="cpu", poison_unused: bool = False,
            block_start=None):
    """Logical K, V [Hkv][num_slots][D] in the pool dtype (FP8 pools: make_kv_fp8).

    poison_unused: slots outside every block's current length hold NaN (they
    must never reach a result).
    """
    if wl.fp8:
        raise ValueError("FP8 workloads: use make_kv_fp8 (codes and scales)")
    K, V = _draw_kv(wl, layer, num_slots, device, poison_unused, block_start)
    return K.to(wl.dtype), V.to(wl.dtype)


def make_kv_fp8(wl: Workload, layer: int, num_slots: int, device="cpu",
                poison_unused: bool = False, block_start=None):
    """FP8 E4M3 pools: logical K, V codes [Hkv][num_slots][D] (torch.float8_e4m3fn)
    of the same draws as make_kv, and per kv head scales k_scale, v_scale [Hkv]
    (amax of the head's plane / 448, so that no code saturates).  The stored
    value is code * scale."""
    K, V = _draw_kv(wl, layer, num_slots, device, poison_unused, block_start)

    def quant(X):
        amax = torch.nan_to_num(X.abs(), nan=0.0).amax(dim=(1, 2))
        scale = (amax / 448.0).clamp_min(2.0 ** -20)
        return (X / scale[:, None, None]).to(torch.float8_e4m3fn), scale.float().cpu()

    K8, ks = quant(K)
    V8, vs = quant(V)
    return K8, V8, ks, vs


def _draw_kv(wl: Workload, layer: int, num_slots: int, device, poison_unused, block_start):
    gk = _gen(wl.seed, layer, 2, device)
    gv = _gen(wl.seed, layer, 3, device)
    shape = (wl.Hkv, num_slots, wl.D)
    K = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
    V = torch.randn(shape, generator=gv, device=device, dtype=torch.float32)
    if wl.offset_sigma > 0:
        go = _gen(wl.seed, layer, 4, device)
        K += wl.offset_sigma * torch.randn(wl.Hkv, 1, wl.D, generator=go, device=device)
        V += wl.offset_sigma * torch.randn(wl.Hkv, 1, wl.D, generator=go, device=device)
    if poison_unused:
        starts = block_start if block_start is not None else np.cumsum([0] + wl.caps[:-1])
        used = torch.zeros(num_slots, dtype=torch.bool, device=device)
        for b, n in enumerate(wl.lens):
            used[int(starts[b]):int(starts[b]) + int(n)] = True
        K[:, ~used] = float("nan")
        V[:, ~used] = float("nan")
    return K, V


def summary(wl: Workload) -> dict:
    return {
        "workload": wl.name, "workers": wl.W, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
        "head_dim": wl.D, "rope_theta": wl.theta, "layers": wl.layers,
        "block_lens": [int(x) for x in wl.lens], "tokens": wl.tokens,
        "kv_dtype": {torch.bfloat16: "bf16", torch.float32: "f32",
                     torch.float8_e4m3fn: "fp8_e4m3"}[wl.dtype],
    }


__all__ = ["Workload", "tiny", "qwq_layer", "qwq_step", "sweep", "qwen3_loop", "loop_appends",
           "with_fp8", "make_q", "make_kv", "make_kv_fp8", "summary", "round_up"]
