"""Test helpers: build a pool from a seeded workload, run the oracle and the library on it."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from decode_attention_shared_hw_amd import hogwild_attn as hw
from decode_attention_shared_hw_amd import workloads

BF16_MAX_ABS, BF16_REL_L2 = 5e-3, 1e-2   # bf16 inputs, fp32 accumulation
F32_REL = 1e-5                           # fp32 inputs


# Entry point of Setup.decode: "decode" (hw_attn_decode: up to 32 stacked MFMA
# rows take the kernel that builds its plan in-kernel) or "plan_run"
# (hw_attn_plan + hw_attn_run: the plan kernel and the run kernels).
API = "decode"


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.abs(got - ref).max())
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel_l2


def assert_close(got, ref, dtype, what=""):
    max_abs, rel_l2 = errors(got, ref)
    if dtype == torch.float32:
        scale = max(float(np.abs(ref).max()), 1e-30)
        assert max_abs <= F32_REL * scale and rel_l2 <= F32_REL, \
            f"{what}: fp32 max_abs {max_abs:.3e} (scale {scale:.3e}) rel_l2 {rel_l2:.3e}"
    else:
        assert max_abs <= BF16_MAX_ABS and rel_l2 <= BF16_REL_L2, \
            f"{what}: bf16 max_abs {max_abs:.3e} rel_l2 {rel_l2:.3e}"
    return max_abs, rel_l2


class Setup:
    """A device pool filled from a workload (layers [0, n_layers)) plus host copies.

    K, V: the stored values per layer (FP8 pools: code * scale in float64);
    K8, V8, k_scale, v_scale: the FP8 codes and scales (FP8 pools only)."""

    def __init__(self, wl: workloads.Workload, n_layers: int = 1, poison_unused=False,
                 gen_device="cpu"):
        self.wl = wl
        slots = sum(wl.caps)
        starts = list(np.cumsum([0] + list(wl.caps[:-1])))
        draws = []
        for layer in range(n_layers):
            if wl.fp8:
                draws.append(workloads.make_kv_fp8(wl, layer, max(slots, 32), device=gen_device,
                                                   poison_unused=poison_unused, block_start=starts))
            else:
                draws.append(workloads.make_kv(wl, layer, max(slots, 32), device=gen_device,
                                               poison_unused=poison_unused, block_start=starts))
        self.k_scale = torch.stack([d[2] for d in draws]) if wl.fp8 else None
        self.v_scale = torch.stack([d[3] for d in draws]) if wl.fp8 else None
        self.pool = hw.Pool(n_layers, wl.Hkv, wl.D, wl.caps, dtype=wl.dtype,
                            k_scale=self.k_scale, v_scale=self.v_scale)
        assert self.pool.block_start == starts and self.pool.num_slots == max(slots, 32)
        self.pool.set_lengths(wl.lens)
        self.K, self.V, self.q, self.K8, self.V8 = [], [], [], [], []
        for layer, d in enumerate(draws):
            K, V = d[0], d[1]
            self.pool.store_layer(layer, K, V)
            if wl.fp8:
                self.K8.append(K.cpu())
                self.V8.append(V.cpu())
                self.K.append(K.cpu().double() * d[2].double()[:, None, None])
                self.V.append(V.cpu().double() * d[3].double()[:, None, None])
            else:
                self.K.append(K.cpu())
                self.V.append(V.cpu())
            self.q.append(workloads.make_q(wl, layer, device=gen_device).cpu())
        self.tables = torch.zeros(wl.W, wl.W + 1, 2, dtype=torch.int32, device="cuda")
        self.num_entries = torch.zeros(wl.W, dtype=torch.int32, device="cuda")
        hw.hw_build_combined_tables(self.pool, wl.W, wl.common_block, wl.worker_block,
                                    self.tables, self.num_entries)
        self.ws = hw.alloc_workspace(self.pool, wl.W, wl.Hq)

    def decode(self, layer=0, q=None, tables=None, num_entries=None, api=None):
        """One attention call through the C ABI: hw_attn_decode (api "decode"), or
        hw_attn_plan + hw_attn_run (api "plan_run"); the module's API by default."""
        wl = self.wl
        api = API if api is None else api
        q = (self.q[layer] if q is None else q).to("cuda")
        tables = self.tables if tables is None else tables
        num_entries = self.num_entries if num_entries is None else num_entries
        out = torch.full((q.shape[0], wl.Hq, wl.D), float("nan"), device="cuda")
        if self.ws.numel() < hw.hw_attn_workspace_bytes(self.pool, q.shape[0], wl.Hq):
            self.ws = hw.alloc_workspace(self.pool, q.shape[0], wl.Hq)
        if api == "plan_run":
            plan = hw.alloc_plan(self.pool, q.shape[0], wl.Hq)
            hw.hw_attn_plan(self.pool, tables, num_entries, plan, wl.Hq)
            hw.hw_attn_run(self.pool, layer, q, plan, wl.theta, out, self.ws)
        else:
            hw.hw_attn_decode(self.pool, layer, q, tables, num_entries, wl.theta, out, self.ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_tables(self, lens=None):
        lens = self.wl.lens if lens is None else lens
        return oracle.build_combined_tables(self.wl.common_block, self.wl.worker_block, lens)

    def oracle_decode(self, layer=0, form=oracle.FORM_METHOD, q=None, lens=None, tables=None):
        lens = np.asarray(self.wl.lens if lens is None else lens, np.int32)
        if tables is None:
            tb, to, ne = self.oracle_tables(lens)
        else:
            tb, to, ne = tables
        q = self.q[layer] if q is None else q
        out, rc = oracle.attn_decode(form, q.double().numpy(), self.K[layer].double().numpy(),
                                     self.V[layer].double().numpy(), tb, to, ne, lens,
                                     np.asarray(self.pool.block_start, np.int64), self.wl.theta)
        return out, rc

    def oracle_one(self, layer, w, h, form=oracle.FORM_METHOD, lens=None):
        lens = np.asarray(self.wl.lens if lens is None else lens, np.int32)
        tb, to, ne = self.oracle_tables(lens)
        g = h // self.wl.G
        out, rc = oracle.attn_one(form, self.q[layer][w, h].double().numpy(),
                                  self.K[layer][g].double().numpy(),
                                  self.V[layer][g].double().numpy(), tb[w], to[w], lens,
                                  np.asarray(self.pool.block_start, np.int64), self.wl.theta)
        return out, rc
