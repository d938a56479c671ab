"""Pool storage layout: logical [..., slots, head_dim] <-> the library's tile layout.

Pure index permutations (no arithmetic on the values).  Slots are grouped in
tiles of 32; inside a tile (t = slot % 32, D = head_dim):

  key   (t, d) -> (t // 16) * 16 * D + (d // 8) * 128 + (t % 16) * 8 + d % 8
  value (t, d) -> ((t % 16) // 4) * 8 * D + d * 8 + (t // 16) * 4 + t % 4

which is the order in which the gfx950 bf16 MFMA kernels load their operand
fragments (one contiguous 16-byte vector per lane).  Works on torch tensors on
any device; the slot count must be a multiple of 32.
"""
from __future__ import annotations

import torch

TILE = 32


def _check(x: torch.Tensor):
    S, D = x.shape[-2], x.shape[-1]
    if S % TILE or D % 8:
        raise ValueError(f"slots ({S}) must be a multiple of 32 and head_dim ({D}) of 8")
    return S, D


def pack_keys(x: torch.Tensor) -> torch.Tensor:
    S, D = _check(x)
    lead = x.shape[:-2]
    y = x.reshape(*lead, S // TILE, 2, 16, D // 8, 8)           # [T, a, i, c, e]
    n = len(lead)
    y = y.permute(*range(n), n, n + 1, n + 3, n + 2, n + 4)     # [T, a, c, i, e]
    return y.contiguous().reshape(*lead, S, D)


def unpack_keys(y: torch.Tensor) -> torch.Tensor:
    S, D = _check(y)
    lead = y.shape[:-2]
    x = y.reshape(*lead, S // TILE, 2, D // 8, 16, 8)           # [T, a, c, i, e]
    n = len(lead)
    x = x.permute(*range(n), n, n + 1, n + 3, n + 2, n + 4)     # [T, a, i, c, e]
    return x.contiguous().reshape(*lead, S, D)


def pack_values(x: torch.Tensor) -> torch.Tensor:
    S, D = _check(x)
    lead = x.shape[:-2]
    y = x.reshape(*lead, S // TILE, 2, 4, 4, D)                 # [T, a, g, v, d]
    n = len(lead)
    y = y.permute(*range(n), n, n + 2, n + 4, n + 1, n + 3)     # [T, g, d, a, v]
    return y.contiguous().reshape(*lead, S, D)


def unpack_values(y: torch.Tensor) -> torch.Tensor:
    S, D = _check(y)
    lead = y.shape[:-2]
    x = y.reshape(*lead, S // TILE, 4, D, 2, 4)                 # [T, g, d, a, v]
    n = len(lead)
    x = x.permute(*range(n), n, n + 3, n + 1, n + 4, n + 2)     # [T, a, g, v, d]
    return x.contiguous().reshape(*lead, S, D)
