"""CPU oracle for Hogwild! concurrent-attention decode (fp64, plain C++).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
package ``decode_attention_shared_hw_amd`` never imports it, and this module
never imports the product package.

Thin ctypes wrappers over ``hogwild_oracle.cpp``; each C function cites the
passage of the pages it follows.  Arrays are numpy float64 holding the stored
values exactly (bf16 / fp32 widened).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hogwild_oracle.cpp")
# (HWO_LIB: another build of the same source, e.g. the sanitizer build of
# tests/sanitize_host.py)
_LIB = os.environ.get("HWO_LIB") or os.path.join(_HERE, "libhogwild_oracle.so")

HWO_OK, HWO_EINVAL, HWO_ENOTOKENS, HWO_ECAPACITY = 0, 1, 2, 3
HWO_F32, HWO_BF16, HWO_FP8 = 0, 1, 2
FORM_DEFINITION, FORM_METHOD = 0, 1


def build(out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with g++ (fp64, no FMA contraction); sanitize: with
    AddressSanitizer and UndefinedBehaviorSanitizer (host code only)."""
    out = out or _LIB
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC"]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=undefined"]
    cmd += ["-o", out + ".tmp", _SRC]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        d, i32, i64 = ctypes.c_double, ctypes.c_int32, ctypes.c_int64
        P = ctypes.c_void_p
        L.hwo_round_bf16.restype = d
        L.hwo_round_bf16.argtypes = [d]
        L.hwo_round_f32.restype = d
        L.hwo_round_f32.argtypes = [d]
        L.hwo_e4m3_value.restype = d
        L.hwo_e4m3_value.argtypes = [i32]
        L.hwo_round_e4m3.restype = d
        L.hwo_round_e4m3.argtypes = [d]
        L.hwo_rope.restype = None
        L.hwo_rope.argtypes = [P, i32, d, d, P]
        L.hwo_build_combined_tables.restype = i32
        L.hwo_build_combined_tables.argtypes = [i32, i32, P, i32, P, P, P, P]
        L.hwo_query_position.restype = i64
        L.hwo_query_position.argtypes = [i32, P, P, P]
        L.hwo_attn_one.restype = i32
        L.hwo_attn_one.argtypes = [i32, i32, d, i32, P, P, i32, P, P, P, P, P, P]
        L.hwo_attn_decode.restype = i32
        L.hwo_attn_decode.argtypes = [i32, i32, i32, i32, i32, d, i32, P, P, P, i32, P, P,
                                      i64, P, P, P, P]
        L.hwo_block_append.restype = i32
        L.hwo_block_append.argtypes = [i32, i32, i32, i64, P, P, i32, P, P, P, i32, i32, d, i32, P]
        L.hwo_attn_chunk.restype = i32
        L.hwo_attn_chunk.argtypes = [i32, i32, i32, i32, i32, i32, d, i32, P, P, P, i32, P, P, i64,
                                     P, P, P, P]
        L.hwo_build_interleaved_tables.restype = i32
        L.hwo_build_interleaved_tables.argtypes = L.hwo_build_combined_tables.argtypes
        L.hwo_block_write.restype = i32
        L.hwo_block_write.argtypes = [i32, i32, i64, P, P, i32, P, P, i32, P, P, P, d, i32, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def round_bf16(x: float) -> float:
    return lib().hwo_round_bf16(float(x))


def round_f32(x: float) -> float:
    return lib().hwo_round_f32(float(x))


def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (0..255)."""
    return lib().hwo_e4m3_value(int(code))


def round_e4m3(x: float) -> float:
    """Nearest OCP FP8 E4M3 value (ties to even, saturating at +-448)."""
    return lib().hwo_round_e4m3(float(x))


def _scales(s):
    if s is None:
        return None, None
    a = _c(s, np.float64).reshape(-1)
    return a, _p(a)


def rope(x, theta: float, pos: float) -> np.ndarray:
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib().hwo_rope(_p(x), x.shape[-1], float(theta), float(pos), _p(y))
    return y


def build_combined_tables(common_block: int, worker_block, block_len):
    """Returns (tbl_block [W][W+1], tbl_off [W][W+1], num_entries [W]) int32, or raises."""
    wb = _c(worker_block, np.int32)
    bl = _c(block_len, np.int32)
    W = wb.shape[0]
    tb = np.zeros((W, W + 1), np.int32)
    to = np.zeros((W, W + 1), np.int32)
    ne = np.zeros((W,), np.int32)
    rc = lib().hwo_build_combined_tables(W, int(common_block), _p(wb), bl.shape[0], _p(bl),
                                         _p(tb), _p(to), _p(ne))
    if rc != HWO_OK:
        raise ValueError(f"hwo_build_combined_tables: code {rc}")
    return tb, to, ne


def build_interleaved_tables(common_block: int, worker_block, block_len):
    """Interleaved layout: [common, own] per worker.  Same return shapes as
    build_combined_tables."""
    wb = _c(worker_block, np.int32)
    bl = _c(block_len, np.int32)
    W = wb.shape[0]
    tb = np.zeros((W, W + 1), np.int32)
    to = np.zeros((W, W + 1), np.int32)
    ne = np.zeros((W,), np.int32)
    rc = lib().hwo_build_interleaved_tables(W, int(common_block), _p(wb), bl.shape[0], _p(bl),
                                            _p(tb), _p(to), _p(ne))
    if rc != HWO_OK:
        raise ValueError(f"hwo_build_interleaved_tables: code {rc}")
    return tb, to, ne


def query_position(tbl_block_row, tbl_off_row, block_len) -> int:
    tb = _c(tbl_block_row, np.int32)
    to = _c(tbl_off_row, np.int32)
    bl = _c(block_len, np.int32)
    return int(lib().hwo_query_position(tb.shape[0], _p(tb), _p(to), _p(bl)))


def attn_one(form, q, K_plane, V_plane, tbl_block_row, tbl_off_row, block_len, block_start,
             theta):
    """One (worker, q-head): q [D]; K_plane/V_plane [num_slots][D].  Returns (out [D], rc)."""
    q = _c(q, np.float64)
    K = _c(K_plane, np.float64)
    V = _c(V_plane, np.float64)
    tb = _c(tbl_block_row, np.int32)
    to = _c(tbl_off_row, np.int32)
    bl = _c(block_len, np.int32)
    bs = _c(block_start, np.int64)
    out = np.zeros(q.shape[0], np.float64)
    rc = lib().hwo_attn_one(int(form), q.shape[0], float(theta), tb.shape[0], _p(tb), _p(to),
                            bl.shape[0], _p(bl), _p(bs), _p(q), _p(K), _p(V), _p(out))
    return out, rc


def attn_decode(form, q, K, V, tbl_block, tbl_off, num_entries, block_len, block_start, theta):
    """Whole call: q [W][Hq][D]; K, V [Hkv][num_slots][D]; tables [W][E].  Returns (out, rc)."""
    q = _c(q, np.float64)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    tb = _c(tbl_block, np.int32)
    to = _c(tbl_off, np.int32)
    ne = _c(num_entries, np.int32)
    bl = _c(block_len, np.int32)
    bs = _c(block_start, np.int64)
    W, Hq, D = q.shape
    Hkv, S, _ = K.shape
    out = np.zeros_like(q)
    rc = lib().hwo_attn_decode(int(form), W, Hq, Hkv, D, float(theta), tb.shape[1], _p(tb),
                               _p(to), _p(ne), bl.shape[0], _p(bl), _p(bs), S, _p(q), _p(K),
                               _p(V), _p(out))
    return out, rc



def attn_chunk(form, q, K, V, tbl_block, tbl_off, num_entries, block_len, block_start, theta):
    """Query chunk: q [W][n][Hq][D]; K, V [Hkv][num_slots][D]; tables [W][E].
    Query j of worker w sits at i_q[w] - (n - 1 - j) with a causal mask over
    the view.  Returns (out [W][n][Hq][D], rc)."""
    q = _c(q, np.float64)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    tb = _c(tbl_block, np.int32)
    to = _c(tbl_off, np.int32)
    ne = _c(num_entries, np.int32)
    bl = _c(block_len, np.int32)
    bs = _c(block_start, np.int64)
    W, n, Hq, D = q.shape
    Hkv, S, _ = K.shape
    out = np.zeros_like(q)
    rc = lib().hwo_attn_chunk(int(form), W, n, Hq, Hkv, D, float(theta), tb.shape[1], _p(tb),
                              _p(to), _p(ne), bl.shape[0], _p(bl), _p(bs), S, _p(q), _p(K),
                              _p(V), _p(out))
    return out, rc

def block_append(K, V, block_start, block_cap, block_len, src, dst, theta, dtype, k_scale=None):
    """In place on float64 arrays K, V [L][Hkv][num_slots][D] and int32 block_len.  Returns rc.
    FP8 pools: K, V hold code * scale and k_scale is [L][Hkv]."""
    assert K.dtype == np.float64 and K.flags.c_contiguous
    assert V.dtype == np.float64 and V.flags.c_contiguous
    assert block_len.dtype == np.int32 and block_len.flags.c_contiguous
    bs = _c(block_start, np.int64)
    bc = _c(block_cap, np.int32)
    L, Hkv, S, D = K.shape
    ks, ksp = _scales(k_scale)
    return lib().hwo_block_append(L, Hkv, D, S, _p(K), _p(V), bl_n(block_len), _p(bs), _p(bc),
                                  _p(block_len), int(src), int(dst), float(theta), int(dtype), ksp)


def block_write(K, V, block_start, block_len, blocks, k_new, v_new, theta, dtype, k_scale=None,
                v_scale=None):
    """In place on float64 arrays K, V [Hkv][num_slots][D] of one layer: the new
    token of every listed block at its slot block_len[b] - 1 (key design 1).
    k_new, v_new: [n][Hkv][D].  FP8 pools: k_scale, v_scale [Hkv].  Returns rc."""
    assert K.dtype == np.float64 and K.flags.c_contiguous
    assert V.dtype == np.float64 and V.flags.c_contiguous
    bs = _c(block_start, np.int64)
    bl = _c(block_len, np.int32)
    bk = _c(blocks, np.int32)
    kn = _c(k_new, np.float64)
    vn = _c(v_new, np.float64)
    Hkv, S, D = K.shape
    ks, ksp = _scales(k_scale)
    vs, vsp = _scales(v_scale)
    return lib().hwo_block_write(Hkv, D, S, _p(K), _p(V), int(bl.shape[0]), _p(bs), _p(bl),
                                 int(bk.shape[0]), _p(bk), _p(kn), _p(vn), float(theta), int(dtype),
                                 ksp, vsp)


def bl_n(block_len) -> int:
    return int(block_len.shape[0])
