"""Python binding of libhogwild_attn (ctypes): the C ABI's calls under the same names.

Argument marshalling only: torch tensors are passed as device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the shared library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import layout

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhogwild_attn.so")

HW_OK, HW_EINVAL, HW_ERANGE, HW_ECAPACITY, HW_EUNSUPPORTED, HW_EWORKSPACE, HW_EHIP = range(7)
HW_DEV_BAD_ENTRY, HW_DEV_BAD_LENGTH, HW_DEV_NO_TOKENS, HW_DEV_APPEND_OVERFLOW = 1, 2, 4, 8
HW_DEV_WRITE_OVERFLOW, HW_DEV_STALE_PLAN, HW_DEV_WORKSPACE, HW_DEV_SPIN_LIMIT = 16, 32, 64, 128
HW_F32, HW_BF16, HW_FP8 = 0, 1, 2
HW_TILE_TOKENS = 32
HW_ABI_VERSION = 3
HW_MAX_BLOCKS, HW_MAX_WORKERS, HW_MAX_ROWS, HW_MAX_ENTRIES, HW_MAX_FP8_KV_HEADS = 64, 32, 80, 64, 64
PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2
HW_LAYOUT_COMBINED, HW_LAYOUT_INTERLEAVED, HW_LAYOUT_CONTIGUOUS = 0, 1, 2


class HWError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {hw_status_str(code)} (code {code})")


class hw_entry(ctypes.Structure):
    _fields_ = [("block_id", ctypes.c_int32), ("view_offset", ctypes.c_int32)]


class hw_pool(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("num_slots", ctypes.c_int64),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_len", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("block_start", ctypes.c_void_p),
        ("block_cap", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


_HW_DTYPES = {torch.bfloat16: HW_BF16, torch.float32: HW_F32, torch.float8_e4m3fn: HW_FP8}


def query_dtype(pool_dtype: torch.dtype) -> torch.dtype:
    """dtype of q for a pool: fp32 for fp32 pools, bf16 for bf16 and FP8 pools."""
    return torch.float32 if pool_dtype == torch.float32 else torch.bfloat16


EXPORTED = [
    "hw_abi_version", "hw_status_str", "hw_attn_plan_bytes", "hw_attn_plan", "hw_attn_run",
    "hw_attn_workspace_bytes", "hw_attn_decode", "hw_attn_decode_noalloc", "hw_attn_chunk",
    "hw_block_append", "hw_block_reset", "hw_block_advance", "hw_block_write",
    "hw_build_combined_tables", "hw_build_view_tables", "hw_pool_status", "hw_set_tuning",
]

_lib = None


def lib() -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run decode_attention_shared_hw_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, d, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                              ctypes.c_size_t)
        PP = ctypes.POINTER(hw_pool)
        L.hw_abi_version.restype = i32
        L.hw_abi_version.argtypes = []
        L.hw_status_str.restype = ctypes.c_char_p
        L.hw_status_str.argtypes = [i32]
        L.hw_attn_plan_bytes.restype = sz
        L.hw_attn_plan_bytes.argtypes = [PP, i32, i32, i32]
        L.hw_attn_plan.restype = i32
        L.hw_attn_plan.argtypes = [PP, i32, i32, i32, P, i32, P, P, sz, P]
        L.hw_attn_run.restype = i32
        L.hw_attn_run.argtypes = [PP, i32, P, i32, i32, i32, P, sz, d, P, P, sz, P]
        L.hw_attn_workspace_bytes.restype = sz
        L.hw_attn_workspace_bytes.argtypes = [PP, i32, i32]
        L.hw_attn_decode.restype = i32
        L.hw_attn_decode.argtypes = [PP, i32, P, i32, i32, P, i32, P, d, P, P, sz, P]
        L.hw_attn_decode_noalloc.restype = i32
        L.hw_attn_decode_noalloc.argtypes = [PP, i32, P, i32, i32, P, i32, P, d, P, P]
        L.hw_attn_chunk.restype = i32
        L.hw_attn_chunk.argtypes = [PP, i32, P, i32, i32, i32, P, i32, P, d, P, P, sz, P]
        L.hw_block_append.restype = i32
        L.hw_block_append.argtypes = [PP, i32, i32, d, P]
        L.hw_block_reset.restype = i32
        L.hw_block_reset.argtypes = [PP, i32, P]
        L.hw_block_advance.restype = i32
        L.hw_block_advance.argtypes = [PP, i32, P, P]
        L.hw_block_write.restype = i32
        L.hw_block_write.argtypes = [PP, i32, i32, P, P, P, d, P]
        L.hw_build_combined_tables.restype = i32
        L.hw_build_combined_tables.argtypes = [PP, i32, i32, P, P, P, P]
        L.hw_build_view_tables.restype = i32
        L.hw_build_view_tables.argtypes = [PP, i32, i32, i32, P, P, P, P]
        L.hw_pool_status.restype = i32
        L.hw_pool_status.argtypes = [PP, P, i32, P]
        L.hw_set_tuning.restype = i32
        L.hw_set_tuning.argtypes = [i32, i32, i32]
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != HW_OK:
        raise HWError(code, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


class Pool:
    """A K/V block pool spanning `num_layers` layers, owned by torch tensors.

    k, v: device tensors [num_layers, num_kv_heads, num_slots, head_dim] in the
    library's tile layout (see `layout`); block_len / status: device int32.
    block b owns slots [block_start[b], block_start[b] + block_cap[b]).
    FP8 pools (dtype torch.float8_e4m3fn) hold E4M3 codes; k_scale / v_scale
    [num_layers][num_kv_heads] (host) give value = code * scale.
    """

    def __init__(self, num_layers, num_kv_heads, head_dim, block_caps, dtype=torch.bfloat16,
                 device="cuda", fill=None, k_scale=None, v_scale=None):
        caps = [int(c) for c in block_caps]
        if any(c % HW_TILE_TOKENS for c in caps):
            raise ValueError("block capacities must be multiples of 32")
        starts, s = [], 0
        for c in caps:
            starts.append(s)
            s += c
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.num_slots = max(s, HW_TILE_TOKENS)
        self.dtype = dtype
        self.hw_dtype = _HW_DTYPES[dtype]
        shape = (num_layers, num_kv_heads, self.num_slots, head_dim)
        if fill is None:
            self.k = torch.zeros(shape, dtype=dtype, device=device)
            self.v = torch.zeros(shape, dtype=dtype, device=device)
        else:
            self.k = torch.full(shape, fill, dtype=dtype, device=device)
            self.v = torch.full(shape, fill, dtype=dtype, device=device)
        self.block_len = torch.zeros(len(caps), dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self._start = (ctypes.c_int64 * len(caps))(*starts)
        self._cap = (ctypes.c_int32 * len(caps))(*caps)
        self.block_start = starts
        self.block_cap = caps
        self._ks = self._vs = None
        if k_scale is not None or v_scale is not None:
            n = num_layers * num_kv_heads
            ks = [float(x) for x in torch.as_tensor(k_scale, dtype=torch.float32).reshape(-1)]
            vs = [float(x) for x in torch.as_tensor(v_scale, dtype=torch.float32).reshape(-1)]
            if len(ks) != n or len(vs) != n:
                raise ValueError("k_scale and v_scale must hold num_layers * num_kv_heads values")
            self._ks = (ctypes.c_float * n)(*ks)
            self._vs = (ctypes.c_float * n)(*vs)
        self.desc = hw_pool(self.hw_dtype, num_layers, num_kv_heads, head_dim, len(caps), 0,
                            self.num_slots, self.k.data_ptr(), self.v.data_ptr(),
                            self.block_len.data_ptr(), self.status.data_ptr(),
                            ctypes.cast(self._start, ctypes.c_void_p),
                            ctypes.cast(self._cap, ctypes.c_void_p),
                            ctypes.cast(self._ks, ctypes.c_void_p) if self._ks else None,
                            ctypes.cast(self._vs, ctypes.c_void_p) if self._vs else None)

    def scales(self, layer):
        """(k_scale, v_scale) lists of one layer's kv heads (FP8 pools)."""
        H = self.num_kv_heads
        return list(self._ks[layer * H:(layer + 1) * H]), list(self._vs[layer * H:(layer + 1) * H])

    @property
    def num_blocks(self):
        return len(self.block_cap)

    # -- layout marshalling (index permutations only) --
    def _bits(self, t):
        # FP8 codes are moved as bytes (index permutations only)
        return t.view(torch.uint8) if self.hw_dtype == HW_FP8 else t

    def store_layer(self, layer, k_logical, v_logical):
        """Write logical [Hkv, num_slots, D] K/V (pool dtype) into `layer`."""
        k = k_logical.to(self.k.device, self.dtype)
        v = v_logical.to(self.v.device, self.dtype)
        self._bits(self.k[layer]).copy_(layout.pack_keys(self._bits(k)))
        self._bits(self.v[layer]).copy_(layout.pack_values(self._bits(v)))

    def load_layer(self, layer):
        """Logical [Hkv, num_slots, D] copies of `layer`'s K/V."""
        k = layout.unpack_keys(self._bits(self.k[layer]))
        v = layout.unpack_values(self._bits(self.v[layer]))
        if self.hw_dtype == HW_FP8:
            return k.view(self.dtype), v.view(self.dtype)
        return k, v

    def set_lengths(self, lens):
        self.block_len.copy_(torch.as_tensor(lens, dtype=torch.int32))


def hw_abi_version() -> int:
    return int(lib().hw_abi_version())


def hw_status_str(code: int) -> str:
    return lib().hw_status_str(int(code)).decode()


def hw_set_tuning(path: int = PATH_AUTO, units_per_head: int = 0, balance: int = 0):
    _check(lib().hw_set_tuning(int(path), int(units_per_head), int(balance)), "hw_set_tuning")


def _expect(t, name, dtype, shape, device):
    """Raise ValueError unless `t` is a contiguous tensor of `dtype` and `shape` on `device`
    (the library sees bare pointers and cannot check sizes itself)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, the pool is on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _expect_bytes(t, name, nbytes, device):
    """A contiguous device byte buffer of at least `nbytes`."""
    if not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor on {device}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _check_views(pool, tables, num_entries, W):
    dev = pool.k.device
    if not isinstance(tables, torch.Tensor) or tables.dim() != 3 or tables.shape[2] != 2:
        raise ValueError("tables: expected int32 [W][E][2]")
    _expect(tables, "tables", torch.int32, (W, tables.shape[1], 2), dev)
    _expect(num_entries, "num_entries", torch.int32, (W,), dev)


def hw_attn_plan_bytes(pool: Pool, num_workers: int, chunk: int, num_q_heads: int) -> int:
    return int(lib().hw_attn_plan_bytes(ctypes.byref(pool.desc), num_workers, chunk, num_q_heads))


def alloc_plan(pool: Pool, num_workers: int, num_q_heads: int, chunk: int = 1) -> torch.Tensor:
    """Device buffer for hw_attn_plan (int32 words)."""
    n = hw_attn_plan_bytes(pool, num_workers, chunk, num_q_heads)
    if n == 0:
        raise HWError(HW_EINVAL, "hw_attn_plan_bytes")
    return torch.empty((n + 3) // 4, dtype=torch.int32, device=pool.k.device)


def hw_attn_workspace_bytes(pool: Pool, num_workers: int, num_q_heads: int) -> int:
    return int(lib().hw_attn_workspace_bytes(ctypes.byref(pool.desc), num_workers, num_q_heads))


def alloc_workspace(pool: Pool, num_workers: int, num_q_heads: int) -> torch.Tensor:
    """Device workspace for hw_attn_decode / hw_attn_chunk / hw_attn_run (zeroed: its merge
    counters must start at zero; every call leaves them zero)."""
    n = hw_attn_workspace_bytes(pool, num_workers, num_q_heads)
    if n == 0:
        raise HWError(HW_EINVAL, "hw_attn_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=pool.k.device)


def hw_attn_plan(pool: Pool, tables: torch.Tensor, num_entries: torch.Tensor, plan: torch.Tensor,
                 num_q_heads: int, chunk: int = 1, stream=None):
    """Plan of the decode (chunk = 1) or chunk calls over these views: tables int32 [W][E][2],
    num_entries int32 [W], plan from alloc_plan."""
    W = int(num_entries.shape[0]) if isinstance(num_entries, torch.Tensor) else 0
    _check_views(pool, tables, num_entries, W)
    nb = hw_attn_plan_bytes(pool, W, chunk, num_q_heads)
    _expect_bytes(plan, "plan", nb, pool.k.device)
    code = lib().hw_attn_plan(ctypes.byref(pool.desc), W, int(chunk), int(num_q_heads),
                              _ptr(tables), int(tables.shape[1]), _ptr(num_entries), _ptr(plan),
                              plan.numel() * plan.element_size(), _stream(stream))
    _check(code, "hw_attn_plan")


def hw_attn_run(pool: Pool, layer: int, q: torch.Tensor, plan: torch.Tensor, rope_theta: float,
                out: torch.Tensor, workspace: torch.Tensor, stream=None):
    """One layer from a plan.  q [W][Hq][D] (decode) or [W][n][Hq][D] (chunk),
    query_dtype(pool.dtype); out fp32 of the same shape."""
    dev = pool.k.device
    if not isinstance(q, torch.Tensor) or q.dim() not in (3, 4):
        raise ValueError("q: expected [W][Hq][D] or [W][n][Hq][D]")
    W, n = int(q.shape[0]), (int(q.shape[1]) if q.dim() == 4 else 1)
    Hq = int(q.shape[-2])
    shape = (W, Hq, pool.head_dim) if q.dim() == 3 else (W, n, Hq, pool.head_dim)
    _expect(q, "q", query_dtype(pool.dtype), shape, dev)
    _expect(out, "out", torch.float32, shape, dev)
    _expect_bytes(plan, "plan", hw_attn_plan_bytes(pool, W, n, Hq), dev)
    _expect_bytes(workspace, "workspace", hw_attn_workspace_bytes(pool, W * n, Hq), dev)
    code = lib().hw_attn_run(ctypes.byref(pool.desc), int(layer), _ptr(q), W, n, Hq, _ptr(plan),
                             plan.numel() * plan.element_size(), float(rope_theta), _ptr(out),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check(code, "hw_attn_run")


def hw_attn_decode(pool: Pool, layer: int, q: torch.Tensor, tables: torch.Tensor,
                   num_entries: torch.Tensor, rope_theta: float, out: torch.Tensor,
                   workspace: torch.Tensor, stream=None):
    """q [W][Hq][D] (query_dtype(pool.dtype)), tables int32 [W][E][2], num_entries int32 [W],
    out fp32 [W][Hq][D]."""
    dev = pool.k.device
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q: expected [W][Hq][D]")
    W, Hq, _ = q.shape
    _expect(q, "q", query_dtype(pool.dtype), (W, Hq, pool.head_dim), dev)
    _expect(out, "out", torch.float32, (W, Hq, pool.head_dim), dev)
    _check_views(pool, tables, num_entries, W)
    _expect_bytes(workspace, "workspace", hw_attn_workspace_bytes(pool, W, Hq), dev)
    code = lib().hw_attn_decode(ctypes.byref(pool.desc), int(layer), _ptr(q), W, Hq, _ptr(tables),
                                int(tables.shape[1]), _ptr(num_entries), float(rope_theta),
                                _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "hw_attn_decode")


NOALLOC_SCRATCH_BYTES = 16 << 20  # HW_NOALLOC_SCRATCH_BYTES


def hw_attn_decode_noalloc(pool: Pool, layer: int, q: torch.Tensor, tables: torch.Tensor,
                           num_entries: torch.Tensor, rope_theta: float, out: torch.Tensor,
                           stream=None):
    """hw_attn_decode with the library's static per-GPU scratch as its workspace: the
    call allocates no device memory (neither here nor in the library).  Calls that may
    overlap on one GPU race on the scratch."""
    dev = pool.k.device
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q: expected [W][Hq][D]")
    W, Hq, _ = q.shape
    _expect(q, "q", query_dtype(pool.dtype), (W, Hq, pool.head_dim), dev)
    _expect(out, "out", torch.float32, (W, Hq, pool.head_dim), dev)
    _check_views(pool, tables, num_entries, W)
    code = lib().hw_attn_decode_noalloc(ctypes.byref(pool.desc), int(layer), _ptr(q), W, Hq,
                                        _ptr(tables), int(tables.shape[1]), _ptr(num_entries),
                                        float(rope_theta), _ptr(out), _stream(stream))
    _check(code, "hw_attn_decode_noalloc")


def hw_attn_chunk(pool: Pool, layer: int, q: torch.Tensor, tables: torch.Tensor,
                  num_entries: torch.Tensor, rope_theta: float, out: torch.Tensor,
                  workspace: torch.Tensor, stream=None):
    """q [W][n][Hq][D] (query_dtype(pool.dtype)): each worker's last n tokens as queries, causal over the
    view; out fp32 [W][n][Hq][D]; workspace sized for W * n workers."""
    dev = pool.k.device
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected [W][n][Hq][D]")
    W, n, Hq, _ = q.shape
    _expect(q, "q", query_dtype(pool.dtype), (W, n, Hq, pool.head_dim), dev)
    _expect(out, "out", torch.float32, (W, n, Hq, pool.head_dim), dev)
    _check_views(pool, tables, num_entries, W)
    _expect_bytes(workspace, "workspace", hw_attn_workspace_bytes(pool, W * n, Hq), dev)
    code = lib().hw_attn_chunk(ctypes.byref(pool.desc), int(layer), _ptr(q), W, n, Hq,
                               _ptr(tables), int(tables.shape[1]), _ptr(num_entries),
                               float(rope_theta), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "hw_attn_chunk")


def hw_block_append(pool: Pool, src_block: int, dst_block: int, rope_theta: float, stream=None):
    _check(lib().hw_block_append(ctypes.byref(pool.desc), int(src_block), int(dst_block),
                                 float(rope_theta), _stream(stream)), "hw_block_append")


def hw_block_reset(pool: Pool, block: int, stream=None):
    _check(lib().hw_block_reset(ctypes.byref(pool.desc), int(block), _stream(stream)),
           "hw_block_reset")


def _blocks(blocks):
    arr = (ctypes.c_int32 * len(blocks))(*[int(b) for b in blocks])
    return len(blocks), ctypes.cast(arr, ctypes.c_void_p), arr


def hw_block_advance(pool: Pool, blocks, stream=None):
    """Reserve the next slot of every listed block (block_len += 1 on the device)."""
    n, p, keep = _blocks(blocks)
    _check(lib().hw_block_advance(ctypes.byref(pool.desc), n, p, _stream(stream)),
           "hw_block_advance")


def hw_block_write(pool: Pool, layer: int, blocks, k_new: torch.Tensor, v_new: torch.Tensor,
                   rope_theta: float, stream=None):
    """Store each listed block's new token of `layer` in slot block_len - 1.
    k_new, v_new: device fp32 [len(blocks)][num_kv_heads][head_dim]."""
    n, p, keep = _blocks(blocks)
    shape = (n, pool.num_kv_heads, pool.head_dim)
    _expect(k_new, "k_new", torch.float32, shape, pool.k.device)
    _expect(v_new, "v_new", torch.float32, shape, pool.k.device)
    _check(lib().hw_block_write(ctypes.byref(pool.desc), int(layer), n, p, _ptr(k_new),
                                _ptr(v_new), float(rope_theta), _stream(stream)),
           "hw_block_write")


def hw_build_combined_tables(pool: Pool, num_workers: int, common_block: int, worker_block,
                             tables: torch.Tensor, num_entries: torch.Tensor, stream=None):
    """tables: device int32 [W][W+1][2]; num_entries: device int32 [W]."""
    _expect(tables, "tables", torch.int32, (num_workers, num_workers + 1, 2), pool.k.device)
    _expect(num_entries, "num_entries", torch.int32, (num_workers,), pool.k.device)
    wb = (ctypes.c_int32 * num_workers)(*[int(b) for b in worker_block])
    _check(lib().hw_build_combined_tables(ctypes.byref(pool.desc), int(num_workers),
                                          int(common_block), ctypes.cast(wb, ctypes.c_void_p),
                                          _ptr(tables), _ptr(num_entries), _stream(stream)),
           "hw_build_combined_tables")


def hw_build_view_tables(pool: Pool, layout: int, num_workers: int, common_block: int,
                         worker_block, tables: torch.Tensor, num_entries: torch.Tensor,
                         stream=None):
    """View tables of one of the HW_LAYOUT_* layouts; shapes as hw_build_combined_tables."""
    _expect(tables, "tables", torch.int32, (num_workers, num_workers + 1, 2), pool.k.device)
    _expect(num_entries, "num_entries", torch.int32, (num_workers,), pool.k.device)
    wb = (ctypes.c_int32 * num_workers)(*[int(b) for b in worker_block])
    _check(lib().hw_build_view_tables(ctypes.byref(pool.desc), int(layout), int(num_workers),
                                      int(common_block), ctypes.cast(wb, ctypes.c_void_p),
                                      _ptr(tables), _ptr(num_entries), _stream(stream)),
           "hw_build_view_tables")


def hw_pool_status(pool: Pool, clear: bool = False, stream=None) -> int:
    """The pool's sticky HW_DEV_* bits once `stream`'s work so far is done (synchronizes it)."""
    flags = ctypes.c_int32(0)
    _check(lib().hw_pool_status(ctypes.byref(pool.desc), ctypes.byref(flags), int(bool(clear)),
                                _stream(stream)), "hw_pool_status")
    return int(flags.value)
