"""ctypes binding of libpagedkv.so: the C ABI of include/pagedkv.h under the
same names.  Argument marshalling only -- every step of the decode path runs
in the library's HIP kernels.  Shapes and sizes of torch tensors are checked
here because the C side receives bare pointers and cannot.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")
# A host-only build of the block manager (csrc/pool.cpp alone, e.g. under
# the host sanitizers) may stand in for the library in CPU tests; it has no
# device entry points.
HOST_LIB_PATH = os.environ.get("PKV_HOST_LIB")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_NO_BLOCKS, PKV_ERR_BAD_BLOCK = 0, -1, -2, -3
PKV_ERR_REFCOUNT, PKV_ERR_CAPACITY, PKV_ERR_HIP, PKV_ERR_WORKSPACE, PKV_ERR_BAD_SEQ = -4, -5, -6, -7, -8
PKV_F32, PKV_BF16, PKV_INT8, PKV_FP8 = 0, 1, 2, 3
_DTYPE_CODE = {"f32": PKV_F32, "bf16": PKV_BF16, "int8": PKV_INT8, "fp8": PKV_FP8}
# One-byte caches: codes plus a float32 scale per (token, kv head) row.
Q8_CODES = (PKV_INT8, PKV_FP8)
BLOCK_SIZE = 16

STATUS_NAMES = {0: "OK", -1: "INVALID", -2: "NO_BLOCKS", -3: "BAD_BLOCK", -4: "REFCOUNT", -5: "CAPACITY",
                -6: "HIP", -7: "WORKSPACE", -8: "BAD_SEQ"}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = STATUS_NAMES.get(code, str(code))


class pkv_layout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]

    @property
    def elem_bytes(self) -> int:
        """Bytes of one stored element (a one-byte code for PKV_INT8 and PKV_FP8)."""
        return {PKV_F32: 4, PKV_BF16: 2}.get(self.kv_dtype, 1)

    @property
    def tile_bytes(self) -> int:
        """Bytes of one (block, kv head) tile; int8 and FP8 tiles end with 16 float32 scales."""
        return BLOCK_SIZE * self.head_dim * self.elem_bytes + (4 * BLOCK_SIZE if self.kv_dtype in Q8_CODES else 0)

    @property
    def pool_elems(self) -> int:
        """Elements of a pool tensor: stored elements, or bytes for PKV_INT8 and PKV_FP8."""
        if self.kv_dtype in Q8_CODES:
            return self.num_blocks * self.num_kv_heads * self.tile_bytes
        return self.num_blocks * self.num_kv_heads * BLOCK_SIZE * self.head_dim


class pkv_stats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_free", ctypes.c_int32), ("num_used", ctypes.c_int32),
                ("num_shared", ctypes.c_int32), ("num_seqs", ctypes.c_int64), ("tokens_logical", ctypes.c_int64),
                ("tokens_stored", ctypes.c_int64), ("usage", ctypes.c_double),
                ("internal_fragmentation", ctypes.c_double)]


class pkv_prefix_stats(ctypes.Structure):
    _fields_ = [("lookups", ctypes.c_int64), ("query_tokens", ctypes.c_int64), ("hit_tokens", ctypes.c_int64),
                ("registered", ctypes.c_int64), ("evictions", ctypes.c_int64), ("cached_blocks", ctypes.c_int32),
                ("idle_blocks", ctypes.c_int32), ("hit_rate", ctypes.c_double)]


class pkv_swap_stats(ctypes.Structure):
    _fields_ = [("host_blocks", ctypes.c_int32), ("host_used", ctypes.c_int32), ("host_free", ctypes.c_int32),
                ("clock_hand", ctypes.c_int32), ("swapped_out", ctypes.c_int64), ("swapped_in", ctypes.c_int64)]


PKV_PLAN_KEY_INTS = 32


class pkv_decode_plan(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_int64 * PKV_PLAN_KEY_INTS)]


class pkv_decode_opts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32), ("waves_per_simd", ctypes.c_int32),
                ("ev_begin", ctypes.c_void_p),
                ("ev_partition_done", ctypes.c_void_p), ("ev_end", ctypes.c_void_p),
                ("xcd_weights", ctypes.c_int32 * 8), ("load_policy", ctypes.c_int32), ("trace", ctypes.c_void_p),
                ("plan", ctypes.c_void_p), ("plan_buffer", ctypes.c_void_p), ("plan_bytes", ctypes.c_size_t)]


PKV_TRACE_WAVES = 8192  # waves a decode trace buffer holds (4 int32 each)


# name -> (restype, argtypes) of every exported symbol of include/pagedkv.h
_P, _I32, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_PL = ctypes.POINTER(pkv_layout)
_PO = ctypes.POINTER(pkv_decode_opts)
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_pool_create": (ctypes.c_int, [_PL, _P, ctypes.POINTER(_P)]),
    "pkv_pool_destroy": (ctypes.c_int, [_P]),
    "pkv_block_alloc": (ctypes.c_int, [_P, ctypes.POINTER(_I32)]),
    "pkv_block_incref": (ctypes.c_int, [_P, _I32]),
    "pkv_block_free": (ctypes.c_int, [_P, _I32]),
    "pkv_block_refcount": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_I32)]),
    "pkv_pool_num_free": (ctypes.c_int, [_P, ctypes.POINTER(_I32)]),
    "pkv_seq_create": (ctypes.c_int, [_P, ctypes.POINTER(_I64)]),
    "pkv_seq_fork": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I64)]),
    "pkv_seq_append_slots": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_batch_append_slots": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_seq_free": (ctypes.c_int, [_P, _I64]),
    "pkv_seq_len": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I32)]),
    "pkv_seq_block_table": (ctypes.c_int, [_P, _I64, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_batch_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pkv_pool_stats": (ctypes.c_int, [_P, ctypes.POINTER(pkv_stats)]),
    "pkv_xcd_weights_from_trace": (ctypes.c_int, [_P, _I32, _P]),
    "pkv_prefix_cache_enable": (ctypes.c_int, [_P, _I32]),
    "pkv_seq_create_from_prefix": (ctypes.c_int, [_P, _P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "pkv_seq_register_prefix": (ctypes.c_int, [_P, _I64, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_prefix_cache_stats": (ctypes.c_int, [_P, ctypes.POINTER(pkv_prefix_stats)]),
    "pkv_swap_configure": (ctypes.c_int, [_P, _I32]),
    "pkv_swap_out": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_seq_swap_in": (ctypes.c_int, [_P, _I64, _P, _I32, ctypes.POINTER(_I32)]),
    "pkv_seq_resident": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I32)]),
    "pkv_swap_space_stats": (ctypes.c_int, [_P, ctypes.POINTER(pkv_swap_stats)]),
    "pkv_swap_copy": (ctypes.c_int, [_PL, _P, _P, _I32, _P, _P, _I32, _P, _I32, _P]),
    "pkv_kv_bytes_per_token": (_I64, [_PL, _I32]),
    "pkv_pool_bytes": (_I64, [_PL]),
    "pkv_validate_tables": (ctypes.c_int, [_PL, _P, _P, _I32, _I32]),
    "paged_kv_append": (ctypes.c_int, [_PL, _P, _P, _P, _P, _P, _I32, _P]),
    "pkv_copy_blocks": (ctypes.c_int, [_PL, _P, _P, _P, _I32, _P]),
    "paged_attention_workspace_bytes": (_SZ, [_PL, _I32, _I32, _I32, _PO]),
    "paged_attention_decode": (ctypes.c_int, [_PL, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _F, _P, _SZ,
                                              _PO, _P]),
    "paged_attention_prefill": (ctypes.c_int, [_PL, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F,
                                               _P]),
    "paged_attention_decode_noalloc": (ctypes.c_int, [_PL, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _F, _PO,
                                                      _P]),
    "paged_attention_plan_bytes": (_SZ, [_PL, _I32, _I32, _I32, _PO]),
}

_lib = None


def lib():
    """Load the in-tree library; fail loudly when it has not been built."""
    global _lib
    if _lib is None:
        if HOST_LIB_PATH:
            L = ctypes.CDLL(HOST_LIB_PATH)
        else:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                  "(hipcc --offload-arch=gfx950); there is no fallback path")
            import torch  # noqa: F401  -- bind to the HIP runtime torch loaded (same soname)
            L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            if HOST_LIB_PATH and not hasattr(L, name):
                continue  # a device entry point: not in a host-only build
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != PKV_OK:
        raise PagedKVError(rc, lib().pkv_last_error().decode(errors="replace"))


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode(errors="replace")


def pkv_version() -> str:
    return lib().pkv_version().decode()


def make_layout(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str) -> pkv_layout:
    return pkv_layout(int(num_blocks), BLOCK_SIZE, int(num_kv_heads), int(head_dim), _DTYPE_CODE[dtype])


# ------------------------------------------------------------------ host pool
def pkv_pool_create(layout: pkv_layout, free_order=None):
    h = ctypes.c_void_p()
    fo = None
    if free_order is not None:
        fo = np.ascontiguousarray(free_order, dtype=np.int32)
        if fo.size != layout.num_blocks:
            raise ValueError("free_order must hold num_blocks entries")
    _check(lib().pkv_pool_create(ctypes.byref(layout), None if fo is None else _np_ptr(fo), ctypes.byref(h)))
    return h


def pkv_pool_destroy(pool):
    _check(lib().pkv_pool_destroy(pool))


def pkv_block_alloc(pool) -> int:
    out = ctypes.c_int32()
    _check(lib().pkv_block_alloc(pool, ctypes.byref(out)))
    return out.value


def pkv_block_incref(pool, block: int):
    _check(lib().pkv_block_incref(pool, int(block)))


def pkv_block_free(pool, block: int):
    _check(lib().pkv_block_free(pool, int(block)))


def pkv_block_refcount(pool, block: int) -> int:
    out = ctypes.c_int32()
    _check(lib().pkv_block_refcount(pool, int(block), ctypes.byref(out)))
    return out.value


def pkv_pool_num_free(pool) -> int:
    out = ctypes.c_int32()
    _check(lib().pkv_pool_num_free(pool, ctypes.byref(out)))
    return out.value


def pkv_seq_create(pool) -> int:
    out = ctypes.c_int64()
    _check(lib().pkv_seq_create(pool, ctypes.byref(out)))
    return out.value


def pkv_seq_fork(pool, parent: int) -> int:
    out = ctypes.c_int64()
    _check(lib().pkv_seq_fork(pool, int(parent), ctypes.byref(out)))
    return out.value


def pkv_batch_append_slots(pool, ids, n: int, cow_cap: int | None = None, slots_out: np.ndarray | None = None):
    """Returns (slots int64 [len(ids) * n], cow pairs int32 [k][2])."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    cap = len(ids) if cow_cap is None else int(cow_cap)
    if slots_out is None:
        slots_out = np.empty(len(ids) * n, dtype=np.int64)
    elif slots_out.dtype != np.int64 or slots_out.size < len(ids) * n or not slots_out.flags["C_CONTIGUOUS"]:
        raise ValueError("slots_out must be a contiguous int64 array of len(ids) * n entries")
    cow = np.empty((max(cap, 1), 2), dtype=np.int32)
    ncow = ctypes.c_int32(0)
    _check(lib().pkv_batch_append_slots(pool, _np_ptr(ids), len(ids), int(n), _np_ptr(slots_out), _np_ptr(cow), cap,
                                        ctypes.byref(ncow)))
    return slots_out, cow[:ncow.value].copy()


def pkv_seq_append_slots(pool, seq: int, n: int, cow_cap: int = 1):
    slots = np.empty(n, dtype=np.int64)
    cow = np.empty((max(cow_cap, 1), 2), dtype=np.int32)
    ncow = ctypes.c_int32(0)
    _check(lib().pkv_seq_append_slots(pool, int(seq), int(n), _np_ptr(slots), _np_ptr(cow), int(cow_cap),
                                      ctypes.byref(ncow)))
    return slots, cow[:ncow.value].copy()


def pkv_seq_free(pool, seq: int):
    _check(lib().pkv_seq_free(pool, int(seq)))


def pkv_seq_len(pool, seq: int) -> int:
    out = ctypes.c_int32()
    _check(lib().pkv_seq_len(pool, int(seq), ctypes.byref(out)))
    return out.value


def pkv_seq_block_table(pool, seq: int) -> list:
    n = ctypes.c_int32()
    rc = lib().pkv_seq_block_table(pool, int(seq), None, 0, ctypes.byref(n))
    if rc not in (PKV_OK, PKV_ERR_CAPACITY):
        _check(rc)
    out = np.empty(max(n.value, 1), dtype=np.int32)
    _check(lib().pkv_seq_block_table(pool, int(seq), _np_ptr(out), out.size, ctypes.byref(n)))
    return out[:n.value].tolist()


def pkv_batch_block_tables(pool, ids, max_blocks: int, tables_out: np.ndarray | None = None,
                           ctx_out: np.ndarray | None = None):
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    B = len(ids)
    if tables_out is None:
        tables_out = np.empty((B, max_blocks), dtype=np.int32)
    if ctx_out is None:
        ctx_out = np.empty(B, dtype=np.int32)
    if tables_out.dtype != np.int32 or tables_out.size != B * max_blocks or not tables_out.flags["C_CONTIGUOUS"]:
        raise ValueError("tables_out must be a contiguous int32 [B][max_blocks] array")
    if ctx_out.dtype != np.int32 or ctx_out.size != B or not ctx_out.flags["C_CONTIGUOUS"]:
        raise ValueError("ctx_out must be a contiguous int32 [B] array")
    _check(lib().pkv_batch_block_tables(pool, _np_ptr(ids), B, int(max_blocks), _np_ptr(tables_out),
                                        _np_ptr(ctx_out)))
    return tables_out, ctx_out


def pkv_pool_stats(pool) -> dict:
    s = pkv_stats()
    _check(lib().pkv_pool_stats(pool, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in pkv_stats._fields_}


def pkv_prefix_cache_enable(pool, enable: bool = True):
    _check(lib().pkv_prefix_cache_enable(pool, 1 if enable else 0))


def pkv_seq_create_from_prefix(pool, token_ids):
    """(sequence id, tokens found cached) for a prompt of token ids."""
    toks = np.ascontiguousarray(token_ids, dtype=np.int32)
    sid, nc = ctypes.c_int64(), ctypes.c_int32()
    _check(lib().pkv_seq_create_from_prefix(pool, _np_ptr(toks), toks.size, ctypes.byref(sid), ctypes.byref(nc)))
    return sid.value, nc.value


def pkv_seq_register_prefix(pool, seq: int, token_ids, n: int | None = None) -> int:
    toks = np.ascontiguousarray(token_ids, dtype=np.int32)
    n = toks.size if n is None else int(n)
    if n > toks.size:
        raise ValueError("n exceeds the token ids given")
    added = ctypes.c_int32()
    _check(lib().pkv_seq_register_prefix(pool, int(seq), _np_ptr(toks), n, ctypes.byref(added)))
    return added.value


def pkv_prefix_cache_stats(pool) -> dict:
    s = pkv_prefix_stats()
    _check(lib().pkv_prefix_cache_stats(pool, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in pkv_prefix_stats._fields_}


def pkv_swap_configure(pool, num_host_blocks: int):
    _check(lib().pkv_swap_configure(pool, int(num_host_blocks)))


def pkv_swap_out(pool, want: int, protect=()) -> np.ndarray:
    """Clock victims: int32 [n][2] of (device block, host slot)."""
    prot = np.ascontiguousarray(np.asarray(list(protect), dtype=np.int64))
    out = np.empty((max(int(want), 1), 2), dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().pkv_swap_out(pool, int(want), _np_ptr(prot) if prot.size else None, prot.size, _np_ptr(out),
                              int(want), ctypes.byref(n)))
    return out[:n.value].copy()


def pkv_seq_swap_in(pool, seq: int) -> np.ndarray:
    """int32 [n][2] of (host slot, device block) to copy back."""
    n = ctypes.c_int32()
    rc = lib().pkv_seq_swap_in(pool, int(seq), None, 0, ctypes.byref(n))
    if rc == PKV_ERR_CAPACITY or (rc == PKV_OK and n.value > 0):
        out = np.empty((max(n.value, 1), 2), dtype=np.int32)
        _check(lib().pkv_seq_swap_in(pool, int(seq), _np_ptr(out), n.value, ctypes.byref(n)))
        return out[:n.value].copy()
    _check(rc)
    return np.zeros((0, 2), dtype=np.int32)


def pkv_seq_resident(pool, seq: int) -> bool:
    r = ctypes.c_int32()
    _check(lib().pkv_seq_resident(pool, int(seq), ctypes.byref(r)))
    return bool(r.value)


def pkv_swap_space_stats(pool) -> dict:
    s = pkv_swap_stats()
    _check(lib().pkv_swap_space_stats(pool, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in pkv_swap_stats._fields_}


def pkv_kv_bytes_per_token(layout: pkv_layout, num_layers: int) -> int:
    return lib().pkv_kv_bytes_per_token(ctypes.byref(layout), int(num_layers))


def pkv_pool_bytes(layout: pkv_layout) -> int:
    return lib().pkv_pool_bytes(ctypes.byref(layout))


def pkv_validate_tables(layout: pkv_layout, tables: np.ndarray, ctx: np.ndarray):
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    _check(lib().pkv_validate_tables(ctypes.byref(layout), _np_ptr(tables), _np_ptr(ctx), ctx.size,
                                     tables.shape[1] if tables.ndim == 2 else 0))


# ---------------------------------------------------------------- device side
def _dev(t, what, dtype=None, numel=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what} must hold {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def pool_torch_dtype(layout):
    """torch dtype of a pool tensor (uint8 bytes for an int8 or FP8 cache)."""
    import torch
    return {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16}.get(layout.kv_dtype, torch.uint8)


def row_torch_dtype(layout):
    """torch dtype of queries and of the rows handed to append."""
    import torch
    return torch.float32 if layout.kv_dtype == PKV_F32 else torch.bfloat16


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def paged_kv_append(layout, k_pool, v_pool, k_new, v_new, slots, stream=None):
    import torch
    pdt, rdt = pool_torch_dtype(layout), row_torch_dtype(layout)
    T = slots.numel()
    row = layout.num_kv_heads * layout.head_dim
    args = (ctypes.byref(layout), _dev(k_pool, "k_pool", pdt, layout.pool_elems),
            _dev(v_pool, "v_pool", pdt, layout.pool_elems), _dev(k_new, "k_new", rdt, T * row),
            _dev(v_new, "v_new", rdt, T * row), _dev(slots, "slots", torch.int64), T, _stream(stream))
    _check(lib().paged_kv_append(*args))


def pkv_copy_blocks(layout, k_pool, v_pool, pairs, stream=None):
    import torch
    dt = pool_torch_dtype(layout)
    if pairs.numel() % 2:
        raise ValueError("pairs must be [n][2]")
    _check(lib().pkv_copy_blocks(ctypes.byref(layout), _dev(k_pool, "k_pool", dt, layout.pool_elems),
                                 _dev(v_pool, "v_pool", dt, layout.pool_elems), _dev(pairs, "pairs", torch.int32),
                                 pairs.numel() // 2, _stream(stream)))


def decode_opts(partition_tokens=0, kernel=0, events=None, waves_per_simd=0, xcd_weights=None,
                trace=None, load_policy=0, plan=None) -> pkv_decode_opts:
    """trace: optional device int32 tensor of 4 * PKV_TRACE_WAVES elements;
    load_policy: 0 auto, 1 streaming (non-temporal) K/V loads, 2 cached;
    plan: (pkv_decode_plan, device buffer of paged_attention_plan_bytes()
    bytes): an all-zero record makes the call record its split there, a
    recorded one makes it run from it (the caller keeps both alive while the
    options are used)."""
    ev = list(events) if events else [None, None, None]
    o = pkv_decode_opts(int(partition_tokens), int(kernel), int(waves_per_simd), *[e if e else None for e in ev])
    o.load_policy = int(load_policy)
    if plan is not None:
        rec, buf = plan
        if not isinstance(rec, pkv_decode_plan):
            raise TypeError("plan must be (pkv_decode_plan, device buffer)")
        o.plan = ctypes.addressof(rec)
        o.plan_buffer = _dev(buf, "plan buffer").value
        o.plan_bytes = buf.numel() * buf.element_size()
    if xcd_weights is not None:
        w = [int(x) for x in xcd_weights]
        if len(w) != 8:
            raise ValueError("xcd_weights must hold 8 values")
        o.xcd_weights[:] = w
    if trace is not None:
        import torch
        o.trace = _dev(trace, "trace", torch.int32, 4 * PKV_TRACE_WAVES).value
    return o


def xcd_weights_from_trace(trace) -> list:
    """Per-XCD weights (1000 = the mean rate) from a decode trace (a host
    or device int32 tensor, or a numpy array, of 4 * PKV_TRACE_WAVES)."""
    arr = np.ascontiguousarray(trace.cpu().numpy() if hasattr(trace, "cpu") else trace, dtype=np.int32).reshape(-1)
    if arr.size < 4:
        raise ValueError("trace too small")
    out = np.zeros(8, np.int32)
    _check(lib().pkv_xcd_weights_from_trace(arr.ctypes.data_as(ctypes.c_void_p), min(arr.size // 4, PKV_TRACE_WAVES),
                                            out.ctypes.data_as(ctypes.c_void_p)))
    return [int(x) for x in out]


def paged_attention_workspace_bytes(layout, num_seqs, num_q_heads, max_context_len, partition_tokens=0,
                                    kernel=0) -> int:
    o = decode_opts(partition_tokens, kernel)
    return lib().paged_attention_workspace_bytes(ctypes.byref(layout), int(num_seqs), int(num_q_heads),
                                                 int(max_context_len), ctypes.byref(o))


def paged_attention_plan_bytes(layout, num_seqs, num_q_heads, max_context_len, partition_tokens=0) -> int:
    o = decode_opts(partition_tokens)
    return lib().paged_attention_plan_bytes(ctypes.byref(layout), int(num_seqs), int(num_q_heads),
                                            int(max_context_len), ctypes.byref(o))


def new_decode_plan(layout, num_seqs, num_q_heads, max_context_len, partition_tokens=0, device="cuda"):
    """(empty pkv_decode_plan, plan buffer) for the decode calls of one step:
    pass it as plan= to each; the first records the split, the others run
    from it.  Zero the record (reset_decode_plan) when tables or lengths
    change."""
    import torch
    n = paged_attention_plan_bytes(layout, num_seqs, num_q_heads, max_context_len, partition_tokens)
    return pkv_decode_plan(), torch.empty(max(-(-n // 4), 1), dtype=torch.int32, device=device)


def reset_decode_plan(plan):
    """Empties a plan record, so that the next call records a new split."""
    ctypes.memset(ctypes.addressof(plan[0] if isinstance(plan, tuple) else plan), 0, ctypes.sizeof(pkv_decode_plan))


def paged_attention_decode(layout, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale,
                           workspace=None, partition_tokens=0, kernel=0, events=None, stream=None, waves_per_simd=0,
                           xcd_weights=None, trace=None, load_policy=0, plan=None):
    """events: optional (begin, partition_done, end) raw hipEvent_t handles."""
    import torch
    pdt, rdt = pool_torch_dtype(layout), row_torch_dtype(layout)
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError("q must be [num_seqs][num_q_heads][head_dim]")
    B, Hq, D = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    mb = block_tables.shape[1]
    ws_need = paged_attention_workspace_bytes(layout, B, Hq, max_context_len, partition_tokens, kernel)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < ws_need:
        raise ValueError(f"workspace of {ws_need} bytes needed, got {ws_bytes}")
    o = decode_opts(partition_tokens, kernel, events, waves_per_simd, xcd_weights, trace, load_policy, plan)
    _check(lib().paged_attention_decode(
        ctypes.byref(layout), _dev(out, "out", torch.float32, B * Hq * D), _dev(q, "q", rdt),
        _dev(k_pool, "k_pool", pdt, layout.pool_elems), _dev(v_pool, "v_pool", pdt, layout.pool_elems),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32, B),
        B, Hq, mb, int(max_context_len), float(scale), ws_ptr, ws_bytes, ctypes.byref(o), _stream(stream)))


def paged_attention_decode_noalloc(layout, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                                   scale, partition_tokens=0, kernel=0, events=None, stream=None, waves_per_simd=0,
                                   xcd_weights=None, trace=None, load_policy=0, plan=None):
    """paged_attention_decode on the library's own per-GPU scratch: no
    workspace argument, no allocation."""
    import torch
    pdt, rdt = pool_torch_dtype(layout), row_torch_dtype(layout)
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError("q must be [num_seqs][num_q_heads][head_dim]")
    B, Hq, D = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    o = decode_opts(partition_tokens, kernel, events, waves_per_simd, xcd_weights, trace, load_policy, plan)
    _check(lib().paged_attention_decode_noalloc(
        ctypes.byref(layout), _dev(out, "out", torch.float32, B * Hq * D), _dev(q, "q", rdt),
        _dev(k_pool, "k_pool", pdt, layout.pool_elems), _dev(v_pool, "v_pool", pdt, layout.pool_elems),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32, B),
        B, Hq, block_tables.shape[1], int(max_context_len), float(scale), ctypes.byref(o), _stream(stream)))


def paged_attention_prefill(layout, out, q, k_pool, v_pool, block_tables, context_lens, query_start, max_query_len,
                            max_context_len, scale, stream=None):
    """Causal attention of the new tokens of every sequence: q and out are
    [T][num_q_heads][head_dim] with sequence b's rows query_start[b] ..
    query_start[b+1]-1, the last tokens of its context_lens[b]."""
    import torch
    pdt = pool_torch_dtype(layout)
    if q.dim() != 3 or q.shape[2] != layout.head_dim:
        raise ValueError("q must be [T][num_q_heads][head_dim]")
    T, Hq, D = q.shape
    B = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    _check(lib().paged_attention_prefill(
        ctypes.byref(layout), _dev(out, "out", torch.float32, T * Hq * D), _dev(q, "q", torch.bfloat16),
        _dev(k_pool, "k_pool", pdt, layout.pool_elems), _dev(v_pool, "v_pool", pdt, layout.pool_elems),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32, B),
        _dev(query_start, "query_start", torch.int32, B + 1), B, Hq, block_tables.shape[1], int(max_query_len),
        int(max_context_len), float(scale), _stream(stream)))


def pkv_swap_copy(layout, dst_k, dst_v, dst_blocks, src_k, src_v, src_blocks, pairs, stream=None):
    """Whole blocks from one pool to another (either may be pinned host
    memory): pairs int32 [n][2] of (source, destination) readable by the
    device."""
    import torch
    if pairs.numel() % 2:
        raise ValueError("pairs must be [n][2]")
    pdt = pool_torch_dtype(layout)
    per_block = layout.pool_elems // layout.num_blocks
    for t, what, nb in ((dst_k, "dst_k", dst_blocks), (dst_v, "dst_v", dst_blocks), (src_k, "src_k", src_blocks),
                        (src_v, "src_v", src_blocks)):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.dtype != pdt or t.numel() != nb * per_block:
            raise ValueError(f"{what} must be a contiguous {pdt} tensor of {nb} blocks")
    if not (pairs.is_cuda or pairs.is_pinned()) or pairs.dtype != torch.int32:
        raise ValueError("pairs must be int32 on the device or in pinned memory")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    _check(lib().pkv_swap_copy(ctypes.byref(layout), p(dst_k), p(dst_v), int(dst_blocks), p(src_k), p(src_v),
                               int(src_blocks), p(pairs), pairs.numel() // 2, _stream(stream)))
