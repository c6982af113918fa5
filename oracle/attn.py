"""ctypes wrapper around the C oracle (``attn.c``) plus the oracle's own
end-to-end run of a workload (bookkeeping -> append -> attention).

TEST INFRASTRUCTURE; see ``oracle/__init__.py`` for who may use it.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

from . import build as _build
from .book import BLOCK_SIZE, build_workload

_DT = {"f32": 0, "bf16": 1, "int8": 2, "fp8": 3}
_NP = {"f32": np.float32, "bf16": np.uint16, "int8": np.uint8, "fp8": np.uint8}
# Element type of queries and of the rows handed to append: an int8 or FP8
# cache is fed bfloat16 rows and quantises them itself.
ROW = {"f32": "f32", "bf16": "bf16", "int8": "bf16", "fp8": "bf16"}
# One-byte caches: codes plus a float32 scale per (token, kv head).
QUANT = ("int8", "fp8")
NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0)}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_append.argtypes = [I, I, I, P, P, P, P, P, I64]
        L.orc_copy_blocks.argtypes = [I, I, I, P, P, P, I]
        L.orc_paged_attention.argtypes = [I, I, I, I, P, P, P, P, I, P, I, D, P]
        L.orc_contiguous_attention.argtypes = [I, I, I, I, P, P, P, I, D, P]
        L.orc_partitioned_attention.argtypes = [I, I, I, I, P, P, P, P, I, P, I, D, I, P]
        L.orc_gather_token.argtypes = [I, I, I, P, P, P, I, P, P]
        L.orc_paged_prefill.argtypes = [I, I, I, I, P, P, P, P, I, P, P, I, D, P]
        L.orc_num_threads.restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def tile_bytes_int8(head_dim: int) -> int:
    """Bytes of one (block, kv head) tile of an int8 pool: 16 * D codes, then
    16 float32 scales."""
    return BLOCK_SIZE * head_dim + 4 * BLOCK_SIZE


def new_pool(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str):
    """K and V pools filled with a NaN sentinel: slots never written stay NaN
    (for int8, zero codes under a NaN scale)."""
    if dtype in QUANT:
        tb = tile_bytes_int8(head_dim)
        tiles = np.zeros((num_blocks * num_kv_heads, tb), dtype=np.uint8)
        tiles[:, BLOCK_SIZE * head_dim:] = np.full((tiles.shape[0], BLOCK_SIZE), np.nan,
                                                   dtype=np.float32).view(np.uint8)
        return tiles.reshape(-1), tiles.reshape(-1).copy()
    n = num_blocks * num_kv_heads * BLOCK_SIZE * head_dim
    k = np.full(n, NAN_BITS[dtype], dtype=_NP[dtype])
    v = np.full(n, NAN_BITS[dtype], dtype=_NP[dtype])
    return k, v


def append(dtype, num_kv_heads, head_dim, kpool, vpool, k_new, v_new, slots):
    k_new = np.ascontiguousarray(k_new, dtype=_NP[ROW[dtype]])
    v_new = np.ascontiguousarray(v_new, dtype=_NP[ROW[dtype]])
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    assert k_new.shape == v_new.shape == (slots.size, num_kv_heads, head_dim)
    # A negative slot is skipped; one past the pool is outside the definition
    # (the C routine has no pool size and would write past the array).
    per_block = num_kv_heads * (tile_bytes_int8(head_dim) if dtype in QUANT else BLOCK_SIZE * head_dim)
    if slots.size and slots.max() >= kpool.size // per_block * BLOCK_SIZE:
        raise ValueError("slot past the end of the pool")
    lib().orc_append(_DT[dtype], num_kv_heads, head_dim, _p(kpool), _p(vpool), _p(k_new), _p(v_new),
                     _p(slots), slots.size)


def copy_blocks(dtype, num_kv_heads, head_dim, kpool, vpool, pairs):
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    lib().orc_copy_blocks(_DT[dtype], num_kv_heads, head_dim, _p(kpool), _p(vpool), _p(pairs),
                          pairs.shape[0])


def paged_attention(dtype, q, kpool, vpool, tables, ctx, num_kv_heads, scale):
    q = np.ascontiguousarray(q, dtype=_NP[ROW[dtype]])
    B, Hq, D = q.shape
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lib().orc_paged_attention(_DT[dtype], Hq, num_kv_heads, D, _p(q), _p(kpool), _p(vpool), _p(tables),
                              tables.shape[1], _p(ctx), B, float(scale), _p(out))
    return out


def partitioned_attention(dtype, q, kpool, vpool, tables, ctx, num_kv_heads, scale, part_tokens):
    q = np.ascontiguousarray(q, dtype=_NP[ROW[dtype]])
    B, Hq, D = q.shape
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lib().orc_partitioned_attention(_DT[dtype], Hq, num_kv_heads, D, _p(q), _p(kpool), _p(vpool),
                                    _p(tables), tables.shape[1], _p(ctx), B, float(scale),
                                    int(part_tokens), _p(out))
    return out


def paged_prefill(dtype, q, kpool, vpool, tables, ctx, qstart, num_kv_heads, scale):
    """Causal attention of every new token of every sequence: q [T][Hq][D]
    (rows of sequence b are qstart[b] .. qstart[b+1]-1, the last tokens of its
    ctx[b]) -> [T][Hq][D] float64."""
    q = np.ascontiguousarray(q, dtype=_NP[ROW[dtype]])
    T, Hq, D = q.shape
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    qstart = np.ascontiguousarray(qstart, dtype=np.int32)
    B = ctx.size
    assert qstart.size == B + 1 and qstart[0] == 0 and qstart[-1] == T
    assert (np.diff(qstart) >= 0).all() and (np.diff(qstart) <= ctx).all()
    out = np.zeros((T, Hq, D), dtype=np.float64)
    if T:
        lib().orc_paged_prefill(_DT[dtype], Hq, num_kv_heads, D, _p(q), _p(kpool), _p(vpool), _p(tables),
                                tables.shape[1], _p(ctx), _p(qstart), B, float(scale), _p(out))
    return out


def contiguous_attention(dtype, q_seq, k_seq, v_seq, scale):
    """q_seq [Hq][D]; k_seq, v_seq [n][Hkv][D] -> [Hq][D] float64 (f32 or
    bf16 elements: a contiguous cache is never quantised)."""
    assert dtype in ("f32", "bf16")
    q_seq = np.ascontiguousarray(q_seq, dtype=_NP[dtype])
    k_seq = np.ascontiguousarray(k_seq, dtype=_NP[dtype])
    v_seq = np.ascontiguousarray(v_seq, dtype=_NP[dtype])
    Hq, D = q_seq.shape
    n, Hkv, _ = k_seq.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    lib().orc_contiguous_attention(_DT[dtype], Hq, Hkv, D, _p(q_seq), _p(k_seq), _p(v_seq), n,
                                   float(scale), _p(out))
    return out


def gather_token(dtype, num_kv_heads, head_dim, kpool, vpool, table, j):
    table = np.ascontiguousarray(table, dtype=np.int32)
    k = np.zeros((num_kv_heads, head_dim))
    v = np.zeros((num_kv_heads, head_dim))
    lib().orc_gather_token(_DT[dtype], num_kv_heads, head_dim, _p(kpool), _p(vpool), _p(table), int(j),
                           _p(k), _p(v))
    return k, v


def num_threads() -> int:
    return lib().orc_num_threads()


def tables_of(book, ids, max_blocks=None):
    rows = [book.block_table(s) for s in ids]
    mb = max_blocks or max(1, max(len(r) for r in rows))
    t = np.zeros((len(ids), mb), dtype=np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    ctx = np.array([book.seq_len(s) for s in ids], dtype=np.int32)
    return t, ctx


def run_workload(inst, with_attention=True):
    """The oracle's own end-to-end decode step for a workload instance."""
    wl = inst.wl
    book, ids, pre_slots, step_slots, cow = build_workload(inst)
    assert not cow, "the workloads never trigger copy-on-write"
    kpool, vpool = new_pool(inst.num_blocks, wl.num_kv_heads, wl.head_dim, wl.cache_dtype)
    append(wl.cache_dtype, wl.num_kv_heads, wl.head_dim, kpool, vpool, inst.prefill_tokens("k"),
           inst.prefill_tokens("v"), np.asarray(pre_slots, dtype=np.int64))
    append(wl.cache_dtype, wl.num_kv_heads, wl.head_dim, kpool, vpool, inst.step_tokens("k"),
           inst.step_tokens("v"), np.asarray(step_slots, dtype=np.int64))
    tables, ctx = tables_of(book, ids)
    assert (ctx == inst.ctx).all()
    res = {"book": book, "ids": ids, "prefill_slots": pre_slots, "step_slots": step_slots,
           "kpool": kpool, "vpool": vpool, "tables": tables, "ctx": ctx}
    if with_attention:
        res["out"] = paged_attention(wl.cache_dtype, inst.q(), kpool, vpool, tables, ctx, wl.num_kv_heads,
                                     1.0 / math.sqrt(wl.head_dim))
    return res


def build_prefill(inst):
    """The build script of a prefill workload instance through the
    bookkeeping model and the oracle's append: tables, lengths and pools."""
    from .book import Book
    wl = inst.wl
    book = Book(inst.num_blocks, inst.free_order)
    kpool, vpool = new_pool(inst.num_blocks, wl.num_kv_heads, wl.head_dim, wl.cache_dtype)

    def put(sid, n, k, v):
        slots, cow = book.append_slots(sid, n)
        assert not cow
        append(wl.cache_dtype, wl.num_kv_heads, wl.head_dim, kpool, vpool, k, v, np.asarray(slots, np.int64))

    if wl.shared_prefix:
        root = book.create()
        put(root, wl.shared_prefix, inst.shared_kv("k"), inst.shared_kv("v"))
        ids = [root] + [book.fork(root) for _ in range(wl.batch - 1)]
    else:
        ids = [book.create() for _ in range(wl.batch)]
    for b, sid in enumerate(ids):
        put(sid, int(inst.own_prefix[b] + inst.nq[b]), inst.own_kv(b, "k"), inst.own_kv(b, "v"))
    tables, ctx = tables_of(book, ids)
    assert (ctx == inst.ctx).all()
    return {"book": book, "ids": ids, "tables": tables, "ctx": ctx, "kpool": kpool, "vpool": vpool}


def run_prefill(inst):
    """The oracle's own prefill of a prefill workload instance: the build,
    then causal attention of every new token."""
    res = build_prefill(inst)
    wl = inst.wl
    res["out"] = paged_prefill(wl.cache_dtype, inst.q(), res["kpool"], res["vpool"], res["tables"], res["ctx"],
                               inst.qstart, wl.num_kv_heads, 1.0 / math.sqrt(wl.head_dim))
    return res
