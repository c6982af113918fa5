"""A paged KV cache on one GPU, driven through the C ABI.

``PagedKVCache`` owns the host block manager (``pkv_pool``) and one K and one
V pool tensor per layer in HBM; every layer shares the block tables, as in a
serving engine where the scheduler assigns slots once per step.  All device
work goes through the library's kernels; torch only allocates memory and
supplies the stream.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib as L

_NAN = {"bf16": 0x7FC0, "f32": float("nan")}


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str, num_layers: int = 1,
                 free_order=None, device="cuda", fill_nan: bool = True):
        self.dtype = dtype  # storage of the cache: "f32", "bf16", "int8" or "fp8"
        self.layout = L.make_layout(num_blocks, num_kv_heads, head_dim, dtype)
        self.pool = L.pkv_pool_create(self.layout, free_order)
        self.device = torch.device(device)
        tdt = L.pool_torch_dtype(self.layout)
        self.k_pools, self.v_pools = [], []
        for _ in range(num_layers):
            k = torch.empty(self.layout.pool_elems, dtype=tdt, device=self.device)
            v = torch.empty_like(k)
            if fill_nan:  # slots never written hold a NaN sentinel
                for t in (k, v):
                    if dtype == "bf16":
                        t.view(torch.int16).fill_(_NAN["bf16"])
                    elif dtype == "f32":
                        t.fill_(_NAN["f32"])
                    else:  # zero codes under a NaN scale
                        tiles = t.view(-1, self.layout.tile_bytes)
                        tiles[:, :16 * head_dim].zero_()
                        sc = torch.full((tiles.shape[0], 16), float("nan"), dtype=torch.float32, device=self.device)
                        tiles[:, 16 * head_dim:] = sc.view(torch.uint8).view(tiles.shape[0], 64)
            self.k_pools.append(k)
            self.v_pools.append(v)

    def close(self):
        if self.pool is not None:
            L.pkv_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- host bookkeeping -----------------------------------------------------
    def create(self) -> int:
        return L.pkv_seq_create(self.pool)

    def fork(self, parent: int) -> int:
        return L.pkv_seq_fork(self.pool, parent)

    def free(self, seq: int):
        L.pkv_seq_free(self.pool, seq)

    def reserve(self, ids, n: int):
        """Slots for n more tokens of every sequence in ids (batch order);
        pending copy-on-write copies run on every layer before returning."""
        slots, cow = L.pkv_batch_append_slots(self.pool, ids, n, cow_cap=max(1, len(ids)))
        if len(cow):
            pairs = torch.from_numpy(np.ascontiguousarray(cow)).to(self.device)
            for k, v in zip(self.k_pools, self.v_pools):
                L.pkv_copy_blocks(self.layout, k, v, pairs)
        return slots, cow

    # -- swap to host memory ------------------------------------------------
    def enable_swap(self, num_host_blocks: int):
        """Pinned host pools (one K and one V per layer) of num_host_blocks
        block slots, in the device pools' tile layout."""
        L.pkv_swap_configure(self.pool, num_host_blocks)
        per_block = self.layout.pool_elems // self.layout.num_blocks
        tdt = L.pool_torch_dtype(self.layout)
        self.num_host_blocks = num_host_blocks
        self.host_k = [torch.empty(num_host_blocks * per_block, dtype=tdt, pin_memory=True)
                       for _ in self.k_pools]
        self.host_v = [torch.empty(num_host_blocks * per_block, dtype=tdt, pin_memory=True)
                       for _ in self.v_pools]

    def swap_out(self, want: int, protect=()):
        """Clock victims moved to host slots on every layer; returns the
        (device block, host slot) pairs."""
        pairs = L.pkv_swap_out(self.pool, want, protect)
        if len(pairs):
            d = torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device)
            for layer in range(len(self.k_pools)):
                L.pkv_swap_copy(self.layout, self.host_k[layer], self.host_v[layer], self.num_host_blocks,
                                self.k_pools[layer], self.v_pools[layer], self.layout.num_blocks, d)
        return pairs

    def swap_in(self, seq: int):
        """Every host block of a sequence back on the device, every layer;
        returns the (host slot, device block) pairs."""
        pairs = L.pkv_seq_swap_in(self.pool, seq)
        if len(pairs):
            d = torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device)
            for layer in range(len(self.k_pools)):
                L.pkv_swap_copy(self.layout, self.k_pools[layer], self.v_pools[layer], self.layout.num_blocks,
                                self.host_k[layer], self.host_v[layer], self.num_host_blocks, d)
        return pairs

    # -- prefix cache ---------------------------------------------------------
    def enable_prefix_cache(self, on: bool = True):
        L.pkv_prefix_cache_enable(self.pool, on)

    def create_from_prefix(self, token_ids):
        """(sequence, tokens already cached): the caller stores K/V for the
        rest of the prompt, then calls register_prefix."""
        return L.pkv_seq_create_from_prefix(self.pool, token_ids)

    def register_prefix(self, seq: int, token_ids, n=None) -> int:
        return L.pkv_seq_register_prefix(self.pool, seq, token_ids, n)

    def prefix_stats(self) -> dict:
        return L.pkv_prefix_cache_stats(self.pool)

    def tables(self, ids, max_blocks: int):
        return L.pkv_batch_block_tables(self.pool, ids, max_blocks)

    def stats(self) -> dict:
        return L.pkv_pool_stats(self.pool)

    # -- device calls ---------------------------------------------------------
    def write(self, layer: int, slots_dev, k_new, v_new):
        L.paged_kv_append(self.layout, self.k_pools[layer], self.v_pools[layer], k_new, v_new, slots_dev)

    def decode(self, layer: int, out, q, tables_dev, ctx_dev, max_ctx: int, scale: float, workspace=None,
               partition_tokens=0, kernel=0, events=None, waves_per_simd=None, xcd_weights=None, trace=None,
               load_policy=0, plan=None):
        if waves_per_simd is None:
            waves_per_simd = self.waves_per_simd()
        L.paged_attention_decode(self.layout, out, q, self.k_pools[layer], self.v_pools[layer], tables_dev, ctx_dev,
                                 max_ctx, scale, workspace, partition_tokens, kernel, events,
                                 waves_per_simd=waves_per_simd, xcd_weights=xcd_weights, trace=trace,
                                 load_policy=load_policy, plan=plan)

    def prefill(self, layer: int, out, q, tables_dev, ctx_dev, qstart_dev, max_query_len: int, max_ctx: int,
                scale: float):
        """Causal attention of each sequence's new tokens (already stored)."""
        L.paged_attention_prefill(self.layout, out, q, self.k_pools[layer], self.v_pools[layer], tables_dev, ctx_dev,
                                  qstart_dev, max_query_len, max_ctx, scale)

    def waves_per_simd(self) -> int:
        """Two resident waves per SIMD when the live sequences read their
        blocks more than twice over on average (shared prompts, parallel
        samples): such blocks are served from L2, where more waves in flight
        pay; otherwise one, which streams from HBM fastest."""
        st = self.stats()
        return 2 if st["tokens_stored"] and st["tokens_logical"] > 2 * st["tokens_stored"] else 1

    def workspace(self, num_seqs, num_q_heads, max_ctx, partition_tokens=0, kernel=0):
        nbytes = L.paged_attention_workspace_bytes(self.layout, num_seqs, num_q_heads, max_ctx, partition_tokens,
                                                   kernel)
        return torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=self.device)


def _bits_to_dev(arr: np.ndarray, dtype: str, device):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


class GpuWorkload:
    """A workload instance built on the GPU path: the instance's build script
    run through the host block manager, its prefill and decode-step tokens
    stored by paged_kv_append, and device tables, lengths and query ready for
    paged_attention_decode."""

    def __init__(self, inst, num_layers: int = 1, device="cuda", extra_blocks: int = 0):
        wl = inst.wl
        self.inst, self.wl = inst, wl
        self.device = torch.device(device)
        order = np.concatenate([inst.free_order, np.arange(inst.num_blocks, inst.num_blocks + extra_blocks,
                                                           dtype=np.int32)])
        self.cache = PagedKVCache(inst.num_blocks + extra_blocks, wl.num_kv_heads, wl.head_dim, wl.cache_dtype,
                                  num_layers=num_layers, free_order=order, device=device)
        c = self.cache
        pre = []
        if wl.prefix_len:
            root = c.create()
            s, _ = c.reserve([root], wl.prefix_len)
            pre.append(s)
            self.ids = [root] + [c.fork(root) for _ in range(wl.batch - 1)]
        else:
            self.ids = [c.create() for _ in range(wl.batch)]
        for b, sid in enumerate(self.ids):
            n = int(inst.own_prefill[b])
            if n:
                s, _ = c.reserve([sid], n)
                pre.append(s)
        self.prefill_slots = np.concatenate(pre) if pre else np.zeros(0, np.int64)
        if self.prefill_slots.size:
            slots_dev = torch.from_numpy(self.prefill_slots).to(self.device)
            kpre = _bits_to_dev(inst.prefill_tokens("k"), wl.dtype, self.device)
            vpre = _bits_to_dev(inst.prefill_tokens("v"), wl.dtype, self.device)
            for layer in range(num_layers):
                c.write(layer, slots_dev, kpre, vpre)
            del kpre, vpre
        self.step_slots, _ = c.reserve(self.ids, 1)
        self.step_slots_dev = torch.from_numpy(self.step_slots).to(self.device)
        self.k_step = _bits_to_dev(inst.step_tokens("k"), wl.dtype, self.device)
        self.v_step = _bits_to_dev(inst.step_tokens("v"), wl.dtype, self.device)
        for layer in range(num_layers):
            c.write(layer, self.step_slots_dev, self.k_step, self.v_step)
        self.max_ctx = int(inst.ctx.max())
        self.max_blocks = -(-self.max_ctx // 16)
        tables, ctx = c.tables(self.ids, self.max_blocks)
        self.tables_host, self.ctx_host = tables, ctx
        self.tables_dev = torch.from_numpy(tables).to(self.device)
        self.ctx_dev = torch.from_numpy(ctx).to(self.device)
        self.q = _bits_to_dev(inst.q(), wl.dtype, self.device)
        self.scale = 1.0 / math.sqrt(wl.head_dim)
        self.out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.float32, device=self.device)

    def decode(self, layer=0, partition_tokens=0, kernel=0, events=None, workspace=None, out=None, waves_per_simd=None,
               xcd_weights=None, trace=None, load_policy=0, plan=None):
        """plan: (pkv_decode_plan, buffer) from new_plan(): recorded by the
        first call given it, used by the next ones."""
        if workspace is None:
            workspace = self.cache.workspace(self.wl.batch, self.wl.num_q_heads, self.max_ctx, partition_tokens,
                                             kernel)
        out = self.out if out is None else out
        self.cache.decode(layer, out, self.q, self.tables_dev, self.ctx_dev, self.max_ctx, self.scale, workspace,
                          partition_tokens, kernel, events, waves_per_simd, xcd_weights, trace, load_policy, plan)
        return out

    def new_plan(self, partition_tokens=0):
        return L.new_decode_plan(self.cache.layout, self.wl.batch, self.wl.num_q_heads, self.max_ctx,
                                 partition_tokens, self.device)


class GpuPrefill:
    """A prefill workload instance built on the GPU path: the build script
    through the host block manager, every token (cached prefix and new ones)
    stored by paged_kv_append, and the queries, tables, lengths and query
    offsets on the device for paged_attention_prefill."""

    def __init__(self, inst, num_layers: int = 1, device="cuda"):
        wl = inst.wl
        self.inst, self.wl = inst, wl
        self.device = torch.device(device)
        self.cache = PagedKVCache(inst.num_blocks, wl.num_kv_heads, wl.head_dim, wl.cache_dtype,
                                  num_layers=num_layers, free_order=inst.free_order, device=device)
        c = self.cache

        def put(sid, k, v):
            slots, cow = c.reserve([sid], k.shape[0])
            assert len(cow) == 0
            sd = torch.from_numpy(slots).to(self.device)
            kd, vd = _bits_to_dev(k, wl.dtype, self.device), _bits_to_dev(v, wl.dtype, self.device)
            for layer in range(num_layers):
                c.write(layer, sd, kd, vd)
            return slots

        if wl.shared_prefix:
            root = c.create()
            put(root, inst.shared_kv("k"), inst.shared_kv("v"))
            self.ids = [root] + [c.fork(root) for _ in range(wl.batch - 1)]
        else:
            self.ids = [c.create() for _ in range(wl.batch)]
        new_slots = []
        for b, sid in enumerate(self.ids):
            new_slots.append(put(sid, inst.own_kv(b, "k"), inst.own_kv(b, "v"))[-int(inst.nq[b]):])
        # The new tokens' slots and rows: a prefill step stores them, then attends.
        self.new_slots_dev = torch.from_numpy(np.concatenate(new_slots)).to(self.device)
        self.k_new = _bits_to_dev(np.concatenate([inst.own_kv(b, "k")[-int(inst.nq[b]):] for b in range(wl.batch)]),
                                  wl.dtype, self.device)
        self.v_new = _bits_to_dev(np.concatenate([inst.own_kv(b, "v")[-int(inst.nq[b]):] for b in range(wl.batch)]),
                                  wl.dtype, self.device)
        self.max_ctx = int(inst.ctx.max())
        self.max_q = int(inst.nq.max())
        tables, ctx = c.tables(self.ids, -(-self.max_ctx // 16))
        self.tables_host = tables
        self.tables_dev = torch.from_numpy(tables).to(self.device)
        self.ctx_dev = torch.from_numpy(ctx).to(self.device)
        self.qstart_dev = torch.from_numpy(inst.qstart).to(self.device)
        self.q = _bits_to_dev(inst.q(), wl.dtype, self.device)
        self.scale = 1.0 / math.sqrt(wl.head_dim)
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device=self.device)

    def run(self, layer=0, out=None):
        out = self.out if out is None else out
        self.cache.prefill(layer, out, self.q, self.tables_dev, self.ctx_dev, self.qstart_dev, self.max_q, self.max_ctx,
                           self.scale)
        return out
