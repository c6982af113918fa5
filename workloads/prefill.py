"""Prefill workloads and their seeded inputs.

A prefill computes the causal attention of a prompt's new tokens; tokens of
a prefix already in the cache are attended to but not recomputed (ch.15
"KV Cache 工程学" §15.1, §15.6; ch.8 "新一代 KV Cache 管理" §8.3).  Shapes
follow the decode workloads: Llama-3-8B grouped-query heads, 16-token blocks,
a shared system prompt of 2000 tokens.

How an instance is built, identically on both sides of a parity test:

* ``shared_prefix > 0``: sequence 0 is created and the ``shared_prefix``
  tokens are appended; sequences 1..B-1 are forks of it (the prefix blocks
  are shared; ``shared_prefix`` is a multiple of 16 in the named workloads).
* Every sequence b then appends, in batch order, ``own[b]`` tokens: a
  private cached part of ``own_prefix[b]`` tokens followed by ``nq[b]`` new
  tokens.  Its context is ``ctx[b] = shared_prefix + own[b]``; the query rows
  of its new tokens are ``qstart[b] .. qstart[b+1]-1``.

Values are N(0, 1) float32 draws from seeded CPU generators, rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import BLOCK, derive_seed, normal_bits


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    number: int                 # seed 2000 + number
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str = "bf16"         # queries and K/V rows handed to append
    cache: str = ""             # "" = dtype, or "int8" / "fp8"
    shared_prefix: int = 0      # cached tokens held once by every sequence
    own_prefix: tuple = (0, 0)  # private cached tokens per sequence: inclusive range
    new_tokens: tuple = (1, 1)  # new tokens per sequence: inclusive range
    same_data_as: str = ""      # draw lengths, order and values as the named workload does
    description: str = ""

    @property
    def cache_dtype(self) -> str:
        return self.cache or self.dtype

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def data_name(self) -> str:
        return self.same_data_as or self.name

    def instantiate(self) -> "PrefillInstance":
        rng = np.random.default_rng(derive_seed(2000 + self.number, self.data_name, "lens"))
        B = self.batch
        own_prefix = rng.integers(self.own_prefix[0], self.own_prefix[1] + 1, size=B).astype(np.int32)
        nq = rng.integers(self.new_tokens[0], self.new_tokens[1] + 1, size=B).astype(np.int32)
        ctx = (self.shared_prefix + own_prefix + nq).astype(np.int32)
        demand = -(-self.shared_prefix // BLOCK) + int(sum(-(-int(n) // BLOCK) + 1 for n in own_prefix + nq))
        num_blocks = int(np.ceil(1.25 * demand)) + 4
        perm = np.random.default_rng(derive_seed(2000 + self.number, self.data_name, "perm")).permutation(
            num_blocks).astype(np.int32)
        return PrefillInstance(self, ctx, own_prefix, nq, num_blocks, perm)


@dataclass
class PrefillInstance:
    wl: PrefillWorkload
    ctx: np.ndarray          # int32 [B] tokens held after the new ones are stored
    own_prefix: np.ndarray   # int32 [B] private cached tokens
    nq: np.ndarray           # int32 [B] new tokens (queries)
    num_blocks: int
    free_order: np.ndarray
    _cache: dict = field(default_factory=dict, repr=False)

    @property
    def qstart(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.nq)]).astype(np.int32)

    def _seed(self, *names) -> int:
        return derive_seed(2000 + self.wl.number, self.wl.data_name, *names)

    def shared_kv(self, which: str) -> np.ndarray:
        w = self.wl
        key = ("shared", which)
        if key not in self._cache:
            self._cache[key] = normal_bits(self._seed(which, "shared"), (w.shared_prefix, w.num_kv_heads, w.head_dim),
                                           w.dtype)
        return self._cache[key]

    def own_kv(self, b: int, which: str) -> np.ndarray:
        """[own_prefix[b] + nq[b]][h_kv][d] values sequence b appends itself."""
        w = self.wl
        key = ("own", which, b)
        if key not in self._cache:
            n = int(self.own_prefix[b] + self.nq[b])
            self._cache[key] = normal_bits(self._seed(which, "own", b), (n, w.num_kv_heads, w.head_dim), w.dtype)
        return self._cache[key]

    def seq_kv(self, b: int, which: str) -> np.ndarray:
        """[ctx[b]][h_kv][d] logical K or V of sequence b."""
        own = self.own_kv(b, which)
        return np.concatenate([self.shared_kv(which), own], axis=0) if self.wl.shared_prefix else own

    def q(self) -> np.ndarray:
        """[T][h_q][d] queries of the new tokens, sequence by sequence."""
        w = self.wl
        if "q" not in self._cache:
            self._cache["q"] = normal_bits(self._seed("q"), (int(self.nq.sum()), w.num_q_heads, w.head_dim), w.dtype)
        return self._cache["q"]

    def flops(self) -> int:
        """Multiply-adds x 2 of both products: every new token t of sequence b
        scores and weights ctx[b] - nq[b] + t + 1 keys for each query head."""
        w = self.wl
        keys = sum(int(self.ctx[b] - self.nq[b]) * int(self.nq[b]) + int(self.nq[b]) * (int(self.nq[b]) + 1) // 2
                   for b in range(w.batch))
        return 4 * w.head_dim * w.num_q_heads * keys

    def kv_bytes(self) -> int:
        """Distinct K/V bytes the tokens attended to occupy (shared prefix once)."""
        w = self.wl
        row = w.head_dim + 4 if w.cache_dtype in ("int8", "fp8") else w.head_dim * 2
        return (w.shared_prefix + int((self.own_prefix + self.nq).sum())) * 2 * w.num_kv_heads * row


PREFILL_WORKLOADS = {
    "prefill_shared_prefix": PrefillWorkload(
        "prefill_shared_prefix", 1, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        shared_prefix=2000, new_tokens=(512, 512),
        description="prefill of 16 prompts of 512 new tokens after a cached 2000-token system prompt held once, "
                    "Llama-3-8B heads, bf16"),
    "prefill_shared_prefix_int8": PrefillWorkload(
        "prefill_shared_prefix_int8", 1, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, cache="int8",
        shared_prefix=2000, new_tokens=(512, 512), same_data_as="prefill_shared_prefix",
        description="prefill_shared_prefix on an int8 cache: the same lengths and bf16 rows, quantised on append"),
    "prefill_shared_prefix_fp8": PrefillWorkload(
        "prefill_shared_prefix_fp8", 1, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, cache="fp8",
        shared_prefix=2000, new_tokens=(512, 512), same_data_as="prefill_shared_prefix",
        description="prefill_shared_prefix on an FP8 E4M3 cache: the same lengths and bf16 rows, quantised on append"),
    "prefill_8b_b4": PrefillWorkload(
        "prefill_8b_b4", 2, batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, new_tokens=(2048, 2048),
        description="prefill of 4 prompts of 2048 new tokens, no cached prefix, Llama-3-8B heads, bf16"),
}


def get(name: str) -> PrefillInstance:
    return PREFILL_WORKLOADS[name].instantiate()


def scaled(name: str, **overrides) -> PrefillWorkload:
    import dataclasses
    return dataclasses.replace(PREFILL_WORKLOADS[name], **overrides)
