"""The five decode workloads and their seeded inputs.

Shapes follow the workloads the pages discuss: Llama-3-8B / 70B grouped-query
head shapes and 16-token blocks (ch.15 "KV Cache 工程学" §15.2, §15.5), 4K
contexts (§15.3), shared system prompts of a few thousand tokens (§15.6),
best-of-8 sampling over a 2000-token prompt (ch.8 "新一代 KV Cache 管理" §8.1)
and attention-sink tokens at the start of long contexts (§8.2).

How a workload is built, identically on both sides of a parity test:

* ``prefix_len == 0``: one sequence per batch row is created and
  ``own_prefill[b] = ctx[b] - 1`` tokens are appended to it (batch order).
* ``prefix_len > 0``: sequence 0 is created and ``prefix_len`` tokens are
  appended; sequences 1..B-1 are forks of sequence 0; then each sequence
  appends ``own_prefill[b] = ctx[b] - prefix_len - 1`` private tokens.
* The decode step then appends one token to every sequence (batch order) and
  attends over ``ctx[b]`` tokens.

Token values: the token at logical position ``p`` of sequence ``b`` carries
``prefix_k[p]`` when ``p < prefix_len`` and ``own_k(b)[p - prefix_len]``
otherwise (likewise V).  Values are N(0, 1) float32 draws from a seeded CPU
``torch.Generator`` (thread-count invariant), rounded to bf16 by round to
nearest even where the workload is bf16.  Sinks multiply K and V of logical
positions ``< sinks`` by ``sink_scale`` (exact in bf16).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 16  # tokens per KV block in every workload


def derive_seed(base: int, *names) -> int:
    """Stable 63-bit seed for a named sub-stream of a workload seed."""
    key = "/".join(str(x) for x in (base,) + names).encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little") & ((1 << 63) - 1)


def normal_bits(seed: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws as raw element bits: uint16 (bf16) or float32."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return x.numpy()
    raise ValueError(dtype)


def _scale_exact(bits: np.ndarray, dtype: str, factor: float) -> np.ndarray:
    """Multiply stored elements by a power of two (exact for these ranges)."""
    if dtype == "f32":
        return bits * np.float32(factor)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return (t * factor).view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    number: int                  # 1..5; the seed is 1000 + number
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                   # "f32" | "bf16": queries and the K/V rows handed to append
    ctx_fixed: tuple = ()        # explicit context lengths, or
    ctx_range: tuple = ()        # (lo, hi) inclusive uniform integers
    prefix_len: int = 0          # tokens shared by every sequence (held once)
    suffix_fixed: int = 0        # private tokens per sequence after the prefix, or
    suffix_range: tuple = ()     # (lo, hi) inclusive uniform integers
    pool_blocks: int = 0         # explicit pool size, else ceil(1.25 x demand)
    sinks: int = 0
    sink_scale: float = 4.0
    shuffled: bool = True        # blocks handed out in a seeded random order, else 0, 1, 2, ...
    cache: str = ""              # storage of the cache: "" = dtype, or "int8" / "fp8" (codes + per-token scales)
    same_data_as: str = ""       # draw lengths, order and values as the named workload does
    description: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def cache_dtype(self) -> str:
        return self.cache or self.dtype

    @property
    def data_name(self) -> str:
        return self.same_data_as or self.name

    @property
    def row_bytes(self) -> int:
        """Cache bytes of one token's K (or V) row of one kv head: an int8 or
        FP8 cache keeps a float32 scale beside its d one-byte codes."""
        if self.cache_dtype in ("int8", "fp8"):
            return self.head_dim + 4
        return self.head_dim * self.elem_bytes

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def instantiate(self) -> "Instance":
        rng = np.random.default_rng(derive_seed(self.seed, self.data_name, "lens"))
        B = self.batch
        if self.prefix_len:
            if self.suffix_range:
                lo, hi = self.suffix_range
                suffix = rng.integers(lo, hi + 1, size=B).astype(np.int64)
            else:
                suffix = np.full(B, self.suffix_fixed, dtype=np.int64)
            ctx = self.prefix_len + suffix
        elif self.ctx_fixed:
            ctx = np.asarray(self.ctx_fixed, dtype=np.int64)
            assert ctx.size == B
        else:
            lo, hi = self.ctx_range
            ctx = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        own_prefill = ctx - self.prefix_len - 1
        assert (own_prefill >= 0).all()
        # Demand counts shared prefix blocks once (pool sizing only).
        demand = -(-self.prefix_len // BLOCK) + int(sum(-(-int(n) // BLOCK) for n in (ctx - self.prefix_len)))
        num_blocks = self.pool_blocks or int(np.ceil(1.25 * demand))
        if self.shuffled:
            perm = np.random.default_rng(derive_seed(self.seed, self.data_name, "perm")).permutation(num_blocks).astype(np.int32)
        else:
            perm = np.arange(num_blocks, dtype=np.int32)
        return Instance(self, ctx.astype(np.int32), own_prefill.astype(np.int32), num_blocks, perm)


@dataclass
class Instance:
    """One seeded draw of a workload: lengths, block hand-out order, values."""
    wl: Workload
    ctx: np.ndarray            # int32 [B]: tokens attended after the step's append
    own_prefill: np.ndarray    # int32 [B]: private tokens appended before the step
    num_blocks: int
    free_order: np.ndarray     # int32 [num_blocks]: order blocks are handed out
    _cache: dict = field(default_factory=dict, repr=False)

    # -- values ---------------------------------------------------------------
    def q(self) -> np.ndarray:
        """[B][h_q][d] query of the decode step."""
        w = self.wl
        if "q" not in self._cache:
            self._cache["q"] = normal_bits(derive_seed(w.seed, w.data_name, "q"), (w.batch, w.num_q_heads, w.head_dim), w.dtype)
        return self._cache["q"]

    def _sinked(self, arr: np.ndarray, start_pos: int) -> np.ndarray:
        w = self.wl
        if w.sinks and start_pos < w.sinks:
            n = min(w.sinks - start_pos, arr.shape[0])
            arr = arr.copy()
            arr[:n] = _scale_exact(arr[:n], w.dtype, w.sink_scale)
        return arr

    def prefix_kv(self, which: str) -> np.ndarray:
        """[prefix_len][h_kv][d] values of the shared prefix tokens."""
        w = self.wl
        key = "prefix_" + which
        if key not in self._cache:
            a = normal_bits(derive_seed(w.seed, w.data_name, which, "prefix"), (w.prefix_len, w.num_kv_heads, w.head_dim), w.dtype)
            self._cache[key] = self._sinked(a, 0)
        return self._cache[key]

    def own_kv(self, b: int, which: str) -> np.ndarray:
        """[ctx[b]-prefix_len][h_kv][d] values of sequence b's private tokens
        (cached: the prefill and the decode step both read them)."""
        w = self.wl
        key = ("own", which, b)
        if key not in self._cache:
            n = int(self.ctx[b]) - w.prefix_len
            a = normal_bits(derive_seed(w.seed, w.data_name, which, "own", b), (n, w.num_kv_heads, w.head_dim), w.dtype)
            self._cache[key] = self._sinked(a, w.prefix_len)
        return self._cache[key]

    def drop_cache(self):
        self._cache.clear()

    def seq_kv(self, b: int, which: str) -> np.ndarray:
        """[ctx[b]][h_kv][d] logical K or V of sequence b (all its tokens)."""
        own = self.own_kv(b, which)
        if self.wl.prefix_len == 0:
            return own
        return np.concatenate([self.prefix_kv(which), own], axis=0)

    # -- the token lists the build script appends, in order -------------------
    def prefill_tokens(self, which: str) -> np.ndarray:
        """Values of every token appended before the decode step, in append
        order: the shared prefix (if any), then each sequence's private
        prefill in batch order.  Shape [T][h_kv][d]."""
        w = self.wl
        parts = []
        if w.prefix_len:
            parts.append(self.prefix_kv(which))
        for b in range(w.batch):
            n = int(self.own_prefill[b])
            if n:
                parts.append(self.own_kv(b, which)[:n])
        if not parts:
            shape = (0, w.num_kv_heads, w.head_dim)
            return np.zeros(shape, dtype=np.float32 if w.dtype == "f32" else np.uint16)
        return np.concatenate(parts, axis=0)

    def step_tokens(self, which: str) -> np.ndarray:
        """Values of the token each sequence appends in the decode step
        (its last logical position).  Shape [B][h_kv][d]."""
        return np.stack([self.own_kv(b, which)[-1] for b in range(self.wl.batch)], axis=0)

    def kv_bytes_logical(self) -> int:
        """K and V bytes the decode step reads: every sequence's whole context."""
        w = self.wl
        return int(self.ctx.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.row_bytes

    def kv_bytes_unique(self) -> int:
        """K and V bytes of distinct stored tokens (a shared prefix counts once)."""
        w = self.wl
        tokens = int(self.ctx.astype(np.int64).sum()) - (w.batch - 1) * w.prefix_len
        return tokens * 2 * w.num_kv_heads * w.row_bytes


WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", 1, batch=4, num_q_heads=4, num_kv_heads=4, head_dim=64, dtype="f32",
        ctx_fixed=(1, 17, 100, 255), pool_blocks=64,
        description="tiny fp32 paged decode: 4 seqs, 4 q = 4 kv heads, d 64, 64-block shuffled pool, ctx {1,17,100,255}"),
    "llama3_8b_b64": Workload(
        "llama3_8b_b64", 2, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        ctx_range=(128, 4096),
        description="Llama-3-8B-shaped single-layer decode: B 64, 32 q / 8 kv heads, d 128, bf16, ctx U[128,4096], shuffled pool 1.25x demand"),
    "llama3_8b_b64_int8": Workload(
        "llama3_8b_b64_int8", 2, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        ctx_range=(128, 4096), cache="int8", same_data_as="llama3_8b_b64",
        description="llama3_8b_b64 with an int8 cache: the same lengths, order and bf16 rows, quantised "
                    "on append to int8 codes with a float32 scale per token and kv head"),
    "llama3_8b_b64_fp8": Workload(
        "llama3_8b_b64_fp8", 2, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        ctx_range=(128, 4096), cache="fp8", same_data_as="llama3_8b_b64",
        description="llama3_8b_b64 with an FP8 E4M3 cache: the same lengths, order and bf16 rows, quantised "
                    "on append to E4M3 codes with a float32 scale per token and kv head"),
    "llama3_70b_b256": Workload(
        "llama3_70b_b256", 3, batch=256, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16",
        ctx_fixed=(4096,) * 256,
        description="Llama-3-70B-shaped single-layer decode: B 256, 64 q / 8 kv heads, d 128, bf16, ctx 4096, shuffled pool 1.25x demand"),
    "llama3_70b_b256_int8": Workload(
        "llama3_70b_b256_int8", 3, batch=256, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16",
        ctx_fixed=(4096,) * 256, cache="int8", same_data_as="llama3_70b_b256",
        description="llama3_70b_b256 with an int8 cache: the same lengths, order and bf16 rows, quantised "
                    "on append to int8 codes with a float32 scale per token and kv head"),
    "shared_prefix_b128": Workload(
        "shared_prefix_b128", 4, batch=128, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        prefix_len=2000, suffix_range=(16, 512),
        description="shared-prefix decode: 128 seqs share one 2000-token prefix held once, private suffixes U[16,512], Llama-3-8B heads, bf16"),
    "best_of_8": Workload(
        "best_of_8", 4, batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        prefix_len=2000, suffix_fixed=100,
        description="best-of-8 decode over a shared 2000-token prompt with 100-token private tails, Llama-3-8B heads, bf16"),
    "mha_long": Workload(
        "mha_long", 5, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128, dtype="bf16",
        ctx_fixed=(1024, 4096, 8192, 16384, 32768, 32768, 20000, 12345), pool_blocks=9968, sinks=4,
        description="long-context MHA decode: B 8, 32 q = 32 kv heads, d 128, bf16, ctx up to 32768, 4 sink positions x4"),
}


def get(name: str) -> Instance:
    return WORKLOADS[name].instantiate()


def scaled(name: str, **overrides) -> Workload:
    """A copy of a named workload with some fields replaced (small parity cases)."""
    import dataclasses
    return dataclasses.replace(WORKLOADS[name], **overrides)
