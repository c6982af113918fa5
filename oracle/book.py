"""Oracle model of the KV block manager (plain Python, slow, obviously correct).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.
It shares no code with the HIP library and never calls it.

What it follows:

* The physical KV cache is cut into fixed 16-token blocks held in one flat
  pool; a sequence owns a block table whose entry i names the physical block
  of its i-th logical block; a new block is taken only when the current one
  is full; a finished sequence hands every block back to the free pool
  [KV Cache 工程学 §15.5; 新一代 KV Cache 管理 §8.1].
* Several block tables may name the same physical block; each block carries
  a reference count [新一代 KV Cache 管理 §8.1], and sharing of a common
  prompt uses copy-on-write [KV Cache 与 PagedAttention, "PagedAttention
  如何解决这个问题"].

Readings where the pages are silent (each one is listed in the design notes):

* free pool = a LIFO stack seeded so that the first allocation returns
  ``free_order[0]``; a freed block is pushed on top;
* a sequence being freed releases its blocks in table order;
* copy-on-write fires only when a token is written into a tail block whose
  reference count is above one: a fresh block is taken, the pair
  (old, new) is reported for a whole-block copy, the old block loses one
  reference and the table points at the new block; the last holder of a
  block writes in place;
* an append reserves all of its tokens or none (state unchanged on
  failure); a batch append is all-or-nothing over the whole batch;
* sequence ids are handed out 0, 1, 2, ... and never reused.
* prefix cache [KV Cache 工程学 §15.6; 新一代 KV Cache 管理 §8.3]: only full
  blocks are cached; a block is identified by the whole token prefix that
  ends with it (here the exact tuple of token ids; the library hashes it);
  a request points its table at the longest run of cached blocks that
  begins its prompt and stops at the first miss; registration after the
  prefill adds the prompt's full blocks whose content is not cached yet; a
  cached block held by no sequence stays cached ("idle") and is taken, least
  recently used first, only when the free stack is empty; a sequence's
  cached blocks that turn idle together enter the LRU deepest first; turning
  the cache off returns idle blocks to the free stack, oldest first.
* swap to host memory ("fine-grained eviction": small pages move to the CPU
  instead of whole sequences [KV Cache 与 PagedAttention, summary]; Clock
  replacement [PagedAttention：大模型KV Cache内存管理革新 §3.3]): host memory
  holds ``num_host`` block slots, handed out from a LIFO stack seeded
  0, 1, 2, ...; every device block has a reference bit, set when the block is
  taken, when a token slot in it is assigned and when a batch's tables naming
  it are exported for a device call; ``swap_out(want, protect)`` moves the Clock hand over device block
  ids from where it stopped: a block held by some sequence, not in the prefix
  cache and not held by a protected sequence is a candidate; a candidate whose
  bit is set has it cleared and is passed over, one whose bit is clear is
  swapped out (a host slot is taken, every table entry naming the block
  becomes ``-(slot + 1)``, the block's references move to the slot and the
  block goes back to the free stack); it stops after ``want`` victims, when
  host slots run out, or after two turns of the hand; ``swap_in(seq)`` brings
  back every host entry of a sequence in table order, all or nothing, each
  into a freshly taken block (sharers follow); a sequence holding host
  entries cannot append or export its table.

Parity unpinned items: none; every behaviour here is checked by the
invariant and worked-number tests in ``tests/test_oracle_book.py`` and
``tests/test_prefix_cache.py`` (the pages' two-user example).
"""
from __future__ import annotations


BLOCK_SIZE = 16


class BookError(Exception):
    """Raised with a ``code`` matching the library's status names."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class Book:
    def __init__(self, num_blocks: int, free_order=None):
        if num_blocks <= 0:
            raise BookError("INVALID", "num_blocks must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BookError("INVALID", "free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.free = order[::-1]          # top of the stack is the list's end
        self.ref = [0] * num_blocks
        self.seqs = {}                   # id -> {"table": [...], "len": n}
        self.next_id = 0
        # Prefix cache: exact keys (the whole token prefix ending with a full
        # block), an idle list of cached blocks held by no sequence (oldest
        # first) and counters.
        self.pc_on = False
        self.pc = {}                     # key tuple -> block
        self.key_of = {}                 # block -> key tuple
        self.lru = []
        self.pst = {"lookups": 0, "query_tokens": 0, "hit_tokens": 0, "registered": 0, "evictions": 0}
        # Host swap space and the Clock state.
        self.refbit = [0] * num_blocks
        self.hand = 0
        self.num_host = 0
        self.host_free = []
        self.host_ref = []
        self.sst = {"swapped_out": 0, "swapped_in": 0}

    # -- blocks ---------------------------------------------------------------
    def alloc(self) -> int:
        """The top of the free stack, else the least recently used idle
        cached block, which leaves the cache."""
        if self.free:
            blk = self.free.pop()
        elif self.lru:
            blk = self.lru.pop(0)
            del self.pc[self.key_of.pop(blk)]
            self.pst["evictions"] += 1
        else:
            raise BookError("NO_BLOCKS", "pool exhausted")
        self.ref[blk] = 1
        self.refbit[blk] = 1
        return blk

    def _check(self, blk: int):
        if not (0 <= blk < self.num_blocks):
            raise BookError("BAD_BLOCK", str(blk))

    def incref(self, blk: int):
        self._check(blk)
        if self.ref[blk] <= 0:
            raise BookError("REFCOUNT", f"incref of free block {blk}")
        self.ref[blk] += 1

    def decref(self, blk: int):
        self._check(blk)
        if self.ref[blk] <= 0:
            raise BookError("REFCOUNT", f"free of free block {blk}")
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self._release(blk)

    def _release(self, blk: int):
        if blk in self.key_of:
            self.lru.append(blk)
        else:
            self.free.append(blk)

    def refcount(self, blk: int) -> int:
        self._check(blk)
        return self.ref[blk]

    def num_free(self) -> int:
        """Blocks that can be handed out: free, or idle in the prefix cache."""
        return len(self.free) + len(self.lru)

    # -- sequences ------------------------------------------------------------
    def _seq(self, sid: int):
        if sid not in self.seqs:
            raise BookError("BAD_SEQ", str(sid))
        return self.seqs[sid]

    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"table": [], "len": 0}
        return sid

    def fork(self, parent: int) -> int:
        p = self._seq(parent)
        for blk in p["table"]:  # a table naming a freed block is corrupt: refuse before changing anything
            if blk >= 0 and self.ref[blk] <= 0:
                raise BookError("REFCOUNT", f"fork of a sequence holding free block {blk}")
        for blk in p["table"]:
            if blk >= 0:
                self.incref(blk)
            else:
                self.host_ref[-blk - 1] += 1
        sid = self.create()
        self.seqs[sid] = {"table": list(p["table"]), "len": p["len"]}
        return sid

    def _append_one_seq(self, sid: int, n: int, slots: list, cow: list):
        s = self._seq(sid)
        for _ in range(n):
            pos = s["len"]
            if pos % BLOCK_SIZE == 0:
                s["table"].append(self.alloc())
            elif self.ref[s["table"][-1]] > 1:
                old = s["table"][-1]
                new = self.alloc()
                cow.append((old, new))
                self.decref(old)
                s["table"][-1] = new
            blk = s["table"][pos // BLOCK_SIZE]
            self.refbit[blk] = 1
            slots.append(blk * BLOCK_SIZE + pos % BLOCK_SIZE)
            s["len"] = pos + 1

    def append_slots(self, sid: int, n: int):
        """Reserve n token slots at the end of sequence sid.
        Returns (slots, cow_pairs); all-or-nothing."""
        return self.batch_append_slots([sid], n)

    def batch_append_slots(self, sids, n: int):
        """Reserve n slots for each sequence of the batch, in batch order."""
        if n < 0:
            raise BookError("INVALID", "negative token count")
        for sid in sids:
            self._seq(sid)
        for sid in sids:
            if not self.resident(sid):
                raise BookError("INVALID", f"sequence {sid} has blocks swapped out")
        # Appending changes the appended sequences' own entries and the block
        # containers below, nothing else: the snapshot for the undo is exactly
        # that (keys and counters are immutable values, so shallow copies do).
        saved = (list(self.free), list(self.ref), dict(self.pc), dict(self.key_of), list(self.lru),
                 dict(self.pst), list(self.refbit),
                 {sid: {"table": list(self.seqs[sid]["table"]), "len": self.seqs[sid]["len"]} for sid in sids})
        slots, cow = [], []
        try:
            for sid in sids:
                self._append_one_seq(sid, n, slots, cow)
        except BookError:
            self.free, self.ref, self.pc, self.key_of, self.lru, self.pst, self.refbit, seqs = saved
            self.seqs.update(seqs)
            raise
        return slots, cow

    def free_seq(self, sid: int):
        s = self._seq(sid)
        # Refuse before changing anything when some block has fewer references
        # than the table holds it (possible only after a caller freed a block
        # the sequence still held): the release is all or nothing.
        held = {}
        for blk in s["table"]:
            if blk >= 0:
                held[blk] = held.get(blk, 0) + 1
        for blk, k in held.items():
            if self.ref[blk] < k:
                raise BookError("REFCOUNT", f"free of a sequence holding block {blk} {k} times, refcount {self.ref[blk]}")
        # Blocks reaching zero go back in table order; cached ones turn idle
        # deepest first (of a prefix released together, the tail is evicted
        # before the head: a cached block is reachable only through its prefix).
        idle = []
        for blk in s["table"]:
            if blk < 0:
                slot = -blk - 1
                self.host_ref[slot] -= 1
                if self.host_ref[slot] == 0:
                    self.host_free.append(slot)
                continue
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                if blk in self.key_of:
                    idle.append(blk)
                else:
                    self.free.append(blk)
        self.lru.extend(reversed(idle))
        del self.seqs[sid]

    # -- prefix cache [KV Cache 工程学 §15.6; 新一代 KV Cache 管理 §8.3] ----------
    def enable_prefix_cache(self, on: bool):
        if not on and self.pc_on:
            while self.lru:
                self.free.append(self.lru.pop(0))
            self.pc.clear()
            self.key_of.clear()
        self.pc_on = bool(on)

    def create_from_prefix(self, tokens):
        """New sequence pointing at the longest run of cached full blocks that
        begins the prompt; returns (id, tokens found cached)."""
        sid = self.create()
        s = self.seqs[sid]
        if self.pc_on:
            for i in range(len(tokens) // BLOCK_SIZE):
                blk = self.pc.get(tuple(tokens[:BLOCK_SIZE * (i + 1)]))
                if blk is None:
                    break
                if self.ref[blk] == 0:
                    self.lru.remove(blk)
                self.ref[blk] += 1
                s["table"].append(blk)
                s["len"] += BLOCK_SIZE
            self.pst["lookups"] += 1
            self.pst["query_tokens"] += len(tokens) // BLOCK_SIZE * BLOCK_SIZE
            self.pst["hit_tokens"] += s["len"]
        return sid, s["len"]

    def register_prefix(self, sid: int, tokens, n: int) -> int:
        """Cache the full blocks of the first n tokens of sequence sid (whose
        K/V are stored); content already cached is left alone."""
        s = self._seq(sid)
        if n < 0 or n > s["len"]:
            raise BookError("INVALID", "register beyond the sequence")
        added = 0
        if self.pc_on:
            for i in range(n // BLOCK_SIZE):
                key = tuple(tokens[:BLOCK_SIZE * (i + 1)])
                blk = s["table"][i]
                if blk < 0:  # swapped out: the cache names device blocks only
                    break
                if key in self.pc or blk in self.key_of:
                    continue
                self.pc[key] = blk
                self.key_of[blk] = key
                added += 1
            self.pst["registered"] += added
        return added

    def prefix_stats(self) -> dict:
        st = dict(self.pst)
        st["cached_blocks"] = len(self.pc)
        st["idle_blocks"] = len(self.lru)
        st["hit_rate"] = st["hit_tokens"] / st["query_tokens"] if st["query_tokens"] else 0.0
        return st

    def seq_len(self, sid: int) -> int:
        return self._seq(sid)["len"]

    def block_table(self, sid: int):
        """The table as stored (host entries as -(slot + 1))."""
        return list(self._seq(sid)["table"])

    def export_tables(self, sids):
        """Tables and lengths of a batch for a device call (every sequence
        must be resident); sets the reference bits of the blocks named."""
        for sid in sids:
            self._seq(sid)
        for sid in sids:
            if not self.resident(sid):
                raise BookError("INVALID", f"sequence {sid} has blocks swapped out")
        tables = [self.block_table(sid) for sid in sids]
        for t in tables:
            for blk in t:
                self.refbit[blk] = 1
        return tables, [self.seq_len(sid) for sid in sids]

    # -- swap to host memory -----------------------------------------------
    def resident(self, sid: int) -> bool:
        return all(blk >= 0 for blk in self._seq(sid)["table"])

    def configure_swap(self, num_host: int):
        if num_host < 0:
            raise BookError("INVALID", "negative host slot count")
        if any(r > 0 for r in self.host_ref):
            raise BookError("INVALID", "host slots in use")
        self.num_host = num_host
        self.host_free = list(range(num_host))[::-1]
        self.host_ref = [0] * num_host

    def swap_out(self, want: int, protect=()):
        """Clock victims: list of (device block, host slot) to copy out."""
        if want < 0:
            raise BookError("INVALID", "negative count")
        for sid in protect:
            self._seq(sid)
        guarded = {blk for sid in protect for blk in self.seqs[sid]["table"] if blk >= 0}
        entries = {}
        for q in self.seqs.values():
            for blk in q["table"]:
                if blk >= 0:
                    entries[blk] = entries.get(blk, 0) + 1
        # Candidates: blocks named by some table whose every reference is a
        # table entry.  A block also held by the caller (pkv_block_alloc or
        # pkv_block_incref) stays: the caller's id must keep naming it.
        named = {blk for blk, k in entries.items() if self.ref[blk] == k}
        pairs = []
        examined = 0
        while len(pairs) < want and self.host_free and examined < 2 * self.num_blocks:
            blk = self.hand
            self.hand = (self.hand + 1) % self.num_blocks
            examined += 1
            if blk not in named or blk in self.key_of or blk in guarded:
                continue
            if self.refbit[blk]:
                self.refbit[blk] = 0
                continue
            slot = self.host_free.pop()
            self.host_ref[slot] = self.ref[blk]
            for s in self.seqs.values():
                s["table"] = [-(slot + 1) if b == blk else b for b in s["table"]]
            self.ref[blk] = 0
            self.free.append(blk)
            named.discard(blk)  # free now: a second turn of the hand passes it over
            pairs.append((blk, slot))
        self.sst["swapped_out"] += len(pairs)
        return pairs

    def swap_in(self, sid: int):
        """Every host entry of sequence sid back on the device, in table
        order: list of (host slot, device block) to copy in."""
        s = self._seq(sid)
        slots = []
        for blk in s["table"]:
            if blk < 0 and -blk - 1 not in slots:
                slots.append(-blk - 1)
        if len(slots) > self.num_free():
            raise BookError("NO_BLOCKS", "not enough device blocks to swap in")
        pairs = []
        for slot in slots:
            blk = self.alloc()
            self.ref[blk] = self.host_ref[slot]
            self.host_ref[slot] = 0
            self.host_free.append(slot)
            for q in self.seqs.values():
                q["table"] = [blk if b == -(slot + 1) else b for b in q["table"]]
            pairs.append((slot, blk))
        self.sst["swapped_in"] += len(pairs)
        return pairs

    def check_invariants(self):
        """Every block is in exactly one of: free stack, idle cache list,
        held (refcount > 0); refcounts equal table references plus loose
        ones; host slots likewise."""
        assert len(set(self.free)) == len(self.free), "block twice on the free stack"
        assert len(set(self.lru)) == len(self.lru)
        held = {b for b in range(self.num_blocks) if self.ref[b] > 0}
        assert not (set(self.free) & set(self.lru)) and not (held & (set(self.free) | set(self.lru)))
        assert len(self.free) + len(self.lru) + len(held) == self.num_blocks
        counts = {}
        for q in self.seqs.values():
            for e in q["table"]:
                counts[e] = counts.get(e, 0) + 1
        for e, k in counts.items():
            if e >= 0:
                assert self.ref[e] >= k, (e, self.ref[e], k)
            else:
                assert self.host_ref[-e - 1] == k, (e, self.host_ref[-e - 1], k)
        assert len(set(self.host_free)) == len(self.host_free)
        used = {i for i, r in enumerate(self.host_ref) if r > 0}
        assert not (used & set(self.host_free)) and len(used) + len(self.host_free) == self.num_host

    def swap_stats(self) -> dict:
        used = sum(1 for r in self.host_ref if r > 0)
        return {"host_blocks": self.num_host, "host_used": used, "host_free": len(self.host_free),
                "swapped_out": self.sst["swapped_out"], "swapped_in": self.sst["swapped_in"], "clock_hand": self.hand}

    # -- statistics -----------------------------------------------------------
    def stats(self) -> dict:
        used = self.num_blocks - self.num_free()
        shared = sum(1 for r in self.ref if r > 1)
        logical = sum(s["len"] for s in self.seqs.values())
        # A block's fill is the largest number of its slots any holder uses.
        fill = {}
        for s in self.seqs.values():
            for j, blk in enumerate(s["table"]):
                if blk < 0:  # on the host: not stored on the device
                    continue
                f = min(BLOCK_SIZE, s["len"] - j * BLOCK_SIZE)
                fill[blk] = max(fill.get(blk, 0), f)
        stored = sum(fill.values())
        return {
            "num_blocks": self.num_blocks,
            "num_free": self.num_free(),
            "num_used": used,
            "num_shared": shared,
            "num_seqs": len(self.seqs),
            "tokens_logical": logical,
            "tokens_stored": stored,
            "usage": used / self.num_blocks,
            "internal_fragmentation": (1.0 - stored / (used * BLOCK_SIZE)) if used else 0.0,
        }


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """K and V of one token across all layers: two tensors of h_kv x d_h
    elements per layer [KV Cache 工程学 §15.2]."""
    return num_layers * 2 * num_kv_heads * head_dim * elem_bytes


def blocks_for_tokens(n: int) -> int:
    """Blocks a sequence of n tokens occupies: whole blocks, the last one
    possibly part-filled [KV Cache 工程学 §15.5]."""
    return -(-n // BLOCK_SIZE)


def build_workload(inst):
    """Run a workload's build script and decode-step append on a fresh Book.

    Returns (book, seq_ids, prefill_slots, step_slots, cow_pairs): slots of
    every prefill token in append order, and the step's slot per sequence."""
    wl = inst.wl
    book = Book(inst.num_blocks, inst.free_order)
    prefill_slots, cow = [], []
    if wl.prefix_len:
        root = book.create()
        s, c = book.append_slots(root, wl.prefix_len)
        prefill_slots += s
        cow += c
        ids = [root] + [book.fork(root) for _ in range(wl.batch - 1)]
    else:
        ids = [book.create() for _ in range(wl.batch)]
    for b, sid in enumerate(ids):
        s, c = book.append_slots(sid, int(inst.own_prefill[b]))
        prefill_slots += s
        cow += c
    step_slots, c = book.batch_append_slots(ids, 1)
    cow += c
    return book, ids, prefill_slots, step_slots, cow
