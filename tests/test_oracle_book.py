"""The oracle's block bookkeeping against the pages' worked numbers and
against invariants that any correct block manager must keep (CPU)."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.book import BLOCK_SIZE, Book, BookError, blocks_for_tokens, build_workload, kv_bytes_per_token
from pins import read_golden
import workloads

KIB, GIB = 1024, 1024 ** 3


def test_bytes_per_token_table():
    """[KV Cache 工程学 §15.2] table, whole-model bytes per token."""
    for name, L, hkv, dh, eb, kib in read_golden("kv_bytes_per_token.txt"):
        assert kv_bytes_per_token(int(L), int(hkv), int(dh), int(eb)) == int(kib) * KIB, name


def test_llama3_70b_sizes():
    """[KV Cache 工程学 §15.3, §15.8]: per-sequence GiB by context, 327,680 B
    per token, INT8 halving."""
    units = {"GiB": GIB, "KiB": KIB, "B": 1}
    for kind, ctx, eb, val, unit in read_golden("llama3_70b_kv_sizes.txt"):
        got = int(ctx) * kv_bytes_per_token(80, 8, 128, int(eb))
        assert got == float(val) * units[unit], (kind, ctx, eb)


def test_best_of_8_counts():
    """[新一代 KV Cache 管理 §8.1]: best-of-8 over a 2,000-token prompt stores
    2,800 instead of 16,800 tokens once blocks are shared by reference."""
    g = {k: int(v) for k, v in read_golden("best_of_8.txt")}
    book = Book(400)
    root = book.create()
    book.append_slots(root, g["prompt_tokens"])
    ids = [root] + [book.fork(root) for _ in range(g["samples"] - 1)]
    for s in ids:
        book.append_slots(s, g["tail_tokens"])
    st_ = book.stats()
    assert st_["tokens_logical"] == g["logical_tokens"]
    assert st_["tokens_stored"] == g["stored_tokens"]
    assert sum(len(book.block_table(s)) for s in ids) == g["table_entries"]
    assert st_["num_used"] == g["distinct_blocks"]
    prompt_blocks = blocks_for_tokens(g["prompt_tokens"])
    for j in range(prompt_blocks):
        assert book.refcount(book.block_table(root)[j]) == g["samples"]
    for s in ids:
        for blk in book.block_table(s)[prompt_blocks:]:
            assert book.refcount(blk) == 1
    # the same numbers come out of the bench workload description
    book2, *_ = build_workload(workloads.get("best_of_8"))
    assert book2.stats()["tokens_stored"] == g["stored_tokens"]
    assert book2.stats()["num_used"] == g["distinct_blocks"]


def test_fragmentation_example():
    """[KV Cache 与 PagedAttention, first article]: a 4096-slot slab used for
    300 tokens wastes ~93%; in 16-token blocks only the tail block wastes."""
    g = {k: int(v) for k, v in read_golden("fragmentation.txt")}
    assert round(100 * (1 - g["used_tokens"] / g["slab_slots"])) == g["slab_waste_pct"]
    book = Book(64)
    s = book.create()
    book.append_slots(s, g["used_tokens"])
    assert len(book.block_table(s)) == g["paged_blocks"]
    st_ = book.stats()
    assert st_["num_used"] * BLOCK_SIZE - st_["tokens_stored"] == g["paged_waste_slots"]


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 31, 32, 33, 4095, 4096, 4097])
def test_blocks_per_sequence(n):
    """A sequence of n tokens holds ceil(n / 16) blocks and wastes < 16 slots."""
    book = Book(300)
    s = book.create()
    book.append_slots(s, n)
    nb = len(book.block_table(s))
    assert nb == math.ceil(n / 16)
    assert 0 <= nb * 16 - n < 16


def test_free_order_and_lifo():
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    book = Book(8, order)
    got = [book.alloc() for _ in range(3)]
    assert got == [5, 2, 7]
    book.decref(2)
    book.decref(5)
    assert book.alloc() == 5  # last freed comes back first
    assert book.alloc() == 2
    assert book.alloc() == 0


def test_slots_follow_table():
    book = Book(8, [3, 1, 6, 0, 2, 4, 5, 7])
    s = book.create()
    slots, cow = book.append_slots(s, 20)
    assert cow == []
    assert slots[:16] == [3 * 16 + i for i in range(16)]
    assert slots[16:] == [1 * 16 + i for i in range(4)]


def test_exhaustion_is_all_or_nothing():
    book = Book(4)
    a = book.create()
    book.append_slots(a, 40)  # 3 blocks
    before = (list(book.free), list(book.ref), book.block_table(a), book.seq_len(a))
    with pytest.raises(BookError) as e:
        book.append_slots(a, 40)  # needs 3 more, 1 free
    assert e.value.code == "NO_BLOCKS"
    assert (list(book.free), list(book.ref), book.block_table(a), book.seq_len(a)) == before
    b = book.create()
    with pytest.raises(BookError):
        book.batch_append_slots([a, b], 9)  # a needs 1 (pos 40..48 crosses 48), b needs 1: 2 > 1
    assert (list(book.free), list(book.ref), book.block_table(a), book.seq_len(a)) == before
    assert (book.block_table(b), book.seq_len(b)) == ([], 0)
    book.batch_append_slots([a, b], 8)  # a stays in its block, b takes the last one
    assert book.num_free() == 0


def test_refcount_errors():
    book = Book(4)
    blk = book.alloc()
    book.decref(blk)
    with pytest.raises(BookError) as e:
        book.decref(blk)
    assert e.value.code == "REFCOUNT"
    with pytest.raises(BookError) as e:
        book.incref(blk)
    assert e.value.code == "REFCOUNT"
    with pytest.raises(BookError) as e:
        book.decref(9)
    assert e.value.code == "BAD_BLOCK"
    with pytest.raises(BookError) as e:
        book.free_seq(123)
    assert e.value.code == "BAD_SEQ"


def test_copy_on_write():
    """A write into a shared, part-filled tail block copies it first
    [KV Cache 与 PagedAttention, first article: copy-on-write for shared prefixes]."""
    book = Book(16, list(range(16)))
    p = book.create()
    book.append_slots(p, 20)            # blocks 0 (full), 1 (4 used)
    c = book.fork(p)
    assert book.refcount(1) == 2
    slots, cow = book.append_slots(p, 1)
    assert cow == [(1, 2)]              # fresh block 2 receives a copy of block 1
    assert book.block_table(p) == [0, 2] and book.block_table(c) == [0, 1]
    assert slots == [2 * 16 + 4]
    assert book.refcount(1) == 1 and book.refcount(0) == 2
    slots, cow = book.append_slots(c, 1)  # last holder writes in place
    assert cow == [] and slots == [1 * 16 + 4]
    # a second fork shares the part-filled tail again; the next write copies it
    d = book.fork(c)
    book.append_slots(c, 11)  # fill block 1 to 16 -> shared tail, CoW on first write
    assert book.block_table(c)[-1] != book.block_table(d)[-1]


OPS = st.lists(st.tuples(st.sampled_from(["create", "fork", "append", "free"]),
                         st.integers(0, 7), st.integers(0, 40)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(OPS)
def test_invariants_random_ops(ops):
    """Reference counts equal the number of tables naming a block; free and
    used blocks partition the pool; slots of unshared positions are unique."""
    book = Book(24, np.random.default_rng(0).permutation(24))
    live = []
    for op, i, n in ops:
        try:
            if op == "create" or not live:
                live.append(book.create())
            elif op == "fork":
                live.append(book.fork(live[i % len(live)]))
            elif op == "append":
                book.append_slots(live[i % len(live)], n)
            else:
                book.free_seq(live.pop(i % len(live)))
        except BookError as e:
            assert e.code == "NO_BLOCKS"
        count = [0] * 24
        for s in live:
            for blk in book.block_table(s):
                count[blk] += 1
            assert len(book.block_table(s)) == blocks_for_tokens(book.seq_len(s))
        assert count == book.ref
        assert sorted(book.free) == [b for b in range(24) if book.ref[b] == 0]
        assert len(set(book.free)) == len(book.free)
        # position -> slot is a function of the physical block only
        where = {}
        for s in live:
            t = book.block_table(s)
            for j in range(book.seq_len(s)):
                slot = t[j // 16] * 16 + j % 16
                where.setdefault(slot, set()).add(j)
        for slot, js in where.items():
            assert len(js) == 1  # one logical position per physical slot
