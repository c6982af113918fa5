"""Parity of the paged prefill (through the C ABI) with the CPU oracle.

The prefill is a causal attention of each sequence's new tokens over its
paged cache (a cached prefix, shared or private, then the new tokens).  The
pools are built on both sides by the same build script; outputs are compared
element by element: max abs error <= 2e-2 (bf16, int8 or FP8 cache, float32
accumulation), on every output of small shapes, on sampled query rows of the
full-size workloads (the oracle evaluates the last new tokens of chosen
sequences, which see the most keys), and on every new token of the
full-size workloads (every output of the bf16 ones; the query heads of one
kv head for the one-byte caches).
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import attn as orc
from paged_kv_cache_381_amd import _lib as L
from paged_kv_cache_381_amd.engine import GpuPrefill, GpuWorkload
from workloads import prefill as PW

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    say(f"  {what}: max abs err {err:.3e} (tol {tol})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"
    return err


SMALL = [
    ("prefill_shared_prefix", dict(batch=3, shared_prefix=48, new_tokens=(1, 40))),          # G 4, shared prefix
    ("prefill_8b_b4", dict(batch=3, new_tokens=(1, 70))),                                      # no prefix
    ("prefill_8b_b4", dict(batch=4, num_q_heads=64, own_prefix=(0, 50), new_tokens=(1, 33))),  # G 8, private prefix
    ("prefill_8b_b4", dict(batch=3, num_q_heads=8, own_prefix=(0, 20), new_tokens=(1, 45))),   # G 1: 16 tokens a wave
    ("prefill_8b_b4", dict(batch=2, num_q_heads=16, num_kv_heads=1, new_tokens=(5, 37))),     # G 16: 1 token a wave
    ("prefill_8b_b4", dict(batch=3, head_dim=64, own_prefix=(10, 30), new_tokens=(1, 50))),   # D 64
    ("prefill_8b_b4", dict(batch=3, num_q_heads=24, own_prefix=(0, 17), new_tokens=(1, 29))),  # G 3: 15 columns used
    ("prefill_shared_prefix", dict(batch=3, shared_prefix=32, new_tokens=(1, 40), cache="int8")),
    ("prefill_8b_b4", dict(batch=3, num_q_heads=64, own_prefix=(0, 40), new_tokens=(1, 30), cache="int8")),
    ("prefill_shared_prefix", dict(batch=3, shared_prefix=32, new_tokens=(1, 40), cache="fp8")),
    ("prefill_8b_b4", dict(batch=3, head_dim=64, own_prefix=(0, 40), new_tokens=(1, 30), cache="fp8")),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small_every_output(case):
    name, kw = SMALL[case]
    inst = PW.scaled(name, **kw).instantiate()
    say(f"[prefill] {name} {kw}: nq {inst.nq.tolist()} ctx {inst.ctx.tolist()}")
    gp = GpuPrefill(inst)
    ref = orc.run_prefill(inst)
    assert np.array_equal(gp.tables_host, ref["tables"])
    out = gp.run().cpu().numpy()
    check_close(out, ref["out"], TOL, f"{name} {kw}")


def _sampled(name, picks, last):
    inst = PW.get(name)
    gp = GpuPrefill(inst)
    out = gp.run().cpu().numpy()
    assert np.isfinite(out).all()
    # The oracle's pools, then the last `last` new tokens of each picked
    # sequence (they see every key before them): a sub-problem of the same
    # definition.
    wl = inst.wl
    built = orc.build_prefill(inst)
    kpool, vpool, tables, ctx = built["kpool"], built["vpool"], built["tables"], built["ctx"]
    assert np.array_equal(tables, gp.tables_host)
    qs = inst.qstart
    q = inst.q()
    for b in picks:
        rows = slice(int(qs[b + 1]) - last, int(qs[b + 1]))
        ref = orc.paged_prefill(wl.cache_dtype, q[rows], kpool, vpool, tables[b:b + 1], ctx[b:b + 1],
                                np.array([0, last], np.int32), wl.num_kv_heads, 1 / math.sqrt(wl.head_dim))
        check_close(out[rows], ref, TOL, f"{name} seq {b}, last {last} of {int(inst.nq[b])} new tokens")


def test_prefill_shared_prefix_sampled():
    _sampled("prefill_shared_prefix", picks=[0, 7, 15], last=48)


def test_prefill_8b_b4_sampled():
    _sampled("prefill_8b_b4", picks=[0, 3], last=32)


def _one_head(pool, num_blocks, num_kv_heads, g):
    """The pool of kv head g alone: tile (block, g) of every block, in block
    order (a pool of the same layout with one kv head)."""
    tiles = pool.reshape(num_blocks, num_kv_heads, -1)
    return np.ascontiguousarray(tiles[:, g, :]).reshape(-1)


FULL = [("prefill_8b_b4", tuple(range(8))), ("prefill_shared_prefix", tuple(range(8))),
        ("prefill_shared_prefix_int8", (3,)), ("prefill_shared_prefix_fp8", (4,))]


@pytest.mark.parametrize("case", range(len(FULL)))
def test_prefill_full_workload_every_token(case):
    """Every new token of every sequence of a full-size workload, for the
    query heads of the listed kv heads: the oracle in float64 over one kv
    head's group at a time (the same definition with that head's pool and
    query heads), every output of those heads compared."""
    name, heads = FULL[case]
    inst = PW.get(name)
    wl = inst.wl
    gp = GpuPrefill(inst)
    out = gp.run().cpu().numpy()
    assert np.isfinite(out).all()
    built = orc.build_prefill(inst)
    assert np.array_equal(built["tables"], gp.tables_host)
    H, G = wl.num_kv_heads, wl.num_q_heads // wl.num_kv_heads
    q = inst.q()
    for g in heads:
        kp = _one_head(built["kpool"], inst.num_blocks, H, g)
        vp = _one_head(built["vpool"], inst.num_blocks, H, g)
        say(f"[prefill] {name}: kv head {g}, {q.shape[0]} new tokens x {G} query heads")
        ref = orc.paged_prefill(wl.cache_dtype, q[:, g * G:(g + 1) * G], kp, vp, built["tables"], built["ctx"],
                                inst.qstart, 1, 1 / math.sqrt(wl.head_dim))
        check_close(out[:, g * G:(g + 1) * G], ref, TOL, f"{name} kv head {g}, every new token")


@pytest.mark.parametrize("cache", ["bf16", "int8"])
def test_prefill_maximum_context_every_output(cache):
    """16 new tokens after a cached prefix that brings the context to the
    largest length the call accepts, 2^22 tokens (262144 blocks in one table
    row); one kv head of four query heads at d 64.  Every wave walks all
    131072 chunks; every output against the oracle."""
    n = 1 << 22
    inst = PW.scaled("prefill_8b_b4", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                     own_prefix=(n - 16, n - 16), new_tokens=(16, 16), cache=cache).instantiate()
    say(f"[prefill] context {inst.ctx.tolist()}, {inst.nq.tolist()} new, {cache}")
    gp = GpuPrefill(inst)
    out = gp.run().cpu().numpy()
    ref = orc.run_prefill(inst)
    assert np.array_equal(gp.tables_host, ref["tables"])
    check_close(out, ref["out"], TOL, f"context 2^22, {cache}")
    del gp
    torch.cuda.empty_cache()


def test_prefill_of_one_token_is_decode():
    """A prefill whose every sequence has one new token is a decode step."""
    import workloads
    inst = workloads.configs.scaled("llama3_8b_b64", batch=6, ctx_range=(1, 700)).instantiate()
    gw = GpuWorkload(inst)
    dec = gw.decode().clone()
    qstart = torch.arange(inst.wl.batch + 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(dec)
    gw.cache.prefill(0, out, gw.q, gw.tables_dev, gw.ctx_dev, qstart, 1, gw.max_ctx, gw.scale)
    check_close(out.cpu().numpy(), dec.cpu().numpy().astype(np.float64), TOL, "prefill of one token vs decode")


def test_prefill_deterministic_and_placement_invariant():
    name, kw = "prefill_8b_b4", dict(batch=3, own_prefix=(0, 40), new_tokens=(1, 60))
    inst = PW.scaled(name, **kw).instantiate()
    a = GpuPrefill(inst)
    x = a.run().clone()
    assert torch.equal(x, a.run().clone())
    inst.free_order = np.arange(inst.num_blocks, dtype=np.int32)
    b = GpuPrefill(inst)
    assert not np.array_equal(a.tables_host, b.tables_host)
    assert torch.equal(x, b.run().clone())


def test_prefill_rejects_bad_calls():
    inst = PW.scaled("prefill_8b_b4", batch=2, new_tokens=(3, 5)).instantiate()
    gp = GpuPrefill(inst)
    with pytest.raises(L.PagedKVError):  # max_query_len beyond max_context_len
        L.paged_attention_prefill(gp.cache.layout, gp.out, gp.q, gp.cache.k_pools[0], gp.cache.v_pools[0],
                                  gp.tables_dev, gp.ctx_dev, gp.qstart_dev, gp.max_ctx + 1, gp.max_ctx, gp.scale)
    c = gp.cache
    f32 = L.make_layout(c.layout.num_blocks, c.layout.num_kv_heads, c.layout.head_dim, "f32")
    kf = torch.zeros(f32.pool_elems, dtype=torch.float32, device="cuda")
    with pytest.raises(L.PagedKVError):  # no float32 prefill
        L.paged_attention_prefill(f32, gp.out, gp.q, kf, kf, gp.tables_dev, gp.ctx_dev, gp.qstart_dev, gp.max_q,
                                  gp.max_ctx, gp.scale)
