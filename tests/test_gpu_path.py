"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Append and copy are compared bit for bit over the whole pool, NaN sentinels
included.  Attention is compared element by element: max abs error <= 1e-5
for the float32 workload and <= 2e-2 for the bf16 workloads (bf16 K/V,
float32 accumulation).  Full-size workloads run in the launch configuration
the bench times (default partition, automatic kernel choice) and are checked
on every output against the oracle's run of the same build.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import attn as orc
from paged_kv_cache_381_amd import _lib as L
from paged_kv_cache_381_amd.engine import GpuWorkload, PagedKVCache

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pool_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def oracle_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


_built = {}


def built(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _built:
        say(f"[build] {name} {kw}")
        inst = workloads.get(name) if not kw else workloads.configs.scaled(name, **kw).instantiate()
        _built[key] = (inst, GpuWorkload(inst))
        torch.cuda.synchronize()
    return _built[key]


def check_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    say(f"  {what}: max abs err {err:.3e} (tol {tol})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"
    return err


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("name", ["tiny_fp32", "best_of_8", "shared_prefix_b128", "llama3_8b_b64"])
def test_append_pool_bit_exact(name):
    inst, gw = built(name)
    say(f"[append] {name}: oracle pool build")
    ref = orc.run_workload(inst, with_attention=False)
    assert gw.step_slots.tolist() == ref["step_slots"]
    assert gw.prefill_slots.tolist() == ref["prefill_slots"]
    assert np.array_equal(gw.tables_host, ref["tables"])
    for got, want in ((gw.cache.k_pools[0], ref["kpool"]), (gw.cache.v_pools[0], ref["vpool"])):
        assert np.array_equal(pool_bits(got), oracle_bits(want))


def test_copy_blocks_and_cow_bit_exact():
    """Copy-on-write: a fork shares a part-filled tail; the next write copies
    the block on the device and stores into the copy."""
    H, D, dt = 2, 64, "bf16"
    order = np.random.default_rng(3).permutation(12).astype(np.int32)
    c = PagedKVCache(12, H, D, dt, free_order=order)
    kpool, vpool = orc.new_pool(12, H, D, dt)
    book_ids = []
    from oracle.book import Book
    book = Book(12, order)
    vals = workloads.configs.normal_bits(7, (64, 2, H, D), dt)
    p = c.create()
    bp = book.create()
    s, cow = c.reserve([p], 21)
    bs, bcow = book.append_slots(bp, 21)
    assert s.tolist() == bs and len(cow) == 0
    sd = torch.from_numpy(s).cuda()
    kn = torch.from_numpy(vals[:21, 0].view(np.int16).copy()).view(torch.bfloat16).cuda()
    vn = torch.from_numpy(vals[:21, 1].view(np.int16).copy()).view(torch.bfloat16).cuda()
    c.write(0, sd, kn, vn)
    orc.append(dt, H, D, kpool, vpool, vals[:21, 0], vals[:21, 1], bs)
    ch = c.fork(p)
    bch = book.fork(bp)
    for seq, bseq, row in ((p, bp, 21), (ch, bch, 22)):
        s, cow = c.reserve([seq], 1)
        bs, bcow = book.append_slots(bseq, 1)
        assert s.tolist() == bs and [tuple(x) for x in cow.tolist()] == bcow
        if bcow:
            orc.copy_blocks(dt, H, D, kpool, vpool, bcow)
        kn = torch.from_numpy(vals[row:row + 1, 0].view(np.int16).copy()).view(torch.bfloat16).cuda()
        vn = torch.from_numpy(vals[row:row + 1, 1].view(np.int16).copy()).view(torch.bfloat16).cuda()
        c.write(0, torch.from_numpy(s).cuda(), kn, vn)
        orc.append(dt, H, D, kpool, vpool, vals[row:row + 1, 0], vals[row:row + 1, 1], bs)
    assert np.array_equal(pool_bits(c.k_pools[0]), kpool)
    assert np.array_equal(pool_bits(c.v_pools[0]), vpool)
    # explicit whole-block copies of random pairs
    pairs = np.array([[int(order[0]), int(order[9])], [int(order[1]), int(order[10])]], np.int32)
    L.pkv_copy_blocks(c.layout, c.k_pools[0], c.v_pools[0], torch.from_numpy(pairs).cuda())
    orc.copy_blocks(dt, H, D, kpool, vpool, pairs)
    assert np.array_equal(pool_bits(c.k_pools[0]), kpool)
    assert np.array_equal(pool_bits(c.v_pools[0]), vpool)
    del book_ids


# --------------------------------------------------------------- attention
def test_tiny_fp32_all_partitions():
    inst, gw = built("tiny_fp32")
    ref = orc.run_workload(inst)["out"]
    for part in (32, 64, 128, 512):
        out = gw.decode(partition_tokens=part).cpu().numpy()
        check_close(out, ref, TOL["f32"], f"tiny_fp32 P={part}")


SMALL = [  # (workload, overrides) small enough for the oracle on every output
    ("llama3_8b_b64", dict(batch=6, ctx_range=(1, 700))),
    ("llama3_70b_b256", dict(batch=5, ctx_fixed=(1, 31, 32, 33, 577))),
    ("mha_long", dict(batch=4, num_q_heads=4, num_kv_heads=4, ctx_fixed=(1, 16, 17, 1100), pool_blocks=0)),
    ("best_of_8", dict(batch=3, prefix_len=48, suffix_fixed=21)),
    ("llama3_8b_b64", dict(batch=3, head_dim=64, ctx_range=(1, 300))),
    ("tiny_fp32", dict(num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_fixed=(3, 64, 65, 200), pool_blocks=0)),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("part", [32, 96, 512])
def test_small_workloads_every_output(case, kernel, part):
    name, kw = SMALL[case]
    inst, gw = built(name, **kw)
    if kernel == 2 and inst.wl.dtype != "bf16":
        pytest.skip("matrix-core kernel is bf16 only")
    key = ("ref", name, tuple(sorted(kw.items())))
    if key not in _built:
        _built[key] = orc.run_workload(inst)["out"]
    out = gw.decode(partition_tokens=part, kernel=kernel).cpu().numpy()
    check_close(out, _built[key], TOL[inst.wl.dtype], f"{name} {kw} kernel={kernel} P={part}")


_full_ref = {}


def full_ref(name, inst):
    if name not in _full_ref:
        say(f"[oracle] {name}: {orc.num_threads()} threads")
        _full_ref[name] = orc.run_workload(inst)["out"]
    return _full_ref[name]


@pytest.mark.parametrize("name", ["llama3_8b_b64", "llama3_70b_b256", "best_of_8", "shared_prefix_b128", "mha_long"])
def test_full_workload_every_output(name):
    """Every output of a full-size workload, in the launch configuration the
    bench times, against the oracle's run of the same build (OpenMP over
    sequence x query head on the host)."""
    inst, gw = built(name)
    ref = full_ref(name, inst)
    out = gw.decode().cpu().numpy()
    check_close(out, ref, TOL["bf16"], f"{name} full")
    if name in ("llama3_70b_b256", "mha_long"):  # the largest pools: give their memory back
        _built.pop((name, ()), None)
        _full_ref.pop(name, None)
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name,hq", [("llama3_8b_b64", 4), ("llama3_8b_b64_int8", 4), ("llama3_8b_b64", 1)])
def test_maximum_context_every_output(name, hq):
    """A context of the largest length the calls accept, 2^22 tokens (262144
    blocks in one table row), beside a short one; one kv head of four query
    heads (the matrix-core kernel) or of one (the wavefront kernel) at d 64
    keeps the pool near 1.3 GiB.  The long context is cut into a piece for
    nearly every wave of the grid and the merge folds them all; every output
    against the oracle."""
    kw = dict(batch=2, num_q_heads=hq, num_kv_heads=1, head_dim=64, ctx_fixed=(1 << 22, 100))
    inst, gw = built(name, **kw)
    say(f"[oracle] {name} contexts {inst.ctx.tolist()}")
    ref = orc.run_workload(inst)["out"]
    check_close(gw.decode().cpu().numpy(), ref, TOL["bf16"], f"{name} context 2^22")
    _built.pop((name, tuple(sorted(kw.items()))), None)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,hq", [("llama3_8b_b64", 8), ("llama3_8b_b64_int8", 8), ("llama3_8b_b64", 2)])
def test_maximum_batch_every_output(name, hq):
    """The largest batch one call takes, 8192 sequences of 1-40 tokens: the
    chunk scan of the whole batch fills most of the workgroup's LDS and
    leaves the result ring a few records; every output against the oracle,
    on the matrix-core kernel (G = 4, bf16 and int8) and the wavefront
    kernel (G = 1)."""
    kw = dict(batch=8192, num_q_heads=hq, num_kv_heads=2, head_dim=64, ctx_range=(1, 40))
    inst, gw = built(name, **kw)
    say(f"[oracle] {name} 8192 sequences, {hq} query heads")
    ref = orc.run_workload(inst)["out"]
    check_close(gw.decode().cpu().numpy(), ref, TOL["bf16"], f"{name} 8192 sequences")
    _built.pop((name, tuple(sorted(kw.items()))), None)


@pytest.mark.parametrize("name", ["llama3_8b_b64", "llama3_8b_b64_int8"])
def test_many_short_segments_every_output(name):
    """2600 sequences of 1-16 tokens: one chunk per segment, about 20
    segment ends per wave, more than its LDS result ring holds (9 records
    of 2080 bytes at this batch, whose chunk scan takes 20 KiB of the
    workgroup's 96 KiB), so pieces past the ring's capacity
    take the direct stores; every output must still match the oracle."""
    inst, gw = built(name, batch=2600, ctx_range=(1, 16))
    say(f"[oracle] {name} 2600 short sequences")
    ref = orc.run_workload(inst)["out"]
    check_close(gw.decode().cpu().numpy(), ref, TOL["bf16"], f"{name} 2600 short sequences")


def test_xcd_weights_every_output_and_trace():
    """Per-XCD weights move the region bounds of the balanced split: the
    outputs still match the oracle everywhere and repeat bit for bit, and the
    trace holds one record per working wave, on all 8 XCDs, whose chunk
    counts add up to the batch's chunks."""
    name = "llama3_8b_b64"
    inst, gw = built(name)
    ref = full_ref(name, inst)
    w = [1000, 870, 1130, 800, 1000, 1200, 950, 1050]
    trace = torch.zeros(4 * L.PKV_TRACE_WAVES, dtype=torch.int32, device="cuda")
    a = gw.decode(xcd_weights=w, trace=trace).clone()
    check_close(a.cpu().numpy(), ref, TOL["bf16"], f"{name} weights {w}")
    assert torch.equal(a, gw.decode(xcd_weights=w).clone())
    t = trace.cpu().numpy().reshape(-1, 4)
    used = t[t[:, 1] > 0]
    assert set(used[:, 0].tolist()) == set(range(8))
    assert int(used[:, 1].sum()) == inst.wl.num_kv_heads * sum(-(-int(n) // 32) for n in inst.ctx)
    got = L.xcd_weights_from_trace(trace)
    say(f"  measured weights {got}")
    assert all(x > 0 for x in got)
    check_close(gw.decode(xcd_weights=got).cpu().numpy(), ref, TOL["bf16"], f"{name} weights {got}")


def test_deterministic_and_placement_invariant():
    """Bitwise: run-to-run, and identity vs shuffled physical placement."""
    name, kw = "llama3_8b_b64", dict(batch=6, ctx_range=(1, 700))
    inst, gw = built(name, **kw)
    a = gw.decode().clone()
    b = gw.decode().clone()
    assert torch.equal(a, b)
    inst2 = workloads.configs.scaled(name, **kw).instantiate()
    inst2.free_order = np.arange(inst2.num_blocks, dtype=np.int32)
    gw2 = GpuWorkload(inst2)
    assert not np.array_equal(gw.tables_host, gw2.tables_host)
    for kernel in (1, 2):
        for wps in (1, 2):
            assert torch.equal(gw.decode(kernel=kernel, waves_per_simd=wps).clone(),
                               gw2.decode(kernel=kernel, waves_per_simd=wps).clone())


class _Unshared:
    """The same logical tokens as a shared-prefix instance, but every
    sequence holds its own copy of the prefix (no sharing)."""

    def __init__(self, inst):
        import dataclasses
        self.src = inst
        self.wl = dataclasses.replace(inst.wl, prefix_len=0)
        self.ctx = inst.ctx
        self.own_prefill = inst.ctx - 1
        demand = int(sum(-(-int(n) // 16) for n in inst.ctx))
        self.num_blocks = demand + 7
        self.free_order = np.random.default_rng(11).permutation(self.num_blocks).astype(np.int32)

    def q(self):
        return self.src.q()

    def prefill_tokens(self, which):
        return np.concatenate([self.src.seq_kv(b, which)[:int(self.ctx[b]) - 1] for b in range(self.wl.batch)])

    def step_tokens(self, which):
        return self.src.step_tokens(which)


def test_shared_prefix_reads_like_private_copies():
    """Outputs through refcounted shared blocks equal those of an unshared
    deep copy at other physical blocks, bit for bit."""
    inst, gw = built("best_of_8")
    st = gw.cache.stats()
    assert st["num_used"] == 181 and st["tokens_stored"] == 2800 and st["num_shared"] == 125
    un = GpuWorkload(_Unshared(inst))
    assert un.cache.stats()["num_shared"] == 0
    # Same launch on both sides: the split of the chunk list follows the grid,
    # and a different cut changes the rounding of the merge.
    for kernel in (1, 2):
        for wps in (1, 2):
            assert torch.equal(gw.decode(kernel=kernel, waves_per_simd=wps).clone(),
                               un.decode(kernel=kernel, waves_per_simd=wps).clone())


def test_empty_and_padding_sequences():
    """A sequence with no tokens (padding) gets zeros; NaN in unused slots
    never reaches an output."""
    H, Hq, D = 2, 8, 128
    c = PagedKVCache(8, H, D, "bf16")
    ids = [c.create(), c.create()]
    s, _ = c.reserve([ids[1]], 5)
    kv = workloads.configs.normal_bits(5, (2, 5, H, D), "bf16")
    mk = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    c.write(0, torch.from_numpy(s).cuda(), mk(kv[0]), mk(kv[1]))
    tables, ctx = c.tables(ids, 2)
    q = workloads.configs.normal_bits(6, (2, Hq, D), "bf16")
    for kernel in (1, 2):
        out = torch.full((2, Hq, D), 7.0, device="cuda")
        ws = c.workspace(2, Hq, 5, 0, kernel)
        c.decode(0, out, mk(q), torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), 5, 1 / math.sqrt(D),
                 ws, 0, kernel)
        o = out.cpu().numpy()
        assert (o[0] == 0).all()
        ref = orc.contiguous_attention("bf16", q[1], kv[0], kv[1], 1 / math.sqrt(D))
        check_close(o[1], ref, TOL["bf16"], f"padding kernel={kernel}")


def test_prefix_cache_hits_read_like_prefill():
    """Requests built through the prefix cache (their prompt's cached blocks
    found, the rest stored) attend exactly over their own prompt: every
    output within tolerance of the oracle's contiguous attention."""
    H, Hq, D = 8, 32, 128
    rng = np.random.default_rng(11)
    system = rng.integers(0, 32000, size=200, dtype=np.int32)  # 12 full blocks + 8 tokens
    c = PagedKVCache(256, H, D, "bf16")
    c.enable_prefix_cache(True)
    sys_k = workloads.configs.normal_bits(21, (200, H, D), "bf16")
    sys_v = workloads.configs.normal_bits(22, (200, H, D), "bf16")
    mk = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    ids, kv = [], []
    for r in range(6):
        own = 20 + 31 * r
        toks = np.concatenate([system, rng.integers(0, 32000, size=own, dtype=np.int32)])
        k_all = np.concatenate([sys_k, workloads.configs.normal_bits(30 + r, (own, H, D), "bf16")])
        v_all = np.concatenate([sys_v, workloads.configs.normal_bits(40 + r, (own, H, D), "bf16")])
        sid, cached = c.create_from_prefix(toks)
        assert cached == (0 if r == 0 else 192)
        slots, _ = c.reserve([sid], len(toks) - cached)
        c.write(0, torch.from_numpy(slots).cuda(), mk(k_all[cached:]), mk(v_all[cached:]))
        c.register_prefix(sid, toks)
        ids.append(sid)
        kv.append((k_all, v_all))
    st = c.prefix_stats()
    assert st["hit_tokens"] == 5 * 192
    mb = max(-(-len(k) // 16) for k, _ in kv)
    tables, ctx = c.tables(ids, mb)
    q = workloads.configs.normal_bits(50, (len(ids), Hq, D), "bf16")
    out = torch.empty(len(ids), Hq, D, device="cuda")
    for wps in (1, 2):
        ws = c.workspace(len(ids), Hq, int(ctx.max()))
        c.decode(0, out, mk(q), torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), int(ctx.max()),
                 1 / math.sqrt(D), ws, waves_per_simd=wps)
        o = out.cpu().numpy()
        for i, (k_all, v_all) in enumerate(kv):
            ref = orc.contiguous_attention("bf16", q[i], k_all, v_all, 1 / math.sqrt(D))
            check_close(o[i], ref, TOL["bf16"], f"prefix-cache request {i} wps={wps}")
