"""Seeded random shapes for decode and prefill, every output against the
oracle.

The named workloads fix one shape each; these draw the parameters the
kernels branch on -- group size G (1..16, including G = 3, whose tiles use
15 of 16 columns), head dim 64 or 128, bf16, float32 or int8 caches, batch
size, context and prompt lengths (including 1 and lengths one either side of
a block or chunk edge), shared prefixes, partition size, waves per SIMD and
the kernel choice -- from a fixed seed, so each case is reproducible by its
index.  Tolerances: 1e-5 for float32 caches, 2e-2 for bf16 and int8.
Every decode draw also records a decode plan and runs from it: both calls
must equal the self-scheduled one bit for bit.
PKV_RANDOM_SHAPES=<decode>,<prefill> runs a longer sweep of the same draws.
"""
import os
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import attn as orc
from paged_kv_cache_381_amd.engine import GpuPrefill, GpuWorkload
from workloads import prefill as PW

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "int8": 2e-2}
# Case counts; a longer sweep sets PKV_RANDOM_SHAPES=<decode>,<prefill>.
N_DECODE, N_PREFILL = (int(x) for x in os.environ.get("PKV_RANDOM_SHAPES", "15,12").split(","))
EDGE = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    say(f"  {what}: max abs err {err:.3e} (tol {tol})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def decode_case(i):
    rng = np.random.default_rng(7000 + i)
    cache = ["bf16", "f32", "int8"][i % 3]
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    hkv = int(rng.choice([1, 2, 4])) if G < 12 else 1
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 9))
    kw = dict(batch=B, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D,
              dtype="f32" if cache == "f32" else "bf16", cache="int8" if cache == "int8" else "")
    if rng.random() < 0.3:  # a shared prefix (whole blocks), then private suffixes
        kw.update(prefix_len=16 * int(rng.integers(1, 20)), suffix_range=(1, int(rng.integers(2, 200))))
    else:
        ctx = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(1, 900)) for _ in range(B)]
        kw.update(ctx_fixed=tuple(ctx))
    kernel = 1 if (cache == "bf16" and rng.random() < 0.3) else 0
    part = int(rng.choice([0, 32, 96]))
    wps = int(rng.choice([1, 2]))
    return kw, kernel, part, wps


@pytest.mark.parametrize("i", range(N_DECODE))
def test_decode_random_shape(i):
    kw, kernel, part, wps = decode_case(i)
    base = "tiny_fp32" if kw["dtype"] == "f32" else "llama3_8b_b64"
    kw = {k: v for k, v in kw.items() if not (k == "cache" and v == "")}
    inst = workloads.configs.scaled(base, ctx_range=(), pool_blocks=0, **kw).instantiate()  # pool: 1.25x demand
    say(f"[decode {i}] {kw} kernel {kernel} partition {part} waves/SIMD {wps}: ctx {inst.ctx.tolist()}")
    gw = GpuWorkload(inst)
    ref = orc.run_workload(inst)["out"]
    first = gw.decode(partition_tokens=part, kernel=kernel, waves_per_simd=wps).clone()
    out = first.cpu().numpy()
    check_close(out, ref, TOL[inst.wl.cache_dtype], f"decode case {i}")
    plan = gw.new_plan(part)
    for what in ("recording a plan", "from the plan"):
        again = gw.decode(partition_tokens=part, kernel=kernel, waves_per_simd=wps, plan=plan)
        assert torch.equal(again, first), f"decode case {i} {what}: differs from the self-scheduled call"


ODD_GROUPS = [(G, cache, kernel) for G in (3, 5, 6, 12) for cache, kernel in
              (("bf16", 1), ("bf16", 2), ("int8", 2), ("fp8", 2))]


@pytest.mark.parametrize("G,cache,kernel", ODD_GROUPS)
def test_decode_group_not_power_of_two(G, cache, kernel):
    """Group sizes that are not powers of two: the matrix-core kernel's
    padded head columns (columns G..15 repeat head G-1) and its ring records
    (G rows, G (m, l) pairs, the place at the next 16-byte boundary), and the
    wavefront kernel's group padded up to a power of two.  Contexts cross
    block and chunk edges and are long enough to be cut between waves."""
    hkv = 2
    ctx = (1, 17, 33, 250, 700, 1500)
    kw = dict(batch=len(ctx), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=128, dtype="bf16", ctx_fixed=ctx)
    if cache != "bf16":
        kw["cache"] = cache
    inst = workloads.configs.scaled("llama3_8b_b64", ctx_range=(), pool_blocks=0, **kw).instantiate()
    say(f"[groups] G {G} {cache} kernel {kernel}: ctx {inst.ctx.tolist()}")
    gw = GpuWorkload(inst)
    ref = orc.run_workload(inst)["out"]
    for part, wps in ((0, 1), (32, 2)):
        out = gw.decode(partition_tokens=part, kernel=kernel, waves_per_simd=wps).cpu().numpy()
        check_close(out, ref, TOL["bf16"], f"G {G} {cache} kernel {kernel} partition {part} waves/SIMD {wps}")


def prefill_case(i):
    rng = np.random.default_rng(8000 + i)
    cache = ["bf16", "int8"][i % 2]
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4])) if G < 16 else 1
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 5))
    nmax = int(rng.choice([1, 17, 40, 97]))
    kw = dict(batch=B, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, cache="int8" if cache == "int8" else "",
              new_tokens=(1, nmax), own_prefix=(0, int(rng.choice([0, 15, 33, 120]))))
    if rng.random() < 0.4:
        kw["shared_prefix"] = 16 * int(rng.integers(1, 8))
    return kw


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_prefill_random_shape(i):
    kw = prefill_case(i)
    inst = PW.scaled("prefill_8b_b4", **kw).instantiate()
    say(f"[prefill {i}] {kw}: nq {inst.nq.tolist()} ctx {inst.ctx.tolist()}")
    gp = GpuPrefill(inst)
    ref = orc.run_prefill(inst)
    out = gp.run().cpu().numpy()
    check_close(out, ref["out"], TOL[inst.wl.cache_dtype], f"prefill case {i}")
