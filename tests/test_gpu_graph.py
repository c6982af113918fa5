"""The allocation-free decode entry under HIP graph capture: captured once,
replayed several times with the program's own eager work and
synchronisations between the replays, every replay bitwise equal to the
eager call (the same kernels and split).  The capture records only the
partition and merge kernels (no memset, no allocation)."""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import attn as orc
from paged_kv_cache_381_amd import _lib as L
from paged_kv_cache_381_amd.engine import GpuWorkload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,kw", [("llama3_8b_b64", dict(batch=12, ctx_range=(1, 2500))),
                                     ("llama3_8b_b64_int8", dict(batch=7, ctx_range=(1, 1800)))])
def test_noalloc_decode_replays_from_a_graph(name, kw):
    inst = workloads.configs.scaled(name, **kw).instantiate()
    say(f"[graph] {name} {kw}: ctx {inst.ctx.tolist()}")
    gw = GpuWorkload(inst)
    c = gw.cache
    wps = c.waves_per_simd()

    def call(out):
        L.paged_attention_decode_noalloc(c.layout, out, gw.q, c.k_pools[0], c.v_pools[0], gw.tables_dev,
                                         gw.ctx_dev, gw.max_ctx, gw.scale, waves_per_simd=wps)

    eager = torch.full_like(gw.out, float("nan"))
    call(eager)  # also looks up the scratch's address, outside the capture
    torch.cuda.synchronize()
    ref = orc.run_workload(inst)["out"]
    err = float(np.abs(eager.cpu().numpy() - ref).max())
    say(f"  eager: max abs err {err:.3e}")
    assert err <= 2e-2

    out = torch.full_like(gw.out, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        scratch_user = torch.full_like(gw.out, 3.0)  # eager work between replays
        call(scratch_user)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: differs from the eager call"
        assert torch.equal(scratch_user, eager)
        say(f"  replay {rep}: bitwise equal to the eager call")
