"""Swap of blocks to pinned host memory and back, on the GPU: the bytes of
every block survive the round trip (compared with the oracle's pools
through the tables), and decode over swapped-in sequences equals decode
before the swap bit for bit (same launch, same logical tokens) and the
oracle within tolerance."""
import math
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


def gathered(cache, tables, ctx, H, D, dtype):
    """Logical K/V of each sequence read through its table: (codes or
    element bits per token) from the device pools."""
    def raw(t):
        return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy().view(np.uint8)
    out = []
    tb = 16 * D * (2 if dtype == "bf16" else 1) + (64 if dtype == "int8" else 0)
    kb, vb = raw(cache.k_pools[0]), raw(cache.v_pools[0])
    for b in range(len(ctx)):
        blocks = [int(x) for x in tables[b][:-(-int(ctx[b]) // 16)]]
        out.append((np.concatenate([kb[(blk * H) * tb:(blk * H + H) * tb] for blk in blocks]),
                    np.concatenate([vb[(blk * H) * tb:(blk * H + H) * tb] for blk in blocks])))
    return out


@pytest.mark.parametrize("name", ["llama3_8b_b64", "llama3_8b_b64_int8"])
def test_swap_round_trip_keeps_blocks_and_outputs(name):
    kw = dict(batch=8, ctx_range=(20, 300))
    inst = workloads.configs.scaled(name, **kw).instantiate()
    wl = inst.wl
    gw = GpuWorkload(inst, extra_blocks=64)
    c = gw.cache
    H, D = wl.num_kv_heads, wl.head_dim
    before = gw.decode(waves_per_simd=1).clone()
    tables0, ctx0 = c.tables(gw.ids, gw.max_blocks)
    data0 = gathered(c, tables0, ctx0, H, D, wl.cache_dtype)
    c.enable_swap(400)
    keep = gw.ids[:3]
    # export the kept batch (sets their bits), then evict: every other block
    # goes to the host within two turns of the hand
    c.tables(keep, gw.max_blocks)
    total = int(sum(-(-int(n) // 16) for n in ctx0[3:]))
    pairs = c.swap_out(10 ** 4, protect=keep)
    say(f"[swap] {name}: {len(pairs)} blocks out of {total} unprotected")
    assert len(pairs) == total
    for sid in gw.ids[3:]:
        assert not L.pkv_seq_resident(c.pool, sid)
    # reuse the freed device blocks: a new sequence overwrites them with other values
    junk = c.create()
    slots, _ = c.reserve([junk], 16 * 40)
    rows = workloads.configs.normal_bits(99, (16 * 40, H, D), "bf16")
    dev = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda()
    c.write(0, torch.from_numpy(slots).cuda(), dev, dev)
    c.free(junk)
    for sid in gw.ids[3:]:
        c.swap_in(sid)
    torch.cuda.synchronize()
    tables1, ctx1 = c.tables(gw.ids, gw.max_blocks)
    assert not np.array_equal(tables0, tables1)
    data1 = gathered(c, tables1, ctx1, H, D, wl.cache_dtype)
    for b in range(wl.batch):
        assert np.array_equal(data0[b][0], data1[b][0]) and np.array_equal(data0[b][1], data1[b][1]), b
    gw.tables_dev = torch.from_numpy(tables1).cuda()
    after = gw.decode(waves_per_simd=1).clone()
    assert torch.equal(before, after)
    ref = orc.run_workload(inst)["out"]
    err = np.abs(after.cpu().numpy() - ref).max()
    say(f"[swap] {name}: decode after swap-in, max abs err {err:.3e}")
    assert err <= 2e-2
    st = L.pkv_swap_space_stats(c.pool)
    assert st["host_used"] == 0 and st["swapped_out"] == st["swapped_in"] == total
