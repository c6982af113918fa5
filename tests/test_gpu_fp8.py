"""Parity of the FP8 E4M3 cache path (through the C ABI) with the CPU oracle.

Append codes each (token, kv head) row in float32 on both sides (scale =
amax / 448, nearest E4M3 value, ties to even), so the whole pool -- codes,
scales and the NaN-scale sentinel of unwritten slots -- is compared byte for
byte.  Attention is compared element by element with the oracle's attention
over the same codes and scales: max abs error <= 2e-2, the bar of a bf16
cache with float32 accumulation (the kernels widen codes exactly to bf16 and
round each softmax weight times its V scale to bf16 for the matrix cores).
Two codes of the format are NaN; slots past a context that hold them must
not reach any output.
"""
import math
import sys

import numpy as np
import pytest
import torch

import pins
import workloads
from oracle import attn as orc
from paged_kv_cache_381_amd import _lib as L
from paged_kv_cache_381_amd.engine import GpuWorkload, PagedKVCache
from workloads import prefill as PW

pytestmark = pytest.mark.gpu

TOL = 2e-2
NAME = "llama3_8b_b64_fp8"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_built = {}


def built(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _built:
        say(f"[build] {name} {kw}")
        inst = workloads.get(name) if not kw else workloads.configs.scaled(name, **kw).instantiate()
        _built[key] = (inst, GpuWorkload(inst))
        torch.cuda.synchronize()
    return _built[key]


def oracle_out(name, **kw):
    key = ("ref", name, tuple(sorted(kw.items())))
    if key not in _built:
        inst, _ = built(name, **kw)
        _built[key] = orc.run_workload(inst)
    return _built[key]


def check_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    say(f"  {what}: max abs err {err:.3e} (tol {tol})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"
    return err


def bf16_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


SMALL = [  # FP8 caches small enough for the oracle on every output
    (NAME, dict(batch=6, ctx_range=(1, 700))),
    (NAME, dict(batch=5, num_q_heads=64, ctx_range=(1, 300))),            # G = 8
    (NAME, dict(batch=4, num_q_heads=8, ctx_range=(1, 600))),             # G = 1
    (NAME, dict(batch=3, head_dim=64, ctx_range=(1, 300))),               # D = 64
    (NAME, dict(batch=5, num_q_heads=16, num_kv_heads=1, ctx_range=(30, 90))),  # G = 16
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_fp8_append_pool_bit_exact(case):
    name, kw = SMALL[case]
    inst, gw = built(name, **kw)
    ref = oracle_out(name, **kw)
    assert gw.step_slots.tolist() == ref["step_slots"]
    assert np.array_equal(gw.tables_host, ref["tables"])
    for got, want in ((gw.cache.k_pools[0], ref["kpool"]), (gw.cache.v_pools[0], ref["vpool"])):
        g = got.cpu().numpy()
        assert g.dtype == np.uint8 and g.shape == want.shape
        bad = np.flatnonzero(g != want)
        assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}"


def test_fp8_full_append_bit_exact():
    inst, gw = built(NAME)
    say(f"[append] {NAME}: oracle pool build")
    ref = orc.run_workload(inst, with_attention=False)
    for got, want in ((gw.cache.k_pools[0], ref["kpool"]), (gw.cache.v_pools[0], ref["vpool"])):
        assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("part", [32, 96, 512])
@pytest.mark.parametrize("wps", [1, 2])
def test_fp8_small_every_output(case, part, wps):
    name, kw = SMALL[case]
    inst, gw = built(name, **kw)
    ref = oracle_out(name, **kw)["out"]
    out = gw.decode(partition_tokens=part, waves_per_simd=wps).cpu().numpy()
    check_close(out, ref, TOL, f"{name} {kw} P={part} wps={wps}")


def test_fp8_full_workload_every_output():
    inst, gw = built(NAME)
    say(f"[oracle] {NAME}: {orc.num_threads()} threads")
    ref = orc.run_workload(inst)["out"]
    out = gw.decode().cpu().numpy()
    check_close(out, ref, TOL, f"{NAME} full")


def test_fp8_close_to_bf16_cache():
    """The same rows stored in bf16 and in FP8: outputs differ only by the
    quantisation (3 mantissa bits), far less than the outputs themselves."""
    kw = dict(batch=6, ctx_range=(1, 700))
    _, g8 = built(NAME, **kw)
    _, g16 = built("llama3_8b_b64", **kw)
    a = g8.decode().cpu().numpy()
    b = g16.decode().cpu().numpy()
    diff = np.abs(a - b).max()
    say(f"  fp8 vs bf16 cache: max abs diff {diff:.3e}, max |out| {np.abs(b).max():.3e}")
    assert diff <= 0.15


def test_fp8_every_code_decodes_exactly():
    """Every finite E4M3 code, placed as the V row of a one-token context
    under a scale of 1, comes back exactly (the softmax weight is 1) from
    decode and from prefill; the values are torch's float8_e4m3fn."""
    H, D = 1, 128
    c = PagedKVCache(4, H, D, "fp8")
    ids = [c.create(), c.create()]
    slots, _ = c.reserve(ids, 1)
    finite = np.array([x for x in range(256) if x & 0x7F != 0x7F], np.uint8)
    codes = np.zeros((2, D), np.uint8)
    codes.reshape(-1)[:finite.size] = finite
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    tb = c.layout.tile_bytes
    k = c.k_pools[0].cpu().numpy()
    v = c.v_pools[0].cpu().numpy()
    one = np.array([1.0], np.float32).view(np.uint8)
    for b in range(2):
        blk, t = int(slots[b]) // 16, int(slots[b]) % 16
        tile = blk * H * tb
        d = np.arange(D)
        k[tile + ((d // 16) * 16 + pins.int8_k_pos(t)) * 16 + d % 16] = 0
        v[tile + d * 16 + t] = codes[b]
        k[tile + 16 * D + 4 * t:tile + 16 * D + 4 * t + 4] = one
        v[tile + 16 * D + 4 * t:tile + 16 * D + 4 * t + 4] = one
    c.k_pools[0].copy_(torch.from_numpy(k))
    c.v_pools[0].copy_(torch.from_numpy(v))
    tables, ctx = c.tables(ids, 1)
    tdev, cdev = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    q = torch.zeros(2, 1, D, dtype=torch.bfloat16, device="cuda")
    out = torch.full((2, 1, D), 7.0, device="cuda")
    c.decode(0, out, q, tdev, cdev, 16, 1 / math.sqrt(D), c.workspace(2, 1, 16))
    got = out.cpu().numpy()[:, 0].astype(np.float64)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
    outp = torch.full((2, 1, D), 7.0, device="cuda")
    qstart = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    c.prefill(0, outp, q, tdev, cdev, qstart, 1, 16, 1 / math.sqrt(D))
    gotp = outp.cpu().numpy()[:, 0].astype(np.float64)
    assert np.array_equal(gotp, want), np.argwhere(gotp != want)[:8]


def _nan_filled_cache(num_blocks, H, D):
    """An FP8 cache whose every code byte is the NaN code 0x7F and every
    scale NaN before anything is appended."""
    c = PagedKVCache(num_blocks, H, D, "fp8", fill_nan=False)
    for t in (c.k_pools[0], c.v_pools[0]):
        tiles = t.view(-1, c.layout.tile_bytes)
        tiles[:, :16 * D].fill_(0x7F)
        sc = torch.full((tiles.shape[0], 16), float("nan"), dtype=torch.float32, device="cuda")
        tiles[:, 16 * D:] = sc.view(torch.uint8).view(tiles.shape[0], 64)
    return c


def test_fp8_nan_codes_past_context_are_masked():
    """Slots past each context hold NaN codes and NaN scales; decode (both
    waves-per-SIMD settings, several partitions) and prefill still match the
    oracle, which never reads those slots."""
    H, Hq, D = 2, 8, 128
    c = _nan_filled_cache(16, H, D)
    lens = [1, 15, 17, 33, 50, 64]
    ids = [c.create() for _ in lens]
    kpool, vpool = orc.new_pool(16, H, D, "fp8")
    kv = workloads.configs.normal_bits(17, (2, sum(lens), H, D), "bf16")
    at = 0
    for sid, n in zip(ids, lens):
        s, _ = c.reserve([sid], n)
        c.write(0, torch.from_numpy(s).cuda(), bf16_dev(kv[0, at:at + n]), bf16_dev(kv[1, at:at + n]))
        orc.append("fp8", H, D, kpool, vpool, kv[0, at:at + n], kv[1, at:at + n], s)
        at += n
    tables, ctx = c.tables(ids, 4)
    tdev, cdev = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    q = workloads.configs.normal_bits(18, (len(lens), Hq, D), "bf16")
    ref = orc.paged_attention("fp8", q, kpool, vpool, tables, ctx, H, 1 / math.sqrt(D))
    for part in (32, 64):
        for wps in (1, 2):
            out = torch.full((len(lens), Hq, D), 7.0, device="cuda")
            c.decode(0, out, bf16_dev(q), tdev, cdev, 64, 1 / math.sqrt(D), c.workspace(len(lens), Hq, 64, part),
                     partition_tokens=part, waves_per_simd=wps)
            check_close(out.cpu().numpy(), ref, TOL, f"fp8 NaN tails P={part} wps={wps}")
    # prefill of each sequence's last min(n, 20) tokens
    nq = np.minimum(np.asarray(lens), 20)
    qstart = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qp = workloads.configs.normal_bits(19, (int(qstart[-1]), Hq, D), "bf16")
    refp = orc.paged_prefill("fp8", qp, kpool, vpool, tables, ctx, qstart, H, 1 / math.sqrt(D))
    outp = torch.full((int(qstart[-1]), Hq, D), 7.0, device="cuda")
    c.prefill(0, outp, bf16_dev(qp), tdev, cdev, torch.from_numpy(qstart).cuda(), int(nq.max()), 64,
              1 / math.sqrt(D))
    check_close(outp.cpu().numpy(), refp, TOL, "fp8 NaN tails prefill")


def test_fp8_special_rows_and_padding():
    """All-zero rows (scale 0), rows with one large element (its code 448;
    in the K row the rest code as subnormals or zero), a padding sequence with
    no tokens (zeros out), and NaN scales in unused slots."""
    H, Hq, D = 2, 8, 128
    c = PagedKVCache(8, H, D, "fp8")
    kpool, vpool = orc.new_pool(8, H, D, "fp8")
    ids = [c.create(), c.create()]
    s, _ = c.reserve([ids[1]], 37)
    kv = workloads.configs.normal_bits(5, (2, 37, H, D), "bf16")
    kv[:, 3] = 0                         # all-zero rows: scale 0, codes 0
    kv[0, 7, 0, 5] = np.uint16(0x4780)   # 65536.0 in one element of a K row: the rest code as subnormals
    kv[1, 9, 1, 0] = np.uint16(0xC2FE)   # -127.0 in one element of a V row (a larger V would put the
    #                                      bf16 rounding of weight x scale above the absolute bar)
    c.write(0, torch.from_numpy(s).cuda(), bf16_dev(kv[0]), bf16_dev(kv[1]))
    orc.append("fp8", H, D, kpool, vpool, kv[0], kv[1], s)
    assert np.array_equal(c.k_pools[0].cpu().numpy(), kpool)
    assert np.array_equal(c.v_pools[0].cpu().numpy(), vpool)
    tables, ctx = c.tables(ids, 3)
    q = workloads.configs.normal_bits(6, (2, Hq, D), "bf16")
    out = torch.full((2, Hq, D), 7.0, device="cuda")
    ws = c.workspace(2, Hq, 37)
    c.decode(0, out, bf16_dev(q), torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), 37,
             1 / math.sqrt(D), ws)
    o = out.cpu().numpy()
    assert (o[0] == 0).all()
    ref = orc.paged_attention("fp8", q, kpool, vpool, tables, ctx, H, 1 / math.sqrt(D))
    check_close(o, ref, TOL, "fp8 special rows")


def test_fp8_copy_blocks_bit_exact():
    """Copying FP8 blocks moves codes and scales byte for byte."""
    H, D = 2, 64
    c = PagedKVCache(6, H, D, "fp8")
    kpool, vpool = orc.new_pool(6, H, D, "fp8")
    sid = c.create()
    s, _ = c.reserve([sid], 40)
    kv = workloads.configs.normal_bits(9, (2, 40, H, D), "bf16")
    c.write(0, torch.from_numpy(s).cuda(), bf16_dev(kv[0]), bf16_dev(kv[1]))
    orc.append("fp8", H, D, kpool, vpool, kv[0], kv[1], s)
    used = sorted({int(x) // 16 for x in s})
    free = [b for b in range(6) if b not in used]
    pairs = np.array([[used[0], free[0]], [used[2], free[1]]], np.int32)
    L.pkv_copy_blocks(c.layout, c.k_pools[0], c.v_pools[0], torch.from_numpy(pairs).cuda())
    orc.copy_blocks("fp8", H, D, kpool, vpool, pairs)
    assert np.array_equal(c.k_pools[0].cpu().numpy(), kpool)
    assert np.array_equal(c.v_pools[0].cpu().numpy(), vpool)


def test_fp8_deterministic_and_placement_invariant():
    name, kw = NAME, dict(batch=6, ctx_range=(1, 700))
    inst, gw = built(name, **kw)
    a = gw.decode().clone()
    assert torch.equal(a, gw.decode().clone())
    inst2 = workloads.configs.scaled(name, **kw).instantiate()
    inst2.free_order = np.arange(inst2.num_blocks, dtype=np.int32)
    gw2 = GpuWorkload(inst2)
    assert not np.array_equal(gw.tables_host, gw2.tables_host)
    for wps in (1, 2):
        assert torch.equal(gw.decode(waves_per_simd=wps).clone(), gw2.decode(waves_per_simd=wps).clone())


def test_fp8_rejects_wavefront_kernel():
    c = PagedKVCache(4, 1, 64, "fp8")
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 4, 64, device="cuda")
    tables = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = c.workspace(1, 4, 16, 0, 1)
    with pytest.raises(L.PagedKVError) as e:
        c.decode(0, out, q, tables, ctx, 16, 0.125, ws, kernel=1)
    assert e.value.name == "INVALID"


def test_fp8_long_prompt_prefill():
    """Prompts of 300+ new tokens after private prefixes: pools byte for byte
    and prefill outputs against the oracle."""
    inst = PW.scaled("prefill_8b_b4", batch=2, own_prefix=(0, 40), new_tokens=(300, 340), cache="fp8").instantiate()
    from paged_kv_cache_381_amd.engine import GpuPrefill
    say(f"[prefill fp8] nq {inst.nq.tolist()} ctx {inst.ctx.tolist()}")
    gp = GpuPrefill(inst)
    ref = orc.run_prefill(inst)
    assert np.array_equal(gp.cache.k_pools[0].cpu().numpy(), ref["kpool"])
    assert np.array_equal(gp.cache.v_pools[0].cpu().numpy(), ref["vpool"])
    check_close(gp.run().cpu().numpy(), ref["out"], TOL, "fp8 prefill")
