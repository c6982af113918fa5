"""Pins of the CPU oracle: checks against facts fixed by the pages or by
mathematics, never against the oracle itself.

Each ``check_*`` function raises AssertionError when the oracle is wrong.
``test_oracle_attention.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on deliberately broken copies of it, to
show that a plausible mistake anywhere in the oracle fails at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import attn as orc
from oracle.book import Book
from workloads.configs import normal_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements -> float64, computed here independently of the oracle."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


class Problem:
    """A small paged decode problem built with the oracle's own bookkeeping
    and append: logical K/V per sequence, pools, tables, lengths."""

    def __init__(self, dtype, B, Hq, Hkv, D, ctx, num_blocks, seed, identity=False, kv=None, q=None):
        self.dtype, self.B, self.Hq, self.Hkv, self.D = dtype, B, Hq, Hkv, D
        self.ctx = np.asarray(ctx, dtype=np.int32)
        rng = np.random.default_rng(seed)
        order = np.arange(num_blocks) if identity else rng.permutation(num_blocks)
        self.book = Book(num_blocks, order)
        self.ids = [self.book.create() for _ in range(B)]
        rt = orc.ROW[dtype]
        if kv is None:
            kv = [(normal_bits(seed * 7919 + 2 * b, (int(ctx[b]), Hkv, D), rt),
                   normal_bits(seed * 7919 + 2 * b + 1, (int(ctx[b]), Hkv, D), rt)) for b in range(B)]
        self.kv = kv
        self.q = normal_bits(seed * 7919 + 99991, (B, Hq, D), rt) if q is None else q
        self.kpool, self.vpool = orc.new_pool(num_blocks, Hkv, D, dtype)
        for b, sid in enumerate(self.ids):
            slots, _ = self.book.append_slots(sid, int(ctx[b]))
            orc.append(dtype, Hkv, D, self.kpool, self.vpool, kv[b][0], kv[b][1], np.asarray(slots))
        self.tables, got_ctx = orc.tables_of(self.book, self.ids)
        assert (got_ctx == self.ctx).all()
        self.scale = 1.0 / math.sqrt(D)

    def paged(self):
        return orc.paged_attention(self.dtype, self.q, self.kpool, self.vpool, self.tables, self.ctx,
                                   self.Hkv, self.scale)

    def contiguous(self, b):
        k, v = self.kv[b]
        return orc.contiguous_attention(self.dtype, self.q[b], k, v, self.scale)


def int8_tile_bytes(D):
    return 16 * D + 64


def int8_k_pos(t):
    """Unit of token slot t along a K row of a one-byte tile: slots 0-3,
    8-11, 4-7, 12-15 in that order (tests/golden/pool_layout_int8.txt)."""
    order = [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]
    return order.index(t)


def int8_read(pool, H, D, blk, g, t, is_v):
    """(codes[D], scale) of slot t of tile (blk, g) of an int8 pool, read with
    the byte layout of tests/golden/pool_layout_int8.txt."""
    tb = int8_tile_bytes(D)
    tile = pool[(blk * H + g) * tb:(blk * H + g + 1) * tb]
    d = np.arange(D)
    at = d * 16 + t if is_v else ((d // 16) * 16 + int8_k_pos(t)) * 16 + d % 16
    codes = tile[at].view(np.int8).astype(np.int64)
    scale = tile[16 * D + 4 * t:16 * D + 4 * t + 4].view(np.float32)[0]
    return codes, scale


def fp8_read(pool, H, D, blk, g, t, is_v):
    """(values[D], scale) of slot t of tile (blk, g) of an FP8 pool: the same
    byte layout as an int8 pool, each code decoded by torch's float8_e4m3fn
    (the OCP E4M3 format) rather than by the oracle."""
    tb = int8_tile_bytes(D)
    tile = pool[(blk * H + g) * tb:(blk * H + g + 1) * tb]
    d = np.arange(D)
    at = d * 16 + t if is_v else ((d // 16) * 16 + int8_k_pos(t)) * 16 + d % 16
    codes = np.ascontiguousarray(tile[at])
    values = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    scale = tile[16 * D + 4 * t:16 * D + 4 * t + 4].view(np.float32)[0]
    return values, scale, codes


def brute_attention(q, K, V, scale):
    """Textbook softmax attention of one query row in pure Python floats
    with exactly rounded sums (math.fsum) and no max subtraction."""
    n, D = len(K), len(q)
    s = [scale * math.fsum(q[d] * K[j][d] for d in range(D)) for j in range(n)]
    e = [math.exp(x) for x in s]
    z = math.fsum(e)
    return [math.fsum(e[j] * V[j][d] for j in range(n)) / z for d in range(D)]


# --------------------------------------------------------------------------
def check_brute_force():
    """Oracle == exactly-summed textbook attention on tiny inputs."""
    for dtype in ("f32", "bf16"):
        p = Problem(dtype, 3, 4, 2, 8, [1, 17, 40], 12, seed=11)
        out = p.paged()
        G = p.Hq // p.Hkv
        for b in range(p.B):
            K, V = widen(p.kv[b][0], dtype), widen(p.kv[b][1], dtype)
            for h in range(p.Hq):
                ref = brute_attention(list(widen(p.q[b, h], dtype)), K[:, h // G, :].tolist(),
                                      V[:, h // G, :].tolist(), p.scale)
                err = np.abs(out[b, h] - np.asarray(ref)).max()
                assert err <= 1e-13, (dtype, b, h, err)


def check_library_sdpa():
    """Oracle == torch's scaled_dot_product_attention in float64 on the
    contiguous cache, with its grouped-query option (h -> h // G)."""
    p = Problem("bf16", 2, 8, 2, 64, [100, 257], 30, seed=5)
    out = p.paged()
    for b in range(p.B):
        q = torch.from_numpy(widen(p.q[b], "bf16"))[None, :, None, :]            # [1,Hq,1,D]
        k = torch.from_numpy(widen(p.kv[b][0], "bf16")).permute(1, 0, 2)[None]    # [1,Hkv,n,D]
        v = torch.from_numpy(widen(p.kv[b][1], "bf16")).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(),
                                                               scale=p.scale, enable_gqa=True)
        err = np.abs(out[b] - ref[0, :, 0, :].numpy()).max()
        assert err <= 1e-12, (b, err)


def check_paged_equals_contiguous():
    """Shuffled physical blocks give exactly the contiguous-cache result."""
    for dtype in ("f32", "bf16"):
        p = Problem(dtype, 4, 4, 4, 16, [1, 16, 33, 100], 20, seed=3)
        out = p.paged()
        for b in range(p.B):
            assert np.array_equal(out[b], p.contiguous(b)), (dtype, b)


def check_placement_invariance():
    """Identity and shuffled block hand-out orders give bitwise-equal results."""
    a = Problem("bf16", 3, 8, 2, 32, [5, 48, 70], 16, seed=9, identity=True)
    b = Problem("bf16", 3, 8, 2, 32, [5, 48, 70], 16, seed=9, identity=False)
    assert not np.array_equal(a.tables, b.tables)
    assert np.array_equal(a.paged(), b.paged())


def check_special_cases():
    dt = "f32"
    # One cached token: the softmax weight is exactly 1, so out == v.
    p = Problem(dt, 2, 2, 2, 8, [1, 1], 4, seed=21)
    out = p.paged()
    for b in range(2):
        for h in range(2):
            assert np.array_equal(out[b, h], widen(p.kv[b][1][0, h], dt))
    # Every key identical: uniform weights, so out == mean of V.
    n = 37
    k1 = normal_bits(77, (1, 1, 8), dt)
    K = np.repeat(k1, n, axis=0)
    V = normal_bits(78, (n, 1, 8), dt)
    p = Problem(dt, 1, 1, 1, 8, [n], 4, seed=22, kv=[(K, V)])
    out = p.paged()[0, 0]
    mean = np.array([math.fsum(widen(V[:, 0, d], dt)) / n for d in range(8)])
    assert np.abs(out - mean).max() <= 1e-13
    # One key far more aligned with q than the rest: out ~= its value row.
    q = np.zeros((1, 1, 8), np.float32)
    q[0, 0, 0] = 1.0
    K = normal_bits(79, (n, 1, 8), dt)
    K[13, 0, :] = 0.0
    for big in (400.0, 4000.0):  # the second puts the top score far past exp's range
        K[13, 0, 0] = big
        p = Problem(dt, 1, 1, 1, 8, [n], 4, seed=23, kv=[(K, V)], q=q)
        assert np.abs(p.paged()[0, 0] - widen(V[13, 0], dt)).max() <= 1e-12
    # Adding one vector c to every key shifts all scores by q.c: no change.
    K = normal_bits(80, (n, 1, 8), dt)
    c = normal_bits(81, (1, 1, 8), dt)
    K2 = (K.astype(np.float64) + c.astype(np.float64)).astype(np.float32)
    q = normal_bits(82, (1, 1, 8), dt)
    base = Problem(dt, 1, 1, 1, 8, [n], 4, seed=24, kv=[(K2, V)], q=q).paged()[0, 0]
    # reference: the same problem with the exact shifted keys computed in float64 by brute force
    qs = widen(q[0, 0], dt).tolist()
    ref = brute_attention(qs, widen(K2[:, 0], dt).tolist(), widen(V[:, 0], dt).tolist(), 1 / math.sqrt(8))
    assert np.abs(base - np.asarray(ref)).max() <= 1e-13
    ref_shift = brute_attention(qs, (widen(K2[:, 0], dt) - widen(c[0, 0], dt)[None]).tolist(),
                                widen(V[:, 0], dt).tolist(), 1 / math.sqrt(8))
    assert np.abs(base - np.asarray(ref_shift)).max() <= 1e-12
    # Reordering the cached tokens (keys with their values) changes nothing.
    perm = np.random.default_rng(5).permutation(n)
    pa = Problem(dt, 1, 1, 1, 8, [n], 4, seed=25, kv=[(K, V)], q=q).paged()[0, 0]
    pb = Problem(dt, 1, 1, 1, 8, [n], 4, seed=25, kv=[(K[perm].copy(), V[perm].copy())], q=q).paged()[0, 0]
    assert np.abs(pa - pb).max() <= 1e-14


def check_merge_identity():
    """Any split of the context into 16-token-aligned spans, merged by
    log-sum-exp, equals the single-pass result."""
    p = Problem("bf16", 3, 8, 2, 32, [16, 300, 1000], 100, seed=31)
    ref = p.paged()
    for P in (16, 32, 48, 512):
        out = orc.partitioned_attention("bf16", p.q, p.kpool, p.vpool, p.tables, p.ctx, p.Hkv, p.scale, P)
        assert np.abs(out - ref).max() <= 1e-13, P


def check_gqa_reduces_to_mha():
    """Grouped-query attention == multi-head attention whose kv heads are
    repeated per group of h_q / h_kv consecutive query heads."""
    Hq, Hkv, D, n = 8, 2, 16, 50
    K = normal_bits(41, (n, Hkv, D), "bf16")
    V = normal_bits(42, (n, Hkv, D), "bf16")
    q = normal_bits(43, (1, Hq, D), "bf16")
    gqa = Problem("bf16", 1, Hq, Hkv, D, [n], 8, seed=44, kv=[(K, V)], q=q).paged()
    Kr = np.repeat(K, Hq // Hkv, axis=1).copy()
    Vr = np.repeat(V, Hq // Hkv, axis=1).copy()
    mha = Problem("bf16", 1, Hq, Hq, D, [n], 8, seed=44, kv=[(Kr, Vr)], q=q).paged()
    assert np.array_equal(gqa, mha)
    # and the groups do read different heads
    assert np.abs(gqa[0, 0] - gqa[0, Hq - 1]).max() > 1e-3


def check_append_roundtrip():
    """Every appended token reads back bit-for-bit through its block table;
    slots never written keep the sentinel; whole-block copies are exact."""
    for dtype in ("f32", "bf16"):
        p = Problem(dtype, 3, 4, 2, 16, [1, 16, 45], 8, seed=51, identity=True)
        written = 0
        for b in range(p.B):
            for j in range(int(p.ctx[b])):
                k, v = orc.gather_token(dtype, p.Hkv, p.D, p.kpool, p.vpool, p.tables[b], j)
                assert np.array_equal(k, widen(p.kv[b][0][j], dtype))
                assert np.array_equal(v, widen(p.kv[b][1][j], dtype))
                written += 1
        for pool in (p.kpool, p.vpool):
            nan = np.isnan(widen(pool, dtype))
            assert int((~nan).sum()) == written * p.Hkv * p.D
        k0, v0 = p.kpool.copy(), p.vpool.copy()
        src = int(p.tables[2][1])
        dst = int(p.book.free[-1])
        orc.copy_blocks(dtype, p.Hkv, p.D, p.kpool, p.vpool, [(src, dst)])
        blk = p.Hkv * 16 * p.D
        for pool, old in ((p.kpool, k0), (p.vpool, v0)):
            assert np.array_equal(pool[dst * blk:(dst + 1) * blk], old[src * blk:(src + 1) * blk])
            rest = np.ones(pool.size, bool)
            rest[dst * blk:(dst + 1) * blk] = False
            assert np.array_equal(pool[rest].view(np.uint8 if dtype == "bf16" else np.uint32),
                                  old[rest].view(np.uint8 if dtype == "bf16" else np.uint32))


def check_layout_golden():
    """The flat pool indices of hand-worked examples (tests/golden/pool_layout.txt)."""
    H, D = 2, 16
    for dtype, slot, head, d, ki, vi in read_golden("pool_layout.txt"):
        slot, head, d, ki, vi = int(slot), int(head), int(d), int(ki), int(vi)
        kpool, vpool = orc.new_pool(slot // 16 + 1, H, D, dtype)
        kn = np.zeros((1, H, D), np.float32)
        kn[0, head, d] = 3.0
        vn = np.zeros((1, H, D), np.float32)
        vn[0, head, d] = 5.0
        if dtype == "bf16":
            kn = (kn.view(np.uint32) >> 16).astype(np.uint16)
            vn = (vn.view(np.uint32) >> 16).astype(np.uint16)
        orc.append(dtype, H, D, kpool, vpool, kn, vn, np.array([slot]))
        kw, vw = widen(kpool, dtype), widen(vpool, dtype)
        assert np.flatnonzero(kw == 3.0).tolist() == [ki], (dtype, slot, head, d)
        assert np.flatnonzero(vw == 5.0).tolist() == [vi], (dtype, slot, head, d)


def check_rejects_per_page_softmax():
    """The per-page softmax of the vendor article's pseudo-code
    [PagedAttention：大模型KV Cache内存管理革新 §3.2] agrees with the oracle
    only while the context fits in one page; beyond that the oracle keeps one
    softmax over the whole context."""
    p = Problem("f32", 2, 1, 1, 16, [16, 80], 8, seed=61)
    out = p.paged()
    for b in range(p.B):
        K, V = widen(p.kv[b][0][:, 0], "f32"), widen(p.kv[b][1][:, 0], "f32")
        q = widen(p.q[b, 0], "f32")
        acc = np.zeros(16)
        for s0 in range(0, int(p.ctx[b]), 16):
            s = K[s0:s0 + 16] @ q * p.scale
            w = np.exp(s - s.max())
            acc += (w / w.sum()) @ V[s0:s0 + 16]
        diff = np.abs(out[b, 0] - acc).max()
        if p.ctx[b] <= 16:
            assert diff <= 1e-13
        else:
            assert diff > 1e-2


def _bf16_bits(values):
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert ((bits & 0xFFFF) == 0).all(), "golden values must be bfloat16-exact"
    return (bits >> 16).astype(np.uint16)


def check_int8_quant_golden():
    """Append of hand-worked rows stores the hand-worked codes and scale
    (tests/golden/int8_quant_example.txt), in both pools."""
    H, D = 1, 16
    for label, scale_hex, _, *rest in read_golden("int8_quant_example.txt"):
        values = [float(x) for x in rest[:16]]
        codes = [int(x) for x in rest[17:33]]
        assert rest[16] == "|" and len(codes) == 16
        want_scale = np.array([int(scale_hex, 16)], np.uint32).view(np.float32)[0]
        kpool, vpool = orc.new_pool(2, H, D, "int8")
        row = _bf16_bits(values).reshape(1, 1, D)
        orc.append("int8", H, D, kpool, vpool, row, row, np.array([16 + 6]))
        for pool, is_v in ((kpool, False), (vpool, True)):
            got, sc = int8_read(pool, H, D, 1, 0, 6, is_v)
            assert got.tolist() == codes, (label, is_v, got.tolist())
            assert sc.view(np.uint32) == want_scale.view(np.uint32), (label, is_v, sc)


def check_int8_layout_golden():
    """Byte offsets of codes and scales in an int8 pool for hand-worked slots
    (tests/golden/pool_layout_int8.txt)."""
    H, D = 2, 32
    for slot, head, d, kb, vb, sb in read_golden("pool_layout_int8.txt"):
        slot, head, d, kb, vb, sb = (int(x) for x in (slot, head, d, kb, vb, sb))
        kpool, vpool = orc.new_pool(slot // 16 + 1, H, D, "int8")
        row = np.zeros((1, H, D), np.float32)
        row[0, head, d] = 3.0
        bits = _bf16_bits(row)
        orc.append("int8", H, D, kpool, vpool, bits, bits, np.array([slot]))
        tb = int8_tile_bytes(D)
        is_code = (np.arange(kpool.size) % tb) < 16 * D  # scale bytes (NaN sentinel) hold 0x7f too
        assert np.flatnonzero((kpool == 127) & is_code).tolist() == [kb], (slot, head, d)
        assert np.flatnonzero((vpool == 127) & is_code).tolist() == [vb], (slot, head, d)
        want = np.float32(3.0) / np.float32(127.0)
        for pool in (kpool, vpool):
            assert pool[sb:sb + 4].view(np.float32)[0] == want
        # the other head of the same slot was written with an all-zero row
        other = sb + (1 - 2 * head) * tb
        for pool in (kpool, vpool):
            assert pool[other:other + 4].view(np.float32)[0] == 0.0


def check_int8_quant_error_bound():
    """Every appended row of an int8 cache: |x - code*scale| <= scale/2 (up to
    the float32 rounding of x/scale), the largest |code| is 127, codes keep
    the sign of x; slots never written read NaN."""
    p = Problem("int8", 3, 4, 2, 32, [1, 16, 45], 8, seed=71, identity=True)
    for b in range(p.B):
        for j in range(int(p.ctx[b])):
            blk, t = int(p.tables[b][j // 16]), j % 16
            for g in range(p.Hkv):
                for which, pool in ((0, p.kpool), (1, p.vpool)):
                    x = widen(p.kv[b][which][j, g], "bf16")
                    codes, sc = int8_read(pool, p.Hkv, p.D, blk, g, t, which == 1)
                    sc = float(sc)
                    assert abs(sc - np.abs(x).max() / 127) <= 1e-6 * sc
                    err = np.abs(x - codes * sc)
                    assert (err <= 0.5 * sc * (1 + 2.0 ** -16)).all(), (b, j, g, which, err.max() / sc)
                    assert np.abs(codes).max() == 127
                    assert (codes * x >= 0).all()
    # a slot past the last token of sequence 0 is still the sentinel
    k, v = orc.gather_token("int8", p.Hkv, p.D, p.kpool, p.vpool, p.tables[0], 1)
    assert np.isnan(k).all() and np.isnan(v).all()


def check_int8_brute_force():
    """Attention over an int8 cache == exactly-summed textbook attention over
    the dequantised values (code * scale, decoded here from the bytes), for
    shuffled blocks, and it stays within the quantisation error of the same
    problem stored in bfloat16."""
    p = Problem("int8", 3, 4, 2, 16, [1, 17, 40], 12, seed=81)
    out = p.paged()
    G = p.Hq // p.Hkv
    ref16 = Problem("bf16", 3, 4, 2, 16, [1, 17, 40], 12, seed=81).paged()
    for b in range(p.B):
        n = int(p.ctx[b])
        for g in range(p.Hkv):
            K, V = [], []
            for j in range(n):
                blk, t = int(p.tables[b][j // 16]), j % 16
                kc, ks = int8_read(p.kpool, p.Hkv, p.D, blk, g, t, False)
                vc, vs = int8_read(p.vpool, p.Hkv, p.D, blk, g, t, True)
                K.append((kc * float(ks)).tolist())
                V.append((vc * float(vs)).tolist())
            for h in range(g * G, (g + 1) * G):
                ref = brute_attention(list(widen(p.q[b, h], "bf16")), K, V, p.scale)
                err = np.abs(out[b, h] - np.asarray(ref)).max()
                assert err <= 1e-13, (b, h, err)
    assert np.abs(out - ref16).max() <= 0.05
    # the split pass merges to the same result on an int8 cache too
    part = orc.partitioned_attention("int8", p.q, p.kpool, p.vpool, p.tables, p.ctx, p.Hkv, p.scale, 16)
    assert np.abs(part - out).max() <= 1e-13


def check_int8_copy_blocks():
    """Copying an int8 block moves its codes and scales byte for byte."""
    p = Problem("int8", 2, 2, 2, 32, [20, 33], 8, seed=91, identity=True)
    src = int(p.tables[1][1])
    dst = int(p.book.free[-1])
    k0, v0 = p.kpool.copy(), p.vpool.copy()
    orc.copy_blocks("int8", p.Hkv, p.D, p.kpool, p.vpool, [(src, dst)])
    blk = p.Hkv * int8_tile_bytes(p.D)
    for pool, old in ((p.kpool, k0), (p.vpool, v0)):
        assert np.array_equal(pool[dst * blk:(dst + 1) * blk], old[src * blk:(src + 1) * blk])
        rest = np.ones(pool.size, bool)
        rest[dst * blk:(dst + 1) * blk] = False
        assert np.array_equal(pool[rest], old[rest])


def check_fp8_quant_golden():
    """Append of hand-worked rows stores the hand-worked E4M3 codes and scale
    (tests/golden/fp8_quant_example.txt), in both pools."""
    H, D = 1, 16
    for label, scale_hex, _, *rest in read_golden("fp8_quant_example.txt"):
        values = [float(x) for x in rest[:16]]
        codes = [int(x) for x in rest[17:33]]
        assert rest[16] == "|" and len(codes) == 16
        want_scale = np.array([int(scale_hex, 16)], np.uint32).view(np.float32)[0]
        kpool, vpool = orc.new_pool(2, H, D, "fp8")
        row = _bf16_bits(values).reshape(1, 1, D)
        orc.append("fp8", H, D, kpool, vpool, row, row, np.array([16 + 6]))
        for pool, is_v in ((kpool, False), (vpool, True)):
            _, sc, got = fp8_read(pool, H, D, 1, 0, 6, is_v)
            assert got.tolist() == codes, (label, is_v, got.tolist())
            assert sc.view(np.uint32) == want_scale.view(np.uint32), (label, is_v, sc)


def _fp8_pool_with_codes(codes, D):
    """A one-block FP8 pool (one kv head) whose slot t holds codes[t] under a
    scale of exactly 1, written byte by byte (K layout in the K pool, V layout
    in the V pool)."""
    kpool, vpool = orc.new_pool(1, 1, D, "fp8")
    for t in range(16):
        d = np.arange(D)
        kpool[((d // 16) * 16 + int8_k_pos(t)) * 16 + d % 16] = codes[t]
        vpool[d * 16 + t] = codes[t]
        one = np.array([1.0], np.float32).view(np.uint8)
        kpool[16 * D + 4 * t:16 * D + 4 * t + 4] = one
        vpool[16 * D + 4 * t:16 * D + 4 * t + 4] = one
    return kpool, vpool


def check_fp8_decode_library():
    """The oracle's value of every finite E4M3 code equals torch's
    float8_e4m3fn widening of the same byte (the two NaN codes are never
    written by append and are left out)."""
    D = 16
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    want = torch.from_numpy(finite.copy()).view(torch.float8_e4m3fn).double().numpy()
    for i0 in range(0, finite.size, 16 * D):
        chunk = np.zeros(16 * D, np.uint8)
        n = min(16 * D, finite.size - i0)
        chunk[:n] = finite[i0:i0 + n]
        codes = chunk.reshape(16, D)
        kpool, vpool = _fp8_pool_with_codes(codes, D)
        for t in range(16):
            k, v = orc.gather_token("fp8", 1, D, kpool, vpool, np.array([0]), t)
            for got in (k[0], v[0]):
                for d in range(D):
                    i = t * D + d
                    if i < n:
                        assert got[d] == want[i0 + i], (hex(finite[i0 + i]), got[d], want[i0 + i])


def check_fp8_encode_library():
    """For values of every binade of E4M3, subnormals, exact ties and the
    largest value, the code append stores equals torch's round-to-nearest-even
    float8_e4m3fn cast (a row holding 448 has a scale of exactly 1, so each
    element is encoded as it is)."""
    H, D = 1, 64
    rng = np.random.default_rng(1234)
    vals = []
    for e in range(-9, 9):
        vals += list((rng.random(24) + 1.0) * 2.0 ** e)
    grid = [(k + 0.5) * 2.0 ** -9 for k in range(16)] + [m * 2.0 ** e for e in range(-6, 8)
                                                         for m in (1.0625, 1.1875, 1.3125, 1.9375)]
    vals = np.asarray(vals + grid)
    vals = vals[vals < 448.0] * np.where(rng.random(vals[vals < 448.0].size) < 0.5, -1.0, 1.0)
    bits = (np.asarray(vals, np.float32).view(np.uint32) + 0x8000) & 0xFFFF0000   # bfloat16-exact
    vals = bits.view(np.float32)
    vals = vals[np.abs(vals) < 448.0]
    rows = []
    for i0 in range(0, vals.size, D - 1):
        row = np.zeros(D, np.float32)
        part = vals[i0:i0 + D - 1]
        row[:part.size] = part
        row[D - 1] = 448.0
        rows.append(row)
    rows = np.stack(rows)
    want = torch.from_numpy(rows).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    n = rows.shape[0]
    kpool, vpool = orc.new_pool((n + 15) // 16, H, D, "fp8")
    orc.append("fp8", H, D, kpool, vpool, _bf16_bits(rows).reshape(n, 1, D), _bf16_bits(rows).reshape(n, 1, D),
               np.arange(n))
    for r in range(n):
        for pool, is_v in ((kpool, False), (vpool, True)):
            _, sc, got = fp8_read(pool, H, D, r // 16, 0, r % 16, is_v)
            assert float(sc) == 1.0
            assert np.array_equal(got, want[r]), (r, is_v, rows[r][got != want[r]])


def check_fp8_quant_error_bound():
    """Every appended row of an FP8 cache: scale = amax / 448, the largest
    code is 448, codes keep the sign, and |x / scale - value(code)| is at
    most half the E4M3 spacing at |x / scale| (2^-4 of the binade's base for
    normals, 2^-10 below 2^-6), up to the float32 rounding of x / scale."""
    p = Problem("fp8", 3, 4, 2, 32, [1, 16, 45], 8, seed=72, identity=True)
    for b in range(p.B):
        for j in range(int(p.ctx[b])):
            blk, t = int(p.tables[b][j // 16]), j % 16
            for g in range(p.Hkv):
                for which, pool in ((0, p.kpool), (1, p.vpool)):
                    x = widen(p.kv[b][which][j, g], "bf16")
                    vals, sc, _ = fp8_read(pool, p.Hkv, p.D, blk, g, t, which == 1)
                    sc = float(sc)
                    assert abs(sc - np.abs(x).max() / 448) <= 1e-6 * sc
                    y = x / sc
                    base = 2.0 ** np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -30))), -6)
                    assert (np.abs(y - vals) <= base / 16 * (1 + 2.0 ** -16) + 1e-12).all(), (b, j, g, which)
                    assert np.abs(vals).max() == 448.0
                    assert (vals * x >= 0).all()
    k, v = orc.gather_token("fp8", p.Hkv, p.D, p.kpool, p.vpool, p.tables[0], 1)
    assert np.isnan(k).all() and np.isnan(v).all()


def check_fp8_brute_force():
    """Attention over an FP8 cache == exactly-summed textbook attention over
    the values torch decodes from the bytes times the scales, for shuffled
    blocks; the split pass merges to the same result; it stays within the
    quantisation error of the same problem stored in bfloat16."""
    p = Problem("fp8", 3, 4, 2, 16, [1, 17, 40], 12, seed=82)
    out = p.paged()
    G = p.Hq // p.Hkv
    ref16 = Problem("bf16", 3, 4, 2, 16, [1, 17, 40], 12, seed=82).paged()
    for b in range(p.B):
        n = int(p.ctx[b])
        for g in range(p.Hkv):
            K, V = [], []
            for j in range(n):
                blk, t = int(p.tables[b][j // 16]), j % 16
                kv_, ks, _ = fp8_read(p.kpool, p.Hkv, p.D, blk, g, t, False)
                vv_, vs, _ = fp8_read(p.vpool, p.Hkv, p.D, blk, g, t, True)
                K.append((kv_ * float(ks)).tolist())
                V.append((vv_ * float(vs)).tolist())
            for h in range(g * G, (g + 1) * G):
                ref = brute_attention(list(widen(p.q[b, h], "bf16")), K, V, p.scale)
                assert np.abs(out[b, h] - np.asarray(ref)).max() <= 1e-13, (b, h)
    assert np.abs(out - ref16).max() <= 0.15
    part = orc.partitioned_attention("fp8", p.q, p.kpool, p.vpool, p.tables, p.ctx, p.Hkv, p.scale, 16)
    assert np.abs(part - out).max() <= 1e-13


class PrefillProblem:
    """Sequences whose last nq_b of ctx_b tokens are new (queries), stored
    with the oracle's own bookkeeping and append; queries packed by row."""

    def __init__(self, dtype, Hq, Hkv, D, ctx, nq, num_blocks, seed, kv=None):
        self.dtype, self.Hq, self.Hkv, self.D = dtype, Hq, Hkv, D
        self.ctx = np.asarray(ctx, np.int32)
        self.nq = np.asarray(nq, np.int32)
        self.qstart = np.concatenate([[0], np.cumsum(self.nq)]).astype(np.int32)
        B = len(ctx)
        rt = orc.ROW[dtype]
        rng = np.random.default_rng(seed)
        self.book = Book(num_blocks, rng.permutation(num_blocks))
        self.ids = [self.book.create() for _ in range(B)]
        self.kv = kv or [(normal_bits(seed * 31 + 2 * b, (int(ctx[b]), Hkv, D), rt),
                          normal_bits(seed * 31 + 2 * b + 1, (int(ctx[b]), Hkv, D), rt)) for b in range(B)]
        self.q = normal_bits(seed * 31 + 777, (int(self.qstart[-1]), Hq, D), rt)
        self.kpool, self.vpool = orc.new_pool(num_blocks, Hkv, D, dtype)
        for b, sid in enumerate(self.ids):
            slots, _ = self.book.append_slots(sid, int(ctx[b]))
            orc.append(dtype, Hkv, D, self.kpool, self.vpool, self.kv[b][0], self.kv[b][1], np.asarray(slots))
        self.tables, _ = orc.tables_of(self.book, self.ids)
        self.scale = 1.0 / math.sqrt(D)

    def out(self):
        return orc.paged_prefill(self.dtype, self.q, self.kpool, self.vpool, self.tables, self.ctx, self.qstart,
                                 self.Hkv, self.scale)


def check_prefill_brute_force():
    """Causal prefill == exactly-summed textbook attention of each new token
    over the positions up to and including its own (cached prefix + new
    tokens), for shuffled blocks, with and without a prefix."""
    for dtype in ("f32", "bf16"):
        p = PrefillProblem(dtype, 4, 2, 8, ctx=[5, 19, 27, 1], nq=[5, 3, 20, 1], num_blocks=12, seed=13)
        out = p.out()
        G = p.Hq // p.Hkv
        for b in range(len(p.ctx)):
            p0 = int(p.ctx[b] - p.nq[b])
            K, V = widen(p.kv[b][0], dtype), widen(p.kv[b][1], dtype)
            for t in range(int(p.nq[b])):
                r = int(p.qstart[b]) + t
                for h in range(p.Hq):
                    n = p0 + t + 1
                    ref = brute_attention(list(widen(p.q[r, h], dtype)), K[:n, h // G].tolist(),
                                          V[:n, h // G].tolist(), p.scale)
                    err = np.abs(out[r, h] - np.asarray(ref)).max()
                    assert err <= 1e-13, (dtype, b, t, h, err)


def check_prefill_library_sdpa():
    """Causal prefill == torch's scaled_dot_product_attention in float64 with
    an explicit mask (query t of the new tokens sees keys 0 .. prefix + t)
    and grouped-query heads."""
    p = PrefillProblem("bf16", 8, 2, 64, ctx=[70, 33], nq=[30, 33], num_blocks=16, seed=17)
    out = p.out()
    for b in range(2):
        n, nq = int(p.ctx[b]), int(p.nq[b])
        rows = slice(int(p.qstart[b]), int(p.qstart[b + 1]))
        q = torch.from_numpy(widen(p.q[rows], "bf16")).permute(1, 0, 2)[None]             # [1,Hq,nq,D]
        k = torch.from_numpy(widen(p.kv[b][0], "bf16")).permute(1, 0, 2)[None].contiguous()  # [1,Hkv,n,D]
        v = torch.from_numpy(widen(p.kv[b][1], "bf16")).permute(1, 0, 2)[None].contiguous()
        mask = torch.arange(n)[None, :] <= (n - nq + torch.arange(nq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q.contiguous(), k, v, attn_mask=mask,
                                                               scale=p.scale, enable_gqa=True)
        err = np.abs(out[rows] - ref[0].permute(1, 0, 2).numpy()).max()
        assert err <= 1e-12, (b, err)


def check_prefill_int8():
    """Prefill over an int8 cache == textbook attention over the values
    decoded from the bytes."""
    p = PrefillProblem("int8", 4, 2, 16, ctx=[40, 9], nq=[12, 9], num_blocks=8, seed=19)
    out = p.out()
    G = p.Hq // p.Hkv
    for b in range(2):
        p0 = int(p.ctx[b] - p.nq[b])
        for g in range(p.Hkv):
            K, V = [], []
            for j in range(int(p.ctx[b])):
                blk, t = int(p.tables[b][j // 16]), j % 16
                kc, ks = int8_read(p.kpool, p.Hkv, p.D, blk, g, t, False)
                vc, vs = int8_read(p.vpool, p.Hkv, p.D, blk, g, t, True)
                K.append((kc * float(ks)).tolist())
                V.append((vc * float(vs)).tolist())
            for t in range(int(p.nq[b])):
                r = int(p.qstart[b]) + t
                for h in range(g * G, (g + 1) * G):
                    ref = brute_attention(list(widen(p.q[r, h], "bf16")), K[:p0 + t + 1], V[:p0 + t + 1], p.scale)
                    assert np.abs(out[r, h] - np.asarray(ref)).max() <= 1e-13, (b, t, h)


def check_prefill_fp8():
    """Prefill over an FP8 cache == textbook attention over the values torch
    decodes from the bytes times the scales."""
    p = PrefillProblem("fp8", 4, 2, 16, ctx=[40, 9], nq=[12, 9], num_blocks=8, seed=29)
    out = p.out()
    G = p.Hq // p.Hkv
    for b in range(2):
        p0 = int(p.ctx[b] - p.nq[b])
        for g in range(p.Hkv):
            K, V = [], []
            for j in range(int(p.ctx[b])):
                blk, t = int(p.tables[b][j // 16]), j % 16
                kv_, ks, _ = fp8_read(p.kpool, p.Hkv, p.D, blk, g, t, False)
                vv_, vs, _ = fp8_read(p.vpool, p.Hkv, p.D, blk, g, t, True)
                K.append((kv_ * float(ks)).tolist())
                V.append((vv_ * float(vs)).tolist())
            for t in range(int(p.nq[b])):
                r = int(p.qstart[b]) + t
                for h in range(g * G, (g + 1) * G):
                    ref = brute_attention(list(widen(p.q[r, h], "bf16")), K[:p0 + t + 1], V[:p0 + t + 1], p.scale)
                    assert np.abs(out[r, h] - np.asarray(ref)).max() <= 1e-13, (b, t, h)


ALL_CHECKS = [check_brute_force, check_library_sdpa, check_paged_equals_contiguous,
              check_placement_invariance, check_special_cases, check_merge_identity,
              check_gqa_reduces_to_mha, check_append_roundtrip, check_layout_golden,
              check_rejects_per_page_softmax, check_int8_quant_golden, check_int8_layout_golden,
              check_int8_quant_error_bound, check_int8_brute_force, check_int8_copy_blocks,
              check_prefill_brute_force, check_prefill_library_sdpa, check_prefill_int8,
              check_fp8_quant_golden, check_fp8_decode_library, check_fp8_encode_library,
              check_fp8_quant_error_bound, check_fp8_brute_force, check_prefill_fp8]
