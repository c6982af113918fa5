"""Paged decode attention benchmark on one MI355X.

One step is one pass of the whole decode path for a batch: the host block
manager assigns every sequence its next token slot (taking a fresh block at a
16-token boundary), the slots, block tables and lengths go to HBM in one
pinned host-to-device copy, and then for every layer the new token's K/V are
stored (paged_kv_append) and attention runs over the whole paged context
(paged_attention_decode: partition kernel plus split-context merge).  Layers
have their own K/V pools and share the block tables; several layers are run
per step so that the bytes read per step exceed the 256 MB Infinity Cache.

Prints one JSON line: KV GB/s of the whole step (inputs resident in HBM), the
roofline of the attention call (partition kernel and split-context merge)
from HIP events recorded around it on the launch stream, the same rate as a
share of a streaming-read probe's, pool usage and internal fragmentation,
and the CPU oracle timed on the host on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "paged decode attention KV GB/s (% of HBM peak) + decode tokens/s, 1 GPU"
MODEL_LAYERS = {"llama3_8b_b64": 32, "llama3_70b_b256": 80, "llama3_70b_b256_int8": 80, "shared_prefix_b128": 32, "best_of_8": 32,
                "mha_long": 32, "tiny_fp32": 1}
PARTITION_KERNELS = ("decode_mfma_kernel", "decode_valu_kernel")


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h: timing only, no system-scope fences


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded, so the
    library can record them between its own launches.  They only time: the
    system-scope release/acquire fences of a default event (a write-back of
    the L2s at every record) are turned off."""

    def __init__(self, flags=HIP_EVENT_DISABLE_SYSTEM_FENCE):
        self.flags = flags
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.flags) == 0
            out.append(e)
        return out

    def record(self, e, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert self.hip.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def kernel_source_hash() -> str:
    """Hash of the decode kernels' sources with comments and blank lines
    removed: a stored traffic measurement applies while the code is
    unchanged, whatever its comments say."""
    h = hashlib.sha256()
    for f in ("decode_mfma.hip", "decode_valu.hip", "decode_merge.hip", "pkv_device.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_381_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", "", src)  # line comments (no string literal in these files holds //)
        code = "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())
        h.update(code.encode("utf-8"))
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per partition-kernel launch from the committed PMC summary,
    or None when there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inst, min_seconds: float):
    """The oracle (fp64 C, OpenMP) on the host: the decode step's append and
    attention over the whole batch, repeated for at least min_seconds."""
    import numpy as np
    from oracle import attn as orc
    from oracle.book import build_workload

    wl = inst.wl
    book, ids, pre_slots, step_slots, _ = build_workload(inst)
    kpool, vpool = orc.new_pool(inst.num_blocks, wl.num_kv_heads, wl.head_dim, wl.cache_dtype)
    orc.append(wl.cache_dtype, wl.num_kv_heads, wl.head_dim, kpool, vpool, inst.prefill_tokens("k"),
               inst.prefill_tokens("v"), np.asarray(pre_slots, np.int64))
    tables, ctx = orc.tables_of(book, ids)
    kstep, vstep, q = inst.step_tokens("k"), inst.step_tokens("v"), inst.q()
    slots = np.asarray(step_slots, np.int64)
    scale = 1.0 / math.sqrt(wl.head_dim)
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.append(wl.cache_dtype, wl.num_kv_heads, wl.head_dim, kpool, vpool, kstep, vstep, slots)
        orc.paged_attention(wl.cache_dtype, q, kpool, vpool, tables, ctx, wl.num_kv_heads, scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    per_step = dt / reps
    return {"value": round(inst.kv_bytes_logical() / per_step / 1e9, 4), "unit": "GB/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"full {wl.name} decode step (append + fp64 attention over all {wl.batch} sequences, "
                      f"{int(inst.ctx.sum())} tokens), {reps} repetition(s) in {dt:.1f} s, "
                      f"{per_step * 1e3:.1f} ms per step; OMP threads = {orc.num_threads()}, "
                      f"host cores = {os.cpu_count()}"}


def _pmc_rows(run_dir: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _pmc_mean_kib(rows, name_part: str, counter: str) -> float:
    vals = [float(r["Counter_Value"]) for r in rows if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel named like {name_part!r}")
    return sum(vals) / len(vals)


def traffic_summary(args):
    """Write profiles/decode_<workload>_traffic.txt from four rocprofv3 --pmc
    runs: FETCH_SIZE and WRITE_SIZE of the bench, and of the plain copy probe
    (1 GiB read + 1 GiB written per copy), which calibrates each counter.
    The traffic of one attention call is its partition kernel's plus its
    merge kernel's."""
    fetch_dir, write_dir, fetch_copy_dir, write_copy_dir, bench_log = args.traffic_summary
    kern = next((k for k in PARTITION_KERNELS if any(k in r["Kernel_Name"] for r in _pmc_rows(fetch_dir))), None)
    if kern is None:
        raise SystemExit("no partition kernel in the FETCH_SIZE run")
    fetch = _pmc_mean_kib(_pmc_rows(fetch_dir), kern, "FETCH_SIZE")
    write = _pmc_mean_kib(_pmc_rows(write_dir), kern, "WRITE_SIZE")
    mfetch = _pmc_mean_kib(_pmc_rows(fetch_dir), "merge_kernel", "FETCH_SIZE")
    mwrite = _pmc_mean_kib(_pmc_rows(write_dir), "merge_kernel", "WRITE_SIZE")
    copy_bytes = 1 << 30
    cfetch = _pmc_mean_kib(_pmc_rows(fetch_copy_dir), "copyBuffer", "FETCH_SIZE")
    cwrite = _pmc_mean_kib(_pmc_rows(write_copy_dir), "copyBuffer", "WRITE_SIZE")
    fscale, wscale = copy_bytes / (cfetch * 1024), copy_bytes / (cwrite * 1024)
    part = fetch * 1024 * fscale + write * 1024 * wscale
    merge = mfetch * 1024 * fscale + mwrite * 1024 * wscale
    hbm = part + merge
    algo = None
    with open(bench_log, encoding="utf-8") as f:
        for line in f:
            if line.startswith("{"):
                algo = json.loads(line)["roofline"]["bytes_per_launch"]
    lines = [
        f"# HBM traffic per attention call (partition kernel {kern} + merge_kernel), workload {args.workload}",
        "# from rocprofv3 --pmc runs, one counter per run, each scaled by what it reads for a plain",
        "# 1 GiB device copy (bench.py --copy-probe):",
        f"#   cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o b -- python3 <repo>/bench.py "
        f"--workload {args.workload} --steps 5 --warmup 2 --no-cpu-baseline --no-stream-probe",
        "#   (the same with --pmc WRITE_SIZE, and both counters over python3 <repo>/bench.py --copy-probe), then",
        f"#   python3 <repo>/bench.py --workload {args.workload} --traffic-summary <fetch dir> <write dir> "
        "<copy fetch dir> <copy write dir> <bench log of the FETCH_SIZE run>",
        f"kernel_source_hash = {kernel_source_hash()}",
        f"fetch_kib_per_dispatch = {fetch:.1f}",
        f"write_kib_per_dispatch = {write:.1f}",
        f"merge_fetch_kib_per_dispatch = {mfetch:.1f}",
        f"merge_write_kib_per_dispatch = {mwrite:.1f}",
        f"copy_fetch_kib_per_gib = {cfetch:.1f}",
        f"copy_write_kib_per_gib = {cwrite:.1f}",
        f"fetch_scale = {fscale:.4f}",
        f"write_scale = {wscale:.4f}",
        f"partition_hbm_bytes_per_launch = {part:.0f}",
        f"merge_hbm_bytes_per_launch = {merge:.0f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
        f"algorithmic_bytes_per_launch = {algo}",
        f"traffic_over_algorithmic = {hbm / algo:.4f}" if algo else "traffic_over_algorithmic = unknown",
    ]
    path = os.path.join(ROOT, "profiles", f"decode_{args.workload}_traffic.txt")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_summary(args):
    """Write profiles/<name>_counters.txt from rocprofv3 --pmc runs of this
    bench (CSV output): per kernel, the mean of each counter over its
    dispatches and the derived busy fractions (per-XCD active cycles =
    GRBM_GUI_ACTIVE / 8; 256 CUs, 1024 SIMDs)."""
    import collections
    name, cmd, *dirs = args.pmc_summary
    vals = collections.defaultdict(list)
    for d in dirs:
        for r in _pmc_rows(d):
            k = r["Kernel_Name"].replace("void (anonymous namespace)::", "").split("(")[0]
            vals[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
    kernels = sorted({k for k, _ in vals if any(t in k for t in ("decode_", "prefill_", "merge_kernel"))})
    lines = [f"# rocprofv3 --pmc counters (MI355X, one GPU): {name}",
             "# command, one run per counter set: cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc <counters> "
             f"--output-format csv -d <dir> -o b -- python3 <repo>/bench.py {cmd}",
             f"# then: python3 <repo>/bench.py --pmc-summary {name} '{cmd}' <dir> ...",
             "# counter sets: " + "; ".join(sorted({' '.join(sorted({c for (k2, c) in vals if k2 == k}))
                                                  for k in kernels})),
             "# mean per dispatch; busy fractions against GRBM_GUI_ACTIVE / 8 (per-XCD active cycles)"]
    for k in kernels:
        cs = {c: sum(v) / len(v) for (k2, c), v in vals.items() if k2 == k}
        n = max(len(v) for (k2, c), v in vals.items() if k2 == k)
        lines.append(f"{k}  ({n} dispatches)")
        for c in sorted(cs):
            lines.append(f"    {c:28s} {cs[c]:16.6g}")
        act = cs.get("GRBM_GUI_ACTIVE", 0) / 8
        if act:
            def frac(c, units, scale=1.0):
                if c in cs:
                    lines.append(f"    {c + ' busy':28s} {100 * cs[c] * scale / (act * units):15.1f} %")
            frac("SQ_VALU_MFMA_BUSY_CYCLES", 1024)
            frac("SQ_ACTIVE_INST_VALU", 1024, 4.0)
            for c in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY"):  # shares of the waves' cycles
                if c in cs and cs.get("SQ_WAVE_CYCLES"):
                    lines.append(f"    {c + ' of wave cycles':28s} {100 * cs[c] / cs['SQ_WAVE_CYCLES']:15.1f} %")
            if "SQ_WAVE_CYCLES" in cs:  # waves resident per SIMD, on average
                lines.append(f"    {'SQ_WAVE_CYCLES waves/SIMD':28s} {cs['SQ_WAVE_CYCLES'] * 4.0 / (act * 1024):15.2f}")
            frac("TA_TA_BUSY", 256)
            frac("TD_TD_BUSY", 256)
    path = os.path.join(ROOT, "profiles", f"{name}_counters.txt")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(args):
    """Write profiles/[decode_]<workload>_kernel_trace.txt from a
    rocprofv3 --kernel-trace --stats run of this bench (CSV output) and the
    bench log of the same run."""
    import csv
    import glob
    out_dir, bench_log, cmd = args.trace_summary
    files = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {out_dir}")
    with open(files[0], newline="") as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    bench_lines = []
    with open(bench_log, encoding="utf-8") as f:
        for line in f:
            if line.startswith("[bench]") and ("attention call" in line or "prefill kernel" in line
                                               or "building" in line):
                bench_lines.append("#   " + line.strip())
    kind = "" if args.workload.startswith("prefill") else "decode_"
    tag = args.workload + ("_identity_tables" if args.tables == "identity" else "") + \
        (f"_batch{args.batch}" if args.batch else "") + (f"_kernel{args.kernel}" if args.kernel else "")
    lines = ["# rocprofv3 --kernel-trace --stats summary (MI355X, one GPU)",
             f"# command: cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d <out> -o kt -- python3 <repo>/bench.py {cmd}",
             f"# then: python3 <repo>/bench.py --workload {args.workload} --trace-summary <out> <bench log> '{cmd}'",
             "# the bench's own lines in that run (HIP events on the launch stream, timed steps only):",
             *bench_lines,
             "# averages below include the warm-up steps and the build of the workload",
             f"{'kernel':<78}{'calls':>6}{'avg_us':>10}{'min_us':>10}{'max_us':>10}"]
    for r in rows:
        name = (r.get("Name") or r.get("KernelName") or "?").replace("void (anonymous namespace)::", "")
        name = name.replace("(SplitParams)", "").replace("(PrefillParams)", "")[:76]
        lines.append(f"{name:<78}{int(r['Calls']):>6}{float(r['AverageNs']) / 1e3:>10.1f}"
                     f"{float(r['MinNs']) / 1e3:>10.1f}{float(r['MaxNs']) / 1e3:>10.1f}")
    path = os.path.join(ROOT, "profiles", f"{kind}{tag}_kernel_trace.txt")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:12]))


N_SPAN_CALLS = 5  # untimed traced steps after the timed ones (wave span of the partition kernel)
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
PREFILL_METRIC = "paged prefill attention TFLOP/s (% of bf16 MFMA peak), 1 GPU"


def cpu_baseline_prefill(inst, min_seconds: float):
    """The fp64 oracle's causal prefill on the host, on a bounded sample: the
    last new tokens of sequence 0 (the rows that see the most keys), doubled
    until the run lasts min_seconds; reported in GFLOP/s of the same count."""
    import numpy as np
    from oracle import attn as orc
    wl = inst.wl
    built = orc.build_prefill(inst)
    q = inst.q()
    qs = inst.qstart
    rows, reps = 1, 0
    while True:
        last = min(rows, int(inst.nq[0]))
        sub = q[int(qs[1]) - last:int(qs[1])]
        t0 = time.perf_counter()
        orc.paged_prefill(wl.cache_dtype, sub, built["kpool"], built["vpool"], built["tables"][:1], built["ctx"][:1],
                          np.array([0, last], np.int32), wl.num_kv_heads, 1.0 / math.sqrt(wl.head_dim))
        dt = time.perf_counter() - t0
        reps += 1
        if dt >= min_seconds or last == int(inst.nq[0]):
            break
        rows *= 2
    n0 = int(inst.ctx[0]) - int(inst.nq[0])
    keys = sum(n0 + t + 1 for t in range(int(inst.nq[0]) - last, int(inst.nq[0])))
    flops = 4 * wl.head_dim * wl.num_q_heads * keys
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"the last {last} new tokens of sequence 0 of {wl.name} ({keys} query-key pairs per head, "
                      f"{flops / 1e9:.2f} GFLOP) in {dt:.1f} s; OMP threads = {orc.num_threads()}, "
                      f"host cores = {os.cpu_count()}"}


def bench_prefill(args):
    """A prefill step per layer: store the new tokens' K/V into their slots
    (paged_kv_append), then the causal attention of every new token over its
    paged context (paged_attention_prefill).  Reports whole-step TFLOP/s and
    the prefill kernel against the bf16 matrix-core peak."""
    import torch
    from workloads import prefill as PW
    from paged_kv_cache_381_amd.engine import GpuPrefill

    inst = PW.get(args.workload)
    wl = inst.wl
    K, W = args.steps, args.warmup
    layers = args.layers or 2
    print(f"[bench] building {wl.name}: B={wl.batch} Hq={wl.num_q_heads} H={wl.num_kv_heads} D={wl.head_dim} "
          f"{wl.cache_dtype} cache, layers/step={layers}, new tokens {int(inst.nq.sum())}", flush=True)
    gp = GpuPrefill(inst, num_layers=layers)
    flops = inst.flops()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]

    def step(timed):
        for layer in range(layers):
            gp.cache.write(layer, gp.new_slots_dev, gp.k_new, gp.v_new)
            if timed is not None and layer == timed % layers:
                ev[timed][0].record()
                gp.run(layer)
                ev[timed][1].record()
            else:
                gp.run(layer)

    import gc
    gc.collect()
    gc.disable()
    for _ in range(W):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    assert torch.isfinite(gp.out).all().item(), "non-finite prefill output"
    avg_ms = sum(a.elapsed_time(b) for a, b in ev) / K
    tflops = flops * layers * K / elapsed / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    print(f"[bench] {K} steps in {elapsed:.3f} s; prefill kernel avg {avg_ms * 1e3:.1f} us "
          f"({achieved:.1f} TFLOP/s)", flush=True)
    res = {
        "metric": PREFILL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.description, "name": wl.name, "batch": wl.batch, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": 16,
                   "kv_cache": wl.cache_dtype, "layers_per_step": layers, "new_tokens": int(inst.nq.sum()),
                   "cached_prefix": wl.shared_prefix, "parallelism": "none"},
        "prefill_tokens_per_s_per_layer": round(int(inst.nq.sum()) * K * layers / elapsed, 1),
        "roofline": {"kernel": "paged_attention_prefill", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(avg_ms * 1e3, 2),
                     "flops_per_launch": flops, "kv_bytes_distinct": inst.kv_bytes(), "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(inst, args.cpu_seconds)
    print(json.dumps(res), flush=True)


PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction
SWAP_METRIC = "block swap GB/s between HBM and pinned host memory (% of PCIe 5.0 x16), 1 GPU"


def bench_swap(args):
    """Swap of a decode workload's blocks: every block of the second half of
    the batch moves to pinned host memory (Clock victims, the first half
    protected) and back, K and V, one layer.  Times the two copy kernels with
    events on the launch stream; the host bookkeeping is reported apart."""
    import numpy as np
    import torch
    import workloads
    from paged_kv_cache_381_amd import _lib as L
    from paged_kv_cache_381_amd.engine import GpuWorkload

    name = args.workload.split(":", 1)[1]
    inst = workloads.get(name)
    wl = inst.wl
    gw = GpuWorkload(inst)
    c = gw.cache
    B = wl.batch
    keep, move = gw.ids[:B // 2], gw.ids[B // 2:]
    need = int(sum(-(-int(n) // 16) for n in inst.ctx[B // 2:]))
    c.enable_swap(need + 16)
    tile = c.layout.pool_elems // c.layout.num_blocks * (c.k_pools[0].element_size())
    K, W = args.steps, args.warmup
    out_ms, in_ms, book_s, moved = [], [], 0.0, 0
    for k in range(W + K):
        c.tables(keep, gw.max_blocks)  # the running half: its blocks are protected and referenced
        t0 = time.perf_counter()
        pairs = L.pkv_swap_out(c.pool, 10 ** 6, keep)
        book_s += time.perf_counter() - t0 if k >= W else 0.0
        d = torch.from_numpy(np.ascontiguousarray(pairs)).cuda()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        L.pkv_swap_copy(c.layout, c.host_k[0], c.host_v[0], c.num_host_blocks, c.k_pools[0], c.v_pools[0],
                        c.layout.num_blocks, d)
        e[1].record()
        back = []
        t0 = time.perf_counter()
        for sid in move:
            back.append(L.pkv_seq_swap_in(c.pool, sid))
        book_s += time.perf_counter() - t0 if k >= W else 0.0
        d2 = torch.from_numpy(np.ascontiguousarray(np.concatenate(back))).cuda()
        e[2].record()
        L.pkv_swap_copy(c.layout, c.k_pools[0], c.v_pools[0], c.layout.num_blocks, c.host_k[0], c.host_v[0],
                        c.num_host_blocks, d2)
        e[3].record()
        torch.cuda.synchronize()
        assert len(pairs) == need and len(d2) == need
        if k >= W:
            out_ms.append(e[0].elapsed_time(e[1]))
            in_ms.append(e[2].elapsed_time(e[3]))
            moved += len(pairs)
    nbytes = need * 2 * tile  # K and V of every block, per direction
    o_ms, i_ms = sum(out_ms) / K, sum(in_ms) / K
    out_gbps, in_gbps = nbytes / (o_ms * 1e-3) / 1e9, nbytes / (i_ms * 1e-3) / 1e9
    gbps = 2 * nbytes / ((o_ms + i_ms) * 1e-3) / 1e9
    print(f"[bench] swap {need} blocks ({nbytes / 1e6:.1f} MB) out {o_ms * 1e3:.0f} us ({out_gbps:.1f} GB/s), "
          f"in {i_ms * 1e3:.0f} us ({in_gbps:.1f} GB/s); bookkeeping {book_s / K * 1e3:.2f} ms per round trip",
          flush=True)
    res = {"metric": SWAP_METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": round(o_ms + i_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": wl.cache_dtype, "data": "synthetic",
           "config": {"workload": f"swap out and back in the blocks of half of: {wl.description}", "name": wl.name,
                      "blocks_per_direction": need, "bytes_per_direction": nbytes, "parallelism": "none"},
           "swap_out_gbps": round(out_gbps, 2), "swap_in_gbps": round(in_gbps, 2),
           "bookkeeping_ms_per_round_trip": round(book_s / K * 1e3, 3),
           "roofline": {"kernel": "pkv_swap_copy (swap_blocks_kernel)", "bound": "pcie", "achieved": round(gbps, 2),
                        "peak": PCIE_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / PCIE_PEAK_GBPS, 4),
                        "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)


def copy_probe(gib: float, reps: int):
    """Plain device-to-device copies of a known size (PMC calibration)."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "reps": reps}))


PROBE_TILES = 1 << 18  # 1 GiB of 4 KiB tiles: four times the Infinity Cache


def stream_probe(reps: int = 5):
    """Achievable read rate for the decode kernels' access pattern: the
    streaming-read probe (libpkvprobe.so) reads 1 GiB of 4 KiB tiles in a
    seeded random order and in address order, with cached and with
    non-temporal loads, one wave per SIMD; returns GB/s per variant (HIP
    events, mean over reps after a warm-up)."""
    import numpy as np
    import torch
    from paged_kv_cache_381_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise SystemExit(f"{B.PROBE_LIB} is not built (run __graft_entry__.build())")
    plib = ctypes.CDLL(B.PROBE_LIB)
    plib.pkv_probe_stream_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    n = PROBE_TILES
    buf = torch.empty(n * 1024, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    orders = {"random": np.random.default_rng(4096).permutation(n).astype(np.int32),
              "sequential": np.arange(n, dtype=np.int32)}
    sink = torch.empty(4 * 2 * plib.pkv_probe_compute_units(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for oname, order in orders.items():
        d_order = torch.from_numpy(order).cuda()
        for loads, nt in (("cached", 0), ("streaming", 1)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
            for r in range(reps + 1):
                if r:
                    ev[2 * r - 2].record()
                rc = plib.pkv_probe_stream_tiles(buf.data_ptr(), n, d_order.data_ptr(), 1, nt, sink.data_ptr(),
                                                 stream)
                assert rc == 0, f"probe launch failed ({rc})"
                if r:
                    ev[2 * r - 1].record()
            torch.cuda.synchronize()
            ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) / reps
            res[f"{oname}_{loads}"] = round(n * 4096 / (ms * 1e-3) / 1e9, 1)
    del buf
    return res


def launch_cost(reps: int = 30):
    """Fixed cost of one launch on the decode kernels' grid: an empty kernel
    (libpkvprobe.so) whose waves record their first and last clock, timed by
    the same events as the attention call.  Returns the median event time, the
    span of the waves (first start to last end) and their difference, in us."""
    import numpy as np
    import torch
    from paged_kv_cache_381_amd import build as B
    plib = ctypes.CDLL(B.PROBE_LIB)
    plib.pkv_probe_launch_cost.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    clock = torch.zeros(8 * plib.pkv_probe_compute_units(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()
    ev = hip.create(2)
    times, spans = [], []
    for r in range(reps + 1):
        hip.record(ev[0], stream)
        assert plib.pkv_probe_launch_cost(clock.data_ptr(), stream) == 0
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        if r:
            times.append(hip.elapsed_ms(ev[0], ev[1]) * 1e3)
            c = clock.cpu().numpy().astype(np.int64).reshape(-1, 2) & 0xFFFFFFFF
            spans.append((c[:, 1].max() - c[:, 0].min()) / 100.0)
    hip.destroy(ev)
    t, sp = float(np.median(times)), float(np.median(spans))
    return {"event_us": round(t, 2), "wave_span_us": round(sp, 2), "outside_waves_us": round(t - sp, 2)}


def pattern_probe(reps: int = 5):
    """Load-pattern probe (libpkvprobe.so): the decode kernels' per-lane loads
    of a chunk with no arithmetic, over random (block, kv head) tiles of about
    0.5 GiB per pool, bf16 (4 KiB tiles) and one-byte (2112-byte tiles), each
    variant (K loads on half or whole 128-byte lines, query slices reloaded
    with every chunk or not) with cached and streaming loads.  Returns GB/s
    of tile bytes per variant (HIP events, mean of reps after a warm-up)."""
    import numpy as np
    import torch
    from paged_kv_cache_381_amd import build as B
    plib = ctypes.CDLL(B.PROBE_LIB)
    plib.pkv_probe_load_pattern.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.empty(4 * plib.pkv_probe_compute_units(), dtype=torch.int32, device="cuda")
    q = torch.full((256 * 1024,), 3, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()
    ev = hip.create(2)
    names = {0: "half-line K, query every chunk", 1: "whole-line K, query every chunk",
             2: "half-line K, no query loads", 3: "whole-line K, no query loads"}
    res = {}
    for one_byte, tb, n_chunks in ((0, 4096, 64 * 1024), (1, 2112, 128 * 1024)):
        n_tiles = 2 * n_chunks
        k = torch.full((n_tiles * tb,), 1, dtype=torch.uint8, device="cuda")
        v = torch.full((n_tiles * tb,), 2, dtype=torch.uint8, device="cuda")
        order = torch.from_numpy(np.random.default_rng(4096).permutation(n_tiles).astype(np.int32)).cuda()
        for variant in range(4):
            for loads, nt in (("cached", 0), ("streaming", 1)):
                ms = 0.0
                for r in range(reps + 1):
                    hip.record(ev[0], stream)
                    rc = plib.pkv_probe_load_pattern(one_byte, variant, nt, k.data_ptr(), v.data_ptr(), q.data_ptr(),
                                                     n_chunks, order.data_ptr(), sink.data_ptr(), stream)
                    assert rc == 0, f"probe launch failed ({rc})"
                    hip.record(ev[1], stream)
                    torch.cuda.synchronize()
                    if r:
                        ms += hip.elapsed_ms(ev[0], ev[1])
                res[f"{'one-byte' if one_byte else 'bf16'}, {names[variant]}, {loads}"] = \
                    round(n_tiles * 2 * tb / (ms / reps * 1e-3) / 1e9, 1)
        del k, v
    hip.destroy(ev)
    return res


def mfma_probe(iters: int = 20000):
    """Matrix-core issue probe (libpkvprobe.so): per iteration 24 independent
    v_mfma_f32_16x16x32_bf16 and/or the vector work that weighs 24 scores, or
    12 v_mfma_f32_32x32x16_bf16, with one and two waves per SIMD.  Returns us per launch and cycles per
    iteration of one wave (at 2.4 GHz), and the products' TFLOP/s."""
    import torch
    from paged_kv_cache_381_amd import build as B
    plib = ctypes.CDLL(B.PROBE_LIB)
    plib.pkv_probe_mfma_issue.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    cus = plib.pkv_probe_compute_units()
    d_in = torch.zeros(96, dtype=torch.float32, device="cuda")
    d_out = torch.empty(2 * 256 * cus, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()
    ev = hip.create(2)
    names = {0: "products", 1: "vector work", 2: "both, in program order", 3: "both, interleaved",
             4: "32x32x16 products"}
    res = {}
    for wps in (1, 2):
        for mode in range(5):
            assert plib.pkv_probe_mfma_issue(mode, wps, iters, d_in.data_ptr(), d_out.data_ptr(), stream) == 0
            hip.record(ev[0], stream)
            assert plib.pkv_probe_mfma_issue(mode, wps, iters, d_in.data_ptr(), d_out.data_ptr(), stream) == 0
            hip.record(ev[1], stream)
            torch.cuda.synchronize()
            us = hip.elapsed_ms(ev[0], ev[1]) * 1e3
            r = {"us": round(us, 1), "cycles_per_iter_per_wave_at_2.4GHz": round(us * 2400 / iters / wps, 1)}
            if mode in (0, 4):  # 24 x 16384 = 12 x 32768 flops per iteration
                r["tflops"] = round(24 * 16384 * iters * 4 * cus * wps / (us * 1e-6) / 1e12, 1)
            res[f"{names[mode]}, {wps} wave(s)/SIMD"] = r
    hip.destroy(ev)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_b64")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per step (0: enough that a step stores >= 1 GiB of distinct K/V, at most 64)")
    ap.add_argument("--partition", type=int, default=0,
                    help="fewest context tokens per wave of the balanced split (0: library default, 128)")
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 wavefront-reduction, 2 matrix-core")
    ap.add_argument("--waves-per-simd", type=int, default=0,
                    help="matrix-core kernel: 1 or 2 resident waves per SIMD (0: chosen from the pool's sharing)")
    ap.add_argument("--xcd-weights", default="none",
                    help="per-XCD work weights of the balanced split: 'none' (equal shares, the default), "
                         "'auto' (from traced untimed steps after the warm-up) or 8 comma-separated integers")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help="run only plain 1 GiB copies (PMC calibration)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run only the matrix-core issue probe (products and vector work, one and two waves per SIMD)")
    ap.add_argument("--pattern-probe", action="store_true",
                    help="run only the load-pattern probe (the decode kernels' loads of bf16 and one-byte tiles)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="run only the streaming-read probe (1 GiB of 4 KiB tiles, random and address order)")
    ap.add_argument("--no-stream-probe", action="store_true", help="skip the probe in a decode run")
    ap.add_argument("--batch", type=int, default=0,
                    help="decode workloads: run the named workload's shapes and draws at this batch size "
                         "(counter checks on a small launch; 0: the workload's own)")
    ap.add_argument("--load-policy", type=int, default=0,
                    help="K/V tile loads: 0 auto, 1 streaming (non-temporal), 2 cached")
    ap.add_argument("--plan", choices=("step", "none"), default="step",
                    help="step: each step's first decode call records the split in a plan and the other layers' "
                         "calls run from it; none: every call schedules itself")
    ap.add_argument("--tables", choices=("shuffled", "identity"), default="shuffled",
                    help="physical block placement: the workload's shuffled pool, or blocks handed out in "
                         "address order (each sequence's blocks consecutive)")
    ap.add_argument("--traffic-summary", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR", "BENCH_LOG"),
                    help="write profiles/decode_<workload>_traffic.txt from rocprofv3 --pmc output (no GPU)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("OUT_DIR", "BENCH_LOG", "BENCH_ARGS"),
                    help="write profiles/<kind>_<workload>_kernel_trace.txt from a rocprofv3 --kernel-trace "
                         "--stats run of this bench (no GPU)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="NAME CMD DIR",
                    help="write profiles/<NAME>_counters.txt from rocprofv3 --pmc runs (CSV dirs) of the bench "
                         "command CMD (no GPU)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "sequences or kv heads would shard across GPUs with no exchange.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(1.0, 10)
        return
    if args.mfma_probe:
        print(json.dumps({"mfma_issue_probe": mfma_probe()}), flush=True)
        return
    if args.pattern_probe:
        print(json.dumps({"load_pattern_probe_gbps": pattern_probe()}), flush=True)
        return
    if args.stream_probe:
        r = stream_probe(10)
        print(json.dumps({"stream_probe_gbps": r, "tiles": PROBE_TILES, "tile_bytes": 4096}), flush=True)
        return

    import workloads
    from workloads import prefill as PW
    from paged_kv_cache_381_amd import _lib as L
    from paged_kv_cache_381_amd.engine import GpuWorkload

    if args.workload in PW.PREFILL_WORKLOADS:
        bench_prefill(args)
        return
    if args.workload.startswith("swap:"):
        bench_swap(args)
        return
    inst = workloads.configs.scaled(args.workload, batch=args.batch).instantiate() if args.batch else \
        workloads.get(args.workload)
    if args.tables == "identity":
        inst.free_order = np.arange(inst.num_blocks, dtype=np.int32)
    wl = inst.wl
    B, H, Hq, D = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim
    K, W = args.steps, args.warmup
    tok_bytes = 2 * H * wl.row_bytes  # K and V of one token, one layer (int8: scales included)
    # Enough layers (own pools) that one step stores more than 1 GiB of
    # distinct K/V, so the 256 MB Infinity Cache cannot hold a step's reads.
    layers = args.layers or min(64, max(1, math.ceil((1 << 30) / inst.kv_bytes_unique())))
    total_steps = K + W + 3 + N_SPAN_CALLS  # warm-up, XCD-weight calibration, timed and traced steps
    extra = B * (total_steps // 16 + 2)
    print(f"[bench] building {wl.name}: B={B} Hq={Hq} H={H} D={D} {wl.cache_dtype} cache, layers/step={layers}",
          flush=True)
    gw = GpuWorkload(inst, num_layers=layers, extra_blocks=extra)
    inst.drop_cache()
    cache, ids = gw.cache, np.asarray(gw.ids, np.int64)
    MB = -(-(int(inst.ctx.max()) + total_steps + 1) // 16)
    ws = cache.workspace(B, Hq, MB * 16, args.partition, args.kernel)
    dev = torch.device("cuda")
    # Slots (int64), lengths and block tables of a step travel in one pinned
    # host-to-device copy; R pinned sets rotate so the host never overwrites
    # one still being copied.
    R = 4
    n32 = 2 * B + B + B * MB
    pin = [torch.empty(n32, dtype=torch.int32, pin_memory=True) for _ in range(R)]
    ring_ev = [torch.cuda.Event() for _ in range(R)]
    dbuf = torch.empty(n32, dtype=torch.int32, device=dev)
    d_slots, d_ctx, d_tables = dbuf[:2 * B].view(torch.int64), dbuf[2 * B:3 * B], dbuf[3 * B:].view(B, MB)
    k_new, v_new = gw.k_step, gw.v_step
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    wps = args.waves_per_simd or cache.waves_per_simd()
    hip = HipEvents()
    # One layer per timed step (rotating) carries the HIP events around its
    # partition kernel: every event record idles the GPU for a few
    # microseconds, which would otherwise be charged to the whole step.
    evs = hip.create(2 * K)
    torch.cuda.synchronize()

    # The step calls the C ABI directly with argument tuples built once: the
    # binding's per-call checks cost the host more than the GPU work of a
    # small layer, and a slow host would otherwise set the step's pace.
    lib = L.lib()
    V = ctypes.c_void_p
    stream = L._stream(None)
    ids_c = np.ascontiguousarray(ids, dtype=np.int64)
    cow = np.empty((B, 2), dtype=np.int32)
    ncow = ctypes.c_int32(0)
    lay = ctypes.byref(cache.layout)
    # One plan per step: the step's first call records the split of its
    # tables and lengths, the other layers' calls run from it.
    use_plan = args.plan == "step"
    step_plan = L.new_decode_plan(cache.layout, B, Hq, MB * 16, args.partition) if use_plan else None
    wps_opts = L.decode_opts(args.partition, args.kernel, None, wps, load_policy=args.load_policy, plan=step_plan)
    def timed_opts(xw=None):
        # Even timed steps bracket the whole attention call (partition kernel
        # and split-context merge), odd ones the partition kernel alone; one
        # event pair per step, since a record in between would idle the GPU.
        return [L.decode_opts(args.partition, args.kernel,
                              (evs[2 * i], None, evs[2 * i + 1]) if i % 2 == 0 else (evs[2 * i], evs[2 * i + 1], None),
                              wps, xw, load_policy=args.load_policy, plan=step_plan) for i in range(K)]

    ev_opts = timed_opts()
    ws_bytes = ws.numel() * ws.element_size()
    append_args = [(lay, V(cache.k_pools[i].data_ptr()), V(cache.v_pools[i].data_ptr()), V(k_new.data_ptr()),
                    V(v_new.data_ptr()), V(d_slots.data_ptr()), B, stream) for i in range(layers)]
    head = [(lay, V(out.data_ptr()), V(gw.q.data_ptr()), V(cache.k_pools[i].data_ptr()),
             V(cache.v_pools[i].data_ptr()), V(d_tables.data_ptr()), V(d_ctx.data_ptr()), B, Hq, MB)
            for i in range(layers)]
    tail = (ctypes.c_float(gw.scale), V(ws.data_ptr()), ws_bytes)
    pin_ptr = [(V(p.data_ptr()), V(p.data_ptr() + 12 * B), V(p.data_ptr() + 8 * B)) for p in pin]

    def step(k: int, timed_idx: int, traced=None):
        r = k % R
        ring_ev[r].synchronize()  # the copy that last read this pinned set is done
        slots_p, tables_p, ctx_p = pin_ptr[r]
        L._check(lib.pkv_batch_append_slots(cache.pool, ids_c.ctypes.data_as(V), B, 1, slots_p,
                                            cow.ctypes.data_as(V), B, ctypes.byref(ncow)))
        assert ncow.value == 0, "the bench's sequences never share a tail block"
        L._check(lib.pkv_batch_block_tables(cache.pool, ids_c.ctypes.data_as(V), B, MB, tables_p, ctx_p))
        ctx_np = pin[r].numpy()[2 * B:3 * B]
        max_ctx = int(ctx_np.max())
        dbuf.copy_(pin[r], non_blocking=True)
        ring_ev[r].record()
        if use_plan:
            L.reset_decode_plan(step_plan)  # new lengths and tables: the first call records again
        # Timed steps 2j and 2j+1 (whole call, partition kernel alone) time
        # the same layer, j mod layers, so both cover every layer alike
        # (with a plan the step's first call records it, the others run
        # from it).
        ev_layer = (timed_idx // 2) % layers if timed_idx >= 0 else -1
        for layer in range(layers):
            opts = ev_opts[timed_idx] if layer == ev_layer else wps_opts
            if traced is not None and layer == traced[0]:
                opts = traced[1]
            L._check(lib.paged_kv_append(*append_args[layer]))
            L._check(lib.paged_attention_decode(*head[layer], max_ctx, *tail, ctypes.byref(opts), stream))
        return int(ctx_np.astype(np.int64).sum())

    import gc
    gc.collect()
    gc.disable()  # a collection pause inside the timed steps would be charged to the GPU path
    for k in range(W):
        step(k, -1)
    torch.cuda.synchronize()
    # Per-XCD weights: XCDs stream K/V at different rates, so equal shares
    # leave the slowest running alone at the end.  'auto' traces the
    # partition kernel of layer 0 on a few untimed steps and weighs each
    # XCD's work by its streaming rate.
    xw, n_cal = None, 0
    if args.xcd_weights == "auto":
        trace = torch.zeros(4 * L.PKV_TRACE_WAVES, dtype=torch.int32, device=dev)
        recs = []
        for c in range(3):
            trace.zero_()
            step(W + c, -1, (0, L.decode_opts(args.partition, args.kernel, None, wps, trace=trace,
                                              load_policy=args.load_policy, plan=step_plan)))
            torch.cuda.synchronize()
            t = trace.cpu().numpy().reshape(-1, 4)
            recs.append(t[t[:, 1] > 0])
        n_cal = 3
        allrec = np.concatenate(recs)[:L.PKV_TRACE_WAVES]
        if len(allrec):
            try:
                xw = L.xcd_weights_from_trace(allrec.reshape(-1))
            except L.PagedKVError:
                xw = None  # some XCD had no traced wave (a small grid): equal shares
    elif args.xcd_weights != "none":
        xw = [int(v) for v in args.xcd_weights.split(",")]
    if xw is not None:
        wps_opts = L.decode_opts(args.partition, args.kernel, None, wps, xw, load_policy=args.load_policy,
                                 plan=step_plan)
        ev_opts = timed_opts(xw)
    W_eff = W + n_cal
    print(f"[bench] warmup done ({W} steps), xcd weights {xw}, timing {K} steps", flush=True)
    ctx_tokens = []
    marks = []
    t0 = time.perf_counter()
    for k in range(K):
        ctx_tokens.append(step(W_eff + k, k))
        marks.append(time.perf_counter())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    if os.environ.get("PKV_BENCH_STEP_TIMES"):
        gaps = np.diff([t0] + marks) * 1e3
        print("[bench] host ms per step (issue):", " ".join(f"{g:.2f}" for g in gaps), flush=True)
    elapsed = t1 - t0
    assert torch.isfinite(out).all().item(), "non-finite attention output"

    kv_bytes = sum(ctx_tokens) * tok_bytes * layers
    gbps = kv_bytes / elapsed / 1e9
    ms_step = elapsed / K * 1e3
    durs_all = [hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(K)]
    hip.destroy(evs)
    durs = durs_all[0::2]  # whole attention call: partition + merge
    durs_part = durs_all[1::2] or durs
    call_us_by_layer = [round(float(np.mean(durs[j::layers])) * 1e3, 2) for j in range(min(layers, len(durs)))]
    avg_ms = sum(durs) / len(durs)
    avg_part_ms = sum(durs_part) / len(durs_part)
    bytes_per_launch = sum(ctx_tokens) / K * tok_bytes  # logical: every sequence's whole context
    # What HBM must deliver: a prefix held once in shared blocks counts once.
    unique_per_launch = bytes_per_launch - (B - 1) * wl.prefix_len * tok_bytes
    achieved = unique_per_launch / (avg_ms * 1e-3) / 1e9
    achieved_logical = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    achieved_part = unique_per_launch / (avg_part_ms * 1e-3) / 1e9
    traffic = stored_traffic(wl.name)
    per_layer_s = elapsed / K / layers
    print(f"[bench] {K} steps in {elapsed:.3f} s; attention call avg {avg_ms * 1e3:.1f} us "
          f"({achieved:.0f} GB/s of distinct K/V, {achieved_logical:.0f} GB/s logical); partition kernel alone "
          f"{avg_part_ms * 1e3:.1f} us", flush=True)
    # Untimed calls with the wave trace: the span of the partition kernel's
    # waves (first start to last end) against its event time, the rate at
    # which its waves read while they run, and how long the last wave runs
    # after the median wave has ended (what a perfectly balanced end would
    # save at most).
    trace = torch.zeros(4 * L.PKV_TRACE_WAVES, dtype=torch.int32, device=dev)
    ev_w = hip.create(2)
    spans, part_us, tails = [], [], []
    for c in range(N_SPAN_CALLS):
        trace.zero_()
        # The last layer's call: with a plan, one that runs from it.
        step(W_eff + K + c, -1, (layers - 1, L.decode_opts(args.partition, args.kernel, (ev_w[0], ev_w[1], None),
                                                           wps, xw, trace=trace, load_policy=args.load_policy,
                                                           plan=step_plan)))
        torch.cuda.synchronize()
        t = trace.cpu().numpy().reshape(-1, 4).astype(np.int64)
        t = t[t[:, 1] > 0]
        if len(t):
            rel = lambda v: (v - t[0, 2] + (1 << 31)) % (1 << 32) - (1 << 31)  # 32-bit clock, 100 MHz
            spans.append((rel(t[:, 3]).max() - rel(t[:, 2]).min()) / 100.0)
            tails.append((rel(t[:, 3]).max() - np.median(rel(t[:, 3]))) / 100.0)
            part_us.append(hip.elapsed_ms(ev_w[0], ev_w[1]) * 1e3)
    hip.destroy(ev_w)
    wave_span = None
    if spans:
        sp, pu = float(np.median(spans)), float(np.median(part_us))
        wave_span = {"partition_event_us": round(pu, 2), "wave_span_us": round(sp, 2),
                     "outside_waves_us": round(pu - sp, 2),
                     "last_end_after_median_end_us": round(float(np.median(tails)), 2),
                     "read_rate_over_span_gbps": round(unique_per_launch / (sp * 1e-6) / 1e9, 1)}
        print(f"[bench] partition kernel waves: span {sp:.1f} us of {pu:.1f} us between events "
              f"({wave_span['read_rate_over_span_gbps']:.0f} GB/s over the span)", flush=True)
    probe, lcost = None, None
    if not args.no_stream_probe:
        probe = stream_probe()
        print(f"[bench] streaming-read probe (1 GiB of 4 KiB tiles), GB/s: {probe}", flush=True)
        lcost = launch_cost()
        print(f"[bench] empty launch on the same grid: {lcost}", flush=True)
    pst = cache.stats()

    res = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,  # queries and matrix-core operands; an int8 cache is widened to it exactly
        "data": "synthetic",
        "config": {"workload": wl.description, "name": wl.name, "batch": B, "num_q_heads": Hq,
                   "num_kv_heads": H, "head_dim": D, "block_size": 16, "kv_cache": wl.cache_dtype,
                   "layers_per_step": layers,
                   "mean_context": round(sum(ctx_tokens) / K / B, 1), "pool_blocks": inst.num_blocks + extra,
                   "min_tokens_per_wave": args.partition or 128, "kernel": args.kernel, "waves_per_simd": wps,
                   "xcd_weights": xw, "tables": args.tables, "load_policy": args.load_policy,
                   "plan": "recorded by each step's first call" if use_plan else "none", "parallelism": "none"},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "attention_pct_of_probe": round(100 * achieved / max(probe[k] for k in probe if k.startswith("random")), 2)
        if probe else None,
        "stream_probe_gbps": probe,
        "launch_cost_us": lcost,
        "partition_wave_span": wave_span,
        "pool": {"blocks": pst["num_blocks"], "usage": round(pst["usage"], 4),
                 "internal_fragmentation": round(pst["internal_fragmentation"], 4),
                 "tokens_logical": pst["tokens_logical"], "tokens_stored": pst["tokens_stored"],
                 "shared_blocks": pst["num_shared"]},
        "decode_tokens_per_s_per_layer": round(B / per_layer_s, 1),
        "decode_tokens_per_s_attention_full_depth": round(B / (per_layer_s * MODEL_LAYERS.get(wl.name, 32)), 1),
        "roofline": {"kernel": "paged_attention_decode (partition kernel + split-context merge)", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "avg_launch_us": round(avg_ms * 1e3, 2),
                     "launch_us_min_median_max": [round(min(durs) * 1e3, 2),
                                                  round(sorted(durs)[len(durs) // 2] * 1e3, 2),
                                                  round(max(durs) * 1e3, 2)],
                     "bytes_per_launch": int(unique_per_launch),
                     "logical_bytes_per_launch": int(bytes_per_launch),
                     "achieved_logical": round(achieved_logical, 2),
                     "call_us_by_layer": call_us_by_layer,
                     "partition_kernel_us": round(avg_part_ms * 1e3, 2),
                     "partition_kernel_frac": round(achieved_part / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_source": "stored rocprofv3 PMC summary of the partition kernel for these kernel sources "
                                       f"(profiles/decode_{wl.name}_traffic.txt), not measured in this run"
                     if traffic else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del gw, cache
        torch.cuda.empty_cache()
        print("[bench] timing the CPU oracle", flush=True)
        base = workloads.configs.scaled(args.workload, batch=args.batch).instantiate() if args.batch else \
            workloads.get(args.workload)
        if args.tables == "identity":
            base.free_order = np.arange(base.num_blocks, dtype=np.int32)
        res["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
