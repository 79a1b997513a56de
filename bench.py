"""Benchmark of the DDTree tree-verify hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
ddtree_build_mask -> ddtree_verify_attn (bf16 MFMA, + split merge when split)
-> ddtree_greedy_accept (vocab argmax + path walk).  Default workload: Kimi-K2
shapes with a long context and the accept step -- 4 requests x 128-node draft
trees x 64 heads, kv_lora 512 + rope 64, 131072-token cached prefixes, logits
[4, 128, 163840] float32.  Inputs are seeded synthetic draws, resident in HBM
before the timed region.

Prints one JSON line.  `value` is the algorithmic attention TFLOP/s over the
whole step (mask + attention + accept); the per-kernel figures, the roofline
of the dominant kernel (the bf16 attention kernel, timed with HIP events on
its launch stream) and the CPU oracle baseline on a bounded sample are in the
same line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
ATTN_KERNEL = "verify_attn_bf16_kernel"
ATTN_SOURCE = os.path.join(ROOT, "mla_tree_verify_absorb_amd", "csrc", "verify_attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_bf16_k2_long_context_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, help="workload number (3, 4 or 5); 5 is the headline")
    ap.add_argument("--heads", type=int, default=0,
                    help="override the workload's head count (8: one GPU's share under 8-way head parallelism)")
    ap.add_argument("--splits", type=int, default=0,
                    help="uniform KV splits (0 = the library's automatic schedule)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget (0 = skip)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the attention-only timings of workloads 3 and 4 in the default run")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB --steps times (HBM counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("ATTN_FETCH", "ATTN_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: write the HBM-traffic file from four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of the default workload's attention, then of --copy-calibration-mb 1024)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """A plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE counters calibrate HBM traffic."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": steps}), flush=True)


def summarize_traffic(dirs, copy_mib=1024, out_path=TRAFFIC_FILE):
    """HBM bytes per launch of the attention kernel from rocprofv3 --pmc runs: each counter's per-dispatch value
    (KiB) averaged over the kernel's dispatches, scaled by copy bytes / the same counter's reading for the plain copy
    of known size.  Writes out_path (the file the bench line reads), keyed to this kernel source's code hash and the
    workload's flops."""
    import csv
    import glob

    import numpy as np

    from synth import make_config

    def mean_counter(d, name):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        with open(files[0]) as f:
            vals = [float(r["Counter_Value"]) for r in csv.DictReader(f) if name in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no {name} dispatch in {files[0]}")
        return sum(vals) / len(vals), len(vals)

    fetch, nf = mean_counter(dirs[0], ATTN_KERNEL)
    write, nw = mean_counter(dirs[1], ATTN_KERNEL)
    cfetch, _ = mean_counter(dirs[2], "copyBuffer")
    cwrite, _ = mean_counter(dirs[3], "copyBuffer")
    copy_kib = copy_mib * 1024.0
    fs, ws = copy_kib / cfetch, copy_kib / cwrite
    w = make_config(5)
    depth = np.zeros_like(w.parents)
    for i in range(1, w.N):
        depth[:, i] = depth[np.arange(w.B), w.parents[:, i]] + 1
    flops, _, _ = algorithmic_work(w, depth)
    base = "rocprofv3 --pmc {c} -d <dir> -o {o} --output-format csv -- python3 bench.py {a}"
    attn = "--steps 2 --warmup 1 --cpu-seconds 0 --no-other-workloads"
    copy = f"--copy-calibration-mb {copy_mib} --steps 3"
    out = {
        "kernel": ATTN_KERNEL,
        "workload": "k2-long-context-accept (B4 N128 H64 Dl512 Dr64 L131072)",
        "source_sha256_16": source_hash(ATTN_SOURCE),
        "launch_flops": int(flops),
        "fetch_kib_per_launch_raw": fetch, "write_kib_per_launch_raw": write, "dispatches": [nf, nw],
        "copy_calibration": {"copy_bytes": copy_mib << 20, "fetch_kib_raw": cfetch, "write_kib_raw": cwrite,
                             "fetch_scale": round(fs, 5), "write_scale": round(ws, 5)},
        "hbm_bytes_per_launch": int(round((fetch * fs + write * ws) * 1024)),
        "commands": [base.format(c="FETCH_SIZE", o="bench", a=attn), base.format(c="WRITE_SIZE", o="bench", a=attn),
                     base.format(c="FETCH_SIZE", o="copy", a=copy), base.format(c="WRITE_SIZE", o="copy", a=copy),
                     "python3 bench.py --summarize-traffic <attn FETCH dir> <attn WRITE dir> <copy FETCH dir> "
                     "<copy WRITE dir>"],
        "source_hash_rule": "sha256 of the kernel source with comments, blank lines and whitespace runs removed "
                            "(bench.py source_hash)",
    }
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps({"hbm_bytes_per_launch": out["hbm_bytes_per_launch"], "file": out_path}))
    return out


def source_hash(path):
    """Hash of the kernel source's code: comments, blank lines and runs of whitespace are dropped, so that only
    a change of the code itself invalidates HBM counters taken on it."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = [" ".join(re.sub(r"//.*$", "", l).split()) for l in text.splitlines()]
    code = "\n".join(l for l in lines if l)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def algorithmic_work(w, depth):
    """Attention flops / bytes and accept bytes of one step (see the design notes)."""
    import numpy as np
    vis = (w.prefix_lens[:, None] + depth.astype(np.int64) + 1)          # keys seen by each node
    keys_total = int(vis.sum())
    flops = 2 * w.H * (2 * w.Dl + w.Dr) * keys_total
    esz = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.N * w.H
    attn_bytes = (int(w.prefix_lens.sum()) * (w.Dl + w.Dr) * esz           # prefix KV read once
                  + w.B * w.N * (w.Dl + w.Dr) * esz                         # tree KV
                  + rows * (w.Dl + w.Dr) * esz                              # queries
                  + rows * w.Dl * 4 + rows * 4                              # o, lse
                  + w.B * w.N * ((w.N + 31) // 32) * 4)                     # mask
    accept_bytes = w.B * w.N * w.V * 4 if w.V else 0
    return flops, attn_bytes, accept_bytes


def cpu_baseline(w, budget_s):
    """The oracle as it stands, on request 0's first n nodes (all heads, full prefix)."""
    import numpy as np
    from oracle import build_mask_ref, verify_attn_ref
    from synth import restrict
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
        blas_name = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or None
    except Exception:
        threads, blas_name = os.cpu_count() or 1, None
    f = w.f32
    kv = f("kv")
    kt = f("kv_tree")
    done_flops = 0
    elapsed = 0.0
    n_done = 0
    n = 1
    while n <= w.N and elapsed < budget_s:
        sub = restrict(w, 0, n)
        mask, depth, _, _ = build_mask_ref(sub.parents, sub.prefix_lens)
        L = int(sub.prefix_lens[0])
        node = n - 1                                   # time node n-1 alone over the full prefix
        t0 = time.perf_counter()
        verify_attn_ref(f("q_lat")[:1, :n], f("q_rope")[:1, :n], kv[:L, :w.Dl], kv[:L, w.Dl:], sub.prefix_offsets,
                        kt[:1, :n, :w.Dl], kt[:1, :n, w.Dl:], mask, w.scale, nodes=[(0, node)])
        elapsed += time.perf_counter() - t0
        done_flops += 2 * w.H * (2 * w.Dl + w.Dr) * (L + int(depth[0, node]) + 1)
        n_done += 1
        n += 1
    return {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"request 0, tree nodes 0..{n_done - 1} one at a time (all {w.H} heads), full "
                      f"{int(w.prefix_lens[0])}-token prefix, float64 NumPy; {elapsed:.1f} s of oracle time",
            "seconds": round(elapsed, 2), "host_cpus": os.cpu_count(), "blas_threads": int(threads),
            "blas": blas_name, "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name (first /proc/cpuinfo entry)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_time_us(torch, dev, fn, steps):
    """Mean GPU time of fn() in microseconds: a GPU-side spin ahead of each pair of events keeps the host's
    call overhead out of the measured interval."""
    fn()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_ms = 0.0
    for _ in range(steps):
        torch.cuda._sleep(200000)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        total_ms += e0.elapsed_time(e1)
    return round(total_ms * 1e3 / steps, 2)


def time_compaction(dd, torch, w, kv_tree, accept_len, accept_nodes, steps):
    """Post-verify KV-cache compaction of this step's accepted paths (outside the timed step): each request's
    path rows go to its own N-row region of a scratch cache.  Latency-bound: a few KB per request."""
    dev = kv_tree.device
    cache = torch.zeros((w.B * w.N, w.Dl + w.Dr), dtype=kv_tree.dtype, device=dev)
    dest = torch.arange(w.B, dtype=torch.int64, device=dev) * w.N
    args = (kv_tree[..., :w.Dl], kv_tree[..., w.Dl:], accept_len, accept_nodes, dest, cache[:, :w.Dl],
            cache[:, w.Dl:])
    us = gpu_time_us(torch, dev, lambda: dd.ddtree_compact_kv(*args), steps)
    rows = int(accept_len.sum()) + w.B
    return {"us_per_call": us, "rows_moved": rows, "bytes_moved": 2 * rows * (w.Dl + w.Dr) * kv_tree.element_size()}


def time_tree_builder(dd, torch, w, dev, steps, tree_spec):
    """The best-first draft-tree builder at this workload's tree shape (outside the timed step): N nodes from
    D draft depths of K proposals each, (D, K) = the workload's depth and branching bounds (12 and 4 for the
    long-context workload), from seeded synthetic drafter proposals."""
    from synth import make_draft_candidates
    D, K = (int(tree_spec[1]), int(tree_spec[2])) if tree_spec[0] == "bounded" else (8, 4)
    c = make_draft_candidates(B=w.B, D=D, K=K, V=max(w.V, 1000), seed=1)
    args = (torch.from_numpy(c.root_tokens).to(dev), torch.from_numpy(c.cand_tokens).to(dev),
            torch.from_numpy(c.cand_logp).to(dev), w.N)
    us = gpu_time_us(torch, dev, lambda: dd.ddtree_build_tree(*args), steps)
    return {"us_per_call": us, "requests": w.B, "nodes": w.N, "depths": D, "proposals": K}


def time_rope(dd, torch, w, dev, q_rope, kv_tree, positions, steps):
    """NeoX rotation of the tree nodes' rotary queries (all heads) and keys at their positions (outside the
    timed step; on copies, so the step's inputs stay as they are)."""
    import numpy as np
    q = q_rope.clone()
    kt = kv_tree.clone()
    inv = torch.from_numpy(10000.0 ** (-np.arange(0, w.Dr, 2, dtype=np.float64) / w.Dr)).to(dev)
    us = gpu_time_us(torch, dev, lambda: dd.ddtree_rope_tree(q, kt[..., w.Dl:], positions, inv), steps)
    rows = w.B * w.N * (w.H + 1)
    return {"us_per_call": us, "rows": rows, "bytes_moved": 2 * rows * w.Dr * q_rope.element_size()}


def reference_rates(torch, dev, accept_bytes=0):
    """Rates this GPU attains on plain work, as context for the vendor peaks: a large dense bf16 GEMM
    (torch.matmul, hipBLASLt), a plain 1 GiB device-to-device copy (read + write bytes), and the library's own
    probes: back-to-back bf16 MFMAs, and a read-only stream of 2 GiB and of the accept call's logits size (the
    best of three workgroup counts each).  None is part of the verify path."""
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    x = torch.ones(((1 << 30) // 4,), device=dev, dtype=torch.float32)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(fn, reps=10):
        for _ in range(3):
            fn()
        times = []
        for _ in range(reps):
            torch.cuda._sleep(100000)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]

    gemm_ms = best_ms(lambda: torch.matmul(a, b, out=c))
    copy_ms = best_ms(lambda: y.copy_(x))
    # the library's own probes: back-to-back bf16 MFMAs on every SIMD, and read-only streams
    from mla_tree_verify_absorb_amd import rates
    wgs, iters = 512, 40000                       # two waves per SIMD on 256 CUs
    sink = torch.empty((wgs * 4,), dtype=torch.float32, device=dev)
    mfma_flops = rates.mfma_loop(wgs, iters, sink)
    mfma_ms = best_ms(lambda: rates.mfma_loop(wgs, iters, sink), reps=5)
    rd_counts = (1024, 2048, 4096)
    rsink = torch.empty((max(rd_counts) * 256,), dtype=torch.int32, device=dev)
    buf = torch.ones(((2 << 30) // 4,), dtype=torch.float32, device=dev)

    def best_stream(nbytes):
        view = buf[: nbytes // 4]
        rd_ms = min(best_ms(lambda: rates.stream_read(view, g, rsink)) for g in rd_counts)
        return round(nbytes / (rd_ms * 1e-3) / 1e9, 1)
    out = {"gemm_bf16_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
           "gemm_shape": [n, n, n],
           "copy_gbps": round(2 * x.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1),
           "copy_bytes_moved": 2 * x.numel() * 4,
           "mfma_loop_bf16_tflops": round(mfma_flops / (mfma_ms * 1e-3) / 1e12, 1),
           "mfma_loop": f"{wgs} workgroups x 4 waves, {iters} iterations of 4 independent "
                        f"v_mfma_f32_32x32x16_bf16 per wave, median of 5",
           "stream_read_gbps": best_stream(buf.numel() * 4),
           "stream_read_bytes": buf.numel() * 4,
           "stream_read": f"contiguous spans per workgroup, 8 nontemporal 16-byte loads in flight per thread, "
                          f"best of {list(rd_counts)} workgroups of 256 threads"}
    if 0 < accept_bytes <= buf.numel() * 4 and accept_bytes % 16 == 0:
        out["stream_read_accept_size_gbps"] = best_stream(accept_bytes)
        out["stream_read_accept_size_bytes"] = accept_bytes
    del a, b, c, x, y, buf
    return out


def attention_only(dd, torch, dev, k, steps, warmup):
    """Mask + attention of workload k (its full shape, the automatic schedule) timed like the main step:
    HIP events around the attention call (attention kernel and split merge) on its stream."""
    import numpy as np
    from synth import make_config
    w = make_config(k)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    parents = torch.from_numpy(w.parents).to(dev)
    offsets = torch.from_numpy(w.prefix_offsets).to(dev)
    q_lat, q_rope = to_dev(w.q_lat), to_dev(w.q_rope)
    kv, kv_tree = to_dev(w.kv), to_dev(w.kv_tree)
    max_len = int(w.prefix_lens.max())
    splits = dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, max_len)
    ws = torch.empty((max(dd.ddtree_verify_attn_workspace_size(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, max_len,
                                                               splits), 1),), dtype=torch.uint8, device=dev)
    mask, depth, _, ok = dd.ddtree_build_mask(parents, offsets)
    o = torch.empty((w.B, w.N, w.H, w.Dl), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.N, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def attn():
        dd.ddtree_verify_attn(q_lat, q_rope, kv[:, :w.Dl], kv[:, w.Dl:], offsets, max_len, kv_tree[..., :w.Dl],
                              kv_tree[..., w.Dl:], mask, w.scale, num_splits=splits, o=o, lse=lse, workspace=ws)

    for _ in range(warmup):
        attn()
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(steps):
        torch.cuda._sleep(100000)                     # keep host launch latency out of the event interval
        e0.record(stream)
        attn()
        e1.record(stream)
        e1.synchronize()
        total += e0.elapsed_time(e1)
    assert int(ok.min()) == 1 and bool(torch.isfinite(o).all())
    attn_ms = total / steps
    flops, attn_bytes, _ = algorithmic_work(w, depth.cpu().numpy())
    tflops = flops / (attn_ms * 1e-3) / 1e12
    out = {"batch": w.B, "tree_nodes": w.N, "heads": w.H, "prefix_len_total": int(w.prefix_lens.sum()),
           "prefix_len_max": max_len, "schedule": "band" if splits == 0 else f"uniform-{splits}",
           "attn_ms": round(attn_ms, 4), "attn_tflops": round(tflops, 2),
           "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
           "algorithmic_bytes": attn_bytes, "workspace_bytes": ws.numel()}
    del q_lat, q_rope, kv, kv_tree, o, lse, ws
    return out


def traffic_for_current_kernel(launch_flops):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(ATTN_SOURCE) or t.get("launch_flops") != launch_flops:
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library runs a GPU's share of the work "
              f"(requests, heads or a prefix slice); the collectives that would join several GPUs are not implemented",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, args.steps)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    import numpy as np
    import torch

    import mla_tree_verify_absorb_amd as dd
    from synth import CONFIGS, make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w = make_config(args.config, heads=args.heads or None)
    gen_s = time.perf_counter() - t_gen

    def to_dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    parents = torch.from_numpy(w.parents).to(dev)
    offsets = torch.from_numpy(w.prefix_offsets).to(dev)
    q_lat, q_rope = to_dev(w.q_lat), to_dev(w.q_rope)
    kv, kv_tree = to_dev(w.kv), to_dev(w.kv_tree)
    ckv, krope = kv[:, :w.Dl], kv[:, w.Dl:]
    ckv_t, krope_t = kv_tree[..., :w.Dl], kv_tree[..., w.Dl:]
    logits = torch.from_numpy(w.logits).to(dev) if w.logits is not None else None
    tokens = torch.from_numpy(w.tokens).to(dev) if w.tokens is not None else None
    max_len = int(w.prefix_lens.max())
    code = dd.DDTREE_BF16 if w.dtype == "bf16" else dd.DDTREE_F32
    splits = args.splits or dd.ddtree_verify_attn_auto_splits(code, w.B, w.N, w.H, w.Dl, w.Dr, max_len)
    schedule = "band" if splits == 0 else f"uniform-{splits}"
    ws_bytes = dd.ddtree_verify_attn_workspace_size(code, w.B, w.N, w.H, w.Dl, w.Dr, max_len, splits)
    workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    W = (w.N + 31) // 32
    mask = torch.empty((w.B, w.N, W), dtype=torch.int32, device=dev)
    depth = torch.empty((w.B, w.N), dtype=torch.int32, device=dev)
    positions = torch.empty((w.B, w.N), dtype=torch.int64, device=dev)
    tree_ok = torch.empty((w.B,), dtype=torch.int32, device=dev)
    o = torch.empty((w.B, w.N, w.H, w.Dl), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.N, w.H), dtype=torch.float32, device=dev)
    acc_out = None
    if logits is not None:
        acc_out = [torch.empty((w.B, w.N), dtype=torch.int32, device=dev), torch.empty((w.B,), dtype=torch.int32,
                   device=dev), torch.empty((w.B, w.N), dtype=torch.int32, device=dev),
                   torch.empty((w.B, w.N), dtype=torch.int32, device=dev)]
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(timed):
        if timed:
            ev[0].record(stream)
        dd.ddtree_build_mask(parents, offsets, mask=mask, depth=depth, positions=positions, tree_ok=tree_ok)
        if timed:
            ev[1].record(stream)
        dd.ddtree_verify_attn(q_lat, q_rope, ckv, krope, offsets, max_len, ckv_t, krope_t, mask, w.scale,
                              num_splits=splits, o=o, lse=lse, workspace=workspace)
        if timed:
            ev[2].record(stream)
        if logits is not None:
            dd.ddtree_greedy_accept(logits, tokens, parents, target_argmax=acc_out[0], accept_len=acc_out[1],
                                    accept_nodes=acc_out[2], commit_tokens=acc_out[3])
        if timed:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t_mask = t_attn = t_acc = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        ev[3].synchronize()
        t_mask += ev[0].elapsed_time(ev[1])
        t_attn += ev[1].elapsed_time(ev[2])
        t_acc += ev[2].elapsed_time(ev[3])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    K = args.steps
    mask_ms, attn_ms, acc_ms = t_mask / K, t_attn / K, t_acc / K
    step_ms = mask_ms + attn_ms + acc_ms
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "non-finite attention output"
    assert int(tree_ok.min()) == 1

    flops, attn_bytes, accept_bytes = algorithmic_work(w, depth.cpu().numpy())
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    value = flops / (step_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for_current_kernel(flops), "kernel": ATTN_KERNEL,
                "launch_ms": round(attn_ms, 4), "algorithmic_flops": flops, "algorithmic_bytes": attn_bytes}
    out = {
        "metric": "tree-verify attn TFLOP/s & HBM GB/s (% roofline); verify steps/sec at K2 shape",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "tree_nodes": w.N, "heads": w.H,
                   "kv_lora": w.Dl, "rope_dim": w.Dr, "prefix_len_max": max_len,
                   "prefix_len_total": int(w.prefix_lens.sum()), "vocab": w.V, "schedule": schedule},
        "verify_steps_per_s": round(1e3 / step_ms, 2),
        "attn_tflops": round(attn_tflops, 2),
        "attn_hbm_gbps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "mask_ms": round(mask_ms, 4), "attn_ms": round(attn_ms, 4), "accept_ms": round(acc_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": roofline,
    }
    if accept_bytes:
        gbps = accept_bytes / (acc_ms * 1e-3) / 1e9
        out["accept_hbm_gbps"] = round(gbps, 1)
        out["accept_hbm_frac"] = round(gbps / HBM_PEAK_GBPS, 4)
        out["compact_kv"] = time_compaction(dd, torch, w, kv_tree, acc_out[1], acc_out[2], args.steps)
    if args.config == 5 and args.heads == 0 and args.splits == 0 and not args.no_other_workloads:
        out["other_workloads"] = {CONFIGS[k]["name"]: attention_only(dd, torch, dev, k, args.steps, args.warmup)
                                  for k in (3, 4)}
    ref = reference_rates(torch, dev, accept_bytes)
    roofline["frac_of_measured_gemm"] = round(attn_tflops / ref["gemm_bf16_tflops"], 4)
    roofline["frac_of_measured_mfma_loop"] = round(attn_tflops / ref["mfma_loop_bf16_tflops"], 4)
    if accept_bytes:
        out["accept_frac_of_measured_copy"] = round(out["accept_hbm_gbps"] / ref["copy_gbps"], 4)
        out["accept_frac_of_measured_stream_read"] = round(out["accept_hbm_gbps"] / ref["stream_read_gbps"], 4)
        if "stream_read_accept_size_gbps" in ref:
            out["accept_frac_of_same_size_stream_read"] = round(
                out["accept_hbm_gbps"] / ref["stream_read_accept_size_gbps"], 4)
    for sub in out.get("other_workloads", {}).values():
        sub["frac_of_measured_mfma_loop"] = round(sub["attn_tflops"] / ref["mfma_loop_bf16_tflops"], 4)
    out["reference_rates"] = ref
    out["build_tree"] = time_tree_builder(dd, torch, w, dev, args.steps, CONFIGS[args.config]["tree"])
    out["rope_tree"] = time_rope(dd, torch, w, dev, q_rope, kv_tree, positions, args.steps)
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    out["input_generation_s"] = round(gen_s, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
