#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

A step is one forward pass (fa_fwd) followed by one backward pass (fa_bwd)
of bf16 causal attention over one batch of seeded synthetic input that is
already resident in device memory.  Default workload: B=8, H=16, N=2048,
d=128 (the bf16 causal configuration the headline metric is quoted on).

Throughput counts 4*B*H*N^2*d FLOP for the forward, halved for causal, and
2.5x that for the backward.  Kernel time is taken with HIP events on the
stream the kernels are launched on (torch's current stream).  Rank 0 prints
one JSON line; see ``--help`` for the options.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # 256 CUs x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz = 2516.6
PEAK_HBM_GBS = 8000.0
# v_exp_f32 throughput measured on the MI355X with a dependent-free exp loop:
# 26.5 results per clock per CU; at 256 CUs and 2.4 GHz that is 16.3e12 exp/s.
EXP_PER_CLK_PER_CU = 26.5
EXP_RATE = 256 * EXP_PER_CLK_PER_CU * 2.4e9
COLD_BUFFER_BYTES = 512 << 20  # larger than the 256 MB MALL: writing it evicts the inputs


def flops(p, passes):
    f = 4.0 * p.B * p.Hq * p.N * p.N * p.d
    if p.causal:
        f /= 2
    total = 0.0
    if "fwd" in passes:
        total += f
    if "bwd" in passes:
        total += 2.5 * f
    return total, f


def alg_bytes_fwd(p):
    """Algorithmic HBM bytes of one forward launch: Q, K, V read once, O
    written once, LSE written (float32)."""
    e = 2 if p.dtype == "bf16" else 4
    return (2 * p.B * p.Hq * p.N * p.d + 2 * p.B * p.Hkv * p.N * p.d) * e + 4 * p.B * p.Hq * p.N


FWD_SOURCES = ["io_aware_transformer_amd/csrc/fa_fwd_bf16.hip", "io_aware_transformer_amd/csrc/fa_device.hpp"]


def fwd_source_hash():
    """sha256 over the forward kernel's sources: ties stored counter data to
    the kernel it was measured on."""
    import hashlib

    h = hashlib.sha256()
    for rel in FWD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(p):
    """HBM bytes per forward launch from profiles/fwd_traffic_<preset>.json
    (FETCH_SIZE / WRITE_SIZE counter runs scaled by the copy calibration),
    or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"fwd_traffic_{p.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != fwd_source_hash():
        return None
    return t


def window_pairs(n, left, right):
    """Number of (query, key) pairs a window (left, right) leaves visible."""
    total = 0
    for i in range(n):
        a = 0 if left < 0 else max(0, i - left)
        b = n - 1 if right < 0 else min(n - 1, i + right)
        total += b - a + 1
    return total


def exp_count(p):
    """Exponentials one forward pass evaluates (one per unmasked score, the
    causal half by the same convention as the FLOP count)."""
    n = float(p.B) * p.Hq * p.N * p.N
    return n / 2 if p.causal else n


def pct(x, q):
    """q-th percentile (nearest rank) of a list."""
    x = sorted(x)
    return x[min(len(x) - 1, max(0, int(math.ceil(q / 100.0 * len(x))) - 1))]


_CPU_LEG = {}  # inputs and GPU results the CPU leg's forked workers read


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_unit(unit):
    """Worker: the fp64 oracle on one (b, h) unit of the workload, timed, and
    the max-abs difference of the GPU's outputs for that unit."""
    import numpy as np

    import oracle

    b, h = unit
    d = _CPU_LEG
    p, passes = d["p"], d["passes"]
    g = h // (p.Hq // p.Hkv)
    q, k, v, do = (d[n][b, h if n in ("q", "do") else g] for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    o, lse = oracle.head_forward(q, k, v, p.scale, p.causal)
    grads = oracle.head_backward(q, k, v, do, p.scale, p.causal) if "bwd" in passes else None
    dt = time.perf_counter() - t0
    err = {"O": (float(np.max(np.abs(d["o"][b, h] - o))), float(np.max(np.abs(o)))),
           "LSE": (float(np.max(np.abs(d["lse"][b, h] - lse))), float(np.max(np.abs(lse))))}
    if grads is not None:
        err["dQ"] = (float(np.max(np.abs(d["dq"][b, h] - grads[0]))), float(np.max(np.abs(grads[0]))))
        if p.Hq == p.Hkv:  # grouped heads: a unit holds only part of dK / dV
            err["dK"] = (float(np.max(np.abs(d["dk"][b, g] - grads[1]))), float(np.max(np.abs(grads[1]))))
            err["dV"] = (float(np.max(np.abs(d["dv"][b, g] - grads[2]))), float(np.max(np.abs(grads[2]))))
    return dt, err


def cpu_baseline(p, passes, budget_s, m):
    """The fp64 oracle timed on the host's cores over (b, h) units of the same
    workload (the GPU's own inputs), a pool of single-threaded workers (one
    BLAS thread each, at most 16: this host's share), in rounds of one unit
    per worker until ``budget_s`` of wall time is spent.  The same units give
    the GPU outputs' max-abs errors against the oracle (and the oracle's
    largest magnitudes), per output."""
    import multiprocessing

    import numpy as np

    t = m["tensors"]
    f64 = lambda x: x.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    _CPU_LEG.clear()
    _CPU_LEG.update({"p": p, "passes": passes})
    for n in ("q", "k", "v", "do", "o", "lse", "dq", "dk", "dv"):
        if t[n] is not None:
            _CPU_LEG[n] = f64(t[n])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores))
    # memory: about 8 N x N float64 arrays live per worker
    mem_per = 8 * 8 * p.N * p.N
    try:
        avail = os.sysconf("SC_AVPHYS_PAGES") * os.sysconf("SC_PAGE_SIZE")
        workers = max(1, min(workers, int(avail * 0.5 // mem_per)))
    except (ValueError, OSError):  # pragma: no cover
        avail = None
    units = m["units"]
    rng = np.random.default_rng(p.seed)
    order = [units[i] for i in rng.permutation(len(units))]
    done, errs = 0, {}
    t0 = time.perf_counter()
    with multiprocessing.get_context("fork").Pool(workers, initializer=_blas_one_thread) as pool:
        while done < len(order) and (done == 0 or time.perf_counter() - t0 < budget_s):
            for _, e in pool.map(_oracle_unit, order[done:done + workers]):
                for name, (err, top) in e.items():
                    a, b = errs.get(name, (0.0, 0.0))
                    errs[name] = (max(a, err), max(b, top))
            done += len(order[done:done + workers])
    dt = time.perf_counter() - t0
    _CPU_LEG.clear()
    unit_flops = flops(p, passes)[0] / (p.B * p.Hq)
    return {
        "value": round(done * unit_flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{done} of {len(units)} (batch, head) units of the workload ({'+'.join(passes)}, N={p.N} "
                  f"d={p.d}, fp64 numpy) on {workers} single-threaded worker processes in {dt:.1f} s, same FLOP "
                  f"count per unit as the GPU line",
        "parity_on_sample": {k: {"max_abs_err": round(v[0], 7), "oracle_max_abs": round(v[1], 5)}
                             for k, v in errs.items()},
    }


def alg_bytes_split(p):
    """Algorithmic HBM bytes of one split forward: Q, K, V read once, O and
    LSE written once (the float32 partials are implementation traffic)."""
    return 2 * (2 * p.B * p.Hq * p.Nq * p.d + 2 * p.B * p.Hkv * p.Nk * p.d) + 4 * p.B * p.Hq * p.Nq


def cpu_baseline_split(p, budget_s):
    """The fp64 oracle on (b, h_kv-group) units of the split workload."""
    import numpy as np

    import oracle
    from io_aware_transformer_amd import inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    G = p.Hq // p.Hkv
    q, k, v = inputs.make_split(1, G, 1, p.Nq, p.Nk, p.d, p.torch_dtype, p.seed)
    q, k, v = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    units = 0
    t0 = time.perf_counter()
    while True:
        oracle.cross_forward(q, k, v, p.scale, p.causal)
        units += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    unit_bytes = alg_bytes_split(p) / (p.B * p.Hkv)
    return {"value": round(units * unit_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} (batch, kv head) units of N_q={p.Nq} x N_k={p.Nk} d={p.d} ({G} query heads each) "
                      f"in {dt:.1f} s, same algorithmic bytes per unit as the GPU line"}


def bench_split(args, p):
    """Split key/value forward (decoding workloads): one step is one
    fa_fwd_split call (partials + merge) over the whole batch."""
    import torch

    from io_aware_transformer_amd import fwd_split, fwd_split_parts, fwd_split_workspace_size, inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs.make_split_preset(p))
    stream = torch.cuda.current_stream(dev)

    def timed(splits, steps, warmup):
        ws = torch.empty(max(1, fwd_split_workspace_size(p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d, splits)), device=dev,
                         dtype=torch.uint8)
        o = torch.empty_like(q)
        lse = torch.empty((p.B, p.Hq, p.Nq), device=dev, dtype=torch.float32)
        for _ in range(warmup):
            fwd_split(q, k, v, scale=p.scale, causal=p.causal, num_splits=splits, out=o, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.min_warmup_seconds:
            for _ in range(20):
                fwd_split(q, k, v, scale=p.scale, causal=p.causal, num_splits=splits, out=o, lse=lse, workspace=ws)
            torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            fwd_split(q, k, v, scale=p.scale, causal=p.causal, num_splits=splits, out=o, lse=lse, workspace=ws)
            e[1].record(stream)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in evs]

    ms = timed(0, args.steps, args.warmup)
    avg = sum(ms) / len(ms)
    gbs = alg_bytes_split(p) / (avg * 1e-3) / 1e9
    one = timed(1, max(5, args.steps // 5), 2)
    one_avg = sum(one) / len(one)
    line = {
        "metric": "split key/value forward: algorithmic HBM GB/s (bf16, decoding shapes)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V rounded to bf16, resident in HBM",
        "config": {"workload": f"{p.name}: split fwd {p.dtype} {'causal' if p.causal else 'non-causal'} B={p.B} "
                               f"H_q={p.Hq} H_kv={p.Hkv} N_q={p.Nq} N_k={p.Nk} d={p.d}",
                   "parts": fwd_split_parts(p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d, 0)},
        "ms_p10_p90": [round(pct(ms, 10), 5), round(pct(ms, 90), 5)],
        "roofline": {"bound": "hbm", "kernel": "fwd_split_kernel + lse_merge_kernel (one fa_fwd_split call)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "alg_bytes": alg_bytes_split(p)},
        "unsplit": {"parts": 1, "ms": round(one_avg, 5),
                    "gbs": round(alg_bytes_split(p) / (one_avg * 1e-3) / 1e9, 1)},
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline_split(p, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def varlen_flops(p):
    """Forward FLOP of a packed batch: 4*H*n^2*d per sequence of n tokens
    (halved for causal, the convention of ``flops``)."""
    f = sum(4.0 * p.Hq * n * n * p.d for n in p.lengths)
    return f / 2 if p.causal else f


def cpu_baseline_varlen(p, budget_s):
    """The fp64 oracle on (sequence, head) units of the pack, sequences taken
    in order, forward and backward, until ``budget_s`` of CPU work is done."""
    import numpy as np

    import oracle
    from io_aware_transformer_amd import inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v, do, cu = inputs.make_varlen_preset(p)
    done_flops, units = 0.0, 0
    t0 = time.perf_counter()
    for s in range(len(p.lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        x = [t[0, a:b].float().numpy().astype(np.float64) for t in (q, k, v, do)]
        oracle.head_forward(x[0], x[1], x[2], p.scale, p.causal)
        oracle.head_backward(*x, p.scale, p.causal)
        n = b - a
        done_flops += 3.5 * 4.0 * n * n * p.d / (2 if p.causal else 1)
        units += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} (sequence, head) units of the pack (fwd+bwd) in {dt:.1f} s, same FLOP "
                      f"convention as the GPU line"}


def bench_varlen(args, p):
    """Packed variable-length batch: one step is fa_fwd_varlen then
    fa_bwd_varlen over the whole pack.  The same sequences padded to the
    longest one and run through fa_fwd / fa_bwd are timed beside it."""
    import torch

    from io_aware_transformer_amd import bwd, bwd_varlen, bwd_varlen_workspace_size, fwd, fwd_varlen, inputs

    dev = torch.device("cuda:0")
    lens = p.lengths
    mx = max(lens)
    q, k, v, do, cu = (t.to(dev) for t in inputs.make_varlen_preset(p))
    o = torch.empty_like(q)
    lse = torch.empty((p.Hq, p.total), device=dev, dtype=torch.float32)
    ws = torch.empty(max(1, bwd_varlen_workspace_size(p.total, p.Hq, p.Hkv, p.d)), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def run(f, b, steps, warmup):
        for _ in range(warmup):
            f()
            b()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.min_warmup_seconds:
            for _ in range(5):
                f()
                b()
            torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            f()
            e[1].record(stream)
            b()
            e[2].record(stream)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in evs], [e[1].elapsed_time(e[2]) for e in evs]

    fwd_ms, bwd_ms = run(lambda: fwd_varlen(q, k, v, cu, mx, scale=p.scale, causal=p.causal, out=o, lse=lse),
                         lambda: bwd_varlen(q, k, v, o, lse, do, cu, mx, scale=p.scale, causal=p.causal,
                                            workspace=ws),
                         args.steps, args.warmup)
    ff = varlen_flops(p)
    fa, ba = sum(fwd_ms) / len(fwd_ms), sum(bwd_ms) / len(bwd_ms)
    ms = fa + ba
    value = 3.5 * ff / (ms * 1e-3) / 1e12

    # Padded comparison: B = number of sequences, N = the longest length.
    B = len(lens)
    pq = torch.zeros((B, p.Hq, mx, p.d), device=dev, dtype=q.dtype)
    pk = torch.zeros((B, p.Hkv, mx, p.d), device=dev, dtype=q.dtype)
    pv, pdo = torch.zeros_like(pk), torch.zeros_like(pq)
    c = cu.cpu()
    for s in range(B):
        a, b = int(c[s]), int(c[s + 1])
        pq[s, :, : b - a] = q[:, a:b]
        pk[s, :, : b - a] = k[:, a:b]
        pv[s, :, : b - a] = v[:, a:b]
        pdo[s, :, : b - a] = do[:, a:b]
    po, plse = fwd(pq, pk, pv, scale=p.scale, causal=p.causal)
    pf, pb = run(lambda: fwd(pq, pk, pv, scale=p.scale, causal=p.causal, out=po, lse=plse),
                 lambda: bwd(pq, pk, pv, po, plse, pdo, scale=p.scale, causal=p.causal),
                 max(5, args.steps // 4), 2)
    pms = sum(pf) / len(pf) + sum(pb) / len(pb)
    line = {
        "metric": "attention fwd/bwd TFLOP/s (bf16, causal, d=128, N=2K-8K) + % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V, dO rounded to bf16, seeded log-uniform lengths, resident in HBM",
        "config": {"workload": f"{p.name}: fwd+bwd packed variable-length {p.dtype} "
                               f"{'causal' if p.causal else 'non-causal'} {len(lens)} sequences, total={p.total} "
                               f"(lengths {min(lens)}..{mx}) H_q={p.Hq} H_kv={p.Hkv} d={p.d}",
                   "lengths": lens},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(ff / (fa * 1e-3) / 1e12, 2),
        "fwd_ms_p10_p90": [round(pct(fwd_ms, 10), 5), round(pct(fwd_ms, 90), 5)],
        "bwd_tflops": round(2.5 * ff / (ba * 1e-3) / 1e12, 2),
        "bwd_ms_p10_p90": [round(pct(bwd_ms, 10), 5), round(pct(bwd_ms, 90), 5)],
        "roofline": {"bound": "mfma", "kernel": "fwd_pp_kernel (fa_fwd_varlen)",
                     "achieved": round(ff / (fa * 1e-3) / 1e12, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(ff / (fa * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(fa, 5)},
        "padded": {"B": B, "N": mx, "ms_per_step": round(pms, 5),
                   "useful_tflops": round(3.5 * ff / (pms * 1e-3) / 1e12, 2),
                   "speedup_of_packed": round(pms / ms, 3)},
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline_varlen(p, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preset", default="c2", help="input preset (default c2: B8 H16 N2048 d128 bf16 causal; "
                                                    "s1..s3: split key/value forward on decoding shapes; "
                                                    "v1, v2: packed variable-length batches)")
    ap.add_argument("--passes", default="fwd,bwd", help="comma list of fwd,bwd")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU baseline budget (0 disables)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 launches) to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters, then exit")
    ap.add_argument("--traffic-json", default=None,
                    help="JSON file with measured HBM bytes per forward launch ({'fetch_bytes': F, "
                         "'write_bytes': W}) to report as roofline.traffic (default: "
                         "profiles/fwd_traffic_<preset>.json when it matches the kernel sources)")
    ap.add_argument("--print-source-hash", action="store_true", help="print the forward sources' sha256 and exit")
    ap.add_argument("--window", default=None,
                    help="LEFT,RIGHT: local attention (query i sees keys i-LEFT .. i+RIGHT, -1 unbounded) through "
                         "fa_fwd_window / fa_bwd_window; FLOP counted over the visible (query, key) pairs")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="repetitions of the cold-MALL variant (a 512 MB buffer is written before each; 0 disables)")
    ap.add_argument("--sparse", default=None,
                    help="band:K or bigbird:K: block-sparse attention (128-position blocks; each query block sees "
                         "itself and the K-1 blocks before it, bigbird also the first block) through "
                         "fa_fwd_blocksparse / fa_bwd_blocksparse; FLOP counted over the visible pairs")
    ap.add_argument("--dropout", default=None, help="P: dropout probability on P through fa_fwd_dropout / "
                                                    "fa_bwd_dropout (FLOP counted as without dropout)")
    ap.add_argument("--no-legs", action="store_true", help="do not add the N=8192 leg to the default run")
    ap.add_argument("--min-warmup-seconds", type=float, default=0.5,
                    help="after the --warmup steps, keep warming up (untimed) until this much time has passed, so "
                         "the timed steps run at the settled shader clock (0: exactly --warmup steps)")
    args = ap.parse_args()

    if args.print_source_hash:
        print(fwd_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no multi-GPU "
              f"path; the per-GPU shard is the single-GPU workload.", file=sys.stderr)
        sys.exit(2)

    import torch

    from io_aware_transformer_amd import FAError, bwd, fwd, inputs

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.arange(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 3}), flush=True)
        return
    if args.preset in inputs.SPLIT_PRESETS:
        bench_split(args, inputs.SPLIT_PRESETS[args.preset])
        return
    if args.preset in inputs.VARLEN_PRESETS:
        bench_varlen(args, inputs.VARLEN_PRESETS[args.preset])
        return
    p = inputs.PRESETS[args.preset]
    passes = [x for x in args.passes.split(",") if x]
    mode = Mode.from_args(args)
    m = measure_fixed(args, p, passes, mode, dev, cold_reps=args.cold_reps)
    line = fixed_line(args, p, m, mode)
    # Long-context leg (the metric spans N = 2K-8K): the default run also
    # times fwd+bwd at B2 H16 N8192 d128 with the same kernels.
    if args.preset == "c2" and mode.kind == "dense" and not args.no_legs:
        m3 = measure_fixed(args, inputs.PRESETS["c3a"], passes, mode, dev, steps=max(3, args.steps // 2),
                           warmup=max(1, args.warmup // 2), cold_reps=0, sample_clock=False)
        line["legs"] = {"c3a": leg_summary(inputs.PRESETS["c3a"], m3)}
    line["clock"] = m["clock"]
    if args.cpu_seconds > 0 and mode.kind == "dense":
        line["cpu_baseline"] = cpu_baseline(p, m["passes"], args.cpu_seconds, m)
    print(json.dumps(line), flush=True)


class Mode:
    """Which entry points a fixed-length run times: dense (fa_fwd / fa_bwd),
    a window, a block map or dropout; and the FLOP it counts."""

    def __init__(self, kind="dense", window=None, sparse=None, dropout=None):
        self.kind, self.window, self.sparse, self.dropout = kind, window, sparse, dropout

    @staticmethod
    def from_args(args):
        if args.window:
            return Mode("window", window=tuple(int(x) for x in args.window.split(",")))
        if args.sparse:
            return Mode("sparse", sparse=args.sparse)
        if args.dropout is not None:
            return Mode("dropout", dropout=float(args.dropout))
        return Mode()

    def block_map(self, p):
        """The block map of --sparse: 'band:K' -- every query block sees itself
        and the K - 1 blocks before it; 'bigbird:K' -- the band plus the first
        key block (a global block)."""
        import numpy as np

        nb = (p.N + 127) // 128
        kind, _, kk = self.sparse.partition(":")
        width = int(kk or 4)
        m = np.zeros((nb, nb), dtype=np.uint8)
        for i in range(nb):
            m[i, max(0, i - width + 1):i + 1] = 1
            if kind == "bigbird":
                m[i, 0] = 1
        return m

    def pairs(self, p):
        """Visible (query, key) pairs of one (b, h) unit, or None for the
        causal / full convention."""
        import numpy as np

        if self.kind == "window":
            return window_pairs(p.N, *self.window)
        if self.kind == "sparse":
            m = self.block_map(p)
            i = np.arange(p.N)
            vis = m[i[:, None] // 128, i[None, :] // 128] != 0
            if p.causal:
                vis &= i[None, :] <= i[:, None]
            return int(vis.sum())
        return None

    def describe(self, p):
        if self.kind == "window":
            return f"window {self.window[0]},{self.window[1]}"
        if self.kind == "sparse":
            return f"block-sparse {self.sparse}{' causal' if p.causal else ''}"
        if self.kind == "dropout":
            return f"dropout p={self.dropout}{' causal' if p.causal else ''}"
        return "causal" if p.causal else "non-causal"


def read_sclk_ghz():
    """Current shader clock of GPU 0 from rocm-smi (a child process), or None."""
    import re
    import subprocess

    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except Exception:
        return None
    for line in r.stdout.splitlines():
        if "sclk" in line:
            mm = re.search(r"\((\d+)\s*Mhz\)", line, re.I)
            if mm:
                return int(mm.group(1)) / 1000.0
    return None


def measure_fixed(args, p, passes, mode, dev, steps=None, warmup=None, cold_reps=0, sample_clock=True):
    """Time `steps` fwd(+bwd) steps of preset p with HIP events on the
    launching stream; returns the per-step times, the outputs and the inputs
    (CPU copies of one sample of units for the CPU leg)."""
    import threading

    import torch

    import io_aware_transformer_amd as fa
    from io_aware_transformer_amd import FAError, inputs

    steps = steps or args.steps
    warmup = warmup if warmup is not None else args.warmup
    q, k, v, do = (t.to(dev) for t in inputs.make_preset(p, with_grad=True))
    extra = {}
    if mode.kind == "window":
        fwd_call = lambda o=None, l=None: fa.fwd_window(q, k, v, mode.window, scale=p.scale, out=o, lse=l)  # noqa
        bwd_call = lambda o, l, ws: fa.bwd_window(q, k, v, o, l, do, mode.window, scale=p.scale, workspace=ws)  # noqa
    elif mode.kind == "sparse":
        bm = torch.from_numpy(mode.block_map(p)).to(dev)
        extra["block_map_density"] = float(bm.float().mean())
        fwd_call = lambda o=None, l=None: fa.fwd_blocksparse(q, k, v, bm, scale=p.scale, causal=p.causal,  # noqa
                                                             out=o, lse=l)
        bwd_call = lambda o, l, ws: fa.bwd_blocksparse(q, k, v, o, l, do, bm, scale=p.scale,  # noqa
                                                       causal=p.causal, workspace=ws)
    elif mode.kind == "dropout":
        fwd_call = lambda o=None, l=None: fa.fwd_dropout(q, k, v, mode.dropout, 1234, 0, scale=p.scale,  # noqa
                                                         causal=p.causal, out=o, lse=l)
        bwd_call = lambda o, l, ws: fa.bwd_dropout(q, k, v, o, l, do, mode.dropout, 1234, 0, scale=p.scale,  # noqa
                                                   causal=p.causal, workspace=ws)
    else:
        fwd_call = lambda o=None, l=None: fa.fwd(q, k, v, scale=p.scale, causal=p.causal, out=o, lse=l)  # noqa
        bwd_call = lambda o, l, ws: fa.bwd(q, k, v, o, l, do, scale=p.scale, causal=p.causal, workspace=ws)  # noqa
    o, lse = fwd_call()
    ws = None
    if "bwd" in passes:
        ws = torch.empty(max(1, fa.bwd_workspace_size(p.B, p.Hq, p.Hkv, p.N, p.d, q.dtype)), device=dev,
                         dtype=torch.uint8)
        try:
            grads = bwd_call(o, lse, ws)
        except FAError as e:
            print(f"backward unavailable ({e}); timing the forward only", file=sys.stderr)
            passes = [x for x in passes if x != "bwd"]
            grads = None
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if "fwd" in passes:
            fwd_call(o, lse)
        if ev is not None:
            ev[1].record(stream)
        if "bwd" in passes:
            bwd_call(o, lse, ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The shader clock settles only after some time under load: the warm-up
    # goes on, untimed, until it has lasted --min-warmup-seconds.
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.min_warmup_seconds:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # Shader clock under this load: rocm-smi (a child process, ~1 s to
    # answer) samples it while the same steps keep running, untimed.
    clock = {"nominal_sclk_ghz": 2.4, "sclk_under_load_ghz": None}
    if sample_clock:
        sampler = threading.Thread(target=lambda: clock.__setitem__("sclk_under_load_ghz", read_sclk_ghz()),
                                   daemon=True)
        sampler.start()
        t0 = time.perf_counter()
        while sampler.is_alive() and time.perf_counter() - t0 < 20:
            for _ in range(5):
                step()
            torch.cuda.synchronize()
        sampler.join(timeout=5)
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]

    cold = None
    if cold_reps > 0:
        # a 512 MB buffer write before every repetition evicts the inputs
        # from the L2 and MALL, so each pass starts from HBM
        buf = torch.empty(COLD_BUFFER_BYTES // 4, device=dev, dtype=torch.float32)
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(cold_reps)]
        for i in range(cold_reps):
            buf.fill_(float(i))
            step(cevs[i])
        torch.cuda.synchronize()
        cold = {"reps": cold_reps, "evict_bytes": COLD_BUFFER_BYTES,
                "fwd_ms_median": round(med([e[0].elapsed_time(e[1]) for e in cevs]), 5) if "fwd" in passes else None,
                "bwd_ms_median": round(med([e[1].elapsed_time(e[2]) for e in cevs]), 5) if "bwd" in passes else None}
        del buf
    # one sample of units for the CPU leg: (b, h) in the order the leg takes them
    units = [(b, h) for b in range(p.B) for h in range(p.Hq)]
    return {"passes": passes, "total_ms": total_ms, "steps": steps, "warmup": warmup, "fwd_ms": fwd_ms,
            "bwd_ms": bwd_ms, "cold": cold, "clock": clock, "extra": extra, "units": units,
            "tensors": {"q": q, "k": k, "v": v, "do": do, "o": o, "lse": lse,
                        "dq": grads[0] if "bwd" in passes else None, "dk": grads[1] if "bwd" in passes else None,
                        "dv": grads[2] if "bwd" in passes else None}}


def med(x):
    x = sorted(x)
    return x[len(x) // 2]


def fixed_flops(p, passes, mode):
    total, fwd_flops = flops(p, passes)
    pairs = mode.pairs(p)
    if pairs is not None:
        fwd_flops = 4.0 * p.B * p.Hq * p.d * pairs
        total = fwd_flops * (("fwd" in passes) + 2.5 * ("bwd" in passes))
    return total, fwd_flops


def leg_summary(p, m):
    passes = m["passes"]
    total_flops, fwd_flops = fixed_flops(p, passes, Mode())
    fa_ = sum(m["fwd_ms"]) / len(m["fwd_ms"])
    ba = sum(m["bwd_ms"]) / len(m["bwd_ms"])
    ms = m["total_ms"] / m["steps"]
    out = {"workload": f"{p.name}: {'+'.join(passes)} {p.dtype} {'causal' if p.causal else 'non-causal'} "
                       f"B={p.B} H_q={p.Hq} H_kv={p.Hkv} N={p.N} d={p.d}",
           "steps": m["steps"], "ms_per_step": round(ms, 5),
           "tflops": round(total_flops / (ms * 1e-3) / 1e12, 2),
           "fwd_tflops": round(fwd_flops / (fa_ * 1e-3) / 1e12, 2),
           "fwd_frac": round(fwd_flops / (fa_ * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "fwd_avg_launch_ms": round(fa_, 5)}
    if "bwd" in passes:
        out["bwd_tflops"] = round(2.5 * fwd_flops / (ba * 1e-3) / 1e12, 2)
        out["bwd_frac"] = round(2.5 * fwd_flops / (ba * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        out["bwd_avg_call_ms"] = round(ba, 5)
    return out


def fixed_line(args, p, m, mode):
    import torch

    passes = m["passes"]
    total_flops, fwd_flops = fixed_flops(p, passes, mode)
    ms_per_step = m["total_ms"] / m["steps"]
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    fwd_ms, bwd_ms = m["fwd_ms"], m["bwd_ms"]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    fwd_tflops = fwd_flops / (fwd_avg * 1e-3) / 1e12 if "fwd" in passes else None
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    bwd_tflops = 2.5 * fwd_flops / (bwd_avg * 1e-3) / 1e12 if "bwd" in passes else None
    dev = torch.device("cuda:0")
    # Roofline of the forward kernel (one launch per forward call, so HIP
    # events around the call time exactly that kernel), bound by bf16 MFMA
    # throughput; the backward (three kernels per call) is given as a whole
    # in roofline_bwd.
    fwd_kernel = "fwd_pp_kernel" if p.dtype == "bf16" else "fwd_f32_kernel"
    mask_id = {"dense": 1 if p.causal else 0, "window": 2, "sparse": 3, "dropout": 1 if p.causal else 0}[mode.kind]
    roofline = {
        "bound": "mfma",
        "kernel": "%s<%d,%d%s>" % (fwd_kernel, p.d, mask_id, ",dropout" if mode.kind == "dropout" else ""),
        "achieved": round(fwd_tflops, 2) if fwd_tflops else None,
        "peak": round(PEAK_BF16_TFLOPS, 1),
        "unit": "TFLOP/s",
        "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4) if fwd_tflops else None,
        "traffic": None,  # filled from --traffic-json / stored counter data when they match the sources
        "avg_launch_ms": round(fwd_avg, 5),
        "alg_hbm_gbs": round(alg_bytes_fwd(p) / (fwd_avg * 1e-3) / 1e9, 1),
    }
    roofline_bwd = None
    if "bwd" in passes:
        roofline_bwd = {"bound": "mfma", "kernels": "bwd_pre + bwd_dkdv + bwd_dq (one backward call)",
                        "achieved": round(bwd_tflops, 2), "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                        "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4), "avg_call_ms": round(bwd_avg, 5),
                        "flop_convention": "2.5 x forward"}
    t = None
    if args.traffic_json:
        with open(args.traffic_json) as f:
            t = json.load(f)
    elif p.dtype == "bf16" and mode.kind == "dense":
        t = stored_traffic(p)
    if t is not None:
        roofline["traffic"] = t["fetch_bytes"] + t["write_bytes"]
        roofline["traffic_detail"] = {"fetch_bytes": t["fetch_bytes"], "write_bytes": t["write_bytes"],
                                      "alg_bytes": alg_bytes_fwd(p), "fetch_factor": t.get("fetch_factor"),
                                      "write_factor": t.get("write_factor"), "source": t.get("source", "")}
    if "fwd" in passes and p.dtype == "bf16":
        # transcendental co-bound: the forward's exponentials at the measured v_exp_f32 rate
        pairs = mode.pairs(p)
        n_exp = exp_count(p) if pairs is None else float(p.B) * p.Hq * pairs
        roofline["exp_bound_ms"] = round(n_exp / EXP_RATE * 1e3, 5)
        roofline["exp_bound_frac_of_launch"] = round(n_exp / EXP_RATE * 1e3 / fwd_avg, 4)
    line = {
        "metric": "attention fwd/bwd TFLOP/s (bf16, causal, d=128, N=2K-8K) + % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": m["warmup"],
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V, dO rounded to bf16, resident in HBM",
        "config": {
            "workload": f"{p.name}: {'+'.join(passes)} {p.dtype} {mode.describe(p)} "
                        f"attention B={p.B} H_q={p.Hq} H_kv={p.Hkv} N={p.N} d={p.d}",
            "window": list(mode.window) if mode.window else None,
            "block_map": mode.sparse, "dropout": mode.dropout,
            "B": p.B, "H_q": p.Hq, "H_kv": p.Hkv, "N": p.N, "d": p.d, "causal": p.causal,
            "passes": passes, "parallelism": "single GPU",
        },
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2) if fwd_tflops else None,
        "fwd_ms_median": round(med(fwd_ms), 5),
        "fwd_ms_p10_p90": [round(pct(fwd_ms, 10), 5), round(pct(fwd_ms, 90), 5)] if "fwd" in passes else None,
        "bwd_tflops": round(bwd_tflops, 2) if bwd_tflops else None,
        "bwd_ms_median": round(med(bwd_ms), 5) if "bwd" in passes else None,
        "bwd_ms_p10_p90": [round(pct(bwd_ms, 10), 5), round(pct(bwd_ms, 90), 5)] if "bwd" in passes else None,
        "cold_mall": m["cold"],
        "peak_inputs": {"cus": torch.cuda.get_device_properties(dev).multi_processor_count, "sclk_ghz": 2.4,
                        "flop_per_clk_per_cu": 4096},
        "roofline": roofline,
        "roofline_bwd": roofline_bwd,
    }
    if m["extra"]:
        line["config"].update(m["extra"])
    return line


if __name__ == "__main__":
    main()
