#!/usr/bin/env python3
"""Throughput of the strict token-logprob path on one MI355X.

A step is one call of the hot path over one batch: rlk_logp_full on 8192 rows
of 152576-wide BF16 logits (151936 real columns, pads -inf), temperature 0.7,
uniform targets - the Qwen3-8B-shaped logits of the RL-Kernel pages (page
"Configurable H100 consistency runs": padded vocabulary 152576, float32
temperature scaling of BF16 logits; page "H100 rollout context parallelism":
8,192 active tokens per validation). Inputs are seeded synthetic normals
(sigma 2.5, one +8 spike per row) generated on the host and uploaded before
the timed region; two copies alternate so that no step reads logits the
previous step left in the 256 MB last-level cache.

Prints one JSON line. `value` is tokens/s over the K timed steps (wall clock
between two device synchronisations); `roofline.achieved` is the algorithmic
bytes of one launch divided by the average launch time measured with HIP
events on the launch stream over the same region. `cpu_baseline` times the
CPU oracle (float64 numpy) on bounded samples of the full-vocab, top-p 0.95 and
per-request workloads, on every usable host core and on one core.
`secondary` reports rlk_logp_nucleus on the top-p 0.95 workload, the
backward (rlk_logp_backward) on it, rlk_logp_nucleus on the per-request
workload (64 requests x 128 rows) and on the invariance-stress workload (64
ragged sequences evaluated as batches of 1, 7 and 64 sequences, with the
byte mismatches between those passes), the vocabulary-parallel form, the
gradient L2 norm and the fused LM-head linear + logprob, for information.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "logp tokens/s and logits HBM GB/s (% of peak), 8192×152576 BF16, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_logp_full_8192x152576.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "invariant_token_log_fp32_amd", "csrc", "rlk_logp.hip"),
    os.path.join(ROOT, "invariant_token_log_fp32_amd", "csrc", "logp_device.hpp"),
    os.path.join(ROOT, "invariant_token_log_fp32_amd", "csrc", "support.hpp"),
    os.path.join(ROOT, "invariant_token_log_fp32_amd", "csrc", "backward.hpp"),
]  # sources of the kernels whose counters the traffic records hold


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def bytes_full(n_rows: int, vocab_real: int) -> int:
    # real logits + int64 target + float32 temperature + float32 output, per row
    return n_rows * (vocab_real * 2 + 8 + 4 + 4)


def bytes_nucleus(n_rows: int, vocab_real: int) -> int:
    # real logits (read once) + target + temperature + top-p + top-k + two outputs
    return n_rows * (vocab_real * 2 + 8 + 4 + 4 + 4 + 8)


def bytes_backward(n_rows: int, vocab_real: int, vocab_padded: int, policy: bool) -> int:
    # real logits read once + gradient row written once (pads included) + per-row
    # temperature, target, ref, lse, upstream gradient (+ policy, support record, upstream gradient)
    return n_rows * (vocab_real * 2 + vocab_padded * 2 + 4 + 8 + 4 + 4 + 4 + (24 if policy else 0))


# Rows the forked oracle workers read: (logits, vocab_real, T, top_p, top_k, targets, kind).
_CPU_ROWS = None


def _oracle_chunk(lo, hi):
    """The oracle over rows [lo, hi) of _CPU_ROWS (in a forked worker or in-process)."""
    from oracle import logp as O
    logits, vr, tt, pp, kk, tg, kind = _CPU_ROWS
    if kind == "ref":
        O.ref_logp(logits[lo:hi], vr, tt[lo:hi], tg[lo:hi])
    else:
        O.nucleus_logp(logits[lo:hi], vr, tt[lo:hi], pp[lo:hi], kk[lo:hi], tg[lo:hi])
    return hi - lo


def _noop(_):
    return 0


def _time_oracle(kind, logits, w, rows, targets, workers, chunk=64):
    """Wall time of the oracle over the sample (generation excluded), on `workers`
    forked processes (rows in 64-row chunks) or in this process when workers == 1."""
    import concurrent.futures as cf
    import multiprocessing as mp
    global _CPU_ROWS
    _CPU_ROWS = (logits, w.vocab_real, w.temperature[rows], w.top_p[rows], w.top_k[rows], targets, kind)
    n = len(rows)
    if workers == 1:
        t0 = time.perf_counter()
        _oracle_chunk(0, n)
        return time.perf_counter() - t0
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork")) as ex:
        list(ex.map(_noop, range(workers)))          # workers started before the clock
        t0 = time.perf_counter()
        done = sum(ex.map(_oracle_chunk, range(0, n, chunk), [min(i + chunk, n) for i in range(0, n, chunk)]))
        dt = time.perf_counter() - t0
    assert done == n
    return dt


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(scale: float = 1.0):
    """The CPU oracle (float64 numpy, as it stands) timed on bounded samples of the
    full-vocabulary, top-p 0.95 and per-request workloads, on every usable host
    core (a forked process per core, at most 16) and on one core. Runs before the
    GPU is touched, so the forked workers never inherit a device context."""
    import datagen
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else
                         (os.cpu_count() or 1)))
    legs = [
        ("full-vocab reference logprob (8192 x 152576 workload, T 0.7)", "ref", datagen.full(), 256, 512),
        ("top-p 0.95 policy + reference logprob (same logits)", "nucleus", datagen.nucleus(), 64, 64),
        ("per-request T/top-p/top-k policy + reference logprob (64 x 128 rows)", "nucleus", datagen.per_request(),
         64, 64),
    ]
    out = []
    for name, kind, w, rows_per_core_multi, rows_single in legs:
        n_multi = max(workers, int(rows_per_core_multi * workers * scale))
        n_single = max(1, min(n_multi, int(rows_single * scale)))
        # a spread of rows (every request of the per-request workload is represented)
        rows = np.linspace(0, w.n_rows - 1, n_multi).astype(np.int64)
        logits, targets = w.generate(rows=rows.tolist())
        one = np.linspace(0, n_multi - 1, n_single).astype(np.int64)   # the one-core sample, spread alike
        for cores, sel in ((workers, np.arange(n_multi)), (1, one)):
            dt = _time_oracle(kind, logits[sel], w, rows[sel], targets[sel], cores)
            out.append({"workload": name, "cores": cores, "rows": int(len(sel)), "seconds": dt,
                        "tokens_per_s": len(sel) / dt})
        del logits
    head = out[0]
    return {
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "cores": head["cores"],
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{head['rows']} rows spread over the 8192-row full-vocab workload (whole 151936-column rows), "
                   f"float64 numpy oracle, {head['cores']} forked processes, {head['seconds']:.1f} s; "
                   "the other legs are listed under 'workloads'"),
        "workloads": out,
    }


def time_calls(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / steps


def time_blocks(fn, steps, warmup, blocks):
    """Secondary legs: `warmup` calls, then `blocks` blocks of `steps` calls each,
    timed with HIP events on the launch stream. Returns the median block's time
    per call (ms) and every block's. The chip's clock moves for tens of
    milliseconds after a change of load (the shader clock measured 2.14 ->
    1.65 -> 1.9 GHz over the first ~30 launches of the full-vocabulary step), so
    the median of several blocks, not one short block, describes a kernel."""
    fn_i = iter(range(1 << 30))
    _, first = time_calls(lambda i: fn(next(fn_i)), steps, warmup)
    per = [first]
    for _ in range(blocks - 1):
        _, ms = time_calls(lambda i: fn(next(fn_i)), steps, 0)
        per.append(ms)
    return float(np.median(per)), per


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--groups", type=int, default=1, help="physical blocks per row (1, 2, 4 or 8)")
    ap.add_argument("--cpu-scale", type=float, default=1.0, help="scales the oracle samples of cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one device copy of the logits (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs the hot path on a single MI355X "
              "(rows are independent, so N GPUs would each run this same benchmark on their own rows); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import datagen
    import invariant_token_log_fp32_amd as rlk

    if not os.path.exists(rlk.LIB_PATH):
        rlk.load_library()  # raises: the HIP library is missing
    # the oracle's forked workers start before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_scale)
    rlk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = datagen.full()
    logits, targets = w.generate()
    lg_a = torch.from_numpy(logits.view(np.int16)).to(dev)
    lg_b = lg_a.clone()
    bufs = (lg_a, lg_b)
    temp = torch.full((w.n_rows,), 0.7, dtype=torch.float32, device=dev)
    tg = torch.from_numpy(targets).to(dev)
    out = torch.empty(w.n_rows, dtype=torch.float32, device=dev)
    ws = None
    need = rlk.workspace_bytes(w.n_rows, w.vocab_padded, w.vocab_real, groups=args.groups)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        rlk.logp_full(bufs[i % 2], temp, tg, vocab_real=w.vocab_real, groups=args.groups, out=out, workspace=ws)

    wall, ms_event = time_calls(step, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = w.n_rows * args.steps / wall
    alg = bytes_full(w.n_rows, w.vocab_real)
    achieved = alg / (ms_event * 1e-3) / 1e9

    if args.calibrate_copy:
        lg_b.copy_(lg_a)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "full-vocab logp: 8192 rows x 152576 BF16 (151936 real), T 0.7, uniform targets",
            "n_rows": w.n_rows, "vocab_padded": w.vocab_padded, "vocab_real": w.vocab_real,
            "temperature": 0.7, "groups": args.groups, "entry_point": "rlk_logp_full",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": stored_traffic(),
            "algorithmic_bytes_per_launch": alg,
            "avg_launch_ms": ms_event,
        },
    }

    if not args.no_secondary:
        sec = []
        pk = torch.full((w.n_rows,), -1, dtype=torch.int32, device=dev)
        pp = torch.full((w.n_rows,), 0.95, dtype=torch.float32, device=dev)
        pol = torch.empty(w.n_rows, dtype=torch.float32, device=dev)
        ref = torch.empty(w.n_rows, dtype=torch.float32, device=dev)
        need_n = rlk.workspace_bytes(w.n_rows, w.vocab_padded, w.vocab_real, groups=args.groups, nucleus=True)
        wsn = torch.empty(need_n, dtype=torch.uint8, device=dev) if need_n else None

        def nstep(i, lgs=bufs, t=temp, p=pp, k=pk, target=tg):
            rlk.logp_nucleus(lgs[i % 2], t, p, k, target, vocab_real=w.vocab_real, groups=args.groups,
                             policy_out=pol, ref_out=ref, workspace=wsn)

        ms_n, blk_n = time_blocks(nstep, 20, 10, 5)
        ab = bytes_nucleus(w.n_rows, w.vocab_real)
        sec.append({"workload": "nucleus: same logits, top-p 0.95, top-k off, T 0.7", "entry_point":
                    "rlk_logp_nucleus", "ms_per_step": ms_n, "ms_blocks": blk_n, "tokens_per_s": w.n_rows / (ms_n * 1e-3),
                    "achieved_GBs": ab / (ms_n * 1e-3) / 1e9, "frac": ab / (ms_n * 1e-3) / 1e9 / HBM_PEAK_GBS})
        # backward of both terms (and of the reference term alone) from the nucleus forward's statistics
        lse = torch.empty(w.n_rows, dtype=torch.float32, device=dev)
        state = torch.empty((w.n_rows, 4), dtype=torch.int32, device=dev)
        rlk.logp_nucleus(lg_a, temp, pp, pk, tg, vocab_real=w.vocab_real, return_state=True, policy_out=pol,
                         ref_out=ref, lse_out=lse, state_out=state, workspace=wsn)
        gen = torch.Generator(device=dev).manual_seed(7)
        g_r = torch.randn(w.n_rows, generator=gen, device=dev)
        g_p = torch.randn(w.n_rows, generator=gen, device=dev)
        grad = torch.empty((w.n_rows, w.vocab_padded), dtype=torch.bfloat16, device=dev)
        for policy in (True, False):
            kw = dict(policy_logp=pol, support_state=state, grad_policy=g_p) if policy else {}
            ms_b, blk_b = time_blocks(lambda i: rlk.logp_backward(
                bufs[0], temp, tg, vocab_real=w.vocab_real, ref_logp=ref, lse=lse, grad_ref=g_r, out=grad, **kw),
                20, 5, 3)
            bb = bytes_backward(w.n_rows, w.vocab_real, w.vocab_padded, policy)
            sec.append({"workload": "backward: same logits, " + ("reference + top-p 0.95 policy terms" if policy
                        else "reference term only") + ", BF16 gradient 8192 x 152576",
                        "entry_point": "rlk_logp_backward", "ms_per_step": ms_b, "ms_blocks": blk_b,
                        "tokens_per_s": w.n_rows / (ms_b * 1e-3), "algorithmic_bytes_per_launch": bb,
                        "achieved_GBs": bb / (ms_b * 1e-3) / 1e9, "frac": bb / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del grad
        wr = datagen.per_request()
        lg_r, tg_r = wr.generate()
        lg_r = (torch.from_numpy(lg_r.view(np.int16)).to(dev),) * 2
        prm = dict(t=torch.from_numpy(wr.temperature).to(dev), p=torch.from_numpy(wr.top_p).to(dev),
                   k=torch.from_numpy(wr.top_k).to(dev), target=torch.from_numpy(tg_r).to(dev))
        ms_r, blk_r = time_blocks(lambda i: nstep(i, lgs=lg_r, **prm), 20, 10, 5)
        sec.append({"workload": "per-request: 64 requests x 128 rows, T {0.7,1.0,1.3}, top-p {0.95,0.99}, "
                    "top-k {-1,128}", "entry_point": "rlk_logp_nucleus", "ms_per_step": ms_r, "ms_blocks": blk_r,
                    "tokens_per_s": wr.n_rows / (ms_r * 1e-3), "achieved_GBs": ab / (ms_r * 1e-3) / 1e9,
                    "frac": ab / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del lg_r
        # invariance stress: 64 ragged sequences (lengths 1..1024), top-p 0.95, evaluated as batches of
        # 1, 7 and 64 sequences; reports each pass's time and the byte mismatches against one call
        wst = datagen.stress()
        lg_s = torch.empty((wst.n_rows, wst.row_stride), dtype=torch.int16, device=dev)
        tg_s = np.empty(wst.n_rows, dtype=np.int64)
        for s0 in range(0, wst.n_rows, 4096):
            blk, tblk = wst.generate(rows=range(s0, min(s0 + 4096, wst.n_rows)))
            tg_s[s0:s0 + len(blk)] = tblk
            lg_s[s0:s0 + len(blk)].copy_(torch.from_numpy(blk.view(np.int16)))
            del blk
        prm_s = dict(t=torch.from_numpy(wst.temperature).to(dev), p=torch.from_numpy(wst.top_p).to(dev),
                     k=torch.from_numpy(wst.top_k).to(dev), target=torch.from_numpy(tg_s).to(dev))
        starts = np.concatenate([[0], np.cumsum(wst.seq_lengths)]).astype(np.int64)
        nseq = len(wst.seq_lengths)
        pol_s = torch.empty(wst.n_rows, dtype=torch.float32, device=dev)
        ref_s = torch.empty(wst.n_rows, dtype=torch.float32, device=dev)
        wss = rlk.workspace_bytes(wst.n_rows, wst.vocab_padded, wst.vocab_real, groups=args.groups, nucleus=True)
        wss = torch.empty(wss, dtype=torch.uint8, device=dev) if wss else None

        def spass(bs):
            for b in range(0, nseq, bs):
                lo, hi = int(starts[b]), int(starts[min(b + bs, nseq)])
                rlk.logp_nucleus(lg_s[lo:hi], prm_s["t"][lo:hi], prm_s["p"][lo:hi], prm_s["k"][lo:hi],
                                 prm_s["target"][lo:hi], vocab_real=wst.vocab_real, vocab_padded=wst.vocab_padded,
                                 groups=args.groups, policy_out=pol_s[lo:hi], ref_out=ref_s[lo:hi], workspace=wss)

        spass(nseq)
        torch.cuda.synchronize()
        base_s = (pol_s.clone(), ref_s.clone())
        modes = {}
        mism = 0
        for bs in (1, 7, nseq):
            # 2 warm-up passes, then the median of 3 blocks of 4 passes (as the other secondary legs)
            ms_s, blk_s = time_blocks(lambda i, bs=bs: spass(bs), 4, 2, 3)
            mism += int((pol_s.view(torch.int32) != base_s[0].view(torch.int32)).sum().item())
            mism += int((ref_s.view(torch.int32) != base_s[1].view(torch.int32)).sum().item())
            modes[f"batches of {bs} sequences"] = {"calls": (nseq + bs - 1) // bs, "ms_per_pass": ms_s,
                                                   "ms_blocks": blk_s, "tokens_per_s": wst.n_rows / (ms_s * 1e-3)}
        ab_s = bytes_nucleus(wst.n_rows, wst.vocab_real)
        ms_one = modes[f"batches of {nseq} sequences"]["ms_per_pass"]
        sec.append({"workload": f"invariance stress: {nseq} ragged sequences ({wst.n_rows} rows) x 152576, "
                    "T 0.7, top-p 0.95, batches of 1, 7 and 64 sequences", "entry_point": "rlk_logp_nucleus",
                    "ms_per_step": ms_one, "tokens_per_s": wst.n_rows / (ms_one * 1e-3),
                    "achieved_GBs": ab_s / (ms_one * 1e-3) / 1e9, "frac": ab_s / (ms_one * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "modes": modes, "byte_mismatches_vs_one_call": mism})
        del lg_s, base_s
        # vocabulary-parallel form: 8 ranks, each with its own 8192 x 19072 slice
        G = 8
        cols = w.vocab_padded // G
        slices = [lg_a[:, r * cols:(r + 1) * cols].contiguous() for r in range(G)]
        summ = torch.empty(rlk.summary_bytes(w.n_rows, w.vocab_padded, w.vocab_real, groups=G) * G,
                           dtype=torch.uint8, device=dev)
        per = summ.numel() // G
        _, ms_ranks = time_calls(lambda i: [rlk.logp_shard_summaries(
            slices[r], temp, tg, rank=r, groups=G, vocab_real=w.vocab_real, vocab_padded=w.vocab_padded,
            out=summ[r * per:(r + 1) * per]) for r in range(G)], 10, 2)
        _, ms_merge = time_calls(lambda i: rlk.logp_merge(
            summ, temp, tg, n_rows=w.n_rows, groups=G, vocab_real=w.vocab_real, vocab_padded=w.vocab_padded,
            out=out), 20, 2)
        rank_bytes = alg / G
        sec.append({"workload": "vocabulary-parallel: 8 ranks x (8192 x 19072 slice) shard summaries, then merge",
                    "entry_point": "rlk_logp_shard_summaries + rlk_logp_merge",
                    "ms_per_rank": ms_ranks / G, "ms_merge": ms_merge,
                    "rank_achieved_GBs": rank_bytes / (ms_ranks / G * 1e-3) / 1e9,
                    "frac": rank_bytes / (ms_ranks / G * 1e-3) / 1e9 / HBM_PEAK_GBS})
        # order-independent gradient L2 norm: the pages' 10M-element microbenchmark, and 2^28 values
        xn = torch.from_numpy(datagen.grad_values(7, datagen.NORM_MICROBENCH_N)).to(dev)
        nb = torch.zeros(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=dev)  # rlk_l2norm leaves it zeroed
        so = torch.empty(1, dtype=torch.float64, device=dev)
        no = torch.empty(1, dtype=torch.float32, device=dev)
        _, ms_norm = time_calls(lambda i: rlk.l2norm(xn, workspace=nb, sumsq_out=so, norm_out=no), 200, 20)
        acc_bins = torch.zeros(rlk.NORM_BIN_WORDS, dtype=torch.int64, device=dev)
        _, ms_acc = time_calls(lambda i: rlk.l2norm_accumulate(xn, acc_bins), 200, 20)
        nbytes = xn.numel() * 4
        sec.append({"workload": "l2norm: 10M BF16-derived fp32 gradient values (accumulate + finalize launches)",
                    "entry_point": "rlk_l2norm", "ms_per_step": ms_norm, "accumulate_ms": ms_acc,
                    "achieved_GBs": nbytes / (ms_norm * 1e-3) / 1e9,
                    "frac": nbytes / (ms_norm * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del xn
        xl = (torch.randn(1 << 28, generator=torch.Generator(device=dev).manual_seed(3), device=dev)
              .to(torch.bfloat16).to(torch.float32))
        _, ms_big = time_calls(lambda i: rlk.l2norm(xl, workspace=nb, sumsq_out=so, norm_out=no), 50, 5)
        nbytes = xl.numel() * 4
        sec.append({"workload": "l2norm: 2^28 BF16-derived fp32 values (1 GiB)", "entry_point": "rlk_l2norm",
                    "ms_per_step": ms_big, "achieved_GBs": nbytes / (ms_big * 1e-3) / 1e9,
                    "frac": nbytes / (ms_big * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del xl
        # fused LM-head linear + logprob at the Qwen3-8B shape (8192 x 4096 hidden, 151936 x 4096 projection)
        d_model = datagen.QWEN3_D_MODEL
        hb, wb = datagen.linear_inputs(41, w.n_rows, d_model, w.vocab_real)
        hid = torch.from_numpy(hb.view(np.int16)).to(dev)
        wt = torch.from_numpy(wb.view(np.int16)).to(dev)
        del hb, wb
        lws = torch.empty(rlk.linear_logp_workspace_bytes(w.n_rows, w.vocab_padded, w.vocab_real),
                          dtype=torch.uint8, device=dev)
        _, ms_ll = time_calls(lambda i: rlk.linear_logp(hid, wt, temp, tg, vocab_padded=w.vocab_padded, out=out,
                                                        workspace=lws), 5, 2)
        lgt = torch.empty((w.n_rows, w.vocab_padded), dtype=torch.bfloat16, device=dev)
        _, ms_lin = time_calls(lambda i: rlk.linear(hid, wt, vocab_padded=w.vocab_padded, out=lgt), 5, 2)
        wt16 = wt.view(torch.bfloat16).t()
        _, ms_lib = time_calls(lambda i: torch.matmul(hid.view(torch.bfloat16), wt16), 5, 2)
        # batch dependence of a row's logits: row block 0..6 computed alone vs inside the 8192-row batch
        lib_full = torch.matmul(hid.view(torch.bfloat16), wt16)
        lib_part = torch.matmul(hid[:7].contiguous().view(torch.bfloat16), wt16)
        lib_var = float((lib_part.view(torch.int16) != lib_full[:7].view(torch.int16)).float().mean())
        del lib_full, lib_part
        own_part = rlk.linear(hid[:7].contiguous(), wt, vocab_padded=w.vocab_padded)
        own_var = float((own_part.view(torch.int16) != lgt[:7].view(torch.int16)).float().mean())
        flops = 2.0 * w.n_rows * w.vocab_real * d_model
        sec.append({"workload": "linear-logp: 8192 x 4096 BF16 hidden states, 151936 x 4096 BF16 projection, T 0.7",
                    "entry_point": "rlk_linear_logp", "ms_per_step": ms_ll, "tokens_per_s": w.n_rows / (ms_ll * 1e-3),
                    "roofline": {"bound": "mfma", "achieved": flops / (ms_ll * 1e-3) / 1e12,
                                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": flops / (ms_ll * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
                    "unfused_ms": {"rlk_linear": ms_lin, "rlk_linear + rlk_logp_full": ms_lin + ms_event,
                                   "hipBLASLt matmul (shape-dependent reduction order)": ms_lib,
                                   "hipBLASLt matmul + rlk_logp_full": ms_lib + ms_event},
                    "logit_bits_changed_by_batch": {"rlk_linear": own_var, "hipBLASLt matmul": lib_var,
                                                    "rows": "0..6 alone vs in the 8192-row batch"}})
        del hid, wt, lgt, lws
        result["secondary"] = sec

    if cpu is not None:
        result["cpu_baseline"] = cpu

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
