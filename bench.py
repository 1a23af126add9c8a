#!/usr/bin/env python3
"""Benchmark of LoopVQ quantized-KV decode attention on one MI355X.

Workload: 0.5 bit per element (T=4 loop steps, T_c=2, G=16, K=256 bf16
codebooks), batch 64, 16 heads, 6144-token context with 8 sinks and a
64-token recent window in bf16 and 759 index pages per request, seeded
synthetic data (the LoopVQ page's "method steps" step 5 quotes its
two-requests-per-block saving at this batch and context).

One step is one decode step of a model with `--layers` attention layers that
each own an independent copy of that cache: for each of the T loop steps,
every layer runs lvq_decode_attn: the index-page partial kernel
(index_mfma_kernel), then the bf16-window kernel that merges the partials
through logsumexp; `--num-splits N` fixes the split count (0: the library's
choice).  Rotating over the
copies (3.4 GB) keeps the 256 MB Infinity Cache from serving repeated reads,
as layers would in a real model.

Printed: one JSON line with the whole-call rate (algorithmic GB/s, fraction
of the 8 TB/s HBM peak, token-heads/s), the roofline entry of the dominant
kernel (the index-page partial timed alone; HIP events on the stream it runs on; its HBM traffic from the
committed counter runs when they match the kernel source), and the fp64
oracle timed on a bounded sample on the host.

Counter runs (rocprofv3 --pmc, one counter per run): `--mode index-only`
launches only the dominant kernel, `--mode copy` a plain 256 MiB device copy
for calibration, and `--pmc-summary` turns the four output directories into
profiles/<kernel>_b64_6k_traffic.json.
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
WORKLOAD = "loopvq-b64-6k"
METRIC = "quantized-KV decode attention HBM GB/s (% of peak) + token-heads/s, B=64 6K"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _positions(g, lengths):
    """(largest index-token count, set of window positions) over the requests."""
    from decode_attention_loopvq_amd.layout import n_index_pages
    max_q, win = 0, set()
    for L in lengths:
        nq = g.page * n_index_pages(L, g)
        max_q = max(max_q, nq)
        win.update(range(min(L, g.sink)))
        win.update(range(g.sink + nq, L))
    return max_q, win


def call_bytes(g, lengths, cb_bytes):
    """Algorithmic bytes of one lvq_decode_attn call, split by stream: every
    input read once, the output written once."""
    from decode_attention_loopvq_amd.layout import index_groups, n_index_pages
    NG = index_groups(g)
    idx = win = pt = 0
    for L in lengths:
        n = n_index_pages(L, g)
        nq = g.page * n
        idx += g.H * nq * 2 * NG                      # K and V index rows
        win += g.H * (L - nq) * 2 * g.D * 2           # bf16 K and V of sinks + recent tokens
        pt += 4 * n                                   # page ids
    cb = g.H * 2 * g.K * g.D * cb_bytes               # the step's K and V slices
    max_q, wpos = _positions(g, lengths)
    rope = max_q * g.D * 2 + len(wpos) * g.D * 4      # fp16 cos/sin of index positions, fp32 of window ones
    qo = len(lengths) * g.H * g.D * (2 + 4)           # bf16 q in, fp32 out
    return {"index": idx, "window": win, "page_table": pt, "codebook": cb, "rope": rope, "q_out": qo}


def quant_kernel_bytes(g, lengths, cb_bytes, splits):
    """Algorithmic bytes of one index-page partial launch (index_mfma_kernel):
    index rows, page ids, codebook slices, fp16 cos/sin of the paged
    positions, q, and the partials written."""
    from decode_attention_loopvq_amd.layout import index_groups, n_index_pages
    NG = index_groups(g)
    idx = pt = 0
    for L in lengths:
        n = n_index_pages(L, g)
        idx += g.H * g.page * n * 2 * NG
        pt += 4 * n
    cb = g.H * 2 * g.K * g.D * cb_bytes
    max_q, _ = _positions(g, lengths)
    rope = max_q * g.D * 2
    q = len(lengths) * g.H * g.D * 2
    parts = len(lengths) * g.H * splits * (g.D + 1) * 4
    return idx + pt + cb + rope + q + parts


def _cpu_rows_worker(path, seconds):
    """One host core: the fp64 oracle's decode step over the stored rows, repeated for `seconds`."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import loopvq as lv

    with np.load(path) as z:
        meta = z["meta"]
        D, T, Tc, G, K, sink, window, page, n = (int(x) for x in meta[:9])
        sm_scale, rope_base = float(meta[9]), float(meta[10])
        rows = [tuple(z[f"{k}{i}"] for k in ("L", "q", "rk", "rv", "ik", "iv", "ek", "ev")) for i in range(n)]
    geo = lv.Geometry(D=D, T=T, Tc=Tc, G=G, K=K, sink=sink, window=window, page=page)
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for (L, q, raw_k, raw_v, idx_k, idx_v, E_k, E_v) in rows:
                for t in range(T):
                    lv.decode_step(q[t], t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, int(L), sm_scale,
                                   rope_base)
                    done += 1
        el = time.perf_counter() - t0
    return done, el


def host_cores():
    """Cores this process may run on (at most 16, the host share of one GPU) and the CPU model."""
    cores = min(len(os.sched_getaffinity(0)), 16)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(prob, rows, seconds, runs=3):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: every allowed host core runs
    the decode step over the sample rows for `seconds`; the rate of each of `runs` runs is the rows done by
    all cores over the run's wall time, and the median is reported."""
    import multiprocessing
    import statistics
    import tempfile
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np

    from oracle import loopvq as lv
    from tests import harness

    cfg = prob.cfg
    geo = lv.Geometry(D=cfg.D, T=cfg.T, Tc=cfg.Tc, G=cfg.G, K=cfg.K, sink=cfg.sink, window=cfg.window,
                      page=cfg.page)
    arrays = {"meta": np.array([cfg.D, cfg.T, cfg.Tc, cfg.G, cfg.K, cfg.sink, cfg.window, cfg.page, len(rows),
                                prob.sm_scale, cfg.rope_base], dtype=np.float64)}
    for i, (b, h) in enumerate(rows):
        L = prob.lengths[b]
        E_k, E_v = harness.host_codebooks(prob, h, "k"), harness.host_codebooks(prob, h, "v")
        raw_k, raw_v = prob.raw[("k", b, h)], prob.raw[("v", b, h)]
        arrays.update({f"L{i}": np.array(L), f"q{i}": prob.q[:, b, h].float().cpu().numpy().astype(np.float64),
                       f"rk{i}": raw_k, f"rv{i}": raw_v, f"ik{i}": lv.encode_request(raw_k, E_k, geo, L),
                       f"iv{i}": lv.encode_request(raw_v, E_v, geo, L), f"ek{i}": E_k, f"ev{i}": E_v})
    cores, model = host_cores()
    rates = []
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "rows.npz")
        np.savez(path, **arrays)
        # spawned workers: fresh interpreters that never touch the GPU
        with ProcessPoolExecutor(max_workers=cores, mp_context=multiprocessing.get_context("spawn")) as pool:
            list(pool.map(_cpu_rows_worker, [path] * cores, [0.0] * cores))   # start the workers, untimed
            for _ in range(runs):
                t0 = time.perf_counter()
                res = list(pool.map(_cpu_rows_worker, [path] * cores, [seconds] * cores))
                wall = time.perf_counter() - t0
                rates.append(sum(r[0] for r in res) / max(wall, max(r[1] for r in res)))
    return statistics.median(rates), rates, cores, model


KERNELS = {"index_mfma_kernel": "index_mfma_kernel<false> (index-page partial, c = 8)"}
KERNEL_SRC = os.path.join(ROOT, "decode_attention_loopvq_amd", "csrc", "attn.hip")
COPY_BYTES = 256 << 20


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_file(kernel):
    return os.path.join(ROOT, "profiles", kernel.replace("_kernel", "") + "_b64_6k_traffic.json")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs, or None when the kernel source has
    changed since they were taken."""
    try:
        with open(traffic_file(kernel)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t["bytes_per_launch"] if t.get("attn_hip_sha256_16") == kernel_source_hash() else None


def _pmc_values(d, counter, name_re):
    """Per-dispatch values of `counter` for kernels whose name matches name_re, from a rocprofv3 csv dir."""
    import csv
    import glob
    import re
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and re.search(name_re, r["Kernel_Name"]):
                vals.append(float(r["Counter_Value"]))
    return vals


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Traffic of the dominant kernel (whichever of KERNELS the counter runs hold) from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for a plain copy of
    COPY_BYTES; writes its traffic file."""
    import statistics
    kernel = next((k for k in KERNELS if _pmc_values(fetch_dir, "FETCH_SIZE", k)), None)
    if kernel is None:
        raise SystemExit("no dispatch of a known kernel in the counter runs")
    kf = _pmc_values(fetch_dir, "FETCH_SIZE", kernel)
    kw = _pmc_values(write_dir, "WRITE_SIZE", kernel)
    cf = [v for v in _pmc_values(copy_fetch_dir, "FETCH_SIZE", "copy|elementwise") if v * 1024 > COPY_BYTES / 8]
    cw = [v for v in _pmc_values(copy_write_dir, "WRITE_SIZE", "copy|elementwise") if v * 1024 > COPY_BYTES / 8]
    if not (kf and kw and cf and cw):
        raise SystemExit(f"missing counter values: kernel fetch {len(kf)} write {len(kw)}, copy {len(cf)} {len(cw)}")
    sf = COPY_BYTES / (statistics.median(cf) * 1024)
    sw = COPY_BYTES / (statistics.median(cw) * 1024)
    fetch = statistics.median(kf) * 1024 * sf
    write = statistics.median(kw) * 1024 * sw
    t = {"kernel": KERNELS[kernel], "workload": WORKLOAD, "attn_hip_sha256_16": kernel_source_hash(),
         "fetch_bytes": round(fetch), "write_bytes": round(write), "bytes_per_launch": round(fetch + write),
         "copy_scale_fetch": round(sf, 4), "copy_scale_write": round(sw, 4), "dispatches": [len(kf), len(kw)]}
    with open(traffic_file(kernel), "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(json.dumps(t))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=6, help="independent cache copies rotated through")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="0: the library's choice; N >= 1: that many splits")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="seconds per CPU-baseline run (3 runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("bench", "index-only", "copy"), default="bench",
                    help="index-only: launch only the dominant kernel (for counter runs); "
                         "copy: a plain device copy of 256 MiB (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output dirs: write the measured traffic of the index-page kernel")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the path "
              "shards by (request, head) with no exchange, so N GPUs run N independent copies of this "
              "benchmark.", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_loopvq_amd as lvq
    from decode_attention_loopvq_amd._lib import lib
    from synth.configs import loopvq_config
    from tests import harness

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.mode == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {COPY_BYTES} bytes x {args.steps}", flush=True)
        return
    cfg = loopvq_config(WORKLOAD)
    sample_rows = [(0, 0), (37, 9)]
    want_cpu = args.mode == "bench" and not args.no_cpu_baseline
    log(f"[bench] building {WORKLOAD}: B={cfg.B} H={cfg.H} L={cfg.L} T={cfg.T} Tc={cfg.Tc} G={cfg.G}")
    t0 = time.perf_counter()
    prob = harness.build_loopvq(cfg, keep=sample_rows if want_cpu else [])
    g, cache = prob.g, prob.cache
    log(f"[bench] built in {time.perf_counter() - t0:.1f}s; copying to {args.layers} layers")
    pools = [cache.pool] + [cache.pool.clone() for _ in range(args.layers - 1)]
    wks = [cache.win_k] + [cache.win_k.clone() for _ in range(args.layers - 1)]
    wvs = [cache.win_v] + [cache.win_v.clone() for _ in range(args.layers - 1)]
    # every layer has its own codebook slices and query rows (the RoPE table is shared, as in a model)
    slices = [prob.slices] + [prob.slices.clone() for _ in range(args.layers - 1)]
    B = cfg.B
    plan = args.num_splits or lvq.lvq_decode_attn_splits(g, B, cache.max_len)
    ws_bytes = lvq.lvq_decode_attn_workspace(g, B, cache.max_len, args.num_splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, g.H, g.D), dtype=torch.float32, device="cuda") for _ in range(args.layers)]
    qs = [[prob.q[t].contiguous() if l == 0 else prob.q[t].contiguous().roll(1 + l, dims=0)
           for t in range(cfg.T)] for l in range(args.layers)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    gref = C.byref(g)
    rope_len = prob.rope_cos.shape[0]

    def full_args(t, l):
        return (gref, t, qs[l][t].data_ptr(), pools[l].data_ptr(), cache.page_table.data_ptr(),
                int(cache.page_table.shape[1]), cache.seq_len.data_ptr(), cache.max_len, None, None, wks[l].data_ptr(),
                wvs[l].data_ptr(), slices[l].data_ptr(), prob.rope_cos.data_ptr(), prob.rope_sin.data_ptr(),
                prob.rope16.data_ptr(), rope_len, C.c_float(prob.sm_scale), outs[l].data_ptr(), None,
                ws.data_ptr(), ws_bytes, args.num_splits, B, sh)

    calls = [full_args(t, l) for t in range(cfg.T) for l in range(args.layers)]

    def one_step():
        for a in calls:
            st = lib.lvq_decode_attn(*a)
            if st != 0:
                raise RuntimeError(lib.lvq_last_error().decode())

    # The dominant kernel alone: the index-page partial (one index_mfma_kernel launch) into its own buffers.
    S = plan
    part_o = torch.empty((B * g.H, S, g.D), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((B * g.H, S), dtype=torch.float32, device="cuda")
    qws_bytes = lvq.lvq_quant_partial_workspace(g, B, cache.max_len)
    qws = torch.empty(max(qws_bytes, 256), dtype=torch.uint8, device="cuda")

    def quant_args(t, l):
        return (gref, t, qs[l][t].data_ptr(), pools[l].data_ptr(), cache.page_table.data_ptr(),
                int(cache.page_table.shape[1]), cache.seq_len.data_ptr(), cache.max_len, None, None,
                slices[l].data_ptr(),
                prob.rope_cos.data_ptr(), prob.rope_sin.data_ptr(), prob.rope16.data_ptr(), rope_len,
                C.c_float(prob.sm_scale), part_o.data_ptr(), part_lse.data_ptr(), S, S, qws.data_ptr(),
                qws.numel(), B, sh)

    qcalls = [quant_args(t, l) for t in range(cfg.T) for l in range(args.layers)]

    def quant_only():
        for a in qcalls:
            st = lib.lvq_quant_partial(*a)
            if st != 0:
                raise RuntimeError(lib.lvq_last_error().decode())

    dominant = quant_only
    if args.mode == "index-only":
        for _ in range(args.warmup + args.steps):
            dominant()
        torch.cuda.synchronize()
        print(f"index-only: {(args.warmup + args.steps) * len(qcalls)} launches", flush=True)
        return

    log(f"[bench] warmup {args.warmup} steps ({len(calls)} calls each, "
        f"{plan} splits)")
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    log(f"[bench] timed {args.steps} steps: {ms_total:.3f} ms")

    # The dominant kernel alone, same rotation, HIP events on the stream it is launched on.
    for _ in range(2):
        quant_only()
    torch.cuda.synchronize()
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0.record(stream)
    for _ in range(args.steps):
        quant_only()
    q1.record(stream)
    torch.cuda.synchronize()
    ms_quant = q0.elapsed_time(q1) / (args.steps * len(qcalls))
    log(f"[bench] index-page partial alone: {ms_quant * 1e3:.2f} us per launch")

    # MALL-warm: the same layer and step over and over (its 199 MB of index rows fit the 256 MB Infinity
    # Cache), for context only: the rotated figure above is the kernel's number.
    warm = qcalls[0]
    for _ in range(3):
        lib.lvq_quant_partial(*warm)
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(20):
        lib.lvq_quant_partial(*warm)
    w1.record(stream)
    torch.cuda.synchronize()
    ms_warm = w0.elapsed_time(w1) / 20

    # A plain device copy of 1 GiB (read + write), the bandwidth a streaming kernel can reach here.
    csrc = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(torch.cuda.current_stream())
    for _ in range(10):
        cdst.copy_(csrc)
    c1.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    copy_gbps = 2 * csrc.numel() * 4 * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del csrc, cdst
    log(f"[bench] MALL-warm index partial {ms_warm * 1e3:.2f} us; device copy {copy_gbps:.0f} GB/s")

    cb_bytes = 2 if cfg.cb_dtype == "bf16" else 4
    parts = call_bytes(g, prob.lengths, cb_bytes)
    per_call = sum(parts.values())
    n_calls = args.steps * len(calls)
    sec = ms_total / 1e3
    gbps = per_call * n_calls / sec / 1e9
    token_heads = sum(prob.lengths) * g.H
    kernel = "index_mfma_kernel"
    qbytes = quant_kernel_bytes(g, prob.lengths, cb_bytes, S)
    q_gbps = qbytes / (ms_quant / 1e3) / 1e9
    traffic = measured_traffic(kernel)

    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD, "B": cfg.B, "H": cfg.H, "L": cfg.L, "T": cfg.T, "Tc": cfg.Tc, "G": cfg.G,
            "K": cfg.K, "codebook": cfg.cb_dtype, "sink": cfg.sink, "window": cfg.window, "page": cfg.page,
            "layers_rotated": args.layers, "calls_per_step": len(calls),
            "path": f"{plan} splits",
            "requests_per_workgroup": 4,
        },
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "token_heads_per_s": round(token_heads * n_calls / sec, 1),
        "us_per_call": round(ms_total * 1e3 / n_calls, 2),
        "bytes_per_call": parts,
        "roofline": {
            "kernel": KERNELS[kernel],
            "bound": "hbm",
            "achieved": round(q_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "us_per_launch": round(ms_quant * 1e3, 2),
            "algorithmic_bytes_per_launch": qbytes,
            "copy_gbps_measured": round(copy_gbps, 1),
            "frac_of_measured_copy": round(q_gbps / copy_gbps, 4),
            "mall_warm_us_per_launch": round(ms_warm * 1e3, 2),
        },
        "cpu_baseline": None,
        "pages_context": {
            "two_requests_per_block": "a further -37% / -48% decode-attention time (0.5 / 0.25 bit) at batch 64, "
                                      "6K context; hardware not stated (LoopVQ page, method steps, step 5)",
            "attention_gpu_time_per_token": "BF16 1.87 ms -> LoopVQ 0.63 ms (0.5 bit) / 0.54 ms (0.25 bit), "
                                            "RTX 6000 Ada, batch 16 (LoopVQ page, Figure 15)",
        },
    }
    if want_cpu:
        log(f"[bench] cpu baseline: fp64 oracle on {len(sample_rows)} rows, every allowed core, "
            f"3 runs of {args.cpu_seconds:.0f}s")
        rate, rates, cores, model = cpu_baseline(prob, sample_rows, args.cpu_seconds)
        share = per_call / (B * g.H)
        result["cpu_baseline"] = {
            "value": round(rate * share / 1e9, 6),
            "unit": "GB/s",
            "cores": cores,
            "kind": "oracle",
            "cpu_model": model,
            "sample": f"(request, head, loop step) rows of {WORKLOAD} from requests/heads {sample_rows}, attention "
                      f"over the cache only (indices from the oracle's own encode, not timed); {cores} worker "
                      f"processes, one BLAS thread each, {args.cpu_seconds:.0f}s per run, median of "
                      f"{len(rates)} runs ({', '.join(f'{r:.1f}' for r in rates)} rows/s); bytes per row = "
                      f"1/(B*H) of one call",
            "token_heads_per_s": round(rate * cfg.L, 1),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
