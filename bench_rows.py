#!/usr/bin/env python3
"""Per-step measurements of the quantized-KV decode path on one MI355X.

bench.py measures the headline workload (LoopVQ B=64, 6K).  This script
times every other step of the path on its own workload, each against the
roofline that bounds it, and prints one JSON line per measurement:

  encode-prefill   lvq_encode of every index page, K and V, 32K context
                   (B=8, H=16, T_c=4, G=32): bf16 distance contraction,
                   2*K*G flops per coupled vector; MFMA and HBM fractions
  encode-page      lvq_encode of one page per request (the decode-time
                   encode of the oldest window page), same workload
  attn-32k         lvq_decode_attn, 32K context, 0.25 bit, all four steps
  attn-deep        lvq_decode_attn, 32 loop steps, ragged lengths, random
                   page order (B=128, H=8), steps 0, 15, 31
  attn-1k          lvq_decode_attn, one request, 1K context, fp32 codebooks
                   (latency)
  kivi-prefill     kivi_append of a 4K prompt (B=16, H=32)
  kivi-append      kivi_append of one decode token
  kivi-attn        kivi_decode_attn after the 4K prefill
  kmeans-step      one Fisher-weighted k-means step (lvq_encode + lvq_codebook_update), 16 x 2048 tokens
  attn-6k-kscale   lvq_decode_attn on the 6K batch-64 workload with a key scale stream (TaSQ+LoopVQ),
                   against the same calls without it
  kivi4-attn       kivi_decode_attn with 4-bit keys and values (KIVI-4), B=16, H=32, 4K
  kivi-gqa-attn    kivi_decode_attn, 2-bit, 32 query heads over 8 KV heads, B=16, 4K

Inputs are seeded and synthetic (synth/), timed with HIP events on the
launch stream after warm-up.  Peaks: HBM 8 TB/s, dense bf16 MFMA
2.5 PFLOP/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12
PEAK_BF16 = 2.5e15


def timed(fn, reps, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3        # seconds per call


def emit(**kw):
    print(json.dumps(kw), flush=True)


def encode_rows(reps):
    import torch
    import decode_attention_loopvq_amd as lvq
    from decode_attention_loopvq_amd.layout import LoopVQCache, index_groups
    from synth import loopvq as syn
    from synth.configs import loopvq_config
    from tests.harness import geom_of

    cfg = loopvq_config("loopvq-b8-32k")
    g = geom_of(cfg)
    lengths = syn.lengths(cfg)
    cache = LoopVQCache(g, lengths, device="cuda")
    cb = syn.codebooks(cfg, "cuda")
    xs = {kind: x for kind in ("k", "v") for beta, x in syn.raw_blocks(cfg, kind, "cuda") if beta == 0}
    NG = index_groups(g)
    n_vec = sum(cache.n_pages) * g.page * g.H * NG * 2                   # coupled vectors, K and V
    flops = 2.0 * g.K * g.G * n_vec
    in_bytes = sum(cache.n_pages) * g.page * g.H * g.Tc * g.D * 2 * 2 + cb[0].numel() * 2
    out_bytes = n_vec

    def prefill():
        lvq.lvq_encode(g, 0, xs["k"], xs["v"], cb, cache.pool, cache.page_table, cache.first_page,
                       cache.n_pages_dev, cache.max_pages, x_tok0=cache.tok0)

    t = timed(prefill, reps, warmup=1)
    emit(row="encode-prefill", workload=cfg.name, B=cfg.B, H=cfg.H, tokens_per_request=cache.n_pages[0] * 8,
         ms=round(t * 1e3, 3), tflops=round(flops / t / 1e12, 3), mfma_frac=round(flops / t / PEAK_BF16, 5),
         hbm_gbps=round((in_bytes + out_bytes) / t / 1e9, 1),
         hbm_frac=round((in_bytes + out_bytes) / t / PEAK_HBM, 5), flops=flops, bytes=in_bytes + out_bytes)

    last = torch.tensor([n - 1 for n in cache.n_pages], dtype=torch.int32, device="cuda")
    one = torch.ones_like(last)
    tok0 = cache.tok0 + last.long() * g.page

    def page():
        lvq.lvq_encode(g, 0, xs["k"], xs["v"], cb, cache.pool, cache.page_table, last, one, 1, x_tok0=tok0)

    t = timed(page, reps * 20)
    cb_bytes = g.H * 2 * NG * g.K * g.G * 2                               # the block's codebooks, read once
    emit(row="encode-page", workload=cfg.name, B=cfg.B, H=cfg.H, us=round(t * 1e6, 2),
         codebook_gbps=round(cb_bytes / t / 1e9, 1), codebook_bytes=cb_bytes)
    del xs


def kmeans_row(reps):
    """One Fisher-weighted k-means step (assignment by lvq_encode, weighted means by
    lvq_codebook_update), every loop block, K and V, on a calibration set of the page's size: 16
    sequences of 2048 tokens (the 6K workload's geometry), log-normal stand-in weights."""
    import torch
    import decode_attention_loopvq_amd as lvq
    import synth.loopvq as syn
    from synth.configs import loopvq_config
    from tests import harness

    cfg = loopvq_config("loopvq-b64-6k", B=16, L=2048)
    p = harness.build_loopvq(cfg)
    g, c = p.g, p.cache
    xs = {kind: dict(syn.raw_blocks(cfg, kind, "cuda")) for kind in ("k", "v")}
    NG = g.D // (g.G // g.Tc)
    gen = torch.Generator(device="cuda").manual_seed(5)
    w = {kind: torch.exp(torch.randn((cfg.B, cfg.H, cfg.L, NG), generator=gen, device="cuda")) for kind in "kv"}
    cb = p.codebooks.clone()

    def step():
        for beta in range(g.T // g.Tc):
            lvq.lvq_encode(g, beta, xs["k"][beta], xs["v"][beta], cb, c.pool, c.page_table, c.first_page,
                           c.n_pages_dev, c.max_pages, x_tok0=c.tok0)
            lvq.lvq_codebook_update(g, beta, xs["k"][beta], xs["v"][beta], w["k"], w["v"], cb, c.pool,
                                    c.page_table, c.first_page, c.n_pages_dev, c.max_pages, x_tok0=c.tok0)

    def update_only():
        for beta in range(g.T // g.Tc):
            lvq.lvq_codebook_update(g, beta, xs["k"][beta], xs["v"][beta], w["k"], w["v"], cb, c.pool,
                                    c.page_table, c.first_page, c.n_pages_dev, c.max_pages, x_tok0=c.tok0)

    t = timed(step, reps)
    t_upd = timed(update_only, reps)
    n_vec = sum(c.n_pages) * g.page * g.H * NG * 2 * (g.T // g.Tc)
    emit(row="kmeans-step", workload="loopvq-b64-6k geometry, 16 x 2048-token calibration set", B=cfg.B,
         H=cfg.H, L=cfg.L, us=round(t * 1e6, 2), update_us=round(t_upd * 1e6, 2), coupled_vectors=n_vec,
         vectors_per_s=round(n_vec / t, 1), assign_flops=2.0 * g.K * g.G * n_vec)


def attn_row(name, cfg_name, steps, reps, kscale=False, **over):
    import torch
    import decode_attention_loopvq_amd as lvq
    from synth.configs import loopvq_config
    from tests import harness
    from bench import call_bytes

    cfg = loopvq_config(cfg_name, **over)
    p = harness.build_loopvq(cfg)
    cb_bytes = 2 if cfg.cb_dtype == "bf16" else 4
    per_call = sum(call_bytes(p.g, p.lengths, cb_bytes).values())
    out = torch.empty((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(lvq.lvq_decode_attn_workspace(p.g, cfg.B, p.cache.max_len), dtype=torch.uint8,
                     device="cuda")
    qs = [p.q[t].contiguous() for t in range(cfg.T)]
    # Ragged batches: the requests grouped by length (one order per decode step, shared by its calls).
    order = lvq.lvq_request_order(p.cache.seq_len, p.cache.max_len) if cfg.ragged else None
    extra = {}
    if order is not None:
        t_ord = timed(lambda: lvq.lvq_request_order(p.cache.seq_len, p.cache.max_len, out=order), reps * 10)
        extra = dict(order="by length (lvq_request_order, once per decode step)", order_us=round(t_ord * 1e6, 2))

    # key scale stream (TaSQ+LoopVQ): fp16 per index token and loop step, 2 bytes per index token per call
    sc = None
    if kscale:
        gen = torch.Generator(device="cuda").manual_seed(3)
        sc = torch.exp(0.25 * torch.randn((p.cache.pool.shape[0], cfg.T, 8), generator=gen, device="cuda"))
        sc = sc.to(torch.float16)
    # The calls are prebuilt ctypes argument tuples (as in bench.py): the Python binding's argument checks
    # would add host time comparable to a call's GPU time.
    import ctypes as C
    from decode_attention_loopvq_amd._lib import lib
    gref = C.byref(p.g)
    sh = torch.cuda.current_stream().cuda_stream
    ws_bytes = ws.numel()

    def call_args(t, ks):
        c = p.cache
        return (gref, t, qs[t].data_ptr(), c.pool.data_ptr(), c.page_table.data_ptr(), int(c.page_table.shape[1]),
                c.seq_len.data_ptr(), c.max_len, order.data_ptr() if order is not None else None,
                ks.data_ptr() if ks is not None else None, c.win_k.data_ptr(), c.win_v.data_ptr(),
                p.slices.data_ptr(), p.rope_cos.data_ptr(), p.rope_sin.data_ptr(), p.rope16.data_ptr(),
                int(p.rope_cos.shape[0]), C.c_float(p.sm_scale), out.data_ptr(), None, ws.data_ptr(), ws_bytes, 0,
                cfg.B, sh)

    def runner(calls):
        def run():
            for a in calls:
                if lib.lvq_decode_attn(*a) != 0:
                    raise RuntimeError(lib.lvq_last_error().decode())
        return run

    if kscale:
        t0 = timed(runner([call_args(t, None) for t in steps]), reps) / len(steps)
        per_call += sum(p.cache.n_pages) * 8 * 2
        extra["unscaled_us_per_call"] = round(t0 * 1e6, 2)

    t = timed(runner([call_args(t, sc) for t in steps]), reps) / len(steps)
    emit(row=name, workload=cfg.name, B=cfg.B, H=cfg.H, L=cfg.L, steps=list(steps), us_per_call=round(t * 1e6, 2),
         gbps=round(per_call / t / 1e9, 1), hbm_frac=round(per_call / t / PEAK_HBM, 4), bytes_per_call=per_call,
         token_heads_per_s=round(sum(p.lengths) * cfg.H / t, 1), **extra)


def kivi_call(g, q, cache, max_len, sm_scale, out, ws):
    """A prebuilt kivi_decode_attn call (ctypes arguments made once, as for the LoopVQ attention rows: the
    binding's checks would add host time comparable to a call's GPU time)."""
    import ctypes as C
    import torch
    from decode_attention_loopvq_amd._lib import lib
    args = (C.byref(g), q.data_ptr(), C.byref(cache.c), int(max_len), C.c_float(sm_scale), out.data_ptr(), None,
            ws.data_ptr(), ws.numel(), 0, int(cache.B), torch.cuda.current_stream().cuda_stream)

    def run():
        if lib.kivi_decode_attn(*args) != 0:
            raise RuntimeError(lib.lvq_last_error().decode())
    return run


def kivi_rows(reps):
    import torch
    import decode_attention_loopvq_amd as lvq
    from synth import kivi as synk
    from synth.configs import kivi_config

    cfg = kivi_config("kivi-b16-4k")
    cap = ((cfg.L + 256 + cfg.group - 1) // cfg.group) * cfg.group
    g = lvq.make_kivi_geom(D=cfg.D, H=cfg.H, bits=cfg.bits, group=cfg.group, R=cfg.R, cap=cap)
    k, v = synk.raw_kv(cfg, "cuda")
    cache = lvq.KiviCache(g, cfg.B, device="cuda")

    def prefill():
        cache.len.zero_()
        cache.n_kq.zero_()
        cache.n_vq.zero_()
        lvq.kivi_append(g, k, v, cache, prefill=True)

    t = timed(prefill, reps)
    raw = k.numel() * 2 * 2
    n_q = cfg.L - cfg.R
    written = cfg.B * cfg.H * (n_q * cfg.D // 4 * 2 + (n_q // cfg.group) * cfg.D * 4 + n_q * (cfg.D // cfg.group) * 4
                               + cfg.R * cfg.D * 2 * 2)
    emit(row="kivi-prefill", workload=cfg.name, B=cfg.B, H=cfg.H, L=cfg.L, us=round(t * 1e6, 2),
         gbps=round((raw + written) / t / 1e9, 1), hbm_frac=round((raw + written) / t / PEAK_HBM, 4),
         bytes=raw + written)

    prefill()
    q = synk.queries(cfg, "cuda")[0].contiguous()
    out = torch.empty((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device="cuda")
    # max_len: the longest request after the prefill (what a server knows on the host), not the capacity
    ws = torch.empty(lvq.kivi_decode_attn_workspace(g, cfg.B, cfg.L), dtype=torch.uint8, device="cuda")

    attn = kivi_call(g, q, cache, cfg.L, synk.softmax_scale(cfg), out, ws)
    t = timed(attn, reps * 10)
    per_bh = n_q * cfg.D // 4 * 2 + (n_q // cfg.group) * cfg.D * 4 + n_q * (cfg.D // cfg.group) * 4 \
        + cfg.R * cfg.D * 2 * 2
    by = cfg.B * cfg.H * (per_bh + cfg.D * (2 + 4))
    emit(row="kivi-attn", workload=cfg.name, B=cfg.B, H=cfg.H, L=cfg.L, us_per_call=round(t * 1e6, 2),
         gbps=round(by / t / 1e9, 1), hbm_frac=round(by / t / PEAK_HBM, 4), bytes_per_call=by,
         token_heads_per_s=round(cfg.B * cfg.H * cfg.L / t, 1))

    k1 = k[:, :, :1].clone()
    v1 = v[:, :, :1].clone()
    n_app = 64

    def appends():
        for _ in range(n_app):
            lvq.kivi_append(g, k1, v1, cache, prefill=False)

    t = timed(appends, 2, warmup=0) / n_app
    emit(row="kivi-append", workload=cfg.name, B=cfg.B, H=cfg.H, us_per_token=round(t * 1e6, 2))


def kivi_variant_row(row, name, reps):
    """Prefill then time decode attention on a KIVI variant workload; algorithmic bytes per call are
    each KV head's codes at their widths, its scales and zero-points and fp16 residual, plus every
    query head's fp16 query and fp32 output."""
    import torch
    import decode_attention_loopvq_amd as lvq
    from synth import kivi as synk
    from synth.configs import kivi_config
    from tests import harness

    cfg = kivi_config(name)
    p = harness.build_kivi(cfg)
    g = p.g
    kb, vb, Hq = lvq.kivi_widths(g)
    out = torch.empty((cfg.B, Hq, cfg.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(lvq.kivi_decode_attn_workspace(g, cfg.B, cfg.L), dtype=torch.uint8, device="cuda")

    attn = kivi_call(g, p.q, p.cache, cfg.L, p.sm_scale, out, ws)
    t = timed(attn, reps * 10)
    n_q = cfg.L - cfg.R
    per_kv = (n_q * cfg.D * kb // 8 + (n_q // cfg.group) * cfg.D * 4 + n_q * cfg.D * vb // 8
              + n_q * (cfg.D // cfg.group) * 4 + cfg.R * cfg.D * 2 * 2)
    by = cfg.B * cfg.H * per_kv + cfg.B * Hq * cfg.D * (2 + 4)
    emit(row=row, workload=cfg.name, B=cfg.B, H=cfg.H, Hq=Hq, key_bits=kb, value_bits=vb, L=cfg.L,
         us_per_call=round(t * 1e6, 2), gbps=round(by / t / 1e9, 1), hbm_frac=round(by / t / PEAK_HBM, 4),
         bytes_per_call=by, token_heads_per_s=round(cfg.B * Hq * cfg.L / t, 1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--only", nargs="*", default=None, help="encode attn-32k attn-deep attn-1k attn-6k-kscale kivi kivi4 kivi-gqa kmeans")
    args = ap.parse_args()
    import torch
    assert torch.cuda.is_available(), "bench_rows.py needs a GPU"
    want = set(args.only) if args.only else {"encode", "attn-32k", "attn-deep", "attn-1k", "attn-6k-kscale", "kivi",
                                                         "kivi4", "kivi-gqa", "kmeans"}
    if "encode" in want:
        encode_rows(args.reps)
    if "attn-32k" in want:
        attn_row("attn-32k", "loopvq-b8-32k", range(4), args.reps)
    if "attn-deep" in want:
        attn_row("attn-deep", "loopvq-deep-ragged", (0, 15, 31), args.reps)
    if "attn-1k" in want:
        attn_row("attn-1k", "loopvq-b1-1k-fp32cb", range(4), args.reps * 20)
    if "attn-6k-kscale" in want:
        attn_row("attn-6k-kscale", "loopvq-b64-6k", range(4), args.reps, kscale=True)
    if "kivi" in want:
        kivi_rows(args.reps)
    if "kmeans" in want:
        kmeans_row(args.reps)
    if "kivi4" in want:
        kivi_variant_row("kivi4-attn", "kivi4-b16-4k", args.reps)
    if "kivi-gqa" in want:
        kivi_variant_row("kivi-gqa-attn", "kivi-gqa-b16-4k", args.reps)


if __name__ == "__main__":
    main()
