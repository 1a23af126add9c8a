"""Decode-attention calls captured in a HIP graph (a serving loop's form): every replay, with the
program's own eager work and synchronizations between replays, must equal the eager calls bit for bit.

Both entry points launch only kernels on the caller's stream (no allocation, no memset, no host
synchronization), so a capture records the same kernels; these tests hold that, for the LoopVQ split path
with and without the packed RoPE table (without it the table is built in the workspace by a kernel of
the call) and for KIVI attention with grouped queries (matrix-core kernel, residual slot, merge).
"""

import sys

import pytest
import torch

from synth.configs import kivi_config, loopvq_config

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _replays_match(graph, outs, refs, n=3):
    for rep in range(n):
        for o in outs:
            o.zero_()
        _ = torch.randn(1 << 16, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"replay {rep}, output {i} differs from the eager call"


@pytest.mark.parametrize("packed", [True, False], ids=["packed-table", "table-in-workspace"])
def test_loopvq_decode_attn_graph_replays(packed):
    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = loopvq_config("loopvq-b64-6k", B=6, H=2, L=700, ragged=(40, 700), random_pages=True, seed=21)
    _say(f"[graph] loopvq B={cfg.B} H={cfg.H} L={cfg.L} packed table {packed}")
    p = harness.build_loopvq(cfg)
    steps = list(range(cfg.T))
    outs = [torch.empty((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device="cuda") for _ in steps]
    lses = [torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda") for _ in steps]
    ws = torch.empty(lvq.lvq_decode_attn_workspace(p.g, cfg.B, p.cache.max_len), dtype=torch.uint8, device="cuda")
    qs = [p.q[t].contiguous() for t in steps]
    s = torch.cuda.Stream()

    def calls():
        for t in steps:
            lvq.lvq_decode_attn(p.g, t, qs[t], p.cache.pool, p.cache.page_table, p.cache.seq_len, p.cache.max_len,
                                p.cache.win_k, p.cache.win_v, p.slices, p.rope_cos, p.rope_sin, p.sm_scale,
                                out=outs[t], lse_out=lses[t], ws=ws, rope_f16=p.rope16 if packed else None)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs + lses]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        calls()
    torch.cuda.synchronize()
    _replays_match(graph, outs + lses, refs)


def test_kivi_decode_attn_graph_replays():
    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = kivi_config("kivi-b16-4k", B=3, H=2, L=700, Hq=8)
    _say(f"[graph] kivi B={cfg.B} H={cfg.H} Hq={cfg.Hq} L={cfg.L}")
    p = harness.build_kivi(cfg)
    Hq = lvq.kivi_widths(p.g)[2]
    max_len = int(p.cache.len.max())
    out = torch.empty((cfg.B, Hq, cfg.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(lvq.kivi_decode_attn_workspace(p.g, cfg.B, max_len), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()

    def calls():
        lvq.kivi_decode_attn(p.g, p.q, p.cache, max_len, p.sm_scale, out=out, lse_out=lse, ws=ws)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    refs = [out.clone(), lse.clone()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        calls()
    torch.cuda.synchronize()
    _replays_match(graph, [out, lse], refs)
