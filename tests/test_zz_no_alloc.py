"""lvq_decode_attn_noalloc (the entry point for callers that cannot allocate) against lvq_decode_attn on
the same inputs: two calls in a row, the second on a smaller batch and context, both through the C ABI, with
and without the packed fp16 RoPE table.
The two share their kernels, so the outputs are expected bit for bit equal; the bar written here is the
attention bar (2e-3 relative per (request, head) row, lse within 2e-3) plus that equality."""

import sys

import pytest
import torch

import decode_attention_loopvq_amd as lvq
from synth.configs import loopvq_config

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
LSE_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(p, t, num_splits=0):
    from tests import harness
    c = p.cache
    B, H = p.cfg.B, p.cfg.H
    ref, lse_ref = harness.run_step(p, t, num_splits=num_splits,
                                    lse=torch.empty((B, H), dtype=torch.float32, device="cuda"))
    out = torch.full((B, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    lvq.lvq_decode_attn_noalloc(p.g, t, p.q[t].contiguous(), c.pool, c.page_table, c.seq_len, c.max_len, c.win_k,
                                c.win_v, p.slices, p.rope_cos, p.rope_sin, p.sm_scale, out, lse_out=lse,
                                num_splits=num_splits, rope_f16=p.rope16)
    torch.cuda.synchronize()
    return ref, lse_ref, out, lse


def _check(ref, lse_ref, out, lse):
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    err = ((out - ref).abs().amax(dim=2) / ref.abs().amax(dim=2)).max().item()
    assert err <= REL_TOL, f"rel err {err:.3e}"
    assert (lse - lse_ref).abs().max().item() <= LSE_TOL
    assert torch.equal(out, ref) and torch.equal(lse, lse_ref)


def test_noalloc_matches_decode_attn_on_two_calls():
    from tests import harness
    big = loopvq_config("loopvq-b64-6k", B=9, H=2, L=3000, ragged=(40, 3000), random_pages=True, seed=31)
    small = loopvq_config("loopvq-b64-6k", B=3, H=2, L=500, seed=32)
    _say(f"[build] {big.name} B={big.B} L={big.L}")
    pb = harness.build_loopvq(big, keep=[])
    _say(f"[build] {small.name} B={small.B} L={small.L}")
    ps = harness.build_loopvq(small, keep=[])
    for t in (0, 3):
        _say(f"[noalloc] big step {t}")
        _check(*_both(pb, t))
        _say(f"[noalloc] small step {t}")
        _check(*_both(ps, t))
    _say("[noalloc] big, 3 splits")
    _check(*_both(pb, 1, num_splits=3))
    # without the packed fp16 RoPE table both calls build it in their workspace from the fp32 tables
    import dataclasses
    _say("[noalloc] big and small without the packed table")
    _check(*_both(dataclasses.replace(pb, rope16=None), 2))
    _check(*_both(dataclasses.replace(ps, rope16=None), 2))
