"""The key scale stream of TaSQ+LoopVQ on the GPU against the oracle (oracle/loopvq.py, decode_step with
k_scales): each index token's reconstructed key times its fp16 scale for the loop step, bf16 window
tokens unscaled.  Scales are seeded stand-ins (the transform that produces them is not on the pages)."""

import sys

import numpy as np
import pytest
import torch

from oracle import loopvq as lv
from synth.configs import loopvq_config
from tests.test_gpu_loopvq import REL_TOL, LSE_TOL, _check_indices, _geo, lv_cb

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _scales(p, seed):
    """fp16 [physical pages][T][8], log-normal around 1 with some zeros."""
    n_phys = p.cache.pool.shape[0]
    gen = torch.Generator(device="cuda").manual_seed(seed)
    s = torch.exp(0.5 * torch.randn((n_phys, p.g.T, 8), generator=gen, device="cuda"))
    s[::7, :, 3] = 0.0
    return s.to(torch.float16).contiguous()


def _request_scales(p, sc_host, b):
    """[n_tok][T] scales of request b's index tokens in token order (through its page table)."""
    n = p.cache.n_pages[b]
    pages = np.asarray(p.cache.page_table_host[b, :n], dtype=np.int64)
    return np.transpose(sc_host[pages], (0, 2, 1)).reshape(n * 8, p.g.T)


def _check(p, t, rows, geo, idx, sc_host, out, lse):
    worst = 0.0
    for (b, h) in rows:
        q = p.q[t, b, h].float().cpu().numpy().astype(np.float64)
        rs = _request_scales(p, sc_host, b)
        o_ref, lse_ref = lv.decode_step(q, t, p.raw[("k", b, h)], p.raw[("v", b, h)], idx[(b, h)]["k"],
                                        idx[(b, h)]["v"], lv_cb(p, h, "k"), lv_cb(p, h, "v"), geo, p.lengths[b],
                                        p.sm_scale, p.cfg.rope_base, k_scales=rs)
        # the kernel's score error is relative to the unscaled score (fp16 query), so a token's scale
        # multiplies it: the logsumexp bound grows with the request's largest scale
        lse_tol = LSE_TOL * max(1.0, float(rs[:, t].max()) if rs.size else 1.0)
        o = out[b, h].double().cpu().numpy()
        err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
        worst = max(worst, err)
        assert err <= REL_TOL, f"step {t} row ({b},{h}): rel err {err:.3e}"
        assert abs(float(lse[b, h]) - lse_ref) <= lse_tol, (t, b, h, float(lse[b, h]), lse_ref, lse_tol)
    return worst


@pytest.mark.parametrize("name,over", [
    ("loopvq-b64-6k", dict(B=5, H=2, L=700)),
    ("loopvq-deep-ragged", dict(B=3, H=2, L=600, T=8, ragged=(100, 600))),
    ("loopvq-b1-1k-fp32cb", dict(B=2, H=2, L=700)),
], ids=["bf16-c8", "bf16-c4", "fp32"])
def test_key_scales_match_oracle(name, over):
    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = loopvq_config(name, **over)
    geo = _geo(cfg)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    _say(f"[kscale] {name} B={cfg.B} H={cfg.H}")
    p = harness.build_loopvq(cfg, keep=rows)
    idx = {r: _check_indices(p, r[0], r[1], geo) for r in rows}
    sc = _scales(p, 31)
    sc_host = sc.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    # ragged batches also with their requests grouped by length: scales follow the physical pages
    order = lvq.lvq_request_order(p.cache.seq_len, p.cache.max_len) if cfg.ragged else None
    for ns, od in ((0, None), (3, None)) + (((0, order),) if order is not None else ()):
        for t in range(cfg.T):
            lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
            out, _ = harness.run_step(p, t, num_splits=ns, lse=lse, k_scales=sc, order=od)
            torch.cuda.synchronize()
            worst = max(worst, _check(p, t, rows, geo, idx, sc_host, out, lse))
    # the standalone partial entry point takes the same stream
    c, S, t = p.cache, 2, cfg.T - 1
    po = torch.empty((cfg.B * cfg.H, S + 1, 128), dtype=torch.float32, device="cuda")
    pl = torch.empty((cfg.B * cfg.H, S + 1), dtype=torch.float32, device="cuda")
    q = p.q[t].contiguous()
    lvq.lvq_quant_partial(p.g, t, q, c.pool, c.page_table, c.seq_len, c.max_len, p.slices, p.rope_cos,
                          p.rope_sin, p.sm_scale, po, pl, S, rope_f16=p.rope16, k_scales=sc)
    lvq.lvq_window_partial(p.g, t, q, c.seq_len, c.max_len, c.win_k, c.win_v, p.rope_cos, p.rope_sin,
                           p.sm_scale, po, pl, slot=S)
    out, lse = lvq.splitk_lse_merge(po, pl)
    torch.cuda.synchronize()
    worst = max(worst, _check(p, t, rows, geo, idx, sc_host, out.view(cfg.B, cfg.H, 128),
                              lse.view(cfg.B, cfg.H)))
    _say(f"[kscale] {name} worst rel err {worst:.3e}")
