"""One Fisher-weighted k-means step on the GPU (lvq_encode for the assignment, lvq_codebook_update for
the weighted means) against the fp64 oracle (oracle/kmeans.py), and Lloyd's monotone objective over
several GPU steps.  Weights are seeded log-normal stand-ins for the page's gradient-based Fisher
weights."""

import sys

import numpy as np
import pytest
import torch

from oracle import kmeans as km
from oracle import loopvq as lv
from synth.configs import loopvq_config

pytestmark = pytest.mark.gpu

TIE = 1e-6          # relative distance band in which the encoder's pick may differ from the exact argmin


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _round_to(x: np.ndarray, bf16: bool) -> np.ndarray:
    """x (float64) rounded once to bf16 or fp32, nearest-even."""
    x = np.asarray(x, dtype=np.float64)
    if not bf16:
        return x.astype(np.float32).astype(np.float64)
    # to fp32 with round-to-odd (no double rounding), then nearest-even on the top 16 bits
    f = x.astype(np.float32)
    u = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != x
    u[inexact & ((u & 1) == 0)] += np.where(np.abs(x) > np.abs(f.astype(np.float64)), 1, -1)[inexact & ((u & 1) == 0)].astype(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.view(np.float32).astype(np.float64)


def _setup(name, over):
    import synth.loopvq as syn
    from tests import harness
    cfg = loopvq_config(name, **over)
    p = harness.build_loopvq(cfg)
    g = p.g
    NG = g.D // (g.G // g.Tc)
    xs = {kind: dict(syn.raw_blocks(cfg, kind, "cuda")) for kind in ("k", "v")}
    gen = torch.Generator(device="cuda").manual_seed(77)
    L = xs["k"][0].shape[2]                          # token rows of the raw data
    w = {kind: torch.exp(torch.randn((cfg.B, cfg.H, L, NG), generator=gen, device="cuda")) for kind in ("k", "v")}
    return cfg, p, xs, w, NG


def _coupled(p, xs, kind, beta, b, h, NG):
    """Coupled vectors [n_tok][NG][G] of the index tokens of (b, h) for block beta, float64."""
    g = p.g
    n_tok = p.cache.n_pages[b] * g.page
    x = xs[kind][beta][b, h, g.sink:g.sink + n_tok].float().cpu().numpy().astype(np.float64)   # [n][Tc][D]
    return lv.couple(np.transpose(x, (1, 0, 2)), g.G)


def _shifted(x):
    """The same values one element past an aligned start (the update's scalar-load path)."""
    buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
    buf[1:] = x.reshape(-1)
    return buf[1:].view(x.shape)


def _update(p, xs, w, cb, beta, shift=False):
    import decode_attention_loopvq_amd as lvq
    c = p.cache
    lvq.lvq_encode(p.g, beta, xs["k"][beta], xs["v"][beta], cb, c.pool, c.page_table, c.first_page,
                   c.n_pages_dev, c.max_pages, x_tok0=c.tok0)
    xk, xv = xs["k"][beta], xs["v"][beta]
    if shift:
        xk, xv = _shifted(xk.contiguous()), _shifted(xv.contiguous())
    lvq.lvq_codebook_update(p.g, beta, xk, xv, w["k"], w["v"], cb, c.pool, c.page_table,
                            c.first_page, c.n_pages_dev, c.max_pages, x_tok0=c.tok0)


# H=4 takes the XCD-grouped workgroup order (2H a multiple of 8), H=1 and H=2 the plain one; "shift"
# hands the update x one element off its aligned start (per-channel loads instead of vector loads).
@pytest.mark.parametrize("name,over,shift", [
    ("loopvq-b64-6k", dict(B=3, H=4, L=600, ragged=(300, 600)), False),
    ("loopvq-b64-6k", dict(B=2, H=2, L=400, ragged=(250, 400)), True),
    ("loopvq-deep-ragged", dict(B=2, H=1, L=500, T=8, ragged=(300, 500)), False),
    ("loopvq-deep-ragged", dict(B=2, H=4, L=400, T=8, ragged=(200, 400)), True),
    ("loopvq-b1-1k-fp32cb", dict(B=2, H=2, L=700), False),
    # lengths 81, 79, 204, 55: one request with a single index page, two with none
    ("loopvq-b64-6k", dict(B=4, H=2, L=600, ragged=(10, 600)), False),
    ("loopvq-deep-ragged", dict(B=2, H=4, L=450, T=8, ragged=(200, 450), cb_dtype="fp32"), False),
], ids=["bf16-c8", "bf16-c8-unaligned", "bf16-c4", "bf16-c4-unaligned-xcd", "fp32", "bf16-c8-short", "fp32-c4-xcd"])
def test_update_matches_oracle(name, over, shift):
    cfg, p, xs, w, NG = _setup(name, over)
    g = p.g
    bf16 = cfg.cb_dtype == "bf16"
    E0 = p.codebooks.clone()
    cb = p.codebooks.clone()
    skipped = compared = near_mid = 0
    for beta in range(g.T // g.Tc):
        _say(f"[kmeans] {cfg.name} H={cfg.H} shift={shift} block {beta}")
        _update(p, xs, w, cb, beta, shift)
        torch.cuda.synchronize()
        for h in range(cfg.H):
            for kv, kind in enumerate(("k", "v")):
                zs, ws = [], []
                for b in range(cfg.B):
                    if p.cache.n_pages[b] == 0:
                        continue
                    zs.append(_coupled(p, xs, kind, beta, b, h, NG))
                    n_tok = p.cache.n_pages[b] * g.page
                    ws.append(w[kind][b, h, g.sink:g.sink + n_tok].cpu().numpy().astype(np.float64))
                z = np.concatenate(zs)                      # [N][NG][G]
                wt = np.concatenate(ws)                     # [N][NG]
                for grp in range(NG):
                    N = z.shape[0]
                    amax = np.max(wt[:, grp, None] * np.abs(z[:, grp]))
                    wmax = np.max(wt[:, grp])
                    E = E0[beta, h, kv, grp].float().cpu().numpy().astype(np.float64)
                    a, d = lv.nearest_codeword(z[:, grp], E)
                    # codewords whose cluster can change within the tie band are not compared
                    best = d[np.arange(len(a)), a]
                    near = d <= best[:, None] * (1 + TIE) + 1e-300
                    ambiguous = np.unique(np.nonzero(near.sum(axis=1) > 1)[0])
                    shaky = set(a[ambiguous].tolist())
                    for n in ambiguous:
                        shaky.update(np.nonzero(near[n])[0].tolist())
                    ref = km.weighted_update(z[:, grp], wt[:, grp], a, E)
                    got = cb[beta, h, kv, grp].float().cpu().numpy().astype(np.float64)
                    for r in range(g.K):
                        if r in shaky:
                            skipped += 1
                            continue
                        compared += 1
                        sel = a == r
                        if not sel.any():
                            np.testing.assert_array_equal(got[r], E[r])     # empty cluster keeps its value
                            continue
                        # the kernel adds w*z and w as integers in steps of 2^-e and 2^-ew, with
                        # 2^-e <= 2 N max|w z| 2^-51 (likewise w): its codeword is the dtype rounding of a
                        # mean within eb of the exact one
                        n_r, den = sel.sum(), np.sum(wt[sel, grp])
                        eb = 1.01 * (n_r * (N * amax * 2.0 ** -51) / den
                                     + np.abs(ref[r]) * n_r * (N * wmax * 2.0 ** -51) / den)
                        lo, hi = _round_to(ref[r] - eb, bf16), _round_to(ref[r] + eb, bf16)
                        assert np.all((got[r] >= lo) & (got[r] <= hi)), (beta, h, kind, grp, r, got[r], ref[r], eb)
                        near_mid += int(np.sum(got[r] != _round_to(ref[r], bf16)))
    _say(f"[kmeans] {compared} codewords compared, {skipped} skipped in the tie band, "
         f"{near_mid} coordinates off the once-rounded mean (within the fixed-point bound)")
    assert skipped <= compared // 100


def test_objective_never_rises_on_gpu():
    """Three GPU Lloyd steps (encode + update) from the synthetic N(0,1) codebooks: the fp64 weighted
    objective of the GPU codebooks does not rise (up to the bf16 rounding of the codewords)."""
    cfg, p, xs, w, NG = _setup("loopvq-b64-6k", dict(B=2, H=1, L=900))
    g = p.g
    h, kind, beta, grp = 0, "v", 0, 5
    z = np.concatenate([_coupled(p, xs, kind, beta, b, h, NG)[:, grp] for b in range(cfg.B)])
    wt = np.concatenate([w[kind][b, h, g.sink:g.sink + p.cache.n_pages[b] * g.page, grp].cpu().numpy()
                         for b in range(cfg.B)]).astype(np.float64)
    cb = p.codebooks.clone()
    prev = km.objective(z, wt, cb[beta, h, 1, grp].float().cpu().numpy().astype(np.float64))
    for it in range(3):
        _update(p, xs, w, cb, beta)
        torch.cuda.synchronize()
        cur = km.objective(z, wt, cb[beta, h, 1, grp].float().cpu().numpy().astype(np.float64))
        _say(f"[kmeans] step {it}: objective {prev:.6g} -> {cur:.6g}")
        assert cur <= prev * (1 + 1e-3)
        prev = cur
