"""The matrix-core encoder against the fp64 oracle's argmin (LoopVQ page, background: a(z) = argmin_r
||z - e_r||^2, the lowest index on ties; method steps, step 4: the prefill encode as a matmul) where the
expansion form z.e - ||e||^2/2 cannot decide on its own:

- codebooks fitted to the data: entries that are the tokens' own coupled vectors (each such token at
  distance 0 from its entry), and codebooks after three GPU Lloyd steps;
- constructed near-ties: two entries a few bf16 ulps from a token whose distances differ by a factor of 4
  or are exactly equal (the lower index wins), both far inside the fp32 error of the expansion.

Bar: every index equals the oracle's, except where the two distances lie within 1e-6 relative."""

import sys

import numpy as np
import pytest
import torch

from oracle import loopvq as lv
from synth.configs import loopvq_config

pytestmark = pytest.mark.gpu

TIE_BAND = 1e-6
GEOMETRIES = [("loopvq-b64-6k", dict(B=2, H=2, L=600)),          # T_c = 2, 16-coordinate codewords
              ("loopvq-b8-32k", dict(B=2, H=1, L=700))]          # T_c = 4, 32-coordinate codewords


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _setup(name, over):
    import synth.loopvq as syn
    from tests import harness
    cfg = loopvq_config(name, **over)
    p = harness.build_loopvq(cfg)
    xs = {kind: dict(syn.raw_blocks(cfg, kind, "cuda")) for kind in ("k", "v")}
    return cfg, p, xs


def _coupled(p, xs, kind, beta, b, h):
    """Coupled vectors [n_tok][NG][G] (float64) of the index tokens of (b, h) in block beta."""
    g = p.g
    n_tok = p.cache.n_pages[b] * g.page
    x = xs[kind][beta][b, h, g.sink:g.sink + n_tok].float().cpu().numpy().astype(np.float64)   # [n][Tc][D]
    return lv.couple(np.transpose(x, (1, 0, 2)), g.G)


def _encode(p, xs, cb):
    import decode_attention_loopvq_amd as lvq
    c = p.cache
    c.pool.zero_()
    for beta in range(p.g.T // p.g.Tc):
        lvq.lvq_encode(p.g, beta, xs["k"][beta], xs["v"][beta], cb, c.pool, c.page_table, c.first_page,
                       c.n_pages_dev, c.max_pages, x_tok0=c.tok0)
    torch.cuda.synchronize()


def _compare(p, xs, cb, exact=None):
    """Every index of every (request, head, K|V, block, group) against the oracle with codebooks cb.
    exact: {(b, h, kind, beta, grp): expected indices of the first tokens} checked for equality."""
    from tests import harness
    g, cfg = p.g, p.cfg
    compared = banded = 0
    for h in range(cfg.H):
        for kv, kind in enumerate(("k", "v")):
            E = cb[:, h, kv].float().cpu().numpy().astype(np.float64)        # [NB][NG][K][G]
            for b in range(cfg.B):
                if p.cache.n_pages[b] == 0:
                    continue
                got_all = harness.gpu_indices(p, b, h, kind)                   # [NB][n][NG]
                for beta in range(g.T // g.Tc):
                    z = _coupled(p, xs, kind, beta, b, h)
                    for grp in range(z.shape[1]):
                        ref, d = lv.nearest_codeword(z[:, grp], E[beta, grp])
                        got = got_all[beta, :, grp].astype(np.int64)
                        rows = np.arange(len(ref))
                        bad = got != ref
                        ok = d[rows, got] <= d[rows, ref] * (1 + TIE_BAND)
                        assert np.all(ok), (f"{kind} b={b} h={h} block {beta} group {grp}: tokens "
                                            f"{np.flatnonzero(~ok)[:8]} got {got[~ok][:8]} oracle {ref[~ok][:8]}")
                        banded += int(bad.sum())
                        compared += len(ref)
                        want = (exact or {}).get((b, h, kind, beta, grp))
                        if want is not None:
                            np.testing.assert_array_equal(got[:len(want)], want)
    return compared, banded


@pytest.mark.parametrize("name,over", GEOMETRIES, ids=["g16", "g32"])
def test_lossless_codebooks(name, over):
    """Entries r < 256 are the coupled vectors of request 0's first 256 index tokens (per head, K|V, block,
    group): those tokens encode to their own entry (distance 0; the first of equal entries), every other
    token to the oracle's nearest entry."""
    cfg, p, xs = _setup(name, over)
    g = p.g
    cb = p.codebooks.clone()
    exact = {}
    for h in range(cfg.H):
        for kv, kind in enumerate(("k", "v")):
            for beta in range(g.T // g.Tc):
                z = _coupled(p, xs, kind, beta, 0, h)[:g.K]                    # [256][NG][G]
                assert z.shape[0] == g.K
                cb[beta, h, kv] = torch.from_numpy(np.transpose(z, (1, 0, 2)).copy()).to(cb.dtype).cuda()
                for grp in range(z.shape[1]):
                    # the first entry equal to each token's own vector
                    _, first, inv = np.unique(z[:, grp], axis=0, return_index=True, return_inverse=True)
                    exact[(0, h, kind, beta, grp)] = first[inv.reshape(-1)]
    _encode(p, xs, cb)
    compared, banded = _compare(p, xs, cb, exact)
    _say(f"[encode] {name} lossless: {compared} indices, {banded} within the tie band")
    assert banded == 0


def _next_bf16_up(v):
    """The bf16 value one ulp further from zero than v (v a bf16 value, nonzero)."""
    u = np.float32(v).view(np.uint32)
    return np.uint32((int(u >> 16) + 1) << 16).view(np.float32).astype(np.float64)


def _pair(v, rng, mode):
    """Two bf16 entries near token v and the index (0 or 1) the exact argmin takes among them.
    "ratio": one coordinate moved one ulp away from zero, the coordinate of largest binade in one entry, of
    smallest binade in the other: distances ulp^2 in different binades, ratio >= 4 (equal binades: equal
    distances, the lower index).  "tie": v + delta and v - delta with delta a whole number (-2 .. 2) of ulps
    per coordinate, kept inside each coordinate's binade: equal distances, the lower index, while the two
    entries differ in most coordinates (so their fp32 scores carry unrelated rounding)."""
    e = np.frexp(np.abs(v))[1].astype(np.int64)
    if mode == "ratio":
        ee = e.copy()
        ee[v == 0] = 10 ** 6
        k_small = int(np.argmin(ee))
        ee[v == 0] = -10 ** 6
        k_big = int(np.argmax(ee))
        near, far = v.copy(), v.copy()
        near[k_small] = _next_bf16_up(v[k_small])
        far[k_big] = _next_bf16_up(v[k_big])
        if e[k_small] == e[k_big]:
            return near, far, 0
        if rng.integers(2):
            return near, far, 0
        return far, near, 1
    ulp = np.ldexp(1.0, e - 8)                       # |v| in [2^(e-1), 2^e): bf16 spacing 2^(e-8)
    a = rng.integers(-2, 3, size=v.shape).astype(np.float64)
    lo, hi = np.ldexp(1.0, e - 1), np.ldexp(1.0, e)
    inside = (v != 0) & (np.abs(v) - np.abs(a) * ulp >= lo) & (np.abs(v) + np.abs(a) * ulp < hi)
    delta = np.where(inside, a * ulp, 0.0)
    return v + delta, v - delta, 0


@pytest.mark.parametrize("mode", ["ratio", "tie"])
@pytest.mark.parametrize("name,over", GEOMETRIES, ids=["g16", "g32"])
def test_constructed_near_ties(name, over, mode):
    """Entries 2 j and 2 j + 1 are two bf16 vectors near token j of request 0 (j < 128; see _pair), with
    distances ~2^-14 ||z||^2 or less, far inside the fp32 error of the expansion form: the exact argmin
    (including the lower index of an exact tie) for each such token, the oracle's pick for every other."""
    cfg, p, xs = _setup(name, over)
    g = p.g
    rng = np.random.default_rng(3)
    cb = p.codebooks.clone()
    exact = {}
    for h in range(cfg.H):
        for kv, kind in enumerate(("k", "v")):
            for beta in range(g.T // g.Tc):
                z = _coupled(p, xs, kind, beta, 0, h)                         # [n][NG][G]
                NG = z.shape[1]
                E = np.empty((NG, g.K, g.G))
                for grp in range(NG):
                    want = []
                    for j in range(g.K // 2):
                        e0, e1, w = _pair(z[j, grp].copy(), rng, mode)
                        E[grp, 2 * j], E[grp, 2 * j + 1] = e0, e1
                        want.append(2 * j + w)
                    exact[(0, h, kind, beta, grp)] = np.array(want)
                Et = torch.from_numpy(E).to(cb.dtype)
                assert torch.equal(Et.double(), torch.from_numpy(E)), "entries must be bf16 values"
                cb[beta, h, kv] = Et.cuda()
    _encode(p, xs, cb)
    compared, banded = _compare(p, xs, cb, exact)
    _say(f"[encode] {name} near ties ({mode}): {compared} indices, {banded} within the tie band")


@pytest.mark.parametrize("name,over", GEOMETRIES, ids=["g16", "g32"])
def test_after_lloyd_steps(name, over):
    """Three GPU Lloyd steps (lvq_encode + lvq_codebook_update with seeded log-normal weights) fit the
    codebooks to the data; the encode with the fitted codebooks against the oracle."""
    import decode_attention_loopvq_amd as lvq
    cfg, p, xs = _setup(name, over)
    g, c = p.g, p.cache
    NG = g.D // (g.G // g.Tc)
    gen = torch.Generator(device="cuda").manual_seed(78)
    L = xs["k"][0].shape[2]
    w = {kind: torch.exp(torch.randn((cfg.B, cfg.H, L, NG), generator=gen, device="cuda")) for kind in ("k", "v")}
    cb = p.codebooks.clone()
    for _ in range(3):
        for beta in range(g.T // g.Tc):
            lvq.lvq_encode(g, beta, xs["k"][beta], xs["v"][beta], cb, c.pool, c.page_table, c.first_page,
                           c.n_pages_dev, c.max_pages, x_tok0=c.tok0)
            lvq.lvq_codebook_update(g, beta, xs["k"][beta], xs["v"][beta], w["k"], w["v"], cb, c.pool,
                                    c.page_table, c.first_page, c.n_pages_dev, c.max_pages, x_tok0=c.tok0)
    _encode(p, xs, cb)
    compared, banded = _compare(p, xs, cb)
    _say(f"[encode] {name} after 3 Lloyd steps: {compared} indices, {banded} within the tie band")
