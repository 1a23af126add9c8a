"""Parity of the HIP LoopVQ path with the fp64 oracle (GPU).

Bars: indices and dequantised values bit-exact (a differing index passes only
if its fp64 distance is within 1e-6 relative of the oracle's, lowest index
on ties); attention outputs within max relative error 2e-3 per (request,
head) row, ||o_gpu - o_ref||_inf / ||o_ref||_inf.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import loopvq as lv
from synth.configs import loopvq_config

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
LSE_TOL = 2e-3
TIE_BAND = 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _geo(cfg):
    return lv.Geometry(D=cfg.D, T=cfg.T, Tc=cfg.Tc, G=cfg.G, K=cfg.K, sink=cfg.sink, window=cfg.window,
                       page=cfg.page)


def _oracle_indices(raw, E, geo, L, blocks=None):
    """The oracle's encode of one (request, head) (encode_request's steps: the coupled vectors of each loop
    block, then each group's nearest codeword), for the loop blocks `blocks` only (all when None; the others
    stay zero), with the (block, group) problems spread over host threads."""
    from concurrent.futures import ThreadPoolExecutor
    _, q_lo, q_hi = lv.cache_regions(L, geo)
    out = np.zeros((geo.NB, q_hi - q_lo, geo.NG), dtype=np.uint8)
    if q_hi == q_lo:
        return out
    blocks = range(geo.NB) if blocks is None else blocks
    with ThreadPoolExecutor(max_workers=16) as ex:
        jobs = []
        for beta in blocks:
            x_block = np.transpose(np.asarray(raw[q_lo:q_hi, beta * geo.Tc:(beta + 1) * geo.Tc, :], np.float64),
                                   (1, 0, 2))
            z = lv.couple(x_block, geo.G)
            for grp in range(geo.NG):
                jobs.append((beta, grp, ex.submit(lv.nearest_codeword, np.ascontiguousarray(z[:, grp]),
                                                  np.asarray(E[beta, grp], np.float64))))
        for beta, grp, job in jobs:
            out[beta, :, grp] = job.result()[0]
    return out


def _check_indices(p, b, h, geo, blocks=None):
    """GPU indices of (b, h) against the oracle's encode (loop blocks `blocks`, all when None); returns the
    oracle's indices."""
    from tests import harness
    L = p.lengths[b]
    _, q_lo, q_hi = lv.cache_regions(L, geo)
    out = {}
    for kind in ("k", "v"):
        E = harness.host_codebooks(p, h, kind)
        ref = _oracle_indices(p.raw[(kind, b, h)], E, geo, L, blocks)
        got = harness.gpu_indices(p, b, h, kind)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        if blocks is not None:
            keep = np.zeros(geo.NB, dtype=bool)
            keep[list(blocks)] = True
            got = np.where(keep[:, None, None], got, ref)
        bad = np.argwhere(got != ref)
        for beta, j, g in bad:
            x = p.raw[(kind, b, h)][q_lo + j, beta * geo.Tc:(beta + 1) * geo.Tc, :]
            z = lv.couple(x[:, None, :], geo.G)[0, g]
            _, d = lv.nearest_codeword(z[None], E[beta, g])
            assert d[0, got[beta, j, g]] <= d[0, ref[beta, j, g]] * (1 + TIE_BAND), \
                f"index mismatch at block {beta} token {j} group {g}"
        out[kind] = ref
    return out


def _check_row(p, t, b, h, geo, idx, out, lse):
    L = p.lengths[b]
    Ek, Ev = (lv_cb(p, h, "k"), lv_cb(p, h, "v"))
    q = p.q[t, b, h].float().cpu().numpy().astype(np.float64)
    o_ref, lse_ref = lv.decode_step(q, t, p.raw[("k", b, h)], p.raw[("v", b, h)], idx["k"], idx["v"], Ek, Ev,
                                    geo, L, p.sm_scale, p.cfg.rope_base)
    o = out[b, h].double().cpu().numpy()
    err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
    assert err <= REL_TOL, f"step {t} row ({b},{h}) L={L}: rel err {err:.3e}"
    assert abs(float(lse[b, h]) - lse_ref) <= LSE_TOL, f"step {t} row ({b},{h}): lse {float(lse[b, h])} vs {lse_ref}"
    return err


def lv_cb(p, h, kind):
    from tests import harness
    return harness.host_codebooks(p, h, kind)


def _run_parity(cfg, rows, steps, splits=(0,), only_needed_blocks=False, packed_table=True):
    """Indices and attention of `rows` against the oracle at loop steps `steps`.  only_needed_blocks: the
    indices of the loop blocks those steps read only (long contexts).  packed_table=False: the calls pass no
    packed fp16 RoPE table (the library builds it from the fp32 tables)."""
    import dataclasses

    from tests import harness
    geo = _geo(cfg)
    _say(f"[build] {cfg.name} B={cfg.B} H={cfg.H} L={cfg.L} T={cfg.T} Tc={cfg.Tc} G={cfg.G} rows={len(rows)}")
    p = harness.build_loopvq(cfg, keep=rows)
    if not packed_table:
        p = dataclasses.replace(p, rope16=None)
    blocks = sorted({t // cfg.Tc for t in steps}) if only_needed_blocks else None
    idx = {}
    for (b, h) in rows:
        _say(f"[indices] {cfg.name} row ({b},{h}) L={p.lengths[b]}")
        idx[(b, h)] = _check_indices(p, b, h, geo, blocks)
    worst = 0.0
    for ns in splits:
        for t in steps:
            lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
            _say(f"[attn] {cfg.name} step {t} num_splits={ns}")
            out, _ = harness.run_step(p, t, num_splits=ns, lse=lse)
            torch.cuda.synchronize()
            for (b, h) in rows:
                worst = max(worst, _check_row(p, t, b, h, geo, idx[(b, h)], out, lse))
    _say(f"[done] {cfg.name} worst rel err {worst:.3e}")
    return p


def test_rope_table_matches_fp64():
    import decode_attention_loopvq_amd as lvq
    cos, sin = lvq.lvq_rope_table(40000, 128, 10000.0)
    phi = lv.rope_angles(np.arange(40000), 128, 10000.0)
    # fp64 evaluation rounded once: within one fp32 rounding of the fp64 values
    assert np.abs(cos.cpu().numpy() - np.cos(phi)).max() <= 6e-8
    assert np.abs(sin.cpu().numpy() - np.sin(phi)).max() <= 6e-8


def test_rope_table_f16_layout_and_rounding():
    """Packed fp16 table: in part A [n][32][8], chunk m < 16 of position p holds cos then sin of frequencies
    4m..4m+3 and chunk 16 + m the same with the sines negated; part B [16][n][8] holds chunks m < 16 again,
    chunk-major; each value is the fp64 one rounded once to binary16."""
    import decode_attention_loopvq_amd as lvq
    n = 9000
    t = lvq.lvq_rope_table_f16(n, 128, 10000.0).cpu().numpy()          # [n * 384] fp16
    ta = t[:n * 256].reshape(n, 32, 8)
    tb = t[n * 256:].reshape(16, n, 8)
    phi = lv.rope_angles(np.arange(n), 128, 10000.0)                  # [n][64]
    for m in range(16):
        c16 = np.cos(phi[:, 4 * m:4 * m + 4]).astype(np.float16)
        s16 = np.sin(phi[:, 4 * m:4 * m + 4]).astype(np.float16)
        np.testing.assert_array_equal(ta[:, m, :4], c16)
        np.testing.assert_array_equal(ta[:, m, 4:], s16)
        np.testing.assert_array_equal(ta[:, 16 + m, :4], c16)
        np.testing.assert_array_equal(ta[:, 16 + m, 4:], -s16)
        np.testing.assert_array_equal(tb[m, :, :4], c16)
        np.testing.assert_array_equal(tb[m, :, 4:], s16)


@pytest.mark.parametrize("cb", ["bf16", "fp32"])
@pytest.mark.parametrize("T,Tc,G", [(4, 2, 16), (4, 4, 32), (32, 4, 16)])
def test_slices_bit_exact(cb, T, Tc, G):
    import decode_attention_loopvq_amd as lvq
    g = lvq.make_geom(T=T, Tc=Tc, G=G, H=3, cb_dtype=cb)
    dt = torch.bfloat16 if cb == "bf16" else torch.float32
    cbk = torch.randn((T // Tc, 3, 2, 128 * Tc // G, 256, G), device="cuda").to(dt)
    sl = lvq.lvq_slice_codebooks(g, cbk)
    host = cbk.float().cpu().numpy()
    got = sl.float().cpu().numpy()
    for t in range(T):
        for h in range(3):
            for kv in range(2):
                np.testing.assert_array_equal(got[t, h, kv], lv.step_slice(host[t // Tc, h, kv], t % Tc, Tc, G))


SMALL = [
    # two requests per workgroup with an odd batch, several tiles and a ragged tail
    loopvq_config("loopvq-b64-6k", B=5, H=2, L=700),
    # fp32 codebooks, the 1K single-request workload as stated
    loopvq_config("loopvq-b1-1k-fp32cb"),
    # T_c = 4, G = 32, 256-token window
    loopvq_config("loopvq-b8-32k", B=3, H=2, L=1500),
    # 32 loop steps, c = 4, ragged lengths from 1 token up, random page order
    loopvq_config("loopvq-deep-ragged", B=7, H=2, L=900, ragged=(1, 900)),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_decode_parity_small(cfg):
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    steps = list(range(cfg.T)) if cfg.T <= 4 else [0, 3, 4, 17, 31]
    _run_parity(cfg, rows, steps, splits=(0, 1, 3))


@pytest.mark.parametrize("T,Tc,G", [(4, 1, 4), (6, 3, 24)], ids=["tc1-g4", "tc3-g24"])
def test_encode_shapes_off_the_matrix_core_path(T, Tc, G):
    """Geometries the matrix-core encoder does not take (a codeword shorter than one 8-coordinate operand
    fragment; three loop steps per index row) go to the exact scan: every index against the oracle, and
    attention at every loop step."""
    cfg = loopvq_config("loopvq-b64-6k", B=3, H=2, L=500, T=T, Tc=Tc, G=G)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    _run_parity(cfg, rows, steps=range(cfg.T), splits=(0,))


def test_decode_edge_lengths(monkeypatch):
    """Lengths shorter than the sinks, exactly sink + window, one page, and
    pages beyond every split boundary; more splits than pages."""
    from tests import harness
    import synth.loopvq as syn
    cfg = loopvq_config("loopvq-b64-6k", B=8, H=1, L=100)
    lengths = [1, 5, 8, 72, 79, 80, 81, 100]
    monkeypatch.setattr(syn, "lengths", lambda c: lengths)
    if True:
        geo = _geo(cfg)
        rows = [(b, 0) for b in range(8)]
        p = harness.build_loopvq(cfg, keep=rows)
        idx = {(b, 0): _check_indices(p, b, 0, geo) for b in range(8)}
        for ns in (0, 1, 2, 7, 50):
            for t in range(cfg.T):
                lse = torch.empty((8, 1), dtype=torch.float32, device="cuda")
                out, _ = harness.run_step(p, t, num_splits=ns, lse=lse)
                torch.cuda.synchronize()
                for (b, h) in rows:
                    _check_row(p, t, b, h, geo, idx[(b, h)], out, lse)


def test_ragged_splits_and_pages():
    """Ragged lengths (requests of one workgroup ending in different splits, one with no index page), random
    page order, a batch that leaves the last workgroup's request group short; split counts 0, 3 and 5."""
    # lengths 3845, 220, 1997, 57, 1548, 143
    cfg = loopvq_config("loopvq-b64-6k", B=6, H=2, L=4000, ragged=(40, 4000), random_pages=True, seed=12)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    _run_parity(cfg, rows, steps=range(cfg.T), splits=(0, 3, 5))


def test_encode_decode_page():
    """The decode-time encode: one page per request (its last index page, as after every 8 generated
    tokens), written into a cleared pool, equals byte for byte the prefill encode of the same tokens and the
    oracle's indices of those tokens, for every request, head, loop block, K and V; a request without an
    index page writes nothing.  Lengths 683, 115, 454, 49, 388, 88, random page order."""
    import decode_attention_loopvq_amd as lvq
    import synth.loopvq as syn
    from tests import harness
    cfg = loopvq_config("loopvq-b64-6k", B=6, H=2, L=700, ragged=(40, 700), random_pages=True, seed=12)
    geo = _geo(cfg)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    p = harness.build_loopvq(cfg, keep=rows)
    ref = {(b, h): _check_indices(p, b, h, geo) for (b, h) in rows}
    c = p.cache
    n = torch.tensor(c.n_pages, dtype=torch.int32, device="cuda")
    last = (n - 1).clamp(min=0)
    one = (n > 0).to(torch.int32)
    tok0 = c.tok0 + last.long() * p.g.page
    pool2 = torch.zeros_like(c.pool)
    _say("[encode page] one page per request, every block, K and V")
    for kind in ("k", "v"):
        for beta, x in syn.raw_blocks(cfg, kind, "cuda"):
            lvq.lvq_encode(p.g, beta, x if kind == "k" else None, x if kind == "v" else None, p.codebooks, pool2,
                           c.page_table, last, one, 1, x_tok0=tok0)
    torch.cuda.synchronize()
    written = []
    NG = geo.NG
    for b in range(cfg.B):
        if c.n_pages[b] == 0:
            continue
        phys = int(c.page_table_host[b, c.n_pages[b] - 1])
        written.append(phys)
        assert torch.equal(pool2[phys], c.pool[phys]), f"request {b}: page {phys} differs"
        # the written page against the oracle's indices of the request's last 8 index tokens
        page = pool2[phys].cpu().numpy()                                  # [NB][H][2][8][NG]
        tau = 8 * (c.n_pages[b] - 1) + np.arange(8)[:, None]
        grp = np.arange(NG)[None, :]
        for h in range(cfg.H):
            for kv, kind in enumerate(("k", "v")):
                for beta in range(geo.NB):
                    got = page[beta, h, kv][np.arange(8)[:, None], harness.index_byte(kind, NG, grp, tau)]
                    np.testing.assert_array_equal(got, ref[(b, h)][kind][beta, -8:],
                                                  err_msg=f"request {b} head {h} {kind} block {beta}")
    rest = torch.ones(pool2.shape[0], dtype=torch.bool, device="cuda")
    rest[torch.tensor(written, device="cuda")] = False
    assert not pool2[rest].any(), "bytes written outside the encoded pages"


@pytest.mark.parametrize("name,over", [
    ("loopvq-b64-6k", dict(B=5, H=2, L=700, ragged=(1, 700), random_pages=True, seed=5)),
    ("loopvq-deep-ragged", dict(B=5, H=2, L=600, ragged=(1, 600), seed=6)),
], ids=["c8", "c4"])
def test_decode_without_packed_table(name, over):
    """lvq_decode_attn given only the fp32 cos/sin tables (no packed fp16 table: the library builds one in
    the workspace on every call), every row and the loop steps 0, 1 and the last, against the oracle."""
    cfg = loopvq_config(name, **over)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    _run_parity(cfg, rows, [0, 1, cfg.T - 1], splits=(0, 3), packed_table=False)


@pytest.mark.parametrize("packed_table", [True, False], ids=["table", "no-table"])
def test_partial_entry_points_compose(packed_table):
    """lvq_quant_partial + lvq_window_partial + splitk_lse_merge give the attention of the oracle (the
    standalone path that lvq_decode_attn fuses), with and without the packed fp16 RoPE table."""
    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = loopvq_config("loopvq-b64-6k", B=5, H=2, L=700)
    geo = _geo(cfg)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    p = harness.build_loopvq(cfg, keep=rows)
    idx = {r: _check_indices(p, r[0], r[1], geo) for r in rows}
    c = p.cache
    S = 2
    for t in range(cfg.T):
        _say(f"[partials] step {t} num_splits={S}")
        po = torch.empty((cfg.B * cfg.H, S + 1, 128), dtype=torch.float32, device="cuda")
        pl = torch.empty((cfg.B * cfg.H, S + 1), dtype=torch.float32, device="cuda")
        q = p.q[t].contiguous()
        lvq.lvq_quant_partial(p.g, t, q, c.pool, c.page_table, c.seq_len, c.max_len, p.slices, p.rope_cos,
                              p.rope_sin, p.sm_scale, po, pl, S, rope_f16=p.rope16 if packed_table else None)
        lvq.lvq_window_partial(p.g, t, q, c.seq_len, c.max_len, c.win_k, c.win_v, p.rope_cos, p.rope_sin,
                               p.sm_scale, po, pl, slot=S)
        out, lse = lvq.splitk_lse_merge(po, pl)
        torch.cuda.synchronize()
        for (b, h) in rows:
            _check_row(p, t, b, h, geo, idx[(b, h)], out.view(cfg.B, cfg.H, 128), lse.view(cfg.B, cfg.H))


def test_merge_parity():
    import decode_attention_loopvq_amd as lvq
    rng = np.random.default_rng(0)
    n, S, D = 37, 6, 128
    po = rng.standard_normal((n, S, D)).astype(np.float32)
    pl = (rng.standard_normal((n, S)) * 5).astype(np.float32)
    pl[3, :] = -np.inf
    pl[5, [0, 2, 4]] = -np.inf
    out, lse = lvq.splitk_lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for r in range(n):
        o_ref, l_ref = lv.merge([(po[r, s].astype(np.float64), float(pl[r, s])) for s in range(S)])
        if l_ref == -np.inf:
            assert lse[r] == -np.inf and not out[r].any()
            continue
        assert np.abs(out[r] - o_ref).max() <= 1e-5 * max(1.0, np.abs(o_ref).max())
        assert abs(lse[r] - l_ref) <= 1e-5 * max(1.0, abs(l_ref))


def test_full_b64_6k_sampled():
    """The serving-scale workload at full size in the benchmark's launch
    configuration, checked on sampled rows."""
    cfg = loopvq_config("loopvq-b64-6k")
    rows = [(0, 0), (37, 9), (63, 15)]
    _run_parity(cfg, rows, steps=range(cfg.T), splits=(0,))


def test_full_b1_1k():
    cfg = loopvq_config("loopvq-b1-1k-fp32cb")
    _run_parity(cfg, [(0, 0)], steps=range(cfg.T), splits=(0,))


def test_full_b8_32k_sampled():
    """The 0.25-bit long-context workload at full size (batch 8, 16 heads, 32768 tokens, 256-token recent
    window, T_c = 4, G = 32), every loop step, checked on sampled rows: indices and attention."""
    cfg = loopvq_config("loopvq-b8-32k")
    _run_parity(cfg, [(0, 0), (7, 15)], steps=range(cfg.T), splits=(0,), only_needed_blocks=True)


def test_full_deep_ragged_sampled():
    """The deep-loop ragged batch at full size (batch 128, 8 heads, 32 loop steps, lengths log-uniform in
    [1024, 16384], random page order), loop steps 0, 15 and 31, checked on the longest and the shortest
    request: indices of the blocks those steps read, and attention."""
    import synth.loopvq as syn
    cfg = loopvq_config("loopvq-deep-ragged")
    lengths = syn.lengths(cfg)
    rows = [(int(np.argmax(lengths)), 0), (int(np.argmin(lengths)), cfg.H - 1)]
    _run_parity(cfg, rows, steps=[0, 15, 31], splits=(0,), only_needed_blocks=True)


def test_channel_permutation():
    """A cache kept in a permuted channel order that maps RoPE pairs to pairs (LoopVQ page, technical novelty:
    TaSQ+LoopVQ's channel permutation P; a random permutation of the 64 frequencies): the synthetic keys,
    values and queries taken as the stored channels, RoPE tables from lvq_rope_table_perm.  Every step against
    the oracle's decode_step_permuted, whose query and output are in the original channel order."""
    import dataclasses

    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = loopvq_config("loopvq-b64-6k", B=3, H=2, L=700)
    geo = _geo(cfg)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    p = harness.build_loopvq(cfg, keep=rows)
    pi = np.random.default_rng(7).permutation(64)
    perm = np.concatenate([pi, pi + 64]).astype(np.int32)
    assert lvq.lvq_channel_perm_check(p.g, perm) == 0
    cos, sin, f16 = lvq.lvq_rope_table_perm(p.g, perm, p.rope_cos.shape[0], cfg.rope_base)
    pp = dataclasses.replace(p, rope_cos=cos, rope_sin=sin, rope16=f16)
    idx = {r: _check_indices(p, r[0], r[1], geo) for r in rows}
    for t in range(cfg.T):
        lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
        out, _ = harness.run_step(pp, t, lse=lse)
        torch.cuda.synchronize()
        for (b, h) in rows:
            q_orig = np.empty(cfg.D)
            q_orig[perm] = p.q[t, b, h].float().cpu().numpy().astype(np.float64)
            o_ref, l_ref = lv.decode_step_permuted(q_orig, t, p.raw[("k", b, h)], p.raw[("v", b, h)],
                                                   idx[(b, h)]["k"], idx[(b, h)]["v"], lv_cb(p, h, "k"),
                                                   lv_cb(p, h, "v"), geo, p.lengths[b], p.sm_scale, cfg.rope_base,
                                                   perm)
            o = out[b, h].double().cpu().numpy()
            err = np.abs(o - o_ref[perm]).max() / np.abs(o_ref).max()
            assert err <= REL_TOL, f"step {t} row ({b},{h}): rel err {err:.3e}"
            assert abs(float(lse[b, h]) - l_ref) <= LSE_TOL, (t, b, h)


def test_check_pages():
    """lvq_check_pages, the debug check of what the kernels take on trust: a valid cache gives no finding;
    page ids outside [0, pool pages) planted inside requests' index ranges are each counted, with the lowest
    such request, while entries past a request's range are not read; lengths outside [0, max_len] are
    counted."""
    import decode_attention_loopvq_amd as lvq
    from decode_attention_loopvq_amd.layout import LoopVQCache
    g = lvq.make_geom(H=2)
    lengths = [700, 75, 300, 1, 512]
    c = LoopVQCache(g, lengths, device="cuda")
    P = c.pool.shape[0]
    assert lvq.lvq_check_pages(g, c.page_table, c.seq_len, c.max_len, P) == (0, -1, 0)
    pt = c.page_table.clone()
    # pt_stride wider than needed, the spare columns holding garbage that must not be read
    wide = torch.full((c.B, pt.shape[1] + 5), -7, dtype=torch.int32, device="cuda")
    wide[:, :pt.shape[1]] = pt
    assert lvq.lvq_check_pages(g, wide, c.seq_len, c.max_len, P) == (0, -1, 0)
    # request 1 has no index page (75 tokens): a bad entry in its row is outside its range
    wide[1, 0] = P + 3
    wide[2, c.n_pages[2] - 1] = P                   # last index page of request 2
    wide[4, 0] = -1                                 # first index page of request 4
    wide[4, 3] = 1 << 30
    wide[0, c.n_pages[0]] = -5                      # just past request 0's range: not read
    assert lvq.lvq_check_pages(g, wide, c.seq_len, c.max_len, P) == (3, 2, 0)
    # lengths past max_len are clamped by the kernels and reported here; negative ones too
    sl = c.seq_len.clone()
    sl[3] = c.max_len + 9
    sl[0] = -4
    assert lvq.lvq_check_pages(g, c.page_table, sl, c.max_len, P) == (0, -1, 2)
    # a pool smaller than the table's ids
    assert lvq.lvq_check_pages(g, c.page_table, c.seq_len, c.max_len, 1)[0] == sum(c.n_pages) - 1


def test_request_order_sorts_by_length():
    """lvq_request_order against a stable host sort of the clamped lengths (longest first, ties by index)."""
    import decode_attention_loopvq_amd as lvq
    rng = np.random.default_rng(21)
    for B, max_len in ((1, 100), (7, 900), (64, 6144), (255, 5000), (1000, 70000)):
        lens = rng.integers(-3, max_len + 50, size=B).astype(np.int32)
        lens[: B // 3] = lens[0]                       # runs of equal lengths
        _say(f"[order] B={B} max_len={max_len}")
        order = lvq.lvq_request_order(torch.from_numpy(lens).cuda(), max_len).cpu().numpy()
        clamped = np.clip(lens, 0, max_len)
        expect = np.lexsort((np.arange(B), -clamped))  # primary key: length descending; then index
        np.testing.assert_array_equal(order, expect)
    lens = np.full(37, 300, dtype=np.int32)
    order = lvq.lvq_request_order(torch.from_numpy(lens).cuda(), 300).cpu().numpy()
    np.testing.assert_array_equal(order, np.arange(37))


@pytest.mark.parametrize("name,over,splits", [
    ("loopvq-b64-6k", dict(B=9, H=2, L=3000, ragged=(40, 3000), random_pages=True, seed=31), (0, 3)),
    ("loopvq-deep-ragged", dict(B=7, H=2, L=900, ragged=(1, 900)), (0, 2)),
    ("loopvq-b1-1k-fp32cb", dict(B=5, H=2, L=1024, ragged=(30, 1024)), (0, 2)),
], ids=["bf16-c8", "bf16-c4", "fp32"])
def test_order_does_not_change_the_output(name, over, splits):
    """The grouping of requests into workgroups changes no bit of the output: no order, the length order and
    a random permutation (every path: the split kernels for bf16 codebooks with c = 8 and c = 4, and fp32)."""
    import decode_attention_loopvq_amd as lvq
    from tests import harness
    cfg = loopvq_config(name, **over)
    _say(f"[build] {cfg.name} B={cfg.B} ragged order invariance")
    p = harness.build_loopvq(cfg, keep=[])
    c = p.cache
    by_len = lvq.lvq_request_order(c.seq_len, c.max_len)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(cfg.B).astype(np.int32)).cuda()
    for ns in splits:
        for t in (0, cfg.T - 1):
            _say(f"[order] {cfg.name} step {t} num_splits={ns}")
            ref, lse_ref = harness.run_step(p, t, num_splits=ns,
                                            lse=torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda"))
            for order in (by_len, perm):
                out, lse = harness.run_step(p, t, num_splits=ns, order=order,
                                            lse=torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda"))
                torch.cuda.synchronize()
                assert torch.equal(out, ref) and torch.equal(lse, lse_ref), f"step {t} splits {ns}"
