"""Pins for the LoopVQ oracle: figures the LoopVQ page states, worked examples,
closed forms, invariants and brute force on tiny inputs.  CPU only."""

import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, logsumexp

from oracle import loopvq as lv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(x):
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Accounting
# ---------------------------------------------------------------------------

def test_bits_per_element_matches_page():
    g = _golden("accounting.json")["loopvq_bits_per_element"]
    for G, bits in zip(g["G"], g["bits"]):
        assert lv.bits_per_element(G) == bits


def test_read_reduction_matches_page():
    """Each loop step reads NG index bytes per token for K (and again for V)
    where bf16 reads 2*D bytes: 2D/NG = 8x at G=16 and 16x at G=32 with T_c=4."""
    g = _golden("accounting.json")["loopvq_read_reduction_vs_bf16"]
    for G, red in zip(g["G"], g["reduction"]):
        geo = lv.Geometry(D=g["D"], T=g["T"], Tc=g["Tc"], G=G)
        assert 2 * geo.D / geo.NG == red


def test_geometry_rejects_tc_not_dividing():
    with pytest.raises(ValueError):
        lv.Geometry(D=128, T=4, Tc=3, G=16)
    with pytest.raises(ValueError):
        lv.Geometry(D=128, T=6, Tc=3, G=16)


# ---------------------------------------------------------------------------
# Loop-axis grouping and dequant
# ---------------------------------------------------------------------------

def test_couple_worked_example():
    g = _golden("loopvq_grouping_example.json")
    x = np.array(g["x"], dtype=np.float64)[:, None, :]   # [T][N=1][D]
    Tc, G = g["Tc"], g["G"]
    for beta, key in ((0, "block0"), (1, "block1")):
        z = lv.couple(x[beta * Tc:(beta + 1) * Tc], G)
        np.testing.assert_array_equal(z[0], np.array(g["coupled"][key], dtype=np.float64))
    E = np.arange(2 * 3 * G, dtype=np.float64).reshape(2, 3, G)   # [NG][K][G]
    for t in range(g["T"]):
        cols = g["slice_coordinates"]["t%d" % t]
        np.testing.assert_array_equal(lv.step_slice(E, t % Tc, Tc, G), E[:, :, cols])


@pytest.mark.parametrize("Tc,G", [(1, 16), (2, 16), (4, 16), (4, 32), (2, 4)])
def test_couple_matches_transpose_view(Tc, G):
    """The coupled vector of group g is the [T_c][c] block of (step, channel)
    values laid out channel-major, step-minor: a transpose then a reshape."""
    rng = np.random.default_rng(0)
    D, N = 128 if G > 4 else 8, 37
    c = G // Tc
    x = rng.standard_normal((Tc, N, D))
    z = lv.couple(x, G)
    ref = x.reshape(Tc, N, D // c, c).transpose(1, 2, 3, 0).reshape(N, D // c, G)
    np.testing.assert_array_equal(z, ref)


def test_tc1_is_per_step_vq():
    """T_c = 1 is the per-loop-step VQ the page compares against: contiguous
    G-channel sub-vectors of one step."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 20, 128))
    z = lv.couple(x, 16)
    np.testing.assert_array_equal(z, x[0].reshape(20, 8, 16))


@pytest.mark.parametrize("T,Tc,G", [(4, 2, 16), (4, 4, 32), (8, 4, 16), (4, 1, 8)])
def test_lossless_codebook_round_trip(T, Tc, G):
    """A codebook whose entries are the data's own coupled vectors: every token
    encodes to its own entry at distance 0 and dequant returns the bf16 input
    of every loop step exactly."""
    rng = np.random.default_rng(2)
    geo = lv.Geometry(D=128, T=T, Tc=Tc, G=G)
    N = 200
    raw = _bf16(rng.standard_normal((T, N, 128)))          # [T][N][D]
    for beta in range(geo.NB):
        xb = raw[beta * Tc:(beta + 1) * Tc]
        z = lv.couple(xb, G)                                 # [N][NG][G]
        E = np.zeros((geo.NG, 256, G))
        E[:, :N, :] = np.transpose(z, (1, 0, 2))
        E[:, N:, :] = 1e3                                    # far-away filler entries
        idx = lv.encode_block(xb, E, G)
        np.testing.assert_array_equal(idx, np.tile(np.arange(N)[:, None], (1, geo.NG)))
        for m in range(Tc):
            np.testing.assert_array_equal(lv.dequant_step(idx, E, m, Tc, G), xb[m])


# ---------------------------------------------------------------------------
# Nearest codeword: brute force
# ---------------------------------------------------------------------------

def _brute_nearest(z, E):
    best, best_d = None, None
    for r in range(len(E)):
        d = 0.0
        for a, b in zip(z, E[r]):
            d += (a - b) * (a - b)
        if best_d is None or d < best_d:
            best, best_d = r, d
    return best


@pytest.mark.parametrize("K,G", [(2, 1), (4, 2), (8, 4), (5, 3)])
def test_nearest_codeword_brute_force(K, G):
    rng = np.random.default_rng(K * 10 + G)
    z = rng.integers(-3, 4, size=(60, G)).astype(np.float64)   # small integers: many exact ties
    E = rng.integers(-3, 4, size=(K, G)).astype(np.float64)
    idx, d = lv.nearest_codeword(z, E)
    for j in range(len(z)):
        assert idx[j] == _brute_nearest(list(z[j]), [list(e) for e in E])
        assert d[j, idx[j]] == min(sum((a - b) ** 2 for a, b in zip(z[j], e)) for e in E)


@pytest.mark.parametrize("N,chunk", [(4096 + 1000, 4096), (9000, 4096), (50, 7)])
def test_nearest_codeword_across_row_chunks(N, chunk):
    """Rows are scanned in chunks of `chunk`; every row of every chunk, the partial last one
    included, gets its own brute-force nearest codeword and its full distance row."""
    rng = np.random.default_rng(N)
    G, K = 3, 12
    z = rng.integers(-3, 4, size=(N, G)).astype(np.float64)
    E = rng.integers(-3, 4, size=(K, G)).astype(np.float64)
    idx, d = lv.nearest_codeword(z, E, chunk=chunk)
    E_list = [list(e) for e in E]
    for j in range(N):
        zj = list(z[j])
        assert idx[j] == _brute_nearest(zj, E_list)
        for r in range(K):
            assert d[j, r] == sum((a - b) ** 2 for a, b in zip(zj, E_list[r]))


def test_duplicate_codewords_pick_lowest_index():
    E = np.array([[1.0, 1.0], [0.0, 0.0], [0.0, 0.0], [5.0, 5.0]])
    idx, _ = lv.nearest_codeword(np.array([[0.1, -0.1], [0.0, 0.0]]), E)
    assert list(idx) == [1, 1]


def test_exhaustive_tiny_grid():
    """Every z on a tiny integer grid against a fixed codebook, brute force."""
    E = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [0.5, 0.5]])
    zs = np.array(list(itertools.product(np.arange(-1, 2.5, 0.5), repeat=2)))
    idx, _ = lv.nearest_codeword(zs, E)
    for j, z in enumerate(zs):
        assert idx[j] == _brute_nearest(list(z), [list(e) for e in E])


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def _rope_complex(x, p, base=10000.0):
    """Independent form: channel pairs (i, i + D/2) as the complex number
    x_i + 1j x_{i+D/2}, multiplied by e^{1j p theta_i}, theta_i = base^(-2i/D)."""
    D = len(x)
    out = [0.0] * D
    for i in range(D // 2):
        theta = base ** (-2.0 * i / D)
        w = complex(x[i], x[i + D // 2]) * cmath.exp(1j * p * theta)
        out[i], out[i + D // 2] = w.real, w.imag
    return np.array(out)


def test_rope_identity_at_zero():
    x = np.random.default_rng(3).standard_normal((4, 128))
    np.testing.assert_array_equal(lv.apply_rope(x, np.zeros(4)), x)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 128))
    pos = np.array([1, 7, 100, 6143, 32767])
    y = lv.apply_rope(x, pos)
    for j in range(5):
        np.testing.assert_allclose(y[j], _rope_complex(list(x[j]), int(pos[j])), rtol=0, atol=1e-10)


def test_rope_known_frequencies():
    """theta_0 = 1 (pair 0 turns by p radians) and theta_{D/4} = base^(-1/2) = 0.01."""
    phi = lv.rope_angles(np.array([1.0, 3.0]), 128)
    assert phi[0, 0] == 1.0 and phi[1, 0] == 3.0
    assert abs(phi[0, 32] - 0.01) < 1e-17
    x = np.zeros((1, 128))
    x[0, 0] = 1.0
    y = lv.apply_rope(x, np.array([2]))
    assert abs(y[0, 0] - math.cos(2.0)) < 1e-15 and abs(y[0, 64] - math.sin(2.0)) < 1e-15


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for pq, pk in [(10, 3), (500, 200), (6000, 5990)]:
        rq = lv.apply_rope(q[None], np.array([pq]))[0]
        rk = lv.apply_rope(k[None], np.array([pk]))[0]
        assert abs(np.linalg.norm(rk) - np.linalg.norm(k)) < 1e-12
        rq2 = lv.apply_rope(q[None], np.array([pq - pk]))[0]
        assert abs(rq @ rk - rq2 @ k) < 1e-9


# ---------------------------------------------------------------------------
# Attention and merge
# ---------------------------------------------------------------------------

def test_attention_q_zero_gives_mean():
    rng = np.random.default_rng(6)
    k, v = rng.standard_normal((50, 16)), rng.standard_normal((50, 16))
    o, lse = lv.attention(np.zeros(16), k, v, 0.3)
    np.testing.assert_allclose(o, v.mean(0), atol=1e-14)
    assert abs(lse - math.log(50)) < 1e-14


def test_attention_single_token_and_dominant_logit():
    rng = np.random.default_rng(7)
    k, v = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    o, _ = lv.attention(rng.standard_normal(16), k, v, 1.0)
    np.testing.assert_allclose(o, v[0], atol=1e-15)
    k = np.zeros((30, 16))
    k[17, 0] = 1.0
    v = rng.standard_normal((30, 16))
    q = np.zeros(16)
    q[0] = 1000.0
    o, _ = lv.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, v[17], atol=1e-12)
    o_neg, _ = lv.attention(-q, k, v, 1.0)     # the sign of the score matters
    np.testing.assert_allclose(o_neg, np.delete(v, 17, 0).mean(0), atol=1e-12)


def test_attention_two_token_logistic_and_lse():
    rng = np.random.default_rng(8)
    a, b, scale = 1.7, -0.6, 0.8
    k = np.zeros((2, 8))
    k[0, 2] = a
    q = np.zeros(8)
    q[2] = b
    v = rng.standard_normal((2, 8))
    o, lse = lv.attention(q, k, v, scale)
    w0 = expit(scale * a * b)
    np.testing.assert_allclose(o, w0 * v[0] + (1 - w0) * v[1], atol=1e-15)
    k = rng.standard_normal((40, 8))
    _, lse = lv.attention(q, k, v[[0] * 40], scale)
    assert abs(lse - logsumexp(scale * (k @ q))) < 1e-12


def test_merge_equals_unsplit():
    rng = np.random.default_rng(9)
    k, v = rng.standard_normal((300, 32)), rng.standard_normal((300, 32))
    q = rng.standard_normal(32) * 3
    o_ref, lse_ref = lv.attention(q, k, v, 0.5)
    for trial in range(20):
        cuts = np.sort(rng.integers(0, 301, size=rng.integers(1, 8)))
        bounds = [0] + list(cuts) + [300]
        parts = [lv.attention(q, k[a:b], v[a:b], 0.5) for a, b in zip(bounds[:-1], bounds[1:])]
        o, lse = lv.merge(parts)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        assert abs(lse - lse_ref) < 1e-12


def test_merge_empty_splits_contribute_nothing():
    rng = np.random.default_rng(10)
    k, v = rng.standard_normal((10, 8)), rng.standard_normal((10, 8))
    q = rng.standard_normal(8)
    ref = lv.attention(q, k, v, 1.0)
    empty = lv.attention(q, k[:0], v[:0], 1.0)
    assert empty[1] == -np.inf
    o, lse = lv.merge([empty, ref, empty])
    np.testing.assert_allclose(o, ref[0], atol=1e-15)
    assert lse == ref[1]


def test_separate_softmax_without_merge_differs():
    """Negative control: averaging per-split normalised outputs is not attention."""
    rng = np.random.default_rng(11)
    k, v = rng.standard_normal((100, 16)), rng.standard_normal((100, 16))
    q = rng.standard_normal(16) * 2
    o_ref, _ = lv.attention(q, k, v, 1.0)
    a, b = lv.attention(q, k[:30], v[:30], 1.0), lv.attention(q, k[30:], v[30:], 1.0)
    assert np.abs((a[0] + b[0]) / 2 - o_ref).max() > 1e-3


# ---------------------------------------------------------------------------
# Cache regions and a whole decode step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 5, 8, 9, 71, 72, 79, 80, 81, 1024, 6144, 32768])
def test_cache_regions(L):
    for W in (64, 256):
        geo = lv.Geometry(D=128, T=4, Tc=2, G=16, window=W)
        n, lo, hi = lv.cache_regions(L, geo)
        assert lo == 8 and hi == 8 + 8 * n
        recent = L - hi
        if L >= 8 + W:
            assert W <= recent < W + 8
        else:
            assert n == 0
    n, _, _ = lv.cache_regions(1024, lv.Geometry(D=128, T=4, Tc=2, G=16))
    assert n == 119


def _tiny_problem(seed, L, D=8, T=4, Tc=2, G=4, K=6, sink=2, window=3, page=2):
    rng = np.random.default_rng(seed)
    geo = lv.Geometry(D=D, T=T, Tc=Tc, G=G, K=K, sink=sink, window=window, page=page)
    raw_k = _bf16(rng.standard_normal((L, T, D)))
    raw_v = _bf16(rng.standard_normal((L, T, D)))
    E_k = rng.standard_normal((geo.NB, geo.NG, K, G))
    E_v = rng.standard_normal((geo.NB, geo.NG, K, G))
    return geo, raw_k, raw_v, E_k, E_v, rng


@pytest.mark.parametrize("seed,L", [(0, 9), (1, 14), (2, 4), (3, 20)])
def test_decode_step_brute_force(seed, L):
    """Pure-Python brute force of a whole decode step on a tiny cache: nearest
    codeword by enumeration, keys rebuilt coordinate by coordinate, complex
    RoPE, math.exp softmax."""
    geo, raw_k, raw_v, E_k, E_v, rng = _tiny_problem(seed, L)
    q = rng.standard_normal(geo.D)
    idx_k = lv.encode_request(raw_k, E_k, geo, L)
    idx_v = lv.encode_request(raw_v, E_v, geo, L)
    _, q_lo, q_hi = lv.cache_regions(L, geo)
    c = geo.c
    for t in range(geo.T):
        beta, m = t // geo.Tc, t % geo.Tc
        keys, vals = [], []
        for p in range(L):
            if q_lo <= p < q_hi:
                kk, vv = [0.0] * geo.D, [0.0] * geo.D
                for g in range(geo.NG):
                    for E, dst, raw in ((E_k, kk, raw_k), (E_v, vv, raw_v)):
                        z = [raw[p, beta * geo.Tc + mm, g * c + i] for i in range(c) for mm in range(geo.Tc)]
                        r = _brute_nearest(z, [list(e) for e in E[beta, g]])
                        for i in range(c):
                            dst[g * c + i] = E[beta, g, r, i * geo.Tc + m]
            else:
                kk, vv = list(raw_k[p, t]), list(raw_v[p, t])
            keys.append(_rope_complex(kk, p))
            vals.append(vv)
        s = [0.7 * sum(a * b for a, b in zip(q, kk)) for kk in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        o_ref = [sum(w[p] * vals[p][d] for p in range(L)) / sum(w) for d in range(geo.D)]
        o, lse = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.7)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        assert abs(lse - (mx + math.log(sum(w)))) < 1e-12


@pytest.mark.parametrize("L", [3, 40, 61])
def test_two_part_split_matches_one_pass(L):
    geo, raw_k, raw_v, E_k, E_v, rng = _tiny_problem(7, L)
    q = rng.standard_normal(geo.D)
    idx_k = lv.encode_request(raw_k, E_k, geo, L)
    idx_v = lv.encode_request(raw_v, E_v, geo, L)
    for t in range(geo.T):
        a = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.5)
        b = lv.decode_step_two_part(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.5)
        np.testing.assert_allclose(a[0], b[0], atol=1e-13)
        assert abs(a[1] - b[1]) < 1e-12


def test_lossless_cache_equals_textbook_attention():
    """With codebooks that hold the data's own coupled vectors, the decode step
    equals plain softmax attention on the raw data rotated by complex RoPE."""
    rng = np.random.default_rng(12)
    geo = lv.Geometry(D=128, T=4, Tc=2, G=16)
    L = 8 + 64 + 8 * 20 + 5
    raw_k = _bf16(rng.standard_normal((L, 4, 128)))
    raw_v = _bf16(rng.standard_normal((L, 4, 128)))
    _, q_lo, q_hi = lv.cache_regions(L, geo)
    E = {}
    for name, raw in (("k", raw_k), ("v", raw_v)):
        E[name] = np.full((geo.NB, geo.NG, 256, 16), 1e3)
        for beta in range(geo.NB):
            z = lv.couple(np.transpose(raw[q_lo:q_hi, 2 * beta:2 * beta + 2], (1, 0, 2)), 16)
            E[name][beta, :, :q_hi - q_lo] = np.transpose(z, (1, 0, 2))
    idx_k = lv.encode_request(raw_k, E["k"], geo, L)
    idx_v = lv.encode_request(raw_v, E["v"], geo, L)
    q = rng.standard_normal(128)
    for t in range(4):
        o, lse = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E["k"], E["v"], geo, L, 1 / math.sqrt(128))
        keys = np.array([_rope_complex(list(raw_k[p, t]), p) for p in range(L)])
        s = keys @ q / math.sqrt(128)
        w = np.exp(s - s.max())
        np.testing.assert_allclose(o, (w @ raw_v[:, t]) / w.sum(), atol=1e-12)
        assert abs(lse - logsumexp(s)) < 1e-12



# ---------------------------------------------------------------------------
# Channel permutation P (TaSQ+LoopVQ plumbing)
# ---------------------------------------------------------------------------

def _perm_problem(seed, geo, L):
    rng = np.random.default_rng(seed)
    raw_k = _bf16(rng.standard_normal((L, geo.T, geo.D)))
    raw_v = _bf16(rng.standard_normal((L, geo.T, geo.D)))
    E_k = _bf16(rng.standard_normal((geo.NB, geo.NG, 256, geo.G)))
    E_v = _bf16(rng.standard_normal((geo.NB, geo.NG, 256, geo.G)))
    q = rng.standard_normal(geo.D)
    return rng, raw_k, raw_v, E_k, E_v, q


def test_permuted_decode_with_identity_is_decode_step():
    """decode_step_permuted with the identity permutation is decode_step (up to the last bit of the BLAS
    products, which may depend on array layout)."""
    geo = lv.Geometry(D=128, T=4, Tc=2, G=16)
    L = 8 + 64 + 8 * 12 + 3
    _, raw_k, raw_v, E_k, E_v, q = _perm_problem(21, geo, L)
    idx_k, idx_v = lv.encode_request(raw_k, E_k, geo, L), lv.encode_request(raw_v, E_v, geo, L)
    for t in range(geo.T):
        o1, l1 = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.09, 10000.0)
        o2, l2 = lv.decode_step_permuted(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.09, 10000.0,
                                         np.arange(geo.D))
        np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
        assert abs(l1 - l2) <= 1e-13 * abs(l1)


@pytest.mark.parametrize("T,Tc,G", [(4, 2, 16), (4, 4, 32)])
def test_permuted_cache_of_whole_groups_is_the_same_attention(T, Tc, G):
    """A permutation that moves whole index groups and maps RoPE pairs to pairs (stored group g' holds original
    group s(g'), stored group g' + NG/2 original group s(g') + NG/2, s not an involution): storing the cache
    in that order (raw values, codebooks and indices moved with their groups) and the query in the original
    order gives the unpermuted attention (up to the last bit of the BLAS products)."""
    geo = lv.Geometry(D=128, T=T, Tc=Tc, G=G)
    L = 8 + 64 + 8 * 12 + 3
    rng, raw_k, raw_v, E_k, E_v, q = _perm_problem(22, geo, L)
    idx_k, idx_v = lv.encode_request(raw_k, E_k, geo, L), lv.encode_request(raw_v, E_v, geo, L)
    c, NG = geo.c, geo.NG
    half = NG // 2
    lo = rng.permutation(half)
    while np.all(lo[lo] == np.arange(half)):            # not an involution, so a transposed use differs
        lo = rng.permutation(half)
    sigma = np.concatenate([lo, lo + half])             # stored group -> original group
    perm = (sigma[:, None] * c + np.arange(c)[None, :]).reshape(-1)   # stored channel -> original channel
    assert np.array_equal(perm[64:], perm[:64] + 64)
    st = dict(raw_k=raw_k[:, :, perm], raw_v=raw_v[:, :, perm], E_k=E_k[:, sigma], E_v=E_v[:, sigma],
              idx_k=idx_k[:, :, sigma], idx_v=idx_v[:, :, sigma])
    for t in range(geo.T):
        o1, l1 = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.09, 10000.0)
        o2, l2 = lv.decode_step_permuted(q, t, st["raw_k"], st["raw_v"], st["idx_k"], st["idx_v"], st["E_k"],
                                         st["E_v"], geo, L, 0.09, 10000.0, perm)
        np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
        assert abs(l1 - l2) <= 1e-13 * abs(l1)


# ---------------------------------------------------------------------------
# Key scale stream (TaSQ+LoopVQ plumbing)
# ---------------------------------------------------------------------------

def _scale_case(seed=21, L=150):
    geo = lv.Geometry(D=16, T=4, Tc=2, G=8, K=16, sink=8, window=16, page=8)
    rng = np.random.default_rng(seed)
    raw_k = rng.standard_normal((L, geo.T, geo.D))
    raw_v = rng.standard_normal((L, geo.T, geo.D))
    E_k = rng.standard_normal((geo.NB, geo.NG, geo.K, geo.G))
    E_v = rng.standard_normal((geo.NB, geo.NG, geo.K, geo.G))
    idx_k = lv.encode_request(raw_k, E_k, geo, L)
    idx_v = lv.encode_request(raw_v, E_v, geo, L)
    q = rng.standard_normal(geo.D)
    return geo, rng, raw_k, raw_v, E_k, E_v, idx_k, idx_v, q


def test_uniform_key_scale_equals_scaled_codebook():
    """A scale alpha on every paged key token equals multiplying the key codebooks by alpha
    (reconstruction is linear in the codeword), for every loop step."""
    geo, rng, raw_k, raw_v, E_k, E_v, idx_k, idx_v, q = _scale_case()
    L = raw_k.shape[0]
    n_tok = idx_k.shape[1]
    for alpha in (0.37, 2.5):
        sc = np.full((n_tok, geo.T), alpha)
        for t in range(geo.T):
            o1, l1 = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.3, k_scales=sc)
            o2, l2 = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, alpha * E_k, E_v, geo, L, 0.3)
            np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
            assert abs(l1 - l2) < 1e-12


def test_zero_key_scales_give_uniform_paged_logits():
    """Zero scales make every paged logit 0: the output is the closed form
    (sum_paged v + sum_bf16 e^{s_j} v_j) / (n_paged + sum_bf16 e^{s_j})."""
    geo, rng, raw_k, raw_v, E_k, E_v, idx_k, idx_v, q = _scale_case(seed=5, L=131)
    L = raw_k.shape[0]
    _, q_lo, q_hi = lv.cache_regions(L, geo)
    sc = np.zeros((idx_k.shape[1], geo.T))
    t = 3
    o, lse = lv.decode_step(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, 0.5, k_scales=sc)
    v = lv.assemble_step(t, raw_v, idx_v, E_v, geo, L)
    bf = np.r_[0:q_lo, q_hi:L]
    ang = lv.rope_angles(bf, geo.D)
    kb = raw_k[bf, t, :]
    half = geo.D // 2
    rot = np.concatenate([kb[:, :half] * np.cos(ang) - kb[:, half:] * np.sin(ang),
                          kb[:, half:] * np.cos(ang) + kb[:, :half] * np.sin(ang)], axis=1)
    e = np.exp(0.5 * rot @ q)
    want = (v[q_lo:q_hi].sum(axis=0) + e @ v[bf]) / ((q_hi - q_lo) + e.sum())
    np.testing.assert_allclose(o, want, rtol=1e-10, atol=1e-12)
    assert abs(lse - np.log((q_hi - q_lo) + e.sum())) < 1e-10
