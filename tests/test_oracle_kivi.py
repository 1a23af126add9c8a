"""Pins for the KIVI oracle: the KIVI page's stated figures, hand-worked
quantizer cases, bounds, the residual-window rules and the joint softmax.  CPU only."""

import json
import math
import os

import numpy as np
import pytest

from oracle import kivi as kv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_memory_formula_matches_page():
    g = _golden("accounting.json")["kivi_memory_formula"]
    per_tok = kv.kv_cache_bytes(g["n_layer"], g["h_kv"], g["d_head"], 1, g["bytes_per_elem"])
    assert per_tok == g["bytes_per_token"]
    assert kv.kv_cache_bytes(g["n_layer"], g["h_kv"], g["d_head"], 4096, 2) == g["bytes_4k_request"]
    assert 16 * kv.kv_cache_bytes(g["n_layer"], g["h_kv"], g["d_head"], 4096, 2) == g["bytes_4k_batch16"]


def test_bytes_per_element_matches_page():
    g = _golden("accounting.json")["kivi_bytes_per_element"]
    assert kv.bytes_per_element(g["bits"], g["group"], g["param_bytes"]) == g["bytes"]


@pytest.mark.parametrize("case", _golden("kivi_quantizer_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_worked_groups(case):
    x = np.array(case["x"], dtype=np.float16)
    s, z = kv.group_params(x)
    assert float(s) == case["s"] and float(z) == case["z"]
    if "s_hex" in case:
        assert int(np.array([s], dtype=np.float16).view(np.uint16)[0]) == int(case["s_hex"], 16)
    codes = kv.quantize(x, s, z)
    assert codes.tolist() == case["codes"]
    assert kv.dequantize(codes, s, z).tolist() == case["x_hat"]


def _groups(seed, n=2000, size=32, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, size)) * scale).astype(np.float16)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("scale", [1.0, 20.0, 1e-3])
def test_codes_in_range_and_error_bound(scale, bits):
    """Every code lies in [0, 2^b - 1]; |x - x_hat| <= s/2 + s|z - z_exact| + a few
    ulps, where z_exact = -min/s before fp16 rounding."""
    for x in _groups(1, scale=scale):
        s, z = kv.group_params(x, bits)
        q = kv.quantize(x, s, z, bits)
        assert q.min() >= 0 and q.max() <= 2 ** bits - 1
        xh = kv.dequantize(q, s, z).astype(np.float64)
        xf = x.astype(np.float64)
        z_exact = -xf.min() / float(s)
        bound = float(s) / 2 + float(s) * abs(float(z) - z_exact) + 4e-7 * (abs(xf).max() + float(s))
        assert np.abs(xf - xh).max() <= bound


@pytest.mark.parametrize("bits", [2, 4])
def test_end_points_map_to_extreme_codes(bits):
    """min -> 0 and max -> 2^b - 1 unless fp16 rounding of z moves the value across a
    rounding boundary (checked by recomputing with the exact z)."""
    top = 2 ** bits - 1
    n_checked = n_top = 0
    for x in _groups(2):
        s, z = kv.group_params(x, bits)
        q = kv.quantize(x, s, z, bits)
        xf = x.astype(np.float32)
        u_min = np.float32(np.float32(xf.min()) / np.float32(s)) + np.float32(z)
        u_max = np.float32(np.float32(xf.max()) / np.float32(s)) + np.float32(z)
        if abs(u_min) < 0.49:
            assert q[np.argmin(xf)] == 0
            n_checked += 1
        if abs(u_max - top) < 0.49:
            assert q[np.argmax(xf)] == top
            n_top += 1
    assert n_checked > 1500 and n_top > 1500


@pytest.mark.parametrize("bits", [2, 4])
def test_exactly_representable_group_is_lossless(bits):
    rng = np.random.default_rng(3)
    top = 2 ** bits - 1
    for _ in range(200):
        s = float(2.0 ** rng.integers(-4, 4))
        a = float(rng.integers(-8, 8)) * s     # min on the grid so z = -a/s is an integer
        levels = np.arange(top + 1)
        x = (a + s * rng.choice(levels, size=32)).astype(np.float16)
        x[0], x[1] = a, a + top * s          # make min and max exact
        s16, z16 = kv.group_params(x, bits)
        q = kv.quantize(x, s16, z16, bits)
        np.testing.assert_array_equal(kv.dequantize(q, s16, z16), x.astype(np.float32))


def test_four_bit_hand_case():
    """Worked by hand: x = 0, 1, ..., 15 (fp16) over a 16-value group: max - min = 15, so
    s = 15 / 15 = 1, z = -0 / 1 = 0 and each value is its own code; x = -1.5 and 6 give
    s = 7.5 / 15 = 0.5, z = 1.5 / 0.5 = 3, and x = 0 -> 0 / 0.5 + 3 = 3."""
    x = np.arange(16, dtype=np.float16)
    s, z = kv.group_params(x, 4)
    assert float(s) == 1.0 and float(z) == 0.0
    assert kv.quantize(x, s, z, 4).tolist() == list(range(16))
    y = np.array([-1.5, 6.0, 0.0, 2.25], dtype=np.float16)
    s, z = kv.group_params(y, 4)
    assert float(s) == 0.5 and float(z) == 3.0
    # 2.25 / 0.5 + 3 = 7.5 -> 8 (ties to even)
    assert kv.quantize(y, s, z, 4).tolist() == [0, 15, 3, 8]


def test_mixed_widths_quantize_each_side_with_its_own():
    """A state with 4-bit keys and 2-bit values: key codes reach 15, value codes stay in [0, 3],
    and each side equals a quantizer call with its own width."""
    rng = np.random.default_rng(9)
    k = rng.standard_normal((300, 32)).astype(np.float16)
    v = rng.standard_normal((300, 32)).astype(np.float16)
    st = kv.KiviState(D=32, bits=4, v_bits=2)
    st.prefill(k, v)
    kc = np.concatenate(st.k_codes)
    vc = np.stack(st.v_codes)
    assert kc.max() == 15 and vc.max() == 3
    codes, _, _ = kv.quantize_keys(k[:st.n_kq], 32, 4)
    np.testing.assert_array_equal(kc, codes)
    codes, _, _ = kv.quantize_values(v[:st.n_vq], 32, 2)
    np.testing.assert_array_equal(vc, codes)


def test_round_half_to_even():
    """x/s + z landing exactly on k + 1/2 rounds to the even neighbour."""
    x = np.array([0.0, 0.5, 1.5, 2.5, 3.0], dtype=np.float16)
    s, z = kv.group_params(x)
    assert kv.quantize(x, s, z).tolist() == [0, 0, 2, 2, 3]


def test_key_and_value_grouping_directions():
    """Keys share (s, z) down a column of `group` tokens; values along a row of
    `group` channels.  A key outlier channel only changes its own column's
    scale; a value outlier only its own row's."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, 128)).astype(np.float16)
    k2 = k.copy()
    k2[:, 5] *= 20
    _, s1, _ = kv.quantize_keys(k)
    _, s2, _ = kv.quantize_keys(k2)
    assert s1.shape == (2, 128)
    changed = np.nonzero((s1 != s2).any(axis=0))[0]
    assert changed.tolist() == [5]
    v = rng.standard_normal((10, 128)).astype(np.float16)
    v2 = v.copy()
    v2[3, 40] = 50
    _, t1, _ = kv.quantize_values(v)
    _, t2, _ = kv.quantize_values(v2)
    assert t1.shape == (10, 4)
    assert np.argwhere(t1 != t2).tolist() == [[3, 1]]


def _state(L, seed=5, D=128, R=128, group=32):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    st = kv.KiviState(D=D, R=R, group=group)
    st.prefill(k, v)
    return st, k, v, rng


def test_prefill_split_matches_pseudo_code():
    """Prefill keeps the last R tokens fp16 (pseudo-code: X_K[:l-R] grouped,
    X_K[l-R:] residual); at L = 4096, R = 128 both quantized parts hold 3968 tokens."""
    st, _, _, _ = _state(4096, D=32)
    assert st.n_kq == 3968 and len(st.k_res) == 128
    assert st.n_vq == 3968 and len(st.v_res) == 128
    st, _, _, _ = _state(300, D=32)          # (L - R) not a multiple of the group
    assert st.n_kq == 160 and len(st.k_res) == 140 and st.n_vq == 172 and len(st.v_res) == 128
    st, _, _, _ = _state(100, D=32)          # shorter than the residual
    assert st.n_kq == 0 and st.n_vq == 0 and len(st.k_res) == 100


def test_decode_appends_follow_flush_rules():
    st, _, _, rng = _state(300, D=32)
    for step in range(400):
        st.append(rng.standard_normal(32).astype(np.float16), rng.standard_normal(32).astype(np.float16))
        assert len(st.k_res) < st.R            # keys flush whole groups once R rows are waiting
        assert st.n_kq % st.group == 0
        assert len(st.v_res) == st.R           # values keep exactly the newest R rows
        assert st.length == 300 + step + 1 == st.n_vq + len(st.v_res)


def test_residual_only_state_is_plain_attention():
    st, k, v, rng = _state(100)
    q = rng.standard_normal(128)
    o, lse = kv.attention(q, st, 1 / math.sqrt(128))
    s = k.astype(np.float64) @ q / math.sqrt(128)
    w = np.exp(s - s.max())
    np.testing.assert_allclose(o, w @ v.astype(np.float64) / w.sum(), atol=1e-13)
    assert abs(lse - (s.max() + math.log(w.sum()))) < 1e-12


def test_joint_softmax_equals_merged_segments_and_differs_from_separate():
    st, _, _, rng = _state(700)
    q = rng.standard_normal(128) * 2
    o, lse = kv.attention(q, st, 1 / math.sqrt(128))
    keys, vals = st.keys(), st.values()
    parts = []
    for sl in (slice(0, 300), slice(300, 700)):
        s = keys[sl] @ q / math.sqrt(128)
        w = np.exp(s - s.max())
        parts.append(((w @ vals[sl]) / w.sum(), s.max() + math.log(w.sum())))
    M = max(p[1] for p in parts)
    lse2 = M + math.log(sum(math.exp(p[1] - M) for p in parts))
    o2 = sum(math.exp(p[1] - lse2) * p[0] for p in parts)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    assert abs(lse - lse2) < 1e-12
    bad = kv.attention_per_segment_softmax(q, st, 1 / math.sqrt(128))
    assert np.abs(bad - o).max() > 1e-2


def _lossless_grid_cache(L, D=128, group=32, bits=2, seed=11):
    """Keys and values whose every quantizer group is an exactly representable grid
    {a, a+s, ..., a+(2^b-1)s} holding both end points, with a scale and an offset of its
    own per group: key groups are (32-token block, channel), aligned at token 0 as the
    flush rule keeps them; value groups are (token, 32-channel block)."""
    rng = np.random.default_rng(seed)
    top = 2 ** bits - 1

    def grid(n):
        s = float(2.0 ** rng.integers(-5, 3))
        a = -float(rng.integers(0, top + 1)) * s       # z = -a/s is an integer
        x = a + s * rng.integers(0, top + 1, size=n)
        i_lo, i_hi = rng.choice(n, size=2, replace=False)
        x[i_lo], x[i_hi] = a, a + top * s
        return x

    k = np.empty((L, D))
    for g0 in range(0, L, group):
        for d in range(D):
            n = min(group, L - g0)
            k[g0:g0 + n, d] = grid(group)[:n]
    v = np.empty((L, D))
    for j in range(L):
        for c0 in range(0, D, group):
            v[j, c0:c0 + group] = grid(group)
    return k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("bits", [2, 4])
def test_state_keys_and_values_reproduce_lossless_inputs(bits):
    """keys() / values() put each dequantized row back at its own position with its own
    group's (s, z): on lossless grids (scale and offset differing from group to group, so a
    misplaced broadcast of s or z, or a row out of order, changes values) the whole cache,
    quantized and fp16 parts, equals the fp16 input exactly, after prefill and after decode
    appends that flush keys and values several times (KIVI page, core design: attention runs
    over the dequantized groups followed by the fp16 residual)."""
    L0, n_app = 300, 150
    k, v = _lossless_grid_cache(L0 + n_app, bits=bits)
    st = kv.KiviState(D=128, R=128, group=32, bits=bits)
    st.prefill(k[:L0], v[:L0])
    assert st.n_kq == 160 and st.n_vq == 172
    np.testing.assert_array_equal(st.keys(), k[:L0].astype(np.float64))
    np.testing.assert_array_equal(st.values(), v[:L0].astype(np.float64))
    for j in range(L0, L0 + n_app):
        st.append(k[j], v[j])
    assert st.n_kq == 416 and st.n_vq == L0 + n_app - 128
    np.testing.assert_array_equal(st.keys(), k.astype(np.float64))
    np.testing.assert_array_equal(st.values(), v.astype(np.float64))
    # the groups really do carry distinct parameters (so the check above can see a wrong broadcast)
    assert len({float(x) for x in np.stack(st.k_s)[:, 0]}) > 1
    assert len({float(x) for x in np.stack(st.v_s)[0]}) > 1
