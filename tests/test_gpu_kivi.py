"""Parity of the HIP KIVI path with the oracle (GPU).

Codes, fp16 scales and zero-points and the fp16 residual rings must match
bit for bit; attention outputs within max relative error 2e-3 per row.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import kivi as kv
from synth.configs import kivi_config

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _unpack(codes: np.ndarray, bits: int = 2) -> np.ndarray:
    """[n][D*b/8] bytes -> [n][D] codes, channel d at bits b*(d % (8/b)) of byte d*b/8."""
    n, nb = codes.shape
    per = 8 // bits
    out = np.empty((n, nb * per), dtype=np.uint8)
    for u in range(per):
        out[:, u::per] = (codes >> (bits * u)) & ((1 << bits) - 1)
    return out


def _u16(x):
    return np.ascontiguousarray(x).view(np.uint16)


def _compare_state(cache, g, b, h, st: kv.KiviState):
    import decode_attention_loopvq_amd as lvq
    kb, vb, _ = lvq.kivi_widths(g)
    ring = g.R + g.group
    L, nk, nv = int(cache.len[b]), int(cache.n_kq[b]), int(cache.n_vq[b])
    assert (L, nk, nv) == (st.length, st.n_kq, st.n_vq), ((L, nk, nv), (st.length, st.n_kq, st.n_vq))
    if nk:
        np.testing.assert_array_equal(_unpack(cache.k_codes[b, h, :nk].cpu().numpy(), kb), np.concatenate(st.k_codes))
        np.testing.assert_array_equal(_u16(cache.k_scale[b, h, :nk // g.group].cpu().numpy()), _u16(np.stack(st.k_s)))
        np.testing.assert_array_equal(_u16(cache.k_zero[b, h, :nk // g.group].cpu().numpy()), _u16(np.stack(st.k_z)))
    if nv:
        np.testing.assert_array_equal(_unpack(cache.v_codes[b, h, :nv].cpu().numpy(), vb), np.stack(st.v_codes))
        np.testing.assert_array_equal(_u16(cache.v_scale[b, h, :nv].cpu().numpy()), _u16(np.stack(st.v_s)))
        np.testing.assert_array_equal(_u16(cache.v_zero[b, h, :nv].cpu().numpy()), _u16(np.stack(st.v_z)))
    kres = cache.k_res[b, h].cpu().numpy()
    vres = cache.v_res[b, h].cpu().numpy()
    for j, p in enumerate(range(nk, L)):
        np.testing.assert_array_equal(_u16(kres[p % ring]), _u16(st.k_res[j]))
    for j, p in enumerate(range(nv, L)):
        np.testing.assert_array_equal(_u16(vres[p % ring]), _u16(st.v_res[j]))


def _check_attn(prob, rows, states):
    """rows: (request, KV head); every query head of those KV heads is checked."""
    import decode_attention_loopvq_amd as lvq
    g, cache = prob.g, prob.cache
    Hq = lvq.kivi_widths(g)[2]
    nrep = Hq // g.H
    max_len = int(cache.len.max())
    worst = 0.0
    for ns in (0, 1, 5):
        lse = torch.empty((cache.B, Hq), dtype=torch.float32, device="cuda")
        out, _ = lvq.kivi_decode_attn(g, prob.q, cache, max_len, prob.sm_scale, lse_out=lse, num_splits=ns)
        torch.cuda.synchronize()
        for (b, h) in rows:
            for hq in range(h * nrep, (h + 1) * nrep):
                q = prob.q[b, hq].float().cpu().numpy().astype(np.float64)
                o_ref, lse_ref = kv.attention(q, states[(b, h)], prob.sm_scale)
                o = out[b, hq].double().cpu().numpy()
                err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
                worst = max(worst, err)
                assert err <= REL_TOL, f"row ({b},{hq}) over KV head {h}, splits {ns}: rel err {err:.3e}"
                assert abs(float(lse[b, hq]) - lse_ref) <= 2e-3
    return worst


def _states(prob, rows):
    k = prob.k.cpu().numpy()
    v = prob.v.cpu().numpy()
    states = {}
    for (b, h) in rows:
        st = kv.KiviState(D=prob.g.D, group=prob.g.group, R=prob.g.R, bits=prob.g.bits, v_bits=prob.g.v_bits)
        st.prefill(k[b, h], v[b, h])
        states[(b, h)] = st
    return states


@pytest.mark.parametrize("L", [1, 100, 128, 160, 300, 700])
def test_prefill_bit_exact_and_attention(L):
    from tests import harness
    cfg = kivi_config("kivi-b16-4k", B=3, H=2, L=L)
    _say(f"[kivi prefill] L={L}")
    prob = harness.build_kivi(cfg)
    rows = [(b, h) for b in range(3) for h in range(2)]
    states = _states(prob, rows)
    for (b, h) in rows:
        _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    _check_attn(prob, rows, states)


def test_decode_appends_bit_exact():
    """Prefill, then 200 single-token appends (several key flushes, a value
    overflow at every step), then attention."""
    import decode_attention_loopvq_amd as lvq
    import synth.kivi as synk
    from tests import harness
    cfg = kivi_config("kivi-b16-4k", B=2, H=2, L=300)
    prob = harness.build_kivi(cfg)
    rows = [(b, h) for b in range(2) for h in range(2)]
    states = _states(prob, rows)
    n = 200
    kn, vn = synk.new_tokens(cfg, n, "cuda")          # [n][B][H][D]
    kn_h, vn_h = kn.cpu().numpy(), vn.cpu().numpy()
    for i in range(n):
        lvq.kivi_append(prob.g, kn[i][:, :, None, :], vn[i][:, :, None, :], prob.cache, prefill=False)
        for (b, h) in rows:
            states[(b, h)].append(kn_h[i, b, h], vn_h[i, b, h])
        if i in (0, 1, 27, 28, 29, 155, 199):
            torch.cuda.synchronize()
            for (b, h) in rows:
                _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    _check_attn(prob, rows, states)


def test_full_b16_4k_sampled():
    from tests import harness
    cfg = kivi_config("kivi-b16-4k")
    _say("[kivi full] B=16 H=32 L=4096")
    prob = harness.build_kivi(cfg)
    rows = [(0, 0), (7, 19), (15, 31)]
    states = _states(prob, rows)
    for (b, h) in rows:
        _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    worst = _check_attn(prob, rows, states)
    _say(f"[kivi full] worst rel err {worst:.3e}")


def _layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    """The same [B][H][L][D] values in another memory layout (a strided view)."""
    B, H, L, D = x.shape
    if layout == "bhld":
        return x
    if layout == "blhd":                      # token-major, as a model's projections write it
        return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if layout == "padded":                    # row stride D + 1: rows off the 16-byte grid
        buf = torch.zeros((B, H, L, D + 1), dtype=x.dtype, device=x.device)
        buf[..., :D] = x
        return buf[..., :D]
    if layout == "offset":                    # contiguous, base one element past an aligned address
        buf = torch.zeros(x.numel() + 8, dtype=x.dtype, device=x.device)
        buf[1:1 + x.numel()] = x.reshape(-1)
        return buf[1:1 + x.numel()].view(B, H, L, D)
    raise ValueError(layout)


@pytest.mark.parametrize("bits,v_bits", [(2, 0), (4, 2), (2, 4)], ids=["k2v2", "k4v2", "k2v4"])
@pytest.mark.parametrize("layout", ["blhd", "padded", "offset"])
def test_prefill_strided_inputs(layout, bits, v_bits):
    """Prefill from views that are not contiguous [B][H][L][D]: token-major rows go through the one-pass
    kernel; rows off the 16-byte grid go through the per-stage kernels.  Both bit-exact, at each code
    width."""
    import decode_attention_loopvq_amd as lvq
    import synth.kivi as synk
    cfg = kivi_config("kivi-b16-4k", B=2, H=3, L=333, bits=bits, v_bits=v_bits)
    _say(f"[kivi prefill strided] layout={layout} k{bits} v{v_bits or bits}")
    g = lvq.make_kivi_geom(D=cfg.D, H=cfg.H, bits=cfg.bits, group=cfg.group, R=cfg.R,
                           cap=((cfg.L + 256 + cfg.group - 1) // cfg.group) * cfg.group, v_bits=cfg.v_bits)
    cache = lvq.KiviCache(g, cfg.B, device="cuda")
    k, v = synk.raw_kv(cfg, "cuda")
    kl, vl = _layout(k, layout), _layout(v, layout)
    assert torch.equal(kl, k) and torch.equal(vl, v)
    lvq.kivi_append(g, kl, vl, cache, prefill=True)
    torch.cuda.synchronize()
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    for b in range(cfg.B):
        for h in range(cfg.H):
            st = kv.KiviState(D=g.D, group=g.group, R=g.R, bits=g.bits, v_bits=g.v_bits)
            st.prefill(kh[b, h], vh[b, h])
            _compare_state(cache, g, b, h, st)


# KIVI-4, mixed key/value widths and grouped-query attention ("core design" with b = 4; the page's note
# on GQA support): prefill of a length with a partial key group and a long value overflow, then 40
# single-token appends (a key flush among them); state bit-exact, every query head's output against
# the oracle over its KV head.
@pytest.mark.parametrize("bits,v_bits,H,Hq", [
    (4, 0, 2, 0), (4, 2, 2, 0), (2, 4, 2, 0), (2, 0, 2, 8), (4, 4, 1, 32), (2, 4, 2, 4), (4, 2, 1, 16),
    (4, 4, 2, 16),
], ids=["k4v4", "k4v2", "k2v4", "k2v2-gqa4", "k4v4-gqa32", "k2v4-gqa2", "k4v2-gqa16", "k4v4-gqa8"])
def test_widths_and_grouped_queries(bits, v_bits, H, Hq):
    import decode_attention_loopvq_amd as lvq
    import synth.kivi as synk
    from tests import harness
    cfg = kivi_config("kivi-b16-4k", B=2, H=H, L=700, bits=bits, v_bits=v_bits, Hq=Hq)
    _say(f"[kivi widths] k{bits} v{v_bits or bits} H={H} Hq={Hq or H}")
    prob = harness.build_kivi(cfg)
    rows = [(b, h) for b in range(2) for h in range(H)]
    states = _states(prob, rows)
    for (b, h) in rows:
        _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    kn, vn = synk.new_tokens(cfg, 40, "cuda")
    kn_h, vn_h = kn.cpu().numpy(), vn.cpu().numpy()
    for i in range(40):
        lvq.kivi_append(prob.g, kn[i][:, :, None, :], vn[i][:, :, None, :], prob.cache, prefill=False)
        for (b, h) in rows:
            states[(b, h)].append(kn_h[i, b, h], vn_h[i, b, h])
    torch.cuda.synchronize()
    for (b, h) in rows:
        _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    worst = _check_attn(prob, rows, states)
    _say(f"[kivi widths] worst rel err {worst:.3e}")


@pytest.mark.parametrize("name", ["kivi4-b16-4k", "kivi-gqa-b16-4k"])
def test_variant_workloads_full_size_sampled(name):
    from tests import harness
    cfg = kivi_config(name)
    _say(f"[kivi full] {name}")
    prob = harness.build_kivi(cfg)
    rows = [(0, 0), (9, cfg.H // 2), (15, cfg.H - 1)]
    states = _states(prob, rows)
    for (b, h) in rows:
        _compare_state(prob.cache, prob.g, b, h, states[(b, h)])
    worst = _check_attn(prob, rows, states)
    _say(f"[kivi full] {name} worst rel err {worst:.3e}")


def _pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """[n][D] codes -> [n][D*b/8] bytes, channel d at bits b*(d % (8/b)) of byte d*b/8 (inverse of _unpack)."""
    n, D = codes.shape
    per = 8 // bits
    out = np.zeros((n, D // per), dtype=np.uint8)
    for u in range(per):
        out |= (codes[:, u::per].astype(np.uint8) << (bits * u)).astype(np.uint8)
    return out


def _put_state(cache, g, b, h, st: kv.KiviState):
    """Write one (request, KV head)'s state, as the oracle holds it, into the device cache (layout in lvq.h)."""
    import decode_attention_loopvq_amd as lvq
    kb, vb, _ = lvq.kivi_widths(g)
    ring = g.R + g.group
    nk, nv, L = st.n_kq, st.n_vq, st.length
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(cache.k_codes.device)
    if nk:
        cache.k_codes[b, h, :nk] = t(_pack(np.concatenate(st.k_codes), kb))
        cache.k_scale[b, h, :nk // g.group] = t(np.stack(st.k_s).astype(np.float16))
        cache.k_zero[b, h, :nk // g.group] = t(np.stack(st.k_z).astype(np.float16))
    if nv:
        cache.v_codes[b, h, :nv] = t(_pack(np.stack(st.v_codes), vb))
        cache.v_scale[b, h, :nv] = t(np.stack(st.v_s).astype(np.float16))
        cache.v_zero[b, h, :nv] = t(np.stack(st.v_z).astype(np.float16))
    for j, p in enumerate(range(nk, L)):
        cache.k_res[b, h, p % ring] = t(st.k_res[j])
    for j, p in enumerate(range(nv, L)):
        cache.v_res[b, h, p % ring] = t(st.v_res[j])


# A ragged batch in one call ("core design": each request's quantized groups and fp16 residual): requests of
# 1000, 5, 0, 300, 37 and 700 tokens, each (request, head) state built by the oracle's prefill and written
# into the cache (the append path cannot make lengths differ within a batch).  Every query head against the
# oracle; the empty request gives out = 0, lse = -inf.
@pytest.mark.parametrize("bits,v_bits,Hq", [(2, 0, 0), (2, 0, 8), (4, 2, 4)], ids=["k2v2", "k2v2-gqa4", "k4v2-gqa2"])
def test_ragged_batch_from_oracle_state(bits, v_bits, Hq):
    import decode_attention_loopvq_amd as lvq
    import synth.kivi as synk
    lengths = [1000, 5, 0, 300, 37, 700]
    B, H, L = len(lengths), 2, max(lengths)
    cfg = kivi_config("kivi-b16-4k", B=B, H=H, L=L, bits=bits, v_bits=v_bits, Hq=Hq)
    _say(f"[kivi ragged] k{bits} v{v_bits or bits} Hq={Hq or H} lengths {lengths}")
    cap = ((L + 256 + cfg.group - 1) // cfg.group) * cfg.group
    g = lvq.make_kivi_geom(D=cfg.D, H=H, bits=bits, group=cfg.group, R=cfg.R, cap=cap, v_bits=v_bits, Hq=Hq)
    cache = lvq.KiviCache(g, B)
    k, v = synk.raw_kv(cfg, "cpu")
    q = synk.queries(cfg, "cuda")[0].contiguous()
    sm = synk.softmax_scale(cfg)
    states = {}
    for b, Lb in enumerate(lengths):
        for h in range(H):
            st = kv.KiviState(D=cfg.D, group=cfg.group, R=cfg.R, bits=bits, v_bits=v_bits)
            if Lb:
                st.prefill(k[b, h, :Lb].numpy(), v[b, h, :Lb].numpy())
            _put_state(cache, g, b, h, st)
            states[(b, h)] = st
        cache.len[b], cache.n_kq[b], cache.n_vq[b] = Lb, states[(b, 0)].n_kq, states[(b, 0)].n_vq
    nrep = lvq.kivi_widths(g)[2] // H
    worst = 0.0
    for ns in (0, 1, 3):
        lse = torch.empty((B, nrep * H), dtype=torch.float32, device="cuda")
        out, _ = lvq.kivi_decode_attn(g, q, cache, L, sm, lse_out=lse, num_splits=ns)
        torch.cuda.synchronize()
        for b, Lb in enumerate(lengths):
            for hq in range(nrep * H):
                o = out[b, hq].double().cpu().numpy()
                if Lb == 0:
                    assert np.all(o == 0.0) and float(lse[b, hq]) == -np.inf, f"empty request {b}, head {hq}"
                    continue
                qv = q[b, hq].float().cpu().numpy().astype(np.float64)
                o_ref, lse_ref = kv.attention(qv, states[(b, hq // nrep)], sm)
                err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
                worst = max(worst, err)
                assert err <= REL_TOL, f"request {b} (length {Lb}), head {hq}, splits {ns}: rel err {err:.3e}"
                assert abs(float(lse[b, hq]) - lse_ref) <= 2e-3
    _say(f"[kivi ragged] worst rel err {worst:.3e}")


# Attention while the cache grows ("core design": appends flush whole key groups and single value rows):
# a prefill of 150 tokens (R = 128: no key group is quantized on both sides yet, the residual slot takes
# every row) and 100 single-token appends, attention checked against the oracle every 10 tokens at the
# library's split count and at 3 splits, so the whole-key-group range and the residual slot move across
# key flushes.
@pytest.mark.parametrize("Hq", [0, 8], ids=["mha", "gqa4"])
def test_attention_while_appending(Hq):
    import decode_attention_loopvq_amd as lvq
    import synth.kivi as synk
    from tests import harness
    cfg = kivi_config("kivi-b16-4k", B=2, H=2, L=150, Hq=Hq)
    _say(f"[kivi grow] Hq={Hq or cfg.H}: prefill 150, 100 appends")
    prob = harness.build_kivi(cfg, cap=((150 + 100 + 256 + 31) // 32) * 32)
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    states = _states(prob, rows)
    kn, vn = synk.new_tokens(cfg, 100, "cuda")
    kn_h, vn_h = kn.cpu().numpy(), vn.cpu().numpy()
    Hq_ = lvq.kivi_widths(prob.g)[2]
    nrep = Hq_ // cfg.H
    checked = 0
    for i in range(100):
        lvq.kivi_append(prob.g, kn[i][:, :, None, :], vn[i][:, :, None, :], prob.cache, prefill=False)
        for (b, h) in rows:
            states[(b, h)].append(kn_h[i, b, h], vn_h[i, b, h])
        if (i + 1) % 10:
            continue
        L = int(prob.cache.len.max())
        for ns in (0, 3):
            lse = torch.empty((cfg.B, Hq_), dtype=torch.float32, device="cuda")
            out, _ = lvq.kivi_decode_attn(prob.g, prob.q, prob.cache, L, prob.sm_scale, lse_out=lse, num_splits=ns)
            torch.cuda.synchronize()
            for (b, h) in rows:
                for hq in range(h * nrep, (h + 1) * nrep):
                    qv = prob.q[b, hq].float().cpu().numpy().astype(np.float64)
                    o_ref, lse_ref = kv.attention(qv, states[(b, h)], prob.sm_scale)
                    o = out[b, hq].double().cpu().numpy()
                    err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
                    st = states[(b, h)]
                    assert err <= REL_TOL, (f"after {i + 1} appends (L={st.length}, n_kq={st.n_kq}, n_vq={st.n_vq}), "
                                            f"row ({b},{hq}), splits {ns}: rel err {err:.3e}")
                    assert abs(float(lse[b, hq]) - lse_ref) <= 2e-3
                    checked += 1
    _say(f"[kivi grow] {checked} rows checked")
