"""Streaming decode (the LoopVQ page, Figure 5): tokens appended one at a time to the bf16 window, the
oldest page encoded every 8 tokens from the window ring, attention at every loop step.  Checked against the
oracle: every index the stream writes, and every attention call along the way (at its length then).  The
state after streaming must also equal, byte for byte, the state a prefill of the same tokens builds, and so
must the attention output."""

import sys

import types

import numpy as np
import pytest
import torch

from oracle import loopvq as lv
from synth.configs import loopvq_config

REL_TOL = 2e-3
LSE_TOL = 2e-3

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,over", [
    ("loopvq-b64-6k", dict(B=5, H=2, L=420, ragged=(200, 420), random_pages=True, seed=41)),
    ("loopvq-deep-ragged", dict(B=3, H=2, L=300, ragged=(120, 300), seed=43)),
], ids=["c8", "c4"])
def test_stream_equals_prefill(name, over):
    import decode_attention_loopvq_amd as lvq
    import synth.loopvq as syn
    from decode_attention_loopvq_amd.layout import LoopVQCache, n_index_pages
    from decode_attention_loopvq_amd.stream import LoopVQStream
    from tests import harness
    cfg = loopvq_config(name, **over)
    N = 40                                              # tokens streamed per request (5 pages)
    _say(f"[stream] {cfg.name} B={cfg.B} prefill reference")
    rows = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    ref = harness.build_loopvq(cfg, keep=rows)          # the final state, by prefill
    geo = lv.Geometry(D=cfg.D, T=cfg.T, Tc=cfg.Tc, G=cfg.G, K=cfg.K, sink=cfg.sink, window=cfg.window,
                      page=cfg.page)
    # the oracle's indices of every row at its final length (a shorter length's are a prefix: the encode is
    # per token)
    oidx = {(kind, b, h): lv.encode_request(ref.raw[(kind, b, h)], harness.host_codebooks(ref, h, kind), geo,
                                            ref.lengths[b])
            for kind in ("k", "v") for (b, h) in rows}

    def check_attend(t, out, lse, lengths):
        """Every row of an attention call against the oracle at the row's current length."""
        for (b, h) in rows:
            L = lengths[b]
            _, q_lo, q_hi = lv.cache_regions(L, geo)
            n = q_hi - q_lo
            q = ref.q[t, b, h].float().cpu().numpy().astype(np.float64)
            o_ref, l_ref = lv.decode_step(q, t, ref.raw[("k", b, h)], ref.raw[("v", b, h)],
                                          oidx[("k", b, h)][:, :n], oidx[("v", b, h)][:, :n],
                                          harness.host_codebooks(ref, h, "k"), harness.host_codebooks(ref, h, "v"),
                                          geo, L, ref.sm_scale, cfg.rope_base)
            o = out[b, h].double().cpu().numpy()
            err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
            assert err <= REL_TOL, f"step {t} row ({b},{h}) L={L}: rel err {err:.3e}"
            if lse is not None:
                assert abs(float(lse[b, h]) - l_ref) <= LSE_TOL, f"step {t} row ({b},{h}): lse {float(lse[b, h])} vs {l_ref}"

    g, final = ref.g, ref.lengths
    start = [L - N for L in final]
    total = sum(n_index_pages(L, g) for L in final)
    cache = LoopVQCache(g, final, phys_perm=syn.page_permutation(cfg, max(1, total)))
    assert np.array_equal(cache.page_table_host, ref.cache.page_table_host)
    n0 = torch.tensor([n_index_pages(L, g) for L in start], dtype=torch.int32, device="cuda")
    xs = {kind: dict(syn.raw_blocks(cfg, kind, "cuda")) for kind in ("k", "v")}
    for beta in range(g.T // g.Tc):                     # prefill of the first `start` tokens
        lvq.lvq_encode(g, beta, xs["k"][beta], xs["v"][beta], ref.codebooks, cache.pool, cache.page_table,
                       cache.first_page, n0, cache.max_pages, x_tok0=cache.tok0)
        harness._fill_window(cache, beta, xs["k"][beta], "k", lengths=start)
        harness._fill_window(cache, beta, xs["v"][beta], "v", lengths=start)
    st = LoopVQStream(cache, ref.codebooks, ref.slices, ref.rope_cos, ref.rope_sin, ref.rope16, ref.sm_scale,
                      start)
    bidx = torch.arange(cfg.B, device="cuda")
    _say(f"[stream] {N} tokens x {g.T} loop steps")
    encoded = 0
    for i in range(N):
        encoded += int(st.begin_token(reorder=(i % 8 == 0)).sum())
        pos = torch.as_tensor(st.len - 1, device="cuda")
        for t in range(g.T):
            beta, m = divmod(t, g.Tc)
            k = xs["k"][beta][bidx, :, pos, m].contiguous()      # [B][H][D]
            v = xs["v"][beta][bidx, :, pos, m].contiguous()
            st.append(t, k, v)
            if i % 13 == 0 or i == N - 1:
                lse_i = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
                out_i, _ = st.attend(t, ref.q[t].contiguous(), lse_out=lse_i)
                torch.cuda.synchronize()
                check_attend(t, out_i, lse_i, list(st.len))
    torch.cuda.synchronize()
    assert encoded == sum(n_index_pages(L, g) - n_index_pages(L0, g) for L, L0 in zip(final, start))
    _say(f"[stream] {encoded} pages encoded from the window; compare with the prefill state")
    assert list(st.len) == list(final)
    assert torch.equal(cache.seq_len, ref.cache.seq_len)
    # every index of the streamed pool against the oracle
    streamed = types.SimpleNamespace(g=g, cache=cache)
    for (b, h) in rows:
        for kind in ("k", "v"):
            np.testing.assert_array_equal(harness.gpu_indices(streamed, b, h, kind), oidx[(kind, b, h)],
                                          err_msg=f"streamed indices of ({b},{h}) {kind}")
    for b in range(cfg.B):
        pages = torch.as_tensor(cache.page_table_host[b, :n_index_pages(final[b], g)], dtype=torch.long,
                                device="cuda")
        assert torch.equal(cache.pool[pages], ref.cache.pool[pages]), f"request {b}: pool pages differ"
        from decode_attention_loopvq_amd.layout import window_positions, window_slot
        slots = torch.as_tensor(window_slot(window_positions(final[b], g), g), dtype=torch.long, device="cuda")
        assert torch.equal(cache.win_k[b][:, :, slots], ref.cache.win_k[b][:, :, slots]), f"request {b}: window K"
        assert torch.equal(cache.win_v[b][:, :, slots], ref.cache.win_v[b][:, :, slots]), f"request {b}: window V"
    for t in range(g.T):
        lse_a = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
        lse_b = torch.empty_like(lse_a)
        out_a, _ = st.attend(t, ref.q[t].contiguous(), lse_out=lse_a)
        out_b, _ = harness.run_step(ref, t, lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), f"step {t}: attention differs"
