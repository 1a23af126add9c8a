"""Streaming decode (the LoopVQ page, Figure 5): tokens appended one at a time to the bf16 window, the
oldest page encoded every 8 tokens from the window ring, attention at every loop step.  The state after
streaming must equal, byte for byte, the state a prefill of the same tokens builds (whose indices and
attention the parity tests check against the oracle), and so must the attention output."""

import sys

import numpy as np
import pytest
import torch

from synth.configs import loopvq_config

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
    ref = harness.build_loopvq(cfg)                     # the final state, by prefill
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
                st.attend(t, ref.q[t].contiguous())
    torch.cuda.synchronize()
    assert encoded == sum(n_index_pages(L, g) - n_index_pages(L0, g) for L, L0 in zip(final, start))
    _say(f"[stream] {encoded} pages encoded from the window; compare with the prefill state")
    assert list(st.len) == list(final)
    assert torch.equal(cache.seq_len, ref.cache.seq_len)
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
