"""Streaming decode with a random-weight looped block: time per generated token and where it goes.

The LoopVQ page's decode loop (Figure 5): for every generated token, each of the T loop steps of a
looped transformer block computes q, k, v, appends the token's pre-RoPE K and V to the bf16 window,
attends (index pages + window, the library's split path) and finishes the block; after every 8
tokens the window's oldest page is encoded into the index pool.  The block here has random bf16
weights (no trained model is available): d_model = H * D = 2048, RMSNorm, fused QKV projection,
rotate-half RoPE on q, output projection, SwiGLU MLP (2048 -> 5632 -> 2048); the same weights at every
loop step.  Its GEMMs and elementwise work are PyTorch (hipBLASLt); the cache steps are the library's
kernels.  The cache is the 6K batch-64 workload (loopvq-b64-6k), streamed from 6144 - N tokens.

Prints one JSON line per measurement: time per token, and the breakdown measured with HIP events
around each phase in a second pass (events add a little time of their own).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--tokens", type=int, default=24, help="timed tokens (3 page encodes)")
    ap.add_argument("--warmup", type=int, default=8)
    args = ap.parse_args()
    import torch
    import decode_attention_loopvq_amd as lvq  # noqa: F401  (fails loudly without the HIP library)
    from decode_attention_loopvq_amd.stream import LoopVQStream
    from synth.configs import loopvq_config
    from tests import harness

    cfg = loopvq_config("loopvq-b64-6k")
    p = harness.build_loopvq(cfg)
    g, B, H, D, T = p.g, cfg.B, cfg.H, cfg.D, cfg.T
    n_tok = args.warmup + args.tokens
    start = [L - n_tok for L in p.lengths]
    st = LoopVQStream(p.cache, p.codebooks, p.slices, p.rope_cos, p.rope_sin, p.rope16, p.sm_scale, start)

    dm, dff = H * D, 5632
    gen = torch.Generator(device="cuda").manual_seed(2024)

    def w(n_in, n_out):
        return (torch.randn((n_in, n_out), generator=gen, device="cuda") / n_in ** 0.5).to(torch.bfloat16)

    W_qkv, W_o, W_gu, W_dn = w(dm, 3 * dm), w(dm, dm), w(dm, 2 * dff), w(dff, dm)
    n1 = torch.ones(dm, dtype=torch.bfloat16, device="cuda")
    n2 = torch.ones(dm, dtype=torch.bfloat16, device="cuda")
    half = D // 2

    def rmsnorm(x, wt):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + 1e-6)).to(torch.bfloat16) * wt

    def rope_q(q, pos):                                  # q [B][H][D] bf16, rotate-half at positions pos [B]
        c = p.rope_cos[pos][:, None, :]
        s = p.rope_sin[pos][:, None, :]
        qf = q.float()
        lo, hi = qf[..., :half], qf[..., half:]
        return torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1).to(torch.bfloat16)

    x0 = (torch.randn((n_tok, B, dm), generator=gen, device="cuda")).to(torch.bfloat16)
    marks = {}

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def token(i, timed_phases):
        ph = []
        if timed_phases:
            ph.append(("start", ev()))
        st.begin_token()
        if timed_phases:
            ph.append(("encode_page", ev()))
        pos = torch.as_tensor(st.len - 1, device="cuda")
        x = x0[i]
        for t in range(T):
            h = rmsnorm(x, n1)
            qkv = (h @ W_qkv).view(B, 3, H, D)
            q = rope_q(qkv[:, 0], pos)
            k, v = qkv[:, 1].contiguous(), qkv[:, 2].contiguous()
            if timed_phases:
                ph.append(("model", ev()))
            st.append(t, k, v)
            if timed_phases:
                ph.append(("append", ev()))
            o, _ = st.attend(t, q)
            if timed_phases:
                ph.append(("attention", ev()))
            x = x + o.to(torch.bfloat16).view(B, dm) @ W_o
            h2 = rmsnorm(x, n2)
            gu = h2 @ W_gu
            x = x + (torch.nn.functional.silu(gu[:, :dff]) * gu[:, dff:]) @ W_dn
            if timed_phases:
                ph.append(("model", ev()))
        return ph

    for i in range(args.warmup):
        token(i, False)
    torch.cuda.synchronize()
    e0 = ev()
    for i in range(args.warmup, n_tok):
        token(i, False)
    e1 = ev()
    torch.cuda.synchronize()
    us_tok = e0.elapsed_time(e1) * 1e3 / args.tokens

    # second pass over the same tokens with events between phases (the stream is rewound)
    st.len = st.len - args.tokens
    st._set_lengths()
    sums = {}
    all_ph = [token(i, True) for i in range(args.warmup, n_tok)]
    torch.cuda.synchronize()
    for ph in all_ph:
        for (_, a), (name, b) in zip(ph, ph[1:]):
            sums[name] = sums.get(name, 0.0) + a.elapsed_time(b) * 1e3 / args.tokens
    total = sum(sums.values())
    print(json.dumps({"row": "decode-stream", "workload": cfg.name, "B": B, "H": H, "L": cfg.L, "T": T,
                      "tokens": args.tokens, "us_per_token": round(us_tok, 1),
                      "breakdown_us_per_token": {k: round(v, 1) for k, v in sums.items()},
                      "attention_share": round(sums.get("attention", 0) / total, 3),
                      "model": "random-weight looped block, d_model 2048, SwiGLU 5632, PyTorch GEMMs"}),
          flush=True)


if __name__ == "__main__":
    main()
