"""GPU parity of packed-sequence training (gda_fwd_train_varlen, gda_bwd_varlen) against the
fp64 oracle, through the C ABI.

Cases: packed documents of ragged lengths (a one-token and an empty document among them),
causal and windowed; chunks whose keys start with a W-1 halo (the sequence-sharded
sliding-window layer, here at full size: 8 chunks of 4096 queries); more queries than keys
(queries at negative positions must get zero gradients and zero path outputs); the Motif-2
layout; the call options; and uniform lengths, whose gradients must equal the batched
backward's bit for bit. Tolerances as the batched backward's: each gradient within 2e-2 (max)
and 2e-3 (mean) of its largest magnitude (at least 0.05).
"""
import numpy as np
import pytest
import torch

import oracle
from attention_gda_fwd_amd import configs as C
from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import (gda_bwd, gda_bwd_varlen, gda_fwd_train,
                                       gda_fwd_train_varlen)

from . import gpu_util as U
from .test_gpu_bwd import assert_grad_close

pytestmark = pytest.mark.gpu

ARGS = ("q_sig", "q_noise", "k", "v", "lam", "gate")
M3 = dict(S=64, N=16, Hkv=16, dqk=192, dv=128, rope_dims=64)
M2 = dict(S=32, N=8, Hkv=16, dqk=128, dv=128)
TINY = dict(S=8, N=2, Hkv=2, dqk=64, dv=64)
DOCS = [120, 1, 70, 0, 45]
CASES = {
    "docs_motif3_causal": (701, M3, DOCS, DOCS, 0, {}),
    "docs_motif3_w50": (702, M3, DOCS, DOCS, 50, {}),
    "halo_motif3_w64": (703, M3, [100, 80], [100, 80 + 63], 64, {}),
    "fewer_keys_motif2": (704, M2, [90, 40], [60, 40], 0, {}),
    "tiny_options": (705, TINY, [70, 33], [70, 48], 16,
                     dict(scale=0.2, lambda_logits=True, gate_logits=True)),
}


def _case(case_id, heads, lens_q, lens_k, logits):
    x = gin.varlen_inputs(case_id, lens_q=lens_q, lens_k=lens_k, dtype="bf16", **heads)
    Tq = int(x["cu_q"][-1])
    if logits:
        x["lam"] = gin.normal(case_id, 41, 0, x["lam"].shape, "bf16")
        x["gate"] = gin.normal(case_id, 42, 0, x["gate"].shape, "bf16")
    x["d_out"] = gin.normal(case_id, 50, 0, (Tq, heads["S"], heads["dv"]), "bf16")
    return x


def _run(x, window, **opts):
    d = {n: U.to_dev(a, "bf16") for n, a in x.items() if n not in ("cu_q", "cu_k")}
    cu_q = torch.from_numpy(x["cu_q"]).cuda()
    cu_k = torch.from_numpy(x["cu_k"]).cuda()
    mq = max(int(np.diff(x["cu_q"]).max()), 1)
    mk = max(int(np.diff(x["cu_k"]).max()), 1)
    out, hs, hn, lse = gda_fwd_train_varlen(*(d[n] for n in ARGS), cu_q, cu_k, mq, window=window,
                                            **opts)
    grads = gda_bwd_varlen(*(d[n] for n in ARGS), hs, hn, lse, d["d_out"], cu_q, cu_k, mq, mk,
                           window=window, **opts)
    return (out, hs, hn, lse), {n: U.to_f64(g) for n, g in grads.items()}


@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_backward(name):
    case_id, heads, lens_q, lens_k, window, opts = CASES[name]
    U.log(f"packed backward {name} lens_q={lens_q} lens_k={lens_k} window={window} {opts}")
    x = _case(case_id, heads, lens_q, lens_k, bool(opts))
    (out, hs, hn, lse), got = _run(x, window, **opts)
    host = [x[n] for n in ARGS]
    r_out, r_hs, r_hn, r_lse = oracle.ref_fwd_train_varlen(*host, x["cu_q"], x["cu_k"],
                                                           window=window, **opts)
    U.assert_close(U.to_f64(out), r_out, "bf16", f"{name} out")
    U.assert_close(U.to_f64(hs), r_hs, "bf16", f"{name} h_sig")
    U.assert_close(U.to_f64(hn), r_hn, "bf16", f"{name} h_noise")
    gl, rl = U.to_f64(lse), r_lse
    fin = np.isfinite(rl)
    assert (np.isfinite(gl) == fin).all(), f"{name}: lse -inf pattern differs"
    assert np.abs(gl[fin] - rl[fin]).max(initial=0.0) <= 1e-3, f"{name}: lse error"
    ref = oracle.ref_bwd_varlen(*host, x["d_out"], x["cu_q"], x["cu_k"], window=window, **opts)
    for n in ref:
        assert_grad_close(got[n], ref[n], f"{name} {n}")
    neg, start = [], 0
    for lq, lk in zip(lens_q, lens_k):
        neg += list(range(start, start + max(lq - lk, 0)))
        start += lq
    if neg:
        for n in ("dq_sig", "dq_noise", "dlam", "dgate"):
            assert (got[n][neg] == 0).all(), f"{name}: {n} not zero at negative positions"


def test_varlen_backward_uniform_lengths_equal_the_batched_call():
    """Two equal sequences (Motif-3 heads, L = 1024, W = 0 and 200): the packed training
    forward and backward give exactly the batched calls' bits."""
    B, L = 2, 1024
    x = gin.fwd_inputs(710, B=B, L=L, dtype="bf16", **M3)
    x["d_out"] = np.stack([gin.normal(710, 50, b, (L, 64, 128), "bf16") for b in range(B)])
    d = {n: U.to_dev(a, "bf16") for n, a in x.items()}
    flat = {n: t.reshape(B * L, *t.shape[2:]) for n, t in d.items()}
    cu = torch.arange(0, B + 1, dtype=torch.int32, device="cuda") * L
    for window in (0, 200):
        U.log(f"packed == batched training, window {window}")
        out, hs, hn, lse = gda_fwd_train(*(d[n] for n in ARGS), window=window)
        g = gda_bwd(*(d[n] for n in ARGS), hs, hn, lse, d["d_out"], window=window)
        pout, phs, phn, plse = gda_fwd_train_varlen(*(flat[n] for n in ARGS), cu, cu, L,
                                                    window=window)
        pg = gda_bwd_varlen(*(flat[n] for n in ARGS), phs, phn, plse, flat["d_out"], cu, cu, L, L,
                            window=window)
        assert torch.equal(pout.reshape(out.shape), out)
        assert torch.equal(phs.reshape(hs.shape), hs)
        # lse: [S+N, B*L] against [B, S+N, L]
        assert torch.equal(plse.reshape(80, B, L).permute(1, 0, 2), lse)
        for n in g:
            assert torch.equal(pg[n].reshape(g[n].shape), g[n]), n


def test_varlen_backward_full_size_sliding_window_chunks():
    """The sliding-window layer (L = 32768, W = 128) as 8 chunks of 4096 queries with
    127-key halos: every gradient of every row against the oracle."""
    cfg = C.MOTIF3_SWA
    P, W = 8, cfg.window
    chunk = cfg.L // P
    lens_q = [chunk] * P
    lens_k = [chunk] + [chunk + W - 1] * (P - 1)
    x = _case(720, M3, lens_q, lens_k, False)
    U.log(f"packed backward at full size: {P} chunks of {chunk} with {W - 1}-key halos")
    _, got = _run(x, W)
    ref = oracle.ref_bwd_varlen(*(x[n] for n in ARGS), x["d_out"], x["cu_q"], x["cu_k"],
                                window=W)
    for n in ref:
        assert_grad_close(got[n], ref[n], f"swa chunks {n}")
