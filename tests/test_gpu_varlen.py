"""GPU parity of packed-sequence prefill (gda_fwd_varlen) against the fp64 oracle.

Cases: packed documents of ragged lengths (a one-token and an empty document among
them), chunks whose keys start with a halo of W-1 earlier keys, sequences with fewer
keys than queries (queries at negative positions must come out as exact zeros), every
compiled bf16 head layout family, the fp32 matrix-core and VALU kernels, the call
options, and two full-size checks: the sliding-window workload cut into 8 chunks with
halos, and the causal Motif 3 workload whose packed form must reproduce the batched call
bit for bit (same kernel, same tiles, same order).
Tolerances: bf16 max |err| <= 2e-2 and mean |err| <= 2e-3; fp32 max |err| <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_gda_fwd_amd import configs as C
from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import gda_fwd, gda_fwd_varlen

from . import gpu_util as U

pytestmark = pytest.mark.gpu

M3 = dict(S=64, N=16, Hkv=16, dqk=192, dv=128, rope_dims=64)
M2 = dict(S=32, N=8, Hkv=16, dqk=128, dv=128)
TINY = dict(S=8, N=2, Hkv=2, dqk=64, dv=64)

DOCS = [200, 1, 77, 130, 0, 64]
CASES = {
    # packed documents (Lq = Lk per document)
    "docs_motif3_causal": (501, M3, "bf16", DOCS, DOCS, 0),
    "docs_motif3_w80": (502, M3, "bf16", DOCS, DOCS, 80),
    "docs_motif2_causal": (503, M2, "bf16", [129, 3, 300], [129, 3, 300], 0),
    "docs_tiny_bf16": (504, TINY, "bf16", [130, 5, 64, 1], [130, 5, 64, 1], 0),
    # chunks with a halo of W-1 earlier keys (Lk = Lq + W - 1), and a first chunk without
    "halo_motif3_w128": (505, M3, "bf16", [300, 257, 40], [300, 257 + 127, 40 + 127], 128),
    "halo_tiny_w16": (506, TINY, "bf16", [100, 33], [115, 48], 16),
    # more queries than keys: the first Lq - Lk queries sit at negative positions
    "fewer_keys_motif2": (507, M2, "bf16", [150, 60, 33], [100, 0, 33], 0),
    "fewer_keys_motif3_w50": (508, M3, "bf16", [140, 20], [90, 19], 50),
    # two KV heads per unit (signal heads per KV head 1 and 2)
    "ns1_r2_d128": (509, dict(S=8, N=4, Hkv=8, dqk=128, dv=128), "bf16", [70, 150], [100, 150],
                    0),
    "ns2_r2_d64": (510, dict(S=16, N=4, Hkv=8, dqk=64, dv=64), "bf16", [90, 45], [90, 60], 30),
    # fp32: matrix-core kernel (64/64 and 192/128) and the VALU kernel (40/24)
    "f32_tiny": (511, TINY, "f32", [100, 37, 1], [100, 50, 1], 0),
    "f32_d192_w37": (512, dict(S=8, N=2, Hkv=2, dqk=192, dv=128), "f32", [90, 60], [120, 60],
                     37),
    "f32_valu_odd_dims": (513, dict(S=4, N=2, Hkv=2, dqk=40, dv=24), "f32", [30, 10], [45, 5],
                          0),
}


def _case(case_id, heads, dtype, lens_q, lens_k):
    return gin.varlen_inputs(case_id, lens_q=lens_q, lens_k=lens_k, dtype=dtype, **heads)


def _run(host, dtype, window, max_seqlen_q=None, **opts):
    d = {k: U.to_dev(v, dtype) for k, v in host.items() if k not in ("cu_q", "cu_k")}
    cu_q = torch.from_numpy(host["cu_q"]).cuda()
    cu_k = torch.from_numpy(host["cu_k"]).cuda()
    mq = int(np.diff(host["cu_q"]).max()) if max_seqlen_q is None else max_seqlen_q
    return gda_fwd_varlen(d["q_sig"], d["q_noise"], d["k"], d["v"], d["lam"], d["gate"], cu_q,
                          cu_k, mq, window=window, **opts)


def _ref(host, window, **opts):
    return oracle.ref_fwd_varlen(host["q_sig"], host["q_noise"], host["k"], host["v"],
                                 host["lam"], host["gate"], host["cu_q"], host["cu_k"],
                                 window=window, **opts)


def _negative_rows(lens_q, lens_k):
    rows, start = [], 0
    for lq, lk in zip(lens_q, lens_k):
        rows += list(range(start, start + max(lq - lk, 0)))
        start += lq
    return rows


@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_full_output(name):
    case_id, heads, dtype, lens_q, lens_k, window = CASES[name]
    U.log(f"varlen parity {name} lens_q={lens_q} lens_k={lens_k} window={window}")
    host = _case(case_id, heads, dtype, lens_q, lens_k)
    got = U.to_f64(_run(host, dtype, window))
    ref = _ref(host, window)
    U.assert_close(got, ref, dtype, f"varlen {name}")
    neg = _negative_rows(lens_q, lens_k)
    if neg:
        assert (got[neg] == 0).all(), f"{name}: queries at negative positions are not zero"


def test_varlen_larger_grid_bound():
    """max_seqlen_q above every length only adds idle tiles."""
    case_id, heads, dtype, lens_q, lens_k, window = CASES["halo_motif3_w128"]
    host = _case(case_id, heads, dtype, lens_q, lens_k)
    a = _run(host, dtype, window)
    b = _run(host, dtype, window, max_seqlen_q=max(lens_q) + 300)
    torch.testing.assert_close(a, b, rtol=0, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_options(dtype):
    heads = M3 if dtype == "bf16" else TINY
    lens_q, lens_k = [120, 7, 64], [150, 7, 40]
    host = _case(520 + (dtype == "f32"), heads, dtype, lens_q, lens_k)
    # logits in place of the sigmoid values: fresh N(0,1) draws
    host["lam"] = gin.normal(520, 41, 0, host["lam"].shape, dtype)
    host["gate"] = gin.normal(520, 42, 0, host["gate"].shape, dtype)
    opts = dict(scale=0.1, lambda_logits=True, gate_logits=True)
    U.log(f"varlen options {dtype}")
    got = U.to_f64(_run(host, dtype, 60, **opts))
    U.assert_close(got, _ref(host, 60, **opts), dtype, f"varlen options {dtype}")


def test_varlen_full_size_sliding_window_chunks():
    """The sliding-window workload (L = 32768, W = 128) cut into 8 chunks of 4096 queries,
    each given the W-1 keys before it as a halo: every output row against the oracle."""
    cfg = C.MOTIF3_SWA
    L, W, P = cfg.L, cfg.window, 8
    chunk, halo = L // P, cfg.window - 1
    lens_q = [chunk] * P
    lens_k = [chunk] + [chunk + halo] * (P - 1)
    U.log(f"varlen full size: {P} chunks of {chunk} with {halo}-key halos")
    host = _case(530, M3, "bf16", lens_q, lens_k)
    got = U.to_f64(_run(host, "bf16", W))
    ref = _ref(host, W)
    U.assert_close(got, ref, "bf16", "varlen swa chunks")


def test_varlen_uniform_lengths_equal_the_batched_call():
    """Causal Motif 3 at full size (B = 2, L = 8192): the packed call with two equal
    sequences must give exactly the batched call's bits."""
    cfg = C.MOTIF3_FULL
    heads = dict(S=cfg.S, N=cfg.N, Hkv=cfg.Hkv, dqk=cfg.dqk, dv=cfg.dv)
    dev = {k: U.to_dev(v, "bf16") for k, v in
           gin.fwd_inputs(cfg.case_id, B=cfg.B, L=cfg.L, dtype="bf16", rope_dims=cfg.rope_dims,
                          **heads).items()}
    batched = gda_fwd(dev["q_sig"], dev["q_noise"], dev["k"], dev["v"], dev["lam"], dev["gate"],
                      window=0)
    flat = {k: v.reshape(cfg.B * cfg.L, *v.shape[2:]) for k, v in dev.items()}
    cu = torch.arange(0, cfg.B + 1, dtype=torch.int32, device="cuda") * cfg.L
    packed = gda_fwd_varlen(flat["q_sig"], flat["q_noise"], flat["k"], flat["v"], flat["lam"],
                            flat["gate"], cu, cu, cfg.L, window=0)
    U.log("varlen uniform == batched")
    assert torch.equal(packed.reshape(batched.shape), batched)
