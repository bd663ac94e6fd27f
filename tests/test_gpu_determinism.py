"""Run-to-run reproducibility of every GPU entry point: the same call on the same
inputs twice gives the same bits (torch.equal). The kernels fix every reduction
order (online softmax over keys in a fixed chunk order, per-wave partials merged
in a fixed wave order, no atomics), so nothing depends on scheduling.

Sizes: the Motif 3 layer's heads and head sizes at L = 2048 (32 query tiles, both
the full-causal and the sliding-window shapes), the Motif-2 two-KV-head layout,
both decode kernels (a 300-token cache takes the short-span kernel, 4096 tokens
the streaming one), the latent-cache decode, and the training forward + backward.
"""
import numpy as np
import pytest
import torch

from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import (gda_bwd, gda_decode, gda_decode_latent, gda_fwd,
                                       gda_fwd_train)

from . import gpu_util as U

pytestmark = pytest.mark.gpu


def _dev(x):
    return {k: U.to_dev(v, "bf16") for k, v in x.items()}


def _twice(fn):
    a = fn()
    torch.cuda.synchronize()
    b = fn()
    torch.cuda.synchronize()
    return a, b


PREFILL = {
    "motif3_causal_L2048": (701, dict(B=1, L=2048, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                      rope_dims=64), 0),
    "motif3_swa128_L2048": (702, dict(B=1, L=2048, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                      rope_dims=64), 128),
    "motif2_causal_L1024": (703, dict(B=1, L=1024, S=32, N=8, Hkv=16, dqk=128, dv=128), 0),
}


@pytest.mark.parametrize("name", sorted(PREFILL))
def test_prefill_bitwise_reproducible(name):
    cid, shp, window = PREFILL[name]
    U.log(f"determinism prefill {name}")
    d = _dev(gin.fwd_inputs(cid, dtype="bf16", **shp))
    a, b = _twice(lambda: gda_fwd(d["q_sig"], d["q_noise"], d["k"], d["v"], d["lam"],
                                  d["gate"], window=window))
    assert torch.equal(a, b), f"{name}: two launches differ"


@pytest.mark.parametrize("lmax", [300, 4096], ids=["short_span", "streaming"])
@pytest.mark.parametrize("window", [0, 128])
def test_decode_bitwise_reproducible(lmax, window):
    U.log(f"determinism decode Lmax={lmax} window={window}")
    x = gin.decode_inputs(704, B=8, Lmax=lmax, S=64, N=16, Hkv=16, dqk=192, dv=128,
                          dtype="bf16", rope_dims=64)
    d = _dev(x)
    lens = torch.tensor([lmax, 1, lmax // 3, lmax - 1, 77, lmax, 2, 129], dtype=torch.int32,
                        device="cuda")
    a, b = _twice(lambda: gda_decode(d["q_sig"], d["q_noise"], d["k_cache"], d["v_cache"],
                                     d["lam"], d["gate"], cache_lens=lens, window=window))
    assert torch.equal(a, b), "two decode launches differ"


def test_latent_decode_bitwise_reproducible():
    U.log("determinism latent decode")
    x = gin.decode_latent_inputs(705, B=6, Lmax=3000, S=64, N=16, Hkv=16, Dn=128, Dr=64,
                                 Dc=512, dv=128, dtype="bf16")
    d = _dev(x)
    a, b = _twice(lambda: gda_decode_latent(d["q_sig"], d["q_noise"], d["c_kv"], d["k_rope"],
                                            d["w_kv_b"], d["lam"], d["gate"], window=0))
    assert torch.equal(a, b), "two latent decode launches differ"


def test_training_bitwise_reproducible():
    U.log("determinism training forward and backward")
    x = gin.fwd_inputs(706, B=1, L=700, S=64, N=16, Hkv=16, dqk=192, dv=128, dtype="bf16",
                       rope_dims=64)
    x["d_out"] = gin.normal(706, 50, 0, (1, 700, 64, 128), "bf16")
    d = _dev(x)
    args = [d[n] for n in ("q_sig", "q_noise", "k", "v", "lam", "gate")]

    def run():
        out, hs, hn, lse = gda_fwd_train(*args, window=0)
        g = gda_bwd(*args, hs, hn, lse, d["d_out"], window=0)
        return [out, hs, hn, lse] + [g[n] for n in sorted(g)]
    a, b = _twice(run)
    for i, (ta, tb) in enumerate(zip(a, b)):
        assert torch.equal(ta, tb), f"training output {i} differs between two runs"
    assert np.isfinite(U.to_f64(a[0])).all()
