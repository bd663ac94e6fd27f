"""GPU parity: libgda (through its C ABI) against the fp64 oracle on the same seeded inputs.

* Full outputs at sizes the oracle finishes in seconds, with every workload's head
  layout, several tiles and a ragged tail.
* The full-size workloads as the bench runs them (both windows for decode),
  every output element.
Tolerances: bf16 max |err| <= 2e-2 and mean |err| <= 2e-3; fp32 max |err| <= 1e-5.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from attention_gda_fwd_amd import configs as C
from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import gda_decode, gda_decode_latent, gda_fwd

from . import gpu_util as U

pytestmark = pytest.mark.gpu

SMALL = {
    # the fp32 workload itself, every output
    "tiny_f32_L256_full": dict(case_id=0, B=1, L=256, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0,
                          dtype="f32"),
    "motif2_layout_L300": dict(case_id=101, B=1, L=300, S=32, N=8, Hkv=16, dqk=128, dv=128,
                               window=0, dtype="bf16"),
    "motif3_layout_B2_L200": dict(case_id=102, B=2, L=200, S=64, N=16, Hkv=16, dqk=192,
                                  dv=128, window=0, dtype="bf16", rope_dims=64),
    "motif3_swa128_L700": dict(case_id=103, B=1, L=700, S=64, N=16, Hkv=16, dqk=192, dv=128,
                               window=128, dtype="bf16", rope_dims=64),
    "tiny_layout_bf16_B2_L130": dict(case_id=104, B=2, L=130, S=8, N=2, Hkv=2, dqk=64, dv=64,
                                     window=0, dtype="bf16"),
    "motif2_layout_f32_L100": dict(case_id=105, B=1, L=100, S=32, N=8, Hkv=16, dqk=128, dv=128,
                                   window=0, dtype="f32"),
    # fp32 matrix-core kernel: head size 192 with a window and a ragged tail; g = 8
    # signal heads per noise head (one wave takes a second head); more noise heads
    # than KV heads
    "f32_d192_w37_B2_L200": dict(case_id=106, B=2, L=200, S=8, N=2, Hkv=2, dqk=192, dv=128,
                                 window=37, dtype="f32"),
    "f32_g8_L77": dict(case_id=107, B=1, L=77, S=16, N=2, Hkv=2, dqk=64, dv=64, window=0,
                       dtype="f32"),
    "f32_n4_hkv2_w16_L90": dict(case_id=108, B=1, L=90, S=8, N=4, Hkv=2, dqk=128, dv=128,
                                window=16, dtype="f32"),
    # fp32 at a head size with no matrix-core instance (the VALU kernel)
    "f32_odd_dims_L50": dict(case_id=109, B=2, L=50, S=4, N=2, Hkv=2, dqk=40, dv=24, window=0,
                             dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_full_output(name):
    kw = SMALL[name]
    U.log(f"parity {name} {kw}")
    case = U.FwdCase(**kw)
    got = U.to_f64(case.run_gpu())
    torch.cuda.synchronize()
    ref = case.run_oracle()
    U.assert_close(got, ref, kw["dtype"], name)


# bf16 prefill head layouts (S, N, Hkv) at every head size, causal and with a
# window: several key tiles and a ragged tail, so every tile shape, the partial
# last tile and every wave split run against the oracle. The names give
# NS = S/Hkv signal heads per KV head, R = Hkv/N KV heads per noise head (or NN =
# N/Hkv noise heads per KV head) and g = S/N signal heads per noise head. The
# first five take one sub-unit per noise head; the rest split a noise head's
# signal heads over several sub-units (g = 3, 5, 6, 8, 16), put several noise
# heads on one KV head (NN = 2, 4) or spread a group over 4 or 8 KV heads.
LAYOUTS = {"ns1_r1": (4, 4, 4), "ns2_r1": (8, 4, 4), "ns4_r1": (16, 4, 4),
           "ns1_r2": (8, 4, 8), "ns2_r2": (16, 4, 8),
           "ns8_r1_g8": (32, 4, 4), "ns3_r1_g3": (12, 4, 4), "ns5_r1_g5": (10, 2, 2),
           "nn2_g2": (16, 8, 4), "nn2_g4": (16, 4, 2), "nn4_g1": (8, 8, 2),
           "ns4_r2_g8": (32, 4, 8), "ns3_r2_g6": (24, 4, 8), "ns1_r4_g4": (8, 2, 8),
           "ns2_r4_g8": (16, 2, 8), "ns2_r8_g16": (16, 1, 8)}
DIMS = {"d64": (64, 64), "d128": (128, 128), "d192": (192, 128)}


@pytest.mark.parametrize("window", [0, 80], ids=["causal", "w80"])
@pytest.mark.parametrize("dims", sorted(DIMS))
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_layout_sweep(layout, dims, window):
    S, N, Hkv = LAYOUTS[layout]
    dqk, dv = DIMS[dims]
    cid = 300 + 10 * sorted(LAYOUTS).index(layout) + sorted(DIMS).index(dims)
    kw = dict(B=1, L=231, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv, window=window, dtype="bf16")
    U.log(f"parity layout {layout} {dims} window={window} {kw}")
    case = U.FwdCase(cid, **kw)
    got = U.to_f64(case.run_gpu())
    torch.cuda.synchronize()
    ref = case.run_oracle()
    U.assert_close(got, ref, "bf16", f"{layout} {dims} window={window}")


# Sliding windows over batches with many sub-units: ragged tails, windows from 1
# key to 194, one to eight signal heads per noise head, two noise heads per KV
# head, and every head size.
SWA_CASES = {
    "motif3_B4_L1000_w128": dict(B=4, L=1000, S=64, N=16, Hkv=16, dqk=192, dv=128, window=128),
    "motif3_B4_L1000_w129": dict(B=4, L=1000, S=64, N=16, Hkv=16, dqk=192, dv=128, window=129),
    "motif3_B4_L1000_w130": dict(B=4, L=1000, S=64, N=16, Hkv=16, dqk=192, dv=128, window=130),
    "motif3_B4_L777_w1": dict(B=4, L=777, S=64, N=16, Hkv=16, dqk=192, dv=128, window=1),
    "motif3_B4_L777_w33": dict(B=4, L=777, S=64, N=16, Hkv=16, dqk=192, dv=128, window=33),
    "g8_B4_L900_w97": dict(B=4, L=900, S=64, N=8, Hkv=8, dqk=192, dv=128, window=97),
    "g3_B8_L600_w64": dict(B=8, L=600, S=24, N=8, Hkv=8, dqk=192, dv=128, window=64),
    "g1_B16_L300_w128": dict(B=16, L=300, S=16, N=16, Hkv=16, dqk=192, dv=128, window=128),
    "nn2_B8_L500_w80": dict(B=8, L=500, S=32, N=16, Hkv=8, dqk=192, dv=128, window=80),
    "d128_B4_L1000_w193": dict(B=4, L=1000, S=64, N=16, Hkv=16, dqk=128, dv=128, window=193),
    "d128_B4_L1000_w194": dict(B=4, L=1000, S=64, N=16, Hkv=16, dqk=128, dv=128, window=194),
    "d128_g2_B8_L700_w128": dict(B=8, L=700, S=32, N=16, Hkv=16, dqk=128, dv=128, window=128),
    "d64_B8_L700_w100": dict(B=8, L=700, S=16, N=4, Hkv=4, dqk=64, dv=64, window=100),
}


@pytest.mark.parametrize("name", sorted(SWA_CASES))
def test_sliding_window_batches(name):
    kw = dict(SWA_CASES[name], dtype="bf16")
    cid = 600 + sorted(SWA_CASES).index(name)
    U.log(f"parity sliding window {name} {kw}")
    case = U.FwdCase(cid, **kw)
    got = U.to_f64(case.run_gpu())
    torch.cuda.synchronize()
    ref = case.run_oracle()
    U.assert_close(got, ref, "bf16", name)


@pytest.mark.parametrize("cfg", [C.MOTIF2, C.MOTIF3_SWA, C.MOTIF3_FULL_SHARD8, C.MOTIF3_FULL],
                         ids=lambda c: c.name)
def test_full_size_full_output(cfg):
    """The full-size prefill workloads as the bench runs them, every output element
    against the oracle (fp64, all host cores; the Motif-3 full layer takes ~2 minutes)."""
    U.log(f"parity {cfg.name}: generating inputs")
    case = U.FwdCase(cfg.case_id, B=cfg.B, L=cfg.L, S=cfg.S, N=cfg.N, Hkv=cfg.Hkv, dqk=cfg.dqk,
                     dv=cfg.dv, window=cfg.window, dtype=cfg.dtype, rope_dims=cfg.rope_dims)
    U.log(f"parity {cfg.name}: running gda_fwd")
    got = U.to_f64(case.run_gpu())
    torch.cuda.synchronize()
    U.log(f"parity {cfg.name}: oracle on all {cfg.B * cfg.L} rows")
    t0 = time.perf_counter()
    ref = case.run_oracle()
    dt = time.perf_counter() - t0
    U.log(f"parity {cfg.name}: oracle {dt:.1f} s = {cfg.flops() / dt / 1e9:.1f} GFLOP/s, "
          f"{cfg.tokens() / dt:.0f} tokens/s ({U.host_cpu()})")
    U.assert_close(got, ref, cfg.dtype, f"{cfg.name} full output")


def _decode_case(case_id, *, B, Lmax, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    host = gin.decode_inputs(case_id, B=B, Lmax=Lmax, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv,
                             dtype=dtype, rope_dims=rope_dims)
    return host, {k: U.to_dev(v, dtype) for k, v in host.items()}


DEC_SMALL = {
    "motif3_layout": dict(case_id=201, B=6, Lmax=300, S=64, N=16, Hkv=16, dqk=192, dv=128,
                          dtype="bf16", rope_dims=64),
    "motif2_layout": dict(case_id=202, B=6, Lmax=300, S=32, N=8, Hkv=16, dqk=128, dv=128,
                          dtype="bf16"),
    "tiny_layout_f32": dict(case_id=203, B=6, Lmax=300, S=8, N=2, Hkv=2, dqk=64, dv=64,
                            dtype="f32"),
}


@pytest.mark.parametrize("window", [0, 128, 1])
@pytest.mark.parametrize("name", sorted(DEC_SMALL))
def test_decode_small_ragged(name, window):
    kw = DEC_SMALL[name]
    U.log(f"decode parity {name} window={window}")
    host, dev = _decode_case(**kw)
    lens = np.array([300, 1, 77, 128, 129, 0], dtype=np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    out = gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"], dev["lam"],
                     dev["gate"], cache_lens=lens_d, window=window)
    got = U.to_f64(out)
    ref = oracle.ref_decode(host["q_sig"], host["q_noise"], host["k_cache"], host["v_cache"],
                            host["lam"], host["gate"], lens, window=window)
    U.assert_close(got, ref, kw["dtype"], f"decode {name} W={window}")
    assert np.all(got[5] == 0.0), "a sequence with no visible key must give zeros"
    # NULL lens = every sequence holds Lmax tokens; lens above Lmax clamp to Lmax
    out_full = U.to_f64(gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"],
                                   dev["lam"], dev["gate"], window=window))
    big = torch.full((kw["B"],), 10**6, dtype=torch.int32, device="cuda")
    out_big = U.to_f64(gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"],
                                  dev["lam"], dev["gate"], cache_lens=big, window=window))
    assert np.array_equal(out_full, out_big)
    np.testing.assert_array_equal(out_full[0], got[0])


# Spans of 2048 keys and more take the streaming decode kernel (K/V chunks copied
# to LDS); shorter ones the kernel above. Ragged lengths: a partial last chunk,
# a single key, an empty cache, chunk-count edges.
DEC_STREAM = {
    "motif3_layout": dict(case_id=211, B=6, Lmax=2100, S=64, N=16, Hkv=16, dqk=192, dv=128,
                          dtype="bf16", rope_dims=64),
    "motif2_layout": dict(case_id=212, B=6, Lmax=2100, S=32, N=8, Hkv=16, dqk=128, dv=128,
                          dtype="bf16"),
    "tiny_layout": dict(case_id=213, B=6, Lmax=2100, S=8, N=2, Hkv=2, dqk=64, dv=64,
                        dtype="bf16"),
}


@pytest.mark.parametrize("window", [0, 2050])
@pytest.mark.parametrize("name", sorted(DEC_STREAM))
def test_decode_stream_ragged(name, window):
    kw = DEC_STREAM[name]
    U.log(f"decode (streaming) parity {name} window={window}")
    host, dev = _decode_case(**kw)
    lens = np.array([2100, 1, 2048, 2049, 1377, 0], dtype=np.int32)
    out = gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"], dev["lam"],
                     dev["gate"], cache_lens=torch.from_numpy(lens).cuda(), window=window)
    got = U.to_f64(out)
    ref = oracle.ref_decode(host["q_sig"], host["q_noise"], host["k_cache"], host["v_cache"],
                            host["lam"], host["gate"], lens, window=window)
    U.assert_close(got, ref, "bf16", f"decode stream {name} W={window}")
    assert np.all(got[5] == 0.0), "a sequence with no visible key must give zeros"


# Decode head layouts whose units hold more than the 16 query heads of one MFMA
# tile, so the workgroups split them (and recompute the noise heads they need):
# a group over two KV heads with 16 signal heads on each; four noise heads on a
# KV head with 16 signal heads; one noise head serving 32 signal heads on one KV
# head; and a group over four KV heads (no split). (S, N, Hkv, dqk, dv), both
# decode kernels (short spans and the streaming one), causal and windowed.
DEC_LAYOUTS = {"ns16_r2_g32": (32, 1, 2, 64, 64), "ns16_nn4_g4": (64, 16, 4, 192, 128),
               "ns32_r1_g32": (32, 1, 1, 128, 128), "ns2_r4_g8": (16, 2, 8, 192, 128)}


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("lmax", [300, 2100], ids=["short", "stream"])
@pytest.mark.parametrize("layout", sorted(DEC_LAYOUTS))
def test_decode_layouts(layout, lmax, window):
    S, N, Hkv, dqk, dv = DEC_LAYOUTS[layout]
    cid = 250 + sorted(DEC_LAYOUTS).index(layout)
    U.log(f"decode layout parity {layout} Lmax={lmax} window={window}")
    host, dev = _decode_case(cid, B=4, Lmax=lmax, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv,
                             dtype="bf16")
    lens = np.array([lmax, 1, lmax // 2 + 3, 0], dtype=np.int32)
    out = gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"], dev["lam"],
                     dev["gate"], cache_lens=torch.from_numpy(lens).cuda(), window=window)
    got = U.to_f64(out)
    ref = oracle.ref_decode(host["q_sig"], host["q_noise"], host["k_cache"], host["v_cache"],
                            host["lam"], host["gate"], lens, window=window)
    U.assert_close(got, ref, "bf16", f"decode {layout} Lmax={lmax} W={window}")
    assert np.all(got[3] == 0.0), "a sequence with no visible key must give zeros"


# Call options: an explicit softmax scale, and lambda/gate given as logits (the kernels
# apply the sigmoid). The logits are fresh N(0,1) draws in place of the sigmoid values.
OPT_FWD = {
    "bf16_motif3_w80_L200": (dict(case_id=121, B=1, L=200, S=64, N=16, Hkv=16, dqk=192,
                                  dv=128, window=80, dtype="bf16", rope_dims=64),
                             dict(scale=0.11, lambda_logits=True, gate_logits=True)),
    "bf16_motif2_L150": (dict(case_id=122, B=1, L=150, S=32, N=8, Hkv=16, dqk=128, dv=128,
                              window=0, dtype="bf16"), dict(scale=0.2, lambda_logits=True)),
    "bf16_tiny_L99": (dict(case_id=123, B=2, L=99, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0,
                           dtype="bf16"), dict(gate_logits=True)),
    "f32_tiny_L100": (dict(case_id=124, B=1, L=100, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0,
                           dtype="f32"), dict(scale=0.3, lambda_logits=True, gate_logits=True)),
    "f32_odd_dims_L40": (dict(case_id=125, B=1, L=40, S=4, N=2, Hkv=2, dqk=40, dv=24, window=7,
                              dtype="f32"), dict(scale=0.25, gate_logits=True)),
}


def _logits(case_id, shape, dtype):
    return np.stack([gin.normal(case_id, 40 + len(shape), b, shape[1:], dtype)
                     for b in range(shape[0])])


@pytest.mark.parametrize("name", sorted(OPT_FWD))
def test_fwd_options(name):
    kw, opts = OPT_FWD[name]
    U.log(f"options parity {name} {opts}")
    case = U.FwdCase(**kw)
    if opts.get("lambda_logits"):
        case.host["lam"] = _logits(kw["case_id"], case.host["lam"].shape, kw["dtype"])
    if opts.get("gate_logits"):
        case.host["gate"] = _logits(kw["case_id"], case.host["gate"].shape, kw["dtype"])
    d = {k: U.to_dev(v, kw["dtype"]) for k, v in case.host.items()}
    got = U.to_f64(gda_fwd(d["q_sig"], d["q_noise"], d["k"], d["v"], d["lam"], d["gate"],
                           window=kw["window"], **opts))
    h = case.host
    ref = oracle.ref_fwd(h["q_sig"], h["q_noise"], h["k"], h["v"], h["lam"], h["gate"],
                         window=kw["window"], **opts)
    U.assert_close(got, ref, kw["dtype"], f"options {name}")


OPT_DEC = {
    "short_motif3": (DEC_SMALL["motif3_layout"], 0,
                     dict(scale=0.09, lambda_logits=True, gate_logits=True)),
    "short_f32": (DEC_SMALL["tiny_layout_f32"], 5, dict(scale=0.3, gate_logits=True)),
    "stream_tiny": (DEC_STREAM["tiny_layout"], 0,
                    dict(scale=0.2, lambda_logits=True, gate_logits=True)),
    "stream_motif2": (DEC_STREAM["motif2_layout"], 0, dict(lambda_logits=True)),
}


@pytest.mark.parametrize("name", sorted(OPT_DEC))
def test_decode_options(name):
    kw, window, opts = OPT_DEC[name]
    U.log(f"decode options parity {name} {opts}")
    host, _ = _decode_case(**kw)
    if opts.get("lambda_logits"):
        host["lam"] = _logits(kw["case_id"], host["lam"].shape, kw["dtype"])
    if opts.get("gate_logits"):
        host["gate"] = _logits(kw["case_id"], host["gate"].shape, kw["dtype"])
    dev = {k: U.to_dev(v, kw["dtype"]) for k, v in host.items()}
    lens = np.array([kw["Lmax"], 1, 77, kw["Lmax"] - 1, 40, 0], dtype=np.int32)
    out = gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"], dev["lam"],
                     dev["gate"], cache_lens=torch.from_numpy(lens).cuda(), window=window, **opts)
    ref = oracle.ref_decode(host["q_sig"], host["q_noise"], host["k_cache"], host["v_cache"],
                            host["lam"], host["gate"], lens, window=window, **opts)
    U.assert_close(U.to_f64(out), ref, kw["dtype"], f"decode options {name}")


# Latent-cache decode (the cache is c_kv [Lmax, 512] + k_rope [Lmax, 64] per sequence,
# expanded by W^KV_b): every query-head count the kernel splits into waves (80, 40 and 10
# heads: 5, 3 and 1 waves), ragged lengths (a partial last chunk, one key, an empty cache),
# windows and the call options.
LAT_SMALL = {
    "motif3_heads": dict(case_id=231, B=5, Lmax=700, S=64, N=16, Hkv=16),
    "motif2_heads": dict(case_id=232, B=5, Lmax=700, S=32, N=8, Hkv=16),
    "tiny_heads": dict(case_id=233, B=5, Lmax=700, S=8, N=2, Hkv=2),
}
LAT_DIMS = dict(Dn=128, Dr=64, Dc=512, dv=128)


def _latent_case(case_id, B, Lmax, S, N, Hkv):
    host = gin.decode_latent_inputs(case_id, B=B, Lmax=Lmax, S=S, N=N, Hkv=Hkv, dtype="bf16",
                                    **LAT_DIMS)
    return host, {k: U.to_dev(v, "bf16") for k, v in host.items()}


def _run_latent(dev, lens, window, **opts):
    return gda_decode_latent(dev["q_sig"], dev["q_noise"], dev["c_kv"], dev["k_rope"],
                             dev["w_kv_b"], dev["lam"], dev["gate"], cache_lens=lens,
                             window=window, **opts)


def _ref_latent(host, lens, window, **opts):
    return oracle.ref_decode_latent(host["q_sig"], host["q_noise"], host["c_kv"],
                                    host["k_rope"], host["w_kv_b"], host["lam"], host["gate"],
                                    lens, window=window, **opts)


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("name", sorted(LAT_SMALL))
def test_latent_small_ragged(name, window):
    kw = LAT_SMALL[name]
    U.log(f"latent decode parity {name} window={window}")
    host, dev = _latent_case(**kw)
    lens = np.array([700, 1, 33, 0, 517], dtype=np.int32)
    got = U.to_f64(_run_latent(dev, torch.from_numpy(lens).cuda(), window))
    ref = _ref_latent(host, lens, window)
    U.assert_close(got, ref, "bf16", f"latent {name} W={window}")
    assert np.all(got[3] == 0.0), "an empty cache must give zeros"


# The merge takes 16 // (1 + g) sequences per workgroup: g = 1 puts 8 sequences in a
# workgroup (9 sequences: a full group and a lone one), g = 8 one; empty caches among
# them.
LAT_GROUPS = {
    "g1_B9": (dict(case_id=234, B=9, Lmax=300, S=16, N=16, Hkv=16),
              [300, 0, 17, 1, 300, 255, 0, 64, 129]),
    "g8_B3": (dict(case_id=235, B=3, Lmax=300, S=64, N=8, Hkv=8), [300, 0, 77]),
}


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("name", sorted(LAT_GROUPS))
def test_latent_merge_groups(name, window):
    kw, lens_l = LAT_GROUPS[name]
    U.log(f"latent decode parity {name} window={window}")
    host, dev = _latent_case(**kw)
    lens = np.array(lens_l, dtype=np.int32)
    got = U.to_f64(_run_latent(dev, torch.from_numpy(lens).cuda(), window))
    ref = _ref_latent(host, lens, window)
    U.assert_close(got, ref, "bf16", f"latent {name} W={window}")
    assert np.all(got[lens == 0] == 0.0), "an empty cache must give zeros"


def test_latent_options_and_null_lengths():
    kw = LAT_SMALL["motif3_heads"]
    host, dev = _latent_case(**kw)
    for k, tid in (("lam", 60), ("gate", 61)):
        host[k] = np.stack([gin.normal(kw["case_id"], tid, b, host[k].shape[1:], "bf16")
                            for b in range(kw["B"])])
        dev[k] = U.to_dev(host[k], "bf16")
    opts = dict(scale=0.07, lambda_logits=True, gate_logits=True)
    got = U.to_f64(_run_latent(dev, None, 0, **opts))
    ref = _ref_latent(host, None, 0, **opts)
    U.assert_close(got, ref, "bf16", "latent options, full caches")


def test_latent_full_size_sampled_sequences():
    """The full latent cache (B=64 sequences of 32768 tokens, Motif 3 heads: 2.4 GB instead
    of the expanded 21.5 GB) at W=0 and W=128; the oracle expands 4 sequences in fp64."""
    cfg = C.MOTIF3_DECODE
    B, Lmax = cfg.B, cfg.L
    shp = dict(Lmax=Lmax, S=cfg.S, N=cfg.N, dtype="bf16", **{k: LAT_DIMS[k] for k in
                                                              ("Dn", "Dr", "Dc", "dv")})
    case_id = 241
    U.log("latent full size: generating the 2.4 GB latent cache")
    dev = None
    keep = {0, 1, 37, 63}
    kept = {}
    for b in range(B):
        row = gin.decode_latent_row(case_id, b, **shp)
        if dev is None:
            dev = {k: torch.empty((B,) + v.shape, dtype=torch.bfloat16, device="cuda")
                   for k, v in row.items()}
        for k, v in row.items():
            dev[k][b].copy_(torch.from_numpy(v).view(torch.bfloat16))
        if b in keep:
            kept[b] = row
    w = gin.latent_weights(case_id, Hkv=cfg.Hkv, Dn=128, dv=128, Dc=512, dtype="bf16")
    dev["w_kv_b"] = U.to_dev(w, "bf16")
    seqs = sorted(keep)
    for window in (0, 128):
        got = U.to_f64(_run_latent(dev, None, window)[seqs])
        host = {k: np.stack([kept[b][k] for b in seqs]) for k in kept[seqs[0]]}
        host["w_kv_b"] = w
        t0 = time.perf_counter()
        ref = _ref_latent(host, None, window)
        U.log(f"latent full size W={window}: oracle on sequences {seqs} "
              f"{time.perf_counter() - t0:.1f} s ({U.host_cpu()})")
        U.assert_close(got, ref, "bf16", f"latent full size W={window}")


def test_decode_full_size_full_output():
    """The full-cache decode (B=64, Lmax=32768, Motif 3 heads) at W=0 and W=128, every
    sequence against the oracle. The 21.5 GB cache is generated on the host 8 sequences
    at a time (a thread each), kept there for the oracle and copied to the device."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = C.MOTIF3_DECODE
    shp = dict(Lmax=cfg.L, S=cfg.S, N=cfg.N, Hkv=cfg.Hkv, dqk=cfg.dqk, dv=cfg.dv,
               dtype=cfg.dtype, rope_dims=cfg.rope_dims)
    host = None
    U.log("decode full size: generating the 21.5 GB cache")
    with ThreadPoolExecutor(8) as ex:
        for b0 in range(0, cfg.B, 8):
            rows = ex.map(lambda b: gin.decode_row(cfg.case_id, b, **shp), range(b0, b0 + 8))
            for b, row in zip(range(b0, b0 + 8), rows):
                if host is None:
                    host = {k: np.empty((cfg.B,) + v.shape, v.dtype) for k, v in row.items()}
                for k, v in row.items():
                    host[k][b] = v
            U.log(f"  generated {b0 + 8}/{cfg.B} sequences")
    dev = {k: U.to_dev(v, cfg.dtype) for k, v in host.items()}
    for window in (0, 128):
        out = gda_decode(dev["q_sig"], dev["q_noise"], dev["k_cache"], dev["v_cache"],
                         dev["lam"], dev["gate"], window=window)
        got = U.to_f64(out)
        U.log(f"decode full size W={window}: oracle on all {cfg.B} sequences")
        t0 = time.perf_counter()
        ref = oracle.ref_decode(host["q_sig"], host["q_noise"], host["k_cache"],
                                host["v_cache"], host["lam"], host["gate"], None, window=window)
        dt = time.perf_counter() - t0
        U.log(f"decode full size W={window}: oracle {dt:.2f} s = "
              f"{cfg.with_(window=window).flops() / dt / 1e9:.1f} GFLOP/s ({U.host_cpu()})")
        U.assert_close(got, ref, "bf16", f"{cfg.name} W={window} full output")
