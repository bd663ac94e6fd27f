"""GPU parity of the training-form forward (gda_fwd_train) and the backward (gda_bwd)
against the fp64 oracle, through the C ABI.

* The training forward's output must match the plain forward's to one bf16 rounding
  (same kernel; the extra stores can change how the compiler fuses multiply-adds) and
  the oracle's; its per-path outputs and log-sum-exps are compared with the oracle's.
* Every gradient (dq_sig, dq_noise, dk, dv, dlambda, dgate) at oracle-friendly sizes for
  the compiled head layouts, causal and windowed, with the call options; and at the
  full Motif-3 sizes on sampled query and key rows (the causal layer's last keys, which
  only the last queries see, and rows anywhere in the sliding-window layer).

Tolerances. The forward's bf16 bar (max |err| <= 2e-2 and mean |err| <= 2e-3 on O(1)
outputs) applied to each gradient tensor relative to its largest magnitude: the
backward rounds P, dS and dO to bf16 before each matrix product (relative error
2^-9 per operand) and accumulates in fp32, so errors scale with the gradient's size (with
a floor of 0.05 for the magnitude, for gradients that vanish identically). Beside it,
a per-row bound: each row (one token's gradient vector for one head, or a token's
dlambda over the signal heads) must be within 5% of that row's own largest magnitude
plus 0.3% of the tensor's, so that small late-row gradients are not judged only
against the tensor's largest row. The absolute part is needed because a row's error
does not shrink with its gradient: dQ and dK come from dS = P (dP - delta), where dP
is formed from the bf16-rounded dO and V, so the rounding error follows |dO| |V|
rather than the (often much smaller) difference. Measured worst rows sit at 0.6 of
this bound; an error of a few tens of percent on a row of 0.05 exceeds it.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_gda_fwd_amd import configs as C
from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import gda_bwd, gda_fwd, gda_fwd_train

from . import gpu_util as U

pytestmark = pytest.mark.gpu

GRADS = ("dq_sig", "dq_noise", "dk", "dv", "dlam", "dgate")
ARGS = ("q_sig", "q_noise", "k", "v", "lam", "gate")


# Per-row bound: max |err| over a row <= ROW_REL * max |ref| over the row
# + ROW_ABS * the tensor's largest magnitude.
ROW_REL, ROW_ABS = 5e-2, 3e-3


def assert_grad_close(got, ref, what):
    # A gradient that vanishes identically (a one-key window makes dS = P (dP - delta)
    # zero) is held to the bound of an O(0.05) gradient: 1e-3 absolute.
    scale = max(float(np.abs(ref).max()), 0.05)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    rows_err = err.reshape(-1, err.shape[-1]).max(axis=1)
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    row_ratio = rows_err / (ROW_REL * rows_ref + ROW_ABS * scale)
    worst = int(np.argmax(row_ratio))
    U.log(f"{what}: max|err| {err.max():.3e} mean|err| {err.mean():.3e} max|ref| {scale:.3e}; "
          f"worst row {worst}: err {rows_err[worst]:.3e} / max|ref| {rows_ref[worst]:.3e} "
          f"= {row_ratio[worst]:.3f} of the row bound")
    assert err.max() <= 2e-2 * scale, f"{what}: max {err.max():.3e} > 2e-2 * {scale:.3e}"
    assert err.mean() <= 2e-3 * scale, f"{what}: mean {err.mean():.3e} > 2e-3 * {scale:.3e}"
    assert row_ratio[worst] <= 1.0, (
        f"{what}: row {worst} error {rows_err[worst]:.3e} > {ROW_REL} * {rows_ref[worst]:.3e}"
        f" + {ROW_ABS} * {scale:.3e}")


def make(case_id, *, B, L, S, N, Hkv, dqk, dv, rope_dims=0, logits=False):
    x = gin.fwd_inputs(case_id, B=B, L=L, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv, dtype="bf16",
                       rope_dims=rope_dims)
    if logits:
        x["lam"] = np.stack([gin.normal(case_id, 41, b, (L, S), "bf16") for b in range(B)])
        x["gate"] = np.stack([gin.normal(case_id, 42, b, (L, S, dv), "bf16") for b in range(B)])
    x["d_out"] = np.stack([gin.normal(case_id, 50, b, (L, S, dv), "bf16") for b in range(B)])
    return x


def run_gpu(x, window, **opts):
    d = {n: U.to_dev(a, "bf16") for n, a in x.items()}
    out, hs, hn, lse = gda_fwd_train(*(d[n] for n in ARGS), window=window, **opts)
    grads = gda_bwd(*(d[n] for n in ARGS), hs, hn, lse, d["d_out"], window=window, **opts)
    return d, (out, hs, hn, lse), {n: U.to_f64(g) for n, g in grads.items()}


SMALL = {
    "motif3_B2_L200_causal": (611, dict(B=2, L=200, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                        rope_dims=64), 0, {}),
    "motif3_L300_w80": (612, dict(B=1, L=300, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                  rope_dims=64), 80, {}),
    "motif2_L150_causal": (613, dict(B=1, L=150, S=32, N=8, Hkv=16, dqk=128, dv=128), 0, {}),
    "tiny_B2_L130_causal": (614, dict(B=2, L=130, S=8, N=2, Hkv=2, dqk=64, dv=64), 0, {}),
    "tiny_L97_w16": (615, dict(B=1, L=97, S=8, N=2, Hkv=2, dqk=64, dv=64), 16, {}),
    "ns1_r2_L120": (616, dict(B=1, L=120, S=8, N=4, Hkv=8, dqk=128, dv=128), 0, {}),
    "motif3_L160_options": (617, dict(B=1, L=160, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                      rope_dims=64), 40,
                            dict(scale=0.1, lambda_logits=True, gate_logits=True)),
    "tiny_L70_gate_logits": (618, dict(B=1, L=70, S=8, N=2, Hkv=2, dqk=64, dv=64), 0,
                             dict(gate_logits=True)),
    # edges: one token; a window of one key (each query sees only itself); a window
    # longer than the sequence (plain causal); a length just past a 32-row tile
    "edge_tiny_B2_L1": (619, dict(B=2, L=1, S=8, N=2, Hkv=2, dqk=64, dv=64), 0, {}),
    "edge_motif3_L40_w1": (620, dict(B=1, L=40, S=64, N=16, Hkv=16, dqk=192, dv=128,
                                     rope_dims=64), 1, {}),
    "edge_motif2_L33_w500": (621, dict(B=2, L=33, S=32, N=8, Hkv=16, dqk=128, dv=128), 500,
                             {}),
    # head layouts whose noise heads' groups span several prefill sub-units: g = 8 on
    # one KV head, a group over four KV heads, two noise heads on one KV head
    "g8_ns8_L140": (622, dict(B=1, L=140, S=32, N=4, Hkv=4, dqk=128, dv=128), 0, {}),
    "g8_r4_L130_w40": (623, dict(B=1, L=130, S=16, N=2, Hkv=8, dqk=192, dv=128), 40, {}),
    "nn2_g2_L110": (624, dict(B=2, L=110, S=16, N=8, Hkv=4, dqk=64, dv=64), 0, {}),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward_small(name):
    case_id, shp, window, opts = SMALL[name]
    U.log(f"backward parity {name} window={window} {opts}")
    x = make(case_id, logits=bool(opts), **shp)
    d, (out, hs, hn, lse), got = run_gpu(x, window, **opts)
    plain = U.to_f64(gda_fwd(*(d[n] for n in ARGS), window=window, **opts))
    o = U.to_f64(out)
    # The same kernel with extra stores: the compiler may fuse the combine's
    # multiply-adds differently, so the two outputs may differ by one bf16 rounding.
    step = np.abs(o - plain) <= 2.0 ** -7 * np.maximum(np.abs(o), np.abs(plain)) + 1e-5
    assert step.all(), "training forward output differs from the plain forward"
    r_out, r_hs, r_hn, r_lse = oracle.ref_fwd_train(*(x[n] for n in ARGS), window=window, **opts)
    U.assert_close(o, r_out, "bf16", f"{name} out")
    U.assert_close(U.to_f64(hs), r_hs, "bf16", f"{name} h_sig")
    U.assert_close(U.to_f64(hn), r_hn, "bf16", f"{name} h_noise")
    lse_err = np.abs(U.to_f64(lse) - r_lse).max()
    U.log(f"{name} lse max|err| {lse_err:.3e}")
    assert lse_err <= 1e-3, f"{name}: lse error {lse_err:.3e}"
    ref = oracle.ref_bwd(*(x[n] for n in ARGS), x["d_out"], window=window, **opts)
    for n in GRADS:
        assert_grad_close(got[n], ref[n], f"{name} {n}")


def _sampled(cfg, q_t, k_s, case_id):
    shp = dict(B=cfg.B, L=cfg.L, S=cfg.S, N=cfg.N, Hkv=cfg.Hkv, dqk=cfg.dqk, dv=cfg.dv,
               rope_dims=cfg.rope_dims)
    x = make(case_id, **shp)
    _, _, got = run_gpu(x, cfg.window)
    torch.cuda.synchronize()
    L = cfg.L
    q_rows = [b * L + t for b in range(cfg.B) for t in q_t]
    k_rows = [b * L + s for b in range(cfg.B) for s in k_s]
    U.log(f"oracle backward on {len(q_rows)} query rows and {len(k_rows)} key rows "
          f"({U.host_cpu()})")
    ref = oracle.ref_bwd(*(x[n] for n in ARGS), x["d_out"], window=cfg.window, q_rows=q_rows,
                         k_rows=k_rows)
    flat = {n: g.reshape((cfg.B * L,) + g.shape[2:]) for n, g in got.items()}
    for n in ("dq_sig", "dq_noise", "dlam", "dgate"):
        assert_grad_close(flat[n][q_rows], ref[n], f"{cfg.name} {n} sampled")
    for n in ("dk", "dv"):
        assert_grad_close(flat[n][k_rows], ref[n], f"{cfg.name} {n} sampled")


def test_backward_full_size_causal_sampled():
    """Motif-3 full layer (B = 2, L = 8192): query rows across the sequence, and the last
    48 keys plus key 8000 (which only the queries after them see)."""
    cfg = C.MOTIF3_FULL
    L = cfg.L
    _sampled(cfg, [0, 1, 63, 64, 2047, 4095, 6000, L - 2, L - 1],
             list(range(L - 48, L)) + [8000], 631)


def test_backward_full_size_causal_early_keys():
    """Motif-3 full layer: dK/dV of early keys of batch row 0 (keys 0, 63, 64 and 4095),
    which accumulate over thousands of queries across many query tiles of the dK/dV
    kernel. The oracle needs every query row of that sequence (about a minute)."""
    cfg = C.MOTIF3_FULL
    shp = dict(B=cfg.B, L=cfg.L, S=cfg.S, N=cfg.N, Hkv=cfg.Hkv, dqk=cfg.dqk, dv=cfg.dv,
               rope_dims=cfg.rope_dims)
    x = make(633, **shp)
    _, _, got = run_gpu(x, cfg.window)
    torch.cuda.synchronize()
    k_rows = [0, 63, 64, 4095]
    U.log(f"oracle backward on key rows {k_rows} of batch row 0 ({U.host_cpu()})")
    ref = oracle.ref_bwd(*(x[n] for n in ARGS), x["d_out"], window=cfg.window, q_rows=[0],
                         k_rows=k_rows)
    for n in ("dk", "dv"):
        flat = got[n].reshape((cfg.B * cfg.L,) + got[n].shape[2:])
        assert_grad_close(flat[k_rows], ref[n], f"{cfg.name} {n} early keys")


def test_backward_full_size_sliding_window_sampled():
    """Motif-3 sliding-window layer (L = 32768, W = 128): rows anywhere."""
    cfg = C.MOTIF3_SWA
    L = cfg.L
    rows = [0, 1, 127, 128, 5000, 16383, 16384, 30001, L - 2, L - 1]
    _sampled(cfg, rows, rows, 632)
