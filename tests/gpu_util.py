"""Helpers of the GPU tests: seeded inputs to the device, oracle comparison.

Inputs come from ``attention_gda_fwd_amd.inputs`` (no method arithmetic);
expected values only from ``oracle`` (fp64 CPU)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from attention_gda_fwd_amd import inputs as gin
from attention_gda_fwd_amd.api import gda_decode, gda_fwd

# Tolerances the target states: bf16 inputs with fp32 accumulation, and fp32.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def log(msg: str) -> None:
    print(f"[gda-test {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def host_cpu() -> str:
    """CPU model and the threads the oracle runs on, for timing logs."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {oracle.threads()} oracle threads"


def to_dev(a: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> dict:
    err = np.abs(got - ref)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 max_ref=float(np.abs(ref).max()))
    log(f"{what}: max|err| {stats['max_abs']:.3e} mean|err| {stats['mean_abs']:.3e} "
        f"max|ref| {stats['max_ref']:.3e}")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "bf16":
        assert stats["max_abs"] <= BF16_MAX_ABS, f"{what}: {stats}"
        assert stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {stats}"
    else:
        assert stats["max_abs"] <= F32_MAX_ABS, f"{what}: {stats}"
    return stats


class FwdCase:
    """A prefill problem: host inputs (storage arrays), device tensors, runners."""

    def __init__(self, case_id, *, B, L, S, N, Hkv, dqk, dv, window, dtype, rope_dims=0):
        self.shape = dict(B=B, L=L, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv)
        self.window, self.dtype = window, dtype
        self.host = gin.fwd_inputs(case_id, B=B, L=L, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv,
                                   dtype=dtype, rope_dims=rope_dims)
        self.dev = {k: to_dev(v, dtype) for k, v in self.host.items()}

    def run_gpu(self, window=None) -> torch.Tensor:
        d = self.dev
        return gda_fwd(d["q_sig"], d["q_noise"], d["k"], d["v"], d["lam"], d["gate"],
                       window=self.window if window is None else window)

    def run_oracle(self, rows=None, window=None) -> np.ndarray:
        h = self.host
        return oracle.ref_fwd(h["q_sig"], h["q_noise"], h["k"], h["v"], h["lam"], h["gate"],
                              window=self.window if window is None else window, rows=rows)

