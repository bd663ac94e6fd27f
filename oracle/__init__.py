"""fp64 CPU oracle for the GDA/GDLA attention core (ctypes front end of ``gda_ref.c``).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package. It imports nothing from the product
package and the product package imports nothing from it.

Inputs are numpy arrays at their storage type: ``uint16`` bf16 bit patterns or
``float32``. Outputs are float64.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDA_ORACLE_LIB names another build of gda_ref.c to load instead (the sanitizer
# test runs the pins against an AddressSanitizer/UBSan build); it is never rebuilt.
_OVERRIDE = os.environ.get("GDA_ORACLE_LIB")
LIB_PATH = _OVERRIDE or os.path.join(_HERE, "libgda_ref.so")
SRC = os.path.join(_HERE, "gda_ref.c")

BF16, F32 = 0, 1
LAMBDA_LOGITS, GATE_LOGITS = 1, 2


def build(force: bool = False) -> str:
    """Compile ``gda_ref.c`` with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _bind(lib):
    """Declare the C signatures on a loaded build of gda_ref.c."""
    i64, vp, ci, f64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.gda_ref_fwd.restype = ci
    lib.gda_ref_fwd.argtypes = [vp] * 7 + [i64] * 8 + [ci, vp, i64]
    lib.gda_ref_decode.restype = ci
    lib.gda_ref_decode.argtypes = [vp] * 8 + [i64] * 8 + [ci]
    lib.gda_ref_fwd_ex.restype = ci
    lib.gda_ref_fwd_ex.argtypes = [vp] * 7 + [i64] * 8 + [ci, vp, i64, f64, ci]
    lib.gda_ref_decode_ex.restype = ci
    lib.gda_ref_decode_ex.argtypes = [vp] * 8 + [i64] * 8 + [ci, f64, ci]
    lib.gda_ref_fwd_varlen.restype = ci
    lib.gda_ref_fwd_varlen.argtypes = [vp] * 9 + [i64] * 7 + [ci, f64, ci]
    lib.gda_ref_decode_latent.restype = ci
    lib.gda_ref_decode_latent.argtypes = [vp] * 9 + [i64] * 10 + [ci, f64, ci]
    lib.gda_ref_fwd_train.restype = ci
    lib.gda_ref_fwd_train.argtypes = [vp] * 10 + [i64] * 8 + [ci, f64, ci]
    lib.gda_ref_bwd.restype = ci
    lib.gda_ref_bwd.argtypes = [vp] * 13 + [i64] * 8 + [ci, f64, ci, vp, i64, vp, i64]
    lib.gda_ref_fwd_train_varlen.restype = ci
    lib.gda_ref_fwd_train_varlen.argtypes = [vp] * 12 + [i64] * 7 + [ci, f64, ci]
    lib.gda_ref_bwd_varlen.restype = ci
    lib.gda_ref_bwd_varlen.argtypes = [vp] * 15 + [i64] * 7 + [ci, f64, ci]
    lib.gda_ref_threads.restype = ci
    lib.gda_ref_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _OVERRIDE:
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


@contextlib.contextmanager
def loaded_from(path: str):
    """Run every oracle function on another build of gda_ref.c while the block runs (the
    tests build copies with one mistake planted, to show that the pins catch it)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs must be uint16 (bf16 bits) or float32, got {a.dtype}")


def _c(a: np.ndarray, code: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if _dtype_code(a) != code:
        raise TypeError("all oracle inputs must share one storage type")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(_load().gda_ref_threads())


def _flags(lambda_logits: bool, gate_logits: bool) -> int:
    return (LAMBDA_LOGITS if lambda_logits else 0) | (GATE_LOGITS if gate_logits else 0)


def ref_fwd(q_sig, q_noise, k, v, lam, gate, *, window: int, rows=None,
            scale: float | None = None, lambda_logits: bool = False,
            gate_logits: bool = False) -> np.ndarray:
    """Prefill oracle. Shapes: q_sig [B,L,S,dqk], q_noise [B,L,N,dqk], k [B,L,Hkv,dqk],
    v [B,L,Hkv,dv], lam [B,L,S], gate [B,L,S,dv]. ``rows`` selects flat (b*L + t) rows;
    the result is [B,L,S,dv] when ``rows`` is None, else [len(rows),S,dv] (float64).
    ``scale`` replaces 1/sqrt(dqk); ``lambda_logits`` / ``gate_logits`` say those inputs
    are logits (the sigmoid is applied here)."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, k, v, lam, gate = (_c(x, code) for x in (q_sig, q_noise, k, v, lam, gate))
    B, L, S, dqk = q_sig.shape
    N = q_noise.shape[2]
    Hkv, dv = v.shape[2], v.shape[3]
    assert q_noise.shape == (B, L, N, dqk) and k.shape == (B, L, Hkv, dqk)
    assert v.shape == (B, L, Hkv, dv) and lam.shape == (B, L, S) and gate.shape == (B, L, S, dv)
    if rows is None:
        out = np.empty((B, L, S, dv), dtype=np.float64)
        rows_arr, n_rows, rp = None, 0, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        n_rows = rows_arr.size
        out = np.empty((n_rows, S, dv), dtype=np.float64)
        rp = _ptr(rows_arr)
    rc = _load().gda_ref_fwd_ex(_ptr(q_sig), _ptr(q_noise), _ptr(k), _ptr(v), _ptr(lam),
                                _ptr(gate), _ptr(out), B, L, S, N, Hkv, dqk, dv, int(window),
                                code, rp, n_rows, float(scale or 0.0),
                                _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_fwd rejected its arguments (code {rc})")
    return out


def ref_decode(q_sig, q_noise, k_cache, v_cache, lam, gate, lens=None, *, window: int,
               scale: float | None = None, lambda_logits: bool = False,
               gate_logits: bool = False) -> np.ndarray:
    """Decode oracle. Shapes: q_sig [B,S,dqk], q_noise [B,N,dqk], k_cache [B,Lmax,Hkv,dqk],
    v_cache [B,Lmax,Hkv,dv], lam [B,S], gate [B,S,dv], lens int32 [B] or None (= Lmax).
    Returns [B,S,dv] float64."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, k_cache, v_cache, lam, gate = (
        _c(x, code) for x in (q_sig, q_noise, k_cache, v_cache, lam, gate))
    B, S, dqk = q_sig.shape
    N = q_noise.shape[1]
    Lmax, Hkv, dv = v_cache.shape[1], v_cache.shape[2], v_cache.shape[3]
    assert q_noise.shape == (B, N, dqk) and k_cache.shape == (B, Lmax, Hkv, dqk)
    assert lam.shape == (B, S) and gate.shape == (B, S, dv)
    lp = None
    if lens is not None:
        lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32).reshape(-1))
        assert lens.size == B
        lp = _ptr(lens)
    out = np.empty((B, S, dv), dtype=np.float64)
    rc = _load().gda_ref_decode_ex(_ptr(q_sig), _ptr(q_noise), _ptr(k_cache), _ptr(v_cache),
                                   lp, _ptr(lam), _ptr(gate), _ptr(out), B, Lmax, S, N, Hkv,
                                   dqk, dv, int(window), code, float(scale or 0.0),
                                   _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_decode rejected its arguments (code {rc})")
    return out


def ref_decode_latent(q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate, lens=None, *,
                      window: int, scale: float | None = None, lambda_logits: bool = False,
                      gate_logits: bool = False) -> np.ndarray:
    """Latent-cache decode oracle. Shapes: q_sig [B,S,Dn+Dr], q_noise [B,N,Dn+Dr],
    c_kv [B,Lmax,Dc], k_rope [B,Lmax,Dr], w_kv_b [Hkv,Dn+dv,Dc], lam [B,S], gate [B,S,dv],
    lens int32 [B] or None. Dr is k_rope's last dim; dv = w_kv_b rows - Dn. Returns
    [B,S,dv] float64."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate = (
        _c(x, code) for x in (q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate))
    B, S, dqk = q_sig.shape
    N = q_noise.shape[1]
    Lmax, Dc = c_kv.shape[1], c_kv.shape[2]
    Dr = k_rope.shape[2]
    Hkv, rows = w_kv_b.shape[0], w_kv_b.shape[1]
    Dn = dqk - Dr
    dv = rows - Dn
    assert q_noise.shape == (B, N, dqk) and c_kv.shape == (B, Lmax, Dc)
    assert k_rope.shape == (B, Lmax, Dr) and w_kv_b.shape == (Hkv, Dn + dv, Dc)
    assert lam.shape == (B, S) and gate.shape == (B, S, dv)
    lp = None
    if lens is not None:
        lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32).reshape(-1))
        assert lens.size == B
        lp = _ptr(lens)
    out = np.empty((B, S, dv), dtype=np.float64)
    rc = _load().gda_ref_decode_latent(
        _ptr(q_sig), _ptr(q_noise), _ptr(c_kv), _ptr(k_rope), _ptr(w_kv_b), lp, _ptr(lam),
        _ptr(gate), _ptr(out), B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, int(window), code,
        float(scale or 0.0), _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_decode_latent rejected its arguments (code {rc})")
    return out


def ref_fwd_varlen(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k, *, window: int,
                   scale: float | None = None, lambda_logits: bool = False,
                   gate_logits: bool = False) -> np.ndarray:
    """Packed-sequence prefill oracle. q_sig [Tq,S,dqk], q_noise [Tq,N,dqk], k [Tk,Hkv,dqk],
    v [Tk,Hkv,dv], lam [Tq,S], gate [Tq,S,dv]; cu_q, cu_k int32 [nseq+1] (host). Local
    query t of sequence i sits at key position (Lk_i - Lq_i) + t. Returns [Tq,S,dv]."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, k, v, lam, gate = (_c(x, code) for x in (q_sig, q_noise, k, v, lam, gate))
    Tq, S, dqk = q_sig.shape
    N, Hkv, dv = q_noise.shape[1], k.shape[1], v.shape[2]
    cu_q = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
    cu_k = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
    nseq = cu_q.size - 1
    assert cu_k.size == nseq + 1 and cu_q[-1] == Tq and cu_k[-1] == k.shape[0]
    out = np.empty((Tq, S, dv), dtype=np.float64)
    rc = _load().gda_ref_fwd_varlen(_ptr(q_sig), _ptr(q_noise), _ptr(k), _ptr(v), _ptr(lam),
                                    _ptr(gate), _ptr(out), _ptr(cu_q), _ptr(cu_k), nseq, S, N,
                                    Hkv, dqk, dv, int(window), code, float(scale or 0.0),
                                    _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_fwd_varlen rejected its arguments (code {rc})")
    return out


def _shape4(q_sig, q_noise, k, v, lam, gate):
    B, L, S, dqk = q_sig.shape
    N, Hkv, dv = q_noise.shape[2], v.shape[2], v.shape[3]
    assert q_noise.shape == (B, L, N, dqk) and k.shape == (B, L, Hkv, dqk)
    assert v.shape == (B, L, Hkv, dv) and lam.shape == (B, L, S) and gate.shape == (B, L, S, dv)
    return B, L, S, N, Hkv, dqk, dv


def ref_fwd_train(q_sig, q_noise, k, v, lam, gate, *, window: int, scale: float | None = None,
                  lambda_logits: bool = False, gate_logits: bool = False):
    """Training form of the prefill oracle. Returns (out [B,L,S,dv], h_sig [B,L,S,dv],
    h_noise [B,L,N,dv], lse [B,S+N,L]): the output, each path's normalised attention output
    and each attention row's log-sum-exp of its scaled scores (natural log; signal heads
    first, then noise heads), all float64."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, k, v, lam, gate = (_c(x, code) for x in (q_sig, q_noise, k, v, lam, gate))
    B, L, S, N, Hkv, dqk, dv = _shape4(q_sig, q_noise, k, v, lam, gate)
    out = np.empty((B, L, S, dv), dtype=np.float64)
    h_sig = np.empty((B, L, S, dv), dtype=np.float64)
    h_noise = np.empty((B, L, N, dv), dtype=np.float64)
    lse = np.empty((B, S + N, L), dtype=np.float64)
    rc = _load().gda_ref_fwd_train(_ptr(q_sig), _ptr(q_noise), _ptr(k), _ptr(v), _ptr(lam),
                                   _ptr(gate), _ptr(out), _ptr(h_sig), _ptr(h_noise), _ptr(lse),
                                   B, L, S, N, Hkv, dqk, dv, int(window), code,
                                   float(scale or 0.0), _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_fwd_train rejected its arguments (code {rc})")
    return out, h_sig, h_noise, lse


def ref_bwd(q_sig, q_noise, k, v, lam, gate, d_out, *, window: int, scale: float | None = None,
            lambda_logits: bool = False, gate_logits: bool = False, q_rows=None,
            k_rows=None) -> dict:
    """Backward oracle: gradients of sum(d_out * out). d_out [B,L,S,dv] at the inputs'
    storage type. Returns float64 dq_sig, dq_noise, dk, dv, dlam, dgate with the inputs'
    shapes, or, with ``q_rows`` / ``k_rows`` (flat b*L+t rows), only those rows:
    dq_sig [nq,S,dqk], dq_noise [nq,N,dqk], dlam [nq,S], dgate [nq,S,dv], dk [nk,Hkv,dqk],
    dv [nk,Hkv,dv]."""
    code = _dtype_code(q_sig)
    q_sig, q_noise, k, v, lam, gate, d_out = (
        _c(x, code) for x in (q_sig, q_noise, k, v, lam, gate, d_out))
    B, L, S, N, Hkv, dqk, dv = _shape4(q_sig, q_noise, k, v, lam, gate)
    assert d_out.shape == (B, L, S, dv)

    def rows_of(r):
        if r is None:
            return None, B * L, None
        a = np.ascontiguousarray(np.asarray(r, dtype=np.int64).reshape(-1))
        return a, a.size, _ptr(a)

    qa, nq, qp = rows_of(q_rows)
    ka, nk, kp = rows_of(k_rows)
    dq_sig = np.empty((nq, S, dqk)); dq_noise = np.empty((nq, N, dqk))
    dlam = np.empty((nq, S)); dgate = np.empty((nq, S, dv))
    dk = np.empty((nk, Hkv, dqk)); dvv = np.empty((nk, Hkv, dv))
    rc = _load().gda_ref_bwd(_ptr(q_sig), _ptr(q_noise), _ptr(k), _ptr(v), _ptr(lam), _ptr(gate),
                             _ptr(d_out), _ptr(dq_sig), _ptr(dq_noise), _ptr(dk), _ptr(dvv),
                             _ptr(dlam), _ptr(dgate), B, L, S, N, Hkv, dqk, dv, int(window), code,
                             float(scale or 0.0), _flags(lambda_logits, gate_logits), qp,
                             nq if qa is not None else 0, kp, nk if ka is not None else 0)
    if rc != 0:
        raise ValueError(f"gda_ref_bwd rejected its arguments (code {rc})")
    out = dict(dq_sig=dq_sig, dq_noise=dq_noise, dk=dk, dv=dvv, dlam=dlam, dgate=dgate)
    if q_rows is None:
        out["dq_sig"] = dq_sig.reshape(B, L, S, dqk)
        out["dq_noise"] = dq_noise.reshape(B, L, N, dqk)
        out["dlam"] = dlam.reshape(B, L, S)
        out["dgate"] = dgate.reshape(B, L, S, dv)
    if k_rows is None:
        out["dk"] = dk.reshape(B, L, Hkv, dqk)
        out["dv"] = dvv.reshape(B, L, Hkv, dv)
    return out


def _varlen_args(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k):
    code = _dtype_code(q_sig)
    q_sig, q_noise, k, v, lam, gate = (_c(x, code) for x in (q_sig, q_noise, k, v, lam, gate))
    Tq, S, dqk = q_sig.shape
    N, Tk, Hkv, dv = q_noise.shape[1], k.shape[0], k.shape[1], v.shape[2]
    cu_q = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
    cu_k = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
    assert cu_k.size == cu_q.size and cu_q[-1] == Tq and cu_k[-1] == Tk
    return code, (q_sig, q_noise, k, v, lam, gate), cu_q, cu_k, Tq, Tk, S, N, Hkv, dqk, dv


def ref_fwd_train_varlen(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k, *, window: int,
                         scale: float | None = None, lambda_logits: bool = False,
                         gate_logits: bool = False):
    """Packed-sequence training forward: (out [Tq,S,dv], h_sig [Tq,S,dv], h_noise [Tq,N,dv],
    lse [S+N,Tq]) in float64 (shapes and positions as ref_fwd_varlen)."""
    code, x, cu_q, cu_k, Tq, Tk, S, N, Hkv, dqk, dv = _varlen_args(q_sig, q_noise, k, v, lam,
                                                                   gate, cu_q, cu_k)
    out = np.empty((Tq, S, dv)); h_sig = np.empty((Tq, S, dv)); h_noise = np.empty((Tq, N, dv))
    lse = np.empty((S + N, Tq))
    rc = _load().gda_ref_fwd_train_varlen(*(_ptr(a) for a in x), _ptr(out), _ptr(h_sig),
                                          _ptr(h_noise), _ptr(lse), _ptr(cu_q), _ptr(cu_k),
                                          cu_q.size - 1, S, N, Hkv, dqk, dv, int(window), code,
                                          float(scale or 0.0), _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_fwd_train_varlen rejected its arguments (code {rc})")
    return out, h_sig, h_noise, lse


def ref_bwd_varlen(q_sig, q_noise, k, v, lam, gate, d_out, cu_q, cu_k, *, window: int,
                   scale: float | None = None, lambda_logits: bool = False,
                   gate_logits: bool = False) -> dict:
    """Packed-sequence backward oracle: gradients of sum(d_out * out), float64, shaped like
    the packed inputs (dq_sig [Tq,S,dqk], dq_noise, dk [Tk,Hkv,dqk], dv, dlam, dgate)."""
    code, x, cu_q, cu_k, Tq, Tk, S, N, Hkv, dqk, dv = _varlen_args(q_sig, q_noise, k, v, lam,
                                                                   gate, cu_q, cu_k)
    d_out = _c(d_out, code)
    assert d_out.shape == (Tq, S, dv)
    g = dict(dq_sig=np.empty((Tq, S, dqk)), dq_noise=np.empty((Tq, N, dqk)),
             dk=np.empty((Tk, Hkv, dqk)), dv=np.empty((Tk, Hkv, dv)), dlam=np.empty((Tq, S)),
             dgate=np.empty((Tq, S, dv)))
    rc = _load().gda_ref_bwd_varlen(*(_ptr(a) for a in x), _ptr(d_out), _ptr(g["dq_sig"]),
                                    _ptr(g["dq_noise"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                    _ptr(g["dlam"]), _ptr(g["dgate"]), _ptr(cu_q), _ptr(cu_k),
                                    cu_q.size - 1, S, N, Hkv, dqk, dv, int(window), code,
                                    float(scale or 0.0), _flags(lambda_logits, gate_logits))
    if rc != 0:
        raise ValueError(f"gda_ref_bwd_varlen rejected its arguments (code {rc})")
    return g
