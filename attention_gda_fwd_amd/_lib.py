"""ctypes loader of libgda.so (the C ABI declared in include/gda.h).

Argument marshalling only. Loading fails loudly if the library has not been
built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# GDA_LIB names another build of the library to load (a host-sanitizer build).
LIB_PATH = os.environ.get("GDA_LIB") or os.path.join(PKG, "libgda.so")

GDA_SUCCESS, GDA_ERROR_INVALID_ARGUMENT, GDA_ERROR_UNSUPPORTED, GDA_ERROR_HIP = range(4)
GDA_BF16, GDA_F32 = 0, 1
GDA_LAMBDA_LOGITS, GDA_GATE_LOGITS = 1, 2

EXPORTED = ("gda_fwd", "gda_decode", "gda_fwd_ex", "gda_decode_ex", "gda_fwd_varlen",
            "gda_fwd_train", "gda_bwd", "gda_bwd_workspace_bytes", "gda_fwd_train_varlen",
            "gda_bwd_varlen", "gda_decode_latent", "gda_decode_latent_noalloc",
            "gda_decode_latent_workspace_bytes", "gda_status_string", "gda_last_error")
# Size of the static scratch of gda_decode_latent_noalloc (GDA_DECODE_LATENT_SCRATCH_BYTES).
DECODE_LATENT_SCRATCH_BYTES = 64 << 20


class Options(ctypes.Structure):
    """gda_options: softmax_scale (0 = 1/sqrt(dqk)) and flags."""
    _fields_ = [("softmax_scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


_lib = None


class GdaError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status
        self.name = name
        self.detail = detail


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libgda.so is not built ({LIB_PATH} missing); run "
            "`python -m attention_gda_fwd_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.gda_fwd.restype = i32
    lib.gda_fwd.argtypes = [vp] * 7 + [i32] * 8 + [i32, vp]
    lib.gda_decode.restype = i32
    lib.gda_decode.argtypes = [vp] * 8 + [i32] * 8 + [i32, vp]
    lib.gda_fwd_ex.restype = i32
    lib.gda_fwd_ex.argtypes = [vp] * 7 + [i32] * 8 + [i32, ctypes.POINTER(Options), vp]
    lib.gda_decode_ex.restype = i32
    lib.gda_decode_ex.argtypes = [vp] * 8 + [i32] * 8 + [i32, ctypes.POINTER(Options), vp]
    lib.gda_fwd_varlen.restype = i32
    lib.gda_fwd_varlen.argtypes = [vp] * 9 + [i32] * 8 + [i32, ctypes.POINTER(Options), vp]
    lib.gda_fwd_train.restype = i32
    lib.gda_fwd_train.argtypes = [vp] * 10 + [i32] * 8 + [i32, ctypes.POINTER(Options), vp]
    lib.gda_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gda_bwd_workspace_bytes.argtypes = [i32] * 5
    lib.gda_bwd.restype = i32
    lib.gda_bwd.argtypes = ([vp] * 16 + [i32] * 8 + [i32, ctypes.POINTER(Options), vp,
                                                     ctypes.c_size_t, vp])
    lib.gda_fwd_train_varlen.restype = i32
    lib.gda_fwd_train_varlen.argtypes = [vp] * 12 + [i32] * 9 + [i32, ctypes.POINTER(Options),
                                                                 vp]
    lib.gda_bwd_varlen.restype = i32
    lib.gda_bwd_varlen.argtypes = ([vp] * 18 + [i32] * 10 + [i32, ctypes.POINTER(Options), vp,
                                                             ctypes.c_size_t, vp])
    lib.gda_decode_latent_workspace_bytes.restype = ctypes.c_size_t
    lib.gda_decode_latent_workspace_bytes.argtypes = [i32] * 5
    lib.gda_decode_latent.restype = i32
    lib.gda_decode_latent.argtypes = ([vp] * 9 + [i32] * 10 + [i32, ctypes.POINTER(Options), vp,
                                                               ctypes.c_size_t, vp])
    lib.gda_decode_latent_noalloc.restype = i32
    lib.gda_decode_latent_noalloc.argtypes = ([vp] * 9 + [i32] * 10 +
                                              [i32, ctypes.POINTER(Options), vp])
    lib.gda_status_string.restype = ctypes.c_char_p
    lib.gda_status_string.argtypes = [i32]
    lib.gda_last_error.restype = ctypes.c_char_p
    lib.gda_last_error.argtypes = []
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != GDA_SUCCESS:
        lib = load()
        name = lib.gda_status_string(status).decode()
        detail = lib.gda_last_error().decode()
        raise GdaError(status, name, detail)


def fwd_raw(q_sig, q_noise, k, v, lam, gate, out, B, L, S, N, Hkv, dqk, dv, window, dtype,
            stream) -> int:
    """Direct call of gda_fwd with integer pointers; returns the status code."""
    return load().gda_fwd(q_sig, q_noise, k, v, lam, gate, out, B, L, S, N, Hkv, dqk, dv,
                          window, dtype, stream)


def decode_raw(q_sig, q_noise, k_cache, v_cache, lens, lam, gate, out, B, Lmax, S, N, Hkv,
               dqk, dv, window, dtype, stream) -> int:
    """Direct call of gda_decode with integer pointers; returns the status code."""
    return load().gda_decode(q_sig, q_noise, k_cache, v_cache, lens, lam, gate, out, B, Lmax,
                             S, N, Hkv, dqk, dv, window, dtype, stream)


def options(scale=None, lambda_logits=False, gate_logits=False):
    """An Options value, or None when every option is the default."""
    if scale is None and not lambda_logits and not gate_logits:
        return None
    flags = (GDA_LAMBDA_LOGITS if lambda_logits else 0) | (GDA_GATE_LOGITS if gate_logits else 0)
    return Options(float(scale or 0.0), flags)


def fwd_ex_raw(q_sig, q_noise, k, v, lam, gate, out, B, L, S, N, Hkv, dqk, dv, window, dtype,
               opts, stream) -> int:
    """Direct call of gda_fwd_ex (opts an Options or None)."""
    return load().gda_fwd_ex(q_sig, q_noise, k, v, lam, gate, out, B, L, S, N, Hkv, dqk, dv,
                             window, dtype, ctypes.byref(opts) if opts is not None else None,
                             stream)


def decode_ex_raw(q_sig, q_noise, k_cache, v_cache, lens, lam, gate, out, B, Lmax, S, N, Hkv,
                  dqk, dv, window, dtype, opts, stream) -> int:
    """Direct call of gda_decode_ex (opts an Options or None)."""
    return load().gda_decode_ex(q_sig, q_noise, k_cache, v_cache, lens, lam, gate, out, B, Lmax,
                                S, N, Hkv, dqk, dv, window, dtype,
                                ctypes.byref(opts) if opts is not None else None, stream)


def latent_workspace_bytes(B, Lmax, S, N, window) -> int:
    return int(load().gda_decode_latent_workspace_bytes(B, Lmax, S, N, window))


def decode_latent_raw(q_sig, q_noise, c_kv, k_rope, w_kv_b, lens, lam, gate, out, B, Lmax, S, N,
                      Hkv, Dn, Dr, Dc, dv, window, dtype, opts, workspace, workspace_bytes,
                      stream) -> int:
    """Direct call of gda_decode_latent (opts an Options or None)."""
    return load().gda_decode_latent(q_sig, q_noise, c_kv, k_rope, w_kv_b, lens, lam, gate, out,
                                    B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, window, dtype,
                                    ctypes.byref(opts) if opts is not None else None, workspace,
                                    workspace_bytes, stream)


def decode_latent_noalloc_raw(q_sig, q_noise, c_kv, k_rope, w_kv_b, lens, lam, gate, out, B,
                              Lmax, S, N, Hkv, Dn, Dr, Dc, dv, window, dtype, opts,
                              stream) -> int:
    """Direct call of gda_decode_latent_noalloc (opts an Options or None)."""
    return load().gda_decode_latent_noalloc(q_sig, q_noise, c_kv, k_rope, w_kv_b, lens, lam, gate,
                                            out, B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, window,
                                            dtype,
                                            ctypes.byref(opts) if opts is not None else None,
                                            stream)


def fwd_varlen_raw(q_sig, q_noise, k, v, lam, gate, out, cu_q, cu_k, nseq, max_seqlen_q, S, N,
                   Hkv, dqk, dv, window, dtype, opts, stream) -> int:
    """Direct call of gda_fwd_varlen (opts an Options or None)."""
    return load().gda_fwd_varlen(q_sig, q_noise, k, v, lam, gate, out, cu_q, cu_k, nseq,
                                 max_seqlen_q, S, N, Hkv, dqk, dv, window, dtype,
                                 ctypes.byref(opts) if opts is not None else None, stream)


def fwd_train_raw(q_sig, q_noise, k, v, lam, gate, out, h_sig, h_noise, lse, B, L, S, N, Hkv,
                  dqk, dv, window, dtype, opts, stream) -> int:
    """Direct call of gda_fwd_train (opts an Options or None)."""
    return load().gda_fwd_train(q_sig, q_noise, k, v, lam, gate, out, h_sig, h_noise, lse, B, L,
                                S, N, Hkv, dqk, dv, window, dtype,
                                ctypes.byref(opts) if opts is not None else None, stream)


def bwd_workspace_bytes(B, L, S, N, dv) -> int:
    return int(load().gda_bwd_workspace_bytes(B, L, S, N, dv))


def bwd_raw(q_sig, q_noise, k, v, lam, gate, h_sig, h_noise, lse, d_out, dq_sig, dq_noise, dk,
            dv_out, dlam, dgate, B, L, S, N, Hkv, dqk, dv, window, dtype, opts, workspace,
            workspace_bytes, stream) -> int:
    """Direct call of gda_bwd (opts an Options or None)."""
    return load().gda_bwd(q_sig, q_noise, k, v, lam, gate, h_sig, h_noise, lse, d_out, dq_sig,
                          dq_noise, dk, dv_out, dlam, dgate, B, L, S, N, Hkv, dqk, dv, window,
                          dtype, ctypes.byref(opts) if opts is not None else None, workspace,
                          workspace_bytes, stream)


def fwd_train_varlen_raw(q_sig, q_noise, k, v, lam, gate, out, h_sig, h_noise, lse, cu_q, cu_k,
                         nseq, max_seqlen_q, total_q, S, N, Hkv, dqk, dv, window, dtype, opts,
                         stream) -> int:
    """Direct call of gda_fwd_train_varlen (opts an Options or None)."""
    return load().gda_fwd_train_varlen(q_sig, q_noise, k, v, lam, gate, out, h_sig, h_noise, lse,
                                       cu_q, cu_k, nseq, max_seqlen_q, total_q, S, N, Hkv, dqk,
                                       dv, window, dtype,
                                       ctypes.byref(opts) if opts is not None else None, stream)


def bwd_varlen_raw(q_sig, q_noise, k, v, lam, gate, h_sig, h_noise, lse, d_out, dq_sig, dq_noise,
                   dk, dv_out, dlam, dgate, cu_q, cu_k, nseq, max_seqlen_q, max_seqlen_k, total_q,
                   S, N, Hkv, dqk, dv, window, dtype, opts, workspace, workspace_bytes,
                   stream) -> int:
    """Direct call of gda_bwd_varlen (opts an Options or None)."""
    return load().gda_bwd_varlen(q_sig, q_noise, k, v, lam, gate, h_sig, h_noise, lse, d_out,
                                 dq_sig, dq_noise, dk, dv_out, dlam, dgate, cu_q, cu_k, nseq,
                                 max_seqlen_q, max_seqlen_k, total_q, S, N, Hkv, dqk, dv, window,
                                 dtype, ctypes.byref(opts) if opts is not None else None,
                                 workspace, workspace_bytes, stream)
