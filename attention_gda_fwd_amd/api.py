"""PyTorch front end of libgda: tensors in, tensors out, same names as the C ABI.

PyTorch only provides device memory and the stream. Every step of the
computation runs in the HIP kernels behind the C entry points.
"""
from __future__ import annotations

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.GDA_BF16, torch.float32: _lib.GDA_F32}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"gda: dtype must be bfloat16 or float32, got {t.dtype}") from None


def _check(name: str, t: torch.Tensor, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"gda: {name} must be a tensor")
    if t.device != device:
        raise ValueError(f"gda: {name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"gda: {name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"gda: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"gda: {name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def gda_fwd(q_sig: torch.Tensor, q_noise: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            lam: torch.Tensor, gate: torch.Tensor, window: int = 0,
            out: torch.Tensor | None = None, scale: float | None = None,
            lambda_logits: bool = False, gate_logits: bool = False) -> torch.Tensor:
    """Prefill. q_sig [B,L,S,dqk], q_noise [B,L,N,dqk], k [B,L,Hkv,dqk], v [B,L,Hkv,dv],
    lam [B,L,S], gate [B,L,S,dv] -> out [B,L,S,dv] = gate*(H_S - lam*Repeat_g(H_N)).
    ``scale`` replaces 1/sqrt(dqk); ``lambda_logits`` / ``gate_logits`` mark those inputs
    as logits (the kernels apply the sigmoid)."""
    if q_sig.dim() != 4 or q_noise.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("gda_fwd: q_sig, q_noise, k, v must be 4-D")
    B, L, S, dqk = q_sig.shape
    N, Hkv, dv = q_noise.shape[2], k.shape[2], v.shape[3]
    dev, dt = q_sig.device, q_sig.dtype
    code = _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError("gda_fwd: tensors must be on a HIP (cuda) device")
    _check("q_sig", q_sig, (B, L, S, dqk), dt, dev)
    _check("q_noise", q_noise, (B, L, N, dqk), dt, dev)
    _check("k", k, (B, L, Hkv, dqk), dt, dev)
    _check("v", v, (B, L, Hkv, dv), dt, dev)
    _check("lam", lam, (B, L, S), dt, dev)
    _check("gate", gate, (B, L, S, dv), dt, dev)
    if out is None:
        out = torch.empty((B, L, S, dv), dtype=dt, device=dev)
    _check("out", out, (B, L, S, dv), dt, dev)
    _lib.check(_lib.fwd_ex_raw(q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(),
                               v.data_ptr(), lam.data_ptr(), gate.data_ptr(), out.data_ptr(), B,
                               L, S, N, Hkv, dqk, dv, int(window), code,
                               _lib.options(scale, lambda_logits, gate_logits), _stream(dev)))
    return out


def gda_decode(q_sig: torch.Tensor, q_noise: torch.Tensor, k_cache: torch.Tensor,
               v_cache: torch.Tensor, lam: torch.Tensor, gate: torch.Tensor,
               cache_lens: torch.Tensor | None = None, window: int = 0,
               out: torch.Tensor | None = None, scale: float | None = None,
               lambda_logits: bool = False, gate_logits: bool = False) -> torch.Tensor:
    """Decode. q_sig [B,S,dqk], q_noise [B,N,dqk], k_cache [B,Lmax,Hkv,dqk],
    v_cache [B,Lmax,Hkv,dv], lam [B,S], gate [B,S,dv], cache_lens int32 [B] on the
    device (or None = Lmax) -> out [B,S,dv]. Options as for gda_fwd."""
    if q_sig.dim() != 3 or q_noise.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("gda_decode: q_sig/q_noise must be 3-D and the caches 4-D")
    B, S, dqk = q_sig.shape
    N, Lmax, Hkv, dv = q_noise.shape[1], k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    dev, dt = q_sig.device, q_sig.dtype
    code = _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError("gda_decode: tensors must be on a HIP (cuda) device")
    _check("q_sig", q_sig, (B, S, dqk), dt, dev)
    _check("q_noise", q_noise, (B, N, dqk), dt, dev)
    _check("k_cache", k_cache, (B, Lmax, Hkv, dqk), dt, dev)
    _check("v_cache", v_cache, (B, Lmax, Hkv, dv), dt, dev)
    _check("lam", lam, (B, S), dt, dev)
    _check("gate", gate, (B, S, dv), dt, dev)
    lens_ptr = None
    if cache_lens is not None:
        _check("cache_lens", cache_lens, (B,), torch.int32, dev)
        lens_ptr = cache_lens.data_ptr()
    if out is None:
        out = torch.empty((B, S, dv), dtype=dt, device=dev)
    _check("out", out, (B, S, dv), dt, dev)
    _lib.check(_lib.decode_ex_raw(q_sig.data_ptr(), q_noise.data_ptr(), k_cache.data_ptr(),
                                  v_cache.data_ptr(), lens_ptr, lam.data_ptr(), gate.data_ptr(),
                                  out.data_ptr(), B, Lmax, S, N, Hkv, dqk, dv, int(window),
                                  code, _lib.options(scale, lambda_logits, gate_logits),
                                  _stream(dev)))
    return out


def gda_fwd_varlen(q_sig: torch.Tensor, q_noise: torch.Tensor, k: torch.Tensor,
                   v: torch.Tensor, lam: torch.Tensor, gate: torch.Tensor,
                   cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                   window: int = 0, out: torch.Tensor | None = None, scale: float | None = None,
                   lambda_logits: bool = False, gate_logits: bool = False) -> torch.Tensor:
    """Packed-sequence prefill. q_sig [Tq,S,dqk], q_noise [Tq,N,dqk], k [Tk,Hkv,dqk],
    v [Tk,Hkv,dv], lam [Tq,S], gate [Tq,S,dv]; cu_seqlens_q / cu_seqlens_k int32 [nseq+1] on
    the device. Local query t of sequence i sits at key position Lk_i - Lq_i + t.
    -> out [Tq,S,dv]."""
    if q_sig.dim() != 3 or q_noise.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("gda_fwd_varlen: q_sig, q_noise, k, v must be 3-D (packed rows)")
    Tq, S, dqk = q_sig.shape
    N, Tk, Hkv, dv = q_noise.shape[1], k.shape[0], k.shape[1], v.shape[2]
    dev, dt = q_sig.device, q_sig.dtype
    code = _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError("gda_fwd_varlen: tensors must be on a HIP (cuda) device")
    nseq = cu_seqlens_q.numel() - 1
    _check("q_sig", q_sig, (Tq, S, dqk), dt, dev)
    _check("q_noise", q_noise, (Tq, N, dqk), dt, dev)
    _check("k", k, (Tk, Hkv, dqk), dt, dev)
    _check("v", v, (Tk, Hkv, dv), dt, dev)
    _check("lam", lam, (Tq, S), dt, dev)
    _check("gate", gate, (Tq, S, dv), dt, dev)
    _check("cu_seqlens_q", cu_seqlens_q, (nseq + 1,), torch.int32, dev)
    _check("cu_seqlens_k", cu_seqlens_k, (nseq + 1,), torch.int32, dev)
    if out is None:
        out = torch.empty((Tq, S, dv), dtype=dt, device=dev)
    _check("out", out, (Tq, S, dv), dt, dev)
    _lib.check(_lib.fwd_varlen_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), out.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), nseq,
        int(max_seqlen_q), S, N, Hkv, dqk, dv, int(window), code,
        _lib.options(scale, lambda_logits, gate_logits), _stream(dev)))
    return out


def _latent_shapes(name, q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate, cache_lens, out):
    if q_sig.dim() != 3 or c_kv.dim() != 3 or k_rope.dim() != 3 or w_kv_b.dim() != 3:
        raise ValueError(f"{name}: q/c_kv/k_rope/w_kv_b must be 3-D")
    B, S, dqk = q_sig.shape
    N = q_noise.shape[1]
    Lmax, Dc = c_kv.shape[1], c_kv.shape[2]
    Dr = k_rope.shape[2]
    Hkv, rows = w_kv_b.shape[0], w_kv_b.shape[1]
    Dn = dqk - Dr
    dv = rows - Dn
    dev, dt = q_sig.device, q_sig.dtype
    _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a HIP (cuda) device")
    _check("q_sig", q_sig, (B, S, dqk), dt, dev)
    _check("q_noise", q_noise, (B, N, dqk), dt, dev)
    _check("c_kv", c_kv, (B, Lmax, Dc), dt, dev)
    _check("k_rope", k_rope, (B, Lmax, Dr), dt, dev)
    _check("w_kv_b", w_kv_b, (Hkv, Dn + dv, Dc), dt, dev)
    _check("lam", lam, (B, S), dt, dev)
    _check("gate", gate, (B, S, dv), dt, dev)
    lens_ptr = None
    if cache_lens is not None:
        _check("cache_lens", cache_lens, (B,), torch.int32, dev)
        lens_ptr = cache_lens.data_ptr()
    if out is None:
        out = torch.empty((B, S, dv), dtype=dt, device=dev)
    _check("out", out, (B, S, dv), dt, dev)
    return B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, dev, lens_ptr, out


def gda_decode_latent(q_sig: torch.Tensor, q_noise: torch.Tensor, c_kv: torch.Tensor,
                      k_rope: torch.Tensor, w_kv_b: torch.Tensor, lam: torch.Tensor,
                      gate: torch.Tensor, cache_lens: torch.Tensor | None = None,
                      window: int = 0, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, scale: float | None = None,
                      lambda_logits: bool = False, gate_logits: bool = False) -> torch.Tensor:
    """Decode over the latent cache. q_sig [B,S,Dn+Dr], q_noise [B,N,Dn+Dr], c_kv [B,Lmax,Dc],
    k_rope [B,Lmax,Dr], w_kv_b [Hkv,Dn+dv,Dc], lam [B,S], gate [B,S,dv], cache_lens int32 [B]
    or None -> out [B,S,dv]. ``workspace``: a uint8 device tensor of at least
    ``latent_workspace_bytes(...)`` bytes (allocated here when None)."""
    B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, dev, lens_ptr, out = _latent_shapes(
        "gda_decode_latent", q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate, cache_lens, out)
    need = _lib.latent_workspace_bytes(B, Lmax, S, N, int(window))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("gda_decode_latent: workspace must be a contiguous uint8 device tensor")
    _lib.check(_lib.decode_latent_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), c_kv.data_ptr(), k_rope.data_ptr(),
        w_kv_b.data_ptr(), lens_ptr, lam.data_ptr(), gate.data_ptr(), out.data_ptr(), B, Lmax, S,
        N, Hkv, Dn, Dr, Dc, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), workspace.data_ptr(), workspace.numel(),
        _stream(dev)))
    return out


def gda_decode_latent_noalloc(q_sig: torch.Tensor, q_noise: torch.Tensor, c_kv: torch.Tensor,
                              k_rope: torch.Tensor, w_kv_b: torch.Tensor, lam: torch.Tensor,
                              gate: torch.Tensor, out: torch.Tensor,
                              cache_lens: torch.Tensor | None = None, window: int = 0,
                              scale: float | None = None, lambda_logits: bool = False,
                              gate_logits: bool = False) -> torch.Tensor:
    """gda_decode_latent without a workspace: the library's static per-GPU scratch
    (DECODE_LATENT_SCRATCH_BYTES) serves instead, and nothing is allocated, so ``out``
    must be given. Calls that may overlap on one GPU must be serialised by the caller."""
    if out is None:
        raise ValueError("gda_decode_latent_noalloc: out must be preallocated")
    B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, dev, lens_ptr, out = _latent_shapes(
        "gda_decode_latent_noalloc", q_sig, q_noise, c_kv, k_rope, w_kv_b, lam, gate, cache_lens,
        out)
    _lib.check(_lib.decode_latent_noalloc_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), c_kv.data_ptr(), k_rope.data_ptr(),
        w_kv_b.data_ptr(), lens_ptr, lam.data_ptr(), gate.data_ptr(), out.data_ptr(), B, Lmax, S,
        N, Hkv, Dn, Dr, Dc, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), _stream(dev)))
    return out


def latent_workspace_bytes(B: int, Lmax: int, S: int, N: int, window: int = 0) -> int:
    """Bytes of workspace gda_decode_latent needs for these sizes."""
    return _lib.latent_workspace_bytes(B, Lmax, S, N, int(window))


def _prefill_shapes(name, q_sig, q_noise, k, v, lam, gate):
    if q_sig.dim() != 4 or q_noise.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError(f"{name}: q_sig, q_noise, k, v must be 4-D")
    B, L, S, dqk = q_sig.shape
    N, Hkv, dv = q_noise.shape[2], k.shape[2], v.shape[3]
    dev, dt = q_sig.device, q_sig.dtype
    _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a HIP (cuda) device")
    _check("q_sig", q_sig, (B, L, S, dqk), dt, dev)
    _check("q_noise", q_noise, (B, L, N, dqk), dt, dev)
    _check("k", k, (B, L, Hkv, dqk), dt, dev)
    _check("v", v, (B, L, Hkv, dv), dt, dev)
    _check("lam", lam, (B, L, S), dt, dev)
    _check("gate", gate, (B, L, S, dv), dt, dev)
    return B, L, S, N, Hkv, dqk, dv, dev, dt


def gda_fwd_train(q_sig: torch.Tensor, q_noise: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  lam: torch.Tensor, gate: torch.Tensor, window: int = 0,
                  scale: float | None = None, lambda_logits: bool = False,
                  gate_logits: bool = False):
    """Training-form prefill (bf16): returns (out [B,L,S,dv], h_sig [B,L,S,dv],
    h_noise [B,L,N,dv], lse float32 [B,S+N,L]) - the output, each path's normalised
    attention output and each attention row's log-sum-exp (natural log)."""
    B, L, S, N, Hkv, dqk, dv, dev, dt = _prefill_shapes("gda_fwd_train", q_sig, q_noise, k, v,
                                                        lam, gate)
    out = torch.empty((B, L, S, dv), dtype=dt, device=dev)
    h_sig = torch.empty((B, L, S, dv), dtype=dt, device=dev)
    h_noise = torch.empty((B, L, N, dv), dtype=dt, device=dev)
    lse = torch.empty((B, S + N, L), dtype=torch.float32, device=dev)
    _lib.check(_lib.fwd_train_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), out.data_ptr(), h_sig.data_ptr(), h_noise.data_ptr(), lse.data_ptr(),
        B, L, S, N, Hkv, dqk, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), _stream(dev)))
    return out, h_sig, h_noise, lse


def bwd_workspace_bytes(B: int, L: int, S: int, N: int, dv: int) -> int:
    return _lib.bwd_workspace_bytes(B, L, S, N, dv)


def gda_bwd(q_sig: torch.Tensor, q_noise: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            lam: torch.Tensor, gate: torch.Tensor, h_sig: torch.Tensor, h_noise: torch.Tensor,
            lse: torch.Tensor, d_out: torch.Tensor, window: int = 0, scale: float | None = None,
            lambda_logits: bool = False, gate_logits: bool = False,
            workspace: torch.Tensor | None = None, grads: dict | None = None) -> dict:
    """Backward (bf16) of the forward gda_fwd_train ran: gradients of sum(d_out * out).
    Returns dict(dq_sig, dq_noise, dk, dv, dlam, dgate) shaped like the inputs.
    ``workspace``: uint8 device tensor of at least bwd_workspace_bytes(...) bytes
    (allocated here when None); ``grads``: preallocated outputs (same keys)."""
    B, L, S, N, Hkv, dqk, dv, dev, dt = _prefill_shapes("gda_bwd", q_sig, q_noise, k, v, lam,
                                                        gate)
    _check("h_sig", h_sig, (B, L, S, dv), dt, dev)
    _check("h_noise", h_noise, (B, L, N, dv), dt, dev)
    _check("lse", lse, (B, S + N, L), torch.float32, dev)
    _check("d_out", d_out, (B, L, S, dv), dt, dev)
    shapes = dict(dq_sig=(B, L, S, dqk), dq_noise=(B, L, N, dqk), dk=(B, L, Hkv, dqk),
                  dv=(B, L, Hkv, dv), dlam=(B, L, S), dgate=(B, L, S, dv))
    if grads is None:
        grads = {n: torch.empty(sh, dtype=dt, device=dev) for n, sh in shapes.items()}
    for n, sh in shapes.items():
        _check(n, grads[n], sh, dt, dev)
    need = _lib.bwd_workspace_bytes(B, L, S, N, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("workspace", workspace, (workspace.numel(),), torch.uint8, dev)
    _lib.check(_lib.bwd_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), h_sig.data_ptr(), h_noise.data_ptr(), lse.data_ptr(), d_out.data_ptr(),
        grads["dq_sig"].data_ptr(), grads["dq_noise"].data_ptr(), grads["dk"].data_ptr(),
        grads["dv"].data_ptr(), grads["dlam"].data_ptr(), grads["dgate"].data_ptr(), B, L, S, N,
        Hkv, dqk, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), workspace.data_ptr(), workspace.numel(),
        _stream(dev)))
    return grads


def _packed_shapes(name, q_sig, q_noise, k, v, lam, gate, cu_seqlens_q, cu_seqlens_k):
    if q_sig.dim() != 3 or q_noise.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError(f"{name}: q_sig, q_noise, k, v must be 3-D (packed rows)")
    Tq, S, dqk = q_sig.shape
    N, Tk, Hkv, dv = q_noise.shape[1], k.shape[0], k.shape[1], v.shape[2]
    dev, dt = q_sig.device, q_sig.dtype
    _dtype_code(q_sig)
    if dev.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a HIP (cuda) device")
    nseq = cu_seqlens_q.numel() - 1
    _check("q_sig", q_sig, (Tq, S, dqk), dt, dev)
    _check("q_noise", q_noise, (Tq, N, dqk), dt, dev)
    _check("k", k, (Tk, Hkv, dqk), dt, dev)
    _check("v", v, (Tk, Hkv, dv), dt, dev)
    _check("lam", lam, (Tq, S), dt, dev)
    _check("gate", gate, (Tq, S, dv), dt, dev)
    _check("cu_seqlens_q", cu_seqlens_q, (nseq + 1,), torch.int32, dev)
    _check("cu_seqlens_k", cu_seqlens_k, (nseq + 1,), torch.int32, dev)
    return Tq, Tk, S, N, Hkv, dqk, dv, nseq, dev, dt


def gda_fwd_train_varlen(q_sig, q_noise, k, v, lam, gate, cu_seqlens_q, cu_seqlens_k,
                         max_seqlen_q: int, window: int = 0, scale: float | None = None,
                         lambda_logits: bool = False, gate_logits: bool = False):
    """Packed-sequence training forward (bf16): (out [Tq,S,dv], h_sig [Tq,S,dv],
    h_noise [Tq,N,dv], lse float32 [S+N,Tq]); sequences as gda_fwd_varlen."""
    Tq, Tk, S, N, Hkv, dqk, dv, nseq, dev, dt = _packed_shapes(
        "gda_fwd_train_varlen", q_sig, q_noise, k, v, lam, gate, cu_seqlens_q, cu_seqlens_k)
    out = torch.empty((Tq, S, dv), dtype=dt, device=dev)
    h_sig = torch.empty((Tq, S, dv), dtype=dt, device=dev)
    h_noise = torch.empty((Tq, N, dv), dtype=dt, device=dev)
    lse = torch.empty((S + N, Tq), dtype=torch.float32, device=dev)
    _lib.check(_lib.fwd_train_varlen_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), out.data_ptr(), h_sig.data_ptr(), h_noise.data_ptr(), lse.data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), nseq, int(max_seqlen_q), Tq, S, N,
        Hkv, dqk, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), _stream(dev)))
    return out, h_sig, h_noise, lse


def gda_bwd_varlen(q_sig, q_noise, k, v, lam, gate, h_sig, h_noise, lse, d_out, cu_seqlens_q,
                   cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, window: int = 0,
                   scale: float | None = None, lambda_logits: bool = False,
                   gate_logits: bool = False, workspace: torch.Tensor | None = None) -> dict:
    """Packed-sequence backward (bf16) of gda_fwd_train_varlen: dict(dq_sig, dq_noise, dk,
    dv, dlam, dgate) shaped like the packed inputs."""
    Tq, Tk, S, N, Hkv, dqk, dv, nseq, dev, dt = _packed_shapes(
        "gda_bwd_varlen", q_sig, q_noise, k, v, lam, gate, cu_seqlens_q, cu_seqlens_k)
    _check("h_sig", h_sig, (Tq, S, dv), dt, dev)
    _check("h_noise", h_noise, (Tq, N, dv), dt, dev)
    _check("lse", lse, (S + N, Tq), torch.float32, dev)
    _check("d_out", d_out, (Tq, S, dv), dt, dev)
    shapes = dict(dq_sig=(Tq, S, dqk), dq_noise=(Tq, N, dqk), dk=(Tk, Hkv, dqk),
                  dv=(Tk, Hkv, dv), dlam=(Tq, S), dgate=(Tq, S, dv))
    grads = {n: torch.empty(sh, dtype=dt, device=dev) for n, sh in shapes.items()}
    need = _lib.bwd_workspace_bytes(1, Tq, S, N, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("workspace", workspace, (workspace.numel(),), torch.uint8, dev)
    _lib.check(_lib.bwd_varlen_raw(
        q_sig.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), h_sig.data_ptr(), h_noise.data_ptr(), lse.data_ptr(), d_out.data_ptr(),
        grads["dq_sig"].data_ptr(), grads["dq_noise"].data_ptr(), grads["dk"].data_ptr(),
        grads["dv"].data_ptr(), grads["dlam"].data_ptr(), grads["dgate"].data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), nseq, int(max_seqlen_q),
        int(max_seqlen_k), Tq, S, N, Hkv, dqk, dv, int(window), _dtype_code(q_sig),
        _lib.options(scale, lambda_logits, gate_logits), workspace.data_ptr(), workspace.numel(),
        _stream(dev)))
    return grads
