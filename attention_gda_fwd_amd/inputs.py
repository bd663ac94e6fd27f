"""Seeded synthetic inputs for the GDA/GDLA attention forward and its checks.

This module only draws tensors. It holds no step of the attention method, so
both the HIP path and the fp64 oracle can take their inputs from it without
sharing any of the method's arithmetic.

Recipe (the pages print no activations; the shapes follow the Motif-2-12.7B and
Motif 3 head layouts, the values stand in for post-RoPE layer activations):

* every tensor of a case is drawn per batch row ``b`` from its own stream,
  ``numpy.random.PCG64(SeedSequence([0x6DA, case_id, tensor_id, b]))``, so any
  sequence can be regenerated on its own (the decode cache one sequence at a
  time);
* Q, K, V: ``standard_normal(float32)``, then rounded to the storage dtype
  (round-to-nearest-even for bf16);
* lambda and gate: ``sigmoid(z)`` of a standard-normal ``z`` evaluated in
  float64, then rounded to the storage dtype. The kernel receives values in
  (0, 1), not logits;
* with ``rope_dims > 0`` (dqk = 192 = 128 + 64 in the Motif 3 layout), the last
  ``rope_dims`` key columns are one draw per (b, token) shared by every KV head,
  mirroring the decoupled rotary key that the Motif 3 walk-through says is
  broadcast to all heads (step 2 and novelty point one).
* latent-cache decode: the KV latent ``c_kv`` is ``standard_normal`` (unit RMS,
  standing in for the RMSNorm output), the rotary key ``k_rope`` likewise; the
  up-projection ``w_kv_b`` [Hkv, Dn + dv, Dc] is ``standard_normal / sqrt(Dc)``
  (so that expanded keys and values have unit variance), drawn once per case.

bf16 tensors are returned as ``uint16`` arrays holding the bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np

SEED_ROOT = 0x6DA

T_QSIG, T_QNOISE, T_K, T_V, T_LAMBDA, T_GATE, T_KROPE, T_CKV, T_WKVB = range(9)

DTYPES = ("bf16", "f32")


def rng(case_id: int, tensor_id: int, b: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED_ROOT, int(case_id), int(tensor_id), int(b)])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1).astype(np.uint32) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values (bf16 bits or float32) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def normal(case_id: int, tensor_id: int, b: int, shape, dtype: str) -> np.ndarray:
    z = rng(case_id, tensor_id, b).standard_normal(size=tuple(shape), dtype=np.float32)
    return to_storage(z, dtype)


def sigmoid_normal(case_id: int, tensor_id: int, b: int, shape, dtype: str) -> np.ndarray:
    z = rng(case_id, tensor_id, b).standard_normal(size=tuple(shape), dtype=np.float32)
    s = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    return to_storage(s.astype(np.float32), dtype)


def keys(case_id: int, b: int, L: int, Hkv: int, dqk: int, rope_dims: int, dtype: str) -> np.ndarray:
    """One batch row of K, [L, Hkv, dqk]; the last ``rope_dims`` columns shared by all KV heads."""
    if rope_dims <= 0:
        return normal(case_id, T_K, b, (L, Hkv, dqk), dtype)
    nope = dqk - rope_dims
    z = rng(case_id, T_K, b).standard_normal(size=(L, Hkv, nope), dtype=np.float32)
    r = rng(case_id, T_KROPE, b).standard_normal(size=(L, 1, rope_dims), dtype=np.float32)
    full = np.empty((L, Hkv, dqk), dtype=np.float32)
    full[:, :, :nope] = z
    full[:, :, nope:] = r
    return to_storage(full, dtype)


def fwd_row(case_id, b, *, L, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    """All prefill inputs of batch row b (no leading batch dim)."""
    return dict(
        q_sig=normal(case_id, T_QSIG, b, (L, S, dqk), dtype),
        q_noise=normal(case_id, T_QNOISE, b, (L, N, dqk), dtype),
        k=keys(case_id, b, L, Hkv, dqk, rope_dims, dtype),
        v=normal(case_id, T_V, b, (L, Hkv, dv), dtype),
        lam=sigmoid_normal(case_id, T_LAMBDA, b, (L, S), dtype),
        gate=sigmoid_normal(case_id, T_GATE, b, (L, S, dv), dtype),
    )


def fwd_inputs(case_id, *, B, L, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    """Prefill inputs with a leading batch dim: q_sig [B,L,S,dqk], q_noise [B,L,N,dqk],
    k [B,L,Hkv,dqk], v [B,L,Hkv,dv], lam [B,L,S], gate [B,L,S,dv]."""
    rows = [fwd_row(case_id, b, L=L, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv, dtype=dtype,
                    rope_dims=rope_dims) for b in range(B)]
    return {name: np.stack([r[name] for r in rows]) for name in rows[0]}


def varlen_inputs(case_id, *, lens_q, lens_k, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    """Packed-sequence prefill inputs. Sequence i draws its query-side tensors with
    lens_q[i] rows and its keys and values with lens_k[i] rows from the streams of batch
    row i, then every sequence is concatenated along the rows: q_sig [Tq,S,dqk],
    q_noise [Tq,N,dqk], k [Tk,Hkv,dqk], v [Tk,Hkv,dv], lam [Tq,S], gate [Tq,S,dv], and
    cu_q, cu_k int32 [nseq+1] (row offsets, from 0)."""
    parts = {n: [] for n in ("q_sig", "q_noise", "k", "v", "lam", "gate")}
    for i, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        parts["q_sig"].append(normal(case_id, T_QSIG, i, (lq, S, dqk), dtype))
        parts["q_noise"].append(normal(case_id, T_QNOISE, i, (lq, N, dqk), dtype))
        parts["k"].append(keys(case_id, i, lk, Hkv, dqk, rope_dims, dtype))
        parts["v"].append(normal(case_id, T_V, i, (lk, Hkv, dv), dtype))
        parts["lam"].append(sigmoid_normal(case_id, T_LAMBDA, i, (lq, S), dtype))
        parts["gate"].append(sigmoid_normal(case_id, T_GATE, i, (lq, S, dv), dtype))
    out = {n: np.concatenate(v) for n, v in parts.items()}
    out["cu_q"] = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    out["cu_k"] = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return out


def decode_row(case_id, b, *, Lmax, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    """All decode inputs of sequence b: q_sig [S,dqk], q_noise [N,dqk], k_cache [Lmax,Hkv,dqk],
    v_cache [Lmax,Hkv,dv], lam [S], gate [S,dv]."""
    return dict(
        q_sig=normal(case_id, T_QSIG, b, (S, dqk), dtype),
        q_noise=normal(case_id, T_QNOISE, b, (N, dqk), dtype),
        k_cache=keys(case_id, b, Lmax, Hkv, dqk, rope_dims, dtype),
        v_cache=normal(case_id, T_V, b, (Lmax, Hkv, dv), dtype),
        lam=sigmoid_normal(case_id, T_LAMBDA, b, (S,), dtype),
        gate=sigmoid_normal(case_id, T_GATE, b, (S, dv), dtype),
    )


def decode_inputs(case_id, *, B, Lmax, S, N, Hkv, dqk, dv, dtype, rope_dims=0):
    rows = [decode_row(case_id, b, Lmax=Lmax, S=S, N=N, Hkv=Hkv, dqk=dqk, dv=dv, dtype=dtype,
                       rope_dims=rope_dims) for b in range(B)]
    return {name: np.stack([r[name] for r in rows]) for name in rows[0]}


def ragged_lens(case_id: int, B: int, Lmax: int) -> np.ndarray:
    """Non-uniform decode cache lengths in [1, Lmax] (int32), always including 1 and Lmax."""
    g = rng(case_id, 99, 0)
    lens = g.integers(1, Lmax + 1, size=B, dtype=np.int64)
    if B >= 1:
        lens[0] = Lmax
    if B >= 2:
        lens[1] = 1
    return lens.astype(np.int32)


def latent_weights(case_id: int, *, Hkv, Dn, dv, Dc, dtype) -> np.ndarray:
    """The up-projection W^KV_b [Hkv, Dn + dv, Dc] of a latent-cache case."""
    z = rng(case_id, T_WKVB, 0).standard_normal(size=(Hkv, Dn + dv, Dc), dtype=np.float32)
    return to_storage(z * np.float32(1.0 / np.sqrt(Dc)), dtype)


def decode_latent_row(case_id, b, *, Lmax, S, N, Dn, Dr, Dc, dv, dtype):
    """Latent-cache decode inputs of sequence b: q_sig [S,Dn+Dr], q_noise [N,Dn+Dr],
    c_kv [Lmax,Dc], k_rope [Lmax,Dr], lam [S], gate [S,dv]."""
    return dict(
        q_sig=normal(case_id, T_QSIG, b, (S, Dn + Dr), dtype),
        q_noise=normal(case_id, T_QNOISE, b, (N, Dn + Dr), dtype),
        c_kv=normal(case_id, T_CKV, b, (Lmax, Dc), dtype),
        k_rope=normal(case_id, T_KROPE, b, (Lmax, Dr), dtype),
        lam=sigmoid_normal(case_id, T_LAMBDA, b, (S,), dtype),
        gate=sigmoid_normal(case_id, T_GATE, b, (S, dv), dtype),
    )


def decode_latent_inputs(case_id, *, B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, dtype):
    rows = [decode_latent_row(case_id, b, Lmax=Lmax, S=S, N=N, Dn=Dn, Dr=Dr, Dc=Dc, dv=dv,
                              dtype=dtype) for b in range(B)]
    out = {name: np.stack([r[name] for r in rows]) for name in rows[0]}
    out["w_kv_b"] = latent_weights(case_id, Hkv=Hkv, Dn=Dn, dv=dv, Dc=Dc, dtype=dtype)
    return out
