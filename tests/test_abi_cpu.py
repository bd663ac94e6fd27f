"""The C ABI of libgda without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (so no pointer is ever
dereferenced here; the pointers below are never valid device memory)."""
import ctypes
import os
import re

import pytest

from attention_gda_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # non-null, never dereferenced: every call below fails validation first
BF16, F32 = _lib.GDA_BF16, _lib.GDA_F32
INVALID, UNSUPPORTED, HIPERR = (_lib.GDA_ERROR_INVALID_ARGUMENT, _lib.GDA_ERROR_UNSUPPORTED,
                                _lib.GDA_ERROR_HIP)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gda_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = _lib.load()
    assert lib.gda_status_string(0) == b"GDA_SUCCESS"
    assert lib.gda_status_string(1) == b"GDA_ERROR_INVALID_ARGUMENT"
    assert lib.gda_status_string(2) == b"GDA_ERROR_UNSUPPORTED"
    assert lib.gda_status_string(3) == b"GDA_ERROR_HIP"
    assert lib.gda_status_string(77) == b"GDA_UNKNOWN_STATUS"


def fwd(**kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, out=FAKE, B=1, L=64, S=8,
             N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16, stream=None)
    a.update(kw)
    return _lib.fwd_raw(a["q"], a["qn"], a["k"], a["v"], a["lam"], a["gate"], a["out"], a["B"],
                        a["L"], a["S"], a["N"], a["Hkv"], a["dqk"], a["dv"], a["window"],
                        a["dtype"], a["stream"])


def dec(**kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lens=None, lam=FAKE, gate=FAKE, out=FAKE, B=1,
             Lmax=64, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16, stream=None)
    a.update(kw)
    return _lib.decode_raw(a["q"], a["qn"], a["k"], a["v"], a["lens"], a["lam"], a["gate"],
                           a["out"], a["B"], a["Lmax"], a["S"], a["N"], a["Hkv"], a["dqk"],
                           a["dv"], a["window"], a["dtype"], a["stream"])


INVALID_CASES = [
    dict(q=None), dict(qn=None), dict(k=None), dict(v=None), dict(lam=None), dict(gate=None),
    dict(out=None), dict(B=0), dict(S=0), dict(N=0), dict(Hkv=0), dict(dqk=0), dict(dv=0),
    dict(B=-1), dict(window=-1), dict(S=8, N=3), dict(S=6, N=2, Hkv=4),
    dict(S=24, N=6, Hkv=4), dict(dtype=7),
    dict(q=FAKE + 8), dict(k=FAKE + 4), dict(gate=FAKE + 2), dict(out=FAKE + 8),  # not 16B aligned
]


@pytest.mark.parametrize("kw", INVALID_CASES, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_fwd_invalid_arguments(kw):
    assert fwd(**kw) == INVALID
    assert _lib.load().gda_last_error() != b""


@pytest.mark.parametrize("kw", INVALID_CASES + [dict(Lmax=0)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_decode_invalid_arguments(kw):
    if "L" in kw:
        kw = dict(kw, Lmax=kw.pop("L"))
    assert dec(**kw) == INVALID


def fwd_ex(opts, **kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, out=FAKE, B=1, L=64, S=8,
             N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16, stream=None)
    a.update(kw)
    return _lib.fwd_ex_raw(a["q"], a["qn"], a["k"], a["v"], a["lam"], a["gate"], a["out"], a["B"],
                           a["L"], a["S"], a["N"], a["Hkv"], a["dqk"], a["dv"], a["window"],
                           a["dtype"], opts, a["stream"])


def dec_ex(opts, **kw):
    return _lib.decode_ex_raw(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 64, 8, 2, 2, 64,
                              64, 0, kw.get("dtype", BF16), opts, None)


@pytest.mark.parametrize("opts", [_lib.Options(-1.0, 0), _lib.Options(float("nan"), 0),
                                  _lib.Options(float("inf"), 0), _lib.Options(0.0, 4),
                                  _lib.Options(0.1, 0x80000000)],
                         ids=["negative_scale", "nan_scale", "inf_scale", "flag4", "flag31"])
def test_invalid_options(opts):
    assert fwd_ex(opts) == INVALID
    assert dec_ex(opts) == INVALID
    assert fwd_ex(opts, dtype=F32) == INVALID


def test_valid_options_reach_the_device_check():
    if _gpu_visible():
        pytest.skip("a GPU is visible: a valid call would launch on the fake pointers")
    for opts in (None, _lib.Options(0.0, 0), _lib.Options(0.125, 3)):
        assert fwd_ex(opts) == HIPERR
        assert dec_ex(opts) == HIPERR


def lat(ws=FAKE, ws_bytes=1 << 30, **kw):
    a = dict(q=FAKE, qn=FAKE, c=FAKE, r=FAKE, w=FAKE, lens=None, lam=FAKE, gate=FAKE, out=FAKE,
             B=2, Lmax=64, S=64, N=16, Hkv=16, Dn=128, Dr=64, Dc=512, dv=128, window=0,
             dtype=BF16)
    a.update(kw)
    return _lib.decode_latent_raw(a["q"], a["qn"], a["c"], a["r"], a["w"], a["lens"], a["lam"],
                                  a["gate"], a["out"], a["B"], a["Lmax"], a["S"], a["N"],
                                  a["Hkv"], a["Dn"], a["Dr"], a["Dc"], a["dv"], a["window"],
                                  a["dtype"], None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(c=None), dict(r=None), dict(w=None),
                                dict(out=None), dict(c=FAKE + 8), dict(w=FAKE + 2), dict(B=0),
                                dict(Dn=0), dict(Dr=-1), dict(S=8, N=3), dict(window=-1),
                                dict(ws=None), dict(ws=FAKE + 8), dict(ws_bytes=100)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_latent_invalid_arguments(kw):
    assert lat(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(dtype=F32), dict(Dc=256), dict(Dn=64), dict(dv=64),
                                dict(S=128, N=16, Hkv=16),   # 144 query heads
                                dict(S=64, N=4, Hkv=4)],     # 16 signal heads per noise head
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_latent_unsupported(kw):
    assert lat(**kw) == UNSUPPORTED


def lat_noalloc(**kw):
    a = dict(q=FAKE, qn=FAKE, c=FAKE, r=FAKE, w=FAKE, lens=None, lam=FAKE, gate=FAKE, out=FAKE,
             B=2, Lmax=64, S=64, N=16, Hkv=16, Dn=128, Dr=64, Dc=512, dv=128, window=0,
             dtype=BF16)
    a.update(kw)
    return _lib.decode_latent_noalloc_raw(a["q"], a["qn"], a["c"], a["r"], a["w"], a["lens"],
                                          a["lam"], a["gate"], a["out"], a["B"], a["Lmax"],
                                          a["S"], a["N"], a["Hkv"], a["Dn"], a["Dr"], a["Dc"],
                                          a["dv"], a["window"], a["dtype"], None, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(out=None), dict(c=FAKE + 8), dict(B=0),
                                dict(S=8, N=3), dict(window=-1)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_latent_noalloc_invalid_arguments(kw):
    assert lat_noalloc(**kw) == INVALID


def test_latent_noalloc_rejects_sizes_beyond_its_scratch():
    # Sizes whose workspace exceeds the static scratch are refused on the host, before
    # any HIP call, with the reason in gda_last_error.
    big = dict(B=512, Lmax=1 << 20)
    assert _lib.latent_workspace_bytes(512, 1 << 20, 64, 16, 0) > _lib.DECODE_LATENT_SCRATCH_BYTES
    assert lat_noalloc(**big) == INVALID
    assert b"scratch" in _lib.load().gda_last_error()
    assert lat_noalloc(dtype=F32) == UNSUPPORTED
    assert lat_noalloc(Dc=256) == UNSUPPORTED
    if not _gpu_visible():
        assert lat_noalloc() == HIPERR


def test_latent_noalloc_scratch_size_matches_the_header():
    src = open(os.path.join(ROOT, "include", "gda.h")).read()
    m = re.search(r"#define GDA_DECODE_LATENT_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DECODE_LATENT_SCRATCH_BYTES


def test_latent_workspace_size():
    n = _lib.latent_workspace_bytes(64, 32768, 64, 16, 0)
    assert 0 < n < 512 << 20
    assert _lib.latent_workspace_bytes(64, 32768, 64, 16, 128) <= n
    assert _lib.latent_workspace_bytes(0, 1, 1, 1, 0) == 0


def varlen(**kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, out=FAKE, cu_q=FAKE,
             cu_k=FAKE, nseq=3, maxq=64, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16,
             opts=None)
    a.update(kw)
    return _lib.fwd_varlen_raw(a["q"], a["qn"], a["k"], a["v"], a["lam"], a["gate"], a["out"],
                               a["cu_q"], a["cu_k"], a["nseq"], a["maxq"], a["S"], a["N"],
                               a["Hkv"], a["dqk"], a["dv"], a["window"], a["dtype"], a["opts"],
                               None)


@pytest.mark.parametrize("kw", [dict(cu_q=None), dict(cu_k=None), dict(q=None), dict(out=None),
                                dict(cu_q=FAKE + 2), dict(k=FAKE + 8), dict(nseq=0),
                                dict(maxq=0), dict(window=-1), dict(S=8, N=3),
                                dict(opts=_lib.Options(-1.0, 0)), dict(dtype=7)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_varlen_invalid_arguments(kw):
    assert varlen(**kw) == INVALID


def test_varlen_unsupported_and_device_check():
    assert varlen(dqk=96, dv=96) == UNSUPPORTED
    if not _gpu_visible():
        assert varlen() == HIPERR
        assert varlen(S=16, N=2, Hkv=2) == HIPERR  # any valid head layout
        assert varlen(dtype=F32, dqk=40, dv=24) == HIPERR


def train(**kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, out=FAKE, hs=FAKE, hn=FAKE,
             lse=FAKE, B=1, L=64, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16)
    a.update(kw)
    return _lib.fwd_train_raw(a["q"], a["qn"], a["k"], a["v"], a["lam"], a["gate"], a["out"],
                              a["hs"], a["hn"], a["lse"], a["B"], a["L"], a["S"], a["N"],
                              a["Hkv"], a["dqk"], a["dv"], a["window"], a["dtype"], None, None)


def bwd(ws=FAKE, ws_bytes=1 << 30, **kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, hs=FAKE, hn=FAKE, lse=FAKE,
             do=FAKE, dqs=FAKE, dqn=FAKE, dk=FAKE, dvo=FAKE, dl=FAKE, dg=FAKE, B=1, L=64, S=8,
             N=2, Hkv=2, dqk=64, dv=64, window=0, dtype=BF16)
    a.update(kw)
    return _lib.bwd_raw(*(a[n] for n in ("q", "qn", "k", "v", "lam", "gate", "hs", "hn", "lse",
                                         "do", "dqs", "dqn", "dk", "dvo", "dl", "dg", "B", "L",
                                         "S", "N", "Hkv", "dqk", "dv", "window", "dtype")),
                        None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(hs=None), dict(lse=None), dict(hn=FAKE + 8),
                                dict(lse=FAKE + 2), dict(B=0), dict(window=-1), dict(S=8, N=3)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_fwd_train_invalid_arguments(kw):
    assert train(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(do=None), dict(dk=None), dict(ws=None), dict(ws=FAKE + 16),
                                dict(ws_bytes=100), dict(dl=FAKE + 8), dict(lse=FAKE + 1),
                                dict(L=0), dict(S=8, N=3)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_bwd_invalid_arguments(kw):
    assert bwd(**kw) == INVALID


def test_training_unsupported_and_device_check():
    assert train(dtype=F32) == UNSUPPORTED
    assert train(dqk=96, dv=96) == UNSUPPORTED
    assert bwd(dtype=F32) == UNSUPPORTED
    assert bwd(dqk=96, dv=96) == UNSUPPORTED
    if not _gpu_visible():
        assert train() == HIPERR
        assert bwd() == HIPERR


def test_bwd_workspace_size():
    n = _lib.bwd_workspace_bytes(2, 8192, 64, 16, 128)
    assert n >= 2 * 8192 * (64 + 16) * (128 * 2 + 4)
    assert _lib.bwd_workspace_bytes(0, 1, 1, 1, 1) == 0


def train_varlen(**kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, out=FAKE, hs=FAKE, hn=FAKE,
             lse=FAKE, cq=FAKE, ck=FAKE, nseq=2, maxq=64, tq=100, S=8, N=2, Hkv=2, dqk=64,
             dv=64, window=0, dtype=BF16)
    a.update(kw)
    return _lib.fwd_train_varlen_raw(*(a[n] for n in ("q", "qn", "k", "v", "lam", "gate", "out",
                                                      "hs", "hn", "lse", "cq", "ck", "nseq",
                                                      "maxq", "tq", "S", "N", "Hkv", "dqk", "dv",
                                                      "window", "dtype")), None, None)


def bwd_varlen(ws=FAKE, ws_bytes=1 << 30, **kw):
    a = dict(q=FAKE, qn=FAKE, k=FAKE, v=FAKE, lam=FAKE, gate=FAKE, hs=FAKE, hn=FAKE, lse=FAKE,
             do=FAKE, dqs=FAKE, dqn=FAKE, dk=FAKE, dvo=FAKE, dl=FAKE, dg=FAKE, cq=FAKE, ck=FAKE,
             nseq=2, maxq=64, maxk=80, tq=100, S=8, N=2, Hkv=2, dqk=64, dv=64, window=0,
             dtype=BF16)
    a.update(kw)
    return _lib.bwd_varlen_raw(*(a[n] for n in ("q", "qn", "k", "v", "lam", "gate", "hs", "hn",
                                                "lse", "do", "dqs", "dqn", "dk", "dvo", "dl", "dg",
                                                "cq", "ck", "nseq", "maxq", "maxk", "tq", "S", "N",
                                                "Hkv", "dqk", "dv", "window", "dtype")),
                               None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(cq=None), dict(ck=FAKE + 2), dict(lse=None), dict(tq=0),
                                dict(nseq=0), dict(maxq=0), dict(hs=FAKE + 8)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_fwd_train_varlen_invalid_arguments(kw):
    assert train_varlen(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(cq=None), dict(ck=FAKE + 1), dict(maxk=0), dict(tq=0),
                                dict(ws_bytes=100), dict(ws=FAKE + 16), dict(do=None)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_bwd_varlen_invalid_arguments(kw):
    assert bwd_varlen(**kw) == INVALID


def test_training_varlen_unsupported_and_device_check():
    assert train_varlen(dtype=F32) == UNSUPPORTED
    assert bwd_varlen(dqk=96, dv=96) == UNSUPPORTED
    if not _gpu_visible():
        assert train_varlen() == HIPERR
        assert bwd_varlen() == HIPERR


def test_decode_misaligned_lengths():
    assert dec(lens=FAKE + 2) == INVALID
    assert b"aligned" in _lib.load().gda_last_error()


# bf16 is compiled for three (dqk, dv) pairs; only other pairs are unsupported.
@pytest.mark.parametrize("kw", [dict(dqk=96, dv=96), dict(dqk=192, dv=192), dict(dqk=128, dv=64)])
def test_fwd_bf16_unsupported(kw):
    assert fwd(**kw) == UNSUPPORTED


def test_decode_bf16_unsupported():
    assert dec(dqk=96, dv=96) == UNSUPPORTED


# Every head layout the validation accepts (S % N == 0, S % Hkv == 0, one of N and
# Hkv dividing the other) is accepted by every bf16 entry point: without a device it
# gets as far as the device check.
VALID_LAYOUTS = [dict(S=16, N=2, Hkv=2),   # 8 signal heads per KV head (g = 8)
                 dict(S=16, N=4, Hkv=2),   # N > Hkv
                 dict(S=16, N=2, Hkv=8),   # Hkv/N = 4
                 dict(S=12, N=4, Hkv=4),   # g = 3
                 dict(S=10, N=2, Hkv=2),   # g = 5
                 dict(S=64, N=2, Hkv=2),   # 32 signal + 1 noise heads per KV head
                 dict(S=32, N=1, Hkv=8),   # a group over 8 KV heads
                 dict(S=8, N=8, Hkv=2)]    # g = 1, 4 noise heads per KV head


@pytest.mark.parametrize("kw", VALID_LAYOUTS, ids=lambda d: "S{S}_N{N}_Hkv{Hkv}".format(**d))
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)], ids=lambda d: f"d{d[0]}")
def test_every_valid_bf16_layout_reaches_the_device(kw, dims):
    if _gpu_visible():
        pytest.skip("a GPU is visible: a valid call would launch on the fake pointers")
    dqk, dv = dims
    assert fwd(dqk=dqk, dv=dv, **kw) == HIPERR
    assert dec(dqk=dqk, dv=dv, **kw) == HIPERR
    assert varlen(dqk=dqk, dv=dv, **kw) == HIPERR
    assert train(dqk=dqk, dv=dv, **kw) == HIPERR


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


def test_valid_call_without_device_returns_hip_error():
    if _gpu_visible():
        pytest.skip("a GPU is visible: a valid call would launch on the fake pointers")
    assert fwd() == HIPERR
    assert fwd(dtype=F32, dqk=96, dv=80, S=12, N=4, Hkv=2) == HIPERR  # f32 takes any layout
    assert dec() == HIPERR
    assert b"device" in _lib.load().gda_last_error()


def test_python_front_end_checks_before_calling():
    import torch
    from attention_gda_fwd_amd import api
    x = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # CPU tensors are refused before the C call
        api.gda_fwd(x, x[:, :, :2], x[:, :, :2], x[:, :, :2], x[..., 0], x)
    with pytest.raises(TypeError):
        api.gda_fwd(x.half(), x, x, x, x[..., 0], x)
