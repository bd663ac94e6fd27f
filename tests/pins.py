"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` function takes the oracle entry points (possibly with a planted
mistake) and returns a list of failure messages (empty = the pin holds). The
tests run them on the exact oracle (all must hold) and on each planted mistake
(at least one must fail).

What each pin rests on:
  * head maps stated by the workload descriptions themselves (layouts A, B, C
    below: "signal head i uses KV head i//4", "noise head j uses KV head 2j and
    is repeated onto signal heads 4j..4j+3", ...), never by the oracle's formula;
  * torch's CPU float64 ``scaled_dot_product_attention`` (a library routine)
    with its default scale;
  * closed forms: uniform weights give the mean of the visible values, a single
    visible key gives that key's value, two visible keys give a logistic mix;
  * invariants of softmax attention: a per-row logit shift, scaling of V or G;
  * a pure-Python brute force on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from attention_gda_fwd_amd import inputs as gin

from . import brute

# Head layouts as the workload descriptions state them.
LAYOUTS = {
    # S=8, N=2, Hkv=2: signal i -> KV i//4; noise j -> KV j; noise j serves signals 4j..4j+3.
    "A": dict(S=8, N=2, Hkv=2, kv_sig=lambda i: i // 4, kv_noise=lambda j: j,
              group=lambda i: i // 4),
    # S=32, N=8, Hkv=16: signal i -> KV i//2; noise j -> KV 2j; noise j serves 4j..4j+3.
    "B": dict(S=32, N=8, Hkv=16, kv_sig=lambda i: i // 2, kv_noise=lambda j: 2 * j,
              group=lambda i: i // 4),
    # S=64, N=16, Hkv=16: signal i -> KV i//4; noise j -> KV j (g=4).
    "C": dict(S=64, N=16, Hkv=16, kv_sig=lambda i: i // 4, kv_noise=lambda j: j,
              group=lambda i: i // 4),
}


def make(layout, *, B=2, L=9, dqk=8, dv=4, dtype="f32", case_id=1000):
    lay = LAYOUTS[layout]
    return gin.fwd_inputs(case_id, B=B, L=L, S=lay["S"], N=lay["N"], Hkv=lay["Hkv"], dqk=dqk,
                          dv=dv, dtype=dtype)


def f64(a, dtype="f32"):
    return gin.storage_to_f64(a, "bf16" if a.dtype == np.uint16 else "f32")


def ones_like_storage(a):
    return gin.to_storage(np.ones(a.shape, dtype=np.float32), "bf16" if a.dtype == np.uint16 else "f32")


def zeros_like_storage(a):
    return gin.to_storage(np.zeros(a.shape, dtype=np.float32), "bf16" if a.dtype == np.uint16 else "f32")


def band_mask(L, window):
    t = torch.arange(L)[:, None]
    s = torch.arange(L)[None, :]
    m = s <= t
    if window:
        m &= (t - s) <= window - 1
    return m


def sdpa(q, k, v, window, scale=None):
    """torch CPU float64 SDPA. q [B,L,d], k [B,L,d], v [B,L,e] -> [B,L,e]."""
    qt = torch.from_numpy(q)[:, None]
    kt = torch.from_numpy(k)[:, None]
    vt = torch.from_numpy(v)[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=band_mask(q.shape[1], window), scale=scale)
    return out[:, 0].numpy()


def _fail(msgs, name, err, tol):
    if not (err <= tol):
        msgs.append(f"{name}: err {err:.3e} > {tol:.1e}")


# ---------------------------------------------------------------------------------------
def pin_library_sdpa(fwd, layouts=("A", "B", "C"), windows=(0, 3)):
    """lambda = 0, gate = 1 -> out_i is plain attention of signal head i over KV kv_sig(i);
    lambda = 1, gate = 1 -> out_i = attn(signal i) - attn(noise group(i)); random lambda and
    gate compose the same two library attentions. dqk != dv so the scale is exercised."""
    msgs = []
    for lay_name in layouts:
        lay = LAYOUTS[lay_name]
        for W in windows:
            x = make(lay_name, dqk=6, dv=4, L=7, case_id=1100)
            qs, qn, k, v = (f64(x[n]) for n in ("q_sig", "q_noise", "k", "v"))
            lamv, gatev = f64(x["lam"]), f64(x["gate"])
            HS = np.stack([sdpa(qs[:, :, i], k[:, :, lay["kv_sig"](i)], v[:, :, lay["kv_sig"](i)], W)
                           for i in range(lay["S"])], axis=2)
            HN = np.stack([sdpa(qn[:, :, j], k[:, :, lay["kv_noise"](j)],
                                v[:, :, lay["kv_noise"](j)], W) for j in range(lay["N"])], axis=2)
            rep = HN[:, :, [lay["group"](i) for i in range(lay["S"])]]
            # lambda = 0, gate = 1
            o0 = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], zeros_like_storage(x["lam"]),
                     ones_like_storage(x["gate"]), window=W)
            _fail(msgs, f"sdpa lam=0 layout {lay_name} W={W}", np.abs(o0 - HS).max(), 1e-12)
            o1 = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], ones_like_storage(x["lam"]),
                     ones_like_storage(x["gate"]), window=W)
            _fail(msgs, f"sdpa lam=1 layout {lay_name} W={W}", np.abs(o1 - (HS - rep)).max(), 1e-12)
            o2 = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], window=W)
            exp2 = gatev * (HS - lamv[..., None] * rep)
            _fail(msgs, f"sdpa random layout {lay_name} W={W}", np.abs(o2 - exp2).max(), 1e-12)
    return msgs


def pin_noise_one_hot(fwd):
    """lambda one-hot on signal head i: only out_i moves, by exactly -attn(noise group(i))."""
    msgs = []
    for lay_name in ("A", "B"):
        lay = LAYOUTS[lay_name]
        x = make(lay_name, L=6, case_id=1200)
        qn, k, v = f64(x["q_noise"]), f64(x["k"]), f64(x["v"])
        zero = zeros_like_storage(x["lam"])
        ones_g = ones_like_storage(x["gate"])
        base = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], zero, ones_g, window=0)
        for i in (0, 3, 5, lay["S"] - 1):
            lam = np.zeros(x["lam"].shape, dtype=np.float32)
            lam[:, :, i] = 1.0
            o = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], gin.to_storage(lam, "f32"), ones_g,
                    window=0)
            j = lay["group"](i)
            hn = sdpa(qn[:, :, j], k[:, :, lay["kv_noise"](j)], v[:, :, lay["kv_noise"](j)], 0)
            _fail(msgs, f"one-hot lambda layout {lay_name} head {i}",
                  np.abs((o[:, :, i] - base[:, :, i]) + hn).max(), 1e-12)
            others = [h for h in range(lay["S"]) if h != i]
            _fail(msgs, f"one-hot lambda leaks, layout {lay_name} head {i}",
                  np.abs(o[:, :, others] - base[:, :, others]).max(), 0.0)
    return msgs


def pin_identical_queries_zero(fwd):
    """q_sig[i] := q_noise[group(i)], lambda = 1: out_i is exactly 0 wherever signal i and
    noise group(i) read the same KV head; nonzero where they do not (layout B, heads 4j+2, 4j+3)."""
    msgs = []
    for lay_name in ("A", "B", "C"):
        lay = LAYOUTS[lay_name]
        x = make(lay_name, L=8, case_id=1300)
        qs = x["q_sig"].copy()
        for i in range(lay["S"]):
            qs[:, :, i] = x["q_noise"][:, :, lay["group"](i)]
        o = fwd(qs, x["q_noise"], x["k"], x["v"], ones_like_storage(x["lam"]), x["gate"], window=0)
        for i in range(lay["S"]):
            same = lay["kv_sig"](i) == lay["kv_noise"](lay["group"](i))
            mx = np.abs(o[:, :, i]).max()
            if same and mx != 0.0:
                msgs.append(f"zero pin layout {lay_name} head {i}: max |out| {mx:.3e} != 0")
            if not same and not (mx > 1e-6):
                msgs.append(f"zero pin layout {lay_name} head {i}: expected nonzero, got {mx:.3e}")
    return msgs


def pin_constant_keys(fwd):
    """All keys of a KV head equal -> uniform weights -> H = mean of the visible V rows."""
    msgs = []
    for lay_name in ("A", "B"):
        lay = LAYOUTS[lay_name]
        for W in (0, 1, 3, 50):
            x = make(lay_name, L=10, case_id=1400)
            k = x["k"].copy()
            k[:] = k[:, :1]  # every key row equal to row 0 of its (b, head)
            vv = f64(x["v"])
            L = vv.shape[1]
            mean = np.zeros_like(vv)
            for t in range(L):
                lo = 0 if W == 0 else max(0, t - W + 1)
                mean[:, t] = vv[:, lo:t + 1].mean(axis=1)
            HS = mean[:, :, [lay["kv_sig"](i) for i in range(lay["S"])]]
            HN = mean[:, :, [lay["kv_noise"](lay["group"](i)) for i in range(lay["S"])]]
            exp = f64(x["gate"]) * (HS - f64(x["lam"])[..., None] * HN)
            o = fwd(x["q_sig"], x["q_noise"], k, x["v"], x["lam"], x["gate"], window=W)
            _fail(msgs, f"constant keys layout {lay_name} W={W}", np.abs(o - exp).max(), 1e-13)
    return msgs


def pin_window(fwd):
    """L <= W equals full causal; W = 1 is the own row's value; W = 2 is a logistic mix of
    two rows; W = L-1 differs from full only at the last query."""
    msgs = []
    x = make("A", L=9, case_id=1500)
    args = (x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"])
    full = fwd(*args, window=0)
    for W in (9, 10, 300):
        o = fwd(*args, window=W)
        _fail(msgs, f"L<=W equality W={W}", np.abs(o - full).max(), 0.0)
    lay = LAYOUTS["A"]
    qs, qn, k, v = (f64(x[n]) for n in ("q_sig", "q_noise", "k", "v"))
    lam, gate = f64(x["lam"]), f64(x["gate"])
    S = lay["S"]
    hs_idx = [lay["kv_sig"](i) for i in range(S)]
    hn_idx = [lay["kv_noise"](lay["group"](i)) for i in range(S)]
    # W = 1: only key t is visible, its weight is exactly 1.
    o1 = fwd(*args, window=1)
    exp1 = gate * (v[:, :, hs_idx] - lam[..., None] * v[:, :, hn_idx])
    _fail(msgs, "W=1 closed form", np.abs(o1 - exp1).max(), 1e-15)
    # W = 2: H = v_t + (v_{t-1} - v_t) * logistic(z_{t-1} - z_t), z = q.k / sqrt(dqk).
    o2 = fwd(*args, window=2)
    dqk = qs.shape[-1]
    exp2 = np.empty_like(o2)
    Bn, L = qs.shape[0], qs.shape[1]
    for b in range(Bn):
        for t in range(L):
            for i in range(S):
                j = lay["group"](i)
                def mix(q, h):
                    if t == 0:
                        return v[b, 0, h]
                    dz = (q @ k[b, t - 1, h] - q @ k[b, t, h]) / math.sqrt(dqk)
                    p = 1.0 / (1.0 + math.exp(-dz))
                    return v[b, t, h] + (v[b, t - 1, h] - v[b, t, h]) * p
                hs = mix(qs[b, t, i], hs_idx[i])
                hn = mix(qn[b, t, j], hn_idx[i])
                exp2[b, t, i] = gate[b, t, i] * (hs - lam[b, t, i] * hn)
    _fail(msgs, "W=2 closed form", np.abs(o2 - exp2).max(), 1e-12)
    # W = L-1: only the last query row loses a key (key 0).
    o8 = fwd(*args, window=8)
    _fail(msgs, "W=L-1 equal before last row", np.abs(o8[:, :8] - full[:, :8]).max(), 0.0)
    if not np.abs(o8[:, 8] - full[:, 8]).max() > 1e-9:
        msgs.append("W=L-1 last row should differ from full attention")
    return msgs


def pin_invariances(fwd):
    """A per-KV-head shift c_h added to every key changes each row's logits by a constant
    (output unchanged); V -> 2V and G -> 2G each double the output exactly."""
    msgs = []
    g = np.random.default_rng(7)
    x = make("B", L=8, case_id=1600)
    # dyadic keys and shifts so that k + c is exact in float32
    k = (g.integers(-16, 17, size=x["k"].shape) / 8.0).astype(np.float32)
    c = (g.integers(-16, 17, size=(1, 1, x["k"].shape[2], x["k"].shape[3])) / 8.0).astype(np.float32)
    c = np.broadcast_to(c, (k.shape[0], 1) + c.shape[2:])
    base_args = [x["q_sig"], x["q_noise"], k, x["v"], x["lam"], x["gate"]]
    for W in (0, 3):
        o = fwd(*base_args, window=W)
        shifted = fwd(x["q_sig"], x["q_noise"], (k + c).astype(np.float32), x["v"], x["lam"],
                      x["gate"], window=W)
        _fail(msgs, f"key shift invariance W={W}", np.abs(shifted - o).max() / np.abs(o).max(),
              1e-12)
        o_v = fwd(x["q_sig"], x["q_noise"], k, (2 * x["v"]).astype(np.float32), x["lam"],
                  x["gate"], window=W)
        _fail(msgs, f"V scaling W={W}", np.abs(o_v - 2 * o).max(), 0.0)
        o_g = fwd(x["q_sig"], x["q_noise"], k, x["v"], x["lam"], (2 * x["gate"]).astype(np.float32),
                  window=W)
        _fail(msgs, f"G scaling W={W}", np.abs(o_g - 2 * o).max(), 0.0)
    return msgs


def pin_decode_is_last_row(fwd, decode):
    """Decode over a cache of length n equals prefill row n-1 over the same K/V."""
    msgs = []
    for lay_name in ("A", "B"):
        for W in (0, 3):
            x = make(lay_name, B=3, L=11, case_id=1700)
            lens = np.array([11, 1, 6], dtype=np.int32)
            full = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], window=W)
            bi = np.arange(3)
            ti = lens - 1
            dec = decode(x["q_sig"][bi, ti], x["q_noise"][bi, ti], x["k"], x["v"], x["lam"][bi, ti],
                         x["gate"][bi, ti], lens, window=W)
            _fail(msgs, f"decode == last prefill row, layout {lay_name} W={W}",
                  np.abs(dec - full[bi, ti]).max(), 0.0)
            # lens above the cache are clamped; lens below 1 give zeros
            dec2 = decode(x["q_sig"][bi, ti], x["q_noise"][bi, ti], x["k"], x["v"],
                          x["lam"][bi, ti], x["gate"][bi, ti], np.array([99, 0, -3], np.int32),
                          window=W)
            _fail(msgs, f"decode clamp, layout {lay_name} W={W}",
                  np.abs(dec2[0] - full[0, 10]).max(), 0.0)
            _fail(msgs, f"decode empty rows, layout {lay_name} W={W}", np.abs(dec2[1:]).max(), 0.0)
    return msgs


def pin_brute_force(fwd):
    """Pure-Python enumeration on tiny shapes, including an N > Hkv layout."""
    msgs = []
    shapes = [
        ("A", LAYOUTS["A"]),
        ("N>Hkv", dict(S=8, N=4, Hkv=2, kv_sig=lambda i: i // 4, kv_noise=lambda j: j // 2,
                       group=lambda i: i // 2)),
        ("g=1", dict(S=2, N=2, Hkv=1, kv_sig=lambda i: 0, kv_noise=lambda j: 0,
                     group=lambda i: i)),
    ]
    for name, lay in shapes:
        for L, W in ((1, 0), (2, 0), (5, 0), (9, 3), (9, 1), (5, 100)):
            for dtype in ("f32", "bf16"):
                x = gin.fwd_inputs(1800 + L, B=2, L=L, S=lay["S"], N=lay["N"], Hkv=lay["Hkv"],
                                   dqk=3, dv=2, dtype=dtype)
                o = fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], window=W)
                ref = brute.gda_fwd(*(f64(x[n]).tolist() for n in
                                      ("q_sig", "q_noise", "k", "v", "lam", "gate")), W,
                                    lay["kv_sig"], lay["kv_noise"], lay["group"])
                ref = np.array(ref)
                err = np.abs(o - ref).max() / max(1e-300, np.abs(ref).max())
                _fail(msgs, f"brute force {name} L={L} W={W} {dtype}", err, 1e-12)
    return msgs


def pin_options(fwd_opt, decode_opt):
    """The call options against library routines: an explicit softmax scale is SDPA's own
    ``scale``; lambda/gate given as logits are torch.sigmoid of them (fp64); a zero logit
    is exactly 0.5; decode with options is the last prefill row with the same options."""
    msgs = []
    for lay_name, W, scale in (("A", 0, 0.37), ("B", 3, 1.9), ("C", 0, 0.05)):
        lay = LAYOUTS[lay_name]
        x = make(lay_name, dqk=6, dv=4, L=7, case_id=1150)
        qs, qn, k, v = (f64(x[n]) for n in ("q_sig", "q_noise", "k", "v"))
        HS = np.stack([sdpa(qs[:, :, i], k[:, :, lay["kv_sig"](i)], v[:, :, lay["kv_sig"](i)], W,
                            scale) for i in range(lay["S"])], axis=2)
        HN = np.stack([sdpa(qn[:, :, j], k[:, :, lay["kv_noise"](j)], v[:, :, lay["kv_noise"](j)],
                            W, scale) for j in range(lay["N"])], axis=2)
        rep_ = HN[:, :, [lay["group"](i) for i in range(lay["S"])]]
        # lam and gate storage reused as logits: N(0,1)-ish values via a shift
        lam_logit = gin.to_storage((f64(x["lam"]) * 6.0 - 3.0).astype(np.float32), "f32")
        gate_logit = gin.to_storage((f64(x["gate"]) * 8.0 - 4.0).astype(np.float32), "f32")
        lamv = torch.sigmoid(torch.from_numpy(f64(lam_logit))).numpy()
        gatev = torch.sigmoid(torch.from_numpy(f64(gate_logit))).numpy()
        args = (x["q_sig"], x["q_noise"], x["k"], x["v"])
        o = fwd_opt(*args, x["lam"], x["gate"], window=W, scale=scale)
        exp_ = f64(x["gate"]) * (HS - f64(x["lam"])[..., None] * rep_)
        _fail(msgs, f"explicit scale layout {lay_name} W={W}", np.abs(o - exp_).max(), 1e-12)
        o = fwd_opt(*args, lam_logit, gate_logit, window=W, scale=scale, lambda_logits=True,
                    gate_logits=True)
        exp_ = gatev * (HS - lamv[..., None] * rep_)
        _fail(msgs, f"logits layout {lay_name} W={W}", np.abs(o - exp_).max(), 1e-12)
        o = fwd_opt(*args, x["lam"], gate_logit, window=W, scale=scale, gate_logits=True)
        exp_ = gatev * (HS - f64(x["lam"])[..., None] * rep_)
        _fail(msgs, f"gate logits only layout {lay_name} W={W}", np.abs(o - exp_).max(), 1e-12)
        # zero logits are exactly one half
        z = zeros_like_storage(x["lam"]), zeros_like_storage(x["gate"])
        half = (gin.to_storage(np.full(x["lam"].shape, 0.5, np.float32), "f32"),
                gin.to_storage(np.full(x["gate"].shape, 0.5, np.float32), "f32"))
        oz = fwd_opt(*args, *z, window=W, lambda_logits=True, gate_logits=True)
        oh = fwd_opt(*args, *half, window=W)
        if not np.array_equal(oz, oh):
            msgs.append(f"zero logits != 0.5 values layout {lay_name}")
        # decode = last prefill row, with the same options
        dec = decode_opt(x["q_sig"][:, -1], x["q_noise"][:, -1], x["k"], x["v"],
                         lam_logit[:, -1], gate_logit[:, -1], window=W, scale=scale,
                         lambda_logits=True, gate_logits=True)
        full = fwd_opt(*args, lam_logit, gate_logit, window=W, scale=scale, lambda_logits=True,
                       gate_logits=True)
        _fail(msgs, f"decode options layout {lay_name}", np.abs(dec - full[:, -1]).max(), 1e-13)
    return msgs


def _latent_expanded(x, w_sel=None):
    """Expanded K/V tensors of a latent case for the (already pinned) expanded-cache
    oracle. With ``w_sel`` = (cols, signs) [Hkv, Dn+dv] the up-projection is a signed
    column selection, so the expansion is an exact copy of latent entries (any dtype);
    otherwise it is a numpy float64 matmul stored as float32."""
    ckv = f64(x["c_kv"])
    B, Lmax, Dc = ckv.shape
    Dr = x["k_rope"].shape[2]
    Dn = x["q_sig"].shape[2] - Dr
    if w_sel is not None:
        cols, signs = w_sel
        kvx = ckv[:, :, cols] * signs  # [B, Lmax, Hkv, Dn+dv], exact
        st = "bf16" if x["c_kv"].dtype == np.uint16 else "f32"
    else:
        kvx = np.einsum("hrc,bsc->bshr", f64(x["w_kv_b"]), ckv)
        st = "f32"
    Hkv = kvx.shape[2]
    k = np.concatenate([kvx[..., :Dn], np.broadcast_to(f64(x["k_rope"])[:, :, None, :],
                                                        (B, Lmax, Hkv, Dr))], axis=-1)
    v = kvx[..., Dn:]
    conv = lambda a: gin.to_storage(np.ascontiguousarray(a).astype(np.float32), st)  # noqa: E731
    return conv(k), conv(v), st


def _pin_latent_layout(decode_latent, decode, shp):
    msgs = []
    lens = np.array([11, 1, 7, 0, 5], dtype=np.int32)
    for dtype in ("f32", "bf16"):
        x = gin.decode_latent_inputs(1300, B=5, Lmax=11, dtype=dtype, **shp)
        rng = np.random.default_rng(1301)
        cols = np.stack([rng.permutation(shp["Dc"])[:shp["Dn"] + shp["dv"]]
                         for _ in range(shp["Hkv"])])
        signs = rng.choice([-1.0, 1.0], size=cols.shape)
        w = np.zeros((shp["Hkv"], shp["Dn"] + shp["dv"], shp["Dc"]), np.float32)
        for h in range(shp["Hkv"]):
            w[h, np.arange(cols.shape[1]), cols[h]] = signs[h]
        xs = dict(x, w_kv_b=gin.to_storage(w, dtype))
        k, v, st = _latent_expanded(xs, (cols, signs))
        for W in (0, 3):
            got = decode_latent(xs["q_sig"], xs["q_noise"], xs["c_kv"], xs["k_rope"], xs["w_kv_b"],
                                xs["lam"], xs["gate"], lens, window=W)
            ref = decode(xs["q_sig"], xs["q_noise"], k, v, xs["lam"], xs["gate"], lens, window=W)
            _fail(msgs, f"latent selection {shp} {dtype} W={W}", np.abs(got - ref).max(), 1e-12)
    x = gin.decode_latent_inputs(1302, B=5, Lmax=11, dtype="f32", **shp)
    k, v, _ = _latent_expanded(x)
    for W in (0, 4):
        got = decode_latent(x["q_sig"], x["q_noise"], x["c_kv"], x["k_rope"], x["w_kv_b"],
                            x["lam"], x["gate"], lens, window=W)
        ref = decode(x["q_sig"], x["q_noise"], k, v, x["lam"], x["gate"], lens, window=W)
        _fail(msgs, f"latent random {shp} W={W}", np.abs(got - ref).max(), 2e-6)
    return msgs


def pin_latent(decode_latent, decode):
    """Latent-cache decode against the expanded-cache decode oracle on explicitly
    expanded K/V: exactly (signed selection up-projections, bf16 and fp32) and to
    float32 rounding (random up-projections), ragged lengths and windows."""
    msgs = []
    for shp in (dict(S=8, N=2, Hkv=2, Dn=6, Dr=4, Dc=16, dv=5),
                dict(S=8, N=2, Hkv=4, Dn=5, Dr=3, Dc=12, dv=4)):  # noise on every other KV head
        msgs += _pin_latent_layout(decode_latent, decode, shp)
    return msgs


ARGS = ("q_sig", "q_noise", "k", "v", "lam", "gate")


def pin_varlen(fwd_varlen):
    """Packed sequences with a query offset against the batched oracle, which is pinned
    above: one whole sequence; packed documents of different lengths each equal to its own
    prefill; a halo chunk (queries = the last rows, keys = all rows) equal to the last
    rows of the full prefill; fewer keys than queries: zeros at negative positions, the
    rest equal to a prefill whose queries are shifted by the difference."""
    msgs = []
    for dtype in ("f32", "bf16"):
        for W in (0, 4):
            x = make("A", B=3, L=23, dqk=6, dv=4, dtype=dtype, case_id=1400)
            one = {n: x[n][0] for n in ARGS}
            full = oracle.ref_fwd(*(x[n][:1] for n in ARGS), window=W)[0]
            o = fwd_varlen(*(one[n] for n in ARGS), [0, 23], [0, 23], window=W)
            if not np.array_equal(o, full):
                msgs.append(f"varlen one sequence {dtype} W={W}")
            # packed documents: lengths 11, 5, 8 taken from three batch rows
            lens = (11, 5, 8)
            pk = {n: np.concatenate([x[n][b, :lens[b]] for b in range(3)]) for n in ARGS}
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            o = fwd_varlen(*(pk[n] for n in ARGS), cu, cu, window=W)
            for b in range(3):
                ref = oracle.ref_fwd(*(x[n][b:b + 1, :lens[b]] for n in ARGS), window=W)[0]
                if not np.array_equal(o[cu[b]:cu[b + 1]], ref):
                    msgs.append(f"varlen packed document {b} {dtype} W={W}")
            # halo: the last 9 queries over all 23 keys
            qa = {n: one[n][14:] if n in ("q_sig", "q_noise", "lam", "gate") else one[n] for n in ARGS}
            o = fwd_varlen(*(qa[n] for n in ARGS), [0, 9], [0, 23], window=W)
            if not np.array_equal(o, full[14:]):
                msgs.append(f"varlen halo {dtype} W={W}")
            # fewer keys than queries: 23 queries over the first 20 keys
            kk = {n: one[n][:20] if n in ("k", "v") else one[n] for n in ARGS}
            o = fwd_varlen(*(kk[n] for n in ARGS), [0, 23], [0, 20], window=W)
            if np.any(o[:3] != 0.0):
                msgs.append(f"varlen negative positions not zero {dtype} W={W}")
            sh = {n: (one[n][3:] if n in ("q_sig", "q_noise", "lam", "gate") else one[n][:20])
                  for n in ARGS}
            ref = oracle.ref_fwd(*(sh[n][None] for n in ARGS), window=W)[0]
            if not np.array_equal(o[3:], ref):
                msgs.append(f"varlen shifted queries {dtype} W={W}")
    return msgs


# ---------------------------------------------------------------------------------------
# The backward and the training form of the forward.
BWD_LAYOUTS = {
    "A": LAYOUTS["A"], "B": LAYOUTS["B"],
    # more noise heads than KV heads: S=4, N=2, Hkv=1, every head on KV 0, groups of 2
    "D": dict(S=4, N=2, Hkv=1, kv_sig=lambda i: 0, kv_noise=lambda j: 0,
              group=lambda i: i // 2),
}


def make_bwd(lay_name, *, B=2, L=7, dqk=6, dv=4, dtype="f32", case_id=1500, logits=False):
    lay = BWD_LAYOUTS[lay_name]
    x = gin.fwd_inputs(case_id, B=B, L=L, S=lay["S"], N=lay["N"], Hkv=lay["Hkv"], dqk=dqk,
                       dv=dv, dtype=dtype)
    if logits:  # logits: unbounded draws in place of the sigmoid values
        x["lam"] = np.stack([gin.normal(case_id, 41, b, x["lam"].shape[1:], dtype)
                             for b in range(B)])
        x["gate"] = np.stack([gin.normal(case_id, 42, b, x["gate"].shape[1:], dtype)
                              for b in range(B)])
    x["d_out"] = np.stack([gin.normal(case_id, 50, b, x["gate"].shape[1:], dtype)
                           for b in range(B)])
    return x


def torch_gda_grads(x, lay, window, scale=None, lambda_logits=False, gate_logits=False):
    """Gradients of sum(d_out * out) by torch autograd in float64, with out composed from
    torch's scaled_dot_product_attention per head as the workload descriptions state the
    head maps (no step of the oracle)."""
    t = {n: torch.from_numpy(f64(x[n])).requires_grad_(n != "d_out") for n in x}
    L = t["q_sig"].shape[1]
    mask = band_mask(L, window)
    F = torch.nn.functional

    def att(q, k, v):
        return F.scaled_dot_product_attention(q[:, None], k[:, None], v[:, None],
                                              attn_mask=mask, scale=scale)[:, 0]

    HS = torch.stack([att(t["q_sig"][:, :, i], t["k"][:, :, lay["kv_sig"](i)],
                          t["v"][:, :, lay["kv_sig"](i)]) for i in range(lay["S"])], dim=2)
    HN = torch.stack([att(t["q_noise"][:, :, j], t["k"][:, :, lay["kv_noise"](j)],
                          t["v"][:, :, lay["kv_noise"](j)]) for j in range(lay["N"])], dim=2)
    lamv = torch.sigmoid(t["lam"]) if lambda_logits else t["lam"]
    G = torch.sigmoid(t["gate"]) if gate_logits else t["gate"]
    rep = HN[:, :, [lay["group"](i) for i in range(lay["S"])]]
    out = G * (HS - lamv[..., None] * rep)
    (out * t["d_out"]).sum().backward()
    return dict(dq_sig=t["q_sig"].grad, dq_noise=t["q_noise"].grad, dk=t["k"].grad,
                dv=t["v"].grad, dlam=t["lam"].grad, dgate=t["gate"].grad)


BWD_CASES = [  # (layout, window, options)
    ("A", 0, {}), ("A", 3, {}), ("B", 0, {}), ("B", 4, {}), ("D", 0, {}), ("D", 2, {}),
    ("A", 0, dict(scale=0.3, lambda_logits=True, gate_logits=True)),
    ("B", 3, dict(scale=0.45, gate_logits=True)),
]


def pin_backward(bwd, cases=BWD_CASES, dtype="f32"):
    """Every gradient against torch autograd through the library attention."""
    msgs = []
    for lay_name, W, opts in cases:
        x = make_bwd(lay_name, dtype=dtype, logits=bool(opts))
        got = bwd(*(x[n] for n in ARGS), x["d_out"], window=W, **opts)
        ref = torch_gda_grads(x, BWD_LAYOUTS[lay_name], W, **opts)
        for name, r in ref.items():
            r = r.numpy()
            tol = 1e-11 * max(1.0, np.abs(r).max())
            _fail(msgs, f"backward {name} layout {lay_name} W={W} {opts}",
                  np.abs(got[name] - r).max(), tol)
    return msgs


def pin_fwd_train(fwd_train, fwd):
    """Training-form outputs: out equals the plain forward, each path's output equals the
    library attention, lse equals torch's logsumexp of the masked, scaled scores."""
    msgs = []
    for lay_name, W, opts in BWD_CASES:
        lay = BWD_LAYOUTS[lay_name]
        x = make_bwd(lay_name, logits=bool(opts))
        out, hs, hn, lse = fwd_train(*(x[n] for n in ARGS), window=W, **opts)
        _fail(msgs, f"train out {lay_name} W={W}",
              np.abs(out - fwd(*(x[n] for n in ARGS), window=W, **opts)).max(), 1e-13)
        qs, qn, k, v = (f64(x[n]) for n in ("q_sig", "q_noise", "k", "v"))
        sc = opts.get("scale") or 1.0 / math.sqrt(qs.shape[-1])
        mask = band_mask(qs.shape[1], W)
        for h in range(lay["S"] + lay["N"]):
            sig = h < lay["S"]
            q = qs[:, :, h] if sig else qn[:, :, h - lay["S"]]
            kv = lay["kv_sig"](h) if sig else lay["kv_noise"](h - lay["S"])
            H = sdpa(q, k[:, :, kv], v[:, :, kv], W, scale=opts.get("scale"))
            got_h = hs[:, :, h] if sig else hn[:, :, h - lay["S"]]
            _fail(msgs, f"train H head {h} {lay_name} W={W}", np.abs(got_h - H).max(), 1e-12)
            z = sc * torch.einsum("bld,bsd->bls", torch.from_numpy(q),
                                  torch.from_numpy(k[:, :, kv]))
            ref_lse = torch.logsumexp(z.masked_fill(~mask, -math.inf), dim=-1).numpy()
            _fail(msgs, f"train lse head {h} {lay_name} W={W}",
                  np.abs(lse[:, h] - ref_lse).max(), 1e-12)
    return msgs


def pin_backward_rows(bwd):
    """Selected query and key rows equal the same rows of the full backward (the sampled
    form the full-size checks use)."""
    msgs = []
    for W in (0, 3):
        x = make_bwd("A", B=2, L=11)
        full = bwd(*(x[n] for n in ARGS), x["d_out"], window=W)
        q_rows, k_rows = [0, 5, 13, 21], [1, 10, 11, 20]
        part = bwd(*(x[n] for n in ARGS), x["d_out"], window=W, q_rows=q_rows, k_rows=k_rows)
        L = 11
        for name in ("dq_sig", "dq_noise", "dlam", "dgate"):
            f = full[name].reshape((2 * L,) + full[name].shape[2:])[q_rows]
            if not np.array_equal(f, part[name]):
                msgs.append(f"rows {name} W={W}")
        for name in ("dk", "dv"):
            f = full[name].reshape((2 * L,) + full[name].shape[2:])[k_rows]
            if not np.array_equal(f, part[name]):
                msgs.append(f"rows {name} W={W}")
    return msgs


def pin_bwd_varlen(bwd_varlen, train_varlen):
    """Packed-sequence backward against the batched backward, which is pinned above:
    packed documents give each document's own gradients; a sequence cut into chunks whose
    keys start with a W-1 halo gives the whole sequence's query-side gradients row for row,
    and its K/V gradients once every chunk's contributions to a key are summed; queries at
    negative positions get zero gradients and the rest are those of the shorter problem.
    The training forward's outputs match the batched ones per document."""
    msgs = []
    Q = ("q_sig", "q_noise", "lam", "gate", "d_out")
    for W in (0, 4):
        x = make_bwd("A", B=3, L=17, case_id=1600)
        # packed documents of lengths 17, 6, 11 taken from three batch rows
        lens = (17, 6, 11)
        pk = {n: np.concatenate([x[n][b, :lens[b]] for b in range(3)]) for n in x}
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        got = bwd_varlen(*(pk[n] for n in ARGS), pk["d_out"], cu, cu, window=W)
        out, hs, hn, lse = train_varlen(*(pk[n] for n in ARGS), cu, cu, window=W)
        for b in range(3):
            one = {n: x[n][b:b + 1, :lens[b]] for n in x}
            ref = oracle.ref_bwd(*(one[n] for n in ARGS), one["d_out"], window=W)
            for name, r in ref.items():
                if not np.array_equal(got[name][cu[b]:cu[b + 1]], r[0]):
                    msgs.append(f"varlen bwd document {b} {name} W={W}")
            r_out, r_hs, r_hn, r_lse = oracle.ref_fwd_train(*(one[n] for n in ARGS), window=W)
            _fail(msgs, f"varlen train out doc {b} W={W}",
                  np.abs(out[cu[b]:cu[b + 1]] - r_out[0]).max(), 1e-13)
            _fail(msgs, f"varlen train h doc {b} W={W}",
                  max(np.abs(hs[cu[b]:cu[b + 1]] - r_hs[0]).max(),
                      np.abs(hn[cu[b]:cu[b + 1]] - r_hn[0]).max()), 1e-13)
            _fail(msgs, f"varlen train lse doc {b} W={W}",
                  np.abs(lse[:, cu[b]:cu[b + 1]] - r_lse[0]).max(), 1e-13)
    # halo chunks: one sequence of 17 rows in chunks of 6, 6, 5; window W = 4 (halo 3)
    W, L = 4, 17
    x = make_bwd("B", B=1, L=L, case_id=1610)
    one = {n: x[n][0] for n in x}
    full = oracle.ref_bwd(*(x[n] for n in ARGS), x["d_out"], window=W)
    starts, C = (0, 6, 12), 6
    q_parts, k_parts, cu_q, cu_k = {n: [] for n in Q}, {"k": [], "v": []}, [0], [0]
    for c0 in starts:
        c1, h0 = min(c0 + C, L), max(0, c0 - (W - 1))
        for n in Q:
            q_parts[n].append(one[n][c0:c1])
        for n in ("k", "v"):
            k_parts[n].append(one[n][h0:c1])
        cu_q.append(cu_q[-1] + c1 - c0)
        cu_k.append(cu_k[-1] + c1 - h0)
    pk = {n: np.concatenate(v) for n, v in {**q_parts, **k_parts}.items()}
    got = bwd_varlen(*(pk[n] for n in ARGS), pk["d_out"], cu_q, cu_k, window=W)
    for name in ("dq_sig", "dq_noise", "dlam", "dgate"):
        if not np.array_equal(got[name], full[name][0]):
            msgs.append(f"halo chunks {name}")
    for name in ("dk", "dv"):
        acc = np.zeros_like(full[name][0])
        for ci, c0 in enumerate(starts):
            c1, h0 = min(c0 + C, L), max(0, c0 - (W - 1))
            acc[h0:c1] += got[name][cu_k[ci]:cu_k[ci + 1]]
        _fail(msgs, f"halo chunks {name} summed", np.abs(acc - full[name][0]).max(), 1e-12)
    # more queries than keys: 17 queries over the first 13 keys
    x = make_bwd("D", B=1, L=17, case_id=1620)
    one = {n: x[n][0] for n in x}
    kk = {n: (one[n][:13] if n in ("k", "v") else one[n]) for n in one}
    got = bwd_varlen(*(kk[n] for n in ARGS), kk["d_out"], [0, 17], [0, 13], window=0)
    for name in ("dq_sig", "dq_noise", "dlam", "dgate"):
        if np.any(got[name][:4] != 0.0):
            msgs.append(f"negative positions: {name} not zero")
    sh = {n: (one[n][4:] if n in Q else one[n][:13]) for n in one}
    ref = oracle.ref_bwd(*(sh[n][None] for n in ARGS), sh["d_out"][None], window=0)
    for name in ("dq_sig", "dq_noise", "dlam", "dgate"):
        if not np.array_equal(got[name][4:], ref[name][0]):
            msgs.append(f"shifted queries {name}")
    for name in ("dk", "dv"):
        _fail(msgs, f"shifted queries {name}", np.abs(got[name] - ref[name][0]).max(), 1e-13)
    return msgs


def all_pins(fwd, decode):
    msgs = []
    for p in (pin_library_sdpa, pin_noise_one_hot, pin_identical_queries_zero,
              pin_constant_keys, pin_window, pin_invariances, pin_brute_force):
        msgs += p(fwd)
    msgs += pin_decode_is_last_row(fwd, decode)
    return msgs


def oracle_entry_points():
    def fwd(*a, window, rows=None):
        return oracle.ref_fwd(*a, window=window, rows=rows)

    def decode(*a, window):
        return oracle.ref_decode(*a, window=window)

    return fwd, decode
