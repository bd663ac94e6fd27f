"""The fp64 oracle against things other than itself (no GPU needed).

Each pin from ``tests/pins.py`` must hold for the exact oracle, and every planted
mistake (a dropped or flipped term, a wrong index map, an off-by-one window, a
transposed operand, ...) must break at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

from . import pins, planted

HERE = os.path.dirname(os.path.abspath(__file__))

EXACT_FWD, EXACT_DEC = pins.oracle_entry_points()

PINS_FWD = [pins.pin_library_sdpa, pins.pin_noise_one_hot, pins.pin_identical_queries_zero,
            pins.pin_constant_keys, pins.pin_window, pins.pin_invariances, pins.pin_brute_force]


@pytest.mark.parametrize("pin", PINS_FWD, ids=lambda p: p.__name__)
def test_exact_oracle_pin(pin):
    assert pin(EXACT_FWD) == []


def test_exact_oracle_decode_pin():
    assert pins.pin_decode_is_last_row(EXACT_FWD, EXACT_DEC) == []


@pytest.mark.parametrize("name", sorted(planted.FWD))
def test_planted_mistake_is_caught(name):
    with oracle.loaded_from(planted.build(name)):
        assert pins.all_pins(EXACT_FWD, EXACT_DEC), f"no pin catches the planted mistake {name!r}"


def test_options_pin():
    """Explicit softmax scale and logit inputs, against torch's SDPA and sigmoid."""
    assert pins.pin_options(oracle.ref_fwd, oracle.ref_decode) == []


def test_options_pin_catches_a_missing_sigmoid():
    def fwd_no_sigmoid(*a, window, scale=None, lambda_logits=False, gate_logits=False):
        return oracle.ref_fwd(*a, window=window, scale=scale, lambda_logits=lambda_logits)

    def dec_no_sigmoid(*a, window, scale=None, lambda_logits=False, gate_logits=False):
        return oracle.ref_decode(*a, window=window, scale=scale, lambda_logits=lambda_logits)

    assert pins.pin_options(fwd_no_sigmoid, dec_no_sigmoid)

    def fwd_default_scale(*a, window, scale=None, lambda_logits=False, gate_logits=False):
        return oracle.ref_fwd(*a, window=window, lambda_logits=lambda_logits,
                              gate_logits=gate_logits)

    assert pins.pin_options(fwd_default_scale, oracle.ref_decode)


def test_options_rejected():
    x = pins.make("A", L=4)
    args = (x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"])
    with pytest.raises(ValueError):
        oracle.ref_fwd(*args, window=0, scale=-1.0)
    with pytest.raises(ValueError):
        oracle.ref_fwd(*args, window=0, scale=float("nan"))


def test_varlen_pin():
    assert pins.pin_varlen(oracle.ref_fwd_varlen) == []


def test_varlen_pin_catches_a_wrong_offset():
    """A plausible mistake: each sequence's queries aligned to its first keys (query t at
    key position t) instead of its last. For a single sequence that is the correct
    computation over only its first Lq keys."""
    def top_left(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k, *, window):
        cu_q, cu_k = np.asarray(cu_q), np.asarray(cu_k)
        if cu_q.size != 2:
            return oracle.ref_fwd_varlen(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k,
                                         window=window)
        lq = int(cu_q[1])
        if lq > int(cu_k[1]):
            return oracle.ref_fwd_varlen(q_sig, q_noise, k, v, lam, gate, cu_q, cu_k,
                                         window=window)
        return oracle.ref_fwd_varlen(q_sig, q_noise, k[:lq], v[:lq], lam, gate, cu_q,
                                     [0, lq], window=window)

    assert pins.pin_varlen(top_left)


def test_latent_pin():
    assert pins.pin_latent(oracle.ref_decode_latent, oracle.ref_decode) == []


@pytest.mark.parametrize("name", sorted(planted.LATENT))
def test_latent_planted_mistake_is_caught(name):
    with oracle.loaded_from(planted.build(name)):
        assert pins.pin_latent(oracle.ref_decode_latent, oracle.ref_decode), \
            f"no pin catches {name!r}"


def test_hand_worked_example():
    with open(os.path.join(HERE, "golden", "hand_worked_example.json")) as f:
        ex = json.load(f)
    x = {k: np.array(v, dtype=np.float32) for k, v in ex["inputs"].items()}
    args = (x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"])
    for key, W in (("window_0", 0), ("window_2", 2)):
        expected = np.array([[eval(s, {"__builtins__": {}}, {"e": math.e}) for s in row]
                             for row in ex["expected"][key]])
        got = oracle.ref_fwd(*args, window=W)[0, :, :, 0]
        np.testing.assert_allclose(got, expected, rtol=0, atol=1e-15)


def test_rows_subset_matches_full():
    x = pins.make("B", L=7, case_id=1900)
    args = (x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"])
    full = oracle.ref_fwd(*args, window=3)
    rows = np.array([13, 0, 6, 7])
    sub = oracle.ref_fwd(*args, window=3, rows=rows)
    np.testing.assert_array_equal(sub, full.reshape(-1, *full.shape[2:])[rows])


def test_rejects_bad_arguments():
    x = pins.make("A", L=4)
    with pytest.raises(ValueError):
        oracle.ref_fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], window=-1)
    with pytest.raises(ValueError):
        oracle.ref_fwd(x["q_sig"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"], window=0,
                       rows=[8])
    with pytest.raises(TypeError):
        oracle.ref_fwd(x["q_sig"].astype(np.float64), x["q_noise"], x["k"], x["v"], x["lam"],
                       x["gate"], window=0)


def _bwd():
    def f(*a, **kw):
        return oracle.ref_bwd(*a, **kw)
    return f


def test_backward_pin():
    assert pins.pin_backward(_bwd()) == []


def test_backward_pin_bf16_inputs():
    assert pins.pin_backward(_bwd(), cases=pins.BWD_CASES[:3], dtype="bf16") == []


@pytest.mark.parametrize("name", sorted(planted.BWD))
def test_backward_planted_mistake_is_caught(name):
    with oracle.loaded_from(planted.build(name)):
        assert pins.pin_backward(_bwd()) != []


def test_fwd_train_pin():
    assert pins.pin_fwd_train(oracle.ref_fwd_train, oracle.ref_fwd) == []


def test_backward_rows_subset():
    assert pins.pin_backward_rows(_bwd()) == []


def test_backward_varlen_pin():
    assert pins.pin_bwd_varlen(oracle.ref_bwd_varlen, oracle.ref_fwd_train_varlen) == []


def test_backward_varlen_pin_catches_a_wrong_offset():
    """An oracle that aligns a sequence's queries with its first keys (not its last)
    fails the halo and fewer-keys checks."""
    def top_left(q_sig, q_noise, k, v, lam, gate, d_out, cu_q, cu_k, *, window, **kw):
        cu_q = np.asarray(cu_q)
        cu_k = np.asarray(cu_k)
        g = {n: [] for n in ("dq_sig", "dq_noise", "dlam", "dgate", "dk", "dv")}
        for i in range(len(cu_q) - 1):
            lq, lk = cu_q[i + 1] - cu_q[i], cu_k[i + 1] - cu_k[i]
            q = slice(cu_q[i], cu_q[i + 1])
            kk = slice(cu_k[i], cu_k[i + 1])
            # queries at key positions 0..lq-1, keys padded or cut to lq rows
            def fit(a):
                out = np.zeros((lq,) + a.shape[1:], a.dtype)
                n = min(lq, lk)
                out[:n] = a[:n]
                return out
            r = oracle.ref_bwd(q_sig[q][None], q_noise[q][None], fit(k[kk])[None],
                               fit(v[kk])[None], lam[q][None], gate[q][None], d_out[q][None],
                               window=window, **kw)
            for n in ("dq_sig", "dq_noise", "dlam", "dgate"):
                g[n].append(r[n][0])
            for n in ("dk", "dv"):
                g[n].append(r[n][0][:lk] if lk <= lq else
                            np.concatenate([r[n][0], np.zeros((lk - lq,) + r[n].shape[2:])]))
        return {n: np.concatenate(v) for n, v in g.items()}
    assert pins.pin_bwd_varlen(top_left, oracle.ref_fwd_train_varlen) != []
