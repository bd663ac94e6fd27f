"""Planted mistakes in the oracle, for the tests that show the pins catch them.

Each entry names one plausible mistake (a dropped or flipped term, a wrong index map, an
off-by-one window, a transposed operand, ...) as a text edit of ``oracle/gda_ref.c``: the
first occurrence of a snippet of the exact source, replaced. ``build(name)`` compiles the
edited copy (same flags as the oracle) into a temporary library that the tests load with
``oracle.loaded_from``; the oracle's own source holds no switch for any of them.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

import oracle

# name -> (exact source snippet, planted replacement)
FWD = {
    "drop_lambda": ("      const double D = Hs[e] - lam * Hn[j * dv + e];",
                    "      const double D = Hs[e];"),
    "plus_lambda": ("      const double D = Hs[e] - lam * Hn[j * dv + e];",
                    "      const double D = Hs[e] + lam * Hn[j * dv + e];"),
    "tiled_repeat": ("    const int64_t j = i / g;\n    double lam = rd(lambda, lam_off + i",
                     "    const int64_t j = i % N;\n    double lam = rd(lambda, lam_off + i"),
    "kv_interleave": ("    const int64_t kvs = (i * Hkv) / S;", "    const int64_t kvs = i % Hkv;"),
    "window_off_by_one": ("  int64_t l = W == 0 ? 0 : t - W + 1;",
                          "  int64_t l = W == 0 ? 0 : t - W;"),
    "scale_dv": ("kv->scale > 0.0 ? kv->scale : 1.0 / sqrt((double)dqk);",
                 "kv->scale > 0.0 ? kv->scale : 1.0 / sqrt((double)dv);"),
    "no_gate": ("      out[i * dv + e] = G * D;", "      out[i * dv + e] = D;"),
    "no_causal": ("  visible_range(t, window, &lo, &hi);\n\n  /* Noise path",
                  "  visible_range(t, window, &lo, &hi);\n  hi = kv->Lk - 1;\n\n  /* Noise path"),
    "k_transposed": ("  return ((b * kv->Lk + s) * kv->Hkv + h) * kv->dqk + d;",
                     "  return ((b * kv->Hkv + h) * kv->Lk + s) * kv->dqk + d;"),
    "lambda_by_group": ("    double lam = rd(lambda, lam_off + i, kv->dtype);",
                        "    double lam = rd(lambda, lam_off + j, kv->dtype);"),
    "no_normalize": ("  for (int64_t e = 0; e < kv->dv; ++e) H[e] /= l;\n}", "}"),
    "decode_position": ("        const int64_t p = len - 1;",
                        "        const int64_t p = len < Lmax ? len : Lmax - 1;"),
    "skip_first_key": ("  if (l < 0) l = 0;\n  *lo = l;",
                       "  if (l < 0) l = 0;\n  if (l == 0) l = 1;\n  *lo = l;"),
}
LATENT = {
    "w_transposed": ("        acc += rd(w, (h * rows + r) * Dc + c, dtype)",
                     "        acc += rd(w, (h * Dc + c) * rows + r, dtype)"),
    "no_rope": ("    for (int64_t r = 0; r < Dr; ++r)\n"
                "      acc += rd(q, q_off + Dn + r, dtype) * "
                "rd(k_rope, (b * Lmax + s) * Dr + r, dtype);\n", ""),
    "value_from_key_rows": ("        acc += rd(w, (h * rows + r) * Dc + c, dtype)",
                            "        acc += rd(w, (h * rows + (r < Dn ? r : r - Dn)) * Dc + c, "
                            "dtype)"),
}
BWD = {
    "no_delta": ("          delta[r * HT + h] = dl;", "          delta[r * HT + h] = 0.0;"),
    "lambda_sign": ("            dlam -= dD * H[(S + j) * dv + e];",
                    "            dlam += dD * H[(S + j) * dv + e];"),
    "noise_not_in_dkv": ("        for (int64_t h = 0; h < HT; ++h) {\n"
                         "          const void* q;\n"
                         "          int64_t q_off, kvh;\n"
                         "          head_of(h, qflat,",
                         "        for (int64_t h = 0; h < HT; ++h) {\n"
                         "          if (h >= S) continue;\n"
                         "          const void* q;\n"
                         "          int64_t q_off, kvh;\n"
                         "          head_of(h, qflat,"),
    "dk_without_scale": ("            dk[(rk * Hkv + kvh) * dqk + d] += scale * dz * "
                         "rd(q, q_off + d, dtype);",
                         "            dk[(rk * Hkv + kvh) * dqk + d] += dz * "
                         "rd(q, q_off + d, dtype);"),
    "gate_logit_derivative": ("            if (flags & GDA_REF_GATE_LOGITS) "
                              "dG *= G * (1.0 - G);\n", ""),
}

_DIR = None
_BUILT = {}


def source(name: str) -> str:
    """The oracle source with mistake ``name`` planted (its first occurrence)."""
    old, new = {**FWD, **LATENT, **BWD}[name]
    with open(oracle.SRC) as f:
        src = f.read()
    if old not in src:
        raise AssertionError(f"planted mistake {name!r}: snippet not in the oracle source")
    return src.replace(old, new, 1)


def build(name: str) -> str:
    """Compile the oracle with mistake ``name`` planted; returns the library path."""
    global _DIR
    if name in _BUILT:
        return _BUILT[name]
    if _DIR is None:
        _DIR = tempfile.mkdtemp(prefix="gda_planted_")
    src = os.path.join(_DIR, f"{name}.c")
    with open(src, "w") as f:
        f.write(source(name))
    lib = os.path.join(_DIR, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-I", os.path.dirname(oracle.SRC), "-o", lib, src, "-lm"],
                   check=True)
    _BUILT[name] = lib
    return lib
