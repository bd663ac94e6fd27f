"""libgda: the Grouped Differential (Latent) Attention forward on MI355X (gfx950).

``gda_fwd`` (prefill) and ``gda_decode`` (one token over a KV cache) call the
hand-written HIP kernels of ``libgda.so`` through its C ABI (include/gda.h).
The torch front end is imported lazily so that ``inputs``/``configs`` load
without torch or the built library.
"""
from __future__ import annotations

__all__ = ["gda_fwd", "gda_decode", "GdaError"]


def __getattr__(name):
    if name in ("gda_fwd", "gda_decode"):
        from . import api
        return getattr(api, name)
    if name == "GdaError":
        from ._lib import GdaError
        return GdaError
    raise AttributeError(name)
