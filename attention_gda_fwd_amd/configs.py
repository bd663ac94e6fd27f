"""The workloads of the GDA forward path (shapes only; no arithmetic).

Head layouts follow the pages: Motif-2-12.7B has 32 signal + 8 noise query heads
over 16 KV heads (overview page, sections 2.1-2.2); Motif 3 has 64 signal + 16
noise query heads over 16 shared KV heads with a 1:3 full:sliding-window (W=128)
layer schedule (Motif 3 release post, architecture and pretraining paragraphs).
Head dims for the Motif 3 layout (dqk = 128 + 64 shared rotary, dv = 128) are
not printed on the pages and are taken as stated by the workload list.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Case:
    name: str
    kind: str          # "fwd" (prefill), "decode" (expanded cache) or "latent" (latent cache)
    dtype: str         # "bf16" or "f32"
    B: int
    L: int             # prefill sequence length, or decode cache length Lmax
    S: int
    N: int
    Hkv: int
    dqk: int
    dv: int
    window: int        # 0 = full causal
    rope_dims: int = 0
    case_id: int = 0   # seed key
    latent: int = 0    # KV latent width Dc of a latent-cache decode (rope_dims = Dr)

    @property
    def g(self) -> int:
        return self.S // self.N

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)

    # Algorithmic work, as the bench reports it -----------------------------------------
    def visible_pairs(self, lens=None) -> int:
        """Visible (query, key) pairs per query head, summed over the batch."""
        W = self.window
        if self.kind == "fwd":
            L = self.L
            if W == 0 or W >= L:
                per = L * (L + 1) // 2
            else:
                per = W * (W + 1) // 2 + (L - W) * W
            return per * self.B
        tot = 0
        for b in range(self.B):
            n = self.L if lens is None else int(min(max(int(lens[b]), 0), self.L))
            tot += n if W == 0 else min(n, W)
        return tot

    def flops(self, lens=None) -> int:
        return 2 * (self.dqk + self.dv) * self.visible_pairs(lens) * (self.S + self.N)

    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self, lens=None) -> int:
        """Every input read once and the output written once, at the stored dtype.
        Decode counts only the cache rows that are visible."""
        e = self.elem_bytes()
        B, L, S, N, H, dqk, dv = self.B, self.L, self.S, self.N, self.Hkv, self.dqk, self.dv
        if self.kind == "fwd":
            n = B * L * (S * dqk + N * dqk + H * dqk + H * dv + S + 2 * S * dv)
            return n * e
        keys = self.visible_pairs(lens)
        if self.kind == "latent":  # per token: the latent and the rotary key; plus W^KV_b
            Dn = dqk - self.rope_dims
            n = (B * (S * dqk + N * dqk + S + 2 * S * dv) + keys * (self.latent + self.rope_dims)
                 + H * (Dn + dv) * self.latent)
            return n * e + (4 * B if lens is not None else 0)
        n = B * (S * dqk + N * dqk + S + 2 * S * dv) + keys * H * (dqk + dv)
        return n * e + (4 * B if lens is not None else 0)

    def bwd_flops(self) -> int:
        """Backward FLOPs per launch: per visible (query, key) pair and query head, the
        score recompute (2 dqk), dP = dO V^T (2 dv), dV (2 dv), dQ (2 dqk), dK (2 dqk)."""
        return 2 * (3 * self.dqk + 2 * self.dv) * self.visible_pairs() * (self.S + self.N)

    def bwd_bytes(self) -> int:
        """Backward bytes: every input read once (Q, K, V, lambda, gate, both paths'
        outputs, the row log-sum-exps, d_out) and every gradient written once."""
        e = self.elem_bytes()
        B, L, S, N, H, dqk, dv = self.B, self.L, self.S, self.N, self.Hkv, self.dqk, self.dv
        reads = (S * dqk + N * dqk + H * dqk + H * dv + S + S * dv + S * dv + N * dv + S * dv)
        writes = S * dqk + N * dqk + H * dqk + H * dv + S + S * dv
        return B * L * (reads + writes) * e + 4 * B * L * (S + N)

    def tokens(self) -> int:
        return self.B * self.L if self.kind == "fwd" else self.B


TINY_F32 = Case("tiny_f32_L256", "fwd", "f32", B=1, L=256, S=8, N=2, Hkv=2, dqk=64, dv=64,
            window=0, case_id=0)
MOTIF2 = Case("motif2_L4096", "fwd", "bf16", B=1, L=4096, S=32, N=8, Hkv=16, dqk=128,
            dv=128, window=0, case_id=1)
MOTIF3_FULL = Case("motif3_full_B2_L8192", "fwd", "bf16", B=2, L=8192, S=64, N=16, Hkv=16,
            dqk=192, dv=128, window=0, rope_dims=64, case_id=2)
MOTIF3_SWA = Case("motif3_swa128_L32768", "fwd", "bf16", B=1, L=32768, S=64, N=16, Hkv=16,
            dqk=192, dv=128, window=128, rope_dims=64, case_id=3)
MOTIF3_DECODE = Case("motif3_decode_B64_Lk32768", "decode", "bf16", B=64, L=32768, S=64, N=16,
            Hkv=16, dqk=192, dv=128, window=0, rope_dims=64, case_id=4)
MOTIF3_DECODE_SWA = MOTIF3_DECODE.with_(name="motif3_decode_swa128_B64_Lk32768", window=128)

# One GPU's share of the Motif 3 full layer when 8 GPUs split its 16 units (whole
# noise groups) with no exchange: 2 units, i.e. 8 signal + 2 noise heads over 2 KV
# heads, at the same batch and length.
MOTIF3_FULL_SHARD8 = MOTIF3_FULL.with_(name="motif3_full_B2_L8192_shard8", S=8, N=2, Hkv=2,
                                       case_id=5)

# The Motif 3 decode over the latent cache (512-wide KV latent + 64-wide rotary key per
# token, expanded by W^KV_b into the 16 KV heads), full and W=128.
MOTIF3_LATENT = MOTIF3_DECODE.with_(name="motif3_latent_decode_B64_Lk32768", kind="latent",
                                    latent=512, case_id=7)
MOTIF3_LATENT_SWA = MOTIF3_LATENT.with_(name="motif3_latent_decode_swa128_B64_Lk32768",
                                        window=128)

CONFIGS = {c.name: c for c in (TINY_F32, MOTIF2, MOTIF3_FULL, MOTIF3_SWA, MOTIF3_DECODE,
                               MOTIF3_DECODE_SWA, MOTIF3_FULL_SHARD8, MOTIF3_LATENT,
                               MOTIF3_LATENT_SWA)}
