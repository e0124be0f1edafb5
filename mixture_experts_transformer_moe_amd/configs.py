"""Workload shapes for the MoE feed-forward layer.

Each workload fixes the layer shape (tokens T, model width D, routed experts E,
experts per token k, routed SwiGLU width F, shared SwiGLU width Fs), the routed
scale alpha, the arithmetic type and the recipe of its seeded synthetic inputs.

Routing constants follow "Laguna M.1/XS.2 Technical Report" (Key claims, the
XS.2 routing item, report section 3.1): sigmoid router over 256 experts,
token-choice top-8, renormalisation after top-k, routed output scaled by 2.5,
one always-on shared expert.  The M.1 widths (D = 4096, expert width 1024)
come from the "Laguna-M.1-base" card (Shape: d_model; Mixture of experts:
Expert dim).  The XS.2 width (D = 2048, F = 512) is not given by any page and
is an assumed value consistent with XS.2's 33.4B total / 3B active.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Dict, Optional


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int            # tokens in the batch
    D: int            # model width (router and expert input / output width)
    E: int            # routed experts
    k: int            # experts selected per token
    F: int            # routed expert SwiGLU width
    Fs: int           # shared expert SwiGLU width (0 = no shared expert)
    alpha: float      # scale on the routed sum
    dtype: str        # "f32" or "bf16": storage and MFMA operand type
    seed: int
    # input recipe
    x_recipe: str = "rmsnorm"          # "normal" (N(0, x_std^2)) or "rmsnorm" (N(0,1) -> RMSNorm)
    x_std: float = 1.0
    w_std: float = 0.02
    bias: Optional[str] = None         # None or "zipf" (log of a Zipf(s) popularity pmf)
    zipf_s: float = 1.2
    outlier_frac: float = 0.0          # share of tokens that carry outliers
    outlier_scale: float = 50.0
    outlier_channels: int = 8
    # training pass: upstream gradient dout ~ N(0, dout_std^2); padding tokens
    # at the tails of sequences of seq_len tokens, pad_frac of the batch on
    # average; auxiliary load-balancing loss coefficient
    dout_std: float = 1.0
    pad_frac: float = 0.0
    seq_len: int = 1024
    aux_coef: float = 1e-3

    @property
    def S(self) -> int:
        """Routed rows: one per (token, selected expert)."""
        return self.k * self.T

    def as_dict(self) -> Dict:
        return asdict(self)

    def flops(self) -> float:
        """Algorithmic FLOPs of one layer pass (multiply-add = 2)."""
        router = 2.0 * self.T * self.D * self.E
        routed = 6.0 * self.S * self.D * self.F
        shared = 6.0 * self.T * self.D * self.Fs
        return router + routed + shared


def variant(base: MoEShape, **kw) -> MoEShape:
    """Same recipe with some fields changed (used for edge cases)."""
    d = base.as_dict()
    d.update(kw)
    return MoEShape(**d)


TINY_F32 = MoEShape("tiny_f32_t64", T=64, D=256, E=16, k=4, F=128, Fs=128, alpha=2.5,
                    dtype="f32", seed=0, x_recipe="normal", x_std=0.02)
XS2_T4096 = MoEShape("xs2_bf16_t4096_d2048", T=4096, D=2048, E=256, k=8, F=512, Fs=512,
                     alpha=2.5, dtype="bf16", seed=1)
M1_T8192 = MoEShape("m1_bf16_t8192_d4096", T=8192, D=4096, E=256, k=8, F=1024, Fs=1024,
                    alpha=2.5, dtype="bf16", seed=2)
DECODE_SKEW_T32 = MoEShape("decode_zipf_bf16_t32_d4096", T=32, D=4096, E=256, k=8, F=1024,
                           Fs=1024, alpha=2.5, dtype="bf16", seed=3, bias="zipf")
PREFILL_OUTLIER_T32768 = MoEShape("prefill_outlier_bf16_t32768_d2048", T=32768, D=2048, E=256,
                                  k=8, F=512, Fs=512, alpha=2.5, dtype="bf16", seed=4,
                                  outlier_frac=0.1)

# M.1's own routing at its widths: top-16 of 256 with routed scale 1
# ("Laguna-M.1-base", Mixture of experts: experts per token, routed scaling
# factor).
M1_TOP16_T8192 = MoEShape("m1_top16_bf16_t8192_d4096", T=8192, D=4096, E=256, k=16, F=1024,
                          Fs=1024, alpha=1.0, dtype="bf16", seed=5)

# The training pass at the XS.2 shape: one padded batch (padding tokens at the
# ends of 1024-token sequences, 1/16 of the batch on average; "Laguna M.1/XS.2
# Technical Report", thread on the report: padding tokens are not routed) and
# an auxiliary-loss coefficient of 1e-3 (the pages give none).
XS2_TRAIN_T4096 = variant(XS2_T4096, name="xs2_train_bf16_t4096_d2048", pad_frac=1 / 16,
                          aux_coef=1e-3)

WORKLOADS: Dict[str, MoEShape] = {s.name: s for s in
                                  (TINY_F32, XS2_T4096, M1_T8192, DECODE_SKEW_T32,
                                   PREFILL_OUTLIER_T32768, M1_TOP16_T8192, XS2_TRAIN_T4096)}

# The single-GPU benchmark workload: the largest single-GPU configuration, the
# long prefill chunk (32768 tokens at the XS.2 widths: 1.89 TFLOP per pass).
BENCH_WORKLOAD = PREFILL_OUTLIER_T32768.name


def get(name: str) -> MoEShape:
    return WORKLOADS[name]


