"""CPU oracle of FP8 expert weights (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does.  It shares no code with the HIP path.

The pages list FP8 as a shipped weight format for the MoE layers ("Laguna M.1/XS.2
Technical Report", Key claims: FP8 / INT4 / NVFP4 quantised releases) but give
no encoding details, so this is a reading, stated here and in the design notes:

  * element format: OCP 8-bit floating point E4M3 -- sign, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
    infinities, S.1111.111 = NaN; largest finite value 448, smallest normal
    2^-6, smallest subnormal 2^-9;
  * one fp32 scale per output row of every weight matrix (per output channel):
    s_r = max_c |w[r, c]| / 448, computed in fp32 (1 for an all-zero row);
  * code[r, c] = the E4M3 value nearest to w[r, c] / s_r (quotient in fp32),
    ties to the even code, magnitudes past 448 saturating to 448;
  * the layer then runs with the weights code * s_r (exact in fp64).

The quotient and the scale are fp32 because they decide integer codes: the
kernel computes them in fp32, and both sides must take that decision in the
same precision.  Rounding itself is exact here: every fp32 quotient is exactly
representable in float64, and the nearest grid point is found by search over
the explicit list of the format's values.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (0..255) from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6          # subnormal: 0.m x 2^(1 - bias)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float64 values of all 256 codes (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_POS = e4m3_table()[:0x7F]        # codes 0x00..0x7E: the non-negative finite values, increasing


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite value (ties to the even code; |v| > 448 -> 448)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_e4m3: non-finite input")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first grid value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(v)
    return (mag | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return e4m3_table()[np.asarray(codes, dtype=np.int64)]


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_rows(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(codes uint8 [..., rows, cols], scales float32 [..., rows]) of bf16 weights.

    ``w_bits`` holds bf16 bit patterns with the output rows on the second-to-last
    axis and the reduction (input) axis last.
    """
    w = _bf16_to_f32(w_bits)
    amax = np.max(np.abs(w), axis=-1)                                    # exact (a max of fp32 values)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (w / scale[..., None]).astype(np.float32)                          # fp32 quotient, as the kernel
    return encode_e4m3(q.astype(np.float64)), scale


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 weights code * scale."""
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[..., None]


class Fp8Weights:
    """A layer's inputs with every expert weight matrix replaced by its FP8 reading.

    Wraps an object with ``x``, ``w_router``, ``bias``, ``expert(e)`` and
    ``shared()`` (bf16 bit patterns) and returns the dequantized expert and
    shared matrices in float64; the router and the tokens are unchanged.
    """

    def __init__(self, inputs):
        self._inputs = inputs
        self.x = inputs.x
        self.w_router = inputs.w_router
        self.bias = inputs.bias

    def expert(self, e: int):
        a, b = self._inputs.expert(e)
        return dequantize_rows(*quantize_rows(a)), dequantize_rows(*quantize_rows(b))

    def shared(self):
        sh = self._inputs.shared()
        if sh is None:
            return None
        return dequantize_rows(*quantize_rows(sh[0])), dequantize_rows(*quantize_rows(sh[1]))
