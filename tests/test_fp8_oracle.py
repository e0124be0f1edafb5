"""Pins of the FP8 (OCP E4M3) weight oracle, CPU only.

What fixes the oracle here, beside its own definition:
  * constants of the E4M3 format (largest finite value 448, smallest normal 2^-6,
    smallest subnormal 2^-9, 1.0 at 0x38, NaN at S.1111.111, no infinities);
  * hand-worked rounding cases (ties to the even code, saturation);
  * an independent library encoder: torch's float8_e4m3fn cast, which rounds to
    nearest even, on random in-range values and on every midpoint of the grid;
  * round trips, the per-row scale rule, and the error bound of the reading;
  * planted mistakes (tie to the odd code, truncation, a scale of max/240) that
    the battery must catch.
"""
import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F


def test_format_constants():
    t = F.e4m3_table()
    assert t[0x38] == 1.0
    assert t[0x40] == 2.0
    assert t[0xB8] == -1.0
    assert t[0x7E] == 448.0                       # largest finite value
    assert t[0x08] == 2.0 ** -6                   # smallest normal
    assert t[0x01] == 2.0 ** -9                   # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9               # largest subnormal
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.count_nonzero(np.isnan(t)) == 2 and np.all(np.isfinite(t[~np.isnan(t)]))
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)               # codes 0x00..0x7E increase strictly
    assert np.array_equal(t[0x80:0xFF], -pos)     # sign bit mirrors


@pytest.mark.parametrize("v, code", [
    (1.0625, 0x38),          # midway 1.0 (m = 0) and 1.125 (m = 1): to the even code, 1.0
    (1.1875, 0x3A),          # midway 1.125 (m = 1) and 1.25 (m = 2): to 1.25
    (1.05, 0x38), (1.07, 0x39), (1.10, 0x39),   # either side of the 1.0625 midpoint
    (448.0, 0x7E), (460.0, 0x7E), (1.0e6, 0x7E), (-1.0e6, 0xFE),   # saturation
    (2.0 ** -10, 0x00),      # half the smallest subnormal: tie to 0 (even)
    (3 * 2.0 ** -10, 0x02),  # midway 2^-9 (code 1) and 2^-8 (code 2): to code 2
    (15 * 2.0 ** -10, 0x08), # midway 7 x 2^-9 (code 7) and 2^-6 (code 8): to code 8
    (-0.0, 0x80), (0.0, 0x00),
])
def test_hand_worked_rounding(v, code):
    assert int(F.encode_e4m3(np.array([v]))[0]) == code


def _torch_codes(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_float8_on_random_and_midpoint_values():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.normal(0, 50, 4000), rng.uniform(-448, 448, 4000),
                        rng.normal(0, 0.01, 2000)]).astype(np.float32)
    pos = F.e4m3_table()[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)       # every midpoint is an fp32 value
    v = np.concatenate([v, mids, -mids, pos.astype(np.float32)])
    assert np.array_equal(F.encode_e4m3(v.astype(np.float64)), _torch_codes(v))


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.encode_e4m3(F.decode_e4m3(codes)), codes)


def _bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_row_scale_rule_and_error_bound():
    rng = np.random.default_rng(3)
    w = _bf16(rng.normal(0, 0.02, (64, 512)))
    w[5] = 0                                                   # an all-zero row
    codes, scales = F.quantize_rows(w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    amax = np.abs(wf).max(axis=1)
    nz = amax > 0
    assert scales.dtype == np.float32
    assert np.array_equal(scales[nz], (amax[nz].astype(np.float32) / np.float32(448)))
    assert scales[5] == 1.0 and np.all(codes[5] == 0)
    # the largest element of each row lands on 448 (code 0x7E or 0xFE)
    assert np.all((codes[nz] & 0x7F).max(axis=1) == 0x7E)
    # error: at most half a grid step (2^-4 relative for normals, 2^-10 absolute
    # below the smallest normal), times the scale, plus the fp32 quotient's rounding
    deq = F.dequantize_rows(codes, scales)
    q = np.abs(wf) / scales.astype(np.float64)[:, None]
    bound = np.where(q >= 2.0 ** -6, q * 2.0 ** -4, 2.0 ** -10) * scales[:, None] * (1 + 1e-6)
    assert np.all(np.abs(deq - wf) <= bound + 1e-30)


def test_fp8_weights_wrapper_changes_only_expert_matrices():
    class Inp:
        x = np.zeros((2, 32), dtype=np.uint16)
        w_router = np.zeros((4, 32), dtype=np.uint16)
        bias = None

        def expert(self, e):
            rng = np.random.default_rng(e)
            return _bf16(rng.normal(0, 0.02, (16, 32))), _bf16(rng.normal(0, 0.02, (32, 8)))

        def shared(self):
            return self.expert(9)

    inp = Inp()
    f = F.Fp8Weights(inp)
    assert f.x is inp.x and f.w_router is inp.w_router and f.bias is None
    a, b = f.expert(2)
    ca, sa = F.quantize_rows(inp.expert(2)[0])
    assert np.array_equal(a, F.decode_e4m3(ca) * sa.astype(np.float64)[:, None])
    assert b.shape == (32, 8) and f.shared()[0].shape == (16, 32)


def test_planted_mistakes_are_caught():
    rng = np.random.default_rng(11)
    v = rng.uniform(-448, 448, 5000).astype(np.float32)
    pos = F.e4m3_table()[:0x7F]
    v = np.concatenate([v, ((pos[1:] + pos[:-1]) / 2).astype(np.float32)])
    ref = _torch_codes(v)

    def ties_to_odd(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        hi = np.minimum(np.searchsorted(pos, a), len(pos) - 1)
        lo = np.maximum(hi - 1, 0)
        pick = (pos[hi] - a < a - pos[lo]) | ((pos[hi] - a == a - pos[lo]) & (hi % 2 == 1))
        return (np.where(pick, hi, lo) | (np.signbit(x) << 7)).astype(np.uint8)

    def truncating(x):
        x = np.asarray(x, dtype=np.float64)
        lo = np.maximum(np.searchsorted(pos, np.abs(x), side="right") - 1, 0)
        return (lo | (np.signbit(x) << 7)).astype(np.uint8)

    for wrong in (ties_to_odd, truncating):
        assert not np.array_equal(wrong(v), ref)
    # a scale for the fnuz variant (largest value 240) leaves codes past 0x77 unused
    w = _bf16(rng.normal(0, 1, (8, 256)))
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    bad = F.encode_e4m3((wf / (np.abs(wf).max(axis=1, keepdims=True) / np.float32(240))).astype(np.float64))
    assert not np.array_equal(bad, F.quantize_rows(w)[0])
