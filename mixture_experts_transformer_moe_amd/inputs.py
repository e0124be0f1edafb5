"""Seeded synthetic inputs for the MoE feed-forward layer.

This module is shared by the GPU path and the CPU oracle and holds none of the
layer's arithmetic: it only draws numbers and encodes them.

Every tensor comes from its own stream,
``numpy.random.default_rng(SeedSequence([seed, tensor_id, expert]))``, so one
expert's weights can be regenerated without drawing the others.  Values are
drawn in fp32 and, for bf16 workloads, encoded to bf16 by round-to-nearest-even
on the bit pattern; both sides consume the same bf16 bits (stored here as
``uint16``).

Recipes (per workload, see ``configs.MoEShape``):
  * weights: N(0, w_std^2), w_std = 0.02;
  * x "normal": N(0, x_std^2);
  * x "rmsnorm": N(0, 1), then scaled per token by 1/sqrt(mean(x^2) + 1e-6) in
    fp32 with unit gain, the pre-norm the pages put before every FFN ("Laguna
    M.1/XS.2 Technical Report", Method: pre-norm with RMSNorm; "Laguna-M.1-base"
    card, Normalization: RMSNorm, eps 1e-6);
  * outliers: after normalisation, round(frac*T) seeded tokens are multiplied by
    ``outlier_scale`` on ``outlier_channels`` seeded channels (late-layer
    activation outliers are reported in the digg.com thread on the report,
    quantization item);
  * router bias "zipf": b_e = -s * ln(r_e) with r a seeded permutation of 1..E,
    i.e. the log of a Zipf(s) popularity law, max-normalised to 0;
  * training pass: the upstream gradient dout ~ N(0, dout_std^2) [T, D]; the
    padding mask cuts the batch into sequences of seq_len tokens (the last one
    may be shorter) and pads the tail of each, its length drawn uniformly from
    0 .. 2 pad_frac seq_len, so pad_frac of the tokens are padding on average
    (padded sequence ends, where a packed batch has them).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os
from typing import Optional, Tuple

import numpy as np

from .configs import MoEShape

# tensor ids of the per-tensor random streams
TID_X, TID_ROUTER, TID_BIAS = 0, 1, 2
TID_GATE, TID_UP, TID_DOWN = 3, 4, 5
TID_SGATE, TID_SUP, TID_SDOWN = 6, 7, 8
TID_OUTLIER = 9
TID_DOUT, TID_PAD = 10, 11


def rng_for(seed: int, tensor_id: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, expert]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _encode(shape: MoEShape, a: np.ndarray) -> np.ndarray:
    return a.astype(np.float32) if shape.dtype == "f32" else f32_to_bf16_bits(a)


def _normal(seed: int, tid: int, expert: int, size, std: float) -> np.ndarray:
    g = rng_for(seed, tid, expert)
    return (g.standard_normal(size, dtype=np.float32) * np.float32(std)).astype(np.float32)


def x_f32(shape: MoEShape) -> np.ndarray:
    """Layer input in fp32, before encoding."""
    T, D = shape.T, shape.D
    if shape.x_recipe == "normal":
        x = _normal(shape.seed, TID_X, 0, (T, D), shape.x_std)
    elif shape.x_recipe == "rmsnorm":
        x = _normal(shape.seed, TID_X, 0, (T, D), 1.0)
        ms = np.mean(x * x, axis=1, dtype=np.float32, keepdims=True)
        x = (x / np.sqrt(ms + np.float32(1e-6))).astype(np.float32)
    else:
        raise ValueError(shape.x_recipe)
    if shape.outlier_frac > 0:
        g = rng_for(shape.seed, TID_OUTLIER, 0)
        n_tok = int(round(shape.outlier_frac * T))
        toks = np.sort(g.choice(T, size=n_tok, replace=False))
        chans = np.sort(g.choice(D, size=shape.outlier_channels, replace=False))
        x[np.ix_(toks, chans)] *= np.float32(shape.outlier_scale)
    return x


def outlier_tokens(shape: MoEShape) -> np.ndarray:
    """Indices of the tokens that carry outliers (empty when there are none)."""
    if shape.outlier_frac <= 0:
        return np.zeros(0, dtype=np.int64)
    g = rng_for(shape.seed, TID_OUTLIER, 0)
    n_tok = int(round(shape.outlier_frac * shape.T))
    return np.sort(g.choice(shape.T, size=n_tok, replace=False))


def router_bias(shape: MoEShape) -> Optional[np.ndarray]:
    if shape.bias is None:
        return None
    if shape.bias == "zipf":
        r = rng_for(shape.seed, TID_BIAS, 0).permutation(shape.E) + 1
        return (-np.float64(shape.zipf_s) * np.log(r.astype(np.float64))).astype(np.float32)
    raise ValueError(shape.bias)


def dout_f32(shape: MoEShape) -> np.ndarray:
    """Upstream gradient of the layer output, fp32 [T, D], before encoding."""
    return _normal(shape.seed, TID_DOUT, 0, (shape.T, shape.D), shape.dout_std)


def dout_encoded(shape: MoEShape) -> np.ndarray:
    return _encode(shape, dout_f32(shape))


def token_mask(shape: MoEShape) -> np.ndarray:
    """uint8 [T]: 1 for a real token, 0 for padding (all 1 when pad_frac is 0)."""
    T = shape.T
    mask = np.ones(T, dtype=np.uint8)
    if shape.pad_frac <= 0 or T == 0:
        return mask
    g = rng_for(shape.seed, TID_PAD, 0)
    L = max(1, shape.seq_len)
    top = int(round(2 * shape.pad_frac * L))
    for start in range(0, T, L):
        end = min(start + L, T)
        n_pad = min(int(g.integers(0, top + 1)), end - start)
        mask[end - n_pad:end] = 0
    return mask


class LayerInputs:
    """All inputs of one layer pass, in storage encoding.

    ``x``          [T, D]      fp32 or bf16 bits (uint16)
    ``w_router``   [E, D]      same encoding
    ``bias``       [E] fp32 or None
    ``expert(e)``  -> (w_gate_up [2F, D], w_down [D, F]); rows 0..F-1 of
                   w_gate_up are the gate projection, rows F..2F-1 the up one.
    ``shared()``   -> (ws_gate_up [2Fs, D], ws_down [D, Fs]) or None if Fs == 0.
    """

    def __init__(self, shape: MoEShape, x: Optional[np.ndarray] = None,
                 w_router: Optional[np.ndarray] = None, bias=Ellipsis):
        self.shape = shape
        self.x = _encode(shape, x_f32(shape)) if x is None else x
        if w_router is None:
            w_router = _encode(shape, _normal(shape.seed, TID_ROUTER, 0, (shape.E, shape.D),
                                              shape.w_std))
        self.w_router = w_router
        self.bias = router_bias(shape) if bias is Ellipsis else bias

    def expert(self, e: int) -> Tuple[np.ndarray, np.ndarray]:
        s = self.shape
        if not 0 <= e < s.E:
            raise IndexError(e)
        g = _normal(s.seed, TID_GATE, e, (s.F, s.D), s.w_std)
        u = _normal(s.seed, TID_UP, e, (s.F, s.D), s.w_std)
        d = _normal(s.seed, TID_DOWN, e, (s.D, s.F), s.w_std)
        return _encode(s, np.concatenate([g, u], axis=0)), _encode(s, d)

    def shared(self) -> Optional[Tuple[np.ndarray, np.ndarray]]:
        s = self.shape
        if s.Fs == 0:
            return None
        g = _normal(s.seed, TID_SGATE, 0, (s.Fs, s.D), s.w_std)
        u = _normal(s.seed, TID_SUP, 0, (s.Fs, s.D), s.w_std)
        d = _normal(s.seed, TID_SDOWN, 0, (s.D, s.Fs), s.w_std)
        return _encode(s, np.concatenate([g, u], axis=0)), _encode(s, d)

    def all_experts(self, threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Stacked routed weights: w_gate_up [E, 2F, D], w_down [E, D, F]."""
        s = self.shape
        dt = np.float32 if s.dtype == "f32" else np.uint16
        wgu = np.empty((s.E, 2 * s.F, s.D), dtype=dt)
        wd = np.empty((s.E, s.D, s.F), dtype=dt)

        def fill(e):
            a, b = self.expert(e)
            wgu[e] = a
            wd[e] = b

        n = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(fill, range(s.E)))
        return wgu, wd


def make_inputs(shape: MoEShape) -> LayerInputs:
    return LayerInputs(shape)
