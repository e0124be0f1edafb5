"""Test helpers: array-backed layer inputs and an independent brute-force layer.

The brute force below is written separately from the oracle on purpose: plain
Python loops over tokens, experts and channels with ``math.exp``, every expert
evaluated for every token, and selection by rank counting (expert e is chosen
iff fewer than k experts beat it under (logit descending, index ascending)).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np


class ArrayInputs:
    """Layer inputs held as arrays (same interface as ``inputs.LayerInputs``)."""

    def __init__(self, x, w_router, bias, w_gate_up, w_down, shared=None):
        self.x = x
        self.w_router = w_router
        self.bias = bias
        self._wgu = w_gate_up      # [E, 2F, D]
        self._wd = w_down          # [E, D, F]
        self._shared = shared      # (ws_gate_up [2Fs, D], ws_down [D, Fs]) or None

    def expert(self, e):
        return self._wgu[e], self._wd[e]

    def shared(self):
        return self._shared


def random_inputs(rng, T, D, E, F, Fs, scale=0.5, bias=False, dtype=np.float64):
    def n(*shape):
        return (rng.standard_normal(shape) * scale).astype(dtype)
    sh = (n(2 * Fs, D), n(D, Fs)) if Fs else None
    b = (rng.standard_normal(E) * 0.7).astype(np.float32) if bias else None
    return ArrayInputs(n(T, D), n(E, D), b, n(E, 2 * F, D), n(E, D, F), sh)


def _sig(a: float) -> float:
    if a < -700:
        return 0.0
    return 1.0 / (1.0 + math.exp(-a))


def swiglu_hidden_loops(xv: Sequence[float], wgu) -> List[float]:
    """h_f = silu(g_f) * u_f with g_f = <W_gate row f, x>, u_f = <W_up row f, x>
    (rows 0..F-1 of wgu are the gate projection, F..2F-1 the up projection)."""
    F = len(wgu) // 2
    D = len(xv)
    h = []
    for f in range(F):
        g = 0.0
        u = 0.0
        for d in range(D):
            g += float(wgu[f][d]) * xv[d]
            u += float(wgu[F + f][d]) * xv[d]
        h.append(g * _sig(g) * u)
    return h


def _swiglu_loops(xv: Sequence[float], wgu, wd) -> List[float]:
    h = swiglu_hidden_loops(xv, wgu)
    return [sum(float(wd[d][f]) * h[f] for f in range(len(h))) for d in range(len(wd))]


def _as64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def brute_force_layer(inp, k: int, alpha: float):
    """Returns (out [T][D] list, chosen experts per token as sets, weights dicts)."""
    x = _as64(inp.x).tolist()
    wr = _as64(inp.w_router).tolist()
    b = None if inp.bias is None else [float(v) for v in np.asarray(inp.bias, dtype=np.float64)]
    T, D, E = len(x), len(x[0]), len(wr)
    experts = [tuple(_as64(a).tolist() for a in inp.expert(e)) for e in range(E)]
    sh = inp.shared()
    sh = None if sh is None else tuple(_as64(a).tolist() for a in sh)
    outs, chosen, weights = [], [], []
    for t in range(T):
        z = []
        for e in range(E):
            acc = 0.0
            for d in range(D):
                acc += x[t][d] * wr[e][d]
            z.append(acc + (b[e] if b is not None else 0.0))
        sel = []
        for e in range(E):
            better = sum(1 for f in range(E) if z[f] > z[e] or (z[f] == z[e] and f < e))
            if better < k:
                sel.append(e)
        tot = sum(_sig(z[e]) for e in sel)
        w = {e: _sig(z[e]) / tot for e in sel}
        dense = [_swiglu_loops(x[t], *experts[e]) for e in range(E)]   # every expert
        y_sh = _swiglu_loops(x[t], *sh) if sh is not None else [0.0] * D
        row = []
        for d in range(D):
            r = 0.0
            for e in sel:
                r += w[e] * dense[e][d]
            row.append(y_sh[d] + alpha * r)
        outs.append(row)
        chosen.append(set(sel))
        weights.append(w)
    return outs, chosen, weights


def rank_count_select(z_row: Sequence[float], k: int) -> List[int]:
    """Selected experts in slot order, by rank counting."""
    E = len(z_row)
    rank = {}
    for e in range(E):
        rank[e] = sum(1 for f in range(E) if z_row[f] > z_row[e] or (z_row[f] == z_row[e] and f < e))
    return sorted([e for e in range(E) if rank[e] < k], key=lambda e: rank[e])
