"""CPU fp64 oracle of the MoE feed-forward layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does.  It shares no code with the HIP path:
it widens the stored inputs to float64 itself and evaluates the layer straight
from its definition with NumPy.

What one token t goes through (notation: x_t in R^D, E routed experts, k
experts per token, routed scale alpha):

 1. router logits  z_t = W_r x_t + b            ("Laguna M.1/XS.2 Technical
    Report", Key claims: sigmoid router, report section 3.1; the bias b is zero
    unless a workload supplies one);
 2. scores         s_{t,e} = 1 / (1 + exp(-z_{t,e}))   (sigmoid, not softmax:
    "Laguna-M.1-base" card, Mixture of experts: Router score);
 3. selection      the k experts first under the order (z descending, expert
    index ascending) -- token-choice top-k (report summary, Key claims: top-8 of
    256); sigma is increasing, so this is the top-k of s with ties to the lower
    index; selection acts on z itself so that fp32 logits keep distinct keys
    where sigma would round them together;
 4. weights        w_{t,j} = s_{t,e_j} / sum_i s_{t,e_i}   (post-top-k
    normalisation: report summary, Key claims; card, Mixture of experts:
    Renormalize top-k = yes);
 5. expert FFN     y = W_d (silu(W_g x) * (W_u x)), silu(a) = a / (1 + e^-a),
    no biases (card, Feed-forward: SwiGLU activation, FFN bias = no);
 6. shared expert  the same SwiGLU with the shared weights, applied to every
    token and added without a gate (report summary, Key claims: "plus a shared
    expert");
 7. output         out_t = ysh_t + alpha * sum_j w_{t,j} y_{t,j}, alpha = 2.5 for
    XS.2 (report summary, Key claims: routed-expert modulation before combining
    with the shared expert).

Bookkeeping for the bit-exact checks of the permutation ("copy expert tokens in
expert order", report summary, Key claims: fused dispatch/grouped GEMM, report
section 3.1.2, Fig. 2): counts_e, offsets = exclusive scan of counts, the tokens
of each expert in ascending token order (sorted_token), and slot_of[t, j], the
position of (t, j) in that order.

Parity pins (tests/test_oracle_pins.py): brute-force per-token dense evaluation
of every expert with rank-counting selection (and of expert_rows' h and y rows),
the routing invariants, closed forms (zero router, k = E, k = 1, zero down
projections, x = 0, E = k = 1), hand-derived single-channel values, and the
parameter counts of the "Laguna-M.1-base" card.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional, Tuple

import numpy as np


# --------------------------------------------------------------------------
# input widening (storage encodings -> float64, exact)
# --------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """fp32 arrays and bf16 bit patterns (uint16) -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


# --------------------------------------------------------------------------
# router: logits, sigmoid scores, top-k, renormalised weights
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """z[t, e] = sum_d x[t, d] * W_r[e, d] + b[e], in float64."""
    z = widen(x) @ widen(w_router).T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(a: np.ndarray) -> np.ndarray:
    return a * sigmoid(a)


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k experts first under (z descending, index ascending).

    Column j of the result is slot j, in that same order.
    """
    z = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite router logits are outside the layer's contract")
    E = z.shape[1]
    if not 1 <= k <= E:
        raise ValueError(f"k={k} outside 1..{E}")
    key = -(z + 0.0)               # +0.0 canonicalises -0.0; equal keys keep index order
    order = np.argsort(key, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def renormalised_weights(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    s = sigmoid(np.take_along_axis(np.asarray(z, dtype=np.float64), idx.astype(np.int64), axis=1))
    return s / s.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# expert order (the on-device form of the dispatch)
# --------------------------------------------------------------------------

@dataclass
class Routing:
    logits: np.ndarray        # [T, E] float64 (self-contained) or widened fp32 logits
    topk_idx: np.ndarray      # [T, k] int32
    topk_w: np.ndarray        # [T, k] float64, sums to 1 per token (alpha not applied)
    counts: np.ndarray        # [E] int32
    offsets: np.ndarray       # [E + 1] int32
    sorted_token: np.ndarray  # [k*T] int32
    slot_of: np.ndarray       # [T, k] int32


def expert_order(topk_idx: np.ndarray, E: int):
    """counts, offsets, sorted_token and slot_of for a routing table."""
    T, k = topk_idx.shape
    counts = np.bincount(topk_idx.ravel(), minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_token = np.empty(T * k, dtype=np.int32)
    slot_of = np.empty((T, k), dtype=np.int32)
    for e in range(E):
        tok, slot = np.nonzero(topk_idx == e)          # row-major: ascending token
        pos = offsets[e] + np.arange(tok.size)
        sorted_token[pos] = tok
        slot_of[tok, slot] = pos
    return counts, offsets.astype(np.int32), sorted_token, slot_of


def route(z: np.ndarray, k: int) -> Routing:
    z = np.asarray(z, dtype=np.float64)
    idx = select_topk(z, k)
    w = renormalised_weights(z, idx)
    counts, offsets, sorted_token, slot_of = expert_order(idx, z.shape[1])
    return Routing(z, idx, w, counts, offsets, sorted_token, slot_of)


def route_from_fp32_logits(logits32: np.ndarray, k: int) -> Routing:
    """Routing decided on given fp32 logits (widened exactly)."""
    return route(np.asarray(logits32, dtype=np.float32).astype(np.float64), k)


# --------------------------------------------------------------------------
# expert evaluation and combine
# --------------------------------------------------------------------------

def swiglu_expert(xrows: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """W_d (silu(W_g x) * (W_u x)) for each row x; w_gate_up rows are [gate; up]."""
    F = w_gate_up.shape[0] // 2
    wg, wu = w_gate_up[:F], w_gate_up[F:]
    g = xrows @ wg.T
    u = xrows @ wu.T
    return (silu(g) * u) @ w_down.T


def shared_output(inputs, xrows64: np.ndarray) -> np.ndarray:
    sh = inputs.shared()
    if sh is None:
        return np.zeros_like(xrows64)
    return swiglu_expert(xrows64, widen(sh[0]), widen(sh[1]))


def forward(inputs, alpha: float, k: int, logits32: Optional[np.ndarray] = None) -> Tuple[np.ndarray, Routing]:
    """Whole-layer output [T, D] in float64, plus the routing used.

    ``inputs`` provides ``x``, ``w_router``, ``bias``, ``expert(e)`` and
    ``shared()`` in storage encoding.  With ``logits32`` the routing is decided
    on those fp32 logits; otherwise the oracle computes its own fp64 logits.
    Experts are evaluated one at a time over their tokens in expert order.
    """
    x = widen(inputs.x)
    E = inputs.w_router.shape[0]
    if logits32 is None:
        r = route(router_logits(inputs.x, inputs.w_router, inputs.bias), k)
    else:
        r = route_from_fp32_logits(logits32, k)
    T, D = x.shape
    y_perm = np.zeros((T * k, D), dtype=np.float64)
    for e in range(E):
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        if hi == lo:
            continue
        a, b = inputs.expert(e)
        y_perm[lo:hi] = swiglu_expert(x[r.sorted_token[lo:hi]], widen(a), widen(b))
    out = shared_output(inputs, x)
    routed = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        routed += r.topk_w[:, j:j + 1] * y_perm[r.slot_of[:, j]]
    out = out + alpha * routed
    return out, r


def forward_tokens(inputs, alpha: float, routing: Routing, tokens: Iterable[int]) -> np.ndarray:
    """Output rows of the given tokens only, under a given routing (float64).

    Each expert used by these tokens is widened once and applied to the tokens
    that selected it.
    """
    tokens = np.asarray(list(tokens), dtype=np.int64)
    x = widen(np.asarray(inputs.x)[tokens])
    out = shared_output(inputs, x)
    routed = np.zeros_like(out)
    sel = routing.topk_idx[tokens]
    for e in np.unique(sel):
        rows, slots = np.nonzero(sel == e)
        a, b = inputs.expert(int(e))
        y = swiglu_expert(x[rows], widen(a), widen(b))
        routed[rows] += routing.topk_w[tokens[rows], slots][:, None] * y
    return out + alpha * routed


def expert_rows(inputs, routing: Routing, e: int, rows: Optional[np.ndarray] = None):
    """Hidden activations h and outputs y of expert e for its rows in expert order.

    ``rows`` are positions inside expert e's segment (default: all).  Returns
    (h [n, F], y [n, D]) in float64.
    """
    lo, hi = int(routing.offsets[e]), int(routing.offsets[e + 1])
    pos = np.arange(lo, hi) if rows is None else lo + np.asarray(rows, dtype=np.int64)
    wgu, wd = (widen(a) for a in inputs.expert(e))
    xr = widen(np.asarray(inputs.x)[routing.sorted_token[pos]])
    F = wgu.shape[0] // 2
    h = silu(xr @ wgu[:F].T) * (xr @ wgu[F:].T)
    return h, h @ wd.T


# --------------------------------------------------------------------------
# invariants (hold for any correct routing)
# --------------------------------------------------------------------------

def check_invariants(topk_idx, topk_w, counts, offsets, sorted_token, slot_of, E: int,
                     w_tol: float = 1e-12) -> None:
    """Raise AssertionError when a routing / expert order breaks an invariant."""
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    S = T * k
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    sorted_token = np.asarray(sorted_token, dtype=np.int64)
    slot_of = np.asarray(slot_of, dtype=np.int64)
    if topk_idx.min(initial=0) < 0 or topk_idx.max(initial=0) >= E:
        raise AssertionError("expert index out of range")
    srt = np.sort(topk_idx, axis=1)
    if k > 1 and np.any(srt[:, 1:] == srt[:, :-1]):
        raise AssertionError("a token selected the same expert twice")
    if topk_w is not None:
        wsum = np.asarray(topk_w, dtype=np.float64).sum(axis=1)
        if np.max(np.abs(wsum - 1.0), initial=0.0) > w_tol:
            raise AssertionError("routing weights do not sum to 1")
        if np.any(np.asarray(topk_w) <= 0):
            raise AssertionError("non-positive routing weight")
    if counts.sum() != S:
        raise AssertionError("expert counts do not sum to k*T")
    if offsets[0] != 0 or offsets[E] != S or np.any(np.diff(offsets) != counts):
        raise AssertionError("offsets are not the exclusive scan of counts")
    if np.any(np.bincount(sorted_token, minlength=T) != k):
        raise AssertionError("a token does not appear exactly k times in expert order")
    if np.any(np.sort(slot_of.ravel()) != np.arange(S)):
        raise AssertionError("slot_of is not a bijection onto [0, kT)")
    tt = np.repeat(np.arange(T), k).reshape(T, k)
    if np.any(sorted_token[slot_of] != tt):
        raise AssertionError("sorted_token[slot_of[t, j]] != t")
    seg = np.searchsorted(offsets, slot_of, side="right") - 1
    if np.any(seg != topk_idx):
        raise AssertionError("slot_of[t, j] is not inside expert topk_idx[t, j]'s segment")
    for e in range(E):
        s = sorted_token[offsets[e]:offsets[e + 1]]
        if s.size > 1 and np.any(np.diff(s) <= 0):
            raise AssertionError(f"expert {e}'s tokens are not strictly ascending")
