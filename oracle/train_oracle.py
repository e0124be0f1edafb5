"""CPU fp64 oracle of the MoE layer's training pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does.  It shares no code with the HIP path.
It builds on the forward oracle (moe_oracle) and adds, in float64:

 * the padding mask.  A padding token is not routed: it selects no expert,
   takes no slot of the expert order and counts in no load statistic; its
   output is the shared expert's alone ("Laguna M.1/XS.2 Technical Report",
   thread on the report: padding tokens always went to one expert and were not
   learnable, so they are neither routed nor load balanced).  Reading: the
   shared expert, a plain dense FFN, still runs over every row.
 * global-batch load statistics and the auxiliary loss (report summary, Key
   claims: load balancing by Qiu et al.'s global-batch auxiliary loss; the
   pages give neither its formula nor its coefficient).  Reading, over the N
   routed tokens of this batch:
       f_e = counts_e / sum_e' counts_e'         share of the routed slots,
             with counts of the GLOBAL batch (the caller's sum over
             micro-batches and data-parallel ranks; this batch's by default),
       p_e = (1/N) sum_t sigma(z_te) / sum_e' sigma(z_te')   mean normalised score,
       L_aux = beta * E * sum_e f_e p_e,
   with the gradient flowing through p only (f is a count).  A uniform
   routing gives L_aux = beta.
 * the backward pass, the chain rule of the forward with the top-k selection
   held fixed (it is piecewise constant), for J = <dout, out> + L_aux:
     combine   dy_{t,j} = alpha w_{t,j} dout_t,  g_{t,j} = alpha <dout_t, y_{t,j}>;
     renorm    ds_j = (g_j - sum_i w_i g_i) / sum_i s_i   over the k slots;
     sigmoid   dz_{t,e_j} += ds_j s_j (1 - s_j);
     aux       with c_e = beta E f_e / N and s' = sigma / Q, Q = sum_e sigma_e:
               dz_{t,m} += (c_m - sum_i c_i s'_i) / Q * sigma_m (1 - sigma_m)
               for every expert m of every routed token;
     SwiGLU    dh = dy W_d, dg = dh u silu'(g), du = dh silu(g),
               silu'(g) = sigma(g) (1 + g (1 - sigma(g)));
     weights   dW_d = dy^T h, dW_g = dg^T a, dW_u = du^T a per expert over its
               rows (the shared expert over all T rows with dy = dout);
     router    dW_r = dz^T x, db = sum_t dz_t;
     input     dx_t = (dg W_g + du W_u)_shared + sum_j (dg W_g + du W_u)_{t,j} + dz_t W_r.

Pins (tests/test_train_oracle.py): central finite differences of J through
the pinned forward, torch.autograd on a dense float64 restatement of the
forward, closed forms (uniform routing, zero upstream gradient, padding-only
batches), and planted mistakes in the helpers below that those checks catch.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional

import numpy as np

from . import moe_oracle as O

widen = O.widen
sigmoid = O.sigmoid


# --------------------------------------------------------------------------
# masked routing and load statistics
# --------------------------------------------------------------------------

def route_masked(z: np.ndarray, k: int, mask: Optional[np.ndarray]) -> O.Routing:
    """Routing of the tokens with mask != 0; padding rows get expert -1,
    weight 0 and slot -1, and take no place in the expert order."""
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    valid = np.ones(T, dtype=bool) if mask is None else np.asarray(mask) != 0
    vt = np.nonzero(valid)[0]
    idx = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    slot_of = np.full((T, k), -1, dtype=np.int32)
    if vt.size:
        idx[vt] = O.select_topk(z[vt], k)
        w[vt] = O.renormalised_weights(z[vt], idx[vt])
    counts, offsets, st_local, so_local = O.expert_order(idx[vt], E)
    sorted_token = vt[st_local].astype(np.int32) if vt.size else np.zeros(0, np.int32)
    slot_of[vt] = so_local
    return O.Routing(z, idx, w, counts, offsets, sorted_token, slot_of)


def routed_tokens(routing: O.Routing) -> np.ndarray:
    return routing.topk_idx[:, 0] >= 0


def normalised_scores(z: np.ndarray) -> np.ndarray:
    """s'_{t,e} = sigma(z_te) / sum_e' sigma(z_te')."""
    s = sigmoid(np.asarray(z, dtype=np.float64))
    return s / s.sum(axis=1, keepdims=True)


def load_stats(routing: O.Routing, counts_global: Optional[np.ndarray] = None):
    """(f, p, N): routed-slot shares of the global counts, mean normalised
    scores over this batch's N routed tokens."""
    valid = routed_tokens(routing)
    N = int(valid.sum())
    c = np.asarray(routing.counts if counts_global is None else counts_global, dtype=np.float64)
    f = c / c.sum() if c.sum() > 0 else np.zeros_like(c)
    E = routing.logits.shape[1]
    p = normalised_scores(routing.logits[valid]).sum(axis=0) / N if N else np.zeros(E)
    return f, p, N


def aux_loss(routing: O.Routing, beta: float, counts_global: Optional[np.ndarray] = None) -> float:
    f, p, _ = load_stats(routing, counts_global)
    return float(beta * f.size * np.dot(f, p))


# --------------------------------------------------------------------------
# forward with the padding mask
# --------------------------------------------------------------------------

def forward(inputs, alpha: float, k: int, mask: Optional[np.ndarray] = None,
            logits32: Optional[np.ndarray] = None):
    """Layer output [T, D] in float64 under the padding mask, and the routing."""
    z = (O.router_logits(inputs.x, inputs.w_router, inputs.bias) if logits32 is None
         else np.asarray(logits32, dtype=np.float32).astype(np.float64))
    r = route_masked(z, k, mask)
    x = widen(inputs.x)
    T, D = x.shape
    out = O.shared_output(inputs, x)
    routed = np.zeros((T, D))
    for e in range(z.shape[1]):
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        if hi == lo:
            continue
        a, b = inputs.expert(e)
        toks = r.sorted_token[lo:hi]
        y = O.swiglu_expert(x[toks], widen(a), widen(b))
        slot = np.argmax(r.topk_idx[toks] == e, axis=1)
        routed[toks] += r.topk_w[toks, slot][:, None] * y
    return out + alpha * routed, r


# --------------------------------------------------------------------------
# backward helpers (each a separate function, so that tests can plant a
# mistake in one and watch the pins fail)
# --------------------------------------------------------------------------

def renorm_backward(w: np.ndarray, s: np.ndarray, g: np.ndarray) -> np.ndarray:
    """d/ds of w_j = s_j / sum s, given g = dJ/dw (rows = tokens)."""
    return (g - np.sum(w * g, axis=1, keepdims=True)) / s.sum(axis=1, keepdims=True)


def silu_grad(g: np.ndarray) -> np.ndarray:
    sg = sigmoid(g)
    return sg * (1.0 + g * (1.0 - sg))


def aux_dsigma(sig: np.ndarray, c: np.ndarray) -> np.ndarray:
    """dL_aux/dsigma for rows of sigmoid scores, with c_e = dL_aux/ds'_e."""
    q = sig.sum(axis=1, keepdims=True)
    sn = sig / q
    return (c[None, :] - np.sum(sn * c[None, :], axis=1, keepdims=True)) / q


def expert_backward_rows(a: np.ndarray, wgu: np.ndarray, wd: np.ndarray, dy: np.ndarray):
    """One SwiGLU expert over rows a [n, D] with output gradient dy [n, D].

    Returns (y, gu, h, dh, dgu, da, dWgu, dWd): y the forward output, gu = [g | u]
    the pre-activations, dgu = [dg | du]."""
    F = wgu.shape[0] // 2
    g = a @ wgu[:F].T
    u = a @ wgu[F:].T
    sg = sigmoid(g)
    h = g * sg * u
    y = h @ wd.T
    dh = dy @ wd
    dg = dh * u * silu_grad(g)
    du = dh * g * sg
    dgu = np.concatenate([dg, du], axis=1)
    da = dgu @ wgu
    return y, np.concatenate([g, u], axis=1), h, dh, dgu, da, dgu.T @ a, dy.T @ h


def dz_rows(z: np.ndarray, idx: np.ndarray, w: np.ndarray, gw: np.ndarray,
            c: Optional[np.ndarray]) -> np.ndarray:
    """Logit gradient rows of routed tokens: top-k weights (renorm, sigmoid)
    plus the auxiliary loss (c = beta E f / N per expert, or None)."""
    T, E = z.shape
    dz = np.zeros((T, E))
    sel = sigmoid(np.take_along_axis(z, idx.astype(np.int64), axis=1))
    ds = renorm_backward(w, sel, gw)
    np.put_along_axis(dz, idx.astype(np.int64), ds * sel * (1.0 - sel), axis=1)
    if c is not None:
        sig = sigmoid(z)
        dz += aux_dsigma(sig, c) * sig * (1.0 - sig)
    return dz


def aux_coefficients(routing: O.Routing, beta: float, counts_global=None) -> Optional[np.ndarray]:
    if beta == 0.0:
        return None
    f, _, N = load_stats(routing, counts_global)
    return beta * f.size * f / N if N else None


# --------------------------------------------------------------------------
# the full backward (small shapes) and sampled pieces (full-size shapes)
# --------------------------------------------------------------------------

@dataclass
class Grads:
    dx: np.ndarray          # [T, D]
    dz: np.ndarray          # [T, E] logit gradient (zero rows for padding)
    dw_router: np.ndarray   # [E, D]
    dbias: np.ndarray       # [E]
    dwgu: np.ndarray        # [E, 2F, D]
    dwd: np.ndarray         # [E, D, F]
    dwsgu: Optional[np.ndarray]   # [2Fs, D]
    dwsd: Optional[np.ndarray]    # [D, Fs]
    dy_perm: np.ndarray     # [S_routed, D] expert-order rows
    gu_perm: np.ndarray     # [S_routed, 2F] forward pre-activations
    dgu_perm: np.ndarray    # [S_routed, 2F]
    dx_perm: np.ndarray     # [S_routed, D]
    gu_shared: Optional[np.ndarray]
    dgu_shared: Optional[np.ndarray]
    dx_shared: np.ndarray   # [T, D]
    dx_router: np.ndarray   # [T, D]


def backward(inputs, alpha: float, routing: O.Routing, dout, beta: float = 0.0,
             counts_global: Optional[np.ndarray] = None) -> Grads:
    """All gradients of J = <dout, out> + L_aux, plus the intermediates the
    GPU path materialises, in float64 (every expert evaluated; small shapes)."""
    x = widen(inputs.x)
    T, D = x.shape
    z = routing.logits
    E = z.shape[1]
    k = routing.topk_idx.shape[1]
    dout = widen(dout) if np.asarray(dout).dtype == np.uint16 else np.asarray(dout, np.float64)
    valid = routed_tokens(routing)
    S = int(routing.offsets[E])
    wgu0, wd0 = (widen(a) for a in inputs.expert(0))
    F = wgu0.shape[0] // 2
    dwgu = np.zeros((E, 2 * F, D))
    dwd = np.zeros((E, D, F))
    y_perm = np.zeros((S, D))
    dy_perm = np.zeros((S, D))
    gu_perm = np.zeros((S, 2 * F))
    dgu_perm = np.zeros((S, 2 * F))
    dx_perm = np.zeros((S, D))
    # dy of slot p: alpha * w of that (token, slot) * dout of its token
    w_of_slot = np.zeros(S)
    for j in range(k):
        sl = routing.slot_of[valid, j]
        w_of_slot[sl] = routing.topk_w[valid, j]
    for e in range(E):
        lo, hi = int(routing.offsets[e]), int(routing.offsets[e + 1])
        if hi == lo:
            continue
        a, b = (widen(m) for m in inputs.expert(e))
        toks = routing.sorted_token[lo:hi]
        dy = alpha * w_of_slot[lo:hi, None] * dout[toks]
        y, gu, _, _, dgu, da, dwgu[e], dwd[e] = expert_backward_rows(x[toks], a, b, dy)
        y_perm[lo:hi], dy_perm[lo:hi], gu_perm[lo:hi] = y, dy, gu
        dgu_perm[lo:hi], dx_perm[lo:hi] = dgu, da
    # routing-weight gradient, then the logit gradient of the routed tokens
    gw = np.zeros((T, k))
    for j in range(k):
        gw[valid, j] = alpha * np.sum(dout[valid] * y_perm[routing.slot_of[valid, j]], axis=1)
    c = aux_coefficients(routing, beta, counts_global)
    dz = np.zeros((T, E))
    if valid.any():
        dz[valid] = dz_rows(z[valid], routing.topk_idx[valid], routing.topk_w[valid], gw[valid], c)
    # shared expert over every row
    sh = inputs.shared()
    dx_shared = np.zeros((T, D))
    dwsgu = dwsd = gu_sh = dgu_sh = None
    if sh is not None:
        _, gu_sh, _, _, dgu_sh, dx_shared, dwsgu, dwsd = expert_backward_rows(
            x, widen(sh[0]), widen(sh[1]), dout)
    wr = widen(inputs.w_router)
    dx_router = dz @ wr
    dx = dx_shared + dx_router
    for j in range(k):
        dx[valid] += dx_perm[routing.slot_of[valid, j]]
    return Grads(dx, dz, dz.T @ x, dz.sum(axis=0), dwgu, dwd, dwsgu, dwsd, dy_perm, gu_perm,
                 dgu_perm, dx_perm, gu_sh, dgu_sh, dx_shared, dx_router)


def token_grads(inputs, alpha: float, routing: O.Routing, dout, tokens: Iterable[int],
                beta: float = 0.0, counts_global: Optional[np.ndarray] = None):
    """(dz rows, dx rows) of the given tokens only, float64.  Each expert the
    tokens use is widened once; the aux coefficients come from the whole
    routing."""
    tokens = np.asarray(list(tokens), dtype=np.int64)
    x = widen(np.asarray(inputs.x)[tokens])
    dout = np.asarray(dout)
    dt = widen(dout[tokens]) if dout.dtype == np.uint16 else dout[tokens].astype(np.float64)
    n, D = x.shape
    k = routing.topk_idx.shape[1]
    idx = routing.topk_idx[tokens]
    w = routing.topk_w[tokens]
    valid = idx[:, 0] >= 0
    gw = np.zeros((n, k))
    dx = np.zeros((n, D))
    for e in np.unique(idx[valid]):
        rows, slots = np.nonzero(idx == e)
        a, b = (widen(m) for m in inputs.expert(int(e)))
        dy = alpha * w[rows, slots][:, None] * dt[rows]
        y, _, _, _, _, da, _, _ = expert_backward_rows(x[rows], a, b, dy)
        gw[rows, slots] = alpha * np.sum(dt[rows] * y, axis=1)
        dx[rows] += da
    c = aux_coefficients(routing, beta, counts_global)
    E = routing.logits.shape[1]
    dz = np.zeros((n, E))
    if valid.any():
        dz[valid] = dz_rows(routing.logits[tokens[valid]], idx[valid], w[valid], gw[valid], c)
    sh = inputs.shared()
    if sh is not None:
        dx += expert_backward_rows(x, widen(sh[0]), widen(sh[1]), dt)[5]
    dx += dz @ widen(inputs.w_router)
    return dz, dx


def expert_grads(inputs, alpha: float, routing: O.Routing, dout, e: int):
    """(dW_gu [2F, D], dW_d [D, F], dgu rows, dy rows) of routed expert e."""
    lo, hi = int(routing.offsets[e]), int(routing.offsets[e + 1])
    toks = routing.sorted_token[lo:hi]
    k = routing.topk_idx.shape[1]
    slot = np.argmax(routing.topk_idx[toks] == e, axis=1) if k else None
    w = routing.topk_w[toks, slot]
    dout = np.asarray(dout)
    dt = widen(dout[toks]) if dout.dtype == np.uint16 else dout[toks].astype(np.float64)
    a, b = (widen(m) for m in inputs.expert(e))
    dy = alpha * w[:, None] * dt
    _, _, _, _, dgu, _, dwgu, dwd = expert_backward_rows(widen(np.asarray(inputs.x)[toks]), a, b, dy)
    return dwgu, dwd, dgu, dy
