"""Pins of the training-pass oracle (padding mask, load statistics, auxiliary
loss, backward), CPU only.

What fixes the oracle here, beside its own definition:
  * the forward it differentiates is the pinned forward oracle: with no padding
    it is that oracle, and with padding every routed token's output equals the
    forward oracle run on the routed tokens alone;
  * central finite differences of J = <dout, out> + L_aux through that
    forward, on float64 inputs, in random directions of every parameter;
  * torch.autograd on a dense float64 restatement of the forward (routing held
    fixed), for every gradient at once;
  * closed forms: equal logits give L_aux = beta whatever the routing; uniform
    counts give no auxiliary gradient; a batch of padding only routes nothing;
  * planted mistakes in the renormalisation backward, the silu derivative and
    the auxiliary-loss score gradient, each of which the checks must catch.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import train_oracle as TR


class F64Inputs:
    """Float64 layer inputs (the oracle widens them as they are)."""

    def __init__(self, T=10, D=24, E=8, k=3, F=16, Fs=16, seed=0, bias=True, scale=1.0):
        g = np.random.default_rng(seed)
        self.x = g.normal(0, 1, (T, D))
        self.w_router = g.normal(0, 0.3 * scale, (E, D))
        self.bias = g.normal(0, 0.2, E) if bias else None
        self.wgu = g.normal(0, 0.2, (E, 2 * F, D))
        self.wd = g.normal(0, 0.2, (E, D, F))
        self.sh = (g.normal(0, 0.2, (2 * Fs, D)), g.normal(0, 0.2, (D, Fs))) if Fs else None
        self.k = k

    def expert(self, e):
        return self.wgu[e], self.wd[e]

    def shared(self):
        return self.sh


def _routing(inp, mask=None):
    return TR.route_masked(O.router_logits(inp.x, inp.w_router, inp.bias), inp.k, mask)


def _objective(inp, alpha, dout, beta, mask, counts_global, want_idx=None):
    out, r = TR.forward(inp, alpha, inp.k, mask)
    if want_idx is not None:
        assert np.array_equal(r.topk_idx, want_idx), "a finite-difference step changed the routing"
    return float(np.sum(dout * out)) + TR.aux_loss(r, beta, counts_global)


# ------------------------------------------------------------------ forward with the mask

def test_no_padding_is_the_forward_oracle():
    inp = F64Inputs(seed=1)
    out, r = TR.forward(inp, 2.5, inp.k, None)
    ref, r0 = O.forward(inp, 2.5, inp.k)
    assert np.allclose(out, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(r.topk_idx, r0.topk_idx) and np.array_equal(r.sorted_token, r0.sorted_token)


def test_padding_tokens_take_the_shared_expert_only():
    inp = F64Inputs(seed=2, T=14)
    mask = np.ones(14, np.uint8)
    mask[[0, 5, 6, 13]] = 0
    out, r = TR.forward(inp, 2.5, inp.k, mask)
    sh = O.shared_output(inp, inp.x)
    pad = mask == 0
    assert np.allclose(out[pad], sh[pad], rtol=0, atol=1e-13)
    assert np.all(r.topk_idx[pad] == -1) and np.all(r.slot_of[pad] == -1) and np.all(r.topk_w[pad] == 0)
    assert r.counts.sum() == inp.k * (~pad).sum() and r.offsets[-1] == r.counts.sum()
    assert set(r.sorted_token.tolist()) == set(np.nonzero(~pad)[0].tolist())
    # the routed tokens alone, through the forward oracle
    sub = F64Inputs(seed=2, T=14)
    sub.x = inp.x[~pad]
    ref, _ = O.forward(sub, 2.5, inp.k)
    assert np.allclose(out[~pad], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # slot_of / sorted_token stay inverse on the routed tokens
    vt = np.nonzero(~pad)[0]
    assert np.all(r.sorted_token[r.slot_of[vt]] == vt[:, None])


def test_all_padding_routes_nothing():
    inp = F64Inputs(seed=3, T=6)
    r = _routing(inp, np.zeros(6, np.uint8))
    assert r.counts.sum() == 0 and r.sorted_token.size == 0
    f, p, N = TR.load_stats(r)
    assert N == 0 and np.all(p == 0)
    g = TR.backward(inp, 2.5, r, np.ones((6, inp.x.shape[1])), beta=0.5)
    assert np.all(g.dz == 0) and np.all(g.dwgu == 0) and np.all(g.dwd == 0)
    assert np.allclose(g.dx, g.dx_shared)


# ------------------------------------------------------------------ load statistics and aux loss

def test_load_stats_sum_to_one_and_equal_logits_give_beta():
    inp = F64Inputs(seed=4, T=40, E=16, k=4)
    r = _routing(inp)
    f, p, N = TR.load_stats(r)
    assert N == 40 and abs(f.sum() - 1) < 1e-15 and abs(p.sum() - 1) < 1e-12
    assert np.allclose(f, r.counts / (4 * 40))
    # equal logits: p = 1/E for every expert, so L = beta E sum f / E = beta
    inp.w_router[:] = 0
    inp.bias = None
    r = _routing(inp)
    assert np.all(r.topk_idx == np.arange(4))                  # ties to the lower index
    assert abs(TR.aux_loss(r, 0.37) - 0.37) < 1e-15


def test_uniform_counts_give_no_aux_gradient():
    inp = F64Inputs(seed=5, T=16, E=8, k=2)
    r = _routing(inp)
    dout = np.zeros_like(inp.x)
    g = TR.backward(inp, 2.5, r, dout, beta=1.0, counts_global=np.full(8, 7))
    assert np.max(np.abs(g.dz)) < 1e-15
    g = TR.backward(inp, 2.5, r, dout, beta=1.0)               # this batch's counts: not uniform
    assert np.max(np.abs(g.dz)) > 1e-6


def test_global_counts_enter_only_through_their_shares():
    inp = F64Inputs(seed=6, T=16, E=8, k=2)
    r = _routing(inp)
    dout = np.random.default_rng(0).normal(size=inp.x.shape)
    a = TR.backward(inp, 2.5, r, dout, beta=0.3)
    b = TR.backward(inp, 2.5, r, dout, beta=0.3, counts_global=3 * r.counts)
    assert np.allclose(a.dz, b.dz, rtol=0, atol=1e-15) and np.allclose(a.dx, b.dx, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ finite differences

@pytest.mark.parametrize("case", ["plain", "padding_aux_global"])
def test_finite_differences_of_every_parameter(case):
    inp = F64Inputs(seed=7, T=9, D=16, E=6, k=2, F=8, Fs=8)
    T, D = inp.x.shape
    g0 = np.random.default_rng(11)
    dout = g0.normal(size=(T, D))
    mask = None
    beta, counts_global = 0.0, None
    if case != "plain":
        mask = np.ones(T, np.uint8)
        mask[[2, 7]] = 0
        beta, counts_global = 0.8, np.array([5, 1, 9, 0, 3, 4])
    r = _routing(inp, mask)
    g = TR.backward(inp, 2.5, r, dout, beta, counts_global)
    # routing must not change under the steps: keep a margin between the k-th
    # and (k+1)-th logits of every routed token
    zs = np.sort(r.logits, axis=1)[:, ::-1]
    assert np.min(zs[:, inp.k - 1] - zs[:, inp.k]) > 1e-4
    params = {
        "x": (inp.x, g.dx), "w_router": (inp.w_router, g.dw_router), "bias": (inp.bias, g.dbias),
        "wgu": (inp.wgu, g.dwgu), "wd": (inp.wd, g.dwd),
        "ws_gu": (inp.sh[0], g.dwsgu), "ws_d": (inp.sh[1], g.dwsd),
    }
    eps = 1e-6
    for name, (arr, grad) in params.items():
        for trial in range(3):
            v = g0.normal(size=arr.shape)
            base = arr.copy()
            arr[...] = base + eps * v
            jp = _objective(inp, 2.5, dout, beta, mask, counts_global, r.topk_idx)
            arr[...] = base - eps * v
            jm = _objective(inp, 2.5, dout, beta, mask, counts_global, r.topk_idx)
            arr[...] = base
            fd = (jp - jm) / (2 * eps)
            an = float(np.sum(grad * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ------------------------------------------------------------------ torch.autograd

def _autograd(inp, alpha, r, dout, beta, counts_global):
    """Dense float64 restatement of J with the routing r held fixed."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x, wr, b = t(inp.x), t(inp.w_router), t(inp.bias)
    wgu, wd = t(inp.wgu), t(inp.wd)
    sgu, sd = t(inp.sh[0]), t(inp.sh[1])
    F, Fs = inp.wgu.shape[1] // 2, inp.sh[0].shape[0] // 2
    z = x @ wr.T + b
    sig = torch.sigmoid(z)
    idx = torch.tensor(np.maximum(r.topk_idx, 0), dtype=torch.int64)
    valid = torch.tensor(r.topk_idx[:, 0] >= 0)
    sel = torch.gather(sig, 1, idx)
    w = sel / sel.sum(1, keepdim=True)
    hs = torch.nn.functional.silu(x @ sgu[:Fs].T) * (x @ sgu[Fs:].T)
    out = hs @ sd.T
    routed = torch.zeros_like(out)
    for j in range(idx.shape[1]):
        e = idx[:, j]
        g = torch.einsum("td,tfd->tf", x, wgu[e, :F])
        u = torch.einsum("td,tfd->tf", x, wgu[e, F:])
        y = torch.einsum("tf,tdf->td", torch.nn.functional.silu(g) * u, wd[e])
        routed = routed + torch.where(valid[:, None], w[:, j:j + 1] * y, torch.zeros_like(y))
    out = out + alpha * routed
    J = (torch.tensor(dout) * out).sum()
    if beta:
        f, _, N = TR.load_stats(r, counts_global)
        sn = sig / sig.sum(1, keepdim=True)
        p = torch.where(valid[:, None], sn, torch.zeros_like(sn)).sum(0) / N
        J = J + beta * len(f) * (torch.tensor(f) * p).sum()
    J.backward()
    return {n: a.grad.numpy() for n, a in
            dict(dx=x, dw_router=wr, dbias=b, dwgu=wgu, dwd=wd, dwsgu=sgu, dwsd=sd).items()}


def _compare_with_autograd(seed=8, beta=0.6, padded=True):
    inp = F64Inputs(seed=seed, T=12, D=16, E=8, k=3, F=8, Fs=8)
    mask = np.ones(12, np.uint8)
    if padded:
        mask[[3, 11]] = 0
    r = _routing(inp, mask)
    dout = np.random.default_rng(seed).normal(size=inp.x.shape)
    counts_global = r.counts + np.arange(8)
    g = TR.backward(inp, 2.5, r, dout, beta, counts_global)
    ref = _autograd(inp, 2.5, r, dout, beta, counts_global)
    worst = 0.0
    for name, a in ref.items():
        b = getattr(g, name)
        worst = max(worst, np.abs(a - b).max() / max(np.abs(a).max(), 1e-30))
    return worst


def test_matches_torch_autograd():
    assert _compare_with_autograd() < 1e-12
    assert _compare_with_autograd(seed=9, beta=0.0, padded=False) < 1e-12


@pytest.mark.parametrize("plant", ["renorm_drops_mean", "silu_grad_is_sigmoid", "aux_not_centred"])
def test_planted_mistakes_are_caught(monkeypatch, plant):
    if plant == "renorm_drops_mean":
        monkeypatch.setattr(TR, "renorm_backward", lambda w, s, g: g / s.sum(axis=1, keepdims=True))
    elif plant == "silu_grad_is_sigmoid":
        monkeypatch.setattr(TR, "silu_grad", lambda g: TR.sigmoid(g))
    else:
        monkeypatch.setattr(TR, "aux_dsigma", lambda sig, c: c[None, :] / sig.sum(axis=1, keepdims=True))
    assert _compare_with_autograd() > 1e-6


# ------------------------------------------------------------------ sampled pieces

def test_sampled_pieces_equal_the_full_backward():
    inp = F64Inputs(seed=10, T=20, D=16, E=8, k=3, F=8, Fs=8)
    mask = np.ones(20, np.uint8)
    mask[[1, 19]] = 0
    r = _routing(inp, mask)
    dout = np.random.default_rng(1).normal(size=inp.x.shape)
    g = TR.backward(inp, 2.5, r, dout, 0.4)
    toks = [0, 1, 7, 19]
    dz, dx = TR.token_grads(inp, 2.5, r, dout, toks, 0.4)
    assert np.allclose(dz, g.dz[toks], rtol=0, atol=1e-13) and np.allclose(dx, g.dx[toks], rtol=0, atol=1e-12)
    for e in range(8):
        if r.counts[e] == 0:
            continue
        dwgu, dwd, dgu, dy = TR.expert_grads(inp, 2.5, r, dout, e)
        lo, hi = r.offsets[e], r.offsets[e + 1]
        assert np.allclose(dwgu, g.dwgu[e], rtol=0, atol=1e-12) and np.allclose(dwd, g.dwd[e], rtol=0, atol=1e-12)
        assert np.allclose(dgu, g.dgu_perm[lo:hi], rtol=0, atol=1e-12)
        assert np.allclose(dy, g.dy_perm[lo:hi], rtol=0, atol=1e-13)
