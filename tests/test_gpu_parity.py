"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Routing and the expert order must be bit-exact (oracle decided on the GPU's
fp32 logits); outputs within 2e-2 * max|oracle| for bf16 and 1e-5 * max|oracle|
for fp32.  Small shapes compare every output element; the full-size workloads
compare sampled tokens (the oracle evaluates them one by one) plus sampled rows
of the intermediate h and y_perm.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from mixture_experts_transformer_moe_amd import binding, configs
from mixture_experts_transformer_moe_amd.inputs import LayerInputs
from tests.gpu_common import (StackedInputs, assert_close_rel, check_routing, out_tolerance,
                              run_layer, say, to_f64)

pytestmark = pytest.mark.gpu

SMALL_BF16 = configs.variant(configs.XS2_T4096, name="small_bf16_t300", T=300, D=256, E=16, k=4,
                             F=256, Fs=256)


def full_parity(s, inp=None, gather=False):
    inp = inp or StackedInputs(LayerInputs(s))
    x, w, b = run_layer(s, inp, gather=gather)
    r = check_routing(s, inp, b)
    ref, _ = O.forward(inp, s.alpha, s.k, logits32=b.logits.cpu().numpy())
    rel = assert_close_rel(to_f64(b.out), ref, out_tolerance(s), "out")
    say(f"{s.name}: out max rel err {rel:.2e}")
    return inp, b, r


def token_rel_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per token: max |gpu - oracle| over its row / max |oracle| over its row."""
    return np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


def sampled_parity(s, n_tokens=40, seed=0, all_outliers=False, expert_rows=3):
    # the benchmark's launch configuration: the first GEMM gathers token rows
    inp = StackedInputs(LayerInputs(s))
    x, w, b = run_layer(s, inp, gather=True)
    r = check_routing(s, inp, b)
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(s.T, size=min(n_tokens, s.T), replace=False).tolist()) | {0, s.T - 1}
    busiest = int(np.argmax(r.counts))
    toks |= set(r.sorted_token[r.offsets[busiest]:r.offsets[busiest] + 4].tolist())
    outl = np.zeros(0, np.int64)
    if s.outlier_frac > 0:
        from mixture_experts_transformer_moe_amd.inputs import outlier_tokens
        outl = np.asarray(outlier_tokens(s), np.int64)
        toks |= set((outl if all_outliers else outl[:6]).tolist())
    toks = np.array(sorted(toks), np.int64)
    say(f"oracle on {len(toks)} sampled tokens")
    ref = O.forward_tokens(inp, s.alpha, r, toks)
    got = to_f64(b.out[torch.from_numpy(toks).cuda()])
    rel = assert_close_rel(got, ref, out_tolerance(s), "sampled out")
    say(f"{s.name}: sampled out max rel err {rel:.2e} (of the sample's largest output)")
    # the outlier rows (x50 activations) dominate max|oracle|: the bar is also
    # applied to the ordinary tokens on their own, and each group's worst
    # per-token error is reported
    is_out = np.isin(toks, outl)
    for name, sel in (("ordinary", ~is_out), ("outlier", is_out)):
        if sel.any():
            g_rel = assert_close_rel(got[sel], ref[sel], out_tolerance(s), f"{name} tokens' out")
            per_tok = token_rel_errors(got[sel], ref[sel])
            say(f"{s.name}: {int(sel.sum())} {name} tokens: max rel err {g_rel:.2e} of their largest "
                f"output; worst per-token error {per_tok.max():.2e} of that token's largest output "
                f"(median {np.median(per_tok):.2e})")
    # intermediate rows of a few experts: busiest, smallest non-empty, random ones
    nz = np.nonzero(r.counts)[0]
    experts = {busiest, int(nz[np.argmin(r.counts[nz])])}
    experts |= set(rng.choice(nz, size=min(expert_rows, len(nz)), replace=False).tolist())
    h = b.h[: s.S * s.F].view(s.S, s.F)
    for e in sorted(experts):
        n = int(r.counts[e])
        rows = np.unique(np.array([0, n - 1, n // 2] + rng.integers(0, n, 8).tolist()))
        h_ref, y_ref = O.expert_rows(inp, r, e, rows)
        pos = int(r.offsets[e]) + rows
        assert_close_rel(to_f64(h[pos]), h_ref, out_tolerance(s), f"h of expert {e}")
        assert_close_rel(to_f64(b.y_perm[pos]), y_ref, out_tolerance(s), f"y_perm of expert {e}")
    return inp, b, r


# ------------------------------------------------------------------ workloads

def test_tiny_f32_full_parity():
    full_parity(configs.TINY_F32)


def test_small_bf16_full_parity_ragged():
    full_parity(SMALL_BF16)


# Shapes with several hundred rows per expert take the LDS-tiled grouped GEMMs
# (256 x 256 tiles, ragged last row tiles of each expert, shared expert first)
LDS_TILED = [
    configs.variant(SMALL_BF16, name="lds_tiled_t1600_e4_k2", T=1600, D=512, E=4, k=2, F=256, Fs=256,
                    seed=31),
    configs.variant(SMALL_BF16, name="lds_tiled_t2000_e8_k4_noshared", T=2000, D=256, E=8, k=4, F=512,
                    Fs=0, seed=32),
    configs.variant(SMALL_BF16, name="lds_tiled_t1700_e2_k1", T=1700, D=768, E=2, k=1, F=256, Fs=512,
                    seed=33),
]


@pytest.mark.parametrize("s", LDS_TILED, ids=lambda s: s.name)
@pytest.mark.parametrize("gather", [False, True])
def test_lds_tiled_gemm_full_parity(s, gather):
    inp, b, r = full_parity(s, gather=gather)
    # every h and y_perm row of every expert, against the oracle's expert rows
    h = b.h[: s.S * s.F].view(s.S, s.F)
    for e in range(s.E):
        h_ref, y_ref = O.expert_rows(inp, r, e)
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        assert_close_rel(to_f64(h[lo:hi]), h_ref, out_tolerance(s), f"h of expert {e}")
        assert_close_rel(to_f64(b.y_perm[lo:hi]), y_ref, out_tolerance(s), f"y_perm of expert {e}")


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_small_bf16_full_parity_other_seeds(seed):
    # other inputs and weights of the same ragged shape
    full_parity(configs.variant(SMALL_BF16, name=f"small_bf16_seed{seed}", seed=seed))


def test_small_bf16_gather_mode_matches_x_perm_mode():
    s = SMALL_BF16
    inp = StackedInputs(LayerInputs(s))
    _, _, b1 = run_layer(s, inp, gather=False)
    _, _, b2 = run_layer(s, inp, gather=True)
    assert torch.equal(b1.out, b2.out)
    assert torch.equal(b1.h, b2.h)


def test_xs2_workload_full_parity():
    """XS.2 shape at full size, in the benchmark's launch configuration: every
    output element, and every expert's h and y_perm rows, against the oracle."""
    s = configs.XS2_T4096
    inp, b, r = full_parity(s, gather=True)
    h = b.h[: s.S * s.F].view(s.S, s.F)
    worst = 0.0
    for e in range(s.E):
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        if hi == lo:
            continue
        h_ref, y_ref = O.expert_rows(inp, r, e)
        assert_close_rel(to_f64(h[lo:hi]), h_ref, out_tolerance(s), f"h of expert {e}")
        worst = max(worst, assert_close_rel(to_f64(b.y_perm[lo:hi]), y_ref, out_tolerance(s),
                                            f"y_perm of expert {e}"))
    say(f"xs2: every expert's rows within tolerance (worst y_perm rel err {worst:.2e})")


def test_prefill_outlier_workload_parity():
    """Long prefill (32768 tokens, 10% of them with x50 outlier channels): all
    3277 outlier tokens and 256 random ones, the bar applied to each group on
    its own."""
    sampled_parity(configs.PREFILL_OUTLIER_T32768, n_tokens=256, all_outliers=True, expert_rows=6)


def test_lds_tiled_many_rounds_sampled_parity():
    """A down launch whose workgroups each run more than 64 tiles (the down
    kernel locates its tiles 64 rounds at a time): 32768 tokens to all 8
    experts, D = 4096 (16 column tiles per 256-row block), F = 256 (the
    shortest K the LDS-tiled kernel takes: 8 stages): 1152 row blocks x 16 =
    18432 tiles, 72 per workgroup on 256 CUs."""
    s = configs.variant(SMALL_BF16, name="lds_rounds_t32768_e8_d4096", T=32768, D=4096, E=8, k=8, F=256,
                        Fs=256, seed=43)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = (cus + 7) // 8 * 8
    row_blocks = s.E * ((s.T * s.k // s.E + 255) // 256) + (s.T + 255) // 256
    assert row_blocks * (s.D // 256) > 64 * grid
    sampled_parity(s, n_tokens=64, expert_rows=2)


@pytest.mark.parametrize("name", [configs.M1_T8192.name, configs.M1_TOP16_T8192.name])
def test_m1_width_workload_sampled_parity(name):
    sampled_parity(configs.get(name), n_tokens=256, expert_rows=4)


def test_decode_workload_full_parity():
    # T = 32: the oracle evaluates the whole layer
    inp, b, r = full_parity(configs.DECODE_SKEW_T32)
    say(f"decode: experts touched {int(np.count_nonzero(r.counts))}, max rows {int(r.counts.max())}")


@pytest.mark.parametrize("shape", ["small_ragged", "lds_tiled"])
def test_nan_in_one_token_stays_in_that_token(shape):
    """A NaN in one input row is outside the contract for that token, but it
    must not fault and must not reach any other token: every other token's
    routing and output are bit-identical to the run without it, and the
    permutation still places every token exactly k times."""
    s = SMALL_BF16 if shape == "small_ragged" else LDS_TILED[0]
    inp = StackedInputs(LayerInputs(s))
    x, w = (None, None)
    from tests.gpu_common import upload_stacked
    x, w = upload_stacked(inp)
    clean = binding.alloc_buffers(s, with_x_perm=False)
    binding.layer_forward(s, x, w, clean)
    bad_tok = s.T // 3
    x_nan = x.clone()
    x_nan[bad_tok] = float("nan")
    b = binding.alloc_buffers(s, with_x_perm=False)
    binding.layer_forward(s, x_nan, w, b)
    torch.cuda.synchronize()
    say(f"{s.name}: NaN in token {bad_tok}")
    keep = torch.ones(s.T, dtype=torch.bool, device="cuda")
    keep[bad_tok] = False
    assert torch.equal(b.topk_idx[keep], clean.topk_idx[keep]), "another token's experts changed"
    assert torch.equal(b.topk_w[keep], clean.topk_w[keep]), "another token's weights changed"
    assert torch.equal(b.out[keep].view(torch.int16), clean.out[keep].view(torch.int16)), \
        "another token's output changed"
    assert torch.isfinite(b.out[keep].float()).all()
    # the NaN token still gets k distinct in-range experts, and the expert order
    # is a valid permutation of every (token, slot)
    idx = b.topk_idx.cpu().numpy()
    O.check_invariants(idx, None, b.counts.cpu().numpy(), b.offsets.cpu().numpy(),
                       b.sorted_token.cpu().numpy(), b.slot_of.cpu().numpy(), s.E)


def test_router_large_batch_with_padding_mask():
    """The router's largest block shape (all 256 experts of 128 tokens per
    workgroup) with a padding mask and a ragged last block (32700 tokens):
    logits within 1e-5 max|z| of fp64, every token's experts bit-exact against
    the oracle's selection on the GPU's fp32 logits, weights within 1e-6,
    padding tokens expert -1 and weight 0."""
    from oracle import train_oracle as TR
    from mixture_experts_transformer_moe_amd.inputs import token_mask
    s = configs.variant(SMALL_BF16, name="router_mask_t32700", T=32700, D=256, E=256, k=8, F=256, Fs=256,
                        pad_frac=0.1, seq_len=700, seed=41)
    assert s.E == 256 and (s.T + 127) // 128 >= 256 and s.T % 128 != 0
    inp = LayerInputs(s)
    x, w = binding.upload(inp)
    mask = token_mask(s)
    n_pad = int((mask == 0).sum())
    assert 0 < n_pad < s.T
    b = binding.alloc_buffers(s, with_x_perm=False)
    c = binding.make_shape(s)
    binding.moe_route_masked(c, x, w.w_router, w.bias, torch.from_numpy(mask).cuda(), b.logits, b.topk_idx,
                             b.topk_w)
    torch.cuda.synchronize()
    logits = b.logits.cpu().numpy()
    z64 = O.router_logits(inp.x, inp.w_router, inp.bias)
    err = np.abs(logits.astype(np.float64) - z64).max()
    assert err <= 1e-5 * np.abs(z64).max(), f"logit error {err}"
    r = TR.route_masked(logits.astype(np.float64), s.k, mask)
    assert np.array_equal(b.topk_idx.cpu().numpy(), r.topk_idx), "topk_idx differs"
    np.testing.assert_allclose(b.topk_w.cpu().numpy(), r.topk_w, rtol=1e-6, atol=0)
    say(f"{s.name}: {n_pad} padding tokens, routing bit-exact")


# ------------------------------------------------------------------ edge cases

EDGE = {
    "k1": dict(k=1),
    "k_eq_E": dict(E=16, k=16),
    "k16_alpha1_E64": dict(E=64, k=16, alpha=1.0),
    "E1_k1": dict(E=1, k=1),
    "no_shared": dict(Fs=0),
    "T1": dict(T=1),
    "T256_one_block": dict(T=256),           # the permutation's single-block path, full
    "T257_two_blocks": dict(T=257),          # two blocks, the second with one token
    "T33_wide_shared": dict(T=33, Fs=512),
    "E256_T70": dict(T=70, E=256, k=8),
    # tile shapes chosen by the mean rows per expert (k T / E)
    "rows37_T300_E32": dict(T=300, E=32, k=4),
    "rows150_T600_E32": dict(T=600, E=32, k=8),
    "rows256_T512_D512": dict(T=512, D=512, E=16, k=8),
    "rows350_T700_D512": dict(T=700, D=512, E=16, k=8, Fs=512),
    # router block shapes at block counts that do not split evenly over the 8
    # XCDs, with ragged token (and expert) tails: 64 x 64 blocks, 132 of them
    "router64_T2050_E256": dict(T=2050, E=256, k=8),
    # 32 x 32 blocks, 132 of them, 72 experts
    "router32_T1400_E72": dict(T=1400, E=72, k=8),
    # 128 x 64 blocks (8 waves), 260 of them, a ragged token tail
    "router128_T8200_E256": dict(T=8200, E=256, k=2),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_shapes_bf16(case):
    s = configs.variant(SMALL_BF16, name=f"edge_{case}", **EDGE[case])
    full_parity(s)


@pytest.mark.parametrize("case", ["rows150_T600_E32", "rows256_T512_D512", "rows350_T700_D512", "T1",
                                  "E256_T70"])
def test_edge_shapes_bf16_gathered(case):
    s = configs.variant(SMALL_BF16, name=f"edge_gather_{case}", **EDGE[case])
    full_parity(s, gather=True)


@pytest.mark.parametrize("case", ["k1", "no_shared", "T1", "k_eq_E"])
def test_edge_shapes_f32(case):
    s = configs.variant(configs.TINY_F32, name=f"edge_f32_{case}", **EDGE[case])
    full_parity(s)


def test_zero_router_ties_go_to_lowest_indices():
    s = configs.variant(SMALL_BF16, name="zero_router", T=100)
    inp = StackedInputs(LayerInputs(s))
    inp.w_router = np.zeros_like(inp.w_router)
    _, b, r = full_parity(s, inp)
    assert (b.topk_idx.cpu().numpy() == np.arange(s.k)).all()
    np.testing.assert_allclose(b.topk_w.cpu().numpy(), 1.0 / s.k, rtol=1e-6)


def test_one_expert_takes_every_token():
    s = configs.variant(SMALL_BF16, name="hot_expert", T=520)
    bias = np.zeros(s.E, np.float32)
    bias[3] = 30.0
    inp = StackedInputs(LayerInputs(s, bias=bias))
    _, b, r = full_parity(s, inp)
    assert int(b.counts[3]) == s.T


def _guarded_like(t: torch.Tensor, pad: int = 4096):
    """A buffer with t's shape followed by a guard region of known bytes."""
    big = torch.empty(t.numel() + pad, dtype=t.dtype, device=t.device)
    ints = big.view(torch.int16 if t.element_size() == 2 else torch.int32)
    ints[t.numel():] = 0x5a5a if t.element_size() == 2 else 0x5a5a5a5a
    return big, big[: t.numel()].view(t.shape)


def _guard_intact(big: torch.Tensor, n: int) -> bool:
    ints = big.view(torch.int16 if big.element_size() == 2 else torch.int32)[n:]
    return bool((ints == (0x5a5a if big.element_size() == 2 else 0x5a5a5a5a)).all())


@pytest.mark.parametrize("fp8", [False, True])
def test_determinism_and_no_out_of_bounds_writes(fp8):
    s = SMALL_BF16
    inp = StackedInputs(LayerInputs(s))
    from tests.gpu_common import upload_stacked
    x, w = upload_stacked(inp, fp8=fp8)
    outs = []
    for rep in range(3):
        say(f"determinism rep {rep}")
        b = binding.alloc_buffers(s)
        guards = {}
        for name in ("logits", "topk_idx", "topk_w", "counts", "offsets", "sorted_token",
                     "slot_of", "x_perm", "h", "y_perm", "y_shared", "out"):
            t = getattr(b, name)
            big, view = _guarded_like(t)
            guards[name] = (big, t.numel())
            setattr(b, name, view)
        binding.layer_forward(s, x, w, b)
        torch.cuda.synchronize()
        for name, (big, n) in guards.items():
            assert _guard_intact(big, n), f"write past the end of {name}"
        outs.append((b.out.clone(), b.sorted_token.clone(), b.h.clone(), b.logits.clone()))
    for o in outs[1:]:
        assert all(torch.equal(p, q) for p, q in zip(o, outs[0]))


@pytest.mark.parametrize("name", ["small_ragged", "xs2"])
def test_shared_expert_on_its_own_stream_matches_the_fused_path(name):
    """moe_shared_ffn on a second stream beside the router, the permutation and
    the routed-only grouped GEMMs gives the fused path's results bit for bit."""
    s = SMALL_BF16 if name == "small_ragged" else configs.XS2_T4096
    say(f"shared expert split {s.name}")
    inp = StackedInputs(LayerInputs(s))
    from tests.gpu_common import upload_stacked
    x, w = upload_stacked(inp)
    fused = binding.alloc_buffers(s)
    binding.layer_forward(s, x, w, fused)
    torch.cuda.synchronize()
    b = binding.alloc_buffers(s)
    c = binding.make_shape(s)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    binding.moe_shared_ffn(c, x, w.ws_gate_up, w.ws_down, b.h[s.T * s.k * s.F:], b.y_shared, side)
    done = torch.cuda.Event()
    done.record(side)
    binding.moe_route(c, x, w.w_router, w.bias, b.logits, b.topk_idx, b.topk_w, main)
    binding.moe_permute(c, b.topk_idx, x, b.counts, b.offsets, b.sorted_token, b.slot_of, b.x_perm,
                        b.workspace, main)
    binding.moe_grouped_gate_up(c, b.x_perm, b.sorted_token, x, b.offsets, w.w_gate_up, None, b.h,
                                main)
    binding.moe_grouped_down(c, b.h, b.offsets, w.w_down, None, b.y_perm, None, main)
    main.wait_event(done)
    binding.moe_combine(c, b.y_perm, b.y_shared, b.slot_of, b.topk_w, b.out, main)
    torch.cuda.synchronize()
    n = s.T * s.k
    assert torch.equal(b.out, fused.out)
    assert torch.equal(b.y_shared, fused.y_shared)
    assert torch.equal(b.h, fused.h)
    assert torch.equal(b.y_perm[:n], fused.y_perm[:n])


@pytest.mark.parametrize("shape", ["small_ragged", "lds_tiled"])
def test_grouped_ffn_entry_point_takes_packed_weights(shape):
    """moe_grouped_ffn, the boundary's single grouped-FFN call, with weights
    packed by moe_pack_weights (its documented precondition) and token rows
    gathered through sorted_token (no x_perm): the same bits as the two GEMM
    calls of the layer pass, whose output the oracle checks."""
    s = SMALL_BF16 if shape == "small_ragged" else LDS_TILED[0]
    inp = StackedInputs(LayerInputs(s))
    x, w, b = run_layer(s, inp, gather=True)
    c = binding.make_shape(s)
    h = torch.full_like(b.h, 3.0)
    y = torch.full_like(b.y_perm, 3.0)
    ys = torch.full_like(b.y_shared, 3.0)
    binding.moe_grouped_ffn(c, None, b.sorted_token, x, b.offsets, w.w_gate_up, w.w_down, w.ws_gate_up,
                            w.ws_down, h, y, ys)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), b.h.view(torch.int16))
    assert torch.equal(y.view(torch.int16), b.y_perm.view(torch.int16))
    assert torch.equal(ys.view(torch.int16), b.y_shared.view(torch.int16))


def test_empty_batch_is_a_no_op():
    s = configs.variant(SMALL_BF16, T=0)
    c = binding.make_shape(s)
    binding.moe_combine(c, None, None, None, None, None)
    binding.moe_route(c, None, None, None, None, None, None)


def test_invalid_arguments_raise_without_launch():
    s = SMALL_BF16
    b = binding.alloc_buffers(s)
    c = binding.make_shape(configs.variant(s, k=0))
    with pytest.raises(binding.MoEError):
        binding.moe_combine(c, b.y_perm, b.y_shared, b.slot_of, b.topk_w, b.out)
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.MoEError):
        binding.moe_permute(binding.make_shape(s), b.topk_idx, b.out, b.counts, b.offsets,
                            b.sorted_token, b.slot_of, None, small_ws)


def _packed_reference(w: np.ndarray) -> np.ndarray:
    """The layout include/moe.h documents for moe_pack_weights, element by element."""
    count, rows, cols = w.shape
    per = rows * cols
    out = np.zeros(count * per, dtype=w.dtype)
    for i in range(count):
        for r in range(rows):
            for c in range(cols):
                o = ((r // 32) * (cols // 16) + c // 16) * 512 + ((r % 32) + 32 * ((c % 16) // 8)) * 8 + c % 8
                out[i * per + o] = w[i, r, c]
    return out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pack_weights_layout_and_padding(dtype):
    say(f"pack layout {dtype}")
    rng = np.random.default_rng(7)
    count, rows, cols = 3, 64, 48
    if dtype == torch.bfloat16:
        host = rng.integers(1, 1 << 15, size=(count, rows, cols), dtype=np.int64).astype(np.int16)
        w = torch.from_numpy(host).view(torch.bfloat16).cuda()
    else:
        host = rng.standard_normal((count, rows, cols)).astype(np.float32)
        w = torch.from_numpy(host).cuda()
    code = binding.MOE_BF16 if dtype == torch.bfloat16 else binding.MOE_F32
    n = binding.moe_packed_bytes(count, rows, cols, code) // w.element_size()
    big, out = _guarded_like(torch.empty(n, dtype=dtype, device="cuda"))
    binding.moe_pack_weights(w, out, count, rows, cols, code)
    torch.cuda.synchronize()
    assert _guard_intact(big, n), "write past the end of the packed buffer"
    got = out.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.float32).numpy()
    assert np.array_equal(got, _packed_reference(host))
