"""moe_permute_static (no allocation, device-resident scratch) against
moe_permute (caller workspace) through the C ABI: identical counts, offsets,
expert order, slots and gathered rows, on consecutive calls of decreasing size
(the second call must not see the first one's scratch contents)."""
import numpy as np
import pytest
import torch

from mixture_experts_transformer_moe_amd import binding, configs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    # k distinct experts per token, skewed so that some experts get many tokens
    keys = rng.random((T, E)) * (1.0 + np.arange(E)[None, :] % 7)
    return np.argsort(-keys, axis=1)[:, :k].astype(np.int32)


def _run_both(T, E, k, D, seed):
    s = configs.variant(configs.XS2_T4096, name=f"perm_t{T}_e{E}_k{k}", T=T, E=E, k=k, D=D, F=256, Fs=256)
    c = binding.make_shape(s)
    idx = torch.from_numpy(_routing(T, E, k, seed)).cuda()
    x = torch.randn(T, D, device="cuda").to(torch.bfloat16)
    outs = []
    for static in (False, True):
        counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        sorted_token = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        slot_of = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        x_perm = torch.zeros(T * k, D, dtype=torch.bfloat16, device="cuda")
        if static:
            binding.moe_permute_static(c, idx, x, counts, offsets, sorted_token, slot_of, x_perm)
        else:
            ws = torch.empty(binding.workspace_bytes(c), dtype=torch.uint8, device="cuda")
            binding.moe_permute(c, idx, x, counts, offsets, sorted_token, slot_of, x_perm, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (counts, offsets, sorted_token, slot_of)] + [x_perm.view(torch.int16).cpu()])
    names = ("counts", "offsets", "sorted_token", "slot_of", "x_perm")
    for n, a, b in zip(names, outs[0], outs[1]):
        assert torch.equal(a, b), f"{s.name}: {n} differs between moe_permute and moe_permute_static"
    assert int(outs[1][1][-1]) == T * k
    say(f"{s.name}: moe_permute_static equals moe_permute bit for bit")


def test_permute_static_equals_permute_on_consecutive_calls():
    # the full long-prefill shape (128 token blocks x 256 experts of scratch),
    # then smaller batches: a few blocks, then one block (no scratch used)
    _run_both(32768, 256, 8, 256, seed=1)
    _run_both(3000, 64, 4, 512, seed=2)
    _run_both(700, 256, 8, 256, seed=3)
    _run_both(200, 16, 2, 256, seed=4)
    # and back to a multi-block batch after the single-block one
    _run_both(1300, 256, 16, 256, seed=5)
