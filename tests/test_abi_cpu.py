"""The C ABI library on the host (no GPU needed): it loads, exports every entry
point include/moe.h declares, and rejects bad arguments before launching."""
import ctypes
import os
import re

import pytest

from mixture_experts_transformer_moe_amd import binding, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_transformer_moe_amd.build import build
        build(verbose=False)
    return binding.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.moe_version() == 1
    for st in range(5):
        assert L.moe_status_string(st)
    assert L.moe_status_string(99) == b"unknown status"


def _shape(**kw):
    s = configs.variant(configs.XS2_T4096, **kw) if kw else configs.XS2_T4096
    return binding.make_shape(s)


def _route(L, shape, ptr=16 * 1024):
    p = ctypes.c_void_p(ptr)
    return L.moe_route(ctypes.byref(shape), p, p, None, p, p, p, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), binding.MOE_ERR_INVALID_ARG),
    (dict(k=300, E=256), binding.MOE_ERR_INVALID_ARG),
    (dict(E=0), binding.MOE_ERR_INVALID_ARG),
    (dict(T=-1), binding.MOE_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), binding.MOE_ERR_INVALID_ARG),
    (dict(E=512), binding.MOE_ERR_UNSUPPORTED),
    (dict(k=17, E=64), binding.MOE_ERR_UNSUPPORTED),
    (dict(D=2000), binding.MOE_ERR_UNSUPPORTED),
    (dict(F=500), binding.MOE_ERR_UNSUPPORTED),
    (dict(Fs=100), binding.MOE_ERR_UNSUPPORTED),
    (dict(F=384), binding.MOE_ERR_UNSUPPORTED),
    (dict(T=1200000), binding.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 28), binding.MOE_ERR_UNSUPPORTED),
])
def test_bad_shapes_are_rejected_before_launch(L, kw, status):
    assert _route(L, _shape(**kw)) == status
    assert L.moe_last_error()
    assert L.moe_workspace_bytes(ctypes.byref(_shape(**kw))) == 0


def test_bad_pointers_are_rejected(L):
    s = _shape()
    p = ctypes.c_void_p(4096)
    assert L.moe_route(ctypes.byref(s), None, p, None, p, p, p, None) == binding.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in L.moe_last_error()
    assert L.moe_route(ctypes.byref(s), ctypes.c_void_p(4098), p, None, p, p, p, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert b"aligned" in L.moe_last_error()
    assert L.moe_route(None, p, p, None, p, p, p, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(s), p, None, p, None, p, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_ffn(ctypes.byref(s), None, None, p, p, p, p, p, p, p, p, p, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert b"sorted_token" in L.moe_last_error()


def test_workspace_checks(L):
    s = _shape()
    need = L.moe_workspace_bytes(ctypes.byref(s))
    assert need >= 16 * 256 * 4 and need % 256 == 0      # one histogram row per 256 tokens
    p = ctypes.c_void_p(4096)
    st = L.moe_permute(ctypes.byref(s), p, p, p, p, p, p, None, p, need - 1, None)
    assert st == binding.MOE_ERR_WORKSPACE
    st = L.moe_permute(ctypes.byref(s), p, p, p, p, p, p, None, None, need, None)
    assert st == binding.MOE_ERR_WORKSPACE


def test_permute_static_checks_before_launch(L):
    # null outputs are rejected like moe_permute's
    s = _shape()
    p = ctypes.c_void_p(4096)
    assert L.moe_permute_static(ctypes.byref(s), p, p, None, p, p, p, None, None) == \
        binding.MOE_ERR_INVALID_ARG
    # its device-resident scratch holds 1 MiB of histograms: ceil(T / 256) * E * 4
    # bytes; one more 256-token block at E = 256 is refused with a clear error
    big = _shape(T=1024 * 256 + 1, E=256, k=1)
    assert L.moe_workspace_bytes(ctypes.byref(big)) > 1 << 20
    st = L.moe_permute_static(ctypes.byref(big), p, p, p, p, p, p, None, None)
    assert st == binding.MOE_ERR_UNSUPPORTED
    assert b"scratch" in L.moe_last_error()
    # an empty batch is a no-op, as for every entry point
    assert L.moe_permute_static(ctypes.byref(_shape(T=0)), None, None, None, None, None, None, None,
                                None) == binding.MOE_OK


def test_empty_batch_is_a_no_op(L):
    s = _shape(T=0)
    assert _route(L, s, ptr=0) == binding.MOE_OK
    assert L.moe_combine(ctypes.byref(s), None, None, None, None, None, None) == binding.MOE_OK


def test_packed_sizes_and_pack_argument_checks(L):
    # packing permutes elements inside each matrix: the size is unchanged
    assert L.moe_packed_bytes(1, 32, 16, binding.MOE_BF16) == 512 * 2
    assert L.moe_packed_bytes(256, 1024, 2048, binding.MOE_BF16) == 256 * 1024 * 2048 * 2
    assert L.moe_packed_bytes(3, 64, 48, binding.MOE_F32) == 3 * 64 * 48 * 4
    assert L.moe_packed_bytes(0, 64, 48, binding.MOE_F32) == 0
    for bad in ((1, 33, 16, binding.MOE_BF16), (1, 32, 20, binding.MOE_BF16), (1, 32, 16, 7),
                (-1, 32, 16, binding.MOE_BF16)):
        assert L.moe_packed_bytes(*bad) == 0
    p, q = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 30)
    assert L.moe_pack_weights(p, q, 1, 33, 16, binding.MOE_BF16, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(p, q, 1, 32, 16, 5, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(None, q, 1, 32, 16, binding.MOE_BF16, None) == binding.MOE_ERR_INVALID_ARG
    # an output that starts inside the input overlaps it
    assert L.moe_pack_weights(p, ctypes.c_void_p((1 << 20) + 512), 1, 32, 16, binding.MOE_BF16,
                              None) == binding.MOE_ERR_INVALID_ARG
    assert b"overlap" in L.moe_last_error()
    assert L.moe_pack_weights(p, q, 0, 32, 16, binding.MOE_BF16, None) == binding.MOE_OK


def test_fp8_sizes_and_argument_checks(L):
    # one byte per weight; rows and columns in whole 32 x 32 blocks
    assert L.moe_fp8_packed_bytes(256, 2048, 4096) == 256 * 2048 * 4096
    assert L.moe_fp8_packed_bytes(1, 32, 32) == 1024
    for bad in ((1, 33, 32), (1, 32, 48), (-1, 32, 32)):
        assert L.moe_fp8_packed_bytes(*bad) == 0
    p, q, r = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 34)
    assert L.moe_quantize_weights_fp8(p, q, r, 1, 32, 48, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_weights_fp8(p, None, r, 1, 32, 32, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_weights_fp8(p, q, None, 1, 32, 32, None) == binding.MOE_ERR_INVALID_ARG
    # the scales may not overlap the codes
    assert L.moe_quantize_weights_fp8(p, q, ctypes.c_void_p((1 << 30) + 512), 1, 32, 32,
                                      None) == binding.MOE_ERR_INVALID_ARG
    assert b"overlap" in L.moe_last_error()
    assert L.moe_quantize_weights_fp8(p, q, r, 0, 32, 32, None) == binding.MOE_OK
    # FP8 weights need bf16 activations; the grouped GEMMs check before launching
    s = binding.make_shape(configs.TINY_F32)
    args = [ctypes.c_void_p(1 << 20)] * 8
    assert L.moe_grouped_gate_up_fp8(ctypes.byref(s), None, *args, None) == binding.MOE_ERR_UNSUPPORTED
    sb = binding.make_shape(configs.variant(configs.XS2_T4096, T=64))
    assert L.moe_grouped_down_fp8(ctypes.byref(sb), *([ctypes.c_void_p(1 << 20)] * 3), None,
                                  *([ctypes.c_void_p(1 << 20)] * 4), None) == binding.MOE_ERR_INVALID_ARG
    assert b"w_down_scale" in L.moe_last_error()


def test_training_entry_points_check_arguments(L):
    s32 = binding.make_shape(configs.TINY_F32)
    s16 = binding.make_shape(configs.variant(configs.XS2_T4096, T=64))
    p = ctypes.c_void_p(1 << 20)
    assert L.moe_train_workspace_bytes(ctypes.byref(s16)) >= 256
    # transposed packing: the transpose's rows (source columns) in 32s, k_padded >= rows in 16s
    assert L.moe_packed_transposed_bytes(4, 2048, 512, 2048) == 4 * 512 * 2048 * 2
    assert L.moe_packed_transposed_bytes(1, 16, 2048, 256) == 2048 * 256 * 2
    for bad in ((1, 32, 48, 32), (1, 40, 64, 32), (1, 32, 64, 40), (-1, 32, 64, 32)):
        assert L.moe_packed_transposed_bytes(*bad) == 0
    assert L.moe_pack_weights_transposed(p, ctypes.c_void_p(1 << 30), 1, 40, 64, 32, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights_transposed(p, ctypes.c_void_p((1 << 20) + 64), 1, 32, 64, 32, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert b"overlap" in L.moe_last_error()
    # the training pass is bf16 only
    args = [p] * 11
    assert L.moe_combine_backward(ctypes.byref(s32), *args) == binding.MOE_ERR_UNSUPPORTED
    assert L.moe_grouped_gate_up_train(ctypes.byref(s32), *([p] * 9)) == binding.MOE_ERR_UNSUPPORTED
    big = binding.make_shape(configs.variant(configs.XS2_T4096, T=600000, Fs=2048))
    assert L.moe_combine_backward(ctypes.byref(big), *args) == binding.MOE_ERR_UNSUPPORTED
    assert b"2 Fs" in L.moe_last_error()
    # missing pointers and workspace are caught before any launch
    assert L.moe_combine_backward(ctypes.byref(s16), None, *([p] * 10)) == binding.MOE_ERR_INVALID_ARG
    assert b"dout" in L.moe_last_error()
    assert L.moe_load_stats(ctypes.byref(s16), p, p, p, None, ctypes.c_float(0.1), p, p, p, p, None, 0,
                            None) == binding.MOE_ERR_WORKSPACE
    assert L.moe_load_stats(ctypes.byref(s16), p, p, p, None, ctypes.c_float(float("nan")), p, p, p, p, p,
                            1 << 20, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_backward_x(ctypes.byref(s16), *([p] * 6), None, *([p] * 5)) == \
        binding.MOE_ERR_INVALID_ARG
    assert b"slot_of" in L.moe_last_error()
    assert L.moe_weight_grads(ctypes.byref(s16), *([p] * 9), None, *([p] * 4), None, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert b"dw_gate_up" in L.moe_last_error()
    assert L.moe_bias_grad(ctypes.byref(s16), p, p, None, 0, None) == binding.MOE_ERR_WORKSPACE


def test_shared_ffn_argument_checks(L):
    p = ctypes.c_void_p(4096)
    s = _shape()
    assert L.moe_shared_ffn(ctypes.byref(s), None, p, p, p, p, None) == binding.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in L.moe_last_error()
    assert L.moe_shared_ffn(ctypes.byref(_shape(Fs=0)), p, p, p, p, p, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert L.moe_shared_ffn(ctypes.byref(_shape(dtype="f32")), p, p, p, p, p, None) == \
        binding.MOE_ERR_UNSUPPORTED
    assert L.moe_shared_ffn(ctypes.byref(_shape(T=0)), None, None, None, None, None, None) == \
        binding.MOE_OK
    # fp32 grouped GEMMs still need the shared expert's weights
    f32 = _shape(dtype="f32")
    assert L.moe_grouped_down(ctypes.byref(f32), p, p, p, None, p, p, None) == \
        binding.MOE_ERR_INVALID_ARG
