"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments
on the host before any launch (no GPU needed: no compute call is made)."""
import ctypes
import os

import pytest

from scale_search_weights_amd import nvfp4

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EHIP, EARG = range(8)
FAKE = 0x7F0000000000  # never dereferenced: validation fails or returns before any use


@pytest.fixture(scope="module")
def L():
    return nvfp4.lib()


def test_exports_every_declared_symbol(L):
    names = nvfp4.declared_symbols()
    assert len(names) == 30
    for n in names:
        assert hasattr(L, n), n
    assert L.nvfp4_version() == 100


def test_status_strings(L):
    for s in range(8):
        assert nvfp4.status_string(s).startswith("NVFP4_")
    assert "unknown" in nvfp4.status_string(99)


def P(v):
    return ctypes.c_void_p(v)


def test_shape_dtype_null_align_checks(L):
    f = L.nvfp4_fakequant
    # cols not a multiple of 16
    assert f(P(FAKE), 1, 1, 4, 17, P(FAKE), None, P(FAKE), None, None, None) == ESHAPE
    assert f(P(FAKE), 1, -1, 4, 16, P(FAKE), None, P(FAKE), None, None, None) == ESHAPE
    # unknown dtype
    assert f(P(FAKE), 7, 1, 4, 16, P(FAKE), None, P(FAKE), None, None, None) == EDTYPE
    # NULL input / output / S
    assert f(None, 1, 1, 4, 16, P(FAKE), None, P(FAKE), None, None, None) == ENULL
    assert f(P(FAKE), 1, 1, 4, 16, None, None, P(FAKE), None, None, None) == ENULL
    assert f(P(FAKE), 1, 1, 4, 16, P(FAKE), None, None, None, None, None) == ENULL
    # misaligned element pointer and codes pointer
    assert f(P(FAKE + 2), 1, 1, 4, 16, P(FAKE), None, P(FAKE), None, None, None) == EALIGN
    assert f(P(FAKE), 1, 1, 4, 16, P(FAKE), None, P(FAKE), P(FAKE + 4), None, None) == EALIGN
    # size overflow
    assert f(P(FAKE), 1, 1 << 40, 1 << 20, 1 << 20, P(FAKE), None, P(FAKE), None, None, None) == ESHAPE


def test_empty_tensors_return_ok_without_launch(L):
    assert L.nvfp4_fakequant(None, 1, 1, 0, 16, None, None, None, None, None, None) == OK
    assert L.nvfp4_fakequant(None, 1, 0, 4, 16, None, None, None, None, None, None) == OK
    assert L.nvfp4_scale_search_mse(None, 0, 1, 4, 0, None, None, None, None) == OK
    assert L.nvfp4_scale_search_four_over_six(None, 1, 0, 4, 16, None, None, None, None) == OK
    assert L.nvfp4_scale_search_local_hessian(None, 1, 1, 0, 32, None, None, None, None, None) == OK
    assert L.nvfp4_global_scale(None, 1, 0, 16, None, None) == OK
    assert L.nvfp4_quantize(None, 1, 1, 0, 16, None, None, None, None, None) == OK
    assert L.nvfp4_dequantize(None, None, None, 1, 0, 16, None, 1, None) == OK


def test_global_scale_workspace_checks(L):
    f = L.nvfp4_global_scale_ws
    need = L.nvfp4_global_scale_workspace_size(1, 4096 * 4096)
    assert need > 0
    assert L.nvfp4_global_scale_workspace_size(1, 12) == 0        # n % 8
    assert L.nvfp4_global_scale_workspace_size(0, 16) == 0        # nothing to do
    assert L.nvfp4_global_scale_workspace_size(-1, 16) == 0
    assert L.nvfp4_global_scale_workspace_size(1 << 40, 1 << 40) == 0
    assert f(P(FAKE), 1, 1, 12, P(FAKE), P(FAKE), need, None) == ESHAPE
    assert f(P(FAKE), 9, 1, 16, P(FAKE), P(FAKE), need, None) == EDTYPE
    assert f(P(FAKE), 1, 1, 4096 * 4096, P(FAKE), None, need, None) == EWS
    assert f(P(FAKE), 1, 1, 4096 * 4096, P(FAKE), P(FAKE), need - 1, None) == EWS
    assert f(P(FAKE), 1, 1, 4096 * 4096, P(FAKE), P(FAKE + 2), need, None) == EALIGN
    assert f(P(FAKE), 1, 1, 4096 * 4096, None, P(FAKE), need, None) == ENULL
    assert f(None, 1, 0, 16, None, None, 0, None) == OK             # empty: no launch


def test_each_entry_point_validates(L):
    assert L.nvfp4_global_scale(P(FAKE), 1, 1, 12, P(FAKE), None) == ESHAPE  # n % 8
    assert L.nvfp4_global_scale(P(FAKE), 9, 1, 16, P(FAKE), None) == EDTYPE
    assert L.nvfp4_scale_search_max(P(FAKE), 1, 1, 2, 16, P(FAKE), None, None) == ENULL
    assert L.nvfp4_scale_search_mse(P(FAKE), 1, 1, 2, 8, P(FAKE), P(FAKE), None, None) == ESHAPE
    assert L.nvfp4_scale_search_mse(P(FAKE), 1, 1, 2, 16, P(FAKE), P(FAKE), P(FAKE + 1), None) == EALIGN
    assert L.nvfp4_calib_histogram(P(FAKE), 1, 12, P(FAKE), None) == ESHAPE
    assert L.nvfp4_calib_histogram(P(FAKE), 1, 16, None, None) == ENULL
    assert L.nvfp4_calib_histogram(P(FAKE), 1, 16, P(FAKE + 4), None) == EALIGN
    assert L.nvfp4_calib_histogram(None, 1, 0, P(FAKE), None) == OK
    assert L.nvfp4_calib_scale(P(FAKE), ctypes.c_double(0.0), P(FAKE), None) == EARG
    assert L.nvfp4_calib_scale(P(FAKE), ctypes.c_double(1.5), P(FAKE), None) == EARG
    assert L.nvfp4_calib_scale(None, ctypes.c_double(0.5), P(FAKE), None) == ENULL
    assert L.nvfp4_ste_backward(P(FAKE), 1, 16, ctypes.c_float(0.0), P(FAKE), None) == EARG
    assert L.nvfp4_ste_backward(P(FAKE), 1, 16, ctypes.c_float(float("nan")), P(FAKE), None) == EARG
    assert L.nvfp4_ste_backward(P(FAKE), 1, 12, ctypes.c_float(1.0), P(FAKE), None) == ESHAPE
    assert L.nvfp4_ste_backward(P(FAKE), 1, 16, ctypes.c_float(1.0), P(FAKE + 8), None) == EALIGN
    assert L.nvfp4_ste_backward(None, 1, 0, ctypes.c_float(1.0), None, None) == OK
    assert L.nvfp4_scale_ema(P(FAKE), P(FAKE), 1, ctypes.c_float(1.5), None) == EARG
    assert L.nvfp4_scale_ema(None, P(FAKE), 1, ctypes.c_float(0.9), None) == ENULL
    assert L.nvfp4_full_hessian(P(FAKE), 1, 8, 24, P(FAKE), 0, P(FAKE), 1 << 20, None) == ESHAPE
    assert L.nvfp4_full_hessian(P(FAKE), 5, 8, 32, P(FAKE), 0, P(FAKE), 1 << 20, None) == EDTYPE
    assert L.nvfp4_full_hessian(P(FAKE), 1, 8, 32, P(FAKE), 0, P(FAKE), 16, None) == EWS
    assert L.nvfp4_gptq_factor(P(FAKE), 32, ctypes.c_double(-1.0), P(FAKE), None, P(FAKE),
                               1 << 30, None) == EARG
    assert L.nvfp4_gptq_factor(P(FAKE), 32, ctypes.c_double(float("nan")), P(FAKE), None,
                               P(FAKE), 1 << 30, None) == EARG
    assert L.nvfp4_gptq_factor(P(FAKE), 32, ctypes.c_double(0.01), P(FAKE + 8), None, P(FAKE),
                               1 << 30, None) == EALIGN
    assert L.nvfp4_gptq_factor(P(FAKE), 32, ctypes.c_double(0.01), P(FAKE), None, P(FAKE),
                               16, None) == EWS
    assert L.nvfp4_gptq(P(FAKE), 1, 4, 40, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                        1 << 30, None) == ESHAPE
    assert L.nvfp4_gptq(P(FAKE), 1, 4, 32, P(FAKE), None, P(FAKE), P(FAKE), P(FAKE),
                        1 << 30, None) == ENULL
    assert L.nvfp4_gptq(P(FAKE), 1, 4, 32, P(FAKE), P(FAKE), P(FAKE), P(FAKE + 4), P(FAKE),
                        1 << 30, None) == EALIGN
    assert L.nvfp4_gptq(P(FAKE), 1, 0, 32, None, None, None, None, None, 0, None) == OK
    assert L.nvfp4_gptq_workspace_size(4, 32) > 0 and L.nvfp4_gptq_factor_workspace_size(32) > 0
    flag = ctypes.c_int32(7)
    old = os.environ.pop("NVFP4_DEBUG_CHECKS", None)
    try:
        assert L.nvfp4_debug_nonfinite(ctypes.byref(flag), None) == EARG  # checks off
        assert L.nvfp4_debug_nonfinite(None, None) == ENULL
    finally:
        if old is not None:
            os.environ["NVFP4_DEBUG_CHECKS"] = old
    f46 = L.nvfp4_scale_search_four_over_six
    assert f46(P(FAKE), 1, 1, 2, 24, P(FAKE), P(FAKE), None, None) == ESHAPE
    assert f46(P(FAKE), 4, 1, 2, 16, P(FAKE), P(FAKE), None, None) == EDTYPE
    assert f46(P(FAKE), 1, 1, 2, 16, None, P(FAKE), None, None) == ENULL
    assert f46(P(FAKE + 8), 1, 1, 2, 16, P(FAKE), P(FAKE), None, None) == EALIGN
    assert f46(P(FAKE), 1, 1, 2, 16, P(FAKE), P(FAKE), P(FAKE + 2), None) == EALIGN
    assert L.nvfp4_scale_search_local_hessian(P(FAKE), 1, 1, 2, 16, P(FAKE), None, P(FAKE), None,
                                              None) == ENULL
    assert L.nvfp4_scale_search_local_hessian(P(FAKE), 1, 1, 2, 16, P(FAKE), P(FAKE), P(FAKE),
                                              P(FAKE + 4), None) == EALIGN
    assert L.nvfp4_quantize(P(FAKE), 1, 1, 2, 16, P(FAKE), None, None, None, None) == ENULL
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 1, 2, 16, P(FAKE), 3, None) == EDTYPE


def test_block_hessian_workspace_and_group_checks(L):
    need = L.nvfp4_block_hessian_workspace_size(4096, 512, 1, 0)
    assert need >= 512 // 16 * 256 * 4
    f = L.nvfp4_block_hessian
    # too small / missing workspace
    assert f(P(FAKE), 1, 4096, 512, 1, None, None, 0, P(FAKE), 0, P(FAKE), need - 1, None) == EWS
    assert f(P(FAKE), 1, 4096, 512, 1, None, None, 0, P(FAKE), 0, None, need, None) == EWS
    # dense form must have exactly one group; grouped form needs both arrays
    assert f(P(FAKE), 1, 4096, 512, 2, None, None, 0, P(FAKE), 0, P(FAKE), need, None) == EARG
    assert f(P(FAKE), 1, 4096, 512, 2, P(FAKE), None, 10, P(FAKE), 0, P(FAKE), need, None) == ENULL
    assert f(P(FAKE), 1, 4096, 500, 1, None, None, 0, P(FAKE), 0, P(FAKE), need, None) == ESHAPE
    # grouped sizing grows with the number of ids
    a = L.nvfp4_block_hessian_workspace_size(1000, 512, 8, 100)
    b = L.nvfp4_block_hessian_workspace_size(1000, 512, 8, 1000000)
    assert b > a


def test_block_hessian_noalloc_checks(L):
    """The allocation-free form validates like the workspace form and refuses calls whose
    workspace would exceed its static scratch, all before touching the device."""
    f = L.nvfp4_block_hessian_noalloc
    assert f(P(FAKE), 1, 4096, 500, 1, None, None, 0, P(FAKE), 0, None) == ESHAPE
    assert f(P(FAKE), 7, 4096, 512, 1, None, None, 0, P(FAKE), 0, None) == EDTYPE
    assert f(P(FAKE), 1, 4096, 512, 2, None, None, 0, P(FAKE), 0, None) == EARG
    assert f(P(FAKE), 1, 4096, 512, 1, None, None, 0, None, 0, None) == ENULL
    assert f(P(FAKE + 2), 1, 4096, 512, 1, None, None, 0, P(FAKE), 0, None) == EALIGN
    assert f(None, 1, 4096, 0, 1, None, None, 0, None, 0, None) == OK
    big_t, big_c = 1 << 20, 16384
    assert L.nvfp4_block_hessian_workspace_size(big_t, big_c, 1, 0) > nvfp4.STATIC_SCRATCH_BYTES
    assert f(P(FAKE), 1, big_t, big_c, 1, None, None, 0, P(FAKE), 0, None) == EWS
    # the two projection-sized and MoE-sized calibration calls fit
    assert L.nvfp4_block_hessian_workspace_size(131072, 4096, 1, 0) <= nvfp4.STATIC_SCRATCH_BYTES
    assert L.nvfp4_block_hessian_workspace_size(65536, 2048, 128, 524288) <= nvfp4.STATIC_SCRATCH_BYTES


def test_route_groups_checks(L):
    need = L.nvfp4_route_groups_workspace_size(1000, 8, 128)
    assert need > 0
    f = L.nvfp4_route_groups
    assert f(P(FAKE), 1000, 8, 0, P(FAKE), P(FAKE), P(FAKE), need, None) == ESHAPE
    assert f(P(FAKE), 1000, 8, 20000, P(FAKE), P(FAKE), P(FAKE), need, None) == EARG
    assert f(P(FAKE), 1000, 8, 128, P(FAKE), P(FAKE), P(FAKE), need - 1, None) == EWS
    assert f(P(FAKE), 1000, 8, 128, None, P(FAKE), P(FAKE), need, None) == ENULL


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nvfp4.fakequant(torch.zeros(4, 16), torch.ones(1))
    with pytest.raises(TypeError):
        nvfp4._dt(torch.zeros(1, dtype=torch.float16))


# ---------------------------------------------------------------- binding argument checks
# The binding checks every tensor argument before the library is called. On this CPU-only
# host the tensors below are CPU tensors dressed up as GPU tensors (only their metadata is
# read); the library loader is replaced so that any call through it fails the test.

import torch  # noqa: E402


class _OnGpu(torch.Tensor):
    """A CPU tensor that reports itself as living on cuda:<index> (metadata only)."""
    index = 0

    @property
    def is_cuda(self):
        return True

    @property
    def device(self):
        return torch.device("cuda", type(self).index)


class _OnGpu1(_OnGpu):
    index = 1


def G(*shape, dtype=torch.float32, cls=_OnGpu):
    return torch.zeros(*shape, dtype=dtype).as_subclass(cls)


@pytest.fixture
def no_launch(monkeypatch):
    def boom():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(nvfp4, "lib", boom)


def _bad_cases():
    x = G(8, 32)                      # fp32 [8, 32]: 16 blocks
    xb = G(8, 32, dtype=torch.bfloat16)
    w3 = G(3, 8, 32)                  # batch 3
    S1 = G(1)
    return [
        ("S on the host", lambda: nvfp4.fakequant(x, torch.ones(1)), ValueError),
        ("S on another GPU", lambda: nvfp4.fakequant(x, G(1, cls=_OnGpu1)), ValueError),
        ("S fp64", lambda: nvfp4.fakequant(x, G(1, dtype=torch.float64)), TypeError),
        ("S with fewer entries than the batch", lambda: nvfp4.scale_search_mse(w3, S1), ValueError),
        ("S with more entries", lambda: nvfp4.quantize(x, G(2)), ValueError),
        ("scales too small", lambda: nvfp4.quantize(x, S1, G(15, dtype=torch.uint8)), ValueError),
        ("scales not uint8", lambda: nvfp4.fakequant(x, S1, G(16, dtype=torch.int32)), TypeError),
        ("out bf16 for an fp32 input", lambda: nvfp4.fakequant(x, S1, out=G(8, 32, dtype=torch.bfloat16)), TypeError),
        ("out too small", lambda: nvfp4.fakequant(xb, S1, out=G(8, 16, dtype=torch.bfloat16)), ValueError),
        ("out not contiguous", lambda: nvfp4.fakequant(x, S1, out=G(32, 8).t()), ValueError),
        ("dequantize with a short S", lambda: nvfp4.dequantize(G(3, 8, 16, dtype=torch.uint8), G(3 * 16, dtype=torch.uint8), S1), ValueError),
        ("dequantize scales too small", lambda: nvfp4.dequantize(G(8, 16, dtype=torch.uint8), G(8, dtype=torch.uint8), S1), ValueError),
        ("Local-Hessian H too small", lambda: nvfp4.scale_search_local_hessian(x, S1, G(1, 16, 16)), ValueError),
        ("Local-Hessian H fp64", lambda: nvfp4.scale_search_local_hessian(x, S1, G(2, 16, 16, dtype=torch.float64)), TypeError),
        ("GPTQ U fp32", lambda: nvfp4.gptq(x, S1, G(16, dtype=torch.uint8), G(32, 32)), TypeError),
        ("GPTQ U too small", lambda: nvfp4.gptq(x, S1, G(16, dtype=torch.uint8), G(16, 32, dtype=torch.float64)), ValueError),
        ("GPTQ S with two entries", lambda: nvfp4.gptq(x, G(2), G(16, dtype=torch.uint8), G(32, 32, dtype=torch.float64)), ValueError),
        ("GPTQ factor of a non-square H", lambda: nvfp4.gptq_factor(G(32, 16)), ValueError),
        ("histogram int32", lambda: nvfp4.calib_histogram(x, G(nvfp4.CALIB_BINS, dtype=torch.int32)), TypeError),
        ("histogram too short", lambda: nvfp4.calib_scale(G(100, dtype=torch.int64), 0.5), ValueError),
        ("block Hessian H too small", lambda: nvfp4.block_hessian(x, H=G(1, 16, 16)), ValueError),
        ("block Hessian ids without offsets", lambda: nvfp4.block_hessian(x, token_ids=G(4, dtype=torch.int32)), ValueError),
        ("block Hessian offsets int64", lambda: nvfp4.block_hessian(x, G(3, dtype=torch.int64), G(4, dtype=torch.int32)), TypeError),
        ("full Hessian H too small", lambda: nvfp4.full_hessian(x, H=G(32, 16)), ValueError),
        ("STE out of another dtype", lambda: nvfp4.ste_backward(xb, 1.0, out=G(8, 32)), TypeError),
        ("scale EMA with a short batch scale", lambda: nvfp4.scale_ema(G(3), G(2), 0.9), ValueError),
        ("routing ids int64", lambda: nvfp4.route_groups(G(4, 2, dtype=torch.int64), 8), ValueError),
    ]


@pytest.mark.parametrize("what,call,exc", _bad_cases(), ids=[c[0] for c in _bad_cases()])
def test_binding_rejects_bad_tensor_arguments(no_launch, what, call, exc):
    with pytest.raises(exc):
        call()
