"""ctypes wrapper around the plain-C NVFP4 oracle (``nvfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg. The product path never imports it.

Arrays are numpy; bf16 inputs must be widened to float32 by the caller (exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libnvfp4_oracle.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        f32 = ctypes.c_float
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [f32]
        L.oracle_bf16_rne_array.restype = None
        L.oracle_bf16_rne_array.argtypes = [P, i64, P]
        L.oracle_tensor_scale.restype = f32
        L.oracle_tensor_scale.argtypes = [P, i64]
        L.oracle_max_byte.restype = ctypes.c_int
        L.oracle_max_byte.argtypes = [f32, f32]
        L.oracle_e2m1_code.restype = ctypes.c_int
        L.oracle_e2m1_code.argtypes = [f32, ctypes.c_int, f32]
        L.oracle_dequant_value.restype = f32
        L.oracle_dequant_value.argtypes = [ctypes.c_int, ctypes.c_int, f32]
        L.oracle_scales_max.restype = None
        L.oracle_scales_max.argtypes = [P, i64, i64, f32, P]
        L.oracle_quantize.restype = None
        L.oracle_quantize.argtypes = [P, i64, i64, f32, P, P]
        L.oracle_dequantize.restype = None
        L.oracle_dequantize.argtypes = [P, P, i64, i64, f32, P]
        L.oracle_block_sq_error.restype = f32
        L.oracle_block_sq_error.argtypes = [P, ctypes.c_int, f32]
        L.oracle_scales_mse.restype = None
        L.oracle_scales_mse.argtypes = [P, i64, i64, f32, P, P]
        L.oracle_ste_clamp.restype = f32
        L.oracle_ste_clamp.argtypes = [f32, f32]
        L.oracle_scale_ema.restype = f32
        L.oracle_scale_ema.argtypes = [f32, f32, f32]
        L.oracle_calib_histogram.restype = None
        L.oracle_calib_histogram.argtypes = [P, i64, P]
        L.oracle_calib_scale.restype = f32
        L.oracle_calib_scale.argtypes = [P, ctypes.c_double]
        L.oracle_byte_for_divisor.restype = ctypes.c_int
        L.oracle_byte_for_divisor.argtypes = [f32, f32, ctypes.c_double]
        L.oracle_scales_four_over_six.restype = None
        L.oracle_scales_four_over_six.argtypes = [P, i64, i64, f32, P, P]
        L.oracle_block_hessian.restype = None
        L.oracle_block_hessian.argtypes = [P, i64, i64, P, i64, P]
        L.oracle_block_lh_objective.restype = ctypes.c_double
        L.oracle_block_lh_objective.argtypes = [P, ctypes.c_int, f32, P]
        L.oracle_scales_local_hessian.restype = None
        L.oracle_scales_local_hessian.argtypes = [P, i64, i64, f32, P, P, P]
        L.oracle_route_groups.restype = ctypes.c_int
        L.oracle_route_groups.argtypes = [P, i64, i64, i64, P, P]
        L.oracle_full_hessian.restype = None
        L.oracle_full_hessian.argtypes = [P, i64, i64, P]
        L.oracle_e2m1_code_d.restype = ctypes.c_int
        L.oracle_e2m1_code_d.argtypes = [ctypes.c_double, ctypes.c_int, f32]
        L.oracle_gptq_factor.restype = i64
        L.oracle_gptq_factor.argtypes = [P, i64, ctypes.c_double, P]
        L.oracle_gptq_rows.restype = None
        L.oracle_gptq_rows.argtypes = [P, i64, i64, f32, P, P, P, P]
        L.oracle_gptq_rows_flip.restype = None
        L.oracle_gptq_rows_flip.argtypes = [P, i64, i64, f32, P, P, P, P, P, i64]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on."""
    lib().oracle_set_num_threads(int(n))


def e4m3_value(byte: int) -> float:
    return lib().oracle_e4m3_value(int(byte))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def bf16_rne(f: float) -> int:
    return lib().oracle_bf16_rne(float(np.float32(f)))


def bf16_rne_array(y: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, rounded to nearest-even."""
    flat = _f32(y).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(y))


def tensor_scale(x) -> np.float32:
    a = _f32(x)
    return np.float32(lib().oracle_tensor_scale(_p(a), a.size))


def ste_backward(grad, c: float) -> np.ndarray:
    """Straight-through gradient of fake-quant, clamped to [-c, c] (fp32 result)."""
    g = _f32(grad)
    f = lib().oracle_ste_clamp
    cf = float(np.float32(c))
    return np.array([f(float(v), cf) for v in g.ravel()], dtype=np.float32).reshape(g.shape)


def scale_ema(S_prev, S_batch, m: float) -> np.ndarray:
    a, b = np.atleast_1d(_f32(S_prev)), np.atleast_1d(_f32(S_batch))
    f = lib().oracle_scale_ema
    return np.array([f(float(x), float(y), float(np.float32(m))) for x, y in zip(a, b)],
                    dtype=np.float32)


CALIB_BINS = 32768


def calib_histogram(x, hist=None) -> np.ndarray:
    """Accumulate the |x| histogram (one bin per bf16 magnitude) into hist (uint64)."""
    a = _f32(x)
    if hist is None:
        hist = np.zeros(CALIB_BINS, dtype=np.uint64)
    lib().oracle_calib_histogram(_p(a), a.size, _p(hist))
    return hist


def calib_scale(hist, fraction: float) -> np.float32:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    return np.float32(lib().oracle_calib_scale(_p(h), float(fraction)))


def max_byte(amax: float, S: float) -> int:
    return lib().oracle_max_byte(float(np.float32(amax)), float(np.float32(S)))


def e2m1_code(x: float, byte: int, S: float) -> int:
    return lib().oracle_e2m1_code(float(np.float32(x)), int(byte), float(np.float32(S)))


def dequant_value(code: int, byte: int, S: float) -> np.float32:
    return np.float32(lib().oracle_dequant_value(int(code), int(byte), float(np.float32(S))))


def scales_max(x, S) -> np.ndarray:
    a = _f32(x)
    rows, cols = a.shape
    out = np.empty((rows, cols // 16), dtype=np.uint8)
    lib().oracle_scales_max(_p(a), rows, cols, float(np.float32(S)), _p(out))
    return out


def quantize(x, S, scales) -> np.ndarray:
    a = _f32(x)
    rows, cols = a.shape
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols // 2), dtype=np.uint8)
    lib().oracle_quantize(_p(a), rows, cols, float(np.float32(S)), _p(sc), _p(out))
    return out


def dequantize(codes, scales, S, rows, cols) -> np.ndarray:
    cd = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float32)
    lib().oracle_dequantize(_p(cd), _p(sc), rows, cols, float(np.float32(S)), _p(out))
    return out


def fakequant(x, S, scales=None):
    """Returns (dequantised fp32, codes, scales); max scaling when scales is None."""
    a = _f32(x)
    rows, cols = a.shape
    sc = scales_max(a, S) if scales is None else np.ascontiguousarray(scales, dtype=np.uint8)
    cd = quantize(a, S, sc)
    return dequantize(cd, sc, S, rows, cols), cd, sc


def block_sq_error(x16, byte, S) -> np.float32:
    a = _f32(x16)
    return np.float32(lib().oracle_block_sq_error(_p(a), int(byte), float(np.float32(S))))


def scales_mse(w, S, with_obj: bool = False):
    a = _f32(w)
    rows, cols = a.shape
    out = np.empty((rows, cols // 16), dtype=np.uint8)
    obj = np.empty((rows, cols // 16), dtype=np.float32)
    lib().oracle_scales_mse(_p(a), rows, cols, float(np.float32(S)), _p(out), _p(obj))
    return (out, obj) if with_obj else out


def byte_for_divisor(amax: float, S: float, k: float) -> int:
    return int(lib().oracle_byte_for_divisor(float(np.float32(amax)), float(np.float32(S)), float(k)))


def scales_four_over_six(w, S, with_obj: bool = False):
    a = _f32(w)
    rows, cols = a.shape
    out = np.empty((rows, cols // 16), dtype=np.uint8)
    obj = np.empty((rows, cols // 16), dtype=np.float32)
    lib().oracle_scales_four_over_six(_p(a), rows, cols, float(np.float32(S)), _p(out), _p(obj))
    return (out, obj) if with_obj else out


def block_hessian(X, token_ids=None) -> np.ndarray:
    """fp64 H [cols/16, 16, 16] of X [tokens, cols] (optionally only the rows token_ids)."""
    a = _f32(X)
    tokens, cols = a.shape
    H = np.empty((cols // 16, 16, 16), dtype=np.float64)
    if token_ids is None:
        lib().oracle_block_hessian(_p(a), tokens, cols, None, 0, _p(H))
    else:
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        lib().oracle_block_hessian(_p(a), tokens, cols, _p(ids), ids.size, _p(H))
    return H


def block_lh_objective(w16, byte, S, Hb) -> float:
    a = _f32(w16)
    h = _f32(Hb)
    return lib().oracle_block_lh_objective(_p(a), int(byte), float(np.float32(S)), _p(h))


def scales_local_hessian(w, S, H, with_obj: bool = False):
    a = _f32(w)
    rows, cols = a.shape
    h = _f32(H)
    assert h.size == (cols // 16) * 256
    out = np.empty((rows, cols // 16), dtype=np.uint8)
    obj = np.empty((rows, cols // 16), dtype=np.float64)
    lib().oracle_scales_local_hessian(_p(a), rows, cols, float(np.float32(S)), _p(h),
                                      _p(out), _p(obj))
    return (out, obj) if with_obj else out


def route_groups(expert_ids, experts: int):
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    tokens, topk = ids.shape
    offsets = np.empty(experts + 1, dtype=np.int32)
    tok = np.empty(tokens * topk, dtype=np.int32)
    rc = lib().oracle_route_groups(_p(ids), tokens, topk, experts, _p(offsets), _p(tok))
    if rc != 0:
        raise ValueError("expert id out of range")
    return offsets, tok


def full_hessian(X) -> np.ndarray:
    """fp64 H [cols, cols] = X^T X of X [tokens, cols]."""
    a = _f32(X)
    tokens, cols = a.shape
    H = np.empty((cols, cols), dtype=np.float64)
    lib().oracle_full_hessian(_p(a), tokens, cols, _p(H))
    return H


def full_hessian_blas(X) -> np.ndarray:
    """The same Gram matrix through a library fp64 matmul (for inputs too large for the
    loop above; the two agree to fp64 rounding)."""
    a = _f32(X).astype(np.float64)
    return a.T @ a


def e2m1_code_d(v: float, byte: int, S: float) -> int:
    return lib().oracle_e2m1_code_d(float(v), int(byte), float(np.float32(S)))


def gptq_factor(H, damp: float = 0.01) -> np.ndarray:
    """U (upper, fp64) with U^T U = (H + damp * mean(diag H) I)^{-1}; H's lower triangle."""
    h = np.ascontiguousarray(H, dtype=np.float64)
    n = h.shape[0]
    U = np.empty((n, n), dtype=np.float64)
    rc = lib().oracle_gptq_factor(_p(h), n, float(damp), _p(U))
    if rc != 0:
        raise ValueError(f"damped H is not positive definite (column {rc - 1})")
    return U


def gptq(w, S, scales, H=None, damp: float = 0.01, U=None, return_v: bool = False, flips=None):
    """GPTQ codes [rows, cols/2] of w at the given block bytes and S (and the values each
    column was rounded from, if asked). Pass U from gptq_factor to reuse it. flips
    ([rows, k] int, -1 = unused): columns where a row takes the other rounding (the grid
    neighbour across the nearer midpoint) instead of the nearest."""
    a = _f32(w)
    rows, cols = a.shape
    if U is None:
        U = gptq_factor(H, damp)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    v = np.empty((rows, cols), dtype=np.float64) if return_v else None
    Uc = np.ascontiguousarray(U)
    if flips is None:
        lib().oracle_gptq_rows(_p(a), rows, cols, float(np.float32(S)), _p(sc), _p(Uc), _p(codes),
                               _p(v) if return_v else None)
    else:
        fl = np.ascontiguousarray(flips, dtype=np.int64)
        assert fl.ndim == 2 and fl.shape[0] == rows
        lib().oracle_gptq_rows_flip(_p(a), rows, cols, float(np.float32(S)), _p(sc), _p(Uc),
                                    _p(codes), _p(v) if return_v else None, _p(fl), fl.shape[1])
    return (codes, v) if return_v else codes
