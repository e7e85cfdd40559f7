"""Python binding of libnvfp4 (ctypes): argument marshalling only.

Every function takes and returns torch tensors on the GPU; the computation runs in the
HIP kernels behind the C ABI declared in ``include/nvfp4.h``. torch supplies device memory
(outputs and workspaces are allocated with torch) and the current stream. There is no
CPU fallback: if the library has not been built, loading it raises.

Shapes: element tensors are [rows, cols] or [batch, rows, cols] (cols % 16 == 0), bf16 or
fp32. Tensor scales S are fp32 [batch] on the same device. Block scales are uint8
[batch, rows, cols/16] (squeezed like the input), packed codes uint8 [..., cols/2].
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "nvfp4.h")

DTYPE_F32 = 0
DTYPE_BF16 = 1
STATIC_SCRATCH_BYTES = 64 << 20  # NVFP4_STATIC_SCRATCH_BYTES: nvfp4_block_hessian_noalloc's scratch

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [_I]),
    "nvfp4_version": (_I, []),
    "nvfp4_global_scale": (_I, [_P, _I, _I64, _I64, _P, _P]),
    "nvfp4_global_scale_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_global_scale_ws": (_I, [_P, _I, _I64, _I64, _P, _P, _SZ, _P]),
    "nvfp4_scale_search_max": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P]),
    "nvfp4_scale_search_mse": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_scale_search_four_over_six": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_calib_histogram": (_I, [_P, _I, _I64, _P, _P]),
    "nvfp4_ste_backward": (_I, [_P, _I, _I64, ctypes.c_float, _P, _P]),
    "nvfp4_scale_ema": (_I, [_P, _P, _I64, ctypes.c_float, _P]),
    "nvfp4_calib_scale": (_I, [_P, ctypes.c_double, _P, _P]),
    "nvfp4_block_hessian_workspace_size": (_SZ, [_I64, _I64, _I64, _I64]),
    "nvfp4_block_hessian": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _I64, _P, _I, _P, _SZ, _P]),
    "nvfp4_block_hessian_noalloc": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _I64, _P, _I, _P]),
    "nvfp4_scale_search_local_hessian": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_quantize": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_dequantize": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "nvfp4_fakequant": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "nvfp4_full_hessian_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_full_hessian": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "nvfp4_gptq_factor_workspace_size": (_SZ, [_I64]),
    "nvfp4_gptq_factor": (_I, [_P, _I64, ctypes.c_double, _P, _P, _P, _SZ, _P]),
    "nvfp4_gptq_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_gptq": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_debug_nonfinite": (_I, [_P, _P]),
    "nvfp4_search_stats_enable": (_I, [_I]),
    "nvfp4_search_stats_read": (_I, [_P, _P]),
    "nvfp4_route_groups_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_route_groups": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def lib():
    """Load libnvfp4.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m scale_search_weights_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Names of every entry point declared in include/nvfp4.h."""
    with open(HEADER) as f:
        txt = f.read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]*?\b(nvfp4_\w+)\s*\(", txt)))


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(int(status)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise NVFP4Error(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _shape3(t: torch.Tensor):
    if t.dim() == 2:
        return 1, t.shape[0], t.shape[1]
    if t.dim() == 3:
        return t.shape[0], t.shape[1], t.shape[2]
    raise ValueError("expected a [rows, cols] or [batch, rows, cols] tensor")


def _out_shape(t: torch.Tensor, last: int):
    return tuple(t.shape[:-1]) + (last,)


def _need(t: torch.Tensor, name: str):
    """The call's main tensor: a contiguous GPU tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _arg(t, name: str, like: torch.Tensor, dtype=None, numel: int | None = None,
         min_numel: int | None = None):
    """Another tensor argument, checked before anything is launched: a contiguous GPU
    tensor on the main tensor's device, of the expected dtype and element count (the kernels
    read and write exactly that many elements)."""
    _need(t, name)
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, got {t.numel()}")
    return t


def _scale_arg(S, like: torch.Tensor, batch: int):
    return _arg(S, "S", like, torch.float32, numel=batch)


def _bytes_arg(scales, like: torch.Tensor, n: int):
    return _arg(scales, "scales", like, torch.uint8, numel=n)


def _elem(x: torch.Tensor, name: str):
    """An element tensor (bf16 or fp32) as the main argument."""
    _need(x, name)
    _dt(x)


def global_scale_workspace_size(batch: int, n: int) -> int:
    return int(lib().nvfp4_global_scale_workspace_size(batch, n))


def global_scale(x: torch.Tensor, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """S[b] = fp32(amax(|x[b]|) / 2688) per batch entry (2-D input: one scale).

    With `workspace` (uint8 on x's device, at least global_scale_workspace_size bytes; no
    initialisation needed) the scale takes two launches instead of three."""
    _elem(x, "x")
    batch = x.shape[0] if x.dim() == 3 else 1
    n = x.numel() // max(batch, 1)
    S = torch.empty(batch, dtype=torch.float32, device=x.device)
    if workspace is None:
        _check(lib().nvfp4_global_scale(_ptr(x), _dt(x), batch, n, _ptr(S), _stream()),
               "nvfp4_global_scale")
        return S
    need = global_scale_workspace_size(batch, n)
    ws = _arg(workspace, "workspace", x, torch.uint8, min_numel=need)
    _check(lib().nvfp4_global_scale_ws(_ptr(x), _dt(x), batch, n, _ptr(S), _ptr(ws), ws.numel(),
                                       _stream()), "nvfp4_global_scale_ws")
    return S


def scale_search_max(w: torch.Tensor, S: torch.Tensor) -> torch.Tensor:
    _elem(w, "w")
    b, r, c = _shape3(w)
    _scale_arg(S, w, b)
    sc = torch.empty(_out_shape(w, c // 16), dtype=torch.uint8, device=w.device)
    _check(lib().nvfp4_scale_search_max(_ptr(w), _dt(w), b, r, c, _ptr(S), _ptr(sc), _stream()),
           "nvfp4_scale_search_max")
    return sc


def scale_search_mse(w: torch.Tensor, S: torch.Tensor, return_obj: bool = False):
    _elem(w, "w")
    b, r, c = _shape3(w)
    _scale_arg(S, w, b)
    sc = torch.empty(_out_shape(w, c // 16), dtype=torch.uint8, device=w.device)
    obj = torch.empty(_out_shape(w, c // 16), dtype=torch.float32, device=w.device) if return_obj else None
    _check(lib().nvfp4_scale_search_mse(_ptr(w), _dt(w), b, r, c, _ptr(S), _ptr(sc), _ptr(obj),
                                        _stream()), "nvfp4_scale_search_mse")
    return (sc, obj) if return_obj else sc


def scale_search_four_over_six(w: torch.Tensor, S: torch.Tensor, return_obj: bool = False):
    _elem(w, "w")
    b, r, c = _shape3(w)
    _scale_arg(S, w, b)
    sc = torch.empty(_out_shape(w, c // 16), dtype=torch.uint8, device=w.device)
    obj = torch.empty(_out_shape(w, c // 16), dtype=torch.float32, device=w.device) if return_obj else None
    _check(lib().nvfp4_scale_search_four_over_six(_ptr(w), _dt(w), b, r, c, _ptr(S), _ptr(sc),
                                                  _ptr(obj), _stream()),
           "nvfp4_scale_search_four_over_six")
    return (sc, obj) if return_obj else sc


def ste_backward(grad: torch.Tensor, clip: float = float("inf"),
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Straight-through gradient of fake-quant: grad clamped to [-clip, clip]."""
    _elem(grad, "grad")
    if out is None:
        out = torch.empty_like(grad)
    else:
        _arg(out, "out", grad, grad.dtype, numel=grad.numel())
    _check(lib().nvfp4_ste_backward(_ptr(grad), _dt(grad), grad.numel(), float(clip), _ptr(out),
                                    _stream()), "nvfp4_ste_backward")
    return out


def scale_ema(S: torch.Tensor, S_batch: torch.Tensor, momentum: float) -> torch.Tensor:
    """In place: S = momentum * S + (1 - momentum) * S_batch (fixed fp32 order)."""
    _need(S, "S")
    _arg(S, "S", S, torch.float32)
    _arg(S_batch, "S_batch", S, torch.float32, numel=S.numel())
    _check(lib().nvfp4_scale_ema(_ptr(S), _ptr(S_batch), S.numel(), float(momentum), _stream()),
           "nvfp4_scale_ema")
    return S


CALIB_BINS = 32768


def calib_histogram(x: torch.Tensor, hist: torch.Tensor | None = None) -> torch.Tensor:
    """Add |x| to a calibration histogram ([CALIB_BINS] int64 on x's device; new if None)."""
    _elem(x, "x")
    if hist is None:
        hist = torch.zeros(CALIB_BINS, dtype=torch.int64, device=x.device)
    else:
        _arg(hist, "hist", x, torch.int64, numel=CALIB_BINS)
    _check(lib().nvfp4_calib_histogram(_ptr(x), _dt(x), x.numel(), _ptr(hist), _stream()),
           "nvfp4_calib_histogram")
    return hist


def calib_scale(hist: torch.Tensor, fraction: float) -> torch.Tensor:
    """Tensor scale S [1] from the clip value at `fraction` of the histogram's values."""
    _need(hist, "hist")
    _arg(hist, "hist", hist, torch.int64, numel=CALIB_BINS)
    S = torch.empty(1, dtype=torch.float32, device=hist.device)
    _check(lib().nvfp4_calib_scale(_ptr(hist), float(fraction), _ptr(S), _stream()),
           "nvfp4_calib_scale")
    return S


def block_hessian_workspace_size(tokens: int, cols: int, groups: int = 1, n_ids: int = 0) -> int:
    return int(lib().nvfp4_block_hessian_workspace_size(tokens, cols, groups, n_ids))


def _workspace(need: int, like: torch.Tensor, workspace: torch.Tensor | None) -> torch.Tensor:
    """The caller's workspace (checked: uint8 on the main tensor's device, large enough),
    or a new one."""
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    return _arg(workspace, "workspace", like, torch.uint8, min_numel=need)


def block_hessian(x: torch.Tensor, group_offsets: torch.Tensor | None = None,
                  token_ids: torch.Tensor | None = None, H: torch.Tensor | None = None,
                  accumulate: bool = False, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Block-diagonal Gram matrices of x [tokens, cols]: [cols/16, 16, 16] (dense) or
    [groups, cols/16, 16, 16] (grouped by group_offsets / token_ids)."""
    _elem(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [tokens, cols]")
    tokens, cols = x.shape
    grouped = group_offsets is not None or token_ids is not None
    if grouped:
        if group_offsets is None or token_ids is None:
            raise ValueError("the grouped form needs both group_offsets and token_ids")
        _arg(group_offsets, "group_offsets", x, torch.int32)
        _arg(token_ids, "token_ids", x, torch.int32)
        if group_offsets.numel() < 1:
            raise ValueError("group_offsets must have groups + 1 entries")
    groups = group_offsets.numel() - 1 if grouped else 1
    n_ids = token_ids.numel() if grouped else 0
    shape = (groups, cols // 16, 16, 16) if grouped else (cols // 16, 16, 16)
    if H is None:
        if accumulate:
            raise ValueError("accumulate needs an existing H")
        H = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        _arg(H, "H", x, torch.float32, numel=groups * (cols // 16) * 256)
    need = block_hessian_workspace_size(tokens, cols, groups, n_ids)
    workspace = _workspace(need, x, workspace)
    _check(lib().nvfp4_block_hessian(_ptr(x), _dt(x), tokens, cols, groups, _ptr(group_offsets),
                                     _ptr(token_ids), n_ids, _ptr(H), int(accumulate),
                                     _ptr(workspace), workspace.numel(), _stream()),
           "nvfp4_block_hessian")
    return H


def debug_nonfinite() -> bool:
    """With NVFP4_DEBUG_CHECKS=1: whether any input since the last call held NaN or inf
    (synchronises the current stream; clears the flag)."""
    flag = ctypes.c_int32(0)
    _check(lib().nvfp4_debug_nonfinite(ctypes.byref(flag), _stream()), "nvfp4_debug_nonfinite")
    return bool(flag.value)


STATS_NAMES = ("mse_blocks", "mse_evals", "lh_pairs", "lh_zero_h", "lh_rel", "lh_abs",
               "lh_noprune", "lh_rescan", "lh_two", "lh_screened", "lh_exact")
STATS_N = 16


def search_stats_enable(on: bool) -> None:
    """Switch the searches' work counters on or off (process-wide; off by default)."""
    _check(lib().nvfp4_search_stats_enable(int(bool(on))), "nvfp4_search_stats_enable")


def search_stats_read() -> dict:
    """The searches' work counters since the last read, by name (synchronises the current
    stream; clears them)."""
    out = (ctypes.c_int64 * STATS_N)()
    _check(lib().nvfp4_search_stats_read(out, _stream()), "nvfp4_search_stats_read")
    return {n: int(out[i]) for i, n in enumerate(STATS_NAMES)}


def full_hessian(x: torch.Tensor, H: torch.Tensor | None = None, accumulate: bool = False,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Full Gram matrix X^T X [cols, cols] (fp32) of x [tokens, cols]."""
    _elem(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [tokens, cols]")
    tokens, cols = x.shape
    if H is None:
        if accumulate:
            raise ValueError("accumulate needs an existing H")
        H = torch.empty(cols, cols, dtype=torch.float32, device=x.device)
    else:
        _arg(H, "H", x, torch.float32, numel=cols * cols)
    need = int(lib().nvfp4_full_hessian_workspace_size(tokens, cols))
    workspace = _workspace(need, x, workspace)
    _check(lib().nvfp4_full_hessian(_ptr(x), _dt(x), tokens, cols, _ptr(H), int(accumulate),
                                    _ptr(workspace), workspace.numel(), _stream()),
           "nvfp4_full_hessian")
    return H


def gptq_factor(H: torch.Tensor, damp: float = 0.01, workspace: torch.Tensor | None = None):
    """GPTQ's factor of H [cols, cols] fp32: (U [cols, cols] fp64 upper with
    U^T U = (H + damp * mean(diag H) I)^-1, status [1] int32: 0 when H was positive definite
    after damping)."""
    _need(H, "H")
    if H.dim() != 2 or H.shape[0] != H.shape[1] or H.dtype != torch.float32:
        raise ValueError("H must be a square fp32 [cols, cols] tensor")
    cols = H.shape[0]
    U = torch.empty(cols, cols, dtype=torch.float64, device=H.device)
    status = torch.empty(1, dtype=torch.int32, device=H.device)
    need = int(lib().nvfp4_gptq_factor_workspace_size(cols))
    workspace = _workspace(need, H, workspace)
    _check(lib().nvfp4_gptq_factor(_ptr(H), cols, float(damp), _ptr(U), _ptr(status),
                                   _ptr(workspace), workspace.numel(), _stream()),
           "nvfp4_gptq_factor")
    return U, status


def gptq(w: torch.Tensor, S: torch.Tensor, scales: torch.Tensor, U: torch.Tensor,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """GPTQ codes [rows, cols/2] of w [rows, cols] at the given block bytes, S and factor U."""
    _elem(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [rows, cols]")
    rows, cols = w.shape
    _scale_arg(S, w, 1)
    _bytes_arg(scales, w, rows * (cols // 16))
    _arg(U, "U", w, torch.float64, numel=cols * cols)
    codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=w.device)
    need = int(lib().nvfp4_gptq_workspace_size(rows, cols))
    workspace = _workspace(need, w, workspace)
    _check(lib().nvfp4_gptq(_ptr(w), _dt(w), rows, cols, _ptr(S), _ptr(scales), _ptr(U),
                            _ptr(codes), _ptr(workspace), workspace.numel(), _stream()),
           "nvfp4_gptq")
    return codes


def scale_search_local_hessian(w: torch.Tensor, S: torch.Tensor, H: torch.Tensor,
                               return_obj: bool = False):
    _elem(w, "w")
    b, r, c = _shape3(w)
    _scale_arg(S, w, b)
    _arg(H, "H", w, torch.float32, numel=b * (c // 16) * 256)
    sc = torch.empty(_out_shape(w, c // 16), dtype=torch.uint8, device=w.device)
    obj = torch.empty(_out_shape(w, c // 16), dtype=torch.float64, device=w.device) if return_obj else None
    _check(lib().nvfp4_scale_search_local_hessian(_ptr(w), _dt(w), b, r, c, _ptr(S), _ptr(H),
                                                  _ptr(sc), _ptr(obj), _stream()),
           "nvfp4_scale_search_local_hessian")
    return (sc, obj) if return_obj else sc


def quantize(x: torch.Tensor, S: torch.Tensor, scales: torch.Tensor | None = None):
    """Returns (codes, scales): packed E2M1 codes and the block bytes used."""
    _elem(x, "x")
    b, r, c = _shape3(x)
    _scale_arg(S, x, b)
    if scales is not None:
        _bytes_arg(scales, x, b * r * (c // 16))
    codes = torch.empty(_out_shape(x, c // 2), dtype=torch.uint8, device=x.device)
    so = None
    if scales is None:
        so = torch.empty(_out_shape(x, c // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize(_ptr(x), _dt(x), b, r, c, _ptr(S), _ptr(scales), _ptr(codes),
                                _ptr(so), _stream()), "nvfp4_quantize")
    return codes, (scales if so is None else so)


def dequantize(codes: torch.Tensor, scales: torch.Tensor, S: torch.Tensor,
               out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    _need(codes, "codes")
    if codes.dtype != torch.uint8 or codes.dim() not in (2, 3):
        raise ValueError("codes must be uint8 [rows, cols/2] or [batch, rows, cols/2]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported dtype {out_dtype} (bf16 or fp32)")
    b, r, half = _shape3(codes)
    c = 2 * half
    _bytes_arg(scales, codes, b * r * (c // 16))
    _scale_arg(S, codes, b)
    y = torch.empty(_out_shape(codes, c), dtype=out_dtype, device=codes.device)
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(S), b, r, c, _ptr(y), _dt(y),
                                  _stream()), "nvfp4_dequantize")
    return y


def fakequant(x: torch.Tensor, S: torch.Tensor, scales: torch.Tensor | None = None,
              return_codes: bool = False, out: torch.Tensor | None = None):
    """Quantise -> dequantise in one pass. Returns y (and codes, scales if asked)."""
    _elem(x, "x")
    b, r, c = _shape3(x)
    _scale_arg(S, x, b)
    if scales is not None:
        _bytes_arg(scales, x, b * r * (c // 16))
    if out is None:
        y = torch.empty_like(x)
    else:
        y = _arg(out, "out", x, x.dtype, numel=x.numel())
    codes = so = None
    if return_codes:
        codes = torch.empty(_out_shape(x, c // 2), dtype=torch.uint8, device=x.device)
        if scales is None:
            so = torch.empty(_out_shape(x, c // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_fakequant(_ptr(x), _dt(x), b, r, c, _ptr(S), _ptr(scales), _ptr(y),
                                 _ptr(codes), _ptr(so), _stream()), "nvfp4_fakequant")
    if return_codes:
        return y, codes, (scales if so is None else so)
    return y


def route_groups(expert_ids: torch.Tensor, experts: int):
    """Per-expert token lists from a [tokens, topk] routing table: (offsets, token_ids)."""
    _need(expert_ids, "expert_ids")
    if expert_ids.dtype != torch.int32 or expert_ids.dim() != 2:
        raise ValueError("expert_ids must be int32 [tokens, topk]")
    tokens, topk = expert_ids.shape
    offsets = torch.empty(experts + 1, dtype=torch.int32, device=expert_ids.device)
    tok = torch.empty(tokens * topk, dtype=torch.int32, device=expert_ids.device)
    need = int(lib().nvfp4_route_groups_workspace_size(tokens, topk, experts))
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=expert_ids.device)
    _check(lib().nvfp4_route_groups(_ptr(expert_ids), tokens, topk, experts, _ptr(offsets),
                                    _ptr(tok), _ptr(ws), ws.numel(), _stream()),
           "nvfp4_route_groups")
    return offsets, tok
