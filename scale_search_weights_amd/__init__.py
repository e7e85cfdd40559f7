"""MI355X-native NVFP4 quantisation engine: fake-quantisation and block-scale selection
(max, MSE over the 126 positive E4M3 scales, Local-Hessian) in HIP kernels for gfx950
behind the C ABI of include/nvfp4.h. ``nvfp4`` is the Python binding."""
from . import nvfp4  # noqa: F401

__all__ = ["nvfp4"]
