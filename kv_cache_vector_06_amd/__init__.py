"""TurboQuant KV-cache compression hot path for AMD MI355X (gfx950).

The computation lives in libtq.so (HIP kernels behind the C ABI of
include/tq.h); `_lib` binds it with ctypes and `torch_api` marshals PyTorch
device tensors and streams into it."""
from . import _lib  # noqa: F401
from ._lib import TQError  # noqa: F401
