"""MI355X-native fully-integer attention (IntAttention IndexSoftmax forward).

The compute path is the HIP library libintattn.so (C ABI declared in
include/intattn.h); the Python names below are thin ctypes marshalling over
it. The binding is imported on first use, and raises if the library has not
been built: there is no CPU fallback.
"""
__all__ = [
    "build_lut", "derive_params", "forward", "forward_debug", "strerror",
    "IntAttnError", "library_path",
]


def __getattr__(name):
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
