"""ctypes declarations of libadafuse's C ABI (include/adafuse.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libadafuse.so")

ADA_OK, ADA_EINVAL, ADA_ESHAPE, ADA_EDTYPE, ADA_EALIGN, ADA_EHIP, ADA_ENOMEM = 0, -1, -2, -3, -4, -5, -6
ADA_F32, ADA_BF16 = 0, 1

c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_float = ctypes.c_float


class AdaProj(ctypes.Structure):
    _fields_ = [
        ("w", c_void_p),
        ("w_out", c_void_p),
        ("a", c_void_p),
        ("b", c_void_p),
        ("d_out", c_int32),
        ("d_in", c_int32),
        ("ld_w", c_int64),
    ]


class AdaLoraProj(ctypes.Structure):
    _fields_ = [
        ("w", c_void_p),
        ("a", c_void_p),
        ("b", c_void_p),
        ("x", c_void_p),
        ("y", c_void_p),
        ("d_out", c_int32),
        ("d_in", c_int32),
        ("ld_w", c_int64),
    ]


class AdaGemvProj(ctypes.Structure):
    _fields_ = [
        ("w", c_void_p),
        ("x", c_void_p),
        ("y", c_void_p),
        ("d_out", c_int32),
        ("d_in", c_int32),
        ("ld_w", c_int64),
    ]


_SIGNATURES = {
    "ada_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ada_model_create": (ctypes.c_int, [ctypes.POINTER(AdaProj), c_int32, c_int32, c_int32, c_int32,
                                        c_void_p, ctypes.POINTER(c_void_p)]),
    "ada_model_destroy": (None, [c_void_p]),
    "ada_model_tiles": (c_int64, [c_void_p]),
    "ada_model_device_bytes": (c_int64, [c_void_p]),
    "ada_pregate": (ctypes.c_int, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                   c_void_p, c_void_p, c_void_p]),
    "ada_merge": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p]),
    "ada_unmerge": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p]),
    "ada_switch": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                  c_float, c_void_p]),
    "ada_decode_gemv": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int64, c_void_p, c_void_p, c_int32,
                                       c_void_p]),
    "ada_decode_gemv_layer": (ctypes.c_int, [ctypes.POINTER(AdaGemvProj), c_int32, c_int32, c_void_p]),
    "ada_lora_apply": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int64, c_void_p, c_void_p, c_int32,
                                      c_int32, c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p,
                                      c_void_p, c_int64, c_int32, c_void_p]),
    "ada_lora_layer": (ctypes.c_int, [ctypes.POINTER(AdaLoraProj), c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                      c_int32, c_float, c_void_p, c_int64, c_int32, c_void_p]),
    "ada_lora_layer_static": (ctypes.c_int, [ctypes.POINTER(AdaLoraProj), c_int32, c_int32, c_int32, c_void_p,
                                             c_void_p, c_int32, c_float, c_int32, c_void_p]),
    "ada_lora_batch": (ctypes.c_int, [ctypes.POINTER(AdaLoraProj), c_int32, c_int32, c_int32, c_int32, c_void_p,
                                      c_void_p, c_int32, c_float, c_void_p, c_int64, c_int32, c_void_p]),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """Load libadafuse.so (built in-tree).  There is no fallback: a missing library
    is an error."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python weight_merge_amd/build.py` first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def declared_functions(header: str) -> list[str]:
    """Function names a C header declares (for the export check)."""
    import re

    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ada_[a-z_]+)\s*\(", text)))
