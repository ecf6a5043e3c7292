"""ctypes view of libmoe.so (the C ABI declared in include/moe.h).

Loading fails loudly if the library has not been built: there is no other
implementation to fall back to.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_F16, MOE_BF16 = 0, 1, 2
MOE_IDX_U32, MOE_IDX_I32, MOE_IDX_I64 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_SHAPE",
          3: "MOE_ERR_DTYPE", 4: "MOE_ERR_UNSUPPORTED", 5: "MOE_ERR_HIP"}

# name -> (restype, argtypes); mirrors include/moe.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
SIGNATURES = {
    "moe_route": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _P, _P, _P]),
    "moe_dispatch_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "moe_dispatch": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _P, _P,
                            _P, _P, _P, _P, _SZ, _P]),
    "moe_dispatch_noalloc": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P,
                                    _P, _P, _P, _P, _P, _P]),
    "moe_experts_forward": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _P,
                                   _P, _P, _P, _P, _P]),
    "moe_experts_forward_clipped": (_INT, [_P, _INT, _I64, _I64, _I64, _I64,
                                           _P, _P, _P, _P, _F32, _F32, _P, _P,
                                           _P]),
    "moe_combine": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _INT, _P,
                           _P, _P]),
    "moe_forward_workspace_size": (_SZ, [_I64, _I64, _I64, _I64, _I64, _INT,
                                         _INT]),
    "moe_forward": (_INT, [_P, _INT, _P, _INT, _I64, _I64, _I64, _I64, _I64,
                           _INT, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_forward_clipped": (_INT, [_P, _INT, _P, _INT, _I64, _I64, _I64, _I64,
                                   _I64, _INT, _F32, _F32, _P, _P, _P, _P, _P,
                                   _SZ, _P]),
    "moe_route_sigmoid_grouped": (_INT, [_P, _INT, _I64, _I64, _P, _I64, _I64,
                                         _I64, _INT, _INT, _F32, _P, _P,
                                         _P]),
    "moe_forward_sigmoid_grouped": (_INT, [_P, _INT, _P, _INT, _P, _I64, _I64,
                                           _I64, _I64, _I64, _I64, _I64, _INT,
                                           _INT, _F32, _P, _P, _P, _P, _P,
                                           _SZ, _P]),
    "moe_selected_router_weights": (_INT, [_P, _INT, _I64, _I64, _P, _INT,
                                           _I64, _INT, _INT, _F32, _P, _P]),
    "moe_selected_router_backward": (_INT, [_P, _INT, _I64, _I64, _P, _INT,
                                            _I64, _P, _INT, _INT, _F32, _P,
                                            _P]),
    "moe_experts_forward_training": (_INT, [_P, _INT, _I64, _I64, _I64, _I64,
                                            _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P]),
    "moe_combine_backward": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P,
                                    _INT, _P, _P, _P, _P, _P]),
    "moe_experts_backward_workspace_size": (_SZ, [_I64, _I64, _I64, _I64,
                                                  _INT]),
    "moe_experts_backward": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _SZ, _P]),
    "moe_dispatch_backward": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _P,
                                     _P]),
    "moe_set_timing_events": (_INT, [_P, _INT]),
    "moe_status_string": (ctypes.c_char_p, [_INT]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


class MoeError(RuntimeError):
    """A nonzero moe_status from libmoe."""

    def __init__(self, status, detail):
        super().__init__("%s: %s" % (STATUS.get(status, status), detail))
        self.status = status


def lib():
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmoe.so is not built (expected at %s); run "
                "`python -m mixture_experts_layer_28_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status):
    if status != 0:
        detail = lib().moe_last_error().decode()
        raise MoeError(status, detail)
