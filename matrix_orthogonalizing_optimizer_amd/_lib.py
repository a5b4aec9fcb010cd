"""ctypes binding of libmuon.so (the C ABI in include/muon.h).

Argument marshalling only: every step of the optimizer runs in the HIP
library.  Importing works without a GPU; there is no fallback of any kind --
if the library is not built, loading raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon.so")

MO_OK, MO_EINVAL, MO_EUNSUPPORTED, MO_EWORKSPACE, MO_EHIP = 0, -1, -2, -3, -4
MO_F32, MO_BF16 = 0, 1
MO_SCALE_SHAPE, MO_SCALE_HIDDEN, MO_SCALE_UPDATE_NORM = 0, 1, 2
(MO_K_MOMENTUM, MO_K_NORM, MO_K_GRAM, MO_K_POLY, MO_K_UPDATE, MO_K_APPLY,
 MO_K_APPLY_X0, MO_K_RMS, MO_K_ADAMW, MO_K_SVD_GRAM, MO_K_SVD_REDUCE,
 MO_K_SVD_COLUMN, MO_K_SVD_EIG, MO_K_SVD_PANEL) = range(14)
KERNEL_CLASS_NAMES = ["momentum", "norm", "gram", "poly", "update", "apply",
                      "apply_x0", "rms", "adamw", "svd_gram", "svd_reduce",
                      "svd_column", "svd_eig", "svd_panel"]

STATUS_NAMES = {MO_OK: "MO_OK", MO_EINVAL: "MO_EINVAL",
                MO_EUNSUPPORTED: "MO_EUNSUPPORTED",
                MO_EWORKSPACE: "MO_EWORKSPACE", MO_EHIP: "MO_EHIP"}


class MoTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("state0", ctypes.c_void_p), ("state1", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MoMatrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MuonError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_c = ctypes
_P = _c.c_void_p
_SIGS = {
    "mo_abi_version": (_c.c_int, []),
    "mo_last_error": (_c.c_char_p, []),
    "mo_muon_workspace_size": (_c.c_int, [_c.POINTER(MoTensor), _c.c_int64, _c.c_int,
                                          _c.POINTER(_c.c_size_t), _c.POINTER(_c.c_size_t)]),
    "mo_muon_step": (_c.c_int, [_c.POINTER(MoTensor), _c.c_int64, _c.c_int, _c.c_int, _c.c_int,
                                _c.c_float, _c.c_float, _c.c_float, _c.c_int, _c.c_int,
                                _c.POINTER(_c.c_float), _c.c_float, _c.c_float,
                                _P, _P, _c.c_size_t, _P]),
    "mo_muon_step_noalloc": (_c.c_int, [_c.POINTER(MoTensor), _c.c_int64, _c.c_int, _c.c_int, _c.c_int,
                                        _c.c_float, _c.c_float, _c.c_float, _c.c_int, _c.c_int,
                                        _c.POINTER(_c.c_float), _c.c_float, _c.c_float, _P, _P]),
    "mo_muon_plan_create": (_c.c_int, [_c.POINTER(MoTensor), _c.c_int64, _c.c_int, _c.c_int,
                                       _c.c_int, _c.POINTER(_P)]),
    "mo_muon_plan_workspace_size": (_c.c_int, [_P, _c.POINTER(_c.c_size_t),
                                               _c.POINTER(_c.c_size_t)]),
    "mo_muon_plan_step": (_c.c_int, [_P, _c.c_float, _c.c_float, _c.c_float, _c.c_int, _c.c_int,
                                     _c.POINTER(_c.c_float), _c.c_float, _c.c_float,
                                     _P, _P, _c.c_size_t, _P]),
    "mo_muon_plan_set_scaling": (_c.c_int, [_P, _c.c_int, _c.c_float]),
    "mo_muon_plan_set_grads": (_c.c_int, [_P, _c.POINTER(_P), _c.c_int64, _P]),
    "mo_muon_plan_destroy": (_c.c_int, [_P]),
    "mo_adamw_step": (_c.c_int, [_c.POINTER(MoTensor), _c.c_int64, _c.c_int, _c.c_float,
                                 _c.c_float, _c.c_double, _c.c_double, _c.c_float, _c.c_int64, _P]),
    "mo_newton_schulz_workspace_size": (_c.c_int, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                                   _c.POINTER(_c.c_size_t)]),
    "mo_newton_schulz": (_c.c_int, [_P, _P, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                    _c.POINTER(_c.c_float), _c.c_float, _P, _c.c_size_t, _P]),
    "mo_svd_entropy_workspace_size": (_c.c_int, [_c.POINTER(MoMatrix), _c.c_int64,
                                                 _c.POINTER(_c.c_size_t), _c.POINTER(_c.c_size_t)]),
    "mo_svd_entropy": (_c.c_int, [_c.POINTER(MoMatrix), _c.c_int64, _c.c_int, _P, _P, _P,
                                  _c.c_size_t, _P]),
    "mo_profile_enable": (_c.c_int, [_c.c_uint]),
    "mo_profile_read": (_c.c_int, [_c.c_int, _c.POINTER(_c.c_int64), _c.POINTER(_c.c_double),
                                   _c.POINTER(_c.c_double)]),
    "mo_profile_reset": (_c.c_int, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m matrix_orthogonalizing_optimizer_amd.build` "
                "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    msg = lib().mo_last_error()
    return msg.decode() if msg else ""


def check(code: int) -> None:
    if code != MO_OK:
        raise MuonError(code, last_error())
