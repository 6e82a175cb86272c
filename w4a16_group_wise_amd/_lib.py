"""ctypes loader for libw4a16q.so and the exported C symbols (see include/w4a16q.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a16q.so")

W4Q_GROUP = 32
W4Q_OK = 0
W4Q_EINVAL = -1
W4Q_ESHAPE = -2
W4Q_EALIGN = -3
W4Q_EUNSUPPORTED = -4
W4Q_EHIP = -5

# every function the header declares, with its ctypes signature
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
class GemvProblem(ctypes.Structure):
    """w4q_gemv_problem of w4a16q.h"""
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scale_f16", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64)]


class AdamParams(ctypes.Structure):
    """w4q_adam_params of w4a16q.h"""
    _fields_ = [(n, ctypes.c_float) for n in ("lr_w", "lr_s", "beta1", "beta2", "eps", "weight_decay",
                                              "bias_c1", "bias_c2", "scale_min")]


SIGNATURES = {
    "w4q_status_string": (ctypes.c_char_p, [_INT]),
    "w4q_version": (_INT, []),
    "quant_hessian": (_INT, [_P, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "quant_hessian_workspace_size": (_INT, [_I64, _I64, _P]),
    "quant_scale_search": (_INT, [_P, _I64, _I64, _P, _I64, _P, _INT, _P, _P, _P, _P, _P]),
    "quant_pack": (_INT, [_P, _P, _I64, _I64, _P, _P, _P]),
    "lsq_fwd": (_INT, [_P, _P, _I64, _I64, _P, _P]),
    "lsq_bwd": (_INT, [_P, _P, _P, _I64, _I64, _F, _P, _P, _P, _P]),
    "lsq_adam_step": (_INT, [_P, _P, _P, _I64, _I64, _F, _P, _P, _P, _P, _P, _P, _P, _P]),
    "w4a16_gemm": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "w4a16_gemm_workspace_size": (_INT, [_I64, _I64, _I64, _P]),
    "w4a16_gemm_dq": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "w4a16_gemm_dq_workspace_size": (_INT, [_I64, _I64, _I64, _P]),
    "w4a16_gemm_dq_noalloc": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _INT, _P]),
    "w4a16_gemv_grouped": (_INT, [_P, _INT, _INT, _P]),
    "quant_scale_search_pc": (_INT, [_P, _I64, _I64, _P, _I64, _P, _INT, _P, _P, _P, _P, _P]),
    "per_channel_workspace_size": (_INT, [_I64, _I64, _I64, _P]),
    "quant_pack_pc": (_INT, [_P, _P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "lsq_fwd_pc": (_INT, [_P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "lsq_bwd_pc": (_INT, [_P, _P, _P, _I64, _I64, _F, _P, _P, _P, _P, _SZ, _P]),
    "w4a16_gemm_pc": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _INT, _INT, _P, _SZ, _P]),
    "joint_workspace_size": (_INT, [_I64, _I64, _P]),
    "quant_joint_objective": (_INT, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "quant_joint_refine": (_INT, [_P, _I64, _I64, _P, _I64, _P, _INT, _P, _P, _INT, _P, _P, _P, _P, _SZ, _P]),
    "gptq_workspace_size": (_INT, [_I64, _I64, _P]),
    "quant_gptq": (_INT, [_P, _I64, _I64, _P, _I64, _P, _F, _P, _P, _P, _SZ, _P]),
    "w4q_probe_read": (_INT, [_P, _I64, _INT, _P, _P]),
    "w4q_probe_mfma_bf16": (_INT, [_P, _I64, _P, _P]),
    "w4q_probe_mfma_f64": (_INT, [_P, _I64, _P, _P]),
}
W4Q_PROBE_SINK_WORDS = 65536


class W4QError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4a16q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m w4a16_group_wise_amd.build` "
                "(hipcc, gfx950).  There is no fallback implementation.")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().w4q_status_string(int(status)).decode()


def version() -> int:
    return int(lib().w4q_version())


def check(fn: str, status: int) -> None:
    if status != W4Q_OK:
        raise W4QError(fn, status)
