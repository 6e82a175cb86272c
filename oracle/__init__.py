"""CPU oracle of the W4A16 group-wise quantization core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``w4a16_group_wise_amd``) never touches it and
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain C, fp64), compiled with
gcc into ``liboracle.so``; this module only marshals numpy arrays.

Functions and the passages they follow (page titles and sections):
  hessian, hessian_entries  -- "Opt.Gear-QAT: Preserving On-Device Performance with QAT",
                               section 2 (second-order view, H = X^T X).
  code, candidate           -- model card "Opt.Gear-1B-qat-int4-per-channel-unquantized",
                               "Quantization Configuration" (symmetric, zero-point 0) and the
                               blog's "Quantization parameters" (group 32).
  scale_search(_groups)     -- model card "Quantization Configuration" objective, per group.
  pack                      -- model card "QAT Highlights" / "Quickstart"; blog "Conclusion".
  lsq_fwd, lsq_bwd          -- blog section 3 (LSQ forward, STE, normalised scale gradient).
  gemm_cols                 -- model card intro (W4A16: INT4 weights, 16-bit activations).
  group=d_in in pack / lsq_* / gemm_cols, scale_search_pc
                            -- model card intro and "Quickstart" (per-channel symmetric INT4:
                               one scale per output row, the whole row as the group).
  joint_objective, joint_refine
                            -- model card "Quantization Configuration" objective over a whole
                               row with the full H, and coordinate descent over the row's groups.
  gptq                      -- the published GPTQ algorithm (static groups on the group-32
                               grid), which the blog's section 2 names as its starting point.
  lsq_adam_step             -- blog section 3 / model card "QAT Highlights" (weights and steps
                               learned together), with Adam as the optimiser.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (OpenMP across independent units, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f16_to_f64.restype = ctypes.c_double
        lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_code.restype = ctypes.c_int
        lib.orc_code.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.orc_candidate.restype = ctypes.c_float
        lib.orc_candidate.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.orc_unpack.restype = ctypes.c_int
        lib.orc_unpack.argtypes = [P, I]
        lib.orc_hessian.argtypes = [P, I, I, P]
        lib.orc_hessian_entries.argtypes = [P, I, I, P, I, P]
        lib.orc_scale_search.argtypes = [P, I, I, P, I, P, ctypes.c_int, P, P, P, P]
        lib.orc_scale_search_groups.argtypes = [P, I, P, I, P, ctypes.c_int, P, P, I, P, P, P, P]
        lib.orc_pack.argtypes = [P, P, I, I, P, P]
        lib.orc_lsq_fwd.argtypes = [P, P, I, I, P]
        lib.orc_lsq_bwd.argtypes = [P, P, P, I, I, ctypes.c_double, P, P, P]
        lib.orc_gemm_cols_mode.argtypes = [P, I, P, P, I, P, I, ctypes.c_int, P, P]
        lib.orc_scale_search_pc.argtypes = [P, I, P, I, P, ctypes.c_int, P, I, P, P, P, P]
        lib.orc_pack_g.argtypes = [P, P, I, I, I, P, P]
        lib.orc_lsq_fwd_g.argtypes = [P, P, I, I, I, P]
        lib.orc_lsq_bwd_g.argtypes = [P, P, P, I, I, I, ctypes.c_double, P, P, P]
        lib.orc_gemm_cols_g.argtypes = [P, I, P, P, I, I, P, I, ctypes.c_int, P, P]
        lib.orc_joint_objective.argtypes = [P, P, I, P, I, P, I, P]
        lib.orc_joint_refine.argtypes = [P, I, P, I, P, ctypes.c_int, P, I, ctypes.c_int, P, P, P, P, P]
        lib.orc_gptq.restype = ctypes.c_int
        lib.orc_gptq.argtypes = [P, I, P, I, P, ctypes.c_double, P, I, P, P, P]
        lib.orc_lsq_adam_step.argtypes = [P, P, P, I, I, ctypes.c_double, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_round_bf16.restype = ctypes.c_double
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return int(_L().orc_threads())


# -------------------------------------------------------------- scalar helpers (for pins)
def f32_to_f16(v: float) -> int:
    return int(_L().orc_f32_to_f16(float(np.float32(v))))


def f16_to_f64(bits: int) -> float:
    return float(_L().orc_f16_to_f64(int(bits)))


def bf16_to_f64(bits: int) -> float:
    return float(_L().orc_bf16_to_f64(int(bits)))


def code(w: float, d: float) -> int:
    return int(_L().orc_code(float(w), float(d)))


def candidate(amax: float, alpha: float) -> float:
    return float(np.float32(_L().orc_candidate(float(np.float32(amax)), float(np.float32(alpha)))))


def round_bf16(v: float) -> float:
    return float(_L().orc_round_bf16(float(v)))


def unpack(packed_row: np.ndarray, k: int) -> int:
    row = _c(packed_row, np.uint8)
    return int(_L().orc_unpack(_p(row), int(k)))


# ----------------------------------------------------------------------- array calls
def hessian(x_bf16: np.ndarray) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    n, d = x.shape
    h = np.empty((d, d), dtype=np.float64)
    _L().orc_hessian(_p(x), n, d, _p(h))
    return h


def hessian_entries(x_bf16: np.ndarray, ij: np.ndarray) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    n, d = x.shape
    ij = _c(ij, np.int64).reshape(-1, 2)
    out = np.empty(ij.shape[0], dtype=np.float64)
    _L().orc_hessian_entries(_p(x), n, d, _p(ij), ij.shape[0], _p(out))
    return out


def scale_search(w: np.ndarray, h: np.ndarray, alpha: np.ndarray, with_all: bool = False):
    """-> (scale f32 [d_out][G], idx u8, obj f64 [d_out][G], obj_all f64 [d_out][G][K] | None)."""
    w = _c(w, np.float32)
    h = _c(h, np.float32)
    alpha = _c(alpha, np.float32)
    d_out, d_in = w.shape
    G, K = d_in // 32, alpha.shape[0]
    scale = np.empty((d_out, G), np.float32)
    idx = np.empty((d_out, G), np.uint8)
    obj = np.empty((d_out, G), np.float64)
    obj_all = np.empty((d_out, G, K), np.float64) if with_all else None
    _L().orc_scale_search(_p(w), d_out, d_in, _p(h), h.shape[1], _p(alpha), K, _p(scale),
                          _p(idx), _p(obj), _p(obj_all))
    return scale, idx, obj, obj_all


def scale_search_groups(w: np.ndarray, h: np.ndarray, alpha: np.ndarray, rows: np.ndarray,
                        groups: np.ndarray, with_all: bool = False):
    w = _c(w, np.float32)
    h = _c(h, np.float32)
    alpha = _c(alpha, np.float32)
    rows = _c(rows, np.int64)
    groups = _c(groups, np.int64)
    cnt, K = rows.shape[0], alpha.shape[0]
    scale = np.empty(cnt, np.float32)
    idx = np.empty(cnt, np.uint8)
    obj = np.empty(cnt, np.float64)
    obj_all = np.empty((cnt, K), np.float64) if with_all else None
    _L().orc_scale_search_groups(_p(w), w.shape[1], _p(h), h.shape[1], _p(alpha), K, _p(rows),
                                 _p(groups), cnt, _p(scale), _p(idx), _p(obj), _p(obj_all))
    return scale, idx, obj, obj_all


def pack(w: np.ndarray, scale: np.ndarray, group: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    """group = 32 ([blog] grid) or d_in (one scale per row)."""
    w = _c(w, np.float32)
    scale = _c(scale, np.float32)
    d_out, d_in = w.shape
    packed = np.empty((d_out, d_in // 2), np.uint8)
    s16 = np.empty((d_out, d_in // group), np.uint16)
    _L().orc_pack_g(_p(w), _p(scale), d_out, d_in, group, _p(packed), _p(s16))
    return packed, s16


def lsq_fwd(w: np.ndarray, scale: np.ndarray, group: int = 32) -> np.ndarray:
    w = _c(w, np.float32)
    scale = _c(scale, np.float32)
    out = np.empty_like(w)
    _L().orc_lsq_fwd_g(_p(w), _p(scale), w.shape[0], w.shape[1], group, _p(out))
    return out


def lsq_bwd(w: np.ndarray, scale: np.ndarray, g: np.ndarray, gs: float, group: int = 32):
    """-> (grad_w f32, grad_scale f64 [d_out][d_in / group], w_hat f32)."""
    w = _c(w, np.float32)
    scale = _c(scale, np.float32)
    g = _c(g, np.float32)
    gw = np.empty_like(w)
    gsc = np.empty((w.shape[0], w.shape[1] // group), np.float64)
    wh = np.empty_like(w)
    _L().orc_lsq_bwd_g(_p(w), _p(scale), _p(g), w.shape[0], w.shape[1], group, float(gs), _p(gw),
                       _p(gsc), _p(wh))
    return gw, gsc, wh


def gemm_cols(x_bf16: np.ndarray, packed: np.ndarray, s16: np.ndarray,
              cols: Optional[np.ndarray] = None, dequant_bf16: bool = False, group: int = 32):
    """-> (y f64 [m][len(cols)], yabs f64 [m][len(cols)]) with yabs = sum |x * w_hat|.
    w_hat = s16 * q exactly, or bf16_RNE(s16 * q) with dequant_bf16; s16 holds d_in / group
    scales per row."""
    x = _c(x_bf16, np.uint16)
    packed = _c(packed, np.uint8)
    s16 = _c(s16, np.uint16)
    m, d_in = x.shape
    if cols is None:
        cols = np.arange(packed.shape[0])
    cols = _c(cols, np.int64)
    y = np.empty((m, cols.shape[0]), np.float64)
    ya = np.empty_like(y)
    _L().orc_gemm_cols_g(_p(x), m, _p(packed), _p(s16), d_in, group, _p(cols), cols.shape[0],
                         1 if dequant_bf16 else 0, _p(y), _p(ya))
    return y, ya


def scale_search_pc(w: np.ndarray, h: np.ndarray, alpha: np.ndarray, rows: Optional[np.ndarray] = None,
                    with_all: bool = False):
    """Per-channel search (whole row, full H) on rows (all by default).
    -> (scale f32 [cnt], idx u8 [cnt], obj f64 [cnt], obj_all f64 [cnt][K] | None)."""
    w = _c(w, np.float32)
    h = _c(h, np.float32)
    alpha = _c(alpha, np.float32)
    rows = _c(np.arange(w.shape[0]) if rows is None else rows, np.int64)
    cnt, K = rows.shape[0], alpha.shape[0]
    scale = np.empty(cnt, np.float32)
    idx = np.empty(cnt, np.uint8)
    obj = np.empty(cnt, np.float64)
    obj_all = np.empty((cnt, K), np.float64) if with_all else None
    _L().orc_scale_search_pc(_p(w), w.shape[1], _p(h), h.shape[1], _p(alpha), K, _p(rows), cnt,
                             _p(scale), _p(idx), _p(obj), _p(obj_all))
    return scale, idx, obj, obj_all


def joint_objective(w: np.ndarray, scale: np.ndarray, h: np.ndarray, rows: Optional[np.ndarray] = None):
    """e^T H e per selected row with the full H, e = w - w_hat on the given group-32 steps."""
    w = _c(w, np.float32)
    scale = _c(scale, np.float32)
    h = _c(h, np.float32)
    rows = _c(np.arange(w.shape[0]) if rows is None else rows, np.int64)
    obj = np.empty(rows.shape[0], np.float64)
    _L().orc_joint_objective(_p(w), _p(scale), w.shape[1], _p(h), h.shape[1], _p(rows), rows.shape[0], _p(obj))
    return obj


def joint_refine(w: np.ndarray, h: np.ndarray, alpha: np.ndarray, idx: np.ndarray,
                 rows: Optional[np.ndarray] = None, n_sweeps: int = 2):
    """Coordinate descent over the groups of each selected row on the joint objective, from the
    start idx [cnt][G].  -> dict idx, scale, obj, margin, sweeps."""
    w = _c(w, np.float32)
    h = _c(h, np.float32)
    alpha = _c(alpha, np.float32)
    rows = _c(np.arange(w.shape[0]) if rows is None else rows, np.int64)
    cnt, G = rows.shape[0], w.shape[1] // 32
    out = {"idx": np.array(idx, dtype=np.uint8, copy=True).reshape(cnt, G),
           "scale": np.empty((cnt, G), np.float32), "obj": np.empty(cnt, np.float64),
           "margin": np.empty(cnt, np.float64), "sweeps": np.empty(cnt, np.int32)}
    _L().orc_joint_refine(_p(w), w.shape[1], _p(h), h.shape[1], _p(alpha), alpha.shape[0], _p(rows), cnt,
                          int(n_sweeps), _p(out["idx"]), _p(out["scale"]), _p(out["obj"]), _p(out["margin"]),
                          _p(out["sweeps"]))
    return out


def gptq(w: np.ndarray, h: np.ndarray, scale: np.ndarray, damp: float = 0.01,
         rows: Optional[np.ndarray] = None):
    """GPTQ error feedback with fixed group-32 steps on selected rows.
    -> dict w_hat f32 [cnt][d_in], w_upd f64 [cnt][d_in], margin f64 [cnt]; raises if H' is not
    positive definite."""
    w = _c(w, np.float32)
    h = _c(h, np.float32)
    scale = _c(scale, np.float32)
    rows = _c(np.arange(w.shape[0]) if rows is None else rows, np.int64)
    cnt, d_in = rows.shape[0], w.shape[1]
    out = {"w_hat": np.empty((cnt, d_in), np.float32), "w_upd": np.empty((cnt, d_in), np.float64),
           "margin": np.empty(cnt, np.float64)}
    rc = _L().orc_gptq(_p(w), d_in, _p(h), h.shape[1], _p(scale), float(damp), _p(rows), cnt,
                       _p(out["w_hat"]), _p(out["w_upd"]), _p(out["margin"]))
    if rc != 0:
        raise ValueError("H + damping is not positive definite")
    return out


ADAM_KEYS = ("lr_w", "lr_s", "beta1", "beta2", "eps", "weight_decay", "step", "scale_min")


def adam_hparams(lr_w, lr_s, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1, scale_min=1e-12):
    """The step's hyperparameters as the array the C oracle takes (bias corrections for step t),
    each rounded to fp32 as the library receives them (0.9 is not an fp32 value: the update is
    defined on the parameters actually passed)."""
    v = [lr_w, lr_s, beta1, beta2, eps, weight_decay, 1.0 - beta1 ** step, 1.0 - beta2 ** step, scale_min]
    return np.array(v, dtype=np.float32).astype(np.float64)


def lsq_adam_step(w, scale, g, gs, m_w, v_w, m_s, v_s, hp, ext_ds=None, with_w_hat=True):
    """-> dict of w, scale, m_w, v_w, m_s, v_s (fp32), ds (f64 step-size gradient), w_hat (fp32)."""
    w, scale, g = _c(w, np.float32), _c(scale, np.float32), _c(g, np.float32)
    m_w, v_w, m_s, v_s = (_c(a, np.float32) for a in (m_w, v_w, m_s, v_s))
    hp = _c(hp, np.float64)
    d_out, d_in = w.shape
    G = d_in // 32
    out = {k: np.empty_like(a) for k, a in (("w", w), ("m_w", m_w), ("v_w", v_w))}
    out.update({k: np.empty((d_out, G), np.float32) for k in ("scale", "m_s", "v_s")})
    out["ds"] = np.empty((d_out, G), np.float64)
    out["w_hat"] = np.empty_like(w) if with_w_hat else None
    ext = None if ext_ds is None else _c(ext_ds, np.float64)
    _L().orc_lsq_adam_step(_p(w), _p(scale), _p(g), d_out, d_in, float(gs), _p(m_w), _p(v_w), _p(m_s), _p(v_s),
                           _p(hp), _p(ext), _p(out["w"]), _p(out["scale"]), _p(out["m_w"]), _p(out["v_w"]),
                           _p(out["m_s"]), _p(out["v_s"]), _p(out["ds"]), _p(out["w_hat"]))
    return out
