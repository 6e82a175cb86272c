"""Torch-tensor front end of the C ABI: metadata checks, output allocation, pointer marshalling.

All tensors must be contiguous CUDA (HIP) tensors on one device; work is enqueued on the
current stream of that device and nothing is synchronised here.
"""
from __future__ import annotations

from typing import Optional, Tuple

import ctypes
import torch

from ._lib import W4Q_GROUP, check, lib


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _out(t: Optional[torch.Tensor], name, shape, dtype, device) -> torch.Tensor:
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, shape, device)
    return t


def _workspace(query: str, sizes, device, workspace: Optional[torch.Tensor]):
    """(pointer, bytes, tensor) of the scratch for one call: the caller's uint8 device tensor, or
    a fresh one of the size the library asks for (torch's caching allocator, on the current
    stream; none when the library needs none)."""
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, device=device)
        return workspace.data_ptr(), workspace.numel(), workspace
    n = ctypes.c_size_t(0)
    check(query, getattr(lib(), query)(*sizes, ctypes.byref(n)))
    if n.value == 0:
        return None, 0, None
    buf = torch.empty(n.value, dtype=torch.uint8, device=device)
    return buf.data_ptr(), n.value, buf


def workspace_size(op: str, *sizes) -> int:
    """Scratch bytes: op in ("quant_hessian", "w4a16_gemm", "w4a16_gemm_dq", "per_channel", "joint",
    "gptq") with (n_tok, d), (m, d_out, d_in) or (d_out, d_in) as the C query takes them."""
    n = ctypes.c_size_t(0)
    check(op + "_workspace_size", getattr(lib(), op + "_workspace_size")(*sizes, ctypes.byref(n)))
    return n.value


def quant_hessian(x: torch.Tensor, h: Optional[torch.Tensor] = None,
                  accumulate: bool = False, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H = X^T X (or H += X^T X) for bf16 X [n_tok][d]; returns fp32 H [d][d].  workspace: a
    uint8 device tensor of scratch (default: allocated per call with torch)."""
    _need(x, "x", torch.bfloat16)
    n_tok, d = x.shape
    if accumulate and h is None:
        raise ValueError("accumulate=True needs h")
    h = _out(h, "h", (d, d), torch.float32, x.device)
    wp, wb, _keep = _workspace("quant_hessian_workspace_size", (n_tok, d), x.device, workspace)
    check("quant_hessian", lib().quant_hessian(x.data_ptr(), n_tok, d, h.data_ptr(),
                                               1 if accumulate else 0, wp, wb, _stream(x)))
    return h


def quant_scale_search(w: torch.Tensor, h: torch.Tensor, alpha: torch.Tensor,
                       with_obj: bool = True, with_obj_all: bool = False,
                       out: Optional[Tuple[torch.Tensor, ...]] = None):
    """-> (scale f32 [d_out][G], idx u8 [d_out][G], obj f32 | None, obj_all f32 | None)."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    if h.dim() != 2 or h.shape[0] != d_in:
        raise ValueError(f"h must be [{d_in}][ldh], got {tuple(h.shape)}")
    _need(h, "h", torch.float32, device=w.device)
    _need(alpha, "alpha", torch.float32, device=w.device)
    G, K = d_in // W4Q_GROUP, alpha.numel()
    dev = w.device
    if out is None:
        out = (None, None, None, None)
    if len(out) != 4:
        raise ValueError("out must be (scale, idx, obj | None, obj_all | None)")
    scale = _out(out[0], "scale", (d_out, G), torch.float32, dev)
    idx = _out(out[1], "idx", (d_out, G), torch.uint8, dev)
    obj = out[2] if out[2] is not None or not with_obj else torch.empty((d_out, G), dtype=torch.float32, device=dev)
    if obj is not None:
        _need(obj, "obj", torch.float32, (d_out, G), dev)
    obj_all = (out[3] if out[3] is not None or not with_obj_all
               else torch.empty((d_out, G, K), dtype=torch.float32, device=dev))
    if obj_all is not None:
        _need(obj_all, "obj_all", torch.float32, (d_out, G, K), dev)
    check("quant_scale_search", lib().quant_scale_search(
        w.data_ptr(), d_out, d_in, h.data_ptr(), h.shape[1], alpha.data_ptr(), K,
        scale.data_ptr(), idx.data_ptr(), obj.data_ptr() if obj is not None else None,
        obj_all.data_ptr() if obj_all is not None else None, _stream(w)))
    return scale, idx, obj, obj_all


def quant_pack(w: torch.Tensor, scale: torch.Tensor,
               out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """-> (packed u8 [d_out][d_in/2], scale_f16 fp16 [d_out][G])."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out, d_in // W4Q_GROUP), w.device)
    packed, s16 = (None, None) if out is None else out
    packed = _out(packed, "packed", (d_out, d_in // 2), torch.uint8, w.device)
    s16 = _out(s16, "scale_f16", (d_out, d_in // W4Q_GROUP), torch.float16, w.device)
    check("quant_pack", lib().quant_pack(w.data_ptr(), scale.data_ptr(), d_out, d_in,
                                         packed.data_ptr(), s16.data_ptr(), _stream(w)))
    return packed, s16


def lsq_fwd(w: torch.Tensor, scale: torch.Tensor, out: Optional[torch.Tensor] = None):
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out, d_in // W4Q_GROUP), w.device)
    w_hat = _out(out, "w_hat", (d_out, d_in), torch.float32, w.device)
    check("lsq_fwd", lib().lsq_fwd(w.data_ptr(), scale.data_ptr(), d_out, d_in,
                                   w_hat.data_ptr(), _stream(w)))
    return w_hat


def lsq_bwd(w: torch.Tensor, scale: torch.Tensor, grad_w_hat: torch.Tensor, grad_scale: float,
            with_w_hat: bool = False, out: Optional[Tuple] = None):
    """-> (grad_w f32, grad_scale_out f32 [d_out][G], w_hat f32 | None)."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out, d_in // W4Q_GROUP), w.device)
    _need(grad_w_hat, "grad_w_hat", torch.float32, (d_out, d_in), w.device)
    gw, gsc, wh = (None, None, None) if out is None else out
    gw = _out(gw, "grad_w", (d_out, d_in), torch.float32, w.device)
    gsc = _out(gsc, "grad_scale_out", (d_out, d_in // W4Q_GROUP), torch.float32, w.device)
    if wh is None and with_w_hat:
        wh = torch.empty_like(w)
    if wh is not None:
        _need(wh, "w_hat", torch.float32, (d_out, d_in), w.device)
    check("lsq_bwd", lib().lsq_bwd(w.data_ptr(), scale.data_ptr(), grad_w_hat.data_ptr(), d_out,
                                   d_in, float(grad_scale), gw.data_ptr(), gsc.data_ptr(),
                                   wh.data_ptr() if wh is not None else None, _stream(w)))
    return gw, gsc, wh


def lsq_adam_step(w: torch.Tensor, scale: torch.Tensor, grad_w_hat: torch.Tensor, grad_scale: float,
                  m_w: torch.Tensor, v_w: torch.Tensor, m_s: torch.Tensor, v_s: torch.Tensor, *,
                  lr_w: float, lr_s: float, step: int, beta1: float = 0.9, beta2: float = 0.999,
                  eps: float = 1e-8, weight_decay: float = 0.0, scale_min: float = 1e-12,
                  with_w_hat_next: bool = False, with_grad_scale: bool = False):
    """One fused QAT step: updates w, scale and the four Adam moments in place; returns
    (w_hat_next | None, grad_scale_out | None)."""
    from ._lib import AdamParams
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    G = d_in // W4Q_GROUP
    for t, n in ((grad_w_hat, "grad_w_hat"), (m_w, "m_w"), (v_w, "v_w")):
        _need(t, n, torch.float32, (d_out, d_in), w.device)
    for t, n in ((scale, "scale"), (m_s, "m_s"), (v_s, "v_s")):
        _need(t, n, torch.float32, (d_out, G), w.device)
    if step < 1:
        raise ValueError("step counts from 1")
    hp = AdamParams(lr_w, lr_s, beta1, beta2, eps, weight_decay, 1.0 - beta1 ** step, 1.0 - beta2 ** step,
                    scale_min)
    wh = torch.empty_like(w) if with_w_hat_next else None
    ds = torch.empty((d_out, G), dtype=torch.float32, device=w.device) if with_grad_scale else None
    check("lsq_adam_step", lib().lsq_adam_step(
        w.data_ptr(), scale.data_ptr(), grad_w_hat.data_ptr(), d_out, d_in, float(grad_scale), m_w.data_ptr(),
        v_w.data_ptr(), m_s.data_ptr(), v_s.data_ptr(), ctypes.byref(hp),
        ds.data_ptr() if ds is not None else None, wh.data_ptr() if wh is not None else None, _stream(w)))
    return wh, ds


def _gemm(name: str, x: torch.Tensor, packed: torch.Tensor, scale_f16: torch.Tensor,
          out_dtype: torch.dtype, out: Optional[torch.Tensor], workspace: Optional[torch.Tensor] = None):
    _need(x, "x", torch.bfloat16)
    m, d_in = x.shape
    _need(packed, "packed", torch.uint8, device=x.device)
    d_out = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] * 2 != d_in:
        raise ValueError(f"packed must be [d_out][{d_in // 2}], got {tuple(packed.shape)}")
    _need(scale_f16, "scale_f16", torch.float16, (d_out, d_in // W4Q_GROUP), x.device)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    y = _out(out, "y", (m, d_out), out_dtype, x.device)
    wp, wb, _keep = _workspace(name + "_workspace_size", (m, d_out, d_in), x.device, workspace)
    check(name, getattr(lib(), name)(x.data_ptr(), m, packed.data_ptr(), scale_f16.data_ptr(),
                                     d_out, d_in, y.data_ptr(),
                                     0 if out_dtype == torch.float32 else 1, wp, wb, _stream(x)))
    return y


def w4a16_gemm(x: torch.Tensor, packed: torch.Tensor, scale_f16: torch.Tensor,
               out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None):
    """y [m][d_out] = x [m][d_in] (bf16) times the dequantised packed weights (s16 * q, exact),
    transposed."""
    return _gemm("w4a16_gemm", x, packed, scale_f16, out_dtype, out, workspace)


def w4a16_gemm_dq(x: torch.Tensor, packed: torch.Tensor, scale_f16: torch.Tensor,
                  out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """As w4a16_gemm with each weight dequantized to bf16 (RNE of s16 * q) before the product;
    d_in must be a multiple of 256."""
    return _gemm("w4a16_gemm_dq", x, packed, scale_f16, out_dtype, out, workspace)


# ------------------------------------------------------------------ per-channel variant
def _h_check(h: torch.Tensor, d_in: int, device) -> None:
    if h.dim() != 2 or h.shape[0] != d_in or h.shape[1] < d_in:
        raise ValueError(f"h must be [{d_in}][ldh >= {d_in}], got {tuple(h.shape)}")
    _need(h, "h", torch.float32, device=device)


def quant_scale_search_pc(w: torch.Tensor, h: torch.Tensor, alpha: torch.Tensor,
                          with_obj: bool = True, with_obj_all: bool = False):
    """One scale per output row, scored with the full H in fp64.
    -> (scale f32 [d_out], idx u8 [d_out], obj f32 [d_out] | None, obj_all f32 [d_out][K] | None)."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _h_check(h, d_in, w.device)
    _need(alpha, "alpha", torch.float32, device=w.device)
    K, dev = alpha.numel(), w.device
    scale = torch.empty(d_out, dtype=torch.float32, device=dev)
    idx = torch.empty(d_out, dtype=torch.uint8, device=dev)
    obj = torch.empty(d_out, dtype=torch.float32, device=dev) if with_obj else None
    obj_all = torch.empty((d_out, K), dtype=torch.float32, device=dev) if with_obj_all else None
    check("quant_scale_search_pc", lib().quant_scale_search_pc(
        w.data_ptr(), d_out, d_in, h.data_ptr(), h.shape[1], alpha.data_ptr(), K, scale.data_ptr(),
        idx.data_ptr(), obj.data_ptr() if obj is not None else None,
        obj_all.data_ptr() if obj_all is not None else None, _stream(w)))
    return scale, idx, obj, obj_all


def _pc_ws(m, d_out, d_in, device, workspace):
    return _workspace("per_channel_workspace_size", (m, d_out, d_in), device, workspace)


def quant_pack_pc(w: torch.Tensor, scale: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """-> (packed u8 [d_out][d_in/2], scale_f16 fp16 [d_out]) on one scale per row."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out,), w.device)
    packed = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=w.device)
    s16 = torch.empty(d_out, dtype=torch.float16, device=w.device)
    wp, wb, _keep = _pc_ws(1, d_out, d_in, w.device, workspace)
    check("quant_pack_pc", lib().quant_pack_pc(w.data_ptr(), scale.data_ptr(), d_out, d_in, packed.data_ptr(),
                                               s16.data_ptr(), wp, wb, _stream(w)))
    return packed, s16


def lsq_fwd_pc(w: torch.Tensor, scale: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out,), w.device)
    w_hat = torch.empty_like(w)
    wp, wb, _keep = _pc_ws(1, d_out, d_in, w.device, workspace)
    check("lsq_fwd_pc", lib().lsq_fwd_pc(w.data_ptr(), scale.data_ptr(), d_out, d_in, w_hat.data_ptr(), wp, wb,
                                         _stream(w)))
    return w_hat


def lsq_bwd_pc(w: torch.Tensor, scale: torch.Tensor, grad_w_hat: torch.Tensor, grad_scale: float,
               with_w_hat: bool = False, workspace: Optional[torch.Tensor] = None):
    """-> (grad_w f32, grad_scale_out f32 [d_out], w_hat f32 | None) on one scale per row."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out,), w.device)
    _need(grad_w_hat, "grad_w_hat", torch.float32, (d_out, d_in), w.device)
    gw = torch.empty_like(w)
    gs = torch.empty(d_out, dtype=torch.float32, device=w.device)
    wh = torch.empty_like(w) if with_w_hat else None
    wp, wb, _keep = _pc_ws(1, d_out, d_in, w.device, workspace)
    check("lsq_bwd_pc", lib().lsq_bwd_pc(w.data_ptr(), scale.data_ptr(), grad_w_hat.data_ptr(), d_out, d_in,
                                         float(grad_scale), gw.data_ptr(), gs.data_ptr(),
                                         wh.data_ptr() if wh is not None else None, wp, wb, _stream(w)))
    return gw, gs, wh


def w4a16_gemm_pc(x: torch.Tensor, packed: torch.Tensor, scale_f16: torch.Tensor,
                  out_dtype: torch.dtype = torch.float32, dequant_bf16: bool = False,
                  workspace: Optional[torch.Tensor] = None):
    """y [m][d_out] = x W_hat^T with one fp16 scale per row (scale_f16 [d_out]); dequant_bf16 as
    w4a16_gemm_dq."""
    _need(x, "x", torch.bfloat16)
    m, d_in = x.shape
    _need(packed, "packed", torch.uint8, device=x.device)
    d_out = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] * 2 != d_in:
        raise ValueError(f"packed must be [d_out][{d_in // 2}], got {tuple(packed.shape)}")
    _need(scale_f16, "scale_f16", torch.float16, (d_out,), x.device)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    y = torch.empty((m, d_out), dtype=out_dtype, device=x.device)
    wp, wb, _keep = _pc_ws(m, d_out, d_in, x.device, workspace)
    check("w4a16_gemm_pc", lib().w4a16_gemm_pc(x.data_ptr(), m, packed.data_ptr(), scale_f16.data_ptr(), d_out,
                                               d_in, y.data_ptr(), 0 if out_dtype == torch.float32 else 1,
                                               1 if dequant_bf16 else 0, wp, wb, _stream(x)))
    return y


# ------------------------------------------------------------------- joint objective
def quant_joint_objective(w: torch.Tensor, scale: torch.Tensor, h: torch.Tensor,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """e^T H e per row with the full H on the group-32 steps scale [d_out][G] -> fp64 [d_out]."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _need(scale, "scale", torch.float32, (d_out, d_in // W4Q_GROUP), w.device)
    _h_check(h, d_in, w.device)
    obj = torch.empty(d_out, dtype=torch.float64, device=w.device)
    wp, wb, _keep = _workspace("joint_workspace_size", (d_out, d_in), w.device, workspace)
    check("quant_joint_objective", lib().quant_joint_objective(
        w.data_ptr(), scale.data_ptr(), d_out, d_in, h.data_ptr(), h.shape[1], obj.data_ptr(), wp, wb,
        _stream(w)))
    return obj


def quant_joint_refine(w: torch.Tensor, h: torch.Tensor, alpha: torch.Tensor, idx: torch.Tensor,
                       n_sweeps: int = 2, inplace: bool = False, workspace: Optional[torch.Tensor] = None):
    """Coordinate descent over the groups of each row on the joint objective, from idx [d_out][G]
    (u8); h must be symmetric (as quant_hessian writes it).  -> (idx, scale f32 [d_out][G],
    obj_before f64, obj_after f64, sweeps i32) per row."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    G = d_in // W4Q_GROUP
    _h_check(h, d_in, w.device)
    _need(alpha, "alpha", torch.float32, device=w.device)
    _need(idx, "idx", torch.uint8, (d_out, G), w.device)
    if not inplace:
        idx = idx.clone()
    dev = w.device
    scale = torch.empty((d_out, G), dtype=torch.float32, device=dev)
    ob = torch.empty(d_out, dtype=torch.float64, device=dev)
    oa = torch.empty(d_out, dtype=torch.float64, device=dev)
    sw = torch.empty(d_out, dtype=torch.int32, device=dev)
    wp, wb, _keep = _workspace("joint_workspace_size", (d_out, d_in), dev, workspace)
    check("quant_joint_refine", lib().quant_joint_refine(
        w.data_ptr(), d_out, d_in, h.data_ptr(), h.shape[1], alpha.data_ptr(), alpha.numel(), idx.data_ptr(),
        scale.data_ptr(), int(n_sweeps), ob.data_ptr(), oa.data_ptr(), sw.data_ptr(), wp, wb, _stream(w)))
    return idx, scale, ob, oa, sw


# -------------------------------------------------------------------- GPTQ feedback
def quant_gptq(w: torch.Tensor, h: torch.Tensor, scale: torch.Tensor, damp: float = 0.01,
               workspace: Optional[torch.Tensor] = None):
    """GPTQ error feedback with the fixed group-32 steps scale [d_out][G].
    -> (w_hat f32 [d_out][d_in] = Delta * q, info int32 [1]: 1 if H + damping was not positive
    definite)."""
    _need(w, "w", torch.float32)
    d_out, d_in = w.shape
    _h_check(h, d_in, w.device)
    _need(scale, "scale", torch.float32, (d_out, d_in // W4Q_GROUP), w.device)
    w_hat = torch.empty_like(w)
    info = torch.zeros(1, dtype=torch.int32, device=w.device)
    wp, wb, _keep = _workspace("gptq_workspace_size", (d_out, d_in), w.device, workspace)
    check("quant_gptq", lib().quant_gptq(w.data_ptr(), d_out, d_in, h.data_ptr(), h.shape[1], scale.data_ptr(),
                                         float(damp), w_hat.data_ptr(), info.data_ptr(), wp, wb, _stream(w)))
    return w_hat, info


class GemvGroupPlan:
    """A prepared w4a16_gemv_grouped call: the problem table is checked and marshalled once, and
    each call of the plan is a single library call (a decode step reuses the same weight, input
    and output buffers, so the table does not change between steps).  The plan keeps references
    to every tensor it points at."""

    def __init__(self, xs, packeds, scales, out_dtype: torch.dtype = torch.float32, outs=None):
        from ._lib import GemvProblem
        n = len(xs)
        if not (len(packeds) == len(scales) == n) or (outs is not None and len(outs) != n):
            raise ValueError("xs, packeds, scales (and outs) must have the same length")
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be float32 or bfloat16")
        arr = (GemvProblem * max(n, 1))()
        ys = []
        for i in range(n):
            x, p, s = xs[i], packeds[i], scales[i]
            _need(x, "x", torch.bfloat16)
            if x.dim() != 2 or x.shape[0] != 1:
                raise ValueError("each x must be [1][d_in]")
            d_in = x.shape[1]
            _need(p, "packed", torch.uint8, device=x.device)
            d_out = p.shape[0]
            if p.dim() != 2 or p.shape[1] * 2 != d_in:
                raise ValueError(f"packed must be [d_out][{d_in // 2}], got {tuple(p.shape)}")
            _need(s, "scale_f16", torch.float16, (d_out, d_in // W4Q_GROUP), x.device)
            y = _out(None if outs is None else outs[i], "y", (1, d_out), out_dtype, x.device)
            ys.append(y)
            arr[i] = GemvProblem(x.data_ptr(), p.data_ptr(), s.data_ptr(), y.data_ptr(), d_out, d_in)
        self.outs = ys
        self._keep = (list(xs), list(packeds), list(scales))
        self._arr = arr
        self._ptr = ctypes.cast(arr, ctypes.c_void_p)
        self._n = n
        self._ydt = 0 if out_dtype == torch.float32 else 1
        self._device = xs[0].device if n else None
        self._fn = lib().w4a16_gemv_grouped

    def __call__(self):
        stream = _stream(self._keep[0][0]) if self._n else 0
        check("w4a16_gemv_grouped", self._fn(self._ptr, self._n, self._ydt, stream))
        return self.outs


def w4a16_gemv_grouped(xs, packeds, scales, out_dtype: torch.dtype = torch.float32, outs=None):
    """One-row products y_i [1][d_out_i] = x_i [1][d_in_i] W_hat_i^T for several independent
    problems in as few launches as possible (64 problems per launch).  For a call repeated on the
    same buffers, GemvGroupPlan marshals the table once."""
    return GemvGroupPlan(xs, packeds, scales, out_dtype, outs)()


def probe_read(buf: torch.Tensor, nontemporal: bool = True, sink: Optional[torch.Tensor] = None) -> None:
    """Enqueue one streaming read of the whole device tensor `buf` (diagnostic: measured HBM
    peak with non-temporal loads; with ordinary loads it also refills the caches).  Time it with
    events on the current stream."""
    from ._lib import W4Q_PROBE_SINK_WORDS
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    sink = _out(sink, "sink", (W4Q_PROBE_SINK_WORDS,), torch.int32, buf.device)
    check("w4q_probe_read", lib().w4q_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                                 1 if nontemporal else 0, sink.data_ptr(), _stream(buf)))


def probe_mfma_bf16(iters: int, device, sink: Optional[torch.Tensor] = None) -> float:
    """Enqueue one launch of independent bf16 matrix-core products (diagnostic: measured MFMA
    peak); returns its flop count."""
    from ._lib import W4Q_PROBE_SINK_WORDS
    device = torch.device(device)
    sink = _out(sink, "sink", (W4Q_PROBE_SINK_WORDS,), torch.float32, device)
    flop = ctypes.c_double(0.0)
    check("w4q_probe_mfma_bf16", lib().w4q_probe_mfma_bf16(sink.data_ptr(), int(iters), ctypes.byref(flop),
                                                           torch.cuda.current_stream(device).cuda_stream))
    return flop.value


def probe_mfma_f64(iters: int, device, sink: Optional[torch.Tensor] = None) -> float:
    """Enqueue one launch of independent fp64 matrix-core products (diagnostic: measured fp64
    MFMA peak); returns its flop count."""
    from ._lib import W4Q_PROBE_SINK_WORDS
    device = torch.device(device)
    sink = _out(sink, "sink", (W4Q_PROBE_SINK_WORDS // 2,), torch.float64, device)
    flop = ctypes.c_double(0.0)
    check("w4q_probe_mfma_f64", lib().w4q_probe_mfma_f64(sink.data_ptr(), int(iters), ctypes.byref(flop),
                                                         torch.cuda.current_stream(device).cuda_stream))
    return flop.value
