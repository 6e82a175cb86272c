"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/w4a16q.h declares, and rejects bad arguments with the documented status codes before
anything reaches the device."""
import ctypes
import os
import re

import pytest

import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16q.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == {"w4q_status_string", "w4q_version", "quant_hessian",
                          "quant_hessian_workspace_size", "quant_scale_search", "quant_pack",
                          "lsq_fwd", "lsq_bwd", "lsq_adam_step", "w4a16_gemm", "w4a16_gemm_workspace_size",
                          "w4a16_gemm_dq", "w4a16_gemm_dq_workspace_size", "w4a16_gemm_dq_noalloc",
                          "w4a16_gemv_grouped",
                          "quant_scale_search_pc", "per_channel_workspace_size", "quant_pack_pc", "lsq_fwd_pc",
                          "lsq_bwd_pc", "w4a16_gemm_pc", "joint_workspace_size", "quant_joint_objective",
                          "quant_joint_refine", "gptq_workspace_size", "quant_gptq",
                          "w4q_probe_read", "w4q_probe_mfma_bf16", "w4q_probe_mfma_f64"}
    l = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(l, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings_and_version():
    assert w4q.version() == 10000
    for s in (0, -1, -2, -3, -4, -5):
        assert w4q.status_string(s) and w4q.status_string(s) != "unknown status"
    assert w4q.status_string(7) == "unknown status"


A = 4096  # a 16-byte aligned fake address: never dereferenced, the checks fail first
B = 4097  # misaligned


def test_hessian_argument_errors():
    L = w4q.lib()
    assert L.quant_hessian(None, 8, 8, A, 0, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 8, 8, None, 0, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 8, 8, A, 2, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 0, 8, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, 12, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, -8, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, 65544, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(B, 8, 8, A, 0, None, 0, None) == w4q.W4Q_EALIGN


def test_workspace_arguments():
    L = w4q.lib()
    n = ctypes.c_size_t(7)
    assert L.quant_hessian_workspace_size(8, 8, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian_workspace_size(0, 8, ctypes.byref(n)) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm_workspace_size(0, 4, 64, ctypes.byref(n)) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm_dq_workspace_size(4, 4, 48, ctypes.byref(n)) == w4q.W4Q_ESHAPE
    # NULL scratch with a size, and misaligned scratch, are refused before anything is enqueued
    assert L.quant_hessian(A, 8, 8, A, 0, None, 64, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 8, 8, A, 0, A + 16, 64, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm(A, 32, A, A, 4, 256, A, 0, None, 16, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm_dq(A, 32, A, A, 4, 256, A, 0, A + 128, 1 << 20, None) == w4q.W4Q_EALIGN


@pytest.mark.parametrize("n_tok,d,want", [(8, 8, 0), (8192, 4096, 256 * 2 * 256 * 256 * 4),
                                          (1 << 20, 12288, 256 * 2 * 256 * 256 * 4)])
def test_hessian_workspace_size(n_tok, d, want):
    # the fastest schedule keeps two 256x256 fp32 partial tiles per workgroup that shares a tile;
    # a single small tile needs none; never more than 128 MB
    n = ctypes.c_size_t(0)
    assert w4q.lib().quant_hessian_workspace_size(n_tok, d, ctypes.byref(n)) == w4q.W4Q_OK
    assert n.value == want
    assert w4q.workspace_size("quant_hessian", n_tok, d) == want


def test_gemm_workspace_size():
    # exact weights use scratch only for m > 16 below 256 output tiles on the tiled kernel; the
    # dequantizing product for its stream-K split
    assert w4q.workspace_size("w4a16_gemm", 16, 4096, 4096) == 0
    assert w4q.workspace_size("w4a16_gemm", 2048, 12288, 4096) == 0          # 384 tiles: per-group kernel
    assert w4q.workspace_size("w4a16_gemm", 256, 8192, 2048) > 0             # 32 tiles: split weights
    assert w4q.workspace_size("w4a16_gemm", 256, 8192, 2080) == 0            # d_in % 256 != 0
    assert 0 < w4q.workspace_size("w4a16_gemm_dq", 2048, 12288, 4096) <= 128 << 20
    assert w4q.workspace_size("w4a16_gemm_dq", 1, 256, 256) == 0             # one tile, no split


def test_search_argument_errors():
    L = w4q.lib()
    ok = dict(w=A, d_out=4, d_in=64, h=A, ldh=64, alpha=A, K=3, scale=A, idx=A)

    def call(**kw):
        a = dict(ok, **kw)
        return L.quant_scale_search(a["w"], a["d_out"], a["d_in"], a["h"], a["ldh"], a["alpha"],
                                    a["K"], a["scale"], a["idx"], None, None, None)
    assert call(w=None) == w4q.W4Q_EINVAL
    assert call(alpha=None) == w4q.W4Q_EINVAL
    assert call(idx=None) == w4q.W4Q_EINVAL
    assert call(K=0) == w4q.W4Q_EINVAL
    assert call(K=256) == w4q.W4Q_EINVAL
    assert call(d_in=48) == w4q.W4Q_ESHAPE
    assert call(d_out=0) == w4q.W4Q_ESHAPE
    assert call(ldh=32) == w4q.W4Q_ESHAPE
    assert call(ldh=66) == w4q.W4Q_ESHAPE                  # rows of H must stay 16-byte aligned
    assert call(w=A + 4) == w4q.W4Q_EALIGN
    assert call(h=A + 4) == w4q.W4Q_EALIGN


def test_pack_lsq_gemm_argument_errors():
    L = w4q.lib()
    assert L.quant_pack(A, A, 4, 40, A, A, None) == w4q.W4Q_ESHAPE
    assert L.quant_pack(A, None, 4, 64, A, A, None) == w4q.W4Q_EINVAL
    assert L.quant_pack(A, A, 4, 64, A + 8, A, None) == w4q.W4Q_EALIGN
    assert L.lsq_fwd(A, A, 4, 64, None, None) == w4q.W4Q_EINVAL
    assert L.lsq_fwd(A, A, -1, 64, A, None) == w4q.W4Q_ESHAPE
    assert L.lsq_bwd(A, A, A, 4, 64, 0.5, A, None, None, None) == w4q.W4Q_EINVAL
    assert L.lsq_bwd(A, A, A, 4, 96, 0.5, A + 4, A, None, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm(A, 1, A, A, 4, 64, A, 2, None, 0, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm(A, 0, A, A, 4, 64, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm(A, 1, A, A, 4, 65, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm(A + 2, 1, A, A, 4, 64, A, 0, None, 0, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm(A, 1, A, A, 4, 64, A + 1, 1, None, 0, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm_dq(A, 1, A, A, 4, 256, A, 2, None, 0, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm_dq(A, 0, A, A, 4, 256, A, 0, None, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm_dq(A + 2, 1, A, A, 4, 256, A, 0, None, 0, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm_dq(A, 1, A, A, 4, 64, A, 0, None, 0, None) == w4q.W4Q_EUNSUPPORTED
    from w4a16_group_wise_amd._lib import GemvProblem
    probs = (GemvProblem * 2)(GemvProblem(A, A, A, A, 4, 64), GemvProblem(A, A, A, A, 4, 64))
    pp = ctypes.cast(probs, ctypes.c_void_p)
    assert L.w4a16_gemv_grouped(None, 0, 0, None) == w4q.W4Q_OK          # nothing to do
    assert L.w4a16_gemv_grouped(None, 1, 0, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemv_grouped(pp, -1, 0, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemv_grouped(pp, 2, 3, None) == w4q.W4Q_EINVAL
    probs[1].d_in = 65
    assert L.w4a16_gemv_grouped(pp, 2, 0, None) == w4q.W4Q_ESHAPE
    probs[1].d_in = 64
    probs[1].x = A + 2
    assert L.w4a16_gemv_grouped(pp, 2, 0, None) == w4q.W4Q_EALIGN
    probs[1].x = 0
    assert L.w4a16_gemv_grouped(pp, 2, 0, None) == w4q.W4Q_EINVAL
    probs[1].x = A
    probs[1].d_out, probs[1].d_in = 4, (1 << 24) + 32   # beyond the 32-bit lane offsets
    assert L.w4a16_gemv_grouped(pp, 2, 0, None) == w4q.W4Q_EUNSUPPORTED


def test_probe_argument_errors():
    L = w4q.lib()
    assert L.w4q_probe_read(None, 16, 1, A, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_read(A, 24, 1, A, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_read(A, 0, 1, A, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_read(A, 16, 2, A, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_read(A, 16, 1, None, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_read(A + 8, 16, 1, A, None) == w4q.W4Q_EALIGN
    assert L.w4q_probe_mfma_bf16(None, 10, None, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_mfma_f64(None, 10, None, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_mfma_f64(A, 0, None, None) == w4q.W4Q_EINVAL
    assert L.w4q_probe_mfma_f64(A + 4, 10, None, None) == w4q.W4Q_EALIGN
    assert L.w4q_probe_mfma_bf16(A, 0, None, None) == w4q.W4Q_EINVAL


def test_python_front_end_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        w4q.lsq_fwd(w, torch.zeros(4, 2))


def test_adam_step_argument_errors():
    from w4a16_group_wise_amd._lib import AdamParams
    L = w4q.lib()
    ok = AdamParams(1e-3, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0.1, 0.001, 1e-12)

    def call(hp=ok, **kw):
        a = dict(w=A, scale=A, g=A, d_out=4, d_in=64, m_w=A, v_w=A, m_s=A, v_s=A, ds=None, wh=None)
        a.update(kw)
        return L.lsq_adam_step(a["w"], a["scale"], a["g"], a["d_out"], a["d_in"], 0.5, a["m_w"], a["v_w"],
                               a["m_s"], a["v_s"], ctypes.byref(hp) if hp is not None else None, a["ds"],
                               a["wh"], None)
    assert call(hp=None) == w4q.W4Q_EINVAL
    assert call(m_w=None) == w4q.W4Q_EINVAL
    for bad in (dict(beta1=1.0), dict(eps=0.0), dict(bias_c1=0.0), dict(bias_c2=1.5), dict(lr_w=-1.0),
                dict(scale_min=0.0), dict(lr_s=float("nan"))):
        hp = AdamParams(*[bad.get(f, getattr(ok, f)) for f, _ in AdamParams._fields_])
        assert call(hp=hp) == w4q.W4Q_EINVAL, bad
    assert call(d_in=48) == w4q.W4Q_ESHAPE
    assert call(v_w=A + 4) == w4q.W4Q_EALIGN
    assert call(wh=A + 8) == w4q.W4Q_EALIGN


def test_per_channel_and_joint_argument_errors():
    L = w4q.lib()
    sz = ctypes.c_size_t(0)
    # per-channel search: as the group search (same shape and H rules)
    assert L.quant_scale_search_pc(None, 4, 64, A, 64, A, 3, A, A, None, None, None) == w4q.W4Q_EINVAL
    assert L.quant_scale_search_pc(A, 4, 64, A, 64, A, 0, A, A, None, None, None) == w4q.W4Q_EINVAL
    assert L.quant_scale_search_pc(A, 4, 48, A, 64, A, 3, A, A, None, None, None) == w4q.W4Q_ESHAPE
    assert L.quant_scale_search_pc(A, 4, 64, A, 66, A, 3, A, A, None, None, None) == w4q.W4Q_ESHAPE
    assert L.quant_scale_search_pc(A, 4, 64, A + 4, 64, A, 3, A, A, None, None, None) == w4q.W4Q_EALIGN
    # per-channel workspace: query, then too small / missing / misaligned
    assert L.per_channel_workspace_size(1, 8, 64, ctypes.byref(sz)) == w4q.W4Q_OK and sz.value > 0
    need = sz.value
    assert L.quant_pack_pc(A, A, 8, 64, A, A, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_pack_pc(A, A, 8, 64, A, A, A, need - 1, None) == w4q.W4Q_EINVAL
    assert L.quant_pack_pc(A, A, 8, 64, A, A, A + 16, need, None) == w4q.W4Q_EALIGN
    assert L.lsq_fwd_pc(A, A, 8, 40, A, A, need, None) == w4q.W4Q_ESHAPE
    assert L.lsq_bwd_pc(A, A, None, 8, 64, ctypes.c_float(1.0), A, A, None, A, need, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm_pc(A, 1, A, A, 8, 64, A, 0, 2, A, need, None) == w4q.W4Q_EINVAL   # w_mode
    assert L.w4a16_gemm_pc(A, 1, A, A, 8, 64, A, 0, 0, A, need - 1, None) == w4q.W4Q_EINVAL
    # joint: workspace must hold at least 64 rows' share (or all rows)
    assert L.joint_workspace_size(8, 64, ctypes.byref(sz)) == w4q.W4Q_OK and sz.value > 0
    need = sz.value
    assert L.quant_joint_refine(A, 8, 64, A, 64, A, 3, A, A, 0, None, None, None, A, need, None) == w4q.W4Q_EINVAL
    assert L.quant_joint_refine(A, 8, 64, A, 64, A, 3, A, A, 1, None, None, None, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_joint_refine(A, 8, 64, A, 64, A, 3, A, A, 1, None, None, None, A + 16, need, None) == w4q.W4Q_EALIGN
    assert L.quant_joint_objective(A, A, 8, 64, A, 60, A, A, need, None) == w4q.W4Q_ESHAPE
    assert L.quant_joint_objective(A, A, 8, 64, A, 64, None, A, need, None) == w4q.W4Q_EINVAL


def test_gptq_argument_errors():
    L = w4q.lib()
    sz = ctypes.c_size_t(0)
    assert L.gptq_workspace_size(8, 64, ctypes.byref(sz)) == w4q.W4Q_OK and sz.value >= 64 * 64 * 8 + 8 * 64 * 8
    need = sz.value
    f = ctypes.c_float
    assert L.quant_gptq(A, 8, 64, A, 64, A, f(0.01), A, None, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_gptq(A, 8, 64, A, 64, A, f(0.01), A, None, A, need - 1, None) == w4q.W4Q_EINVAL
    assert L.quant_gptq(A, 8, 64, A, 64, A, f(-1.0), A, None, A, need, None) == w4q.W4Q_EINVAL
    assert L.quant_gptq(A, 8, 64, A, 64, A, f(float("nan")), A, None, A, need, None) == w4q.W4Q_EINVAL
    assert L.quant_gptq(A, 8, 40, A, 64, A, f(0.01), A, None, A, need, None) == w4q.W4Q_ESHAPE
    assert L.quant_gptq(A, 8, 64, A, 62, A, f(0.01), A, None, A, need, None) == w4q.W4Q_ESHAPE
    assert L.quant_gptq(A, 8, 64, A + 4, 64, A, f(0.01), A, None, A, need, None) == w4q.W4Q_EALIGN
    assert L.quant_gptq(A, 8, 64, A, 64, A, f(0.01), A, None, A + 16, need, None) == w4q.W4Q_EALIGN
