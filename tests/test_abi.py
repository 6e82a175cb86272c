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
                          "quant_scale_search", "quant_pack", "lsq_fwd", "lsq_bwd", "w4a16_gemm",
                          "w4a16_gemm_dq", "w4a16_gemv_grouped", "w4q_probe_read",
                          "w4q_probe_mfma_bf16"}
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
    assert L.quant_hessian(None, 8, 8, A, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 8, 8, None, 0, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 8, 8, A, 2, None) == w4q.W4Q_EINVAL
    assert L.quant_hessian(A, 0, 8, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, 12, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, -8, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(A, 8, 65544, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.quant_hessian(B, 8, 8, A, 0, None) == w4q.W4Q_EALIGN


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
    assert call(w=A + 4) == w4q.W4Q_EALIGN


def test_pack_lsq_gemm_argument_errors():
    L = w4q.lib()
    assert L.quant_pack(A, A, 4, 40, A, A, None) == w4q.W4Q_ESHAPE
    assert L.quant_pack(A, None, 4, 64, A, A, None) == w4q.W4Q_EINVAL
    assert L.quant_pack(A, A, 4, 64, A + 8, A, None) == w4q.W4Q_EALIGN
    assert L.lsq_fwd(A, A, 4, 64, None, None) == w4q.W4Q_EINVAL
    assert L.lsq_fwd(A, A, -1, 64, A, None) == w4q.W4Q_ESHAPE
    assert L.lsq_bwd(A, A, A, 4, 64, 0.5, A, None, None, None) == w4q.W4Q_EINVAL
    assert L.lsq_bwd(A, A, A, 4, 96, 0.5, A + 4, A, None, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm(A, 1, A, A, 4, 64, A, 2, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm(A, 0, A, A, 4, 64, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm(A, 1, A, A, 4, 65, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm(A + 2, 1, A, A, 4, 64, A, 0, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm(A, 1, A, A, 4, 64, A + 1, 1, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm_dq(A, 1, A, A, 4, 256, A, 2, None) == w4q.W4Q_EINVAL
    assert L.w4a16_gemm_dq(A, 0, A, A, 4, 256, A, 0, None) == w4q.W4Q_ESHAPE
    assert L.w4a16_gemm_dq(A + 2, 1, A, A, 4, 256, A, 0, None) == w4q.W4Q_EALIGN
    assert L.w4a16_gemm_dq(A, 1, A, A, 4, 64, A, 0, None) == w4q.W4Q_EUNSUPPORTED
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
    assert L.w4q_probe_mfma_bf16(A, 0, None, None) == w4q.W4Q_EINVAL


def test_python_front_end_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        w4q.lsq_fwd(w, torch.zeros(4, 2))
