"""w4a16_gemm_dq_noalloc (scratch in a static device array, no allocation) against w4a16_gemm_dq
(caller's scratch) through the C ABI: two calls in a row on the same array, the second smaller,
each equal to the workspace entry point's output and within the product's bound of the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import check_gemm, dev_bf16

pytestmark = pytest.mark.gpu


def _fn():
    return w4q.lib().w4a16_gemm_dq_noalloc


def test_noalloc_matches_workspace_entry_point(dev):
    f = _fn()
    stream = torch.cuda.current_stream().cuda_stream
    # first a shape whose split uses most of the array, then a smaller one (fewer partial tiles,
    # the array still holding the first call's)
    for m, d_out, d_in in ((2048, 12288, 4096), (300, 1000, 768)):
        print("[case] noalloc", m, d_out, d_in, flush=True)
        sys.stdout.flush()
        w = synth.weights(60, 0, d_in, d_out, d_in, 0.005)
        scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 7).astype(np.float32)
        packed, s16 = oracle.pack(w, scale)
        x = synth.calib_x(60, 0, m, m, d_in, 1.0)
        xt = dev_bf16(x, dev)
        pt = torch.from_numpy(packed).to(dev)
        st = torch.from_numpy(s16.view(np.float16)).to(dev)
        want = w4q.w4a16_gemm_dq(xt, pt, st)
        assert w4q.workspace_size("w4a16_gemm_dq", m, d_out, d_in) > 0
        y = torch.full((m, d_out), float("nan"), dtype=torch.float32, device=dev)
        rc = f(xt.data_ptr(), m, pt.data_ptr(), st.data_ptr(), d_out, d_in, y.data_ptr(), 0, stream)
        assert rc == w4q.W4Q_OK, w4q.status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        cols = np.arange(0, d_out, 97)
        yr, ya = oracle.gemm_cols(x, packed, s16, cols, dequant_bf16=True)
        check_gemm(y.cpu().numpy()[:, cols], yr, ya)


def test_noalloc_argument_errors():
    f = _fn()
    A = 4096
    assert f(None, 1, A, A, 4, 256, A, 0, None) == w4q.W4Q_EINVAL
    assert f(A, 0, A, A, 4, 256, A, 0, None) == w4q.W4Q_ESHAPE
    assert f(A + 2, 1, A, A, 4, 256, A, 0, None) == w4q.W4Q_EALIGN
