"""GPU checks of the C-ABI boundary itself: caller-owned scratch (every schedule the library picks
for full, partial or no scratch gives the oracle's result), calls on two streams at once with
their own scratch, and HIP-graph capture and replay of the calls that use scratch."""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import check_gemm, check_hessian, dev_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _ws(nbytes, dev):
    return torch.empty(max(nbytes, 0), dtype=torch.uint8, device=dev) if nbytes > 0 else None


def _packed(stream, d_out, d_in):
    w = synth.weights(stream, 0, 1, d_out, d_in, 0.005)
    scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 7).astype(np.float32)
    return oracle.pack(w, scale)


@pytest.mark.parametrize("n_tok,d", [(2048, 2048), (1000, 1288)])
def test_hessian_any_scratch(dev, n_tok, d):
    # the fastest schedule, a small scratch (fewer, longer ranges) and none (whole tiles): each
    # is exactly symmetric and matches the oracle
    x = synth.calib_x(50, 0, d, n_tok, d, 1.0)
    ref = oracle.hessian(x)
    full = w4q.workspace_size("quant_hessian", n_tok, d)
    assert full > 0
    xt = dev_bf16(x, dev)
    for nb in (full, 3 << 20, 0):
        say("hessian scratch", n_tok, d, nb)
        # through the C ABI: NULL scratch with zero bytes for nb == 0
        h = torch.empty((d, d), dtype=torch.float32, device=dev)
        ws = _ws(nb, dev)
        rc = w4q.lib().quant_hessian(xt.data_ptr(), n_tok, d, h.data_ptr(), 0,
                                     ws.data_ptr() if ws is not None else None, nb,
                                     torch.cuda.current_stream().cuda_stream)
        assert rc == w4q.W4Q_OK
        hn = h.cpu().numpy()
        assert np.array_equal(hn, hn.T)
        check_hessian(hn, ref)


@pytest.mark.parametrize("m,d_out,d_in", [(2048, 2048, 2048), (256, 8192, 2048), (300, 1000, 768)])
def test_gemm_dq_any_scratch(dev, m, d_out, d_in):
    packed, s16 = _packed(51, d_out, d_in)
    x = synth.calib_x(51, 0, m, m, d_in, 1.0)
    cols = np.arange(0, d_out, 7)
    yr, ya = oracle.gemm_cols(x, packed, s16, cols, dequant_bf16=True)
    ye, yea = oracle.gemm_cols(x, packed, s16, cols)
    full = w4q.workspace_size("w4a16_gemm_dq", m, d_out, d_in)
    xt, pt, st = dev_bf16(x, dev), torch.from_numpy(packed).to(dev), torch.from_numpy(s16.view(np.float16)).to(dev)
    for nb in sorted({full, 1 << 20, 0}, reverse=True):
        say("gemm_dq scratch", m, d_out, d_in, nb)
        y = torch.empty((m, d_out), dtype=torch.float32, device=dev)
        ws = _ws(nb, dev)
        rc = w4q.lib().w4a16_gemm_dq(xt.data_ptr(), m, pt.data_ptr(), st.data_ptr(), d_out, d_in,
                                     y.data_ptr(), 0, ws.data_ptr() if ws is not None else None, nb,
                                     torch.cuda.current_stream().cuda_stream)
        assert rc == w4q.W4Q_OK
        check_gemm(y.cpu().numpy()[:, cols], yr, ya)
        # exact weights: the split-weight tiled kernel with full scratch, the per-group kernel
        # otherwise; both follow the exact reading
        ye_g = w4q.w4a16_gemm(xt, pt, st, workspace=ws).cpu().numpy()
        check_gemm(ye_g[:, cols], ye, yea)


def test_two_streams_own_scratch(dev):
    # the same calls on two streams at once, each with its own scratch, give the single-stream
    # results bit for bit (same schedules, no shared state)
    xs = [synth.calib_x(52, i, 0, 4096, 2048, 1.0) for i in range(2)]
    packed, s16 = _packed(52, 8192, 2048)
    pt, st = torch.from_numpy(packed).to(dev), torch.from_numpy(s16.view(np.float16)).to(dev)
    xts = [dev_bf16(x, dev) for x in xs]
    say("two streams")
    want_h = [w4q.quant_hessian(xt) for xt in xts]
    want_y = [w4q.w4a16_gemm_dq(xt[:512], pt, st) for xt in xts]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wsh = [_ws(w4q.workspace_size("quant_hessian", 4096, 2048), dev) for _ in range(2)]
    wsy = [_ws(w4q.workspace_size("w4a16_gemm_dq", 512, 8192, 2048), dev) for _ in range(2)]
    hs = [torch.full((2048, 2048), float("nan"), device=dev) for _ in range(2)]
    ys = [torch.full((512, 8192), float("nan"), device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                w4q.quant_hessian(xts[i], h=hs[i], workspace=wsh[i])
                w4q.w4a16_gemm_dq(xts[i][:512], pt, st, out=ys[i], workspace=wsy[i])
        torch.cuda.synchronize()
        for i in (0, 1):
            assert torch.equal(hs[i], want_h[i]), f"rep {rep} stream {i} hessian"
            assert torch.equal(ys[i], want_y[i]), f"rep {rep} stream {i} gemm_dq"


def test_graph_capture_replay(dev):
    # quant_hessian and w4a16_gemm_dq (both with partial tiles in scratch) captured in one HIP
    # graph: every replay, with eager calls on other buffers in between, equals the eager result
    x = synth.calib_x(53, 0, 0, 2048, 4096, 1.0)
    packed, s16 = _packed(53, 4096, 4096)
    xt = dev_bf16(x, dev)
    pt, st = torch.from_numpy(packed).to(dev), torch.from_numpy(s16.view(np.float16)).to(dev)
    say("graph capture")
    want_h = w4q.quant_hessian(xt)
    want_y = w4q.w4a16_gemm_dq(xt[:1024], pt, st)
    torch.cuda.synchronize()
    wsh = _ws(w4q.workspace_size("quant_hessian", 2048, 4096), dev)
    wsy = _ws(w4q.workspace_size("w4a16_gemm_dq", 1024, 4096, 4096), dev)
    assert wsh is not None and wsy is not None
    h = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
    y = torch.empty((1024, 4096), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, on the capture stream
        w4q.quant_hessian(xt, h=h, workspace=wsh)
        w4q.w4a16_gemm_dq(xt[:1024], pt, st, out=y, workspace=wsy)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4q.quant_hessian(xt, h=h, workspace=wsh)
        w4q.w4a16_gemm_dq(xt[:1024], pt, st, out=y, workspace=wsy)
    xo = dev_bf16(synth.calib_x(53, 1, 0, 512, 4096, 1.0), dev)
    for rep in range(3):
        h.fill_(float("nan"))
        y.fill_(float("nan"))
        other_h = w4q.quant_hessian(xo)                    # eager work between replays
        other_y = w4q.w4a16_gemm_dq(xo, pt, st)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, want_h), f"replay {rep} hessian"
        assert torch.equal(y, want_y), f"replay {rep} gemm_dq"
        del other_h, other_y
    hn = h.cpu().numpy()
    check_hessian(hn, oracle.hessian(x))
