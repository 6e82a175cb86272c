"""GPU parity of every step against the CPU oracle (the 256x512 and 2048x2048 layers in full, edge
cases, ragged shapes).  Inputs are the seeded synthetic layers of w4a16_group_wise_amd.synth; each stage is
fed identical inputs on both sides (e.g. the search gets the GPU's fp32 H on both sides)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import (GEMM_REL, LSQ_REL, bf16_bits_to_np, check_gemm, check_hessian,
                      check_search, dev_bf16, dev_f32, host_bf16_bits, host_f16_bits, search_bound)

pytestmark = pytest.mark.gpu
GS = 1.0 / np.sqrt(32 * 7)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _search_both(w, h_gpu, alpha, dev, with_all=True):
    wt, ht, at = dev_f32(w, dev), dev_f32(h_gpu, dev), dev_f32(alpha, dev)
    sc, ix, ob, oa = w4q.quant_scale_search(wt, ht, at, with_obj=True, with_obj_all=with_all)
    torch.cuda.synchronize()
    so, io, oo, oao = oracle.scale_search(w, h_gpu, alpha, with_all=True)
    return (sc.cpu().numpy(), ix.cpu().numpy(), ob.cpu().numpy(),
            None if oa is None else oa.cpu().numpy(), so, io, oo, oao)


def _cand_fn(w, alpha):
    G = w.shape[1] // 32
    amax = np.abs(w.reshape(w.shape[0], G, 32)).max(axis=2).reshape(-1)
    return lambda i, k: oracle.candidate(float(amax[i]), float(alpha[k]))


# ---------------------------------------------------------------------------------- Hessian
@pytest.mark.parametrize("wl", ["linear_256x512", "proj_2048x2048"])
def test_hessian_workload(dev, wl):
    c = synth.WORKLOADS[wl]
    x = c.x(0, "attn")
    say("hessian", wl, x.shape)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    assert np.array_equal(h, h.T)
    check_hessian(h, oracle.hessian(x))


# (45, 5640): wide enough for the 256-wide tiles, ragged in features (22 * 256 + 8) and tokens
@pytest.mark.parametrize("n_tok,d", [(1, 8), (100, 136), (65, 256), (130, 520), (45, 5640)])
def test_hessian_ragged(dev, n_tok, d):
    x = synth.calib_x(31, 0, n_tok, n_tok, d, 1.0)
    say("hessian ragged", n_tok, d)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    assert np.array_equal(h, h.T)
    check_hessian(h, oracle.hessian(x))


@pytest.mark.parametrize("d", [264, 5888])
def test_hessian_accumulate(dev, d):
    x = synth.calib_x(31, 1, 0, 192, d, 1.5)
    say("hessian accumulate", d)
    h = w4q.quant_hessian(dev_bf16(x[:100], dev))
    w4q.quant_hessian(dev_bf16(x[100:], dev), h=h, accumulate=True)
    hn = h.cpu().numpy()
    assert np.array_equal(hn, hn.T)
    check_hessian(hn, oracle.hessian(x))


# ------------------------------------------------------------------------------ scale search
@pytest.mark.parametrize("wl", ["linear_256x512", "proj_2048x2048"])
def test_search_workload(dev, wl):
    c = synth.WORKLOADS[wl]
    lin = c.linears[0]
    w = c.weight(0, lin)
    x = c.x(0, lin.inp)
    say("search", wl, w.shape)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    alpha = c.alpha()
    sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev)
    n_tie = check_search(ix, sc, ob, io, so, oo, oao, _cand_fn(w, alpha))
    assert n_tie <= max(2, ix.size // 5000)
    # every candidate's objective, not only the chosen one
    err = np.abs(oa.astype(np.float64) - oao)
    assert np.all(err <= 1e-5 * oao + 1e-30)


def test_search_identity_hessian_and_edges(dev):
    # all-zero groups, outlier-only groups, weights on midpoints, fp16-subnormal scales
    d_out, d_in = 70, 32 * 7
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    w[0, :] = 0.0                                          # all-zero row
    w[1, 32:64] = 0.0
    w[1, 40] = 0.7                                         # outlier-only group
    w[2, :] = (rng.standard_normal(d_in) * 1e-6).astype(np.float32)  # subnormal fp16 scales
    w[3, :32] = np.float32(0.25) * (np.arange(32) % 16 - 7.5).astype(np.float32)  # midpoints
    w[4, :32] = np.float32(1e-7)
    h = np.eye(d_in, dtype=np.float32) * np.float32(2.0)
    alpha = synth.alpha_grid(17, 0.3, 1.0)
    say("search edges")
    sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev)
    check_search(ix, sc, ob, io, so, oo, oao, _cand_fn(w, alpha))
    assert np.all(sc[0] == 0) and np.all(ix[0] == 0)


def test_search_ragged_and_single_candidate(dev):
    x = synth.calib_x(31, 2, 0, 96, 96, 1.0)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    w = synth.weights(31, 2, 1, 300, 96, 0.01)
    for K in (1, 3, 255):
        alpha = synth.alpha_grid(K, 0.4, 1.0)
        say("search ragged K", K)
        sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev)
        check_search(ix, sc, ob, io, so, oo, oao, _cand_fn(w, alpha))


@pytest.mark.parametrize("sigma", [1.5, 2.5])
def test_search_wide_channel_spread(dev, sigma):
    # lognormal(0, sigma) channel scales spread each H_gg over many binades (about 2^40 between
    # its largest and smallest entries at sigma 2.5), the hard case for a split-precision score
    x = synth.calib_x(32, 0, 0, 1024, 1024, sigma)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    w = synth.weights(32, 0, 1, 192, 1024, 0.005)
    alpha = synth.alpha_grid(40, 0.4, 1.0)
    say("search channel spread", sigma)
    sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev)
    check_search(ix, sc, ob, io, so, oo, oao, _cand_fn(w, alpha))
    err = np.abs(oa.astype(np.float64) - oao)
    assert np.all(err <= 1e-5 * oao + 1e-30), f"worst rel {np.max(err / (oao + 1e-30)):.3g}"


# Correlated calibration activations: X = (Z M + eps N) c, a shared rank-r mixing plus a small
# independent part, so every 32x32 block of H is nearly rank r (condition numbers 1e5 .. 1e9 with
# the lognormal channel factors).  Errors along the shared directions are weighted far more than
# the others (the blog's case for the Hessian objective), and e^T H e cancels heavily: the
# fp32-level first pass can then neither rank the candidates nor give the objective to 1e-5, and
# the kernel must detect it from its error bound.  Both output modes run: with obj_all every
# candidate's objective must be accurate; without it only the chosen one, and the re-scoring is
# restricted to the candidates the bound cannot rule out.
@pytest.mark.parametrize("d_out,d,n_tok,rank,eps", [(256, 512, 128, 4, 0.3), (256, 512, 2048, 4, 0.1),
                                                    (512, 2048, 2048, 2, 0.01), (96, 4096, 1024, 8, 0.03)])
@pytest.mark.parametrize("with_all", [False, True])
def test_search_correlated(dev, d_out, d, n_tok, rank, eps, with_all):
    x = synth.correlated_x(41, rank, d, n_tok, d, rank, eps)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    w = synth.weights(41, rank, d_out, d_out, d, 0.005)
    alpha = synth.alpha_grid(40, 0.4, 1.0)
    say("search correlated", d_out, d, n_tok, rank, eps, "obj_all" if with_all else "")
    sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev, with_all=with_all)
    n_tie = check_search(ix, sc, ob, io, so, oo, oao, _cand_fn(w, alpha))
    assert n_tie <= max(2, ix.size // 5000)
    if with_all:
        err = np.abs(oa.astype(np.float64) - oao)
        assert np.all(err <= 1e-5 * oao + 1e-30), f"worst rel {np.max(err / (oao + 1e-30)):.3g}"


@pytest.mark.parametrize("corr", [False, True])
def test_search_error_within_radius(dev, corr):
    # every first-pass score the kernel keeps lies within its radius 2^-18 |e|^T |H_gg| |e| of
    # the fp64 value (re-scored ones are fp64-accurate), on iid lognormal(0, 2.5) channels and
    # on correlated activations
    if corr:
        x = synth.correlated_x(42, 0, 0, 1024, 512, 4, 0.05)
    else:
        x = synth.calib_x(42, 0, 1, 1024, 512, 2.5)
    h = w4q.quant_hessian(dev_bf16(x, dev)).cpu().numpy()
    w = synth.weights(42, 0, 2, 192, 512, 0.005)
    alpha = synth.alpha_grid(40, 0.4, 1.0)
    say("search radius", "correlated" if corr else "iid sigma 2.5")
    sc, ix, ob, oa, so, io, oo, oao = _search_both(w, h, alpha, dev, with_all=True)
    B = search_bound(w, h, alpha, _cand_fn(w, alpha))
    err = np.abs(oa.astype(np.float64) - oao)
    assert np.all(err <= 2.0 ** -18 * B + 1e-30), f"worst err/B {np.max(err / (B + 1e-300)):.3g}"


def test_search_deterministic(dev):
    c = synth.WORKLOADS["linear_256x512"]
    w = c.weight(0, c.linears[0])
    h = w4q.quant_hessian(dev_bf16(c.x(0, "attn"), dev))
    wt, at = dev_f32(w, dev), dev_f32(c.alpha(), dev)
    say("search determinism")
    a = [t.cpu() for t in w4q.quant_scale_search(wt, h, at)[:3]]
    b = [t.cpu() for t in w4q.quant_scale_search(wt, h, at)[:3]]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ---------------------------------------------------------------------------------- pack
@pytest.mark.parametrize("wl", ["linear_256x512", "proj_2048x2048"])
def test_pack_workload(dev, wl):
    c = synth.WORKLOADS[wl]
    w = c.weight(0, c.linears[0])
    G = w.shape[1] // 32
    # scales: max-based candidates stretched per group (fp32, not yet on the fp16 grid)
    rng = np.random.default_rng(c.stream)
    scale = (np.abs(w.reshape(-1, G, 32)).max(axis=2) / 7 * rng.uniform(0.4, 1.0, (w.shape[0], G))).astype(np.float32)
    say("pack", wl)
    p, s16 = w4q.quant_pack(dev_f32(w, dev), dev_f32(scale, dev))
    po, so = oracle.pack(w, scale)
    assert np.array_equal(p.cpu().numpy(), po)
    assert np.array_equal(host_f16_bits(s16), so)


def test_pack_edges(dev):
    d = np.float32(0.25)
    mids = ((np.arange(-9, 8) + 0.5) * d).astype(np.float32)
    w = np.zeros((3, 64), np.float32)
    w[0, :mids.size] = mids
    w[0, 17:19] = [7 * d, -8 * d]
    w[1, :] = 1e-3
    scale = np.array([[d, d], [0.0, 1e-7], [6e-8, 65504.0]], np.float32)
    say("pack edges")
    p, s16 = w4q.quant_pack(dev_f32(w, dev), dev_f32(scale, dev))
    po, so = oracle.pack(w, scale)
    assert np.array_equal(p.cpu().numpy(), po)
    assert np.array_equal(host_f16_bits(s16), so)


# ------------------------------------------------------------------------------------ LSQ
def _lsq_check(w, scale, g, dev, fused):
    wt, st, gt = dev_f32(w, dev), dev_f32(scale, dev), dev_f32(g, dev)
    wh = w4q.lsq_fwd(wt, st).cpu().numpy()
    gw, gsc, wh2 = w4q.lsq_bwd(wt, st, gt, GS, with_w_hat=fused)
    gw, gsc = gw.cpu().numpy(), gsc.cpu().numpy()
    gwo, gsco, who = oracle.lsq_bwd(w, scale, g, GS)
    assert np.array_equal(wh, who)
    assert np.array_equal(oracle.lsq_fwd(w, scale), who)
    if fused:
        assert np.array_equal(wh2.cpu().numpy(), who)
    assert np.array_equal(gw, gwo)
    # tolerance: 1e-4 * gs * sum|G f| + gs * 2^-20 * sum|G|
    d = np.repeat(scale.astype(np.float64), 32, axis=1)
    q = who.astype(np.float64) / np.where(d == 0, 1, d)
    m = (w >= -8 * d) & (w <= 7 * d)
    f = np.where(m, q - w / d, q)
    G = w.shape[1] // 32
    gf = np.abs(g * f).reshape(w.shape[0], G, 32).sum(axis=2)
    ga = np.abs(g).reshape(w.shape[0], G, 32).sum(axis=2)
    tol = LSQ_REL * GS * gf + GS * 2.0 ** -20 * ga
    assert np.all(np.abs(gsc - gsco) <= tol)


@pytest.mark.parametrize("fused", [False, True])
def test_lsq_linear_256x512(dev, fused):
    c = synth.WORKLOADS["linear_256x512"]
    lin = c.linears[0]
    w = c.weight(0, lin)
    g = c.grad(0, lin)
    G = w.shape[1] // 32
    rng = np.random.default_rng(5)
    scale = (np.abs(w.reshape(-1, G, 32)).max(axis=2) / 7 * rng.uniform(0.3, 1.1, (w.shape[0], G))).astype(np.float32)
    say("lsq linear_256x512 fused", fused)
    _lsq_check(w, scale, g, dev, fused)


def test_lsq_edges(dev):
    d = np.float32(0.25)
    w = np.zeros((3, 64), np.float32)
    w[0, :8] = [0.375, 1.875, 1.75, -2.125, -2.0, 0.1, 7 * 0.25, -8 * 0.25]
    w[0, 8:32] = ((np.arange(24) - 12) * 0.125).astype(np.float32)
    w[1, :] = np.linspace(-3, 3, 64, dtype=np.float32)
    # fp32-subnormal steps: 2^-127 (its reciprocal 2^127 is finite) and 1e-40 (reciprocal overflows)
    tiny = [np.float32(2.0 ** -127), np.float32(1e-40)]
    for j in range(2):
        k = np.arange(32) - 16.0
        w[2, 32 * j:32 * j + 32] = (k * 0.7 * np.float64(tiny[j])).astype(np.float32)
    scale = np.array([[d, np.float32(0.013)], [np.float32(1e-30), np.float32(100.0)], tiny], np.float32)
    g = np.random.default_rng(9).standard_normal((3, 64)).astype(np.float32)
    say("lsq edges")
    _lsq_check(w, scale, g, dev, True)


# ----------------------------------------------------------------------------------- GEMM
def _packed_layer(wl, layer=0):
    c = synth.WORKLOADS[wl]
    lin = c.linears[0]
    w = c.weight(layer, lin)
    G = w.shape[1] // 32
    scale = (np.abs(w.reshape(-1, G, 32)).max(axis=2) / 7).astype(np.float32)
    packed, s16 = oracle.pack(w, scale)
    return c, lin, packed, s16


@pytest.mark.parametrize("wl,m", [("linear_256x512", 1), ("proj_2048x2048", 1), ("proj_2048x2048", 4),
                                  ("proj_2048x2048", 16), ("proj_2048x2048", 3), ("proj_2048x2048", 17),
                                  ("proj_2048x2048", 256)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_gemm_workload(dev, wl, m, bf16_out):
    c, lin, packed, s16 = _packed_layer(wl)
    x = c.x(0, lin.inp)[:m]
    say("gemm", wl, "m", m, "bf16", bf16_out)
    y = w4q.w4a16_gemm(dev_bf16(x, dev), torch.from_numpy(packed).to(dev),
                       torch.from_numpy(s16.view(np.float16)).to(dev),
                       out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    yg = bf16_bits_to_np(host_bf16_bits(y)) if bf16_out else y.cpu().numpy()
    cols = np.arange(packed.shape[0]) if m <= 16 else np.arange(0, packed.shape[0], 7)
    yr, ya = oracle.gemm_cols(x, packed, s16, cols)
    check_gemm(yg[:, cols], yr, ya, bf16_out)


# 2..16 rows run on the matrix-core kernel: G % 8 == 0 (16-byte scale loads) or not, fewer
# groups than wavefronts, ragged weight rows, one or two 16-row tiles per workgroup
# (d_out below or above 8192), 8 or 16 wavefronts per workgroup (d_in >= 8192 with M <= 8)
@pytest.mark.parametrize("m,d_out,d_in", [(1, 1, 32), (1, 3, 96), (2, 130, 224), (5, 64, 1056),
                                          (3, 1000, 256), (16, 33, 8192), (9, 257, 2048), (16, 31, 64),
                                          (4, 8200, 64), (11, 8224, 512),
                                          (5, 40, 8192), (3, 50, 8224), (8, 17, 16384), (2, 9, 12320),
                                          (1, 77, 3072), (33, 200, 160), (130, 129, 96)])
def test_gemm_ragged(dev, m, d_out, d_in):
    w = synth.weights(32, 0, d_out, d_out, d_in, 0.01)
    scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 6).astype(np.float32)
    scale[0, 0] = 0.0                                        # an all-zero code group
    packed, s16 = oracle.pack(w, scale)
    x = synth.calib_x(32, 0, m, m, d_in, 1.0)
    say("gemm ragged", m, d_out, d_in)
    y = w4q.w4a16_gemm(dev_bf16(x, dev), torch.from_numpy(packed).to(dev),
                       torch.from_numpy(s16.view(np.float16)).to(dev))
    yr, ya = oracle.gemm_cols(x, packed, s16)
    check_gemm(y.cpu().numpy(), yr, ya)


def test_gemm_rows_agree_with_m1(dev):
    c, lin, packed, s16 = _packed_layer("proj_2048x2048")
    x = c.x(0, lin.inp)[:40]
    pt = torch.from_numpy(packed).to(dev)
    st = torch.from_numpy(s16.view(np.float16)).to(dev)
    say("gemm row consistency")
    yb = w4q.w4a16_gemm(dev_bf16(x, dev), pt, st).cpu().numpy()
    yr, ya = oracle.gemm_cols(x, packed, s16)
    for r in (0, 17, 39):
        y1 = w4q.w4a16_gemm(dev_bf16(x[r:r + 1], dev), pt, st).cpu().numpy()
        assert np.all(np.abs(y1[0] - yb[r]) <= 2 * GEMM_REL * ya[r])


def test_gemm_zero_codes_exact(dev):
    packed = np.zeros((64, 1024), np.uint8)
    s16 = np.full((64, 64), 0x3C00, np.uint16)
    x = synth.calib_x(33, 0, 0, 4, 2048, 1.0)
    say("gemm zero codes")
    for m in (1, 4, 32):
        y = w4q.w4a16_gemm(dev_bf16(x[:m] if m <= 4 else np.tile(x, (8, 1)), dev),
                           torch.from_numpy(packed).to(dev),
                           torch.from_numpy(s16.view(np.float16)).to(dev))
        assert torch.count_nonzero(y).item() == 0


# ------------------------------------------------ matrix-core product, both weight readings
# shapes on the 256x256-tile kernel (d_in % 256 == 0): ragged rows / columns, K split over
# workgroups (partial tiles) or not, and several tiles per workgroup; the last shape has enough
# output tiles that exact weights take the per-group kernel instead
@pytest.mark.parametrize("m,d_out,d_in", [(17, 40, 256), (300, 520, 512), (64, 256, 4096),
                                          (513, 1000, 768), (256, 2304, 1024), (1100, 4100, 256)])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_mma_shapes(dev, m, d_out, d_in, dq):
    w = synth.weights(34, 0, d_out, d_out, d_in, 0.01)
    scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 7).astype(np.float32)
    scale[1 % d_out, 0] = 0.0                                  # an all-zero code group
    packed, s16 = oracle.pack(w, scale)
    x = synth.calib_x(34, 0, m, m, d_in, 1.0)
    say("gemm mma", m, d_out, d_in, "dq" if dq else "exact")
    fn = w4q.w4a16_gemm_dq if dq else w4q.w4a16_gemm
    y = fn(dev_bf16(x, dev), torch.from_numpy(packed).to(dev), torch.from_numpy(s16.view(np.float16)).to(dev))
    yg = y.cpu().numpy()
    cols = np.arange(d_out) if d_out * m <= 200000 else np.arange(0, d_out, 5)
    yr, ya = oracle.gemm_cols(x, packed, s16, cols, dequant_bf16=dq)
    check_gemm(yg[:, cols], yr, ya)
    # each entry point follows its own weight reading: its distance to the other reading's
    # reference is far above its distance to its own (fp32 accumulation only)
    yo, _ = oracle.gemm_cols(x, packed, s16, cols, dequant_bf16=not dq)
    e_own = np.max(np.abs(yg[:, cols] - yr) / ya)
    e_other = np.max(np.abs(yg[:, cols] - yo) / ya)
    assert e_own * 4 < e_other, (e_own, e_other)


@pytest.mark.parametrize("wl,m", [("linear_256x512", 1), ("proj_2048x2048", 16), ("proj_2048x2048", 2048)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_gemm_dq_workload(dev, wl, m, bf16_out):
    c, lin, packed, s16 = _packed_layer(wl)
    x = c.x(0, lin.inp)[:m]
    say("gemm dq", wl, "m", m, "bf16", bf16_out)
    y = w4q.w4a16_gemm_dq(dev_bf16(x, dev), torch.from_numpy(packed).to(dev),
                          torch.from_numpy(s16.view(np.float16)).to(dev),
                          out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    yg = bf16_bits_to_np(host_bf16_bits(y)) if bf16_out else y.cpu().numpy()
    cols = np.arange(packed.shape[0]) if m <= 16 else np.arange(0, packed.shape[0], 7)
    yr, ya = oracle.gemm_cols(x, packed, s16, cols, dequant_bf16=True)
    check_gemm(yg[:, cols], yr, ya, bf16_out)
    if not bf16_out:
        # the kernel follows the bf16 reading, not the exact one: its distance to the bf16-weight
        # reference (fp32 accumulation only) is far below its distance to the exact weights
        ye, _ = oracle.gemm_cols(x, packed, s16, cols)
        e_dq = np.max(np.abs(yg[:, cols] - yr) / ya)
        e_ex = np.max(np.abs(yg[:, cols] - ye) / ya)
        assert e_dq * 4 < e_ex, (e_dq, e_ex)


# ------------------------------------------------------------ grouped one-row products (decode)
@pytest.mark.parametrize("bf16_out", [False, True])
def test_gemv_grouped(dev, bf16_out):
    # the shapes of the 28-layer decoder's linears, a ragged one (3 groups per row: one lane per
    # row) and enough problems for two launches (64 per launch)
    shapes = [(2048, 1024), (1024, 1024), (1024, 1024), (1024, 2048), (3072, 1024), (3072, 1024),
              (1024, 3072), (77, 96)] * 9
    xs, ps, ss, refs = [], [], [], []
    for i, (d_out, d_in) in enumerate(shapes):
        w = synth.weights(36, i, d_out, d_out, d_in, 0.01)
        scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 7).astype(np.float32)
        packed, s16 = oracle.pack(w, scale)
        x = synth.calib_x(36, i, 0, 1, d_in, 1.0)
        xs.append(dev_bf16(x, dev))
        ps.append(torch.from_numpy(packed).to(dev))
        ss.append(torch.from_numpy(s16.view(np.float16)).to(dev))
        refs.append((x, packed, s16))
    say("gemv grouped", len(shapes), "problems, bf16" if bf16_out else "fp32")
    ys = w4q.w4a16_gemv_grouped(xs, ps, ss, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    for y, (x, packed, s16) in zip(ys, refs):
        yg = bf16_bits_to_np(host_bf16_bits(y)) if bf16_out else y.cpu().numpy()
        yr, ya = oracle.gemm_cols(x, packed, s16)
        check_gemm(yg, yr, ya, bf16_out)


def test_gemv_plan_graph_replays(dev):
    # a prepared grouped call captured in a HIP graph: every replay (with eager work on the same
    # buffers between replays) gives the eager result, which matches the oracle
    shapes = [(2048, 1024), (1024, 3072), (77, 96), (4096, 4096)]
    xs, ps, ss, refs = [], [], [], []
    for i, (d_out, d_in) in enumerate(shapes):
        w = synth.weights(37, i, d_out, d_out, d_in, 0.01)
        scale = (np.abs(w.reshape(d_out, -1, 32)).max(axis=2) / 7).astype(np.float32)
        packed, s16 = oracle.pack(w, scale)
        x = synth.calib_x(37, i, 0, 1, d_in, 1.0)
        xs.append(dev_bf16(x, dev))
        ps.append(torch.from_numpy(packed).to(dev))
        ss.append(torch.from_numpy(s16.view(np.float16)).to(dev))
        refs.append((x, packed, s16))
    say("gemv plan in a graph", len(shapes), "problems")
    plan = w4q.GemvGroupPlan(xs, ps, ss)
    eager = [y.clone() for y in plan()]
    torch.cuda.synchronize()
    for y, (x, packed, s16) in zip(eager, refs):
        yr, ya = oracle.gemm_cols(x, packed, s16)
        check_gemm(y.cpu().numpy(), yr, ya, False)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    for rep in range(3):
        for y in plan.outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(plan.outs, eager):
            assert torch.equal(y, e), f"replay {rep}"


# Rows whose codes are zero except on a few of the channels where |x| is smallest, with widely
# spread channel scales (lognormal sigma 2.5): the product is tiny next to sum |x|, so an error that
# scales with sum |x| instead of sum |x * w_hat| would break the bound.  One-row (vector) and
# 2..16-row (matrix-core) paths, single and grouped calls.
@pytest.mark.parametrize("m", [1, 4, 16])
def test_gemv_sparse_codes_on_small_activations(dev, m):
    d_out, d_in = 256, 4096
    x = synth.calib_x(38, 0, m, m, d_in, 2.5)
    order = np.argsort(np.abs(bf16_bits_to_np(x[0])))          # smallest |x| first
    rng = np.random.default_rng(38 + m)
    q = np.zeros((d_out, d_in), np.int64)
    for r in range(d_out):
        nz = 1 + r % 4
        pos = order[rng.choice(16, nz, replace=False)]          # among the 16 smallest channels
        q[r, pos] = rng.choice([-8, -5, -1, 1, 3, 7], nz)
    s = (rng.uniform(1e-3, 1e-2, (d_out, d_in // 32))).astype(np.float16).astype(np.float32)
    w = (q * np.repeat(s, 32, axis=1)).astype(np.float32)      # exactly s * q
    packed, s16 = oracle.pack(w, s)
    pt = torch.from_numpy(packed).to(dev)
    st = torch.from_numpy(s16.view(np.float16)).to(dev)
    say("gemv sparse codes, m", m)
    y = w4q.w4a16_gemm(dev_bf16(x, dev), pt, st).cpu().numpy()
    yr, ya = oracle.gemm_cols(x, packed, s16)
    check_gemm(y, yr, ya)
    if m == 1:
        yg = w4q.w4a16_gemv_grouped([dev_bf16(x, dev)] * 3, [pt] * 3, [st] * 3)
        for t in yg:
            check_gemm(t.cpu().numpy(), yr, ya)


# ------------------------------------------------------- fused QAT update (LSQ + Adam, in place)
def _adam_check(w0, s0, g, st, dev, step, rows=None, lr_w=1e-3, lr_s=1e-4, wd=0.01):
    """One GPU step from state st (host arrays); checks it against the oracle fed the same inputs
    and returns the GPU's new state."""
    wt, sct, gt = dev_f32(w0, dev), dev_f32(s0, dev), dev_f32(g, dev)
    mw, vw, ms, vs = (dev_f32(a, dev) for a in st)
    wh, ds = w4q.lsq_adam_step(wt, sct, gt, GS, mw, vw, ms, vs, lr_w=lr_w, lr_s=lr_s, step=step,
                               weight_decay=wd, scale_min=1e-8, with_w_hat_next=True, with_grad_scale=True)
    torch.cuda.synchronize()
    out = {k: t.cpu().numpy() for k, t in (("w", wt), ("scale", sct), ("m_w", mw), ("v_w", vw), ("m_s", ms),
                                           ("v_s", vs), ("w_hat", wh), ("ds", ds))}
    sel = slice(None) if rows is None else rows
    hp = oracle.adam_hparams(lr_w, lr_s, weight_decay=wd, step=step, scale_min=1e-8)
    o = oracle.lsq_adam_step(w0[sel], s0[sel], g[sel], GS, *(a[sel] for a in st), hp, with_w_hat=False)
    # step-size gradient: the LSQ backward's bound
    d = np.repeat(s0[sel].astype(np.float64), 32, axis=1)
    wr = w0[sel].astype(np.float64)
    q = np.array([[oracle.code(a, b) for a, b in zip(ra, rb)] for ra, rb in zip(wr, d)], np.float64)
    m = (wr >= -8 * d) & (wr <= 7 * d)
    f = np.where(m, q - wr / d, q)
    G = w0.shape[1] // 32
    gf = np.abs(g[sel] * f).reshape(-1, G, 32).sum(axis=2)
    ga = np.abs(g[sel]).reshape(-1, G, 32).sum(axis=2)
    assert np.all(np.abs(out["ds"][sel] - o["ds"]) <= LSQ_REL * GS * gf + GS * 2.0 ** -20 * ga)
    # weights and their moments: a few fp32 roundings of each update
    u = 2.0 ** -22
    gw = np.where(m, g[sel], 0.0)
    # the first moment can cancel (b1 m0 against (1 - b1) g): its rounding error scales with
    # b1 |m0| + (1 - b1) |g|, not with |m|, and so does the update's
    b1, b2, c1, c2 = hp[2], hp[3], hp[6], hp[7]
    a_w = b1 * np.abs(st[0][sel]) + (1 - b1) * np.abs(gw)
    assert np.all(np.abs(out["m_w"][sel] - o["m_w"]) <= u * a_w + 1e-37)
    assert np.all(np.abs(out["v_w"][sel] - o["v_w"]) <= u * (b2 * st[1][sel] + (1 - b2) * gw * gw) + 1e-37)
    upd = (a_w / c1) / (np.sqrt(o["v_w"].astype(np.float64) / c2) + 1e-8)
    tol_w = 2.0 ** -22 * np.abs(o["w"]) + lr_w * 8 * 2.0 ** -24 * (upd + wd * np.abs(w0[sel]))
    assert np.all(np.abs(out["w"][sel] - o["w"]) <= tol_w + 1e-37)
    # the steps' update from the GPU's own gradient (stage-isolated), then the next forward on the
    # GPU's updated weights and steps
    o2 = oracle.lsq_adam_step(w0[sel], s0[sel], g[sel], GS, *(a[sel] for a in st), hp,
                              ext_ds=out["ds"][sel].astype(np.float64), with_w_hat=False)
    a_s = b1 * np.abs(st[2][sel]) + (1 - b1) * np.abs(out["ds"][sel].astype(np.float64))
    us = (a_s / c1) / (np.sqrt(o2["v_s"].astype(np.float64) / c2) + 1e-8)
    assert np.all(np.abs(out["m_s"][sel] - o2["m_s"]) <= u * a_s + 1e-37)
    assert np.all(np.abs(out["v_s"][sel] - o2["v_s"]) <= u * np.abs(o2["v_s"]) + 1e-37)
    assert np.all(np.abs(out["scale"][sel] - o2["scale"]) <= 2.0 ** -22 * np.abs(o2["scale"]) + lr_s * 8 * 2.0 ** -24 * us)
    assert np.array_equal(out["w_hat"][sel], oracle.lsq_fwd(out["w"][sel], out["scale"][sel]))
    return out


@pytest.mark.parametrize("wl,rows", [("linear_256x512", None), ("mlp_8192x2048", 40)])
def test_lsq_adam_steps(dev, wl, rows):
    c = synth.WORKLOADS[wl]
    lin = c.linears[0]
    w = c.weight(0, lin)
    g = c.grad(0, lin)
    G = w.shape[1] // 32
    rng = np.random.default_rng(8)
    s = (np.abs(w.reshape(-1, G, 32)).max(axis=2) / 7 * rng.uniform(0.5, 1.1, (w.shape[0], G))).astype(np.float32)
    st = (np.zeros_like(w), np.zeros_like(w), np.zeros_like(s), np.zeros_like(s))
    sel = None if rows is None else np.sort(rng.choice(w.shape[0], rows, replace=False))
    for step in (1, 2, 3):
        say("lsq adam", wl, "step", step)
        out = _adam_check(w, s, g, st, dev, step, rows=sel)
        w, s = out["w"], out["scale"]
        st = (out["m_w"], out["v_w"], out["m_s"], out["v_s"])
        g = (g * np.float32(0.9) + np.float32(0.1)).astype(np.float32)     # a different upstream gradient


# The one-row product converts codes through an LDS table on launches of >= 48 MB of codes (and
# by byte selects below): four 8192 x 4096 problems in one grouped launch take the table path.
# One problem holds rows whose codes are zero except on a few of the smallest activations
# (lognormal sigma 2.5), the case an offset encoding of the codes would fail.
def test_gemv_grouped_table_path(dev):
    d_out, d_in = 8192, 4096
    rng = np.random.default_rng(61)
    probs = []
    for p in range(4):
        x = synth.calib_x(61, p, 0, 1, d_in, 2.5 if p == 0 else 1.0)
        if p == 0:
            order = np.argsort(np.abs(bf16_bits_to_np(x[0])))
            q = np.zeros((d_out, d_in), np.int8)
            for r in range(0, d_out):
                nz = 1 + r % 4
                q[r, order[rng.choice(16, nz, replace=False)]] = rng.choice([-8, -5, -1, 1, 3, 7], nz)
        else:
            q = rng.integers(-8, 8, (d_out, d_in)).astype(np.int8)
        nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
        packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
        s16 = rng.uniform(1e-3, 1e-2, (d_out, d_in // 32)).astype(np.float16).view(np.uint16)
        probs.append((x, packed, s16))
    say("gemv grouped table path, 4 x 8192 x 4096")
    xs = [dev_bf16(x, dev) for x, _, _ in probs]
    ps = [torch.from_numpy(pk).to(dev) for _, pk, _ in probs]
    ss = [torch.from_numpy(s.view(np.float16)).to(dev) for _, _, s in probs]
    ys = w4q.w4a16_gemv_grouped(xs, ps, ss)
    for i, (x, packed, s16) in enumerate(probs):
        cols = np.sort(rng.choice(d_out, 48, replace=False))
        yr, ya = oracle.gemm_cols(x, packed, s16, cols)
        check_gemm(ys[i].cpu().numpy()[:, cols], yr, ya)
        y1 = w4q.w4a16_gemm(xs[i], ps[i], ss[i]).cpu().numpy().astype(np.float64)
        yg = ys[i].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(yg - y1) <= 1e-5 * (np.abs(y1).max() + 1e-30))
