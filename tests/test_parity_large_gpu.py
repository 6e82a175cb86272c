"""GPU parity at the full synthetic sizes (MLP block, 28- and 36-layer decoders), in the launch
configuration the benchmark uses: the GPU computes every output, the oracle recomputes a seeded
sample of them one by one (entries of H, groups of the search, rows of pack/LSQ, output columns
of the W4A16 product), plus properties that hold at any size (bitwise symmetry of H)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import (LSQ_REL, bf16_bits_to_np, check_gemm, check_hessian, check_search, dev_bf16,
                      dev_f32, host_f16_bits)

pytestmark = pytest.mark.gpu
GS = 1.0 / np.sqrt(32 * 7)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _hessian_sampled(x, dev, n_samples=3000, seed=0):
    h = w4q.quant_hessian(dev_bf16(x, dev))
    hn = h.cpu().numpy()
    assert np.array_equal(hn, hn.T)
    d = x.shape[1]
    rng = np.random.default_rng(seed)
    ij = np.stack([rng.integers(0, d, n_samples), rng.integers(0, d, n_samples)], 1)
    ij = np.concatenate([ij, np.stack([np.arange(0, d, 97)] * 2, 1)])  # some diagonal entries
    ref = oracle.hessian_entries(x, ij)
    dref = oracle.hessian_entries(x, np.stack([ij[:, 0], ij[:, 0]], 1))
    dref2 = oracle.hessian_entries(x, np.stack([ij[:, 1], ij[:, 1]], 1))
    check_hessian(hn[ij[:, 0], ij[:, 1]], ref, np.sqrt(dref * dref2))
    return h


def _search_sampled(w, h, alpha, dev, n_samples=2000, seed=1):
    d_out, d_in = w.shape
    G = d_in // 32
    sc, ix, ob, _ = w4q.quant_scale_search(dev_f32(w, dev), h, dev_f32(alpha, dev))
    sc, ix, ob = sc.cpu().numpy(), ix.cpu().numpy(), ob.cpu().numpy()
    rng = np.random.default_rng(seed)
    rows = np.concatenate([rng.integers(0, d_out, n_samples), np.zeros(G, np.int64), np.full(G, d_out - 1)])
    groups = np.concatenate([rng.integers(0, G, n_samples), np.arange(G), np.arange(G)])
    hn = h.cpu().numpy()
    so, io, oo, oao = oracle.scale_search_groups(w, hn, alpha, rows, groups, with_all=True)
    amax = np.abs(w.reshape(d_out, G, 32)).max(axis=2)
    cand = lambda i, k: oracle.candidate(float(amax[rows[i], groups[i]]), float(alpha[k]))
    check_search(ix[rows, groups], sc[rows, groups], ob[rows, groups], io, so, oo, oao, cand)
    return sc


def _pack_rows(w, sc, dev, rows):
    p, s16 = w4q.quant_pack(dev_f32(w, dev), dev_f32(sc, dev))
    pn, sn = p.cpu().numpy(), host_f16_bits(s16)
    po, so = oracle.pack(w[rows], sc[rows])
    assert np.array_equal(pn[rows], po)
    assert np.array_equal(sn[rows], so)
    return p, s16


def _gemm_cols(x, p, s16, dev, cols, bf16_out=False, dq=False):
    fn = w4q.w4a16_gemm_dq if dq else w4q.w4a16_gemm
    y = fn(dev_bf16(x, dev), p, s16, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    if bf16_out:
        yg = bf16_bits_to_np(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        yg = y.cpu().numpy()
    pn = p.cpu().numpy()
    sn = host_f16_bits(s16)
    yr, ya = oracle.gemm_cols(x, pn, sn, cols, dequant_bf16=dq)
    check_gemm(yg[:, cols], yr, ya, bf16_out)


def _lsq_rows(w, sc, g, dev, rows):
    wt, st, gt = dev_f32(w, dev), dev_f32(sc, dev), dev_f32(g, dev)
    gw, gsc, wh = w4q.lsq_bwd(wt, st, gt, GS, with_w_hat=True)
    wh1 = w4q.lsq_fwd(wt, st)
    gw, gsc, wh, wh1 = gw.cpu().numpy(), gsc.cpu().numpy(), wh.cpu().numpy(), wh1.cpu().numpy()
    gwo, gso, who = oracle.lsq_bwd(w[rows], sc[rows], g[rows], GS)
    assert np.array_equal(wh[rows], who) and np.array_equal(wh1[rows], who)
    assert np.array_equal(gw[rows], gwo)
    wr = w[rows].astype(np.float64)
    d = np.repeat(sc[rows].astype(np.float64), 32, axis=1)
    q = np.round(who.astype(np.float64) / np.where(d == 0, 1, d))
    m = (wr >= -8 * d) & (wr <= 7 * d)
    f = np.where(m, q - wr / d, q)
    G = w.shape[1] // 32
    gf = np.abs(g[rows] * f).reshape(len(rows), G, 32).sum(axis=2)
    ga = np.abs(g[rows]).reshape(len(rows), G, 32).sum(axis=2)
    assert np.all(np.abs(gsc[rows] - gso) <= LSQ_REL * GS * gf + GS * 2.0 ** -20 * ga)


# ------------------------------------------------------------- MLP block (8192x2048 gate/up)
@pytest.mark.parametrize("name", ["gate", "up", "down"])
def test_mlp_block(dev, name):
    c = synth.WORKLOADS["mlp_8192x2048"]
    lin = {l.name: l for l in c.linears}[name]
    say("mlp_8192x2048", name, lin.d_out, lin.d_in)
    x = c.x(0, lin.inp)
    w = c.weight(0, lin)
    h = _hessian_sampled(x, dev)
    sc = _search_sampled(w, h, c.alpha(), dev)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(lin.d_out, 24, replace=False))
    p, s16 = _pack_rows(w, sc, dev, rows)
    _lsq_rows(w, sc, c.grad(0, lin), dev, rows)
    cols = np.sort(rng.choice(lin.d_out, 48, replace=False))
    for m in c.gemm_m:                    # 1, 16, 256
        _gemm_cols(x[:m], p, s16, dev, cols)
    _gemm_cols(x[:256], p, s16, dev, cols, dq=True)


# ------------------------------------------- 28-layer decoder stack: search, pack, decode
def test_decoder28_stack_search_pack_decode(dev):
    c = synth.WORKLOADS["decoder28_h1024"]
    rng = np.random.default_rng(4)
    alpha = c.alpha()
    at = dev_f32(alpha, dev)
    n_lin = 0
    decode = []  # (x, packed, scales, y of the single call) of every linear
    for layer in range(c.layers):
        xs = {inp: c.x(layer, inp) for inp in c.inputs()}
        hs = {inp: w4q.quant_hessian(dev_bf16(xv, dev)) for inp, xv in xs.items()}
        for lin in c.linears:
            say("decoder28_h1024 layer", layer, lin.name)
            w = c.weight(layer, lin)
            G = lin.d_in // 32
            sc, ix, ob, _ = w4q.quant_scale_search(dev_f32(w, dev), hs[lin.inp], at)
            p, s16 = w4q.quant_pack(dev_f32(w, dev), sc)
            y = w4q.w4a16_gemm(dev_bf16(xs[lin.inp][:1], dev), p, s16)       # decode, M = 1
            # oracle on a sample of every linear of the stack
            rows = rng.integers(0, lin.d_out, 24)
            groups = rng.integers(0, G, 24)
            hn = hs[lin.inp].cpu().numpy()
            so, io, oo, oao = oracle.scale_search_groups(w, hn, alpha, rows, groups, with_all=True)
            scn, ixn, obn = sc.cpu().numpy(), ix.cpu().numpy(), ob.cpu().numpy()
            amax = np.abs(w.reshape(lin.d_out, G, 32)).max(axis=2)
            check_search(ixn[rows, groups], scn[rows, groups], obn[rows, groups], io, so, oo, oao,
                         lambda i, k: oracle.candidate(float(amax[rows[i], groups[i]]), float(alpha[k])))
            prow = np.unique(rows[:4])
            po, s16o = oracle.pack(w[prow], scn[prow])
            assert np.array_equal(p.cpu().numpy()[prow], po)
            cols = rng.integers(0, lin.d_out, 16)
            yr, ya = oracle.gemm_cols(xs[lin.inp][:1], p.cpu().numpy(), host_f16_bits(s16), cols)
            check_gemm(y.cpu().numpy()[:, cols], yr, ya)
            decode.append((dev_bf16(xs[lin.inp][:1], dev), p, s16, y))
            n_lin += 1
    assert n_lin == 196
    # the whole decode pass as grouped launches (64 problems each): every output agrees with the
    # single call to fp32 rounding of the lane split (relative to the sum of |terms|)
    say("decoder28_h1024 grouped decode over", n_lin, "linears")
    ys = w4q.w4a16_gemv_grouped([d[0] for d in decode], [d[1] for d in decode], [d[2] for d in decode])
    for (xd, p, s16, y1), yg in zip(decode, ys):
        a, b = y1.cpu().numpy().astype(np.float64), yg.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(a - b) <= 1e-5 * (np.abs(a).max() + 1e-30)), np.abs(a - b).max()


# ------------------------------------ 36-layer decoder stack, representative layers
@pytest.mark.parametrize("layer", [0, 35])
def test_decoder36_layer(dev, layer):
    c = synth.WORKLOADS["decoder36_h4096"]
    rng = np.random.default_rng(50 + layer)
    alpha = c.alpha()
    hs, xs = {}, {}
    for inp in c.inputs():
        say("decoder36_h4096 layer", layer, "hessian", inp)
        xs[inp] = c.x(layer, inp)
        hs[inp] = _hessian_sampled(xs[inp], dev, n_samples=1500, seed=layer)
    for lin in c.linears:
        say("decoder36_h4096 layer", layer, lin.name, lin.d_out, lin.d_in)
        w = c.weight(layer, lin)
        sc = _search_sampled(w, hs[lin.inp], alpha, dev, n_samples=1000, seed=layer)
        rows = np.sort(rng.choice(lin.d_out, 8, replace=False))
        p, s16 = _pack_rows(w, sc, dev, rows)
        if lin.name in c.lsq:
            _lsq_rows(w, sc, c.grad(layer, lin), dev, rows)
        x = xs[lin.inp]
        cols = np.sort(rng.choice(lin.d_out, 8, replace=False))
        _gemm_cols(x[:1], p, s16, dev, cols)                    # decode
        if lin.name in ("gate", "down"):
            _gemm_cols(x[:2048], p, s16, dev, cols, bf16_out=(lin.name == "down"))   # prefill
            _gemm_cols(x[:2048], p, s16, dev, cols, bf16_out=(lin.name == "gate"), dq=True)
