"""The 36-layer hidden-4096 decoder stack run whole, layer by layer, as the benchmark runs it: the
Hessians of the 4 layer inputs, search and pack of all 7 linears, LSQ forward and backward on gate
and up, the M=2048 prefill product (exact and bf16-dequantized weights) and the M=1 decode product
(single and grouped per decoder phase) on all 7 linears.  Inputs are drawn on the GPU with the
seeded device generators (per layer); the oracle recomputes a seeded sample of every output from
the same tensors: Hessian entries, groups of the search, rows of pack and LSQ, output columns of
the products.  Layers run in chunks of 6 so that every test stays short."""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import LSQ_REL, check_gemm, check_hessian, check_search, host_bf16_bits, host_f16_bits

pytestmark = pytest.mark.gpu
GS = 1.0 / np.sqrt(32 * 7)
C = synth.WORKLOADS["decoder36_h4096"]
CHUNK = 6


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _hessian_sample(xt, h, rng, n=200):
    d = xt.shape[1]
    ij = np.stack([rng.integers(0, d, n), rng.integers(0, d, n)], 1)
    ij = np.concatenate([ij, np.stack([ij[:8, 0]] * 2, 1)])
    cols = np.unique(ij)
    sub = host_bf16_bits(xt[:, torch.from_numpy(cols).to(xt.device)])       # [n_tok][len(cols)]
    loc = {c: i for i, c in enumerate(cols)}
    lij = np.vectorize(loc.get)(ij)
    ref = oracle.hessian_entries(sub, lij)
    dii = oracle.hessian_entries(sub, np.stack([lij[:, 0]] * 2, 1))
    djj = oracle.hessian_entries(sub, np.stack([lij[:, 1]] * 2, 1))
    hv = h[torch.from_numpy(ij[:, 0]).to(h.device), torch.from_numpy(ij[:, 1]).to(h.device)].cpu().numpy()
    hm = h[torch.from_numpy(ij[:, 1]).to(h.device), torch.from_numpy(ij[:, 0]).to(h.device)].cpu().numpy()
    assert np.array_equal(hv, hm)                                             # bitwise symmetric
    check_hessian(hv, ref, np.sqrt(dii * djj))


def _search_sample(w, h, alpha_np, sc, ix, ob, rng, n=48):
    d_out, d_in = w.shape
    G = d_in // 32
    rows = rng.integers(0, d_out, n)
    groups = rng.integers(0, G, n)
    wr = w[torch.from_numpy(rows).to(w.device)].cpu().numpy()
    so, io, oo, oao = [], [], [], []
    amax = []
    for i, (r, g) in enumerate(zip(rows, groups)):
        wg = np.ascontiguousarray(wr[i, 32 * g:32 * g + 32][None, :])
        hb = h[32 * g:32 * g + 32, 32 * g:32 * g + 32].cpu().numpy()
        a, b, c_, d_ = oracle.scale_search(wg, hb, alpha_np, with_all=True)
        so.append(a[0, 0]), io.append(b[0, 0]), oo.append(c_[0, 0]), oao.append(d_[0, 0])
        amax.append(np.abs(wg).max())
    rt, gt = torch.from_numpy(rows).to(w.device), torch.from_numpy(groups).to(w.device)
    cand = lambda i, k: oracle.candidate(float(amax[i]), float(alpha_np[k]))
    check_search(ix[rt, gt].cpu().numpy(), sc[rt, gt].cpu().numpy(), ob[rt, gt].cpu().numpy(),
                 np.array(io), np.array(so, np.float32), np.array(oo), np.array(oao), cand)


def _pack_rows(w, sc, packed, s16, rows):
    rt = torch.from_numpy(rows).to(w.device)
    po, so = oracle.pack(w[rt].cpu().numpy(), sc[rt].cpu().numpy())
    assert np.array_equal(packed[rt].cpu().numpy(), po)
    assert np.array_equal(host_f16_bits(s16[rt]), so)


def _lsq_rows(w, sc, g, rows):
    rt = torch.from_numpy(rows).to(w.device)
    gw, gsc, wh = w4q.lsq_bwd(w, sc, g, GS, with_w_hat=True)
    wh1 = w4q.lsq_fwd(w, sc)
    wn, sn, gn = w[rt].cpu().numpy(), sc[rt].cpu().numpy(), g[rt].cpu().numpy()
    gwo, gso, who = oracle.lsq_bwd(wn, sn, gn, GS)
    assert np.array_equal(wh[rt].cpu().numpy(), who) and np.array_equal(wh1[rt].cpu().numpy(), who)
    assert np.array_equal(gw[rt].cpu().numpy(), gwo)
    wr = wn.astype(np.float64)
    d = np.repeat(sn.astype(np.float64), 32, axis=1)
    q = np.round(who.astype(np.float64) / np.where(d == 0, 1, d))
    m = (wr >= -8 * d) & (wr <= 7 * d)
    f = np.where(m, q - wr / d, q)
    G = w.shape[1] // 32
    gf = np.abs(gn * f).reshape(len(rows), G, 32).sum(axis=2)
    ga = np.abs(gn).reshape(len(rows), G, 32).sum(axis=2)
    assert np.all(np.abs(gsc[rt].cpu().numpy() - gso) <= LSQ_REL * GS * gf + GS * 2.0 ** -20 * ga)


def _product_cols(x_host, y, packed, s16, cols, dq):
    ct = torch.from_numpy(cols).to(packed.device)
    pr, sr = packed[ct].cpu().numpy(), host_f16_bits(s16[ct])
    yr, ya = oracle.gemm_cols(x_host, pr, sr, np.arange(len(cols)), dequant_bf16=dq)
    check_gemm(y[:, ct].cpu().numpy(), yr, ya)


@pytest.mark.parametrize("chunk", range(C.layers // CHUNK))
def test_stack36_layers(dev, chunk):
    alpha_np = C.alpha()
    alpha = torch.from_numpy(alpha_np).to(dev)
    for layer in range(chunk * CHUNK, (chunk + 1) * CHUNK):
        g = synth.device_generator(dev, 1000 + layer)
        rng = np.random.default_rng(2000 + layer)
        xs = {inp: synth.device_calib_x(g, C.n_tok, d, C.sigma, dev) for inp, d in C.inputs().items()}
        say("decoder36 layer", layer, "hessians")
        hs = {inp: w4q.quant_hessian(xt) for inp, xt in xs.items()}
        for inp in xs:
            _hessian_sample(xs[inp], hs[inp], rng)
        x_pre = {inp: host_bf16_bits(xt[:2048]) for inp, xt in xs.items()}
        for lin in C.linears:
            say("decoder36 layer", layer, lin.name, lin.d_out, lin.d_in)
            w = synth.device_weights(g, lin.d_out, lin.d_in, C.outlier_frac, dev)
            sc, ix, ob, _ = w4q.quant_scale_search(w, hs[lin.inp], alpha)
            _search_sample(w, hs[lin.inp], alpha_np, sc, ix, ob, rng)
            packed, s16 = w4q.quant_pack(w, sc)
            _pack_rows(w, sc, packed, s16, np.sort(rng.choice(lin.d_out, 6, replace=False)))
            if lin.name in C.lsq:
                gr = synth.device_grad(g, lin.d_out, lin.d_in, dev)
                _lsq_rows(w, sc, gr, np.sort(rng.choice(lin.d_out, 6, replace=False)))
                del gr
            cols = np.sort(rng.choice(lin.d_out, 4, replace=False))
            xt = xs[lin.inp]
            for dq in (False, True):                                          # prefill, M = 2048
                fn = w4q.w4a16_gemm_dq if dq else w4q.w4a16_gemm
                _product_cols(x_pre[lin.inp], fn(xt[:2048], packed, s16), packed, s16, cols, dq)
            cols = np.sort(rng.choice(lin.d_out, 16, replace=False))           # decode, M = 1
            y1 = w4q.w4a16_gemm(xt[:1], packed, s16)
            _product_cols(x_pre[lin.inp][:1], y1, packed, s16, cols, False)
            yg = w4q.w4a16_gemv_grouped([xt[:1]], [packed], [s16])[0]
            a, b = y1.cpu().numpy().astype(np.float64), yg.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(a - b) <= 1e-5 * (np.abs(a).max() + 1e-30))
            del w, sc, ix, ob, packed, s16, y1, yg
        del xs, hs
        torch.cuda.empty_cache()
