"""GPU parity of the per-channel variant and of the joint objective with its coordinate descent,
against the oracle on identical inputs (the GPU's own H, fetched to the host).

Per-channel (one scale per output row): search on iid and correlated calibration activations,
ragged widths (d_in not a multiple of 64), K = 1 .. 200; pack / LSQ forward and backward / the
product (vector, matrix-core and tiled paths, exact and bf16-dequantized weights).
Joint: the whole-row objective e^T H e, and the descent from the group search's choice: the
same indices and steps as the oracle's descent wherever the oracle saw no near-tie, and on every
row an objective that never rises and matches the oracle's evaluation of the GPU's own result.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import (LSQ_REL, check_gemm, check_search, dev_bf16, dev_f32, host_f16_bits)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _problem(dev, seed, d_out, d_in, n_tok, corr, k, lo=0.4):
    x = (synth.correlated_x(seed, 0, 0, n_tok, d_in, 4, 1e-3) if corr
         else synth.calib_x(seed, 0, 0, n_tok, d_in, 1.0))
    h = w4q.quant_hessian(dev_bf16(x, dev))
    w = synth.weights(seed, 0, 1, d_out, d_in, 0.005)
    alpha = synth.alpha_grid(k, lo, 1.0)
    return x, h, h.cpu().numpy(), w, alpha


def _abs_form(w, steps, h_np, group):
    """|e|^T |H| |e| per row: the scale of fp64 rounding in e^T H e."""
    wh = oracle.lsq_fwd(w, steps, group=group)        # fp32 of an exact product: exact
    e = np.abs(w.astype(np.float64) - wh.astype(np.float64))
    return np.einsum("ri,ij,rj->r", e, np.abs(h_np.astype(np.float64)), e)


# ------------------------------------------------------------------------- per-channel
PC_CASES = [  # d_out, d_in, n_tok, correlated, K
    (48, 256, 512, False, 20),
    (40, 224, 384, True, 7),      # 224 = 3.5 column blocks of 64
    (33, 512, 640, True, 40),
    (16, 128, 256, False, 1),
    (20, 96, 200, True, 70),
    (12, 160, 256, False, 200),   # two candidate blocks of 128
]


@pytest.mark.parametrize("case", PC_CASES, ids=lambda c: "x".join(map(str, c)))
def test_per_channel_search(dev, case):
    d_out, d_in, n_tok, corr, k = case
    say("pc search", case)
    x, h, h_np, w, alpha = _problem(dev, 60 + d_in, d_out, d_in, n_tok, corr, k)
    at = torch.from_numpy(alpha).to(dev)
    sc, ix, ob, oa = w4q.quant_scale_search_pc(dev_f32(w, dev), h, at, with_obj_all=True)
    so, io, oo, oao = oracle.scale_search_pc(w, h_np, alpha, with_all=True)
    amax = np.abs(w).max(axis=1)
    cand = lambda i, kk: oracle.candidate(float(amax[i]), float(alpha[kk]))
    check_search(ix.cpu().numpy(), sc.cpu().numpy(), ob.cpu().numpy(), io, so, oo, oao, cand)
    # every candidate's objective: fp64 rounding of e^T H e (a few 2^-53 d_in of |e|^T |H| |e|),
    # then one rounding to fp32
    ha = np.abs(h_np.astype(np.float64))
    oag = oa.cpu().numpy().astype(np.float64)
    for r in range(d_out):
        d = np.array([cand(r, kk) for kk in range(k)], np.float64)[:, None]
        wr = w[r].astype(np.float64)[None, :]
        q = np.clip(np.round(wr / np.where(d == 0, 1, d)), -8, 7)
        e = np.abs(wr - d * q)
        b = np.einsum("ki,ij,kj->k", e, ha, e)
        assert np.all(np.abs(oag[r] - oao[r]) <= 2.0 ** -24 * np.abs(oao[r]) + 1e-12 * b + 1e-300)


def test_per_channel_zero_row_and_ldh(dev):
    d_out, d_in, k = 6, 128, 9
    x, h, h_np, w, alpha = _problem(dev, 77, d_out, d_in, 256, False, k)
    w[2] = 0.0
    hp = torch.zeros((d_in, d_in + 12), dtype=torch.float32, device=dev)
    hp[:, :d_in] = h
    sc, ix, ob, _ = w4q.quant_scale_search_pc(dev_f32(w, dev), hp, torch.from_numpy(alpha).to(dev))
    so, io, oo, _ = oracle.scale_search_pc(w, h_np, alpha)
    assert np.array_equal(ix.cpu().numpy(), io) and np.array_equal(sc.cpu().numpy(), so)
    assert ix[2].item() == 0 and sc[2].item() == 0.0 and ob[2].item() == 0.0


@pytest.mark.parametrize("d_out,d_in", [(64, 256), (37, 96), (130, 512)])
def test_per_channel_pack_and_lsq(dev, d_out, d_in):
    say("pc pack/lsq", d_out, d_in)
    rng = np.random.default_rng(d_in + d_out)
    w = synth.weights(80, 0, d_in, d_out, d_in, 0.005)
    s = (np.abs(w).max(axis=1) / 7 * rng.uniform(0.4, 1.2, d_out)).astype(np.float32)
    s[0] = np.float32(3e-7)                                   # an fp16-subnormal step
    g = synth.upstream_grad(80, 0, d_in, d_out, d_in)
    wt, st, gt = dev_f32(w, dev), dev_f32(s, dev), dev_f32(g, dev)
    packed, s16 = w4q.quant_pack_pc(wt, st)
    po, so = oracle.pack(w, s[:, None], group=d_in)
    assert np.array_equal(packed.cpu().numpy(), po)
    assert np.array_equal(host_f16_bits(s16), so[:, 0])
    wh = w4q.lsq_fwd_pc(wt, st).cpu().numpy()
    assert np.array_equal(wh, oracle.lsq_fwd(w, s[:, None], group=d_in))
    gs = 1.0 / np.sqrt(d_in * 7)
    gw, gsc, wh2 = w4q.lsq_bwd_pc(wt, st, gt, gs, with_w_hat=True)
    gwo, gso, who = oracle.lsq_bwd(w, s[:, None], g, gs, group=d_in)
    assert np.array_equal(gw.cpu().numpy(), gwo) and np.array_equal(wh2.cpu().numpy(), who)
    d = s.astype(np.float64)[:, None]
    q = np.round(who.astype(np.float64) / np.where(d == 0, 1, d))
    wr = w.astype(np.float64)
    m = (wr >= -8 * d) & (wr <= 7 * d)
    f = np.where(m, q - wr / d, q)
    bound = LSQ_REL * gs * np.abs(g * f).sum(axis=1) + gs * 2.0 ** -20 * np.abs(g).sum(axis=1)
    assert np.all(np.abs(gsc.cpu().numpy() - gso[:, 0]) <= bound)


@pytest.mark.parametrize("m", [1, 4, 16, 64])
@pytest.mark.parametrize("dq", [False, True])
def test_per_channel_product(dev, m, dq):
    d_out, d_in = 192, 512
    say("pc product m", m, "dq", dq)
    w = synth.weights(81, 0, 0, d_out, d_in, 0.005)
    s = (np.abs(w).max(axis=1) / 7).astype(np.float32)
    packed, s16 = oracle.pack(w, s[:, None], group=d_in)
    x = synth.calib_x(81, 0, 1, m, d_in, 1.5)
    pt = torch.from_numpy(packed).to(dev)
    st = torch.from_numpy(s16[:, 0].view(np.float16)).to(dev)
    for out_dtype in (torch.float32, torch.bfloat16):
        y = w4q.w4a16_gemm_pc(dev_bf16(x, dev), pt, st, out_dtype=out_dtype, dequant_bf16=dq)
        yr, ya = oracle.gemm_cols(x, packed, s16, dequant_bf16=dq, group=d_in)
        check_gemm(y.float().cpu().numpy(), yr, ya, bf16_out=out_dtype == torch.bfloat16)


# ------------------------------------------------------------------------------- joint
JOINT_CASES = [  # d_out, d_in, n_tok, correlated, K, sweeps
    (32, 256, 512, True, 20, 3),
    (70, 96, 256, True, 12, 4),     # ragged: two row blocks, 1.5 column blocks
    (16, 512, 768, False, 12, 2),
]


def _bound(w, steps, h_np):
    return _abs_form(w, steps, h_np, 32)


@pytest.mark.parametrize("case", JOINT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_joint_objective_and_refine(dev, case):
    d_out, d_in, n_tok, corr, k, sweeps = case
    say("joint", case)
    x, h, h_np, w, alpha = _problem(dev, 90 + d_in, d_out, d_in, n_tok, corr, k)
    wt, at = dev_f32(w, dev), torch.from_numpy(alpha).to(dev)
    sc, ix, _, _ = w4q.quant_scale_search(wt, h, at)
    sc_np, ix_np = sc.cpu().numpy(), ix.cpu().numpy()
    # the objective of the group search's choice
    og = w4q.quant_joint_objective(wt, sc, h).cpu().numpy()
    oo = oracle.joint_objective(w, sc_np, h_np)
    b0 = _bound(w, sc_np, h_np)
    assert np.all(np.abs(og - oo) <= 1e-12 * b0 + 1e-300)
    # descent from that choice on both sides
    idx_g, sc_g, ob_g, oa_g, sw_g = (t.cpu().numpy() for t in w4q.quant_joint_refine(wt, h, at, ix, n_sweeps=sweeps))
    ref = oracle.joint_refine(w, h_np, alpha, ix_np, n_sweeps=sweeps)
    assert np.all(np.abs(ob_g - oo) <= 1e-12 * b0 + 1e-300)
    b1 = _bound(w, sc_g, h_np)
    assert np.all(oa_g <= ob_g + 1e-12 * b0)                       # never rises
    assert np.all(np.abs(oa_g - oracle.joint_objective(w, sc_g, h_np)) <= 1e-11 * b1 + 1e-300)
    clean = ref["margin"] > 1e-8
    assert clean.mean() > 0.8
    assert np.array_equal(idx_g[clean], ref["idx"][clean])
    assert np.array_equal(sc_g[clean], ref["scale"][clean])
    assert np.array_equal(sw_g[clean], ref["sweeps"][clean])
    assert np.all(np.abs(oa_g[clean] - ref["obj"][clean]) <= 1e-11 * b1[clean] + 1e-300)
    # the steps are the candidates of the chosen indices
    for r in range(0, d_out, max(1, d_out // 5)):
        for g in range(d_in // 32):
            amax = float(np.abs(w[r, 32 * g:32 * g + 32]).max())
            assert sc_g[r, g] == oracle.candidate(amax, float(alpha[idx_g[r, g]]))
    say("joint", case, "rows changed", int((idx_g != ix_np).any(axis=1).sum()), "of", d_out,
        "objective ratio", float(np.mean(oa_g / np.maximum(ob_g, 1e-300))))


def test_joint_refine_chunked_workspace(dev):
    d_out, d_in, k = 150, 128, 10
    x, h, h_np, w, alpha = _problem(dev, 95, d_out, d_in, 256, True, k)
    wt, at = dev_f32(w, dev), torch.from_numpy(alpha).to(dev)
    _, ix, _, _ = w4q.quant_scale_search(wt, h, at)
    full = [t.cpu().numpy() for t in w4q.quant_joint_refine(wt, h, at, ix, n_sweeps=3)]
    small = torch.empty(64 * (d_in * 8 + 8 * 2) + 256, dtype=torch.uint8, device=dev)   # 64 rows a chunk
    part = [t.cpu().numpy() for t in w4q.quant_joint_refine(wt, h, at, ix, n_sweeps=3, workspace=small)]
    for a, b in ((0, 0), (1, 1), (3, 3), (4, 4)):
        assert np.array_equal(full[a], part[b])
    assert np.allclose(full[2], part[2], rtol=1e-12)
