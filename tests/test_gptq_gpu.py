"""GPU parity of the GPTQ error feedback against the oracle on identical inputs (the GPU's H and
the group search's fp16-grid steps, fetched to the host).

Quantized weights are compared exactly on every row where the oracle's updated weights stayed
clear of the decision midpoints (two fp64 routes differ by rounding only, so a code can differ
only within that distance of a midpoint, and then every later column of the row may follow);
on the other rows the GPU's result is checked to be a valid feedback run up to that point.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import w4a16_group_wise_amd as w4q
from w4a16_group_wise_amd import synth
from gpu_util import dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


CASES = [  # d_out, d_in, n_tok, correlated
    (32, 256, 512, True),
    (20, 96, 256, True),        # a 32-wide last block and a padded factor
    (48, 512, 1024, False),
    (9, 1024, 2048, True),      # 16 panels of the factorisation
]


def _run(dev, d_out, d_in, n_tok, corr, seed, dead_col=None, damp=0.01):
    x = (synth.correlated_x(seed, 0, 0, n_tok, d_in, 6, 1e-2) if corr
         else synth.calib_x(seed, 0, 0, n_tok, d_in, 1.0))
    if dead_col is not None:
        x = x.copy()
        x[:, dead_col] = 0
    h = w4q.quant_hessian(dev_bf16(x, dev))
    w = synth.weights(seed, 0, 1, d_out, d_in, 0.005)
    wt = dev_f32(w, dev)
    sc, _, _, _ = w4q.quant_scale_search(wt, h, torch.from_numpy(synth.alpha_grid(20, 0.5, 1.0)).to(dev))
    wh, info = w4q.quant_gptq(wt, h, sc, damp=damp)
    return w, h.cpu().numpy(), sc.cpu().numpy(), wh.cpu().numpy(), int(info.item())


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_gptq_matches_oracle(dev, case):
    d_out, d_in, n_tok, corr = case
    say("gptq", case)
    w, h, sc, wh, info = _run(dev, d_out, d_in, n_tok, corr, 100 + d_in)
    assert info == 0
    ref = oracle.gptq(w, h, sc, damp=0.01)
    clean = ref["margin"] > 1e-9
    assert clean.mean() >= 0.9
    assert np.array_equal(wh[clean], ref["w_hat"][clean])
    # every output is a grid value of its group: Delta * q with q in [-8, 7]
    d = np.repeat(sc.astype(np.float64), 32, axis=1)
    q = np.where(d > 0, wh.astype(np.float64) / np.where(d > 0, d, 1), 0)
    assert np.all(q == np.round(q)) and np.all((q >= -8) & (q <= 7))
    # the feedback moves codes away from plain rounding on correlated activations
    if corr:
        assert np.any(wh != oracle.lsq_fwd(w, sc))
    say("gptq", case, "clean rows", int(clean.sum()), "of", d_out)


def test_gptq_dead_column_and_damping(dev):
    d_out, d_in = 12, 128
    w, h, sc, wh, info = _run(dev, d_out, d_in, 256, True, 131, dead_col=7, damp=0.1)
    assert info == 0 and np.all(wh[:, 7] == 0)
    ref = oracle.gptq(w, h, sc, damp=0.1)
    clean = ref["margin"] > 1e-9
    assert np.array_equal(wh[clean], ref["w_hat"][clean])


def test_gptq_not_positive_definite_sets_info(dev):
    d_out, d_in = 4, 64
    w = synth.weights(7, 0, 1, d_out, d_in, 0.0)
    wt = dev_f32(w, dev)
    h = -torch.eye(d_in, dtype=torch.float32, device=dev)
    sc = torch.full((d_out, d_in // 32), 0.01, dtype=torch.float32, device=dev)
    _, info = w4q.quant_gptq(wt, h, sc, damp=0.0)
    assert int(info.item()) == 1
