"""Pins of the oracle's fused QAT update (one Adam step on the weights and the LSQ steps), against
properties that do not come from retyping its formulas: Adam's bias-correction identity (a
constant gradient gives the normalised step g / (|g| + eps) at every step), the closed form of
the first step from zero moments, the limit lr = 0 (moments move, weights and steps do not, and
the fake-quantised output is the plain LSQ forward), the step-size gradient of the LSQ backward,
and the clamp of the step at its minimum."""
import numpy as np

import oracle

GS = 1.0 / np.sqrt(32 * 7)


def _zeros(w):
    G = w.shape[1] // 32
    return (np.zeros_like(w), np.zeros_like(w), np.zeros((w.shape[0], G), np.float32),
            np.zeros((w.shape[0], G), np.float32))


def test_constant_gradient_gives_normalised_steps():
    # weights far inside the clamp range, steps frozen (lr_s = 0): with g constant, m_t / c1 = g and
    # v_t / c2 = g^2 for every t (bias correction), so each step moves w by lr g / (|g| + eps)
    rng = np.random.default_rng(0)
    w = (rng.uniform(-0.5, 0.5, (4, 64))).astype(np.float32)
    scale = np.full((4, 2), 1.0, np.float32)                    # range [-8, 7]: every w inside
    g = rng.choice([-2.0, -0.5, 0.25, 3.0], (4, 64)).astype(np.float32)
    m_w, v_w, m_s, v_s = _zeros(w)
    cur = w.copy()
    for t in range(1, 6):
        hp = oracle.adam_hparams(1e-3, 0.0, eps=1e-8, step=t)
        lr, eps = hp[0], hp[4]
        o = oracle.lsq_adam_step(cur, scale, g, GS, m_w, v_w, m_s, v_s, hp)
        cur, m_w, v_w, m_s, v_s = o["w"], o["m_w"], o["v_w"], o["m_s"], o["v_s"]
        assert np.array_equal(o["scale"], scale)
    want = w.astype(np.float64) - 5 * lr * g / (np.abs(g) + eps)
    assert np.allclose(cur, want, rtol=0, atol=5 * 2.0 ** -24)


def test_first_step_closed_form_and_mask():
    # from zero moments the first step is lr (g / (|g| + eps) + wd w) for weights inside the range;
    # outside it the straight-through gradient is 0, so only the decay moves them
    d = np.float32(0.25)
    w = np.zeros((1, 32), np.float32)
    w[0, :6] = [0.375, 1.875, 1.75, -2.125, -2.0, 0.1]          # inside: 1.75, -2.0, 0.375, 0.1
    g = np.linspace(-1, 1, 32).astype(np.float32)
    g[g == 0] = 0.5
    scale = np.array([[d]], np.float32)
    m_w, v_w, m_s, v_s = _zeros(w)
    hp = oracle.adam_hparams(1e-2, 0.0, eps=1e-8, weight_decay=0.1, step=1)
    lr, b1, eps, wd = hp[0], hp[2], hp[4], hp[5]          # the fp32 values the update is defined on
    o = oracle.lsq_adam_step(w, scale, g, GS, m_w, v_w, m_s, v_s, hp)
    inside = (w >= -8 * d) & (w <= 7 * d)
    gi = np.where(inside, g, 0.0).astype(np.float64)
    # from zero moments: m / c1 = g and v / c2 = g^2 (c = 1 - beta at t = 1)
    want = w - lr * (gi / (np.abs(gi) + eps) + wd * w.astype(np.float64))
    assert np.allclose(o["w"], want, rtol=0, atol=2.0 ** -24 * np.abs(want).max() + 1e-12)
    assert not inside[0, 1] and not inside[0, 3] and inside[0, 2] and inside[0, 4]
    assert np.array_equal(o["m_w"], ((1 - b1) * gi).astype(np.float32))


def test_zero_rate_keeps_weights_and_forward_matches_lsq():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 96)) * 0.02).astype(np.float32)
    G = 3
    scale = (np.abs(w.reshape(8, G, 32)).max(axis=2) / 7 * rng.uniform(0.5, 1.1, (8, G))).astype(np.float32)
    g = rng.standard_normal((8, 96)).astype(np.float32)
    m_w, v_w, m_s, v_s = _zeros(w)
    o = oracle.lsq_adam_step(w, scale, g, GS, m_w, v_w, m_s, v_s, oracle.adam_hparams(0.0, 0.0))
    assert np.array_equal(o["w"], w) and np.array_equal(o["scale"], scale)
    assert np.array_equal(o["w_hat"], oracle.lsq_fwd(w, scale))
    # the step-size gradient is the LSQ backward's, and the moments take (1 - beta) of it
    _, ds, _ = oracle.lsq_bwd(w, scale, g, GS)
    assert np.array_equal(o["ds"], ds)
    hp = oracle.adam_hparams(0.0, 0.0)
    assert np.array_equal(o["m_s"], ((1 - hp[2]) * ds).astype(np.float32))
    assert np.array_equal(o["v_s"], ((1 - hp[3]) * ds * ds).astype(np.float32))


def test_step_clamped_at_minimum_and_given_gradient():
    w = np.full((1, 32), 0.01, np.float32)
    scale = np.full((1, 1), 1e-3, np.float32)
    g = np.ones((1, 32), np.float32)
    m_w, v_w, m_s, v_s = _zeros(w)
    hp = oracle.adam_hparams(0.0, 1.0, scale_min=1e-4)          # a huge step on D
    ext = np.full((1, 1), 5.0)
    o = oracle.lsq_adam_step(w, scale, g, GS, m_w, v_w, m_s, v_s, hp, ext_ds=ext)
    assert o["scale"][0, 0] == np.float32(1e-4)                 # 1e-3 - 1.0 * 1 clamps
    assert o["ds"][0, 0] == 5.0
