"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks one oracle function against something independent of its code: a
hand-derived worked example (tests/golden), brute force over all codes with exact rational
arithmetic, a closed form, an invariant, or a library routine the oracle does not use
(numpy's float16 cast, numpy's matmul).  Planted mistakes (a dropped term, a wrong sign or
index, a transposed operand) fail at least one of these.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from w4a16_group_wise_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                parts = line.split()
                rows.setdefault(parts[0], []).append(parts[1:])
    return rows


def _brute_code(w: float, d: float) -> int:
    """Nearest of the 16 grid points in exact rational arithmetic, ties to even."""
    if d == 0:
        return 0
    W, D = Fraction(w), Fraction(d)
    best = None
    for c in range(-8, 8):
        dist = abs(W - c * D)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1]


# --------------------------------------------------------------------------- 16-bit floats
def test_f16_matches_numpy_cast():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-6).astype(np.float32),           # fp16 subnormals
        (rng.standard_normal(500) * 1e-8).astype(np.float32),            # underflow to 0
        (rng.uniform(6.0e4, 7.0e4, 500)).astype(np.float32),             # overflow region
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf],
                 dtype=np.float32),
    ])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([oracle.f16_to_f64(b) for b in ref])
    assert np.array_equal(back, ref.view(np.float16).astype(np.float64))


def test_bf16_decode_matches_bit_shift():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    want = synth.bf16_bits_to_f32(bits).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(b) for b in bits])
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------ codes
def test_code_golden_ties():
    with open(os.path.join(GOLD, "code_ties.txt")) as f:
        rows = [l.split("#")[0].split() for l in f if l.split("#")[0].strip()]
    assert len(rows) >= 10
    for w, d, q in rows:
        assert oracle.code(float(w), float(d)) == int(q), (w, d, q)
        assert _brute_code(float(w), float(d)) == int(q)


def test_code_brute_force_random_and_midpoints():
    rng = np.random.default_rng(3)
    deltas = [float(np.float32(v)) for v in rng.uniform(1e-3, 0.2, 40)]
    deltas += [float(oracle.f16_to_f64(b)) for b in (0x0001, 0x0203, 0x2E66, 0x3C00)]
    for d in deltas:
        ws = list(rng.uniform(-10 * d, 10 * d, 40).astype(np.float32))
        # exact midpoints (c + 1/2) D whenever they are fp32 numbers, plus their neighbours
        for c in range(-9, 8):
            m = np.float32((c + 0.5) * d)
            ws += [m, np.nextafter(m, np.float32(np.inf)), np.nextafter(m, np.float32(-np.inf))]
        for w in ws:
            assert oracle.code(float(w), d) == _brute_code(float(w), d), (w, d)


def test_code_idempotent_on_grid():
    for d in (0.25, 0.0999755859375, float(np.float32(0.013))):
        for q in range(-8, 8):
            w = float(np.float32(d * q))
            if Fraction(w) == Fraction(d) * q:
                assert oracle.code(w, d) == q


# ---------------------------------------------------------------------------- candidates
def test_candidate_worked_example():
    (row,) = _golden("worked_examples.txt")["candidate"]
    amax, alpha, bits, val = float(row[0]), float(row[1]), int(row[2], 16), float(row[3])
    assert oracle.f32_to_f16(np.float32(amax) / np.float32(7.0)) == bits
    assert oracle.candidate(amax, alpha) == val


def test_candidate_matches_numpy_float32_order():
    rng = np.random.default_rng(4)
    amax = rng.uniform(1e-4, 2.0, 2000).astype(np.float32)
    alpha = rng.uniform(0.3, 1.0, 2000).astype(np.float32)
    t = alpha * amax                          # numpy float32 ops are IEEE single
    u = t / np.float32(7.0)
    want = u.astype(np.float16).astype(np.float32)
    got = np.array([oracle.candidate(a, b) for a, b in zip(amax, alpha)], dtype=np.float32)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------- Hessian
def test_hessian_worked_example():
    g = _golden("worked_examples.txt")
    x = np.array([[float(v) for v in r.split(",")] for r in g["hessian_x"][0][0].split(";")],
                 dtype=np.float32)
    h_want = np.array([[float(v) for v in r.split(",")] for r in g["hessian_h"][0][0].split(";")])
    h = oracle.hessian(synth.f32_to_bf16_bits(x))
    assert np.array_equal(h, h_want)


def test_hessian_against_numpy_and_invariants():
    x = synth.calib_x(9, 0, 0, 96, 64, 1.0)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    h = oracle.hessian(x)
    ref = xf.T @ xf
    assert np.allclose(h, ref, rtol=1e-13, atol=0)
    assert np.array_equal(h, h.T)
    assert np.isclose(np.trace(h), np.sum(xf * xf), rtol=1e-13)
    np.linalg.cholesky(h + 1e-9 * np.trace(h) * np.eye(64))          # PSD
    x2 = synth.f32_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(x))      # exact doubling
    assert np.array_equal(oracle.hessian(x2), 4.0 * h)
    ij = np.array([[0, 0], [3, 17], [63, 1], [5, 5]])
    assert np.array_equal(oracle.hessian_entries(x, ij), h[ij[:, 0], ij[:, 1]])


# ---------------------------------------------------------------------------- scale search
def _explicit_obj(w_g, x_g, d):
    """||X_g e||^2 with the codes from brute force: no H involved."""
    e = np.array([Fraction(float(v)) - Fraction(d) * _brute_code(float(v), d) for v in w_g])
    out = Fraction(0)
    for row in x_g:
        s = sum(Fraction(float(a)) * b for a, b in zip(row, e))
        out += s * s
    return float(out)


def test_objective_equals_explicit_reconstruction_error():
    # small-integer activations: H = X^T X is exact in fp32, so e^T H e must equal ||X e||^2
    rng = np.random.default_rng(5)
    n_tok, d_in, d_out = 12, 64, 3
    x = rng.integers(-3, 4, (n_tok, d_in)).astype(np.float64)
    h = (x.T @ x).astype(np.float32)
    assert np.array_equal(h.astype(np.float64), x.T @ x)
    w = synth.weights(9, 0, 1, d_out, d_in, 0.02)
    alpha = synth.alpha_grid(7, 0.5, 1.0)
    scale, idx, obj, obj_all = oracle.scale_search(w, h, alpha, with_all=True)
    for r in range(d_out):
        for g in range(d_in // 32):
            wg = w[r, 32 * g:32 * g + 32]
            xg = x[:, 32 * g:32 * g + 32]
            amax = float(np.max(np.abs(wg)))
            want = []
            for k, a in enumerate(alpha):
                d = float((np.float32(a) * np.float32(amax) / np.float32(7)).astype(np.float16))
                want.append(_explicit_obj(wg, xg, d))
            assert np.allclose(obj_all[r, g], want, rtol=1e-12, atol=1e-300)
            kb = int(np.argmin(want))                     # numpy argmin: first minimum
            assert idx[r, g] == kb
            assert obj[r, g] == obj_all[r, g, kb]


def test_identity_hessian_is_plain_mse_grid_search():
    w = synth.weights(9, 0, 2, 16, 128, 0.02)
    alpha = synth.alpha_grid(20, 0.5, 1.0)
    h = np.eye(128, dtype=np.float32) * np.float32(3.0)
    scale, idx, obj, obj_all = oracle.scale_search(w, h, alpha, with_all=True)
    for r in range(16):
        for g in range(4):
            wg = w[r, 32 * g:32 * g + 32].astype(np.float64)
            amax = np.float32(np.max(np.abs(wg)))
            mse = []
            for a in alpha:
                d = float((np.float32(a) * amax / np.float32(7)).astype(np.float16))
                q = np.clip(np.round(wg / d), -8, 7)       # numpy round: half to even
                mse.append(3.0 * np.sum((wg - d * q) ** 2))
            assert np.allclose(obj_all[r, g], mse, rtol=1e-12)
            assert idx[r, g] == int(np.argmin(mse))


def test_search_invariants():
    x = synth.calib_x(9, 0, 3, 64, 96, 1.0)
    h = oracle.hessian(x).astype(np.float32)
    w = synth.weights(9, 0, 3, 24, 96, 0.05)
    alpha = synth.alpha_grid(12, 0.4, 1.0)  # contains alpha = 1 (max-based scale) last
    scale, idx, obj, obj_all = oracle.scale_search(w, h, alpha, with_all=True)
    assert np.all(obj <= obj_all[:, :, -1])                # never worse than max-based scale
    assert np.all(obj == obj_all.min(axis=2))
    # power-of-two scaling of H scales every objective exactly and keeps the choice
    s2, i2, o2, _ = oracle.scale_search(w, h * np.float32(4.0), alpha)
    assert np.array_equal(i2, idx) and np.array_equal(s2, scale) and np.array_equal(o2, 4 * obj)
    # chosen scale is the candidate at idx
    for r in range(24):
        for g in range(3):
            amax = float(np.max(np.abs(w[r, 32 * g:32 * g + 32])))
            assert scale[r, g] == oracle.candidate(amax, alpha[idx[r, g]])
    # group subset call agrees with the full call
    rows = np.array([0, 5, 23, 7])
    groups = np.array([2, 0, 1, 1])
    sc, ix, ob, _ = oracle.scale_search_groups(w, h, alpha, rows, groups)
    assert np.array_equal(sc, scale[rows, groups]) and np.array_equal(ix, idx[rows, groups])


def test_all_zero_group():
    w = np.zeros((2, 64), np.float32)
    w[1, 40] = 0.5
    h = np.eye(64, dtype=np.float32)
    scale, idx, obj, _ = oracle.scale_search(w, h, synth.alpha_grid(5, 0.5, 1.0))
    assert scale[0, 0] == 0 and idx[0, 0] == 0 and obj[0, 0] == 0
    assert scale[1, 0] == 0 and idx[1, 0] == 0


# ---------------------------------------------------------------------------------- pack
def test_pack_worked_example_and_roundtrip():
    (row,) = _golden("worked_examples.txt")["pack"]
    codes = [int(v) for v in row[0].split(",")]
    want = [int(v, 16) for v in row[1].split(",")]
    w = np.zeros((1, 32), np.float32)
    w[0, :4] = codes
    packed, s16 = oracle.pack(w, np.ones((1, 1), np.float32))
    assert list(packed[0, :2]) == want and s16[0, 0] == 0x3C00
    # every code survives pack -> unpack
    w = np.tile(np.arange(-8, 8, dtype=np.float32), 4).reshape(2, 32) * np.float32(0.5)
    packed, s16 = oracle.pack(w, np.full((2, 1), 0.5, np.float32))
    for r in range(2):
        assert [oracle.unpack(packed[r], k) for k in range(32)] == list((w[r] / 0.5).astype(int))


def test_pack_codes_match_brute_force():
    w = synth.weights(9, 0, 4, 8, 64, 0.05)
    scale = np.abs(w.reshape(8, 2, 32)).max(axis=2) / np.float32(5.3)
    packed, s16 = oracle.pack(w, scale)
    assert np.array_equal(s16, scale.astype(np.float16).view(np.uint16))
    for r in range(8):
        for k in range(64):
            d = float(s16[r, k // 32:k // 32 + 1].view(np.float16)[0])
            assert oracle.unpack(packed[r], k) == _brute_code(float(w[r, k]), d)


# ----------------------------------------------------------------------------------- LSQ
def test_lsq_worked_example():
    g = _golden("worked_examples.txt")
    wv = [float(v) for v in g["lsq_w"][0][0].split(",")]
    d = float(g["lsq_scale"][0][0])
    w = np.zeros((1, 32), np.float32)
    w[0, :len(wv)] = wv
    sc = np.full((1, 1), d, np.float32)
    gw, gsc, wh = oracle.lsq_bwd(w, sc, np.ones_like(w), 1.0)
    mask = [int(v) for v in g["lsq_mask"][0][0].split(",")]
    assert list(gw[0, :6]) == [float(m) for m in mask] and np.all(gw[0, 6:] == 1.0)
    # 0.1 is not an fp32 number: w/D = 0.4000000059604645 for the fp32 weight
    assert np.isclose(gsc[0, 0], float(g["lsq_sumf"][0][0]), rtol=0, atol=1e-8)
    assert list(wh[0, :6]) == [float(v) for v in g["lsq_what"][0][0].split(",")]
    assert np.array_equal(oracle.lsq_fwd(w, sc), wh)


def _surrogate(w, d, gup, r0):
    """L(W, D) = sum G * D * (clamp(W/D, -8, 7) + R0): the STE / LSQ surrogate."""
    return float(np.sum(gup * d[:, :, None] * (np.clip(w / d[:, :, None], -8, 7) + r0)))


def test_lsq_gradients_match_finite_differences():
    rng = np.random.default_rng(6)
    d_out, d_in = 3, 64
    w = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    sc = (np.abs(w.reshape(d_out, 2, 32)).max(axis=2) / 6.0).astype(np.float32)
    sc[0, 1] *= np.float32(0.5)                      # force clamping in one group
    gup = rng.standard_normal((d_out, d_in)).astype(np.float32)
    gs = 1.0 / np.sqrt(32 * 7)
    gw, gsc, _ = oracle.lsq_bwd(w, sc, gup, gs)
    w64 = w.astype(np.float64).reshape(d_out, 2, 32)
    d64 = sc.astype(np.float64)
    g64 = gup.astype(np.float64).reshape(d_out, 2, 32)
    q = np.array([[oracle.code(v, d64[r, k // 32]) for k, v in enumerate(w[r])]
                  for r in range(d_out)], dtype=np.float64).reshape(d_out, 2, 32)
    r0 = q - np.clip(w64 / d64[:, :, None], -8, 7)
    h = 1e-7
    for r in range(d_out):
        for g in range(2):
            dp, dm = d64.copy(), d64.copy()
            dp[r, g] += h * d64[r, g]
            dm[r, g] -= h * d64[r, g]
            fd = (_surrogate(w64, dp, g64, r0) - _surrogate(w64, dm, g64, r0)) / (2 * h * d64[r, g])
            near = np.abs(np.abs(w64[r, g] / d64[r, g] + 0.5) - 8.5) < 1e-4
            if not near.any():
                assert np.isclose(gs * fd, gsc[r, g], rtol=1e-6, atol=1e-9)
            for i in range(0, 32, 5):
                k = g * 32 + i
                t = w64[r, g, i] / d64[r, g]
                if abs(t - 7) < 1e-4 or abs(t + 8) < 1e-4:
                    continue
                wp, wm = w64.copy(), w64.copy()
                wp[r, g, i] += 1e-9
                wm[r, g, i] -= 1e-9
                fdw = (_surrogate(wp, d64, g64, r0) - _surrogate(wm, d64, g64, r0)) / 2e-9
                assert np.isclose(fdw, gw[r, k], rtol=1e-5, atol=1e-7)


def test_lsq_closed_forms():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((2, 32)) * 0.01).astype(np.float32)
    gup = rng.standard_normal((2, 32)).astype(np.float32)
    gs = 0.5
    big = np.full((2, 1), 100.0, np.float32)          # D >> |w|: every code 0, all in range
    gw, gsc, wh = oracle.lsq_bwd(w, big, gup, gs)
    assert np.array_equal(gw, gup) and np.all(wh == 0)
    want = -gs * np.sum(gup.astype(np.float64) * w.astype(np.float64) / 100.0, axis=1)
    assert np.allclose(gsc[:, 0], want, rtol=1e-12)
    tiny = np.full((2, 1), 1e-9, np.float32)          # every weight clamped
    w2 = w.copy()
    w2[w2 == 0] = 1e-3
    gw, gsc, _ = oracle.lsq_bwd(w2, tiny, gup, gs)
    assert np.all(gw == 0)
    lev = np.where(w2 > 0, 7.0, -8.0)
    assert np.allclose(gsc[:, 0], gs * np.sum(gup * lev, axis=1), rtol=1e-12)


# ---------------------------------------------------------------------------------- GEMM
def _numpy_dequant(packed, s16):
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    nib = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
    q = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    s = s16.view(np.float16).astype(np.float64)
    return q * np.repeat(s, 32, axis=1)


def test_gemm_worked_example():
    (row,) = _golden("worked_examples.txt")["gemm_y"]
    codes = np.tile(np.arange(-8, 8), 2).astype(np.float32)
    packed, s16 = oracle.pack((codes * np.float32(0.5))[None, :], np.full((1, 1), 0.5, np.float32))
    x = synth.f32_to_bf16_bits(np.ones((1, 32), np.float32))
    y, ya = oracle.gemm_cols(x, packed, s16)
    assert y[0, 0] == float(row[0]) and ya[0, 0] == 0.5 * 2 * 64


def test_gemm_matches_numpy_matmul():
    w = synth.weights(9, 0, 5, 40, 96, 0.01)
    sc = np.abs(w.reshape(40, 3, 32)).max(axis=2) / np.float32(7)
    packed, s16 = oracle.pack(w, sc)
    x = synth.calib_x(9, 0, 5, 5, 96, 1.0)
    y, ya = oracle.gemm_cols(x, packed, s16)
    wh = _numpy_dequant(packed, s16)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(y, xf @ wh.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(ya, np.abs(xf) @ np.abs(wh).T, rtol=1e-12)
    cols = np.array([39, 0, 7])
    y2, _ = oracle.gemm_cols(x, packed, s16, cols)
    assert np.array_equal(y2, y[:, cols])


# ------------------------------------------------- GEMM with weights dequantized to bf16
def _bf16_nearest_bruteforce(v):
    """Nearest bf16 value by enumeration of the bf16 patterns around v (ties: even pattern)."""
    from fractions import Fraction
    f = np.float32(v)
    base = int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
    best = None
    for b in range(max(base - 2, 0), base + 3):
        cand = np.array([b << 16], np.uint32).view(np.float32)[0]
        dist = abs(Fraction(float(cand)) - Fraction(float(v)))
        key = (dist, b & 1)
        if best is None or key < best[0]:
            best = (key, float(cand))
    return best[1]


def test_round_bf16_worked_ties():
    # s = 1 + 2^-8 (fp16 0x3C04): s*1 and s*2 sit exactly halfway between bf16 neighbours
    s = oracle.f16_to_f64(0x3C04)
    assert s == 1.00390625
    assert oracle.round_bf16(s * 1) == 1.0            # tie -> even significand
    assert oracle.round_bf16(s * 2) == 2.0            # tie -> even
    assert oracle.round_bf16(s * 3) == 3.015625       # 0.75 ulp above 3 -> up
    assert oracle.round_bf16(-s * 3) == -3.015625
    assert oracle.round_bf16(s * -8) == -8.0          # 1/2 ulp at 8 (2^-4): tie -> even


def test_round_bf16_bruteforce():
    rng = np.random.default_rng(11)
    s16 = rng.integers(0x0001, 0x7BFF, 300)            # positive finite fp16 patterns
    for sb in s16:
        s = oracle.f16_to_f64(int(sb))
        for q in (-8, -7, -3, 1, 5, 7):
            v = s * q
            assert oracle.round_bf16(v) == _bf16_nearest_bruteforce(v)


def test_gemm_dequant_bf16_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    w = synth.weights(9, 0, 6, 24, 128, 0.01)
    sc = np.abs(w.reshape(24, 4, 32)).max(axis=2) / np.float32(7)
    packed, s16 = oracle.pack(w, sc)
    x = synth.calib_x(9, 0, 6, 3, 128, 1.0)
    y, ya = oracle.gemm_cols(x, packed, s16, dequant_bf16=True)
    wh = _numpy_dequant(packed, s16).astype(np.float32)         # s * q, exact in fp32
    wb = torch.from_numpy(wh).to(torch.bfloat16).to(torch.float64).numpy()  # library RNE
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(y, xf @ wb.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(ya, np.abs(xf) @ np.abs(wb).T, rtol=1e-12)
    # and it differs from the exact reading somewhere (the rounding is really applied)
    ye, _ = oracle.gemm_cols(x, packed, s16)
    assert not np.array_equal(y, ye)


def test_gemm_dequant_bf16_power_of_two_scales_is_exact():
    # scales that are powers of two make s * q exact in bf16: both readings agree bit for bit
    codes = np.random.default_rng(3).integers(-8, 8, (16, 64)).astype(np.float32)
    sc = np.float32(2.0) ** np.random.default_rng(4).integers(-6, 3, (16, 2)).astype(np.float32)
    w = codes * np.repeat(sc, 32, axis=1)
    packed, s16 = oracle.pack(w, sc)
    x = synth.calib_x(9, 0, 7, 4, 64, 1.0)
    y1, _ = oracle.gemm_cols(x, packed, s16, dequant_bf16=True)
    y0, _ = oracle.gemm_cols(x, packed, s16)
    assert np.array_equal(y0, y1)
