"""Pins of the sign-bias sweep oracle (oracle/sweep.py, oracle/codebook_sweep.c).

The C version is checked against exact rational arithmetic (every candidate exponent's error
evaluated with Fractions), against the 2-bit re-quantizer's own exact search for the symmetric
codebook, and against invariants the definition fixes: power-of-two scaling, sign reflection, exact
cancellation of +-x pairs under symmetric codebooks, and the tensor statistics rebuilt from blocks.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, requant, sweep
import workloads

SYM = np.array([-4, -1, 1, 4], np.float32)


def _family_sample(rng, k):
    fam = workloads.codebook_family()
    idx = rng.choice(len(fam), size=k, replace=False)
    return [fam[i] for i in idx] + [SYM, np.array([-6, -1, 1, 6], np.float32), np.array([-2, -1, 0, 1], np.float32)]


def _random_block(rng, kind):
    if kind == "normal":
        return (rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
    if kind == "lognormal":
        return (rng.choice([-1, 1], 32) * np.exp(rng.normal(0, 3, 32))).astype(np.float32)
    if kind == "grid":     # values on a coarse grid, so that exact ties with midpoints occur
        return (rng.integers(-16, 17, 32) * 0.25 * 2.0 ** rng.integers(-3, 4)).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "lognormal", "grid"])
def test_block_choice_matches_exact_rationals(kind):
    rng = np.random.default_rng({"normal": 1, "lognormal": 2, "grid": 3}[kind])
    cbs = _family_sample(rng, 12)
    for _ in range(12):
        x = _random_block(rng, kind)
        for q in cbs:
            e, sse, err = sweep.block_choice_c(x, q)
            e_ex, sse_ex, err_ex = sweep.block_choice_fraction(x, q)
            if e != e_ex:   # only a float64 near-tie may choose differently
                _, sse_e, _ = sweep.block_choice_fraction(x, q, exps=[e])
                assert abs(sse_e - sse_ex) <= Fraction(1, 10 ** 12) * sse_ex, (x, q, e, e_ex)
                continue
            scale = float(sse_ex) + 1e-300
            assert abs(sse - float(sse_ex)) <= 1e-13 * scale, (x, q)
            assert abs(err - float(err_ex)) <= 1e-13 * (float(sum(abs(Fraction(float(v))) for v in x)) + 1e-300)


def test_block_choice_edge_blocks_exact():
    """Zeros of both signs, fp32 subnormals, the largest fp32 values, all-zero blocks, and values at
    code midpoints: the C choice equals the exact one, and sse/err equal the exact values."""
    rng = np.random.default_rng(7)
    tiny = np.float32(2.0 ** -149)
    big = np.float32(3.0e38)
    blocks = [
        np.zeros(32, np.float32),
        -np.zeros(32, np.float32),
        np.array([0.0, -0.0] * 16, np.float32),
        np.array([tiny, -tiny] * 16, np.float32),
        np.array([big, -big, 1.0, -1.0] * 8, np.float32),
        np.array([2.5, -2.5, 0.0, -0.0, 1.0, 4.0, -1.0, -4.0] * 4, np.float32),   # midpoints of {-4,-1,1,4}
        np.array([0.5, -0.5, 1.5, -1.5, 0.0, -0.0, 3.0, -3.0] * 4, np.float32),
        np.concatenate([[1.0], np.zeros(31)]).astype(np.float32),
        np.concatenate([[-0.0], np.full(31, 1e-30)]).astype(np.float32),
    ]
    cbs = _family_sample(rng, 10) + [np.array([-1, 0, 1, 2], np.float32), np.array([-3, -1, 1, 3], np.float32)]
    for x in blocks:
        for q in cbs:
            e, sse, err = sweep.block_choice_c(x, q)
            e_ex, sse_ex, err_ex = sweep.block_choice_fraction(x, q)
            assert e == e_ex, (x, q)
            assert sse == float(sse_ex) or abs(sse - float(sse_ex)) <= 1e-15 * float(sse_ex), (x, q)
            assert abs(err - float(err_ex)) <= 1e-15 * max(abs(float(err_ex)), 1e-300) or err == float(err_ex)


def test_zero_tie_follows_sign_bit():
    """x = +0 and -0 between -1 and +1 (a zero midpoint): +0 takes +1, -0 takes -1 at any exponent."""
    q = [Fraction(-4), Fraction(-1), Fraction(1), Fraction(4)]
    assert sweep.nearest_code_fraction((Fraction(0), False), q, -3) == 2
    assert sweep.nearest_code_fraction((Fraction(0), True), q, -3) == 1
    # block of +0 and a 1: the +0 elements cost (2^e)^2 each, as +1 * 2^e
    x = np.array([1.0] + [0.0] * 31, np.float32)
    e, sse, err = sweep.block_choice_c(x, SYM)
    e_ex, sse_ex, err_ex = sweep.block_choice_fraction(x, SYM)
    assert e == e_ex and err == float(err_ex) and err > 0
    xn = -x
    e2, sse2, err2 = sweep.block_choice_c(xn, SYM)
    assert e2 == e and sse2 == sse and err2 == -err


def test_symmetric_codebook_agrees_with_requantizer_search():
    """For {-4,-1,1,4} the sweep's choice is the 2-bit re-quantizer's (an independent exact integer
    search over all 255 exponents): same exponent, and the same exact squared error."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        nib = rng.integers(0, 256, 16, dtype=np.uint8)
        sb = int(rng.integers(100, 150))
        vals = [formats.e2m1_value(int(b) >> (4 * h) & 15) for b in nib for h in (0, 1)]
        x = np.array([v * 2.0 ** (sb - 127) for v in vals], np.float32)
        if not np.any(x):
            continue
        codes, sbyte = requant.requant_block_c_mxfp4(nib, sb, window=False)
        e_rq = sbyte - 127
        sse_rq = sum((Fraction(float(xi)) - Fraction(formats.CODEBOOK[c]) * Fraction(2) ** e_rq) ** 2
                     for xi, c in zip(x, codes))
        e, sse, err = sweep.block_choice_c(x, SYM)
        e_ex, sse_ex, _ = sweep.block_choice_fraction(x, SYM)
        assert sse_ex == sse_rq, trial
        assert e_ex == e_rq or e_rq < e_ex - 7   # an equal error below the window goes to the lower exponent
        assert e == e_ex


def test_power_of_two_scaling_and_reflection():
    rng = np.random.default_rng(5)
    x = workloads.sweep_tensor(0, R=8, C=256)[None]
    cbs = np.stack(_family_sample(rng, 20))
    st, mo, best = sweep.codebook_sweep(x, cbs)
    for k in (-3, 5):
        st2, mo2, best2 = sweep.codebook_sweep(x * np.float32(2.0 ** k), cbs)
        assert np.array_equal(st2[..., 0], st[..., 0] * 4.0 ** k)
        assert np.array_equal(st2[..., 1], st[..., 1] * 2.0 ** k)
        assert np.array_equal(st2[..., 2:], st[..., 2:]) and np.array_equal(best2, best)
    # x -> -x with q -> (-q3, -q2, -q1, -q0): same error, negated bias
    refl = -cbs[:, ::-1].copy()
    st3, _, _ = sweep.codebook_sweep(-x, refl)
    assert np.array_equal(st3[..., 0], st[..., 0])
    assert np.array_equal(st3[..., 1], -st[..., 1])


def test_symmetric_codebooks_cancel_on_signed_pairs():
    """Blocks of interleaved pairs (y, -y): under a sign-symmetric codebook every pair's errors
    cancel exactly (running sum returns to 0 after each pair), so err = bias = 0; an asymmetric
    codebook leaves a bias."""
    rng = np.random.default_rng(9)
    y = (rng.standard_normal((4, 16 * 64)) * 0.02).astype(np.float32)
    x = np.empty((4, 32 * 64), np.float32)
    x[:, 0::2], x[:, 1::2] = y, -y
    cbs = np.array([[-4, -1, 1, 4], [-6, -1.5, 1.5, 6], [-3, -0.5, 0.5, 3], [-4, -1, 0, 1], [-6, -2, 1, 4]], np.float32)
    st, mo, best = sweep.codebook_sweep(x.reshape(1, 4, -1), cbs)
    assert np.all(st[0, :3, 1] == 0.0) and np.all(st[0, :3, 3] == 0.0)
    assert np.all(st[0, 3:, 1] != 0.0)
    assert mo[0, 1] == 0.0
    assert best[0, 0] in (0, 1, 2) and best[0, 1] in (3, 4)


def test_tensor_stats_from_blocks_and_best():
    rng = np.random.default_rng(13)
    x = np.stack([workloads.sweep_tensor(i, R=4, C=128) for i in range(2)])
    cbs = np.stack(_family_sample(rng, 25))
    st, mo, best = sweep.codebook_sweep(x, cbs)
    for t in range(2):
        flat = x[t].reshape(-1, 32)
        N = x[t].size
        s2 = float(np.sum(x[t].astype(np.float64) ** 2))
        assert mo[t, 0] == pytest.approx(s2, rel=1e-14)
        for m in range(len(cbs)):
            sse = err = 0.0
            for blk in flat:
                _, s, e = sweep.block_choice_c(blk, cbs[m])
                sse += s
                err += e
            assert st[t, m, 0] == sse and st[t, m, 1] == err
            assert st[t, m, 2] == pytest.approx(np.sqrt(sse / s2), rel=1e-15)
            assert st[t, m, 3] == pytest.approx(err / np.sqrt(N * s2), rel=1e-15)
        sym = np.array([c[0] == -c[3] and c[1] == -c[2] for c in cbs])
        for kind, mask in ((0, sym), (1, ~sym)):
            cand = np.where(mask)[0]
            want = cand[np.argmin(st[t, cand, 0])]
            assert best[t, kind] == want


def test_codebook_family_definition():
    fam = workloads.codebook_family()
    assert fam.shape == (1239, 4)
    assert np.all(np.diff(fam, axis=1) > 0)
    assert any(np.array_equal(c, SYM) for c in fam)
    grid = set(formats.E2M1_MAGNITUDE) | {-v for v in formats.E2M1_MAGNITUDE}
    assert all(float(v) in grid for v in fam.ravel())
