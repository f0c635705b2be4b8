"""Pins for the oracle's reduced-precision mode (CPU only).

'fp16_weights' rounds every dequantised weight (q - 4) * s once to fp16 and
keeps x and h unrounded.  These tests restate the rounding from the definition
of IEEE binary16 (11-bit significand, exponents -14..15, subnormal spacing
2^-24, round to nearest with ties to even) in exact rationals, work small
cases by hand with ``fractions``, and check that each plausible slip --
rounding x or h too, leaving W unrounded, rounding (q s) instead of
((q - 4) s), breaking ties away from even -- moves the result far beyond the
tolerance the comparison uses.
"""
import math
from fractions import Fraction

import numpy as np

import oracle
from test_oracle_format import _make_blob


def rne_fp16(v) -> Fraction:
    """v rounded to the nearest binary16 value, ties to the even significand."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)               # below 2^-14 the spacing stays 2^-24
    ulp = Fraction(2) ** (e - 10)
    q, r = divmod(a, ulp)
    q = int(q)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    out = q * ulp
    assert out <= 65504, "outside the finite fp16 range"
    return sign * out


def test_rne_fp16_helper_against_known_values():
    assert rne_fp16(Fraction(3, 100)) == Fraction(1024 + 0x3AE, 2 ** 16)  # fp16(0.03) = 0x27AE
    assert float(rne_fp16(0.03)) == float(np.float16(0.03))
    assert rne_fp16(1 + Fraction(1, 2 ** 11)) == 1                  # tie -> even (1.0)
    assert rne_fp16(1 + Fraction(3, 2 ** 11)) == 1 + Fraction(2, 2 ** 10)  # tie -> even (up)
    assert rne_fp16(Fraction(1, 2 ** 25)) == 0                      # half the smallest subnormal: tie to 0
    assert rne_fp16(Fraction(3, 2 ** 26)) == Fraction(1, 2 ** 24)


def _blob(d, f, codes, scales):
    return _make_blob(d, f, [np.asarray(c) for c in codes], [np.asarray(s, dtype=np.float16) for s in scales])


def test_weight_rounding_ties_both_ways():
    # s = 1 + 2^-10: 3 s = 3 + 3 * 2^-10 sits halfway between the fp16 values
    # 3 + 2^-9 and 3 + 2^-8 (spacing 2^-9 in [2, 4)), and rounds up to the even
    # one; s = 1 + 3 * 2^-10: 3 s = 3 + 9 * 2^-10 is halfway between 3 + 4 * 2^-9
    # and 3 + 5 * 2^-9 and rounds down to the even one.  A code of 1 gives -3 s.
    d = f = 32
    for s, want in ((1 + 2 ** -10, 3 + 2 ** -8), (1 + 3 * 2 ** -10, 3 + 2 ** -7)):
        codes = [np.full((f, d), 4), np.full((f, d), 4), np.full((d, f), 4)]
        codes[0][0, 0] = 7
        codes[0][0, 1] = 1
        scales = [np.full((f, 1), s), np.full((f, 1), s), np.full((d, 1), s)]
        wg, _, _ = oracle.expert_weights(_blob(d, f, codes, scales), d, f, fp16_round=True)
        assert wg[0, 0] == want and wg[0, 1] == -want
        assert float(rne_fp16(Fraction(3) * Fraction(s))) == want
        wg_exact, _, _ = oracle.expert_weights(_blob(d, f, codes, scales), d, f)
        assert wg_exact[0, 0] == 3 * s


def _hand_ffn(x, codes, scales, round_w, round_h, round_x):
    """One token through one expert with exact rational sums; silu in float64."""
    (qg, qu, qd), (sg, su, sd) = codes, scales

    def w(q, s, r, c):
        sc = Fraction(float(s[r, c // 32]))
        if round_w == "qs":  # the slip: q * s rounded, 4 s taken off exactly
            return rne_fp16(int(q[r, c]) * sc) - 4 * sc
        v = Fraction(int(q[r, c]) - 4) * sc
        return rne_fp16(v) if round_w else v

    xs = [Fraction(float(v)) for v in x]
    if round_x:
        xs = [rne_fp16(v) for v in xs]
    f, d = qg.shape
    h = []
    for r in range(f):
        g = sum(w(qg, sg, r, c) * xs[c] for c in range(d))
        u = sum(w(qu, su, r, c) * xs[c] for c in range(d))
        gf = float(g)
        hv = Fraction(gf / (1.0 + math.exp(-gf)) * float(u))
        h.append(rne_fp16(hv) if round_h else hv)
    return np.array([float(sum(w(qd, sd, r, c) * h[c] for c in range(f))) for r in range(d)])


def _worked_case(seed):
    d = f = 32
    rng = np.random.default_rng(seed)
    codes = [rng.integers(0, 8, (f, d)), rng.integers(0, 8, (f, d)), rng.integers(0, 8, (d, f))]
    scales = [rng.uniform(0.01, 0.05, (f, 1)).astype(np.float16), rng.uniform(0.01, 0.05, (f, 1)).astype(np.float16),
              rng.uniform(0.01, 0.05, (d, 1)).astype(np.float16)]
    # x with more bits than fp16 keeps, spread so that g and u are O(1)
    x = (rng.standard_normal(d) * 3.0).astype(np.float32)
    return d, f, codes, scales, x


def _close(a, b, tol):
    return np.abs(a - b).max() <= tol * np.abs(b).max()


def test_fp16_weights_hand_worked():
    for seed in (21, 22, 23):
        d, f, codes, scales, x = _worked_case(seed)
        blob = _blob(d, f, codes, scales)
        got = oracle.expert_ffn(x[None, :], oracle.expert_weights(blob, d, f, True), "fp16_weights")[0]
        want = _hand_ffn(x, codes, scales, round_w=True, round_h=False, round_x=False)
        assert _close(got, want, 1e-13)
        # each slip moves the result by far more than the tolerance above
        for slip in (dict(round_w=False, round_h=False, round_x=False),
                     dict(round_w="qs", round_h=False, round_x=False),
                     dict(round_w=True, round_h=True, round_x=False),
                     dict(round_w=True, round_h=False, round_x=True)):
            assert not _close(_hand_ffn(x, codes, scales, **slip), want, 1e-7), slip


def test_reduced_modes_equal_exact_on_representable_operands():
    # Power-of-two scales make every weight an fp16 value.  Token t is
    # x = m_t * p with p a +-1 pattern and m_t in {1, 2, 4}; gate codes are
    # 4 + 3 p_c, so g = 3 * 32 * m_t * s_g(r) = 48 m_t 2^(r mod 3) >= 48, where
    # silu(g) == g in float64 (exp(-40) < 2^-53).  u is m_t times a multiple
    # of 2^-5 with |u / m_t| <= 4, so h = g u has at most 10 significant bits:
    # every h is an fp16 value too (no rounding of h could hide here), and the
    # reduced mode must give the exact result bit for bit.
    d = f = 32
    rng = np.random.default_rng(5)
    p = np.where(rng.random(d) < 0.5, -1, 1)
    qg = np.tile(4 + 3 * p, (f, 1))
    sg = np.array([[0.5 * 2 ** (r % 3)] for r in range(f)])
    qu = rng.integers(0, 8, (f, d))
    su = np.full((f, 1), 2.0 ** -5)
    qd = rng.integers(0, 8, (d, f))
    sd = np.full((d, 1), 2.0 ** -3)
    blob = _blob(d, f, [qg, qu, qd], [sg, su, sd])
    x = np.stack([m * p for m in (1, 2, 4)]).astype(np.float32)
    we = oracle.expert_weights(blob, d, f)
    g = x.astype(np.float64) @ we[0].T
    assert np.all(g >= 48)
    h = oracle.silu(g) * (x.astype(np.float64) @ we[1].T)
    assert np.array_equal(h, h.astype(np.float16).astype(np.float64))  # h representable
    ex = oracle.expert_ffn(x, we, "exact")
    got = oracle.expert_ffn(x, oracle.expert_weights(blob, d, f, True), "fp16_weights")
    assert np.array_equal(got, ex)


def test_unknown_precision_is_refused():
    import pytest
    d = f = 32
    rng = np.random.default_rng(1)
    blob = _blob(d, f, [rng.integers(0, 8, (f, d)), rng.integers(0, 8, (f, d)), rng.integers(0, 8, (d, f))],
                 [np.full((f, 1), 0.03), np.full((f, 1), 0.03), np.full((d, 1), 0.03)])
    with pytest.raises(ValueError):
        oracle.expert_ffn(np.ones((1, d), np.float32), oracle.expert_weights(blob, d, f, True), "fp16_wh")
