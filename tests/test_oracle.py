"""Pins for the CPU oracle: each test ties it to something other than itself.

Pages cited: "MIT 6.5940 L13 LLM Deployment" guide (AWQ section, slides 25-28;
TinyChat; QServe table), "CMU 11-868 Model Quantization" guide (L19 absmax and
zero-point), "MIT 6.5940 Lab 4 + Lab 5" guide (Lab 4 setup), "Quantization for
LLMs" chapter 11 (section 11.3).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- helpers
def _half_bits_exact(v):
    """Binary16 round-to-nearest-even of an exact rational, from the IEEE rules."""
    v = Fraction(v)
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    if a == 0:
        return sign

    def rne(r):
        f = r.numerator // r.denominator
        rem = r - f
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
            f += 1
        return f

    if a < Fraction(1, 2 ** 14):
        m = rne(a * 2 ** 24)
        return sign | m  # m == 1024 is the smallest normal, same bits
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    m = rne(a / Fraction(2) ** (e - 10))
    if m == 2048:
        e, m = e + 1, 1024
    if e + 15 >= 31:
        return sign | 0x7C00
    return sign | ((e + 15) << 10) | (m - 1024)


def _f16_to_fraction(bits):
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    m = bits & 1023
    if e == 0:
        return s * Fraction(m, 2 ** 24)
    return s * Fraction(m + 1024, 2 ** 25) * Fraction(2) ** e


# ---------------------------------------------------------------- R8: f64 -> f16
def test_f64_to_f16_matches_exact_rational_rne():
    vals = []
    # random magnitudes over the whole fp16 range, including subnormals
    for _ in range(3000):
        vals.append(float(RNG.uniform(-1, 1) * 2.0 ** RNG.integers(-26, 16)))
    # exact midpoints between neighbours, and midpoint +- one double ulp
    for b in list(range(1, 40)) + list(range(1000, 1100)) + list(range(0x3BF0, 0x3C10)) + list(range(0x7BF0, 0x7BFF)):
        lo, hi = _f16_to_fraction(b), _f16_to_fraction(b + 1)
        mid = float((lo + hi) / 2)
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    vals += [1 + 2 ** -11 + 2 ** -40, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -25 + 2.0 ** -60, 3 * 2.0 ** -26]
    got = oracle.f64_to_f16(np.array(vals, dtype=np.float64)).view(np.uint16)
    for v, g in zip(vals, got):
        assert int(g) == _half_bits_exact(Fraction(v)), (v, hex(int(g)))
    # the double-rounding probe: a float32 intermediate would give 0x3C00
    assert int(oracle.f64_to_f16(np.float64(1 + 2 ** -11 + 2 ** -40)).view(np.uint16)) == 0x3C01


# ---------------------------------------------------------------- P1: brute force nearest level
@pytest.mark.parametrize("bits,group", [(4, 4), (4, 8), (4, 16), (3, 4), (3, 8), (3, 16)])
def test_rtn_picks_nearest_level_brute_force(bits, group):
    n, g = 24, 6
    w = RNG.standard_normal((n, g * group)) * 0.02
    w[0, :group] = np.linspace(-1, 1, group)          # hand-built group
    w[1, :group] = np.arange(group) * 0.125 - 0.25     # dyadic, exact halves possible
    w[2, :group] = 0.3                                  # constant
    w[3, :group] = np.abs(w[3, :group]) + 0.5          # one-signed
    q, delta, z = oracle.quantize_groups(w, bits=bits, group=group)
    levels = 2 ** bits
    for r in range(n):
        for gi in range(g):
            d = Fraction(float(delta[r, gi]))
            zz = Fraction(float(z[r, gi]))
            for c in range(group):
                k = gi * group + c
                x = Fraction(float(w[r, k]))
                dist = [abs(x - (qq - zz) * d) for qq in range(levels)]
                best = min(dist)
                winners = [qq for qq in range(levels) if dist[qq] == best]
                qo = int(q[r, k])
                if qo in winners:
                    continue
                # allowed only where exact w/Delta sits within 2 float64 ulps of k + 1/2
                t = x / d
                frac = t - (t.numerator // t.denominator)
                ulp = Fraction(abs(float(t))) * Fraction(2) ** -51 + Fraction(2) ** -1074
                assert abs(frac - Fraction(1, 2)) <= 2 * ulp, (r, k, qo, winners)
                assert dist[qo] - best <= 4 * ulp * d


def test_delta_and_zero_are_the_stated_quotients():
    """Delta = (max - min)/15 and z = rint(-min/Delta), correctly rounded (R5, R7)."""
    w = RNG.standard_normal((16, 512)) * 0.02
    q, delta, z = oracle.quantize_groups(w, 4, 128)
    wg = w.reshape(16, 4, 128)
    for r in range(16):
        for g in range(4):
            mn, mx = Fraction(float(wg[r, g].min())), Fraction(float(wg[r, g].max()))
            rng64 = Fraction(float(mx - mn))          # step 2: the range, rounded to float64
            assert float(delta[r, g]) == float(rng64 / 15)  # step 3: correctly rounded quotient
            t = -mn / Fraction(float(delta[r, g]))
            assert abs(Fraction(float(z[r, g])) - t) <= Fraction(1, 2) + Fraction(1, 10 ** 9)
            # the minimum lands on code 0, the maximum on code 15 (up to ties)
            k_min = int(np.argmin(wg[r, g]))
            assert q[r, g * 128 + k_min] == 0


def test_round_half_to_even_and_round_before_adding_zero():
    """R2/R3: rint(2.5) = 2, and q = rint(w/Delta) + z (not rint(w/Delta + z))."""
    # group of 4 with min -1.5*D... choose Delta = 1 via range 15
    w = np.array([[-5.0, 10.0, 2.5, 3.5]])  # range 15 -> Delta = 1, z = rint(5) = 5
    q, delta, z = oracle.quantize_groups(w, 4, 4)
    assert float(delta[0, 0]) == 1.0 and float(z[0, 0]) == 5.0
    assert list(q[0]) == [0, 15, 7, 9]  # rint(2.5)=2 -> 7; rint(3.5)=4 -> 9
    # with z odd, round-after-add would differ: w = 2.5, z = 6 -> 8 here vs rint(8.5)=8 too;
    w = np.array([[-6.0, 9.0, 2.5, -0.5]])  # Delta 1, z = 6
    q, _, z = oracle.quantize_groups(w, 4, 4)
    assert float(z[0, 0]) == 6.0
    assert list(q[0]) == [0, 15, 8, 6]  # rint(-0.5) = -0 -> 6 ; rint(-0.5 + 6) would be 6 as well
    w = np.array([[-7.0, 8.0, 1.5, 0.5]])  # z = 7: round-first gives 2+7=9, 0+7=7
    q, _, _ = oracle.quantize_groups(w, 4, 4)
    assert list(q[0]) == [0, 15, 9, 7]  # round-after-add would give rint(8.5)=8, rint(7.5)=8


# ---------------------------------------------------------------- P2/P3: invariants
@pytest.mark.parametrize("bits,group", [(4, 128), (4, 64), (4, 32), (3, 128), (3, 32)])
@pytest.mark.parametrize("kind", ["normal", "ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
def test_error_within_half_step_and_code_range(kind, bits, group):
    import synth

    if kind == "normal":
        W = synth.weights(1, 0, 64, 1024)
    else:
        W = synth.edge_weights(kind, 64, 1024, seed=3)
    w = W.astype(np.float64)
    q, delta, z = oracle.quantize_groups(w, bits, group)
    assert q.min() >= 0 and q.max() <= 2 ** bits - 1
    assert np.all(z == np.rint(z))
    qw = oracle.pseudo_quantize(w, bits, group)
    d = np.repeat(delta, group, axis=1)
    assert np.all(np.abs(w - qw) <= d / 2 * (1 + 2.0 ** -40))
    # the group's minimum maps to code 0 exactly (rint(-a) = -rint(a)); its maximum to the top
    # code, or one below where -min/Delta sits at a rounding tie
    wg = w.reshape(64, -1, group)
    qg = q.reshape(64, -1, group)
    spread = wg.max(axis=2) > wg.min(axis=2)
    assert np.all(np.take_along_axis(qg, wg.argmin(axis=2)[:, :, None], 2)[:, :, 0][spread] == 0)
    top = np.take_along_axis(qg, wg.argmax(axis=2)[:, :, None], 2)[:, :, 0][spread]
    assert np.all(top >= 2 ** bits - 2)
    if kind == "normal":
        assert np.mean(top == 2 ** bits - 1) > 0.9


def test_zero_offset_is_positive_zero():
    """R4: a group whose minimum is +0 or -0 stores the zero offset as +0."""
    w = np.zeros((2, 128), dtype=np.float16)
    w[0, 5] = 0.5
    w[1, 5] = 0.5
    w[1, 0] = np.float16(-0.0)
    _, _, zeros = oracle.quantize_pack(w)
    assert list(zeros.view(np.uint16)[:, 0]) == [0, 0]


def test_constant_group_reading():
    """R6: a constant group uses range 1, so Delta = 1/15; all-zero groups give q = z = 0."""
    w = np.zeros((2, 256))
    w[1] = 0.3
    q, delta, z = oracle.quantize_groups(w, 4, 128)
    assert np.all(delta == 1.0 / 15.0)
    assert np.all(q[0] == 0) and np.all(z[0] == 0)
    assert np.all(oracle.pseudo_quantize(w, 4, 128)[0] == 0.0)


# ---------------------------------------------------------------- P4: the pages' error statistic
@pytest.mark.parametrize("bits,group", [(4, 128), (3, 128), (4, 32)])
def test_mean_round_error_is_a_quarter_step(bits, group):
    """L13 AWQ slides 26/28: the expected rounding error is about 0.25 (in steps)."""
    import synth

    W = synth.weights(9, 0, 1024, 1024)
    w = W.astype(np.float64)
    _, delta, _ = oracle.quantize_groups(w, bits, group)
    err = np.abs(w - oracle.pseudo_quantize(w, bits, group)) / np.repeat(delta, group, axis=1)
    assert abs(err.mean() - 0.25) < 0.01


def test_scaling_a_salient_channel_divides_its_error():
    """L13 AWQ slides 26/28: multiply a channel by s, divide back: if Delta barely
    changes the error on that channel shrinks by about s."""
    rng = np.random.default_rng(5)
    n, k = 4096, 1024
    w = rng.standard_normal((n, k)) * 0.02
    sal = np.arange(3, k, 128)          # one channel per group
    s = np.ones(k)
    s[sal] = 2.0
    # keep the salient weights small so max|w| of the group is unchanged
    w[:, sal] *= 0.25
    e0 = np.abs(oracle.pseudo_quantize(w, 4, 128) - w)[:, sal].mean()
    ws = w * s
    e1 = np.abs(oracle.pseudo_quantize(ws, 4, 128) / s - w)[:, sal].mean()
    assert 0.45 < e1 / e0 < 0.55


# ---------------------------------------------------------------- P5: scaling identity
def test_power_of_two_scaling_is_exact_end_to_end():
    """Chapter 11 section 11.3 / L13 slide 13: (X diag(s)^-1)(diag(s) W) = XW.

    With s a power of two, constant over each group, every rounding step is
    exact: codes and zeros are unchanged, Delta scales by s, x/s is exact, and
    the float64 outputs are bit-identical.
    """
    rng = np.random.default_rng(11)
    n, k, m = 96, 1024, 3
    W = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    x = rng.standard_normal((m, k))
    x = (np.sign(x) * np.maximum(np.abs(x), 2.0 ** -6)).astype(np.float16)
    j = rng.integers(-2, 3, size=k // 128)
    s = np.repeat(2.0 ** j, 128).astype(np.float32)
    qa, sa, za = oracle.quantize_pack(W, None)
    qb, sb, zb = oracle.quantize_pack(W, s)
    assert np.array_equal(qa, qb) and np.array_equal(za, zb)
    assert np.array_equal(sb.astype(np.float64), sa.astype(np.float64) * 2.0 ** j[None, :])
    xs = oracle.scale_input(x, s)
    assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) / s.astype(np.float64))
    ya, _ = oracle.linear(x, qa, sa, za)
    yb, _ = oracle.linear(xs, qb, sb, zb)
    assert np.array_equal(ya, yb)


def test_general_scaling_identity_holds_in_float64():
    rng = np.random.default_rng(12)
    n, k, m = 64, 512, 4
    w = rng.standard_normal((n, k)) * 0.02
    x = rng.standard_normal((m, k))
    s = rng.uniform(0.5, 4.0, size=k)
    y0 = x @ w.T
    y1 = (x / s) @ (w * s).T
    bound = k * 2.0 ** -50 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(y1 - y0) <= bound)


def test_group_power_of_two_leaves_codes_and_zero():
    rng = np.random.default_rng(13)
    w = rng.standard_normal((8, 256)) * 0.02
    q0, d0, z0 = oracle.quantize_groups(w, 4, 128)
    w2 = w.copy()
    w2[:, 128:] *= 8.0
    q1, d1, z1 = oracle.quantize_groups(w2, 4, 128)
    assert np.array_equal(q0, q1) and np.array_equal(z0, z1)
    assert np.array_equal(d1[:, 1], d0[:, 1] * 8.0) and np.array_equal(d1[:, 0], d0[:, 0])


# ---------------------------------------------------------------- P6: b = 8 vs the page-2 zero-point quantizer
def _zeropoint_int8_from_description(X):
    """The CMU L19 slide 10 zero-point quantizer, restated from its description:
    scale = 255 / (max - min) (range 0 -> 1), zero point = round(-scale*min - 128),
    codes = clip(round(X*scale + zp), -128, 127), half-to-even rounding."""
    rng_ = X.max() - X.min()
    rng_ = 1.0 if rng_ == 0 else rng_
    scale = 255.0 / rng_
    zp = np.round(-scale * X.min() - 128.0)
    return np.clip(np.round(X * scale + zp), -128, 127)


def test_eight_bit_case_matches_page_two_zero_point_quantizer():
    rng = np.random.default_rng(21)
    rows = rng.standard_normal((200, 1024)) * rng.uniform(0.01, 3.0, size=(200, 1))
    rows[:20] += rng.uniform(-2, 2, size=(20, 1))
    total = 0
    diff = 0
    for r in rows:
        q, delta, z = oracle.quantize_groups(r[None, :], bits=8, group=r.size)
        ours = q[0] - 128
        page = _zeropoint_int8_from_description(r)
        d = np.abs(ours - page)
        assert d.max() <= 1
        diff += int((d != 0).sum())
        total += r.size
    assert diff / total <= 1e-4


# ---------------------------------------------------------------- P8: linear exactness
def _exact_linear(x, qw, sc, zr, k, bits=4, group=128):
    codes = oracle.unpack_codes(qw, k) if bits == 4 else oracle.unpack_codes3(qw, k)
    m, n = x.shape[0], qw.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for r in range(n):
            acc = Fraction(0)
            for c in range(k):
                g = c // group
                wv = (codes[r, c] - Fraction(float(zr[r, g]))) * Fraction(float(sc[r, g]))
                acc += Fraction(float(x[i, c])) * wv
            out[i, r] = acc
    return out


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 32), (3, 128), (3, 64)])
def test_linear_matches_exact_rationals(bits, group):
    import synth

    k, n, m = 256, 5, 2
    W = synth.weights(1, 7, n, k)
    x = synth.activations(1, 7, m, k)
    qw, sc, zr = oracle.quantize_pack(W, bits=bits, group=group)
    y, b = oracle.linear(x, qw, sc, zr, group=group, bits=bits)
    ex = _exact_linear(x, qw, sc, zr, k, bits, group)
    for i in range(m):
        for r in range(n):
            assert abs(Fraction(float(y[i, r])) - ex[i, r]) <= Fraction(k) * Fraction(2) ** -52 * Fraction(float(b[i, r]))


def test_linear_special_cases():
    rng = np.random.default_rng(3)
    k, n, m = 512, 6, 3
    x = rng.standard_normal((m, k)).astype(np.float16)
    # every code equal to its zero -> y = 0 exactly
    codes = rng.integers(0, 16, size=(n, k // 128))
    q = np.repeat(codes, 128, axis=1)
    qw = oracle.pack_codes(q)
    sc = rng.uniform(0.001, 0.1, size=(n, k // 128)).astype(np.float16)
    zr = codes.astype(np.float16)
    y, b = oracle.linear(x, qw, sc, zr)
    assert np.all(y == 0.0) and np.all(b == 0.0)
    # q - z = 1 and Delta = 1 -> y = sum_k x (textbook sum)
    zr1 = (codes - 1).astype(np.float16)
    sc1 = np.ones_like(sc)
    y, _ = oracle.linear(x, qw, sc1, zr1)
    ref = np.array([sum(Fraction(float(v)) for v in row) for row in x])
    for i in range(m):
        assert np.all(y[i] == float(ref[i]))


def test_within_tolerance_rule():
    y_ref = np.array([1.0, -2.0, 0.0])
    b = np.array([10.0, 100.0, 0.0])
    ok = oracle.within_tolerance(np.array([1.0 + 0.0099, -2.0 - 0.11, 1e-5]), y_ref, b)
    assert list(ok) == [True, False, True]


def test_tolerance_rule_accepts_fp16_overflow_only_beyond_range():
    """R11: fp16 outputs saturate to +-inf at 65520; only then is inf acceptable."""
    inf = np.inf
    y_ref = np.array([2.0e6, -7.0e4, 65519.0, 1000.0, 2.0e6])
    b = np.array([3.0e6, 7.0e4, 1.0, 1000.0, 3.0e6])
    y = np.array([inf, -inf, inf, inf, -inf])
    assert list(oracle.within_tolerance(y, y_ref, b)) == [True, True, False, False, False]
    # 65504 + half an ulp (16) is the exact binary16 overflow threshold
    assert np.float64(65519.99).astype(np.float16) == np.float16(65504)
    from oracle.linear import F16_OVERFLOW

    with np.errstate(over="ignore"):
        assert np.isinf(np.float64(F16_OVERFLOW).astype(np.float16))


# ---------------------------------------------------------------- a1: AWQ statistic and input fold
def test_channel_scale_closed_forms():
    t, k = 512, 256
    x = np.zeros((t, k), dtype=np.float16)
    x[:, 0] = 4.0
    x[::2, 1] = -2.0                  # mean |x| = 1
    x[:, 2] = np.where(np.arange(t) % 2 == 0, 1.0, -9.0)  # mean 5
    s = oracle.channel_scale(x, 0.5)
    assert s[0] == 2.0 and s[1] == 1.0
    assert s[3] == 1.0                # all-zero channel: reading R9
    assert oracle.channel_scale(x, 1.0)[2] == 5.0
    assert np.all(oracle.channel_scale(x, 0.0) == 1.0)


def test_channel_scale_is_correctly_rounded_sqrt_of_mean():
    import synth

    xc = synth.calibration(2, 3, 1024)
    s = oracle.channel_scale(xc, 0.5)
    for kk in range(0, 1024, 37):
        mean = sum(abs(Fraction(float(v))) for v in xc[:, kk]) / xc.shape[0]
        # float64 sqrt of the float64 mean, then float32: bracket with exact rationals
        m64 = Fraction(float(mean))
        assert abs(m64 - mean) <= mean * Fraction(2) ** -53
        sv = Fraction(float(s[kk]))
        ulp = Fraction(float(np.spacing(np.float32(s[kk]))))
        assert (sv - ulp / 2) ** 2 <= m64 * (1 + Fraction(2) ** -50)
        assert (sv + ulp / 2) ** 2 >= m64 * (1 - Fraction(2) ** -50)


def test_channel_scale_on_the_alpha_grid_brackets_the_exact_power():
    """s = m^(i/20) for every point of the search grid (L13 AWQ section: s = s_X^alpha), pinned
    in exact rationals: with m the exact mean of |x| (a rational: fp16 magnitudes summed, over
    T), the float32 s must satisfy (s - ulp/2)^20 <= m^i <= (s + ulp/2)^20, up to the float64
    arithmetic before the final rounding (a relative 2^-45 after the 20th power)."""
    import synth

    xc = synth.calibration(2, 5, 1024)
    t = xc.shape[0]
    chans = list(range(0, 1024, 61)) + [int(c) for c in synth.outlier_channels(2, 5, 1024)[:4]]
    eps = Fraction(1, 2 ** 45)
    for i in range(21):
        s = oracle.channel_scale(xc, i / 20)
        for kk in chans:
            m = sum(abs(Fraction(float(v))) for v in xc[:, kk]) / t
            sv = Fraction(float(s[kk]))
            ulp = Fraction(float(np.spacing(np.float32(s[kk]))))
            target = m ** i
            assert (sv - ulp / 2) ** 20 <= target * (1 + eps), (i, kk)
            assert (sv + ulp / 2) ** 20 >= target * (1 - eps), (i, kk)
    # the oracle's own alpha argument is the float64 i/20; alpha = 0 gives 1 exactly
    assert np.all(oracle.channel_scale(xc, 0.0) == 1.0)


def test_channel_scale_outlier_statistics():
    import synth

    xc = synth.calibration(3, 0, 8192)
    s = oracle.channel_scale(xc, 0.5).astype(np.float64)
    outl = synth.outlier_channels(3, 0, 8192)
    normal = np.setdiff1d(np.arange(8192), outl)
    # E|N(0,1)| = sqrt(2/pi); s = sqrt of it, and sqrt(20x) on outlier channels
    assert abs(s[normal].mean() - np.sqrt(np.sqrt(2 / np.pi))) < 0.01
    assert abs(s[outl].mean() - np.sqrt(20 * np.sqrt(2 / np.pi))) < 0.05


def test_scale_input_is_single_rounded_division():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 512)).astype(np.float16)
    s = rng.uniform(0.3, 5.0, size=512).astype(np.float32)
    xs = oracle.scale_input(x, s)
    for i in range(4):
        for kk in range(0, 512, 7):
            exact = Fraction(float(x[i, kk])) / Fraction(float(s[kk]))
            # the one double rounding of the quotient then RNE to half: compare with
            # the exact half rounding of the double quotient
            q64 = Fraction(float(exact))
            assert int(xs[i, kk].view(np.uint16)) == _half_bits_exact(q64)
