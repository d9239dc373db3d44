"""Pins for the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or the mathematics
fix: exact rational brute force (Python ``fractions``/``decimal``), closed
forms, the Sylvester-Hadamard special case (fast Walsh-Hadamard transform),
hand-derived worked examples in ``tests/golden/``, tie and subnormal rules,
and library conversions. Shapes are non-square on purpose so that a swapped
index or transposed operand fails.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import bgb_synth as syn
from conftest import read_golden

getcontext().prec = 80


# ------------------------------------------------------------ exact helpers --

def frac_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest-even) float32 of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, -149)
    n = round(a / Fraction(2) ** q)  # Fraction rounding is half-to-even
    v = np.float32(float(Fraction(n) * Fraction(2) ** q))
    return np.float32(-v) if neg else v


def unpack_format(P: np.ndarray, K: int, N: int) -> np.ndarray:
    """Independent reader of the packed format: word (t, j) at (t//4)*4N + 4j + t%4,
    bit b = row 32t + b, 1 -> +1, 0 -> -1."""
    S = np.empty((K, N), np.int8)
    for i in range(K):
        t, b = divmod(i, 32)
        for j in range(N):
            w = int(P[(t // 4) * 4 * N + 4 * j + (t % 4)])
            S[i, j] = 1 if (w >> b) & 1 else -1
    return S


def fwht(v: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis (Sylvester order)."""
    a = np.array(v, dtype=np.float64 if v.dtype.kind == "f" else np.int64, copy=True)
    n = a.shape[-1]
    h = 1
    while h < n:
        a = a.reshape(a.shape[:-1] + (n // (2 * h), 2, h))
        x, y = a[..., 0, :].copy(), a[..., 1, :].copy()
        a[..., 0, :] = x + y
        a[..., 1, :] = x - y
        a = a.reshape(a.shape[:-3] + (n,))
        h *= 2
    return a


def sylvester(n: int) -> np.ndarray:
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def small_case(seed, K, N, M):
    W = syn.normal_f32(seed, 0, (K, N), std=0.02)
    x = syn.f32_to_bf16_bits(syn.normal_f32(seed, 1, (M, K)))
    return W, x


# ------------------------------------------------------------- brute force --

@pytest.mark.parametrize("K,N,M", [(32, 5, 2), (64, 9, 3), (96, 7, 1)])
def test_fbi_exact_rational(orc, K, N, M):
    W, xb = small_case(10 + K, K, N, M)
    alpha = orc.fbi_alpha(W)
    for j in range(N):
        exact = sum(abs(Fraction(float(W[i, j]))) for i in range(K)) / K
        assert alpha[j] == frac_to_f32(exact), (j, alpha[j], float(exact))
    y = orc.fbi_linear(xb, W, alpha)
    xf = syn.bf16_bits_to_f32(xb)
    for m in range(M):
        for j in range(N):
            s = sum((Fraction(float(xf[m, i])) if W[i, j] > 0 else -Fraction(float(xf[m, i])))
                    for i in range(K))
            exact = Fraction(float(alpha[j])) * s
            # the fp64 sum of <= 96 bf16 values and the product are exact here
            assert y[m, j] == float(exact), (m, j)


@pytest.mark.parametrize("K,N", [(32, 6), (64, 3)])
def test_bitnet_scalars_exact_rational(orc, K, N):
    W = syn.normal_f32(7, 0, (K, N), mean=0.001, std=0.02)
    c, beta = orc.bitnet_scalars(W)
    tot = sum(Fraction(float(v)) for v in W.ravel())
    tot_abs = sum(abs(Fraction(float(v))) for v in W.ravel())
    assert c == frac_to_f32(tot / (K * N))
    assert beta == frac_to_f32(tot_abs / (K * N))
    S = orc.sign_bitnet(W, c)
    ref = np.where(W.astype(np.float64) - float(c) > 0, 1, -1)
    assert np.array_equal(S, ref)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (2, 96)])
def test_ln_statistics_exact(orc, M, K):
    x = syn.normal_f32(21, 1, (M, K))
    q, gamma, mu32, rs32 = orc.ln_absmax_quant(x)
    for m in range(M):
        xs = [Fraction(float(v)) for v in x[m]]
        mu = sum(xs) / K
        var = sum((v - mu) ** 2 for v in xs) / K
        d = Decimal(var.numerator) / Decimal(var.denominator) + Decimal(Fraction(1e-5).numerator) / Decimal(
            Fraction(1e-5).denominator)
        r = Decimal(1) / d.sqrt()
        assert mu32[m] == frac_to_f32(mu)
        assert rs32[m] == frac_to_f32(Fraction(r))
    # gamma is the largest |h| and its element quantizes to exactly +-(Q_b - 1)
    h = (x - mu32[:, None]) * rs32[:, None]
    assert gamma == np.max(np.abs(h))
    am = np.unravel_index(np.argmax(np.abs(h)), h.shape)
    assert abs(int(q[am])) == 127


def test_bitlinear_acc_brute_force(orc):
    K, N, M = 64, 5, 3
    W = syn.normal_f32(5, 0, (K, N), mean=0.001, std=0.02)
    c, _ = orc.bitnet_scalars(W)
    q = syn.rng_for(5, 9).integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = orc.bitlinear_acc(q, W, c)
    for m in range(M):
        for j in range(N):
            ref = sum(int(q[m, i]) * (1 if float(W[i, j]) > float(c) else -1) for i in range(K))
            assert acc[m, j] == ref


# ------------------------------------------------------- packing round trip --

@pytest.mark.parametrize("K,N", [(32, 1), (96, 5), (160, 3), (256, 7)])
def test_pack_round_trip_and_popcount(orc, K, N):
    W = syn.normal_f32(3, 0, (K, N), std=0.02)
    S = orc.sign_fbi(W)
    P = orc.pack(S)
    T = K // 32
    assert P.size == ((T + 3) // 4) * N * 4
    assert np.array_equal(unpack_format(P, K, N), S)
    for j in range(N):
        words = [int(P[(t // 4) * 4 * N + 4 * j + t % 4]) for t in range(T)]
        assert sum(bin(w).count("1") for w in words) == int(np.sum(S[:, j] > 0))
    # padding words are zero
    used = {(t // 4) * 4 * N + 4 * j + t % 4 for t in range(T) for j in range(N)}
    assert all(P[k] == 0 for k in range(P.size) if k not in used)


# ------------------------------------------------------------ closed forms --

@pytest.mark.parametrize("cval", [0.02, 0.5, 3.0])
def test_fbi_closed_forms(orc, cval):
    K, N, M = 64, 6, 2
    xb = syn.f32_to_bf16_bits(syn.normal_f32(1, 1, (M, K)))
    xf = syn.bf16_bits_to_f32(xb).astype(np.float64)
    Wp = np.full((K, N), cval, np.float32)
    a = orc.fbi_alpha(Wp)
    assert np.all(a == np.float32(cval))
    y = orc.fbi_linear(xb, Wp, a)
    assert np.allclose(y, float(np.float32(cval)) * xf.sum(1)[:, None], rtol=0, atol=1e-12)
    Wn = -Wp
    y = orc.fbi_linear(xb, Wn, orc.fbi_alpha(Wn))
    assert np.allclose(y, -float(np.float32(cval)) * xf.sum(1)[:, None], rtol=0, atol=1e-12)
    Wz = np.zeros((K, N), np.float32)
    a0 = orc.fbi_alpha(Wz)
    assert np.all(a0 == 0)
    assert np.all(orc.fbi_linear(xb, Wz, a0) == 0)
    assert np.all(orc.sign_fbi(Wz) == -1)


def test_ties_and_subnormals(orc):
    tiny = np.float32(np.ldexp(1.0, -149))
    W = np.array([[0.0, -0.0, tiny, -tiny, np.inf, -np.inf, np.nan, 1.0]], np.float32)
    W = np.repeat(W, 32, axis=0)
    S = orc.sign_fbi(W)
    assert list(S[0]) == [-1, -1, 1, -1, 1, -1, -1, 1]
    P = orc.pack(S)
    assert int(P[4 * 2]) == 0xFFFFFFFF and int(P[4 * 3]) == 0


def test_bitnet_constant_weights_all_tie(orc):
    W = np.full((64, 5), 0.37, np.float32)
    c, beta = orc.bitnet_scalars(W)
    assert c == np.float32(0.37) and beta == np.float32(0.37)
    assert np.all(orc.sign_bitnet(W, c) == -1)
    q = syn.rng_for(2, 2).integers(-127, 128, size=(2, 64)).astype(np.int8)
    acc = orc.bitlinear_acc(q, W, c)
    assert np.array_equal(acc, np.repeat(-q.astype(np.int64).sum(1, keepdims=True), 5, 1))
    Wp = np.where(np.arange(64)[:, None] % 2 == 0, 1.0, 2.0).astype(np.float32) * np.ones((1, 5), np.float32)
    cp, _ = orc.bitnet_scalars(Wp)   # c = 1.5; half the entries above it
    assert cp == np.float32(1.5)


@pytest.mark.parametrize("n", [64, 256])
def test_hadamard_special_case(orc, n):
    """W = c * H_n (Sylvester): sign(W) = H, alpha = beta = c, x @ W = c * FWHT(x)."""
    cval = np.float32(0.03125)
    H = sylvester(n)
    W = (H * cval).astype(np.float32)
    M = 3
    xb = syn.f32_to_bf16_bits(syn.normal_f32(8, 1, (M, n)))
    xf = syn.bf16_bits_to_f32(xb).astype(np.float64)
    a = orc.fbi_alpha(W)
    assert np.all(a == cval)
    y = orc.fbi_linear(xb, W, a)
    assert np.allclose(y, float(cval) * fwht(xf), rtol=1e-13, atol=1e-13)
    # BitNet on the same W: c = cval/n > 0, so sign(W - c) = H again
    c, beta = orc.bitnet_scalars(W)
    assert beta == cval
    assert np.array_equal(orc.sign_bitnet(W, c), H.astype(np.int8))
    q = syn.rng_for(8, 3).integers(-127, 128, size=(M, n)).astype(np.int8)
    assert np.array_equal(orc.bitlinear_acc(q, W, c), fwht(q.astype(np.int64)))


def test_unit_vector_probes_read_back_signs(orc):
    K, N = 96, 11
    W = syn.normal_f32(4, 0, (K, N), std=0.02)
    a = orc.fbi_alpha(W)
    S = orc.sign_fbi(W)
    for k in (0, 1, 31, 32, 63, 95):
        e = np.zeros((1, K), np.float32)
        e[0, k] = 1.0
        y = orc.fbi_linear(syn.f32_to_bf16_bits(e), W, a)
        assert np.array_equal(y[0], a.astype(np.float64) * S[k])


# ------------------------------------------------------------ quantization --

def test_quant_bounds_and_invariants(orc):
    M, K = 6, 512
    x = syn.normal_f32(11, 1, (M, K)) * np.float32(3.0)
    x[2] = 1.25  # constant row -> LN gives 0 -> q = 0
    q, gamma, mu32, rs32 = orc.ln_absmax_quant(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(q[2] == 0)
    assert np.any(np.abs(q.astype(np.int32)) == 127)
    xd = x.astype(np.float64)
    for m in (0, 1, 3):
        h = (xd[m] - mu32[m]) * rs32[m]
        var = xd[m].var()
        assert abs(h.mean()) < 1e-6
        assert abs(h.var() - var / (var + 1e-5)) < 1e-5
    # all-zero tensor: gamma = 0 and q = 0
    q0, g0, _, _ = orc.ln_absmax_quant(np.zeros((2, 64), np.float32))
    assert g0 == 0 and np.all(q0 == 0)


def test_quant_golden_closed_forms(orc):
    g = read_golden("quant_closed_forms.txt")
    for pat, qk in (("pattern_a", "q_a"), ("pattern_b", "q_b"), ("pattern_c", "q_c")):
        period = np.array([float(v) for v in g[pat]], np.float32)
        expect = np.array([int(v) for v in g[qk]], np.int8)
        reps = 96 // period.size
        x = np.tile(period, (2, reps))
        q, gamma, _, _ = orc.ln_absmax_quant(x)
        assert np.array_equal(q, np.tile(expect, (2, reps))), pat


def test_quant_rounding_mode_is_truncation(orc):
    """Values just under an integer boundary truncate; the argmax maps to 127, not 128."""
    x = np.tile(np.array([-3, -1, 1, 3], np.float32), (1, 8))
    q, _, _, _ = orc.ln_absmax_quant(x, bits=8)
    assert set(np.unique(q).tolist()) == {-127, -42, 42, 127}
    q4, _, _, _ = orc.ln_absmax_quant(x, bits=4)   # Q_b = 8: 3 -> 7.999 -> 7; 1 -> 2.67 -> 2
    assert set(np.unique(q4).tolist()) == {-7, -2, 2, 7}


# ------------------------------------------------------ worked examples -----

def test_golden_fbi_tiny(orc):
    g = read_golden("fbi_tiny.txt")
    K, N = int(g["K"][0]), int(g["N"][0])
    i = np.arange(K)
    W = np.zeros((K, N), np.float32)
    W[:, 0] = 0.5
    W[:, 1] = np.where(i % 2 == 0, 0.25, -0.75)
    W[0, 2] = 1.0
    x = np.stack([i + 1.0, np.ones(K)]).astype(np.float32)
    xb = syn.f32_to_bf16_bits(x)
    a = orc.fbi_alpha(W)
    assert list(a) == [float(v) for v in g["alpha"]]
    y = orc.fbi_linear(xb, W, a)
    assert list(y[0]) == [float(v) for v in g["y0"]]
    assert list(y[1]) == [float(v) for v in g["y1"]]
    P = orc.pack(orc.sign_fbi(W))
    assert [int(v) for v in P] == [int(v, 16) if v.startswith("0x") else int(v) for v in g["packed"]]


def test_golden_bitnet_tiny(orc):
    g = read_golden("bitnet_tiny.txt")
    K, N = int(g["K"][0]), int(g["N"][0])
    i = np.arange(K)
    p = np.where(i % 3 == 0, 0.0, np.where(i % 3 == 1, 1.0, -1.0))
    W = np.stack([0.25 + 0.125 * p, 0.25 - 0.125 * p], axis=1).astype(np.float32)
    c, beta = orc.bitnet_scalars(W)
    assert c == np.float32(float(g["c"][0])) and beta == np.float32(float(g["beta"][0]))
    S = orc.sign_bitnet(W, c)
    P = orc.pack(S)
    assert [int(v) for v in P] == [int(v, 16) if v.startswith("0x") else int(v) for v in g["packed"]]
    x = np.tile(np.array([-3, -1, 1, 3], np.float32), (1, K // 4))
    q, gamma, _, _ = orc.ln_absmax_quant(x)
    assert list(q[0, :4]) == [int(v) for v in g["q_period"]]
    assert abs(float(gamma) - float(g["gamma_exact"][0])) < 2e-7
    acc = orc.bitlinear_acc(q, W, c)
    assert list(acc[0]) == [int(v) for v in g["acc"]]
    y = orc.bitlinear_out(acc, beta, gamma)
    assert np.allclose(y[0], acc[0] * float(beta) * float(gamma) / 128.0, rtol=0, atol=0)


# ------------------------------------------------------------ conversions --

def test_f16_conversion_matches_ieee_library(orc):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * np.float32(0.02),
        rng.standard_normal(2000).astype(np.float32) * np.float32(100.0),
        (rng.standard_normal(500) * 1e-6).astype(np.float32),   # f16 subnormals
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 6.1035156e-05,
                  5.9604645e-08, 2.9802322e-08, 2.9802326e-08, np.inf, -np.inf], np.float32),
    ])
    mine = orc.f32_to_f16(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)
    back = orc.f16_to_f32(ref)
    assert np.array_equal(back, ref.view(np.float16).astype(np.float32))


def test_quant_rne_closed_forms(orc):
    """Round-to-nearest option: hand-derived codes (golden file), the argmax
    still clamps to Q_b - 1, and every code is the truncated one or one step
    away from zero from it."""
    g = read_golden("quant_closed_forms.txt")
    for pat, key, bits in (("pattern_a", "rne_q_a", 8), ("pattern_c", "rne_q_c", 8), ("pattern_a", "rne4_q_a", 4)):
        period = np.array([float(v) for v in g[pat]], np.float32)
        expect = np.array([int(v) for v in g[key]], np.int8)
        x = np.tile(period, (2, 96 // period.size))
        q, _, _, _ = orc.ln_absmax_quant(x, bits=bits, round_mode=1)
        assert np.array_equal(q, np.tile(expect, (2, 96 // period.size))), key
    x = syn.normal_f32(12, 1, (5, 768)) * np.float32(2.0)
    qt, gt, _, _ = orc.ln_absmax_quant(x)
    qr, gr, _, _ = orc.ln_absmax_quant(x, round_mode=1)
    assert gt == gr
    d = qr.astype(np.int32) - qt.astype(np.int32)
    assert np.all((d == 0) | (d == np.sign(qt.astype(np.int32)) + (qt == 0) * np.sign(x - x.mean(1, keepdims=True)).astype(np.int32)))
    assert np.all(np.abs(qr.astype(np.int32)) <= 127) and np.any(d != 0)


def test_quant_token_scope(orc):
    """Per-token gamma: the closed form of the golden file, and quantizing a
    tensor per token equals quantizing each token alone with one gamma."""
    g = read_golden("quant_closed_forms.txt")
    x = np.stack([np.tile(np.array([-3, -1, 1, 3], np.float32), 24),
                  np.tile(np.array([-0.7, 0.7], np.float32), 48)])
    qa = np.array([int(v) for v in g["q_a"]], np.int8)
    qt, gt, _, _ = orc.ln_absmax_quant(x)
    qk, gk, _, _ = orc.ln_absmax_quant(x, gamma_scope=1)
    assert np.array_equal(qt[0], np.tile(qa, 24)) and np.array_equal(qk[0], np.tile(qa, 24))
    assert np.array_equal(qt[1], np.tile(np.array([int(v) for v in g["tensor_q1"]], np.int8), 48))
    assert np.array_equal(qk[1], np.tile(np.array([int(v) for v in g["token_q1"]], np.int8), 48))
    assert gk.shape == (2,) and gk[0] == gt and gk[1] < gt
    xs = syn.normal_f32(13, 1, (6, 512)) * (np.arange(1, 7, dtype=np.float32)[:, None] ** 2)
    xs[3] = 0.5                                            # constant token: gamma 0, codes 0
    for rm in (0, 1):
        qk, gk, _, _ = orc.ln_absmax_quant(xs, round_mode=rm, gamma_scope=1)
        for m in range(xs.shape[0]):
            q1, g1, _, _ = orc.ln_absmax_quant(xs[m:m + 1], round_mode=rm)
            assert np.array_equal(qk[m], q1[0]) and gk[m] == g1
    # one token: both scopes agree
    q1t, g1t, _, _ = orc.ln_absmax_quant(xs[:1])
    q1k, g1k, _, _ = orc.ln_absmax_quant(xs[:1], gamma_scope=1)
    assert np.array_equal(q1t, q1k) and g1k[0] == g1t


def test_bitlinear_out_per_token_gamma(orc):
    acc = np.array([[3, -5, 0], [7, 1, -2]], np.int64)
    y = orc.bitlinear_out(acc, 0.25, np.array([0.5, 2.0], np.float32))
    assert np.array_equal(y, np.array([[3, -5, 0], [7 * 4, 4, -8]], np.float64) * 0.25 * 0.5 / 128)


# ------------------------------------------------- BitNet b1.58 (ternary) --

def test_ternary_closed_form(orc):
    """W = c * pattern, pattern in {-1, 0, 1} with a fraction f of nonzeros:
    gamma_w = c f and W / gamma_w = pattern / f, which rounds and clips back
    to the pattern (|1/f| >= 1)."""
    rng = syn.rng_for(41, 0)
    for f_keep in (0.55, 0.8, 1.0):
        K, N = 96, 7
        pat = np.where(rng.random((K, N)) < f_keep, np.where(rng.random((K, N)) < 0.5, -1, 1), 0).astype(np.int8)
        pat[0, 0] = 1                                             # at least one nonzero
        c = np.float32(0.0371)
        T, g = orc.ternary(pat.astype(np.float32) * c)
        assert np.array_equal(T, pat)
        f = np.count_nonzero(pat) / pat.size
        assert abs(float(g) - float(c) * f) <= 1e-6 * float(c)


def test_ternary_round_half_to_even(orc):
    """The tie rule of round() (eq. (10)): with eps = 0 and |W| taking the
    values 0.5 and 1.5 equally often, gamma_w = 1 exactly; W / gamma_w = 0.5
    rounds to 0 under ties-to-even (half away from zero would give 1), 1.5
    rounds to 2 and clips to 1."""
    w = np.array([0.5] * 16 + [1.5] * 16 + [-0.5] * 16 + [-1.5] * 16, np.float32).reshape(64, 1)
    T, g = orc.ternary(np.repeat(w, 3, axis=1), eps_w=0.0)
    assert g == 1.0
    assert np.array_equal(T[:, 0], np.array([0] * 16 + [1] * 16 + [0] * 16 + [-1] * 16, np.int8))


def test_ternary_exact_brute_force(orc):
    """RoundClip(W / (gamma + eps), -1, 1) against exact rationals: gamma_w from
    an exact sum rounded once, the divisor rounded to fp32, the quotient exact;
    entries whose exact quotient sits within 2^-20 of a half-integer are
    skipped (the fp32 quotient may round either way there)."""
    W = syn.normal_f32(42, 0, (64, 9), std=0.02)
    W[3, 2] = 0.0
    T, g = orc.ternary(W, eps_w=1e-5)
    n = W.size
    g_exact = sum(Fraction(float(abs(v))) for v in W.ravel()) / n
    assert g == frac_to_f32(g_exact)
    den = Fraction(float(np.float32(g) + np.float32(1e-5)))
    checked = 0
    for (i, j), v in np.ndenumerate(W):
        t = Fraction(float(v)) / den
        frac_part = abs(t - int(t))
        if abs(frac_part - Fraction(1, 2)) < Fraction(1, 2 ** 20):
            continue
        r = round(t)                                              # Fraction: half to even
        assert T[i, j] == max(-1, min(1, r)), (i, j, float(t))
        checked += 1
    assert checked > n - 3 and T[3, 2] == 0


def test_ternary_pack_and_product(orc):
    """Two planes in the packed format (+1 plane, then -1 plane) read back by
    the independent reader; the int8 product against an int64 matmul."""
    rng = syn.rng_for(43, 0)
    K, N, M = 160, 11, 3
    T = rng.integers(-1, 2, size=(K, N)).astype(np.int8)
    P2 = orc.pack_ternary(T)
    half = P2.size // 2
    pos = unpack_format(P2[:half], K, N)
    neg = unpack_format(P2[half:], K, N)
    assert not np.any((pos > 0) & (neg > 0))
    assert np.array_equal((pos > 0).astype(np.int8) - (neg > 0).astype(np.int8), T)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = orc.int8_acc(q, T)
    assert np.array_equal(acc, q.astype(np.int64) @ T.astype(np.int64))
    assert np.all(orc.int8_acc(q, np.zeros((K, N), np.int8)) == 0)
    assert np.array_equal(orc.int8_acc(q, np.ones((K, N), np.int8))[:, 0], q.astype(np.int64).sum(1))


# ------------------------------------------------ FBI-linear backward (STE) --

def _bwd_case(seed, M, K, N):
    W = syn.normal_f32(seed, 0, (K, N), std=0.02)
    x = syn.f32_to_bf16_bits(syn.normal_f32(seed, 1, (M, K)))
    dy = syn.f32_to_bf16_bits(syn.normal_f32(seed, 2, (M, N)))
    alpha = np.linspace(0.25, 1.75, N).astype(np.float32)   # distinct per column: a swapped axis shows
    return W, x, dy, alpha


@pytest.mark.parametrize("M,K,N", [(3, 64, 40), (5, 96, 33)])
def test_fbi_backward_against_the_forward(orc, M, K, N):
    """The forward is linear in x and in alpha, so its gradients are read off the
    forward oracle itself: with L = <dY, y(x, alpha)>, dX[m][i] = L at x = e_mi,
    i.e. dY times the forward of the identity batch transposed; dalpha_j = L at
    alpha = e_j, i.e. sum_m dY z with z the forward at alpha = 1."""
    W, x, dy, alpha = _bwd_case(11 + M, M, K, N)
    dx, da, dw = orc.fbi_backward(x, dy, W, alpha)
    dyf = syn.bf16_bits_to_f32(dy).astype(np.float64)
    eye = syn.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    rows = orc.fbi_linear(eye, W, alpha)                    # [K][N]: alpha_j s_ij, through the forward
    assert np.allclose(dx, dyf @ rows.T, rtol=1e-12, atol=1e-12)
    z = orc.fbi_linear(x, W, np.ones(N, np.float32))        # [M][N]: x S
    assert np.allclose(da, (dyf * z).sum(0), rtol=1e-12, atol=1e-12)
    # Euler: each argument enters linearly, so <dX, x> = <dalpha, alpha> =
    # <dW, S> = <dY, y>
    y = orc.fbi_linear(x, W, alpha)
    L = float((dyf * y).sum())
    xf = syn.bf16_bits_to_f32(x).astype(np.float64)
    S = orc.sign_fbi(W).astype(np.float64)
    for v in (float((dx * xf).sum()), float((da * alpha).sum()), float((dw * S).sum())):
        assert abs(v - L) <= 1e-10 * max(1.0, abs(L))


def test_fbi_backward_unit_probes(orc):
    """x = e_i and dY = e_j (one token) give dW = alpha_j at (i, j) and zero
    elsewhere, dX = alpha_j s_(., j) and dalpha_j = s_ij: pins the index order of
    all three outputs."""
    K, N = 64, 40
    W = syn.normal_f32(21, 0, (K, N), std=0.02)
    alpha = np.linspace(0.5, 2.0, N).astype(np.float32)
    S = orc.sign_fbi(W)
    for i, j in [(0, 0), (5, 17), (63, 39), (31, 1)]:
        x = np.zeros((1, K), np.float32)
        x[0, i] = 1.0
        dy = np.zeros((1, N), np.float32)
        dy[0, j] = 1.0
        dx, da, dw = orc.fbi_backward(syn.f32_to_bf16_bits(x), syn.f32_to_bf16_bits(dy), W, alpha)
        want = np.zeros((K, N))
        want[i, j] = alpha[j]
        assert np.array_equal(dw, want)
        assert np.array_equal(dx[0], alpha[j] * S[:, j].astype(np.float64))
        want_da = np.zeros(N)
        want_da[j] = S[i, j]
        assert np.array_equal(da, want_da)


def test_fbi_backward_exact_rational(orc):
    """Tiny case recomputed in exact rationals by this test's own loops; the fp64
    oracle must agree to fp64 rounding."""
    M, K, N = 2, 32, 5
    W, x, dy, alpha = _bwd_case(31, M, K, N)
    dx, da, dw = orc.fbi_backward(x, dy, W, alpha)
    xf = [[Fraction(float(v)) for v in row] for row in syn.bf16_bits_to_f32(x)]
    gf = [[Fraction(float(v)) for v in row] for row in syn.bf16_bits_to_f32(dy)]
    af = [Fraction(float(a)) for a in alpha]
    s = [[1 if W[i, j] > 0 else -1 for j in range(N)] for i in range(K)]
    for m in range(M):
        for i in range(K):
            e = sum(gf[m][j] * af[j] * s[i][j] for j in range(N))
            assert abs(Fraction(dx[m, i]) - e) <= abs(e) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    for j in range(N):
        e = sum(gf[m][j] * sum(xf[m][i] * s[i][j] for i in range(K)) for m in range(M))
        assert abs(Fraction(da[j]) - e) <= abs(e) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    for i in range(K):
        for j in range(N):
            e = af[j] * sum(xf[m][i] * gf[m][j] for m in range(M))
            assert abs(Fraction(dw[i, j]) - e) <= abs(e) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


# ------------------------------------------------ non-negative quantizer (6) --

def test_nonneg_quant_golden_closed_forms(orc):
    g = read_golden("quant_nonneg_closed_forms.txt")
    cases = [("pattern_a", "nn_q_a", 8, 0), ("pattern_a", "nn4_q_a", 4, 0), ("pattern_a", "nn4_q_a", 4, 1),
             ("pattern_d", "nn4_q_d", 4, 0), ("pattern_d", "nn4_rne_q_d", 4, 1), ("pattern_d", "nn_q_d", 8, 0),
             ("pattern_d", "nn_q_d", 8, 1)]
    for pat, qk, bits, rm in cases:
        period = np.array([float(v) for v in g[pat]], np.float32)
        expect = np.array([int(v) for v in g[qk]], np.int8)
        reps = 64 // period.size
        x = np.tile(period, (3, reps))
        x[1] *= 10.0                                   # LN removes the scale: same codes
        for scope in (0, 1):
            q, gamma, eta = orc.ln_nonneg_quant(x, bits=bits, round_mode=rm, gamma_scope=scope)
            assert np.array_equal(q, np.tile(expect, (3, reps))), (pat, qk, rm, scope)
    q, gamma, eta = orc.ln_nonneg_quant(np.full((2, 64), 0.37, np.float32))
    assert not q.any() and gamma == 0


def test_nonneg_quant_invariants(orc):
    """Codes lie in [0, Q_b - 1]; the minimum of the scope maps to 0; codes are
    monotone in the LayerNorm output (hence in x within a token); the symmetric
    quantizer's gamma is the same quantity."""
    x = syn.normal_f32(90, 1, (5, 256)) * np.float32(3.0)
    x[2, 7] = 40.0                                     # an outlier sets gamma
    for scope in (0, 1):
        q, gamma, eta = orc.ln_nonneg_quant(x, gamma_scope=scope)
        q0, g0, _, _ = orc.ln_absmax_quant(x, gamma_scope=scope)
        assert np.array_equal(np.asarray(gamma), np.asarray(g0))
        assert q.min() == 0 and q.max() <= 127
        for m in range(x.shape[0]):
            order = np.argsort(x[m], kind="stable")
            assert np.all(np.diff(q[m][order].astype(int)) >= 0)
        if scope == 1:
            assert all(q[m][np.argmin(x[m])] == 0 for m in range(x.shape[0]))
        else:
            m, i = np.unravel_index(np.argmin((x - x.mean(1, keepdims=True)) / x.std(1, keepdims=True)), x.shape)
            assert q[m, i] == 0


# ------------------------------------- exact quotients and subnormal scale --

def subnormal_rows(M: int, K: int, exponent: int) -> np.ndarray:
    """Token m: x = 2^exponent at index (37 m) mod K, zeros elsewhere."""
    x = np.zeros((M, K), np.float32)
    for m in range(M):
        x[m, (37 * m) % K] = np.float32(2.0 ** exponent)
    return x


def test_quant_golden_exact_quotients(orc):
    """Rows whose quotients h Q_b / gamma are exact integers (truncation boundary)
    or exact half-integers (rounding boundary), hand-derived in the golden file."""
    g = read_golden("quant_closed_forms.txt")
    gn = read_golden("quant_nonneg_closed_forms.txt")
    for pat, keys in (("pattern_e", ("q_e", "rne_q_e")), ("pattern_f", ("q_f", "rne_q_f"))):
        period = np.array([float(v) for v in g[pat]], np.float32)
        x = np.tile(period, (3, 64 // period.size))
        for rm, key in enumerate(keys):
            for scope in (0, 1):
                q, gamma, _, _ = orc.ln_absmax_quant(x, round_mode=rm, gamma_scope=scope)
                expect = np.tile(np.array([int(v) for v in g[key]], np.int8), (3, 64 // period.size))
                assert np.array_equal(q, expect), (pat, key, scope)
    x = np.tile(np.array([float(v) for v in gn["pattern_e"]], np.float32), (2, 16))
    for rm in (0, 1):
        q, _, _ = orc.ln_nonneg_quant(x, round_mode=rm)
        assert np.array_equal(q, np.tile(np.array([int(v) for v in gn["nn_q_e"]], np.int8), (2, 16)))


def test_quant_golden_subnormal_scale(orc):
    """gamma below Q_b / FLT_MAX: the codes are still those of eq. (4)."""
    g = read_golden("quant_closed_forms.txt")
    gn = read_golden("quant_nonneg_closed_forms.txt")
    e, K = int(g["subnormal_exponent"][0]), int(g["subnormal_K"][0])
    x = subnormal_rows(3, K, e)
    assert x[0, 0] == np.float32(2.0 ** e) and x[0, 0] < np.finfo(np.float32).tiny   # a subnormal
    qb_over_max = np.float32(128.0) / np.finfo(np.float32).max
    for rm in (0, 1):
        for scope in (0, 1):
            q, gamma, _, _ = orc.ln_absmax_quant(x, round_mode=rm, gamma_scope=scope)
            assert np.all(np.asarray(gamma) < qb_over_max)
            hot = q[np.arange(3), (37 * np.arange(3)) % K]
            assert np.all(hot == int(g["subnormal_q0"][0]))
            assert np.count_nonzero(q) == 3 and int(g["subnormal_qrest"][0]) == 0
            qn, gn_, eta = orc.ln_nonneg_quant(x, round_mode=rm, gamma_scope=scope)
            assert np.all(qn[np.arange(3), (37 * np.arange(3)) % K] == int(gn["nn_subnormal_q0"][0]))
            assert np.count_nonzero(qn) == 3 and int(gn["nn_subnormal_qrest"][0]) == 0
