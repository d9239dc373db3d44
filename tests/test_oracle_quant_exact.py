"""The oracle's quantizer against eq. (4)-(6) and eq. (8) in exact arithmetic.

"BitNet b1.58: 1bit LLM时代" blog, section 一: eq. (8) LayerNorm, eq. (4)-(5)
absmax quantization Clip(x Q_b / gamma, -Q_b + eps, Q_b - eps) with gamma the
largest |LN(x)|, eq. (6) the non-negative range Clip((x - eta) Q_b / gamma,
eps, Q_b - eps) with eta the smallest value.

The oracle decides the integer code in fp32 (mu32, rstd32, h = fl32(fl32(x -
mu32) rstd32), v = fl32(h Q_b / gamma)). This file recomputes every step in
real arithmetic (exact rationals for the mean and variance, 60-digit decimals
for the square root and the quotients) on random rows and checks that:

  * gamma (and eta) lie within the proven error of the fp32 chain of the
    exact values;
  * every code equals trunc (or round-half-even) of clip(v_exact) unless
    v_exact lies within that element's error bound of a point where the code
    changes -- there either neighbour is correct, and the count of such
    elements is printed and bounded.

Error bound (u = 2^-24, per element i of a token with mean mu and exact
reciprocal deviation r; primes denote the fp32 chain):
  mu32 = mu (1 + t1), rstd32 = r (1 + t2), and the subtraction and the product
  add one rounding each, so
      |h'_i - h_i| <= E_i = |h_i| (3u + 3u^2 + u^3) + |mu| r u (1 + u)^3.
  gamma' and gamma are maxima over the same elements, so |gamma' - gamma| <=
  Emax = max_i E_i (same for eta = min h). With |h_i| <= gamma,
      |h'_i / gamma' - h_i / gamma| <= (E_i + Emax) / (gamma - Emax),
  and the final quotient adds one rounding of at most |v'| u <= Q_b u, so
      |v'_i - v_i| <= Q_b (E_i + Emax) / (gamma - Emax) + Q_b u.
  For eq. (6), d = h - eta <= 2 gamma adds |d| u and Emax of eta:
      |v'_i - v_i| <= Q_b (E_i + 2 Emax + 2 gamma u) / (gamma - Emax) + 2 Q_b u.
The tests use twice these bounds (the fp64 statistics add ~1e-16 relative).
"""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import bgb_synth as syn

U = Decimal(2) ** -24
QB = 128
Q_EPS = Fraction(1, 1000)
LN_EPS = Fraction(1, 100000)


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def exact_ln(x: np.ndarray):
    """Per token: exact mean (Fraction) and the LayerNorm output h (Decimal, 60
    digits), plus r = 1/sqrt(Var + eps) (Decimal); eq. (8), biased variance."""
    out = []
    for row in x:
        xs = [Fraction(float(v)) for v in row]
        K = len(xs)
        mu = sum(xs) / K
        var = sum((v - mu) ** 2 for v in xs) / K
        r = Decimal(1) / _dec(var + LN_EPS).sqrt()
        h = [_dec(v - mu) * r for v in xs]
        out.append((mu, r, h))
    return out


def code_of(v: Decimal, lo: Decimal, hi: Decimal, rne: bool, qmax: int) -> int:
    """trunc (or round half to even) of clip(v, lo, hi), clamped to +-qmax."""
    vc = min(hi, max(lo, v))
    if rne:
        c = int(vc.to_integral_value(rounding="ROUND_HALF_EVEN"))
    else:
        c = int(vc)                      # Decimal -> int truncates toward zero
    return max(-qmax, min(qmax, c))


def boundary_distance(v: Decimal, rne: bool, nonneg: bool) -> Decimal:
    """Distance from v to the nearest point where the code changes: nonzero
    integers (truncation) or half-integers (rounding) up to the clip."""
    a = v if nonneg else abs(v)
    if a > QB:                           # beyond the clip every code is Q_b - 1
        a = Decimal(QB)
    if rne:
        k = (a - Decimal("0.5")).to_integral_value(rounding="ROUND_HALF_EVEN")
        cands = [k + Decimal("0.5"), k - Decimal("0.5"), k + Decimal("1.5")]
        cands = [c for c in cands if Decimal("0.5") <= c <= QB - Decimal("1.5")]
    else:
        k = a.to_integral_value(rounding="ROUND_HALF_EVEN")
        cands = [c for c in (k - 1, k, k + 1) if 1 <= c <= QB - 1]
    return min(abs(a - c) for c in cands) if cands else Decimal(QB)


def rows(seed: int, M: int, K: int, kind: str) -> np.ndarray:
    x = syn.normal_f32(seed, 1, (M, K))
    if kind == "shifted":                 # mean far from zero: stresses mu32's rounding
        x = x * np.float32(0.5) + np.float32(3.0)
    elif kind == "heavy":                 # an outlier per token sets gamma
        x[:, 5] = np.float32(25.0) * (1 + np.arange(M, dtype=np.float32))
    elif kind == "scaled":                # tokens of very different scales (tensor gamma)
        x = x * (np.float32(10.0) ** np.arange(M, dtype=np.float32))[:, None]
    return np.ascontiguousarray(x, np.float32)


CASES = [(s, M, K, kind) for (s, M, K) in ((101, 1, 512), (102, 4, 256), (103, 2, 512), (104, 3, 160))
         for kind in ("normal", "shifted", "heavy", "scaled")]


def _check_codes(q, x, nonneg, rne, scope, gamma, eta=None):
    M, K = x.shape
    ln = exact_ln(x)
    hi = _dec(QB - Q_EPS)
    lo = _dec(Q_EPS) if nonneg else -hi
    with localcontext() as ctx:
        ctx.prec = 60
        E = []
        for (mu, r, h) in ln:
            E.append([abs(hv) * (3 * U + 3 * U * U + U ** 3) + abs(_dec(mu)) * r * U * (1 + U) ** 3 for hv in h])
        scopes = [list(range(M))] if scope == 0 else [[m] for m in range(M)]
        band = 0
        for rows_ in scopes:
            g_ex = max(abs(hv) for m in rows_ for hv in ln[m][2])
            emax = max(e for m in rows_ for e in E[m])
            g_dev = Decimal(float(np.asarray(gamma).reshape(-1)[rows_[0] if scope == 1 else 0]))
            assert abs(g_dev - g_ex) <= 2 * emax, ("gamma", g_dev, g_ex, emax)
            eta_ex = min(hv for m in rows_ for hv in ln[m][2])
            if nonneg:
                e_dev = Decimal(float(np.asarray(eta).reshape(-1)[rows_[0] if scope == 1 else 0]))
                assert abs(e_dev - eta_ex) <= 2 * emax, ("eta", e_dev, eta_ex)
            for m in rows_:
                for i in range(K):
                    hv = ln[m][2][i]
                    if nonneg:
                        v = (hv - eta_ex) * QB / g_ex
                        dlt = QB * (E[m][i] + 2 * emax + 2 * g_ex * U) / (g_ex - emax) + 2 * QB * U
                    else:
                        v = hv * QB / g_ex
                        dlt = QB * (E[m][i] + emax) / (g_ex - emax) + QB * U
                    want = code_of(v, lo, hi, rne, QB - 1)
                    got = int(q[m, i])
                    if boundary_distance(v, rne, nonneg) <= 2 * dlt:
                        band += 1
                        assert abs(got - want) <= 1, (m, i, got, want, v)
                    else:
                        assert got == want, (m, i, got, want, v, dlt)
    return band


@pytest.mark.parametrize("rne", [0, 1])
@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("seed,M,K,kind", CASES)
def test_absmax_quant_against_exact_arithmetic(orc, seed, M, K, kind, scope, rne):
    x = rows(seed, M, K, kind)
    q, gamma, mu32, rs32 = orc.ln_absmax_quant(x, round_mode=rne, gamma_scope=scope)
    band = _check_codes(q, x, False, bool(rne), scope, gamma)
    print(f"absmax seed={seed} M={M} K={K} {kind} scope={scope} rne={rne}: {band} of {M * K} codes in the band")
    assert band <= max(2, M * K // 200)


@pytest.mark.parametrize("rne", [0, 1])
@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("seed,M,K,kind", CASES[::2])
def test_nonneg_quant_against_exact_arithmetic(orc, seed, M, K, kind, scope, rne):
    x = rows(seed, M, K, kind)
    q, gamma, eta = orc.ln_nonneg_quant(x, round_mode=rne, gamma_scope=scope)
    band = _check_codes(q, x, True, bool(rne), scope, gamma, eta)
    print(f"nonneg seed={seed} M={M} K={K} {kind} scope={scope} rne={rne}: {band} of {M * K} codes in the band")
    assert band <= max(2, M * K // 200)


def test_exact_check_catches_planted_mistakes(orc):
    """The check above is sharp enough to fail a plausible slip in a quantizer:
    each variant below (built here from the oracle's own outputs) must fail it."""
    x = rows(102, 4, 256, "scaled")
    q, gamma, mu32, rs32 = orc.ln_absmax_quant(x)
    # (a) a token's codes computed with the token's own gamma under tensor scope
    q_tok, g_tok, _, _ = orc.ln_absmax_quant(x, gamma_scope=1)
    with pytest.raises(AssertionError):
        _check_codes(q_tok, x, False, False, 0, gamma)
    # (b) round to nearest where truncation is the reading
    q_rn, _, _, _ = orc.ln_absmax_quant(x, round_mode=1)
    with pytest.raises(AssertionError):
        _check_codes(q_rn, x, False, False, 0, gamma)
    # (c) the sign of one token flipped
    q_neg = q.copy()
    q_neg[1] = -q_neg[1]
    with pytest.raises(AssertionError):
        _check_codes(q_neg, x, False, False, 0, gamma)
    # (d) a gamma off by the unbiased-variance factor sqrt(K/(K-1))
    g_bad = np.float32(float(gamma) * np.sqrt(256 / 255))
    with pytest.raises(AssertionError):
        _check_codes(q, x, False, False, 0, g_bad)
