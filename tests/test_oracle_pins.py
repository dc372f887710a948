"""Pins for the CPU oracle: each test checks it against something other than itself.

What the stable-diffusion.cpp page "INT8 Convrot Safetensors" fixes:
  * H4 as printed (section "How INT8 convrot works"), stored in tests/golden;
  * R is orthogonal and symmetric, R R^T = I (same section);
  * X_rot W_rot^T = X W^T before quantisation (same section);
  * the scale and code formulas (sections "Weight quantization" and
    "Runtime activation quantization");
  * A in signed 32-bit integers and Y = A s_x s_w + b (same section).
Independent checks used here: closed forms derived from the digit structure of
a Kronecker power, exact rational arithmetic (fractions.Fraction), brute force
on tiny inputs, integer identities, and textbook values of the normal CDF.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import convrot_oracle as orc

GROUPS = [1, 4, 16, 64, 256, 1024]


# --------------------------------------------------------------------------
# H4 and R_G
# --------------------------------------------------------------------------

def _read_printed_h4(golden_dir):
    rows, div = [], None
    with open(os.path.join(golden_dir, "h4_printed.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("divisor"):
                div = int(line.split()[1])
            else:
                rows.append([int(t) for t in line.split()])
    return np.array(rows, dtype=np.float64), div


def test_h4_matches_printed_matrix(golden_dir):
    signs, div = _read_printed_h4(golden_dir)
    assert signs.shape == (4, 4) and div == 2
    assert np.array_equal(orc.h4(), signs / div)


def test_h4_structure():
    h = orc.h4()
    j = np.ones((4, 4))
    p = np.fliplr(np.eye(4))  # reversal permutation
    assert np.array_equal(2 * h, j - 2 * p)  # regular Hadamard: J - 2P
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, np.eye(4))
    assert np.array_equal(h.sum(axis=1), np.ones(4))  # row sums 1 (regular)


def _closed_form_r(g):
    """R[i, j] = 2^-n (-1)^{#digits k with i_k + j_k == 3}, from the digits of i, j."""
    n = int(round(math.log(g, 4)))
    r = np.empty((g, g))
    for i in range(g):
        for jj in range(g):
            neg = 0
            a, b = i, jj
            for _ in range(n):
                if (a % 4) + (b % 4) == 3:
                    neg += 1
                a //= 4
                b //= 4
            r[i, jj] = (-1.0) ** neg * 2.0 ** (-n)
    return r


@pytest.mark.parametrize("g", [1, 4, 16, 64, 256])
def test_rotation_matrix_closed_form(g):
    assert np.array_equal(orc.rotation_matrix(g), _closed_form_r(g))


@pytest.mark.parametrize("g", GROUPS + [4096])
def test_rotation_matrix_properties(g):
    r = orc.rotation_matrix(g)
    n = orc.log4_group(g)
    assert r.shape == (g, g)
    assert np.array_equal(np.abs(r), np.full((g, g), 2.0 ** -n))
    assert np.array_equal(r, r.T)  # symmetric
    if g <= 1024:
        assert np.array_equal(r @ r, np.eye(g))  # involutive, so R R^T = I exactly
    assert np.array_equal(r @ np.ones(g), np.ones(g))  # regular: R 1 = 1
    x = np.random.default_rng(g).standard_normal(g)
    assert abs(np.linalg.norm(r @ x) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)


@pytest.mark.parametrize("bad", [0, 2, 3, 8, 32, 128, 255, 512, -4])
def test_group_size_must_be_power_of_four(bad):
    with pytest.raises(ValueError):
        orc.log4_group(bad)


def test_group_must_divide_k():
    with pytest.raises(ValueError):
        orc.check_group(1000, 16)  # 1000 % 16 != 0
    orc.check_group(1024, 256)


@pytest.mark.parametrize("g", [4, 16, 64])
def test_rotate_is_block_diagonal_product(g):
    rng = np.random.default_rng(7)
    k = 4 * g
    x = rng.standard_normal((5, k))
    big = scipy.linalg.block_diag(*([_closed_form_r(g)] * (k // g)))
    assert np.allclose(orc.rotate(x, g), x @ big, rtol=0, atol=1e-13)


@pytest.mark.parametrize("g", [16, 256])
def test_rotate_special_rows(g):
    k = 2 * g
    # constant rows map to themselves (R 1 = 1 and R symmetric)
    c = np.full((1, k), 3.25)
    assert np.array_equal(orc.rotate(c, g), c)
    # a spike a*e_j spreads to +-a/sqrt(G) over its own group only
    x = np.zeros((1, k))
    j = g + 5
    x[0, j] = 8.0
    y = orc.rotate(x, g)
    assert np.array_equal(y[0, :g], np.zeros(g))
    assert np.array_equal(np.abs(y[0, g:]), np.full(g, 8.0 / math.sqrt(g)))
    assert np.array_equal(y[0, g:], 8.0 * _closed_form_r(g)[j - g])
    # involution: rotating twice gives the input back
    z = np.random.default_rng(3).standard_normal((3, k))
    assert np.allclose(orc.rotate(orc.rotate(z, g), g), z, rtol=0, atol=1e-13)


@pytest.mark.parametrize("m,k,n,g", [(16, 1024, 512, 256), (64, 4096, 256, 1024), (32, 256, 48, 4)])
def test_rotation_preserves_the_linear(m, k, n, g):
    """X_rot W_rot^T == X W^T before quantisation, to 1e-9 in float64."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((m, k))
    x[:, rng.choice(k, 4, replace=False)] *= 50
    w = rng.standard_normal((n, k)) * 0.02
    lhs = orc.rotate(x, g) @ orc.rotate(w, g).T
    rhs = x @ w.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-9 * max(1.0, np.max(np.abs(rhs)))


def test_rotation_spreads_outliers():
    """One outlier per group shrinks by sqrt(G) after the rotation."""
    x = np.zeros((1, 256))
    x[0, 17] = 100.0
    assert np.max(np.abs(orc.rotate(x, 256))) == pytest.approx(100.0 / 16)


# --------------------------------------------------------------------------
# Rounding and quantisation
# --------------------------------------------------------------------------

def test_round_half_away_ties_and_neighbours():
    f32 = np.float32
    below_half = np.nextafter(f32(0.5), f32(0))  # 0.49999997
    v = np.array([0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5, below_half,
                  -below_half, 0.0, 3.49999, 3.5, 127.0], dtype=np.float32)
    want = np.array([1, -1, 2, -2, 3, -3, 127, -127, 0, 0, 0, 3, 4, 127], dtype=np.float32)
    assert np.array_equal(orc.round_half_away(v), want)
    vd = v.astype(np.float64)
    assert np.array_equal(orc.round_half_away(vd), want.astype(np.float64))


def _exact_round_half_away(q: Fraction) -> int:
    a = abs(q)
    t = a.numerator // a.denominator
    if a - t >= Fraction(1, 2):
        t += 1
    return t if q >= 0 else -t


def _rn_float32(q: Fraction) -> np.float32:
    """Nearest float32 to the rational q, ties to even (from the IEEE definition)."""
    lo = np.float32(float(q))
    # walk to the two float32 neighbours bracketing q
    while Fraction(float(lo)) > q:
        lo = np.nextafter(lo, np.float32(-np.inf))
    while Fraction(float(np.nextafter(lo, np.float32(np.inf)))) <= q:
        lo = np.nextafter(lo, np.float32(np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dlo = q - Fraction(float(lo))
    dhi = Fraction(float(hi)) - q
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if (lo.view(np.int32) & 1) == 0 else hi


def test_weight_quantiser_brute_force():
    """float64 weight codes equal exact rational round(W_rot / s_w) with s_w = fp32(max/127)."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((6, 40)) * rng.lognormal(0, 2, (6, 1))
    w[2] = 0.0
    q, s = orc.quantize_weight_rows(w)
    for o in range(w.shape[0]):
        m = max(abs(Fraction(float(v))) for v in w[o])
        s_exact = _rn_float32(m / 127) if m != 0 else np.float32(0)
        # s_w is the float64 quotient rounded to float32; for these rows it equals the
        # directly rounded float32 quotient
        assert s[o] == s_exact
        for i in range(w.shape[1]):
            if s[o] == 0:
                want = 0
            else:
                want = _exact_round_half_away(Fraction(float(w[o, i])) / Fraction(float(s[o])))
                want = max(-127, min(127, want))
            assert q[o, i] == want, (o, i)
    assert np.all(q[2] == 0) and s[2] == 0


def test_activation_quantiser_brute_force():
    """float32 activation codes: s = RN32(max/127), v = RN32(x/s), then round-half-away."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((5, 48)) * rng.lognormal(0, 2, (5, 1))).astype(np.float32)
    x[3] = 0.0
    q, s = orc.quantize_activation_rows(x)
    for r in range(x.shape[0]):
        m = max(abs(Fraction(float(v))) for v in x[r])
        s_want = _rn_float32(m / 127) if m != 0 else np.float32(0)
        assert s[r] == s_want
        for i in range(x.shape[1]):
            if s_want == 0:
                want = 0
            else:
                v = _rn_float32(Fraction(float(x[r, i])) / Fraction(float(s_want)))
                want = max(-127, min(127, _exact_round_half_away(Fraction(float(v)))))
            assert q[r, i] == want, (r, i)


def test_quantiser_ties_with_unit_scale():
    """A row whose absmax is 127 has scale exactly 1, so the codes are round(x)."""
    row = np.array([[127.0, 0.5, -0.5, 1.5, 2.5, -2.5, 126.5, -126.5, 0.25, -0.75, 3.0, 0.0]])
    want = np.array([[127, 1, -1, 2, 3, -3, 127, -127, 0, -1, 3, 0]])
    qw, sw = orc.quantize_weight_rows(row)
    qa, sa = orc.quantize_activation_rows(row.astype(np.float32))
    assert sw[0] == 1.0 and sa[0] == 1.0
    assert np.array_equal(qw, want) and np.array_equal(qa, want)


def test_quantiser_invariants():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((200, 64)) * rng.lognormal(0, 3, (200, 1))).astype(np.float32)
    x[7] = 0
    for q, s in (orc.quantize_activation_rows(x), orc.quantize_weight_rows(x.astype(np.float64))):
        assert q.dtype == np.int8
        assert q.min() >= -127 and q.max() <= 127  # never -128
        nz = s != 0
        assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 127)
        assert np.all(q[~nz] == 0)
        # dequantised error within half a step of the row scale
        err = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None] - x)
        assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-6) + 1e-30)


def test_zero_and_tiny_rows():
    x = np.zeros((2, 16), dtype=np.float32)
    x[1, 3] = np.float32(1e-45)  # smallest subnormal: m/127 underflows to 0
    q, s = orc.quantize_activation_rows(x)
    assert np.all(s == 0) and np.all(q == 0)


def test_pack_of_crafted_rows_is_exact():
    """X = y R with half-integer y: the packed codes are round-half-away(y)."""
    from workloads import crafted_rotated_rows

    for g in (1, 4, 16, 256, 1024):
        y = crafted_rotated_rows(g, 2048, 6, seed=g)
        x = orc.rotate(y, g)  # R is its own inverse, so X R = y
        q, s = orc.pack_activations(x, g)
        assert np.all(s == 1.0)
        want = np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -127, 127)  # exact: y is a half-integer
        assert np.array_equal(q, want.astype(np.int8))


# --------------------------------------------------------------------------
# Integer GEMM and scale restoration
# --------------------------------------------------------------------------

def test_int_gemm_matches_int64_brute_force():
    rng = np.random.default_rng(12)
    qx = rng.integers(-127, 128, size=(33, 1024)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(17, 1024)).astype(np.int8)
    a = orc.int_gemm(qx, qw)
    brute = np.zeros((33, 17), dtype=np.int64)
    for r, o in itertools.product(range(33), range(17)):
        brute[r, o] = int(np.dot(qx[r].astype(np.int64), qw[o].astype(np.int64)))
    assert np.array_equal(a, brute)
    assert np.array_equal(a, orc.int_gemm_int64(qx, qw))


def test_int_gemm_closed_forms():
    k = 4096
    ones = np.ones((2, k), dtype=np.int8)
    assert np.all(orc.int_gemm(ones, ones) == k)
    full = np.full((2, k), 127, dtype=np.int8)
    assert np.all(orc.int_gemm(full, full) == 16129 * k)
    assert np.all(orc.int_gemm(full, -full) == -16129 * k)
    kmax = orc.MAX_K_INT32
    assert kmax * 16129 <= 2**31 - 1 < (kmax + 1) * 16129
    big = np.full((1, kmax), 127, dtype=np.int8)
    assert orc.int_gemm(big, big)[0, 0] == 16129 * kmax  # still exact at the limit


def test_dequantize_exact_small_case():
    """Y = A s_x[r] s_w[o] + b[o] with distinct row and column scales (no transposition)."""
    a = np.array([[3, -5, 7], [11, 0, -2]])
    sx = np.array([0.5, 0.25], dtype=np.float32)
    sw = np.array([2.0, 4.0, 8.0], dtype=np.float32)
    b = np.array([1.0, -1.0, 0.5], dtype=np.float32)
    want = np.array([[3 * 0.5 * 2 + 1, -5 * 0.5 * 4 - 1, 7 * 0.5 * 8 + 0.5],
                     [11 * 0.25 * 2 + 1, 0 - 1, -2 * 0.25 * 8 + 0.5]])
    assert np.array_equal(orc.dequantize(a, sx, sw, b), want)
    assert np.array_equal(orc.dequantize(a, sx, sw, None), want - b[None, :])


def test_zero_weight_row_gives_bias_column():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 64))
    w = rng.standard_normal((4, 64))
    w[1] = 0
    b = rng.standard_normal(4).astype(np.float32)
    qx, sx = orc.pack_activations(x, 16)
    qw, sw = orc.quantize_weights(w, 16)
    y = orc.linear(qx, sx, qw, sw, b)
    assert np.array_equal(y[:, 1], np.full(8, np.float64(b[1])))


def test_linear_approximates_fp64_layer():
    """End-to-end oracle error against the unquantised layer is within the int8 step bound."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 1024))
    w = rng.standard_normal((64, 1024)) * 0.02
    b = rng.standard_normal(64) * 0.01
    qx, sx = orc.pack_activations(x, 256)
    qw, sw = orc.quantize_weights(w, 256)
    y = orc.linear(qx, sx, qw, sw, b)
    ref = orc.reference_linear_fp64(x, w, b)
    rel = np.sum(np.abs(y - ref)) / np.sum(np.abs(ref))
    assert rel < 0.05


# --------------------------------------------------------------------------
# GELU (not on the page; the erf form)
# --------------------------------------------------------------------------

def test_gelu_textbook_values():
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    # Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208 (standard normal CDF tables)
    assert orc.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert orc.gelu(np.array([2.0]))[0] == pytest.approx(2 * 0.9772498680518208, rel=1e-15)
    x = np.linspace(-6, 6, 101)
    assert np.allclose(orc.gelu(x) - orc.gelu(-x), x, rtol=0, atol=1e-15)  # x*Phi(x) + x*Phi(-x)*... identity
    assert orc.gelu(np.array([40.0]))[0] == 40.0
    assert orc.gelu(np.array([-40.0]))[0] == 0.0


def test_activation_codes_use_division_not_reciprocal():
    """Codes follow round(RN32(x / s)), not round(RN32(x * RN32(1 / s))).

    Searches float32 values near code ties where the two differ, then checks
    the oracle against the exact-rational form of the division.
    """
    m = np.float32(100.37)
    s = np.float32(m / np.float32(127))
    r = np.float32(np.float32(1) / s)
    found = []
    for k in range(1, 127):
        x0 = np.float32((k + 0.5) * float(s))
        x = x0
        for _ in range(8):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(16):
            exact = _exact_round_half_away(Fraction(float(_rn_float32(Fraction(float(x)) / Fraction(float(s))))))
            recip = _exact_round_half_away(Fraction(float(np.float32(x * r))))
            if exact != recip:
                found.append((x, exact))
            x = np.nextafter(x, np.float32(np.inf))
    assert found, "no distinguishing value found near the ties"
    row = np.array([[m] + [v for v, _ in found]], dtype=np.float32)
    q, s_row = orc.quantize_activation_rows(row)
    assert s_row[0] == s
    assert list(q[0, 1:]) == [want for _, want in found]


# ---------------------------------------------------------------------------
# Low-rank adapter correction (LoRA form, from the unrotated activation)
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_conversion():
    """Rounding to bfloat16 agrees with torch's float32 -> bfloat16 conversion
    (round to nearest even) on float32 inputs, ties and neighbours included."""
    import torch

    rng = np.random.default_rng(11)
    v = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties: bfloat16 value plus half a bfloat16 ulp
    base = torch.from_numpy(v[:2000]).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    f, e = np.frexp(base)
    ties = (base + np.ldexp(np.sign(base), e - 9)).astype(np.float32)
    v = np.concatenate([v, ties])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_bf16(v.astype(np.float64)), want)


def test_lora_rank_one_closed_form():
    """A = e_j (one down row selecting feature j), B = ones: the correction is
    scale * X[:, j] in every output column (exact: scale is a power of two)."""
    rng = np.random.default_rng(12)
    x = orc.round_bf16(rng.standard_normal((5, 64)))
    a = np.zeros((1, 64))
    a[0, 17] = 1.0
    b = np.ones((7, 1))
    corr = orc.lora_correction(x, a, b, 0.5)
    assert np.array_equal(corr, np.repeat(0.5 * x[:, 17:18], 7, axis=1))


def test_lora_scale_applies_before_the_bf16_rounding():
    """x = 1 + 2^-7 (a bfloat16 value), scale 3: 3 x = 3.0234375 lies halfway
    between the bfloat16 neighbours 3.015625 and 3.03125 and rounds to the even
    one, 3.03125; scaling after the rounding would give 3.0234375."""
    x = np.full((1, 16), 0.0)
    x[0, 3] = 1.0 + 2.0**-7
    a = np.zeros((1, 16))
    a[0, 3] = 1.0
    u = orc.lora_down(x, a, 3.0)
    assert u[0, 0] == 3.03125
    assert orc.lora_correction(x, a, np.array([[2.0]]), 3.0)[0, 0] == 6.0625


def test_lora_equals_merged_weight_update():
    """bf16(scale X A^T) B^T equals X (scale B A)^T (the merged low-rank
    weight) up to the bfloat16 rounding of the intermediate."""
    rng = np.random.default_rng(13)
    x = orc.round_bf16(rng.standard_normal((9, 128)))
    a = orc.round_bf16(rng.standard_normal((16, 128)) * 0.05)
    b = orc.round_bf16(rng.standard_normal((24, 16)) * 0.05)
    scale = 2.0
    corr = orc.lora_correction(x, a, b, scale)
    merged = x @ (scale * b @ a).T
    u_exact = scale * (x @ a.T)
    bound = (np.abs(u_exact) * 2.0 ** -8) @ np.abs(b).T  # half-ulp per U element
    assert np.all(np.abs(corr - merged) <= bound + 1e-12)
    assert not np.allclose(orc.lora_correction(x, a, b, -scale), merged)  # sign matters
    # transposed operands would not even have matching shapes
    with pytest.raises(ValueError):
        orc.lora_correction(x, a.T, b, scale)
