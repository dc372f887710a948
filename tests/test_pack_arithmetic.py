"""The activation pack's float32 code arithmetic, emulated on the host.

The kernels decide a code as trunc(RN(x_un r + copysign(0.5 - 2^-25, x_un)))
with r = RN(1 / s_un), pre-scaling rows with a tiny absmax by 2^64 and
clamping their codes (tests/pack_arith_emulation.c restates those steps in C
with correctly rounded host float32 operations).  These CPU tests check that
arithmetic against the oracle's decision ([ICS, Runtime activation
quantization]: s = max|X_rot| / 127, Q = clamp(round(X_rot / s), -127, 127),
round half away from zero), including rows whose scale is subnormal or
underflows, where a reciprocal of the scale would overflow float32.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import convrot_oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))
HALF = float(np.float32(0.5) - np.float32(2.0**-25))  # 0.5 - 2^-25, exact in float32


def _bits(f):
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0])


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("emu") / "pack_arith_emulation.so")
    flags = ["-O3", "-fno-math-errno", "-ffp-contract=off", "-shared", "-fPIC"]
    try:
        with open("/proc/cpuinfo") as f:
            if " fma " in f.read():
                flags.append("-mfma")  # inline fused multiply-adds (same results as libm's fmaf)
    except OSError:
        pass
    subprocess.run(["gcc", *flags, os.path.join(HERE, "pack_arith_emulation.c"), "-o", out, "-lm"],
                   check=True)
    lib = ctypes.CDLL(out)
    lib.round_step_mismatches.restype = ctypes.c_longlong
    lib.round_step_mismatches.argtypes = [ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32]
    lib.rne_step_mismatches.restype = ctypes.c_longlong
    lib.rne_step_mismatches.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_long,
                                        ctypes.c_uint64]
    lib.emulate_row.restype = None
    lib.emulate_row.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    return lib


def emulate(lib, x_un, n):
    """Codes and scales of every row of x_un (float32 2^n X_rot) as the kernels form them."""
    x_un = np.ascontiguousarray(x_un, dtype=np.float32)
    m, k = x_un.shape
    q = np.zeros((m, k), dtype=np.int8)
    s = np.zeros(m, dtype=np.float32)
    for i in range(m):
        lib.emulate_row(x_un[i].ctypes.data, k, n, q[i].ctypes.data, s[i:].ctypes.data)
    return q, s


def test_round_step_exhaustive(emu):
    """Every float32 |v| <= 128: trunc(RN(v + copysign(0.5 - 2^-25, v))) == round(v)."""
    assert emu.round_step_mismatches(HALF, 0, _bits(128.0)) == 0


def test_round_step_check_has_teeth(emu):
    """With 0.5 in place of 0.5 - 2^-25 the largest float below 0.5 (and others)
    rounds up: the exhaustive check must see that on a small range."""
    lo, hi = _bits(0.4999), _bits(0.5001)
    assert emu.round_step_mismatches(0.5, lo, hi) > 0
    assert emu.round_step_mismatches(HALF, lo, hi) == 0


def _rne_mismatches(lib, rs, xs_per_r=2000, seed=1):
    rs = np.ascontiguousarray(rs, dtype=np.float32)
    return lib.rne_step_mismatches(rs.ctypes.data, rs.size, xs_per_r, seed)


def test_rne_step_exact_when_r_has_nine_bits(emu):
    """r with at least 9 significant bits (low 16 encoding bits not all zero):
    the low byte of RN(x r + 1.5 2^23) is round half away from zero of the
    exact product for every x -- no exact ties exist -- checked on the x
    nearest every half-integer and on random x, for random r over 2^-20..2^20
    and for the reciprocals r = RN(1/s) of scales s = RN(m/127) of random
    maxima m."""
    rng = np.random.default_rng(7)
    bits = (rng.integers(127 - 20, 127 + 20, 3000).astype(np.uint32) << 23) | \
        rng.integers(0, 1 << 23, 3000).astype(np.uint32)
    rs = bits.view(np.float32)
    m = rng.lognormal(0.0, 3.0, 3000).astype(np.float32)
    rs2 = (np.float32(1.0) / (m / np.float32(127.0))).astype(np.float32)
    rs = np.concatenate([rs, rs2])
    rs = rs[(rs.view(np.uint32) & 0xFFFF) != 0]
    assert rs.size > 5900
    assert _rne_mismatches(emu, rs) == 0


def test_exact_ties_round_away_at_any_scale(emu):
    """x / s exactly a half-integer at a scale that is not a power of two:
    the row's codes are decided with r raised by two ulps (above 1 / s), so
    every such tie rounds away from zero as the oracle's does.  Scales with
    at most 16 significant bits make (k + 1/2) s exactly representable; each
    row holds 127 s (its maximum, so its scale is s) and ties for k = -127 ..
    126."""
    rng = np.random.default_rng(11)
    for _ in range(400):
        e = int(rng.integers(-30, 30))
        mant = (int(rng.integers(1 << 15, 1 << 16)) | 1) << 8  # 16 significant bits, odd part > 255
        s32 = np.float32(np.ldexp(mant / float(1 << 23), e))
        ks = np.arange(-127, 127)
        xt = ((ks + 0.5) * np.float64(s32)).astype(np.float32)
        assert np.array_equal(xt.astype(np.float64), (ks + 0.5) * np.float64(s32))  # exact ties
        row = np.concatenate([[np.float32(127.0) * s32], xt]).astype(np.float32)
        m = float(row.astype(np.float64).__abs__().max())
        q, sc = emulate(emu, row[None, :], 0)
        if sc[0] != s32:
            continue  # m / 127 rounded to another scale: not this case
        want = np.where(ks >= 0, ks + 1, ks)  # half away from zero
        assert np.array_equal(q[0, 1:].astype(np.int64), want), (s32, m)


def test_rne_step_check_has_teeth(emu):
    """For r with fewer significant bits exact ties exist and nearest-even
    differs from half away (which is why such rows take the other decision):
    the check must see that."""
    for r in (1.0, 2.0, 0.5, 1.5, 3.0, 0.75):
        assert (int(np.float32(r).view(np.uint32)) & 0xFFFF) == 0
        assert _rne_mismatches(emu, [r], xs_per_r=0) > 0, r


def _exact_quotient(x32, s32):
    """x / s as exact rationals would give, to float64 precision (ample for the band)."""
    return x32.astype(np.float64) / s32.astype(np.float64)[:, None]


def _check_codes(q_emu, s_emu, q_or, s_or, t, band, what):
    """Scales equal; codes equal except one-step changes where t (the exact
    quotient the decision rounds) lies within band of a half-integer."""
    assert np.array_equal(s_emu, s_or), f"{what}: scale"
    d = q_emu.astype(np.int32) - q_or.astype(np.int32)
    assert np.abs(d).max(initial=0) <= 1, f"{what}: code differs by {np.abs(d).max()}"
    a = np.abs(t)
    near = np.abs(a - np.floor(a) - 0.5) < band
    off = np.count_nonzero((d != 0) & ~near)
    assert off == 0, f"{what}: {off} changed codes away from a rounding tie"
    assert q_emu.min(initial=0) >= -127


def test_unit_scale_near_ties_exact(emu):
    """G = 1, scale 1 (the row holds 127): values next to a tie keep their side."""
    vals = np.array([127.0, 0.49999997, 1.4999999, 2.4999998, 126.49999, -0.49999997,
                     -126.49999, 0.5, -0.5, 1.5, 2.5, -2.5, 126.5, -126.5, 0.0, -0.0],
                    dtype=np.float32)
    want = np.array([127, 0, 1, 2, 126, 0, -126, 1, -1, 2, 3, -3, 127, -127, 0, 0])
    q, s = emulate(emu, vals[None, :], 0)
    assert s[0] == 1.0
    assert np.array_equal(q[0].astype(np.int64), want)
    q_or, s_or = orc.pack_activations(vals[None, :].astype(np.float64), 1)
    assert np.array_equal(q_or[0].astype(np.int64), want) and s_or[0] == 1.0


@pytest.mark.parametrize("g", [1, 16, 64, 256, 16384])
@pytest.mark.parametrize("absmax", [1e-37, 1e-38, 1e-40, 1e-44, 1e-30, 3.0, 1e30])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_tiny_and_wide_scale_rows(emu, g, absmax, x_dtype):
    """Rows of every magnitude, down to a subnormal scale and one that
    underflows to 0: the emulated kernel arithmetic against the oracle.

    The emulation is fed the oracle's own float32 rotation (scaled by 2^n), so
    the two decisions differ only by x r against RN(x / s): one step, and only
    within a few ulp of a tie.  An overflowing reciprocal would instead give
    NaN codes (0 after conversion) where the oracle has +-127."""
    n = orc.log4_group(g)
    k = max(g, 1024)
    rng = np.random.default_rng(g * 2 + (x_dtype == "bf16"))
    x = rng.standard_normal((6, k))
    x[1] = np.where(rng.random(k) < 0.02, 30.0, 1.0) * rng.standard_normal(k)  # outliers
    x[2, :] = 0.0
    x[2, 5] = 1.0  # a single spike
    x[3, :] = 1.0  # constant row
    x[5] = rng.integers(-3, 4, size=k)  # small integers: ties after rotation
    x = x / np.max(np.abs(x), axis=1, keepdims=True) * absmax
    if x_dtype == "bf16":
        x = orc.round_bf16(x)
    x = x.astype(np.float32).astype(np.float64)  # the input as the device receives it
    xr32 = orc.rotate(x, g).astype(np.float32)
    q_or, s_or = orc.pack_activations(x, g)
    q, s = emulate(emu, np.ldexp(xr32.astype(np.float64), n).astype(np.float32), n)
    if absmax <= 1e-44:
        assert np.all(s_or == 0) and np.all(q_or == 0)  # max / 127 underflows: zero rows
    nz = s_or != 0
    t = np.zeros(q.shape)
    t[nz] = _exact_quotient(xr32[nz], s_or[nz])
    band = 2.0**-20 * np.maximum(np.abs(t), 1.0)
    _check_codes(q, s, q_or, s_or, t, band, f"G={g} absmax={absmax} {x_dtype}")
    # every row with a normal scale reaches +-127 somewhere, as on the oracle
    # (a subnormal scale keeps so few bits that max / s can fall below 126.5)
    normal = s_or >= np.float32(2.0**-126)
    assert np.all(np.abs(q[normal].astype(np.int32)).max(axis=1) == 127)


def test_subnormal_scale_rotation_precision(emu):
    """The kernels hold the rotation unnormalised (2^n X_rot) in float32, which
    keeps bits that the oracle's float32 X_rot loses when X_rot is subnormal.
    The codes then differ from the oracle's only where the oracle's decision
    lies within that rounding (|X_rot - fl32(X_rot)| / s) of a tie, and the
    clamp holds them in [-127, 127] even when the scale's own rounding puts
    |x r| past 127.5."""
    rng = np.random.default_rng(5)
    for g in (4, 16, 256):
        n = orc.log4_group(g)
        for absmax in (3e-43, 1e-41, 1e-40, 5e-39):
            x = rng.standard_normal((8, 1024))
            x = x / np.max(np.abs(x), axis=1, keepdims=True) * absmax
            x = x.astype(np.float32).astype(np.float64)
            xr64 = orc.rotate(x, g)
            q_or, s_or = orc.pack_activations(x, g)
            x_un = np.ldexp(xr64, n).astype(np.float32)  # what the butterfly holds
            q, s = emulate(emu, x_un, n)
            assert np.all(np.abs(q.astype(np.int32)) <= 127)
            nz = (s_or != 0) & (s != 0)
            assert np.array_equal(s == 0, s_or == 0)
            xr32 = xr64.astype(np.float32).astype(np.float64)
            x_dev = np.ldexp(x_un.astype(np.float64), -n)
            t = xr32[nz] / s_or[nz].astype(np.float64)[:, None]
            band = (np.abs(x_dev[nz] - xr32[nz]) / s_or[nz].astype(np.float64)[:, None]
                    + 2.0**-20 * np.maximum(np.abs(t), 1.0))
            rel = np.abs(s[nz].astype(np.float64) - s_or[nz]) / s_or[nz]
            # the scale comes from the maximum of the unnormalised values,
            # itself rounded to the subnormal grid: equal up to that grid step
            assert np.all(np.abs(s[nz].astype(np.float64) - s_or[nz])
                          <= 2.0**-149 / 127 + 2.0**-24 * s_or[nz]), f"scale {rel.max()}"
            d = q[nz].astype(np.int32) - q_or[nz].astype(np.int32)
            a = np.abs(t)
            near = np.abs(a - np.floor(a) - 0.5) < band
            assert np.abs(d).max(initial=0) <= 1
            assert np.count_nonzero((d != 0) & ~near) == 0, f"G={g} absmax={absmax}"


def test_scale_formula_cases():
    """Closed cases of s = fl32(m / 127) that the tiny rows rely on."""
    assert np.float32(1e-44) / np.float32(127) == 0  # underflow: a zero scale
    s = np.float32(1e-40) / np.float32(127)
    assert 0 < s < np.float32(2.0**-126)  # subnormal scale
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(1.0) / s)  # 1/s is past float32's range
