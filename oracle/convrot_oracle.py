"""Plain CPU oracle for the INT8 convrot linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product path.

Source of truth: the stable-diffusion.cpp documentation page
"INT8 Convrot Safetensors" (docs/int8_convrot.md), cited below as [ICS] with the
section name.  The method is an encoding with a heuristic scale, so the oracle
follows the page's steps in the page's order and notation, one plain
definition per step, with no blocking, fusion or reordering:

    1. H4 and its normalised Kronecker power R_G      [ICS, How INT8 convrot works]
    2. X_rot = X R  and  W_rot = W R  (block diagonal) [ICS, How INT8 convrot works]
    3. per-row absmax scale and int8 code             [ICS, Weight quantization;
                                                        ICS, Runtime activation quantization]
    4. A = Q_x Q_w^T in exact integers                [ICS, Runtime activation quantization]
    5. Y = A s_x[r] s_w[o] + b[o]                     [ICS, Runtime activation quantization]

Readings where the page is silent:

* ``round`` is round-half-away-from-zero (the C ``round`` function).
* A row whose absmax is 0 gets scale 0 and all-zero codes.
* Scales are float32 (the page says "floating-point"; the checkpoint stores one
  float per output row).  Codes are computed by dividing by the *stored* float32
  scale, so that dequantisation uses exactly the scale the division used.
* The precision in which a float decides an int8 code is not stated.  The
  oracle takes each decision in the precision the device path uses for it:
  - weights (offline): rotation, absmax, division and rounding in float64;
    the scale is float64(max)/127 rounded once to float32;
  - activations (runtime): the float64 rotation rounded once to float32, then
    absmax, ``s = max/127`` and ``v = x/s`` as correctly rounded float32
    operations, then round-half-away on v.
* GELU (used between the two linears of a DiT MLP block) is not on the page;
  the erf form x * Phi(x) is used, evaluated in float64.

All arrays are NumPy; floats are float64 unless a step states float32.
"""

from __future__ import annotations

import functools
import math

import numpy as np

# ---------------------------------------------------------------------------
# 1. H4 and R_G                                    [ICS, How INT8 convrot works]
# ---------------------------------------------------------------------------

# The +-1 pattern printed on the page; the page divides the whole matrix by 2.
_H4_SIGNS = (
    (1, 1, 1, -1),
    (1, 1, -1, 1),
    (1, -1, 1, 1),
    (-1, 1, 1, 1),
)

MAX_LOG4_GROUP = 7  # largest supported group: 4**7 = 16384


def h4() -> np.ndarray:
    """The normalised regular Hadamard matrix H4 (printed +-1 pattern / 2)."""
    return np.array(_H4_SIGNS, dtype=np.float64) / 2.0


def log4_group(group_size: int) -> int:
    """n with group_size == 4**n; ValueError if group_size is not a power of four.

    [ICS, Checkpoint format]: the group size must be a power of four.
    """
    g = int(group_size)
    n = 0
    while g > 1 and g % 4 == 0:
        g //= 4
        n += 1
    if g != 1 or group_size < 1:
        raise ValueError(f"group size {group_size} is not a power of four")
    return n


@functools.lru_cache(maxsize=4)
def rotation_matrix(group_size: int) -> np.ndarray:
    """R_G, the normalised Kronecker power of H4 with G = 4**n rows (read-only, cached).

    [ICS, How INT8 convrot works]: for G = 4^n the transform is the Kronecker
    power of H4; H4 already carries the 1/2, so the power is orthonormal and no
    further factor is applied.  G = 1 (n = 0) gives the 1x1 identity.
    """
    n = log4_group(group_size)
    r = np.ones((1, 1), dtype=np.float64)
    for _ in range(n):
        r = np.kron(r, h4())
    r.flags.writeable = False
    return r


def check_group(k: int, group_size: int) -> None:
    """[ICS, Checkpoint format]: G is a power of four and divides in_features."""
    log4_group(group_size)
    if k % group_size != 0:
        raise ValueError(f"group size {group_size} does not divide in_features {k}")


def rotate(x: np.ndarray, group_size: int) -> np.ndarray:
    """X R: R_G applied independently to every contiguous group of G features.

    [ICS, How INT8 convrot works]: the block-diagonal rotation acts on each
    contiguous group of G input features of a row; X_rot = X R (row vectors
    times R).  Returns float64 of the same shape.
    """
    x = np.asarray(x, dtype=np.float64)
    m, k = x.shape
    check_group(k, group_size)
    r = rotation_matrix(group_size)
    groups = x.reshape(m * (k // group_size), group_size)  # one group per row
    return (groups @ r).reshape(m, k)


# ---------------------------------------------------------------------------
# 3. Scale and int8 code        [ICS, Weight quantization; Runtime activation q.]
# ---------------------------------------------------------------------------

QMAX = 127


def round_half_away(v: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, ties away from zero, exactly for finite v.

    |v| - floor(|v|) is exact in binary floating point, so the comparison with
    one half is exact (unlike floor(v + 0.5), which misrounds the largest value
    below one half).
    """
    v = np.asarray(v)
    a = np.abs(v)
    t = np.floor(a)
    up = (a - t) >= 0.5
    return np.sign(v) * (t + up)


def quantize_weight_rows(w_rot: np.ndarray):
    """Per-output-row int8 code of already rotated weights, decided in float64.

    [ICS, Weight quantization]:
        s_w[o]    = max_i |W_rot[o, i]| / 127
        Q_w[o, i] = clamp(round(W_rot[o, i] / s_w[o]), -127, 127)
    The scale is stored as float32; the division uses that stored value.
    Returns (Q_w int8 [N, K], s_w float32 [N]).
    """
    w_rot = np.asarray(w_rot, dtype=np.float64)
    m = np.max(np.abs(w_rot), axis=1)
    s = (m / QMAX).astype(np.float32)
    q = np.zeros(w_rot.shape, dtype=np.int8)
    nz = s != 0
    v = w_rot[nz] / s[nz].astype(np.float64)[:, None]
    q[nz] = np.clip(round_half_away(v), -QMAX, QMAX).astype(np.int8)
    return q, s


def quantize_activation_rows(x_rot32: np.ndarray):
    """Per-row dynamic int8 code of rotated activations, decided in float32.

    [ICS, Runtime activation quantization]:
        s_x[r]    = max_i |X_rot[r, i]| / 127
        Q_x[r, i] = clamp(round(X_rot[r, i] / s_x[r]), -127, 127)
    Input: X_rot as float32.  max/127 and X_rot/s_x are correctly rounded
    float32 operations (NumPy float32 arithmetic).
    Returns (Q_x int8 [M, K], s_x float32 [M]).
    """
    x = np.asarray(x_rot32)
    if x.dtype != np.float32:
        raise TypeError("activation codes are decided on float32 X_rot")
    m = np.max(np.abs(x), axis=1)
    s = m / np.float32(QMAX)
    assert s.dtype == np.float32
    q = np.zeros(x.shape, dtype=np.int8)
    nz = s != 0
    v = x[nz] / s[nz][:, None]
    assert v.dtype == np.float32
    q[nz] = np.clip(round_half_away(v), -QMAX, QMAX).astype(np.int8)
    return q, s


def quantize_weights(w: np.ndarray, group_size: int):
    """Offline weight prep: W_rot = W R in float64, then per-row int8.

    [ICS, How INT8 convrot works] (W_rot = W R) and [ICS, Weight quantization].
    Returns (Q_w int8 [N, K], s_w float32 [N]).
    """
    return quantize_weight_rows(rotate(w, group_size))


def pack_activations(x: np.ndarray, group_size: int):
    """The packed runtime activation: int8 rows and their float row scales.

    [ICS, Runtime activation quantization]: rotate every row group-wise, then
    one dynamic scale over the whole rotated row.  The float64 rotation is
    rounded once to float32, the precision the codes are decided in.
    Returns (Q_x int8 [M, K], s_x float32 [M]).
    """
    x_rot32 = rotate(x, group_size).astype(np.float32)
    return quantize_activation_rows(x_rot32)


# ---------------------------------------------------------------------------
# 4. Integer GEMM                     [ICS, Runtime activation quantization]
# ---------------------------------------------------------------------------

# Largest K for which every int32 sum of K products of codes in [-127, 127]
# is representable: K * 127 * 127 <= 2**31 - 1.
MAX_K_INT32 = (2**31 - 1) // (QMAX * QMAX)


def int_gemm(q_x: np.ndarray, q_w: np.ndarray) -> np.ndarray:
    """A[r, o] = sum_i Q_x[r, i] * Q_w[o, i] as exact integers (int64 result).

    Evaluated with float64 BLAS: every product is an integer of magnitude
    <= 16129 and every partial sum is an integer below 2**31 < 2**53, so every
    float64 addition is exact whatever order the library sums in.
    """
    q_x = np.asarray(q_x)
    q_w = np.asarray(q_w)
    if q_x.shape[1] != q_w.shape[1]:
        raise ValueError("K mismatch")
    if q_x.shape[1] > MAX_K_INT32:
        raise ValueError("K too large for an int32 accumulator")
    a = q_x.astype(np.float64) @ q_w.astype(np.float64).T
    return a.astype(np.int64)


def int_gemm_int64(q_x: np.ndarray, q_w: np.ndarray) -> np.ndarray:
    """Same A with int64 arithmetic (slow; for small cross-checks)."""
    return np.asarray(q_x, dtype=np.int64) @ np.asarray(q_w, dtype=np.int64).T


# ---------------------------------------------------------------------------
# 5. Scale restoration and bias       [ICS, Runtime activation quantization]
# ---------------------------------------------------------------------------


def dequantize(a: np.ndarray, s_x: np.ndarray, s_w: np.ndarray, bias=None) -> np.ndarray:
    """Y[r, o] = A[r, o] * s_x[r] * s_w[o] + b[o], in float64.

    ``bias`` may be None (no bias).
    """
    y = np.asarray(a, dtype=np.float64) * np.asarray(s_x, dtype=np.float64)[:, None]
    y = y * np.asarray(s_w, dtype=np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def gelu(x: np.ndarray) -> np.ndarray:
    """x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))), float64 (not on the page)."""
    from scipy.special import erf

    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(q_x, s_x, q_w, s_w, bias=None, act: str | None = None) -> np.ndarray:
    """The convrot linear on a packed activation and quantised weights.

    A = Q_x Q_w^T exactly, then Y = A s_x s_w + b, then optionally GELU.
    """
    y = dequantize(int_gemm(q_x, q_w), s_x, s_w, bias)
    if act == "gelu":
        y = gelu(y)
    elif act is not None:
        raise ValueError(f"unknown activation {act!r}")
    return y


def reference_linear_fp64(x, w, bias=None) -> np.ndarray:
    """Y = X W^T + b with no rotation and no quantisation (float64).

    The layer convrot approximates [ICS, How INT8 convrot works]; used for the
    rotation-invariance check and for informational quality numbers.
    """
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


# ---------------------------------------------------------------------------
# 6. Low-rank adapter correction          [ICS, Backend support]
# ---------------------------------------------------------------------------
# The page applies LoRA-style adapters at run time: the convrot path computes
# the base output, and the adapter computes its correction from the original,
# *unrotated* activation and adds it.  The page gives no formula; the standard
# low-rank form is used: with down weights A [r, K], up weights B [N, r] and a
# scalar scale (alpha / r), the correction is  scale * (X A^T) B^T.
#
# Readings: the device computes in bfloat16
# operands with float32 accumulation, so the oracle takes the same operand
# values -- X (bfloat16 as given, float32 inputs rounded to bfloat16), A and B
# as bfloat16 values.  The rank-r intermediate carries the scale and is
# rounded to bfloat16 (nearest even): U = bf16(scale * X A^T); the
# correction is then U B^T.  All sums are float64.


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), as float64.

    bfloat16 keeps 8 significant bits: with v = f * 2**e, 0.5 <= |f| < 1, the
    result is rint(f * 2**8) * 2**(e - 8) (np.rint rounds half to even).
    Values are assumed finite and in bfloat16's normal range.
    """
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)


def lora_down(x: np.ndarray, a: np.ndarray, scale: float) -> np.ndarray:
    """U = scale * X A^T over the unrotated activation, rounded to bfloat16.

    x: [M, K] (values already bfloat16), a: [r, K] bfloat16 values.
    Returns float64 [M, r] holding bfloat16 values.
    """
    u = np.asarray(x, dtype=np.float64) @ np.asarray(a, dtype=np.float64).T
    return round_bf16(float(scale) * u)


def lora_up(u: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The correction U B^T (float64 [M, N]); b: [N, r]."""
    return np.asarray(u, dtype=np.float64) @ np.asarray(b, dtype=np.float64).T


def lora_correction(x, a, b, scale) -> np.ndarray:
    """bf16(scale * X A^T) B^T (see above)."""
    return lora_up(lora_down(x, a, scale), b)
