"""Seeded synthetic inputs for the convrot linear workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no scale, no quantisation).  The oracle and
the HIP path both receive exactly the arrays made here, so their comparison
starts from the same bits.

Recipe: ``numpy.random.default_rng(seed)``, draws in
the fixed order X -> outlier columns or channel scales -> each W -> each b.

* X ~ N(0, 1) float32, then either a set of outlier columns multiplied by a
  factor (``rng.choice(K, n, replace=False)``) or every column multiplied by a
  LogNormal(0, 1) channel scale.  Where X is bf16 it is converted from the
  float32 draw once, round-to-nearest-even, with torch on the CPU; the float64
  view handed to the oracle is the exact value of those bf16 bits.
* W ~ N(0, 0.02) float32 (0.02 is the standard deviation), b ~ N(0, 0.01).
* Low-rank adapters (``lora_adapter``): A ~ N(0, 1) / sqrt(K) and
  B ~ N(0, 0.02), both rounded to bf16 once; scale = alpha / rank with
  alpha = 16; a base output Y0 ~ N(0, 1) float32 for the in-place update.

Shapes are those of DiT blocks (attention projections, an MLP pair, a long
video-token sequence); real checkpoints and prompts are not used.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LinearSpec:
    name: str
    n: int  # out_features
    k: int  # in_features


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    x_dtype: str  # "bf16" or "f32"
    seed: int
    linears: tuple
    group_sizes: tuple = (256,)
    outlier_cols: int = 0  # number of outlier columns
    outlier_factor: float = 1.0
    channel_lognormal: bool = False
    gelu_chain: bool = False  # MLP: up -> GELU -> down (down input is produced)
    bias: bool = True
    description: str = ""
    extra: dict = field(default_factory=dict)


TINY = Workload(
    name="tiny_16x1024x512",
    m=16, k=1024, x_dtype="f32", seed=1,
    linears=(LinearSpec("proj", 512, 1024),),
    outlier_cols=8, outlier_factor=50.0,
    description="fp32 X [16,1024] with 8 outlier columns x50; W [512,1024]; G=256",
)

GSWEEP = Workload(
    name="gsweep_256x4096x4096",
    m=256, k=4096, x_dtype="bf16", seed=2,
    linears=(LinearSpec("proj", 4096, 4096),),
    group_sizes=(4, 16, 64, 256, 1024),
    outlier_cols=round(0.005 * 4096), outlier_factor=30.0,
    description="bf16 X [256,4096], 0.5% outlier columns x30; W [4096,4096]; "
    "G in {4,16,64,256,1024} on the same X and W",
)

QKV = Workload(
    name="qkv_4096x3072x9216",
    m=4096, k=3072, x_dtype="bf16", seed=3,
    linears=(LinearSpec("q", 3072, 3072), LinearSpec("k", 3072, 3072),
             LinearSpec("v", 3072, 3072)),
    channel_lognormal=True,
    description="bf16 X [4096,3072] with LogNormal(0,1) channel scales; "
    "Q/K/V weights [3072,3072] each on one packed activation (N total 9216); G=256",
)

MLP = Workload(
    name="mlp_4096x3072x12288",
    m=4096, k=3072, x_dtype="bf16", seed=4,
    linears=(LinearSpec("up", 12288, 3072), LinearSpec("down", 3072, 12288)),
    channel_lognormal=True, gelu_chain=True,
    description="bf16 X [4096,3072] (LogNormal channel scales); up [12288,3072], "
    "GELU, down [3072,12288] on the fp32 GELU output; G=256",
)

VIDEO = Workload(
    name="video_32760x5120x13824",
    m=32760, k=5120, x_dtype="bf16", seed=5,
    linears=(LinearSpec("wide", 13824, 5120), LinearSpec("square", 5120, 5120)),
    outlier_cols=round(0.01 * 5120), outlier_factor=50.0,
    description="bf16 X [32760,5120], 1% outlier columns x50; W [13824,5120] and "
    "W [5120,5120] on one packed activation; G=256",
)

WORKLOADS = {w.name: w for w in (TINY, GSWEEP, QKV, MLP, VIDEO)}
ORDER = (TINY, GSWEEP, QKV, MLP, VIDEO)


def _bf16_round(x32: np.ndarray):
    """float32 -> bf16 (round to nearest even) with torch on the CPU.

    Returns (torch bf16 tensor, float64 numpy array of the same values).
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


def generate(w: Workload, m: int | None = None, n_limit: int | None = None,
             seed: int | None = None) -> dict:
    """Draw the inputs of workload ``w``.

    ``m`` overrides the number of rows (smaller parity cases keep the same
    distribution); ``n_limit`` truncates every weight to its first rows.
    Returns a dict with
      x      : torch CPU tensor (bf16 or float32), the bits the device receives
      x64    : float64 numpy array with exactly the same values (oracle input)
      weights: list of float32 numpy arrays [N, K]
      biases : list of float32 numpy arrays [N] (or None when w.bias is False)
    """
    import torch

    rows = w.m if m is None else int(m)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x32 = rng.standard_normal((rows, w.k), dtype=np.float32)
    if w.outlier_cols:
        cols = rng.choice(w.k, w.outlier_cols, replace=False)
        x32[:, cols] *= np.float32(w.outlier_factor)
    if w.channel_lognormal:
        c = rng.lognormal(0.0, 1.0, w.k).astype(np.float32)
        x32 *= c[None, :]
    weights = []
    for spec in w.linears:
        wt = rng.standard_normal((spec.n, spec.k), dtype=np.float32)
        wt *= np.float32(0.02)
        if n_limit is not None:
            wt = np.ascontiguousarray(wt[:n_limit])
        weights.append(wt)
    biases = []
    for spec, wt in zip(w.linears, weights):
        if w.bias:
            b = rng.standard_normal(spec.n, dtype=np.float32) * np.float32(0.01)
            biases.append(np.ascontiguousarray(b[: wt.shape[0]]))
        else:
            biases.append(None)
    if w.x_dtype == "bf16":
        x, x64 = _bf16_round(x32)
    elif w.x_dtype == "f32":
        x = torch.from_numpy(x32)
        x64 = x32.astype(np.float64)
    else:
        raise ValueError(w.x_dtype)
    return {"x": x, "x64": x64, "weights": weights, "biases": biases}


def lora_adapter(k: int, n: int, rank: int, m: int = 0, seed: int = 0, alpha: float = 16.0) -> dict:
    """Draw a rank-``rank`` adapter for a [n, k] linear (and a base output [m, n]).

    Returns a (torch bf16 CPU tensor [rank, k]), a64 (float64, same values),
    b, b64 ([n, rank]), y0 (float32 numpy [m, n]) and scale = alpha / rank.
    """
    rng = np.random.default_rng(seed)
    a32 = rng.standard_normal((rank, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(k))
    b32 = rng.standard_normal((n, rank), dtype=np.float32) * np.float32(0.02)
    y0 = rng.standard_normal((m, n), dtype=np.float32)
    a, a64 = _bf16_round(a32)
    b, b64 = _bf16_round(b32)
    return {"a": a, "a64": a64, "b": b, "b64": b64, "y0": y0, "scale": alpha / rank}


def crafted_rotated_rows(group_size: int, k: int, rows: int, seed: int = 0):
    """Rows y with half-integer entries, |y| <= 127 and a 127 in every row.

    Used by exactness tests: X = y R_G is formed by the caller (the oracle side
    computes R_G); each entry of y is a multiple of 1/2, so every butterfly
    intermediate of the rotation is a short dyadic number, exact in float32.
    Returns a float64 array [rows, k].
    """
    rng = np.random.default_rng(seed)
    y = rng.integers(-254, 255, size=(rows, k)).astype(np.float64) / 2.0
    pos = rng.integers(0, k, size=rows)
    sign = np.where(rng.integers(0, 2, size=rows) == 0, -1.0, 1.0)
    y[np.arange(rows), pos] = 127.0 * sign
    return y
