"""The hot path captured in a HIP graph (GPU).

Every entry point launches asynchronously on the caller's stream, allocates
nothing and clears memory with kernels, never with a memset, so a caller
may capture a whole layer step in a graph: the activation pack, grouped
linears on the persistent GEMM (plain and with the GELU epilogue), linears
with adapters (down projection and the fused up projection) and a
short-output linear on the split-K kernel.

Each replay runs on new input values copied into the captured input
buffers, with eager launches and synchronisations between replays, and its
outputs must equal those of the same calls made eagerly on the same values,
bit for bit (the same kernels on the same data).  The first replay's
split-K output is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import hadamard_rotated_int8_amd as cr
import workloads as wl
from oracle import convrot_oracle as orc

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _inputs():
    """Two activations (long rows for the persistent GEMM, a short block
    for the split-K path), their weights and two adapters."""
    rng = np.random.default_rng(77)
    xa = wl.generate(wl.QKV, m=2048, n_limit=1)["x"][:, :1024].contiguous().cuda()
    xb = torch.from_numpy((rng.standard_normal((200, 4000)) *
                           np.exp(rng.standard_normal(4000))).astype(np.float32))
    xb = xb.to(torch.bfloat16).cuda()
    ns = (3072, 3072, 3072)
    wa = [cr.quantize_weights(torch.from_numpy((rng.standard_normal((n, 1024)) * 0.02)
                                               .astype(np.float32)).cuda(), 256,
                              torch.from_numpy((rng.standard_normal(n) * 0.01)
                                               .astype(np.float32)).cuda())
          for n in ns]
    wb_host = (rng.standard_normal((1040, 4000)) * 0.02).astype(np.float32)
    wb = cr.quantize_weights(torch.from_numpy(wb_host).cuda(), 16)
    ads = [wl.lora_adapter(1024, n, r, seed=5 + i) for i, (n, r) in enumerate(zip(ns[:2], (32, 64)))]
    ads = [(ad["a"].cuda(), ad["b"].cuda(), ad["scale"]) for ad in ads]
    return xa, xb, wa, wb, wb_host, ads


def _step(xa, xb, wa, wb, ads):
    pa = cr.pack_activations(xa, 256)
    plain = cr.linear_grouped(pa, wa)
    plain_gelu = cr.linear_grouped(pa, wa[:2], gelu=True)  # GELU at store time, no adapters
    us = [cr.lora_down(xa, a, scale) for a, _, scale in ads]
    fused = cr.linear_lora(pa, wa, [(u, b) for u, (_, b, _) in zip(us, ads)] + [None], gelu=True)
    pb = cr.pack_activations(xb, 16)
    short = cr.linear(pb, wb)
    short_gelu = cr.linear(pb, wb, gelu=True)
    return [pa.q, pa.scale, *plain, *plain_gelu, *us, *fused, pb.q, pb.scale, short, short_gelu]


def _variant(x0, i):
    """Input values of replay i: rows rolled and rescaled."""
    return (torch.roll(x0.float(), shifts=37 * i, dims=0) * (1.0 + 0.25 * i)).to(x0.dtype)


def test_hot_path_replays_in_a_graph():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    torch.cuda.set_device(0)
    xa0, xb0, wa, wb, wb_host, ads = _inputs()
    xa, xb = xa0.clone(), xb0.clone()

    # warm up (first-call device queries) off the capture, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(xa, xb, wa, wb, ads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    _say("capture: pack, grouped linears, adapters, split-K")
    with torch.cuda.graph(graph):
        captured = _step(xa, xb, wa, wb, ads)
    torch.cuda.synchronize()

    for i in range(1, REPLAYS + 1):
        va, vb = _variant(xa0, i), _variant(xb0, i)
        xa.copy_(va)
        xb.copy_(vb)
        _say(f"replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        eager = _step(va, vb, wa, wb, ads)  # eager work between replays
        torch.cuda.synchronize()
        for j, (c, e) in enumerate(zip(captured, eager)):
            assert torch.equal(c, e), f"replay {i}: output {j} differs from the eager call"
        if i == 1:
            # the split-K output against the oracle (same bounds as the parity tests)
            x64 = vb.float().cpu().numpy().astype(np.float64)
            qx, sx = orc.pack_activations(x64, 16)
            qw, sw = orc.quantize_weights(wb_host, 16)
            y_or = orc.linear(qx, sx, qw, sw, None)
            y = captured[-2].cpu().numpy().astype(np.float64)
            bound = 1e-3 * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * 4000 * 127
            assert np.all(np.abs(y - y_or) <= bound)
            assert np.abs(y - y_or).sum() / np.abs(y_or).sum() <= 1e-4
