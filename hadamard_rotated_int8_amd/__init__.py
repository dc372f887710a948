"""Python binding of libconvrot.so, the INT8 convrot linear layer for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libconvrot.so.  The functions named ``convrot_*`` mirror the C ABI
in include/convrot.h one to one (raw device pointers and sizes); the
torch-level helpers below them only allocate outputs with torch and pass
pointers plus torch's current HIP stream.

torch is imported before the library is loaded so that the process holds a
single HIP runtime (torch's), which the library then binds to.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # noqa: F401  (must precede loading the library; see above)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libconvrot.so")

# Status codes and enums (include/convrot.h).
OK = 0
ERR_NULL = 1
ERR_SHAPE = 2
ERR_GROUP = 3
ERR_GROUP_MISMATCH = 4
ERR_DTYPE = 5
ERR_UNSUPPORTED = 6
ERR_HIP = 7
F32 = 0
BF16 = 1
I32 = 2
ACT_NONE = 0
ACT_GELU = 1
MAX_K = 133136
MAX_LOG4_GROUP = 7
MAX_GROUPED = 8
MAX_LORA_RANK = 256

EXPORTED = (
    "convrot_quantize_weights",
    "convrot_pack_activations",
    "convrot_linear",
    "convrot_linear_grouped",
    "convrot_lora_down",
    "convrot_lora_up_add",
    "convrot_linear_lora",
    "convrot_status_string",
    "convrot_version",
)


class ConvrotError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class ConvrotPacked(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("m", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("group_size", ctypes.c_int32),
    ]


class ConvrotWeights(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("group_size", ctypes.c_int32),
    ]


class ConvrotLora(ctypes.Structure):
    _fields_ = [
        ("u", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("ldu", ctypes.c_int64),
        ("rank", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libconvrot.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m hadamard_rotated_int8_amd.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.convrot_quantize_weights.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp]
        L.convrot_quantize_weights.restype = ctypes.c_int
        L.convrot_pack_activations.argtypes = [vp, i32, i64, i64, i64, i32,
                                               ctypes.POINTER(ConvrotPacked), vp]
        L.convrot_pack_activations.restype = ctypes.c_int
        L.convrot_linear.argtypes = [ctypes.POINTER(ConvrotPacked), ctypes.POINTER(ConvrotWeights),
                                     vp, i32, i64, i32, vp]
        L.convrot_linear.restype = ctypes.c_int
        L.convrot_linear_grouped.argtypes = [ctypes.POINTER(ConvrotPacked),
                                             ctypes.POINTER(ConvrotWeights), i32,
                                             ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32, vp]
        L.convrot_linear_grouped.restype = ctypes.c_int
        L.convrot_lora_down.argtypes = [vp, i32, i64, i64, i64, vp, i32, ctypes.c_float, vp, i64,
                                        vp]
        L.convrot_lora_down.restype = ctypes.c_int
        L.convrot_lora_up_add.argtypes = [vp, i64, vp, i64, i64, i32, vp, i64, vp]
        L.convrot_lora_up_add.restype = ctypes.c_int
        L.convrot_linear_lora.argtypes = [ctypes.POINTER(ConvrotPacked),
                                          ctypes.POINTER(ConvrotWeights),
                                          ctypes.POINTER(ConvrotLora), i32, ctypes.POINTER(vp),
                                          ctypes.POINTER(i64), i32, vp]
        L.convrot_linear_lora.restype = ctypes.c_int
        L.convrot_status_string.argtypes = [ctypes.c_int]
        L.convrot_status_string.restype = ctypes.c_char_p
        L.convrot_version.argtypes = []
        L.convrot_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().convrot_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# Raw C ABI (device pointers as ints, stream as an int handle or None)
# ---------------------------------------------------------------------------

def convrot_quantize_weights(w, n, k, ldw, group_size, q_out, scale_out, stream=None) -> int:
    return lib().convrot_quantize_weights(w, n, k, ldw, group_size, q_out, scale_out, stream)


def convrot_pack_activations(x, x_dtype, m, k, ldx, group_size, out: ConvrotPacked,
                             stream=None) -> int:
    return lib().convrot_pack_activations(x, x_dtype, m, k, ldx, group_size, ctypes.byref(out),
                                          stream)


def convrot_linear(x: ConvrotPacked, w: ConvrotWeights, y, y_dtype, ldy, act=ACT_NONE,
                   stream=None) -> int:
    return lib().convrot_linear(ctypes.byref(x), ctypes.byref(w), y, y_dtype, ldy, act, stream)


def convrot_linear_grouped(x: ConvrotPacked, ws, ys, ldys, y_dtype, act=ACT_NONE,
                           stream=None) -> int:
    """ws: sequence of ConvrotWeights; ys: device pointers; ldys: row strides."""
    n = len(ws)
    warr = (ConvrotWeights * max(n, 1))(*ws)
    yarr = (ctypes.c_void_p * max(n, 1))(*ys)
    larr = (ctypes.c_int64 * max(n, 1))(*ldys)
    return lib().convrot_linear_grouped(ctypes.byref(x), warr, n, yarr, larr, y_dtype, act,
                                        stream)


def convrot_lora_down(x, x_dtype, m, k, ldx, a, rank, scale, u, ldu, stream=None) -> int:
    return lib().convrot_lora_down(x, x_dtype, m, k, ldx, a, rank, scale, u, ldu, stream)


def convrot_lora_up_add(u, ldu, b, m, n, rank, y, ldy, stream=None) -> int:
    return lib().convrot_lora_up_add(u, ldu, b, m, n, rank, y, ldy, stream)


def convrot_linear_lora(x: ConvrotPacked, ws, loras, ys, ldys, act=ACT_NONE, stream=None) -> int:
    """ws: ConvrotWeights; loras: ConvrotLora (rank 0 = none); ys, ldys as for grouped."""
    n = len(ws)
    warr = (ConvrotWeights * max(n, 1))(*ws)
    larr_ = (ConvrotLora * max(n, 1))(*loras)
    yarr = (ctypes.c_void_p * max(n, 1))(*ys)
    ldarr = (ctypes.c_int64 * max(n, 1))(*ldys)
    return lib().convrot_linear_lora(ctypes.byref(x), warr, larr_, n, yarr, ldarr, act, stream)


def convrot_version() -> int:
    return int(lib().convrot_version())


# ---------------------------------------------------------------------------
# torch helpers: allocate outputs, pass pointers and the current stream
# ---------------------------------------------------------------------------

def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require_cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


@dataclass
class PackedActivation:
    """int8 rows and float32 row scales of one rotated activation."""

    q: torch.Tensor       # int8 [m, k]
    scale: torch.Tensor   # float32 [m]
    group_size: int

    def as_c(self) -> ConvrotPacked:
        m, k = self.q.shape
        return ConvrotPacked(_ptr(self.q), _ptr(self.scale), m, k, self.group_size)


@dataclass
class QuantizedWeights:
    """int8 [n, k] codes, float32 [n] scales and optional float32 [n] bias."""

    q: torch.Tensor
    scale: torch.Tensor
    bias: torch.Tensor | None
    group_size: int

    def as_c(self) -> ConvrotWeights:
        n, k = self.q.shape
        return ConvrotWeights(_ptr(self.q), _ptr(self.scale), _ptr(self.bias), n, k,
                              self.group_size)


# The C ABI sees only pointers and sizes, so the extents, dtypes, layouts and
# device of every tensor are checked here: a wrong one would otherwise make a
# kernel read or write outside it.
def _same_device(dev, *ts):
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError("all tensors of one call must be on the same device")


def _check_packed(x: PackedActivation) -> torch.device:
    q, s = x.q, x.scale
    _require_cuda(q, "the packed codes")
    if q.dtype != torch.int8 or q.dim() != 2 or not q.is_contiguous():
        raise ValueError("the packed codes must be a contiguous int8 [m, k] device tensor")
    if s.dtype != torch.float32 or tuple(s.shape) != (q.shape[0],) or not s.is_contiguous():
        raise ValueError("the packed scales must be a contiguous float32 [m] tensor")
    _same_device(q.device, s)
    return q.device


def _check_weights(w: "QuantizedWeights", dev):
    q = w.q
    if q.dtype != torch.int8 or q.dim() != 2 or not q.is_contiguous():
        raise ValueError("weight codes must be a contiguous int8 [n, k] tensor")
    n = q.shape[0]
    for t, what in ((w.scale, "weight scales"), (w.bias, "bias")):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (n,)
                              or not t.is_contiguous()):
            raise ValueError(f"the {what} must be a contiguous float32 [n] tensor")
    _same_device(dev, q, w.scale, w.bias)


def _check_out(o: torch.Tensor, m: int, n: int, dtype, dev):
    if o.dtype != dtype or tuple(o.shape) != (m, n) or o.stride(1) != 1:
        raise ValueError(f"an output must be a {dtype} [{m}, {n}] view with unit column stride")
    _same_device(dev, o)


def quantize_weights(w: torch.Tensor, group_size: int, bias: torch.Tensor | None = None
                     ) -> QuantizedWeights:
    """Offline W_rot = W R and per-row int8 codes (float32 W [n, k] on the device)."""
    _require_cuda(w, "w")
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a float32 [n, k] device tensor with unit column stride")
    n, k = w.shape
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (n,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [n] tensor")
    _same_device(w.device, bias)
    q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    s = torch.empty((n,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        st = convrot_quantize_weights(_ptr(w), n, k, w.stride(0), group_size, _ptr(q), _ptr(s),
                                      _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_quantize_weights")
    return QuantizedWeights(q, s, bias, group_size)


def pack_activations(x: torch.Tensor, group_size: int, out: PackedActivation | None = None
                     ) -> PackedActivation:
    """Rotate and quantise the rows of x (bf16 or float32 [m, k] on the device)."""
    _require_cuda(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [m, k] with unit column stride")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    m, k = x.shape
    if out is None:
        out = PackedActivation(torch.empty((m, k), dtype=torch.int8, device=x.device),
                               torch.empty((m,), dtype=torch.float32, device=x.device),
                               group_size)
    if tuple(out.q.shape) != (m, k) or _check_packed(out) != x.device:
        raise ValueError("out must hold [m, k] codes and [m] scales on x's device")
    c = ConvrotPacked(_ptr(out.q), _ptr(out.scale), 0, 0, 0)
    with torch.cuda.device(x.device):
        st = convrot_pack_activations(_ptr(x), dt, m, k, x.stride(0), group_size, c, _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_pack_activations")
    out.group_size = group_size
    return out


def linear(x: PackedActivation, w: QuantizedWeights, out: torch.Tensor | None = None,
           raw_i32: bool = False, gelu: bool = False) -> torch.Tensor:
    """Y = (Q_x Q_w^T) s_x s_w + b (float32 [m, n]); raw_i32 returns the int32 A."""
    dev = _check_packed(x)
    _check_weights(w, dev)
    m = x.q.shape[0]
    n = w.q.shape[0]
    dtype = torch.int32 if raw_i32 else torch.float32
    if out is None:
        out = torch.empty((m, n), dtype=dtype, device=dev)
    _check_out(out, m, n, dtype, dev)
    with torch.cuda.device(dev):
        st = convrot_linear(x.as_c(), w.as_c(), _ptr(out), I32 if raw_i32 else F32,
                            out.stride(0), ACT_GELU if gelu else ACT_NONE, _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_linear")
    return out


def linear_grouped(x: PackedActivation, ws, outs=None, raw_i32: bool = False,
                   gelu: bool = False):
    """Several linears on one packed activation in one launch; returns the outputs."""
    dev = _check_packed(x)
    for w in ws:
        _check_weights(w, dev)
    m = x.q.shape[0]
    dtype = torch.int32 if raw_i32 else torch.float32
    if outs is None:
        outs = [torch.empty((m, w.q.shape[0]), dtype=dtype, device=dev) for w in ws]
    if len(outs) != len(ws):
        raise ValueError("one output per weight")
    for o, w in zip(outs, ws):
        _check_out(o, m, w.q.shape[0], dtype, dev)
    with torch.cuda.device(dev):
        st = convrot_linear_grouped(x.as_c(), [w.as_c() for w in ws], [_ptr(o) for o in outs],
                                    [o.stride(0) for o in outs], I32 if raw_i32 else F32,
                                    ACT_GELU if gelu else ACT_NONE, _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_linear_grouped")
    return outs


def lora_down(x: torch.Tensor, a: torch.Tensor, scale: float,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """U = bf16(scale X A^T) for a low-rank adapter, on the unrotated X.

    ``out`` may be a column slice of a wider bfloat16 buffer (unit column
    stride, row stride a multiple of 8); by default a new [m, rank] tensor.
    """
    _require_cuda(x, "x")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a float32 or bfloat16 [m, k] tensor with unit column stride")
    if a.dtype != torch.bfloat16 or a.dim() != 2 or not a.is_contiguous():
        raise ValueError("a must be a contiguous bfloat16 [rank, k] tensor")
    m, k = x.shape
    rank = a.shape[0]
    if a.shape[1] != k:
        raise ValueError("a must have k columns")
    if out is None:
        out = torch.empty((m, rank), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or out.shape != (m, rank) or out.stride(1) != 1:
        raise ValueError("out must be a bfloat16 [m, rank] view with unit column stride")
    _same_device(x.device, a, out)
    with torch.cuda.device(x.device):
        st = convrot_lora_down(_ptr(x), dt, m, k, x.stride(0), _ptr(a), rank, float(scale),
                               _ptr(out), out.stride(0), _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_lora_down")
    return out


def _check_u(u: torch.Tensor, m: int):
    if u.dtype != torch.bfloat16 or u.dim() != 2 or u.stride(1) != 1 or u.shape[0] != m:
        raise ValueError("u must be a bfloat16 [m, rank] tensor with unit column stride")


def lora_up_add(u: torch.Tensor, b: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """y += U B^T in place (y float32 [m, n]), a separate pass; returns y."""
    _require_cuda(y, "y")
    if y.dtype != torch.float32 or y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be a float32 [m, n] tensor with unit column stride")
    m, n = y.shape
    _check_u(u, m)
    rank = u.shape[1]
    if b.dtype != torch.bfloat16 or not b.is_contiguous() or b.shape != (n, rank):
        raise ValueError("b must be a contiguous bfloat16 [n, rank] tensor")
    _same_device(y.device, u, b)
    with torch.cuda.device(y.device):
        st = convrot_lora_up_add(_ptr(u), u.stride(0), _ptr(b), m, n, rank, _ptr(y), y.stride(0),
                                 _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_lora_up_add")
    return y


def linear_lora(x: PackedActivation, ws, adapters, outs=None, gelu: bool = False):
    """Grouped linears with each weight's adapter added in the epilogue.

    adapters: one (u, b) pair per weight -- u from ``lora_down`` (bfloat16
    [m, rank]), b bfloat16 [n, rank] -- or None for a weight without one.
    Returns the float32 outputs act(Y + U B^T).
    """
    dev = _check_packed(x)
    for w in ws:
        _check_weights(w, dev)
    m = x.q.shape[0]
    if len(adapters) != len(ws):
        raise ValueError("one adapter (or None) per weight")
    if outs is None:
        outs = [torch.empty((m, w.q.shape[0]), dtype=torch.float32, device=dev) for w in ws]
    if len(outs) != len(ws):
        raise ValueError("one output per weight")
    loras = []
    for w, ad in zip(ws, adapters):
        if ad is None:
            loras.append(ConvrotLora(None, None, 0, 0))
            continue
        u, b = ad
        _check_u(u, m)
        rank = u.shape[1]
        if b.dtype != torch.bfloat16 or not b.is_contiguous() or b.shape != (w.q.shape[0], rank):
            raise ValueError("b must be a contiguous bfloat16 [n, rank] tensor")
        _same_device(dev, u, b)
        loras.append(ConvrotLora(_ptr(u), _ptr(b), u.stride(0), rank))
    for o, w in zip(outs, ws):
        _check_out(o, m, w.q.shape[0], torch.float32, dev)
    with torch.cuda.device(dev):
        st = convrot_linear_lora(x.as_c(), [w.as_c() for w in ws], loras, [_ptr(o) for o in outs],
                                 [o.stride(0) for o in outs], ACT_GELU if gelu else ACT_NONE,
                                 _stream())
    if st != OK:
        raise ConvrotError(st, "convrot_linear_lora")
    return outs
