"""C-ABI boundary tests that need no GPU.

libconvrot.so validates every argument on the host before any HIP call, so
each invalid call below returns its status code without touching a device.
Every call here fails validation; none of them launches a kernel.
"""

import ctypes
import os
import re

import pytest

import hadamard_rotated_int8_amd as cr

# Every call here passes FAKE device addresses and relies on validation
# failing first; on a host with a visible GPU a mistake in a test would launch
# a kernel on them, so these tests run only where no GPU is visible.
pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="passes fake device pointers; host-validation tests run on GPU-less hosts only")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

FAKE = 0x10000  # a 16-byte aligned non-null address; only used where validation fails first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(cr.EXPORTED)
    L = cr.lib()
    for name in names:
        assert hasattr(L, name), name


def test_ceiling_library_exports_its_declared_functions():
    """libconvrot_ceiling.so (the benchmark's measurement kernels) exports what
    include/convrot_ceiling.h declares, and refuses bad arguments on the host."""
    text = open(os.path.join(ROOT, "include", "convrot_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", text)))
    assert names == ["convrot_ceiling_mfma_i8", "convrot_ceiling_stream"]
    L = ctypes.CDLL(os.path.join(ROOT, "hadamard_rotated_int8_amd", "libconvrot_ceiling.so"))
    s = L.convrot_ceiling_stream
    s.restype = ctypes.c_int32
    s.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p]
    assert s(None, FAKE, 1024, 2, 1, None) == -1      # null source
    assert s(FAKE, FAKE, 1000, 2, 1, None) == -1      # not a multiple of 16 bytes
    assert s(FAKE, FAKE, 0, 2, 1, None) == -1         # nothing to move
    assert s(FAKE, FAKE, 1024, 3, 1, None) == -1      # ratio not 1, 2 or 4
    assert s(FAKE, FAKE, 1024, 2, 0, None) == -1      # no workgroups
    assert s(FAKE + 8, FAKE, 1024, 2, 1, None) == -1  # misaligned
    f = L.convrot_ceiling_mfma_i8
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 128, 32, FAKE, 128, 32, 1, 1, FAKE, None) == -1      # null operand
    assert f(FAKE, 120, 32, FAKE, 128, 32, 1, 1, FAKE, None) == -1      # row stride < 128
    assert f(FAKE, 128, 31, FAKE, 128, 32, 1, 1, FAKE, None) == -1      # fewer than 32 rows
    assert f(FAKE, 128, 32, FAKE, 128, 32, 0, 1, FAKE, None) == -1      # no iterations
    assert f(FAKE + 8, 128, 32, FAKE, 128, 32, 1, 1, FAKE, None) == -1  # misaligned


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define CONVROT_MAX_K (\d+)", text).group(1)) == cr.MAX_K
    assert cr.MAX_K % 16 == 0 and cr.MAX_K * 127 * 127 < 2**31
    assert (cr.MAX_K + 16) * 127 * 127 >= 2**31
    for name, val in [("CONVROT_OK", 0), ("CONVROT_ERR_NULL", 1), ("CONVROT_ERR_SHAPE", 2),
                      ("CONVROT_ERR_GROUP", 3), ("CONVROT_ERR_GROUP_MISMATCH", 4),
                      ("CONVROT_ERR_DTYPE", 5), ("CONVROT_ERR_UNSUPPORTED", 6),
                      ("CONVROT_ERR_HIP", 7)]:
        assert re.search(rf"{name} = {val}\b", text), name


def test_version_and_status_strings():
    assert cr.convrot_version() == 100
    for s in range(8):
        assert cr.status_string(s)
    assert cr.status_string(99) == "unknown status"


def _pack(x=FAKE, dt=cr.BF16, m=4, k=1024, ldx=None, g=256, q=FAKE, s=FAKE, out=True):
    p = cr.ConvrotPacked(q, s, 0, 0, 0)
    if not out:
        return cr.lib().convrot_pack_activations(x, dt, m, k, k if ldx is None else ldx, g,
                                                 None, None)
    return cr.convrot_pack_activations(x, dt, m, k, k if ldx is None else ldx, g, p), p


@pytest.mark.parametrize("g", [0, -4, 2, 3, 8, 32, 128, 255, 512, 4**8, 2**31 - 1])
def test_pack_rejects_bad_group(g):
    st, _ = _pack(g=g, k=4**8 * 2)
    assert st == cr.ERR_GROUP


def test_pack_rejects_group_not_dividing_k():
    st, _ = _pack(g=256, k=1024 + 64)
    assert st == cr.ERR_GROUP
    st, _ = _pack(g=16384, k=8192)  # G > K
    assert st == cr.ERR_GROUP


def test_pack_shape_errors():
    assert _pack(k=0, g=1)[0] == cr.ERR_SHAPE
    assert _pack(k=cr.MAX_K + 16, g=16)[0] == cr.ERR_SHAPE
    assert _pack(m=-1)[0] == cr.ERR_SHAPE
    assert _pack(m=2**31)[0] == cr.ERR_SHAPE
    assert _pack(ldx=1000)[0] == cr.ERR_SHAPE


def test_pack_unsupported_and_dtype():
    assert _pack(k=20, g=4)[0] == cr.ERR_UNSUPPORTED          # k % 16 != 0 (a valid G)
    assert _pack(x=FAKE + 8)[0] == cr.ERR_UNSUPPORTED          # misaligned input
    assert _pack(q=FAKE + 4)[0] == cr.ERR_UNSUPPORTED          # misaligned codes
    assert _pack(ldx=1028, dt=cr.BF16)[0] == cr.ERR_UNSUPPORTED  # row stride not 16 bytes
    assert _pack(dt=cr.I32)[0] == cr.ERR_DTYPE
    assert _pack(dt=7)[0] == cr.ERR_DTYPE


def test_pack_null_pointers():
    assert _pack(out=False) == cr.ERR_NULL
    assert _pack(x=None)[0] == cr.ERR_NULL
    assert _pack(q=None)[0] == cr.ERR_NULL
    assert _pack(s=None)[0] == cr.ERR_NULL


def test_pack_empty_is_a_no_op():
    st, p = _pack(x=None, q=None, s=None, m=0, k=3072, g=256)
    assert st == cr.OK
    assert (p.m, p.k, p.group_size) == (0, 3072, 256)


def _lin(m=16, k=1024, gx=256, n=512, kw=None, gw=None, y=FAKE, ydt=cr.F32, ldy=None,
         act=cr.ACT_NONE, qx=FAKE, sx=FAKE, qw=FAKE, sw=FAKE, bias=None):
    px = cr.ConvrotPacked(qx, sx, m, k, gx)
    w = cr.ConvrotWeights(qw, sw, bias, n, k if kw is None else kw, gx if gw is None else gw)
    return cr.convrot_linear(px, w, y, ydt, n if ldy is None else ldy, act)


def test_linear_group_mismatch():
    assert _lin(gw=64) == cr.ERR_GROUP_MISMATCH
    assert _lin(kw=2048) == cr.ERR_GROUP_MISMATCH


def test_linear_validation():
    assert cr.lib().convrot_linear(None, None, None, 0, 0, 0, None) == cr.ERR_NULL
    assert _lin(gx=255) == cr.ERR_GROUP
    assert _lin(m=-1) == cr.ERR_SHAPE
    assert _lin(n=-5) == cr.ERR_SHAPE
    assert _lin(ldy=100) == cr.ERR_SHAPE
    assert _lin(ydt=cr.BF16) == cr.ERR_DTYPE
    assert _lin(act=5) == cr.ERR_DTYPE
    assert _lin(ydt=cr.I32, act=cr.ACT_GELU) == cr.ERR_DTYPE
    assert _lin(y=None) == cr.ERR_NULL
    assert _lin(qx=None) == cr.ERR_NULL
    assert _lin(sw=None) == cr.ERR_NULL
    assert _lin(y=FAKE + 2) == cr.ERR_UNSUPPORTED  # y needs 4-byte alignment only
    assert _lin(qw=FAKE + 1) == cr.ERR_UNSUPPORTED
    assert _lin(qx=FAKE + 8) == cr.ERR_UNSUPPORTED
    assert _lin(k=1040, gx=16, kw=1040, gw=16, qx=None) == cr.ERR_NULL  # ragged K is accepted
    # each extent fits, but the number of 256 x 192 output tiles would not fit 32 bits
    big = 2**31 - 1
    assert _lin(m=big, n=big, ldy=big) == cr.ERR_SHAPE


def test_linear_empty_is_a_no_op():
    assert _lin(m=0, y=None, qx=None) == cr.OK
    assert _lin(n=0, y=None, qw=None, ldy=0) == cr.OK


def _qw(w=FAKE, n=512, k=1024, ldw=None, g=256, q=FAKE, s=FAKE):
    return cr.convrot_quantize_weights(w, n, k, k if ldw is None else ldw, g, q, s)


def test_quantize_weights_validation():
    assert _qw(g=8) == cr.ERR_GROUP
    assert _qw(k=1024 + 64) == cr.ERR_GROUP
    assert _qw(k=0, g=1) == cr.ERR_SHAPE
    assert _qw(n=-1) == cr.ERR_SHAPE
    assert _qw(ldw=512) == cr.ERR_SHAPE
    assert _qw(w=None) == cr.ERR_NULL
    assert _qw(q=None) == cr.ERR_NULL
    assert _qw(s=None) == cr.ERR_NULL
    assert _qw(q=FAKE + 2) == cr.ERR_UNSUPPORTED
    assert _qw(n=0, w=None, q=None, s=None) == cr.OK


def test_struct_layouts_match_c():
    # int8_t* q; float* scale; int64 m; int64 k; int32 group_size  -> 36 bytes + padding
    assert ctypes.sizeof(cr.ConvrotPacked) == 40
    assert cr.ConvrotPacked.m.offset == 16 and cr.ConvrotPacked.group_size.offset == 32
    assert ctypes.sizeof(cr.ConvrotWeights) == 48
    assert cr.ConvrotWeights.n.offset == 24 and cr.ConvrotWeights.group_size.offset == 40


def _grp(count=3, ws=None, ys=None, ldys=None, ydt=cr.F32, act=cr.ACT_NONE, gx=256, k=1024):
    px = cr.ConvrotPacked(FAKE, FAKE, 16, k, gx)
    if ws is None:
        ws = [cr.ConvrotWeights(FAKE, FAKE, None, 512, k, gx) for _ in range(count)]
    ys = [FAKE] * len(ws) if ys is None else ys
    ldys = [w.n for w in ws] if ldys is None else ldys
    return cr.convrot_linear_grouped(px, ws, ys, ldys, ydt, act)


def test_linear_grouped_validation():
    L = cr.lib()
    assert L.convrot_linear_grouped(None, None, 1, None, None, 0, 0, None) == cr.ERR_NULL
    assert _grp(ws=[]) == cr.ERR_SHAPE                          # count 0
    assert _grp(count=cr.MAX_GROUPED + 1) == cr.ERR_SHAPE
    bad_g = [cr.ConvrotWeights(FAKE, FAKE, None, 512, 1024, 256),
             cr.ConvrotWeights(FAKE, FAKE, None, 512, 1024, 64)]
    assert _grp(ws=bad_g) == cr.ERR_GROUP_MISMATCH              # second weight's G differs
    bad_k = [cr.ConvrotWeights(FAKE, FAKE, None, 512, 1024, 256),
             cr.ConvrotWeights(FAKE, FAKE, None, 512, 2048, 256)]
    assert _grp(ws=bad_k) == cr.ERR_GROUP_MISMATCH
    assert _grp(ldys=[512, 100, 512]) == cr.ERR_SHAPE
    assert _grp(ys=[FAKE, None, FAKE]) == cr.ERR_NULL
    assert _grp(ys=[FAKE, FAKE, FAKE + 2]) == cr.ERR_UNSUPPORTED
    assert _grp(ydt=cr.BF16) == cr.ERR_DTYPE
    assert _grp(ydt=cr.I32, act=cr.ACT_GELU) == cr.ERR_DTYPE
    empty = [cr.ConvrotWeights(None, None, None, 0, 1024, 256) for _ in range(2)]
    assert _grp(ws=empty, ys=[None, None], ldys=[0, 0]) == cr.OK   # nothing to launch


def _down(x=FAKE, dt=cr.BF16, m=64, k=1024, ldx=None, a=FAKE, r=32, u=FAKE, ldu=None):
    return cr.convrot_lora_down(x, dt, m, k, k if ldx is None else ldx, a, r, 0.5, u,
                                r if ldu is None else ldu)


def _up(u=FAKE, b=FAKE, m=64, n=512, r=32, y=FAKE, ldy=None, ldu=None):
    return cr.convrot_lora_up_add(u, r if ldu is None else ldu, b, m, n, r, y,
                                  n if ldy is None else ldy)


def test_lora_rank_limits_match_header():
    text = open(HEADER).read()
    assert int(re.search(r"#define CONVROT_MAX_LORA_RANK (\d+)", text).group(1)) == cr.MAX_LORA_RANK


@pytest.mark.parametrize("r", [0, 8, 15, 24, 136, 264, 272, -16])
def test_lora_rejects_bad_rank(r):
    assert _down(r=r, ldu=max(r, 8)) == cr.ERR_SHAPE
    assert _up(r=r, ldu=max(r, 8)) == cr.ERR_SHAPE


def test_lora_down_validation():
    assert _down(k=0) == cr.ERR_SHAPE
    assert _down(m=-1) == cr.ERR_SHAPE
    assert _down(ldx=512) == cr.ERR_SHAPE           # ldx < k
    assert _down(ldx=(1 << 21) + 8) == cr.ERR_SHAPE
    assert _down(ldu=16) == cr.ERR_SHAPE            # ldu < rank
    assert _down(ldu=(1 << 20) + 8) == cr.ERR_SHAPE
    assert _down(dt=2) == cr.ERR_DTYPE
    assert _down(k=1000) == cr.ERR_UNSUPPORTED       # k % 16
    assert _down(ldu=36) == cr.ERR_UNSUPPORTED       # U rows not whole 16-byte units
    assert _down(x=None) == cr.ERR_NULL
    assert _down(a=None) == cr.ERR_NULL
    assert _down(u=None) == cr.ERR_NULL
    assert _down(x=FAKE + 8) == cr.ERR_UNSUPPORTED   # misaligned
    assert _down(u=FAKE + 2) == cr.ERR_UNSUPPORTED
    assert _down(ldx=1028) == cr.ERR_UNSUPPORTED     # bf16 row stride not a 16-byte multiple
    assert _down(m=0, x=None, a=None, u=None) == cr.OK  # empty: no work, no pointers needed


def test_lora_up_add_validation():
    assert _up(n=-1) == cr.ERR_SHAPE
    assert _up(ldy=100) == cr.ERR_SHAPE              # ldy < n
    assert _up(ldu=16) == cr.ERR_SHAPE
    assert _up(ldu=36) == cr.ERR_UNSUPPORTED
    assert _up(u=None) == cr.ERR_NULL
    assert _up(b=None) == cr.ERR_NULL
    assert _up(y=None) == cr.ERR_NULL
    assert _up(u=FAKE + 4) == cr.ERR_UNSUPPORTED
    assert _up(b=FAKE + 2) == cr.ERR_UNSUPPORTED
    assert _up(y=FAKE + 2) == cr.ERR_UNSUPPORTED
    assert _up(m=0, u=None, b=None, y=None) == cr.OK
    assert _up(n=0, u=None, b=None, y=None) == cr.OK


def test_lora_struct_layout_matches_c():
    # const void* u; const void* b; int64 ldu; int32 rank -> 28 bytes + padding
    assert ctypes.sizeof(cr.ConvrotLora) == 32
    assert cr.ConvrotLora.ldu.offset == 16 and cr.ConvrotLora.rank.offset == 24


def _fused(loras=None, count=3, ws=None, act=cr.ACT_NONE, m=16, k=1024):
    px = cr.ConvrotPacked(FAKE, FAKE, m, k, 256)
    if ws is None:
        ws = [cr.ConvrotWeights(FAKE, FAKE, None, 512, k, 256) for _ in range(count)]
    if loras is None:
        loras = [cr.ConvrotLora(FAKE, FAKE, 32, 32) for _ in ws]
    return cr.convrot_linear_lora(px, ws, loras, [FAKE] * len(ws), [w.n for w in ws], act)


def test_linear_lora_validation():
    L = cr.lib()
    assert L.convrot_linear_lora(None, None, None, 1, None, None, 0, None) == cr.ERR_NULL
    px = cr.ConvrotPacked(FAKE, FAKE, 16, 1024, 256)
    w1 = (cr.ConvrotWeights * 1)(cr.ConvrotWeights(FAKE, FAKE, None, 512, 1024, 256))
    y1 = (ctypes.c_void_p * 1)(FAKE)
    l1 = (ctypes.c_int64 * 1)(512)
    assert L.convrot_linear_lora(ctypes.byref(px), w1, None, 1, y1, l1, 0, None) == cr.ERR_NULL
    assert _fused(count=cr.MAX_GROUPED + 1) == cr.ERR_SHAPE
    assert _fused(act=7) == cr.ERR_DTYPE
    lo = lambda **kw: [cr.ConvrotLora(**{**dict(u=FAKE, b=FAKE, ldu=32, rank=32), **kw})] * 3
    assert _fused(loras=lo(rank=24)) == cr.ERR_SHAPE
    assert _fused(loras=lo(rank=272, ldu=272)) == cr.ERR_SHAPE
    assert _fused(loras=lo(ldu=16)) == cr.ERR_SHAPE            # ldu < rank
    assert _fused(loras=lo(ldu=36)) == cr.ERR_UNSUPPORTED
    assert _fused(loras=lo(u=None)) == cr.ERR_NULL
    assert _fused(loras=lo(b=None)) == cr.ERR_NULL
    assert _fused(loras=lo(u=FAKE + 2)) == cr.ERR_UNSUPPORTED
    assert _fused(loras=lo(b=FAKE + 8)) == cr.ERR_UNSUPPORTED
    # rank 0: no adapter, pointers ignored -- validation passes through to the
    # weights, where a bad ldy is the first error
    none = [cr.ConvrotLora(None, None, 0, 0)] * 3
    px = cr.ConvrotPacked(FAKE, FAKE, 16, 1024, 256)
    ws = [cr.ConvrotWeights(FAKE, FAKE, None, 512, 1024, 256)] * 3
    assert cr.convrot_linear_lora(px, ws, none, [FAKE] * 3, [512, 100, 512]) == cr.ERR_SHAPE
    # empty m: nothing to launch, adapters unchecked beyond their shape
    assert _fused(m=0, loras=lo(u=None, b=None)) == cr.OK
