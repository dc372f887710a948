"""The built libraries' gfx950 kernels use no private scratch memory (CPU).

Every kernel of libconvrot.so and libconvrot_ceiling.so is checked through
the metadata the compiler writes into each code object (the AMDGPU note of
the gfx950 ELF inside the host library's offload bundles): no fixed private
segment and no vector registers spilled.  Scalar registers that the compiler
parks in vector-register lanes are not memory and are not counted.  Skipped
when the libraries have not been built.
"""

import os
import struct

import msgpack
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "hadamard_rotated_int8_amd")
LIBS = [os.path.join(PKG, "libconvrot.so"), os.path.join(PKG, "libconvrot_ceiling.so")]
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32


def _sections(elf: bytes):
    """(name, type, offset, size) of every section of a little-endian ELF64 file."""
    assert elf[:4] == b"\x7fELF" and elf[4] == 2 and elf[5] == 1, "ELF64 little-endian expected"
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdrs = []
    for i in range(shnum):
        name, typ, _flags, _addr, off, size = struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize)
        hdrs.append((name, typ, off, size))
    str_off, str_size = hdrs[shstrndx][2], hdrs[shstrndx][3]
    strtab = elf[str_off:str_off + str_size]
    out = []
    for name, typ, off, size in hdrs:
        end = strtab.index(b"\0", name)
        out.append((strtab[name:end].decode(), typ, off, size))
    return out


def _device_code_objects(lib_bytes: bytes):
    """The gfx950 code objects of every offload bundle in the .hip_fatbin section."""
    sec = [s for s in _sections(lib_bytes) if s[0] == ".hip_fatbin"]
    assert len(sec) == 1, "no .hip_fatbin section"
    _, _, off, size = sec[0]
    fat = lib_bytes[off:off + size]
    objs = []
    start = fat.find(BUNDLE_MAGIC)
    while start >= 0:
        count = struct.unpack_from("<Q", fat, start + len(BUNDLE_MAGIC))[0]
        p = start + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            e_off, e_size, t_len = struct.unpack_from("<QQQ", fat, p)
            p += 24
            triple = fat[p:p + t_len].decode()
            p += t_len
            if triple.startswith("hip") and e_size:
                objs.append((triple, fat[start + e_off:start + e_off + e_size]))
        start = fat.find(BUNDLE_MAGIC, start + 1)
    return objs


def _kernels(code_object: bytes):
    """Kernel metadata maps from the AMDGPU note of a device ELF."""
    kernels = []
    for _name, typ, off, size in _sections(code_object):
        if typ != 7:  # SHT_NOTE
            continue
        p, end = off, off + size
        while p + 12 <= end:
            namesz, descsz, ntype = struct.unpack_from("<III", code_object, p)
            p += 12
            name = code_object[p:p + namesz].rstrip(b"\0")
            p += (namesz + 3) & ~3
            desc = code_object[p:p + descsz]
            p += (descsz + 3) & ~3
            if name == b"AMDGPU" and ntype == NT_AMDGPU_METADATA:
                meta = msgpack.unpackb(desc, raw=False)
                kernels += meta.get("amdhsa.kernels", [])
    return kernels


@pytest.mark.parametrize("lib", LIBS, ids=os.path.basename)
def test_kernels_use_no_scratch(lib):
    if not os.path.exists(lib):
        pytest.skip(f"{os.path.basename(lib)} not built")
    objs = _device_code_objects(open(lib, "rb").read())
    assert objs, "no device code objects found"
    assert all(t.endswith("gfx950") for t, _ in objs), [t for t, _ in objs]
    kernels = [k for _, co in objs for k in _kernels(co)]
    assert kernels, "no kernel metadata found"
    bad = [(k[".name"], k.get(".private_segment_fixed_size"), k.get(".vgpr_spill_count"))
           for k in kernels
           if k.get(".private_segment_fixed_size", 0) != 0 or k.get(".vgpr_spill_count", 0) != 0]
    assert not bad, bad
