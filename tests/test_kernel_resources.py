"""Every kernel in the built library keeps its working set in registers: no
scratch (private segment) memory and no VGPR spills, for every instantiation
that is compiled in. (Scalar registers that the compiler parks in spare VGPR
lanes are not memory traffic and are allowed; with a zero private segment no
spill of any kind reaches memory.)

The register-resident accumulator is part of the method (the TIRx `gemm`
page, "Algorithm" step 3: loop bounds are compile-time so fragments stay in
registers); a kernel that spills pays a memory round trip per spilled value in
its inner loop. This test reads the AMDGPU code-object metadata (the
NT_AMDGPU_METADATA note, msgpack) of the gfx950 objects embedded in the
library's offload bundles, so it runs on the CPU without a GPU. It also checks
that each kernel's LDS fits gfx950's 160 KiB per workgroup and that the
combined register count fits the 512 registers one wave may address.
"""
import os
import struct
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dense_gemm_tile_amd", "libdense_gemm_tile_amd.so")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32


def _bundles(data: bytes):
    """(target triple, code object bytes) for every entry of every offload
    bundle in the file (the uncompressed clang offload-bundle layout: magic,
    entry count, then offset/size/triple per entry, offsets from the magic)."""
    i = 0
    while True:
        i = data.find(BUNDLE_MAGIC, i)
        if i < 0:
            return
        (n,) = struct.unpack_from("<Q", data, i + len(BUNDLE_MAGIC))
        p = i + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            yield triple, data[i + off:i + off + size]
        i += len(BUNDLE_MAGIC)


def _metadata_notes(elf: bytes):
    """Decoded NT_AMDGPU_METADATA notes of a 64-bit little-endian ELF."""
    import msgpack
    assert elf[:4] == b"\x7fELF" and elf[4] == 2 and elf[5] == 1, "not an ELF64 LE object"
    (shoff,) = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    for s in range(shnum):
        base = shoff + s * shentsize
        (sh_type,) = struct.unpack_from("<I", elf, base + 4)
        if sh_type != 7:  # SHT_NOTE
            continue
        off, size = struct.unpack_from("<QQ", elf, base + 0x18)
        p = off
        while p + 12 <= off + size:
            namesz, descsz, ntype = struct.unpack_from("<III", elf, p)
            p += 12 + ((namesz + 3) & ~3)
            desc = elf[p:p + descsz]
            p += (descsz + 3) & ~3
            if ntype == NT_AMDGPU_METADATA:
                yield msgpack.unpackb(desc, raw=False)


def _kernels():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "dense_gemm_tile_amd", "build.py")],
                       check=True)
    with open(LIB, "rb") as f:
        data = f.read()
    out = []
    for triple, obj in _bundles(data):
        if "gfx950" not in triple:
            continue
        for md in _metadata_notes(obj):
            out.extend(md.get("amdhsa.kernels", []))
    return out


@pytest.fixture(scope="module")
def kernels():
    ks = _kernels()
    assert ks, "no gfx950 kernels found in the library's offload bundles"
    return ks


def test_library_holds_the_expected_kernel_families(kernels):
    names = " ".join(k[".name"] for k in kernels)
    for fam in ("gemm_mfma_pingpong_kernel", "gemm_mfma_kernel", "gemm_fma_kernel",
                "gemm_pp_byte_kernel", "gemm_byte_kernel", "gemm_pp_f32_kernel",
                "scale_c_kernel"):
        assert fam in names, fam


def test_no_kernel_uses_scratch_or_spills(kernels):
    bad = [(k[".name"], k[".private_segment_fixed_size"], k.get(".vgpr_spill_count"))
           for k in kernels
           if k[".private_segment_fixed_size"] or k.get(".vgpr_spill_count", 0)]
    assert not bad, f"{len(bad)} kernels spill or use scratch, e.g. {bad[:3]}"


def test_lds_and_registers_fit_gfx950(kernels):
    for k in kernels:
        assert k[".group_segment_fixed_size"] <= 160 * 1024, k[".name"]
        assert k[".vgpr_count"] <= 512, k[".name"]
