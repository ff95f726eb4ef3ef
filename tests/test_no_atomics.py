"""Single-writer design: no atomics anywhere in the attention kernels.

The backward section of "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels" (nanless.github.io digest) gives every per-offset
gradient entry exactly one writing block, so no atomic update is needed and
the summation order is fixed.  Two checks, both on the CPU:

* the HIP sources of the kernels use no atomic operation (comments aside);
* the gfx950 machine code of the built library, disassembled, holds no
  atomic memory instruction (global, buffer, flat or LDS) in any kernel.
"""

import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_relative_position_amd", "csrc")
LIB = os.path.join(ROOT, "exact_relative_position_amd", "librelpos_attn.so")
LLVM = "/opt/rocm/llvm/bin"

KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hpp", "attn_bwd_q.hpp", "attn_bwd_k.hpp",
                  "attn_bwd_f16.hip", "attn_bwd_bf16.hip", "attn_bwd_f32.hip", "qside.hpp",
                  "tiles.hpp", "device.hpp", "dropout.hpp", "geometry.hpp", "buckets.hpp",
                  "prep.hip", "proj.hip", "contract.hip"]


def _strip_comments(src):
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    return re.sub(r"//[^\n]*", " ", src)


@pytest.mark.parametrize("name", KERNEL_SOURCES)
def test_kernel_sources_use_no_atomics(name):
    with open(os.path.join(CSRC, name)) as fh:
        code = _strip_comments(fh.read())
    hits = re.findall(r"\w*atomic\w*", code, flags=re.I)
    assert not hits, f"{name}: {sorted(set(hits))}"


def _device_code_objects(path):
    """gfx950 code objects of every translation unit in the library's
    offload-bundle section (one bundle per source file)."""
    out = os.path.join(os.path.dirname(path), ".fatbin.tmp")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={out}",
                    path, os.devnull], check=True, capture_output=True)
    try:
        data = open(out, "rb").read()
    finally:
        os.remove(out)
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    objs, pos = [], 0
    while (i := data.find(magic, pos)) >= 0:
        off = i + len(magic)
        (n,) = struct.unpack_from("<Q", data, off)
        off += 8
        for _ in range(n):
            eo, es, tl = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tl].decode()
            off += tl
            if "gfx950" in triple:
                objs.append(data[i + eo:i + eo + es])
        pos = i + len(magic)
    return objs


ATOMIC_INSN = re.compile(r"^\s+((?:global|buffer|flat)_atomic\w*|ds_(?:add|sub|rsub|inc|dec|min|"
                         r"max|and|or|xor|mskor|cmpst|cmpswap|wrxchg\w*|pk_add)\w*)\b", re.M)


def test_atomic_pattern_matches_atomic_mnemonics():
    for line in ("\tglobal_atomic_add_f32 v1, v2, s[0:1]", "\tbuffer_atomic_add v1, off",
                 "\tflat_atomic_cmpswap v[0:1], v[2:3]", "\tds_add_u32 v1, v2",
                 "\tds_max_rtn_f32 v0, v1, v2", "\tds_wrxchg_rtn_b32 v0, v1, v2"):
        assert ATOMIC_INSN.search(line), line
    for line in ("\tds_read_b128 v[0:3], v4", "\tds_write_b64 v1, v[2:3]",
                 "\tglobal_load_lds_dwordx4 v[0:1], off", "\tds_bpermute_b32 v0, v1, v2",
                 "\tds_read_b64_tr_b16 v[0:1], v2"):
        assert not ATOMIC_INSN.search(line), line


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "llvm-objdump")),
                    reason="llvm-objdump not installed")
def test_machine_code_has_no_atomic_instructions(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("librelpos_attn.so is not built; run __graft_entry__.build()")
    lib = tmp_path / "lib.so"
    shutil.copy(LIB, lib)
    objs = _device_code_objects(str(lib))
    assert len(objs) >= 7, "expected one gfx950 code object per HIP source"
    kernels = set()
    for k, blob in enumerate(objs):
        f = tmp_path / f"co{k}.elf"
        f.write_bytes(blob)
        asm = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn",
                              str(f)], check=True, capture_output=True, text=True).stdout
        kernels |= set(re.findall(r"^[0-9a-f]+ <(\S+)>:", asm, flags=re.M))
        hits = ATOMIC_INSN.findall(asm)
        assert not hits, f"code object {k}: {sorted(set(hits))}"
    # the attention kernels were among those disassembled
    assert any("fwd_kernel" in n for n in kernels)
    assert any("bwd_kernel" in n for n in kernels)
