"""Properties of the built device code (CPU only, no GPU needed).

The gfx950 code objects are read out of libsv.so's offload bundles and checked with the
ROCm LLVM tools (llvm-readobj for the kernel metadata, llvm-objdump for the
instructions):
  - no kernel uses scratch memory (private segment size 0, no VGPR spills): on gfx9 a
    scratch access counts in vmcnt, and the attention and FFN kernels wait for their
    LDS-DMA tiles with exact vmcnt counts;
  - no packed-fp32 VALU instructions (v_pk_add/mul/fma_f32): the library is built
    without them;
  - M0 is the compiler's: no inline asm in the sources writes it (the LDS address of a
    DMA goes in through an M0 operand, so the compiler materialises and tracks M0), and
    in the code M0 is only ever the destination of a scalar instruction, and nothing but
    the LDS-DMA loads reads it (no relative register indexing, messages, GWS, append/consume or
    interpolation).
"""

import os
import re
import shutil
import struct
import subprocess

import pytest

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import build as B

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _llvm_tool(name):
    cands = [os.path.join(os.path.dirname(os.path.realpath(B.hipcc())), "..", "llvm", "bin", name),
             os.path.join("/opt/rocm/llvm/bin", name), shutil.which(name)]
    for c in cands:
        if c and os.path.exists(c):
            return os.path.realpath(c)
    raise RuntimeError(f"{name} not found")


def _have_tools():
    try:
        _llvm_tool("llvm-objdump")
        _llvm_tool("llvm-readobj")
        return True
    except RuntimeError:
        return False


pytestmark = [
    pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libsv.so not built"),
    pytest.mark.skipif(not _have_tools(), reason="ROCm LLVM tools not found"),
]


def _elf_section(path, wanted):
    """Bytes of the named section of an ELF64 little-endian file."""
    data = open(path, "rb").read()
    assert data[:4] == b"\x7fELF" and data[4] == 2 and data[5] == 1, "not an ELF64 LE file"
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):
        # name, type, flags, addr, offset, size
        return struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)

    strtab = header(shstrndx)
    for i in range(shnum):
        name_off, _, _, _, off, size = header(i)
        start = strtab[4] + name_off
        name = data[start:data.index(b"\0", start)].decode()
        if name == wanted:
            return data[off:off + size]
    raise KeyError(wanted)


def _gfx950_code_objects(fatbin):
    """The gfx950 entries of every offload bundle in a .hip_fatbin section."""
    out = []
    pos = 0
    while True:
        i = fatbin.find(BUNDLE_MAGIC, pos)
        if i < 0:
            return out
        n, = struct.unpack_from("<Q", fatbin, i + len(BUNDLE_MAGIC))
        off = i + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            o, size, tlen = struct.unpack_from("<QQQ", fatbin, off)
            off += 24
            triple = fatbin[off:off + tlen].decode()
            off += tlen
            if triple.endswith("gfx950"):
                out.append(fatbin[i + o:i + o + size])
        pos = i + len(BUNDLE_MAGIC)


@pytest.fixture(scope="module")
def code(tmp_path_factory):
    d = tmp_path_factory.mktemp("co")
    objs = _gfx950_code_objects(_elf_section(L.LIB_PATH, ".hip_fatbin"))
    assert objs, "no gfx950 code object in libsv.so"
    notes, asm = [], []
    for k, blob in enumerate(objs):
        p = d / f"{k}.co"
        p.write_bytes(blob)
        notes.append(subprocess.run([_llvm_tool("llvm-readobj"), "--notes", str(p)],
                                    capture_output=True, text=True, check=True).stdout)
        asm.append(subprocess.run([_llvm_tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(p)],
                                  capture_output=True, text=True, check=True).stdout)
    return notes, asm


def _kernels(notes):
    """(name, private segment bytes, VGPR spills) of every kernel in the metadata."""
    out = []
    for text in notes:
        for block in re.split(r"\n\s*- \.", text)[1:]:
            name = re.search(r"\.name:\s+(\S+)", block)
            priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
            spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
            if name and priv and spill:
                out.append((name.group(1), int(priv.group(1)), int(spill.group(1))))
    return out


def _instructions(asm):
    for text in asm:
        for line in text.splitlines():
            s = line.strip()
            if not s or s.endswith(":") or s.startswith(("Disassembly", ";")) or "file format" in s:
                continue
            yield s.split("//")[0].strip()


def test_no_kernel_uses_scratch(code):
    notes, _ = code
    ks = _kernels(notes)
    names = " ".join(k[0] for k in ks)
    for part in ("attn_kernel", "merge_kernel", "score_kernel", "topk", "block_repr",
                 "ffn_gate_up_kernel", "ffn_down_kernel", "ffn_reduce_kernel"):
        assert part in names, f"no {part} in the code objects"
    bad = [k for k in ks if k[1] != 0 or k[2] != 0]
    assert not bad, f"kernels with scratch: {bad[:5]}"


def test_no_packed_fp32_instructions(code):
    _, asm = code
    pk = [s for s in _instructions(asm) if re.match(r"v_pk_(add|mul|fma)_f32\b", s)]
    assert not pk, pk[:5]


def test_m0_only_feeds_the_lds_dma(code):
    _, asm = code
    implicit = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_append|ds_consume|v_interp|"
                          r"ds_param_load|ds_direct_load|lds_param_load|lds_direct_load|"
                          r"buffer_load\S*.*\blds\b)")
    n_dma = n_m0 = 0
    for s in _instructions(asm):
        assert not implicit.match(s), f"instruction reading M0 implicitly: {s}"
        if re.search(r"\bm0\b", s):
            # only ever the destination of a scalar instruction, never a source
            assert re.match(r"s_\w+ m0,", s) and not re.search(r",.*\bm0\b", s), \
                f"M0 read by {s}"
            n_m0 += 1
        n_dma += s.startswith("global_load_lds")
    assert n_dma > 0 and n_m0 > 0


def test_no_inline_asm_writes_m0():
    # every asm statement's template string in the device sources
    for name in sorted(os.listdir(B.CSRC)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        text = open(os.path.join(B.CSRC, name)).read()
        for m in re.finditer(r"\basm\s+(?:volatile\s*)?\(\s*((?:\"[^\"]*\"\s*)+)", text):
            assert not re.search(r"\bm0\b", m.group(1)), f"{name}: asm names M0: {m.group(1)!r}"


def _wait_states(s):
    m = re.match(r"s_nop (\d+)", s)
    return int(m.group(1)) + 1 if m else 1


def _sgprs(ops):
    regs = set()
    for a, b in re.findall(r"s\[(\d+):(\d+)\]", ops):
        regs |= set(range(int(a), int(b) + 1))
    regs |= {int(x) for x in re.findall(r"\bs(\d+)\b", ops)}
    return regs


def test_vmem_sgpr_and_m0_wait_states(code):
    _, asm = code
    for text in asm:
        ins = list(_instructions([text]))
        n_checked = 0
        for i, s in enumerate(ins):
            m = re.match(r"(global|buffer|flat|scratch)_\w+\s+(.*)", s)
            if not m:
                continue
            reads = _sgprs(m.group(2))
            is_dma = s.startswith("global_load_lds")
            waits, j = 0, i - 1
            # walk back through the straight-line code before the instruction
            while j >= 0 and waits < 5:
                p = ins[j]
                if re.match(r"s_(cbranch|branch|setpc|swappc|endpgm)", p):
                    break
                w = re.match(r"v_\w+\s+(s\d+|s\[\d+:\d+\]|vcc)\b", p)
                if w and reads & _sgprs(w.group(1)):
                    raise AssertionError(f"VMEM reads an SGPR {waits} wait states after a VALU "
                                         f"write: {p!r} ... {s!r}")
                if is_dma and waits < 1 and re.match(r"s_\w+ m0,", p):
                    raise AssertionError(f"LDS DMA reads M0 right after its write: {p!r} {s!r}")
                waits += _wait_states(p)
                j -= 1
            n_checked += 1
        assert n_checked > 0 or "global_" not in text
