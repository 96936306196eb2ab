"""Checks on the gfx950 machine code of libpa.so, run by build.build() after every
build (the AMD assembly of our own code objects, disassembled with ROCm's llvm-objdump).

1. No packed fp32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32).  The device
   pass is compiled with the target feature that forbids them; this check makes sure
   that stays true, whatever the compiler version.
2. M0 is touched only by the multi-token kernel's global -> LDS loads.  Those loads are
   inline assembly that sets M0 (the LDS destination) right before each load; the
   compiler cannot keep a value of its own live in M0 across such a statement, so the
   check requires that no compiler-generated instruction reads or writes M0 at all:
   every instruction naming M0 must be `s_mov_b32 m0, <SGPR>` (sN, or the VCC halves
   the allocator may also hand an "s" operand) directly followed by
   `s_nop 0` and a `global_load_lds_*`, every `global_load_lds_*` must come right after
   such a pair, and no instruction that uses M0 implicitly (indexed register moves,
   messages, GWS, LDS-append, other LDS-DMA forms) may appear.
3. No kernel uses scratch memory (a private segment: spilled registers, or a private
   array indexed at run time), except those in SCRATCH_ALLOWED.  A spill in a chunk
   loop costs a memory round trip on every chunk; the fp32 fused decode once ran 3.5x
   slower for a runtime index into its chunk buffers.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# kernels allowed a private segment, each with the reason
SCRATCH_ALLOWED = {
    # the prompt-chunk instances at head size 128 and block size 4 (eight blocks a
    # chunk, so more block ids live) spill a few registers at the 168-VGPR budget of
    # three workgroups a compute unit; no timed workload uses them
    "_ZN2pa12_GLOBAL__N_118multi_token_kernelIDF16_Li128ELi4ELb0EEEvNS_16MultiTokenParamsE",
    "_ZN2pa12_GLOBAL__N_118multi_token_kernelIDF16bLi128ELi4ELb0EEEvNS_16MultiTokenParamsE",
}

PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
NAMES_M0 = re.compile(r"\bm0\b")
SETUP_M0 = re.compile(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)")
IMPLICIT_M0 = re.compile(r"\b(s_movrel\w*|v_movrel\w*|s_sendmsg\w*|ds_gws_\w+|ds_append|ds_consume|"
                         r"ds_read_addtid\w*|ds_write_addtid\w*|buffer_load_\w+\s.*\blds\b|"
                         r"buffer_store_lds\w*|s_set_gpr_idx_\w+)")


def _tool(name: str) -> str:
    p = os.path.join(LLVM, name)
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found (ROCm llvm tools are needed to check the code objects)")
    return p


def disassemble(lib_path: str, notes: list = None) -> list:
    """Disassembly text of every gfx950 code object bundled in lib_path (one per
    translation unit); with `notes`, also append each code object's metadata notes
    (llvm-readelf --notes) to it."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fat.bin")
        subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib_path,
                        os.path.join(tmp, "stripped")], check=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        out = []
        for k, p in enumerate(starts):
            end = starts[k + 1] if k + 1 < len(starts) else len(data)
            bundle, co = os.path.join(tmp, f"b{k}.bin"), os.path.join(tmp, f"co{k}.o")
            open(bundle, "wb").write(data[p:end])
            subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--targets={TARGET}", f"--input={bundle}", f"--output={co}"],
                           check=True)
            out.append(subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", co],
                                      check=True, capture_output=True, text=True).stdout)
            if notes is not None:
                notes.append(subprocess.run([_tool("llvm-readelf"), "--notes", co],
                                            check=True, capture_output=True, text=True).stdout)
        if not out:
            raise RuntimeError(f"{lib_path}: no offload bundle found")
        return out


def _instructions(text: str):
    """(function, instruction text) pairs, comments and encodings dropped."""
    fn = "?"
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.*)>:", line)
        if m:
            fn = m.group(1)
            continue
        if not line.startswith("\t"):
            continue
        ins = line.split("//")[0].strip()
        if ins:
            yield fn, ins


def problems(texts: list) -> list:
    """Violations of the two rules above, as readable strings (empty: all good)."""
    bad = []
    for text in texts:
        ins = list(_instructions(text))
        for i, (fn, s) in enumerate(ins):
            if PACKED_FP32.search(s):
                bad.append(f"packed fp32 instruction in {fn}: {s}")
            if IMPLICIT_M0.search(s):
                bad.append(f"instruction that uses M0 implicitly in {fn}: {s}")
            if s.startswith("global_load_lds"):
                ok = (i >= 2 and SETUP_M0.fullmatch(ins[i - 2][1])
                      and ins[i - 1][1] == "s_nop 0")
                if not ok:
                    bad.append(f"LDS-DMA load without its own M0 set-up in {fn}: {s}")
            elif NAMES_M0.search(s):
                ok = (SETUP_M0.fullmatch(s) and i + 2 < len(ins)
                      and ins[i + 1][1] == "s_nop 0" and ins[i + 2][1].startswith("global_load_lds"))
                if not ok:
                    bad.append(f"M0 used outside an LDS-DMA load sequence in {fn}: {s}")
    return bad


def scratch_sizes(notes: list) -> dict:
    """Kernel name -> private segment bytes, from the code objects' metadata notes."""
    sizes = {}
    for text in notes:
        for entry in text.split("- .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", entry)
            size = re.search(r"\.private_segment_fixed_size:\s+(\d+)", entry)
            if name and size:
                sizes[name.group(1)] = int(size.group(1))
    return sizes


def scratch_problems(sizes: dict) -> list:
    """Rule 3: kernels with a private segment that SCRATCH_ALLOWED does not list."""
    return [f"kernel uses {n} bytes of scratch memory: {k}" for k, n in sorted(sizes.items())
            if n > 0 and k not in SCRATCH_ALLOWED]


def check(lib_path: str) -> dict:
    """Raise RuntimeError listing every violation; return counts otherwise."""
    notes = []
    texts = disassemble(lib_path, notes)
    sizes = scratch_sizes(notes)
    if not sizes:
        raise RuntimeError(f"{lib_path}: no kernel metadata found in the code objects")
    bad = problems(texts) + scratch_problems(sizes)
    if bad:
        head = "\n  ".join(bad[:20])
        raise RuntimeError(f"{lib_path}: {len(bad)} machine-code check failure(s):\n  {head}")
    n_lds = sum(t.count("global_load_lds") for t in texts)
    return {"code_objects": len(texts), "lds_dma_loads": n_lds, "kernels": len(sizes)}
