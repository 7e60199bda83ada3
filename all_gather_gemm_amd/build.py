"""Builds libagmm.so (gfx950 kernels + C ABI) in-tree with hipcc, and records the resources
of every kernel in the built gfx950 code object (kernel_resources.json)."""
import hashlib
import json
import os
import re
import struct
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libagmm.so")
RESOURCES = os.path.join(HERE, "kernel_resources.json")
SOURCES = ["agmm_kernels.hip", "agmm_static.hip", "agmm_api.cpp"]
LLVM_BIN = "/opt/rocm/llvm/bin"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# per-kernel metadata fields kept from the code object
_FIELDS = ("vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count", "sgpr_spill_count",
           "group_segment_fixed_size", "private_segment_fixed_size", "kernarg_segment_size",
           "max_flat_workgroup_size")


def _gfx950_code_object(obj: str) -> bytes:
    """The gfx950 code object inside an object file's .hip_fatbin section (a clang offload
    bundle: magic, entry count, then per entry offset, size, triple length and triple)."""
    with tempfile.TemporaryDirectory() as td:
        fat = os.path.join(td, "fatbin")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fat}", obj, os.path.join(td, "copy.o")], check=True)
        with open(fat, "rb") as fh:
            b = fh.read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    if not b.startswith(magic):
        raise RuntimeError(f"{obj}: no offload bundle")
    n = struct.unpack_from("<Q", b, len(magic))[0]
    off = len(magic) + 8
    for _ in range(n):
        o, size, tl = struct.unpack_from("<QQQ", b, off)
        off += 24
        triple = b[off:off + tl].decode()
        off += tl
        if triple.endswith("gfx950"):
            return b[o:o + size]
    raise RuntimeError(f"{obj}: no gfx950 code object")


def kernel_resources(obj: str) -> dict:
    """Registers, spills and LDS of every kernel in obj's gfx950 code object, from its
    metadata note, the sha256 of each kernel's machine code, and the code object's sha256."""
    co = _gfx950_code_object(obj)
    with tempfile.NamedTemporaryFile(suffix=".co") as fh:
        fh.write(co)
        fh.flush()
        notes = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "--notes", fh.name],
                               check=True, capture_output=True, text=True).stdout
        syms = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "--symbols", "--wide",
                               "--sections", fh.name], check=True, capture_output=True,
                              text=True).stdout
    # the machine code of each kernel: its symbol's bytes in .text (address - section address
    # + section file offset)
    text = re.search(r"\]\s+\.text\s+PROGBITS\s+([0-9a-f]+)\s+([0-9a-f]+)\s+([0-9a-f]+)", syms)
    code = {}
    if text:
        t_addr, t_off = int(text.group(1), 16), int(text.group(2), 16)
        for m in re.finditer(r"^\s*\d+:\s+([0-9a-f]+)\s+(\d+)\s+FUNC\s+\S+\s+\S+\s+\S+\s+(\S+)$",
                             syms, re.M):
            addr, size, name = int(m.group(1), 16), int(m.group(2)), m.group(3)
            off = addr - t_addr + t_off
            code[name] = hashlib.sha256(co[off:off + size]).hexdigest()
    kernels = {}
    for block in notes.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        rec = {}
        for f in _FIELDS:
            m = re.search(r"\." + f + r":\s+(\d+)", block)
            if m:
                rec[f] = int(m.group(1))
        if name.group(1) in code:
            rec["code_sha256"] = code[name.group(1)]
        kernels[name.group(1)] = rec
    return {"code_object_sha256": hashlib.sha256(co).hexdigest(), "kernels": kernels}


def build(verbose: bool = False) -> str:
    def compile_one(src):
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    res = kernel_resources(objs[0])
    with open(RESOURCES + ".tmp", "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    os.replace(RESOURCES + ".tmp", RESOURCES)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
