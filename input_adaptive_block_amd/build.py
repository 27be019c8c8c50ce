"""Build libspade.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspade.so")
SOURCES = ["api.cpp", "summarize.hip", "select.hip", "bsattn.hip", "static_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 VALU ops off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wno-unused-result",
]


# host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is
# built as usual): a CPU-test build of the library's host validation, sizing
# and launch code, loaded with SPADE_LIB and the ASan runtime preloaded
SANITIZE = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libspade_asan.so")


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = ASAN_DIR if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    flags = [f for f in FLAGS if f != "-O3"] + SANITIZE if sanitize else FLAGS
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link the shared library; returns its path.
    sanitize=True builds the host-sanitizer variant at ASAN_LIB instead."""
    os.makedirs(ASAN_DIR if sanitize else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), SOURCES))
    lib = ASAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    extra = ["-shared-libasan", "-fsanitize=address,undefined"] if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def kernel_resources() -> dict:
    """Per-kernel register and memory figures of the device code, read from
    the code-object metadata of a device-only assembly build of every HIP
    source: {kernel symbol: {"vgpr": n, "vgpr_spill": n, "sgpr_spill": n,
    "scratch": bytes of private (scratch) memory per lane}}."""
    import re
    asm_dir = os.path.join(BUILD, "asm")
    os.makedirs(asm_dir, exist_ok=True)

    def one(src: str) -> str:
        out = os.path.join(asm_dir, src + ".s")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
        return out

    hips = [f for f in SOURCES if f.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=len(hips)) as ex:
        outs = list(ex.map(one, hips))
    res = {}
    for out in outs:
        text = open(out).read()
        # the metadata block of each kernel: ".name: <symbol>" then its fields
        for m in re.finditer(r"\.name:\s+(\S+)\n((?:\s+\.[a-z_]+:.*\n)+)", text):
            body = m.group(2)

            def field(k):
                f = re.search(r"\." + k + r":\s+(\d+)", body)
                return int(f.group(1)) if f else None

            if field("vgpr_count") is None:
                continue
            res[m.group(1)] = {"vgpr": field("vgpr_count"), "vgpr_spill": field("vgpr_spill_count"),
                               "sgpr_spill": field("sgpr_spill_count"),
                               "scratch": field("private_segment_fixed_size")}
    return res


def first_mfma_offsets(src: str = "bsattn.hip") -> dict:
    """Byte offset of the first MFMA instruction from the entry of each kernel
    of src, in a device-only build of it (the disassembly of the code object
    built here): {kernel symbol: offset}.  Kernel entries are 256-byte aligned,
    so the offset fixes where the kernel's loops sit relative to the
    instruction fetch boundaries."""
    import re
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm", "bin")
    out_dir = os.path.join(BUILD, "codeobj")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, src + ".o")
    co = os.path.join(out_dir, src + ".gfx950.co")
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
    cmd = [os.path.join(llvm, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + obj,
           "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"unbundling failed:\n{' '.join(cmd)}\n{r.stderr}")
    r = subprocess.run([os.path.join(llvm, "llvm-objdump"), "-d", co], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-objdump failed:\n{r.stderr}")
    res, cur = {}, None
    for line in r.stdout.splitlines():
        m = re.match(r"^([0-9a-f]+) <(\S+)>:", line)
        if m:
            cur = (int(m.group(1), 16), m.group(2))
            continue
        if cur and cur[1] not in res and "v_mfma" in line:
            a = re.search(r"// ([0-9A-F]+):", line)
            if a:
                res[cur[1]] = int(a.group(1), 16) - cur[0]
    return res


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
