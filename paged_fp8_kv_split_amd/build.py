"""Build ``libpfkv.so`` (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m paged_fp8_kv_split_amd.build`` from the repository root.

After linking, the device assembly of every kernel source is checked: no
scratch (register spills would put the hot loop on slow memory), and M0 written
only by the page-transfer sequences, which save and restore it.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpfkv.so")

KERNEL_SOURCES = ["splitkv_main.hip", "splitkv_main_rm.hip", "splitkv_main_fp8p.hip", "splitkv_main_fp8.hip",
                  "splitkv_main_hd128.hip",
                  "segment_reduce.hip",
                  "stream_read.hip", "debug_check.hip", "prefill.hip", "noalloc.hip"]
SOURCES = ["pfkv_host.cpp", *KERNEL_SOURCES]
# headers the kernel sources include (a change to one rebuilds everything anyway)
HEADERS = ["pfkv_internal.h", "splitkv_kernel.h", "segment_merge.h", "prefill_config.h"]

ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    path = shutil.which("hipcc")
    if path:
        return path
    fallback = "/opt/rocm/bin/hipcc"
    if os.path.exists(fallback):
        return fallback
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out)
    return out


def check_device_asm(asm: str, source: str) -> None:
    """Reject spills and foreign M0 writes in one source's gfx950 assembly."""
    for m in re.finditer(r"\.private_segment_fixed_size:\s+(\d+)", asm):
        if int(m.group(1)) != 0:
            raise RuntimeError(f"{source}: a kernel uses {m.group(1)} bytes of scratch (register spills)")
    lines = [l.strip() for l in asm.splitlines()]
    for k, line in enumerate(lines):
        if re.match(r"s_\w+\s+m0\s*,", line):
            # allowed: "s_mov_b32 m0, sX" directly followed by s_nop and the LDS transfer,
            # and the restore right after the transfer
            nxt = lines[k + 1] if k + 1 < len(lines) else ""
            prev = lines[k - 1] if k > 0 else ""
            if nxt.startswith("s_nop") and lines[k + 2].startswith("global_load_lds_dword"):
                continue
            if prev.startswith("global_load_lds_dword"):
                continue
            raise RuntimeError(f"{source}: unexpected M0 write: {line}")


def build(verbose: bool = False, check: bool = True) -> str:
    """Compile every HIP source into ``libpfkv.so``; returns its path.

    Each source compiles to an object (and, for the check, to device assembly)
    in parallel; the objects are then linked.
    """
    hipcc = _hipcc()
    fd, tmp = tempfile.mkstemp(prefix="libpfkv.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    try:
        with tempfile.TemporaryDirectory() as td:
            jobs = [[hipcc, *FLAGS, "-c", "-o", os.path.join(td, s + ".o"), os.path.join(CSRC, s)] for s in SOURCES]
            if check:
                jobs += [[hipcc, *FLAGS, "--cuda-device-only", "-S", "-o", os.path.join(td, s + ".s"),
                          os.path.join(CSRC, s)] for s in KERNEL_SOURCES]
            workers = max(1, min(len(jobs), os.cpu_count() or 4, 16))
            with ThreadPoolExecutor(workers) as pool:
                list(pool.map(lambda cmd: _run(cmd, verbose), jobs))
            _run([hipcc, *FLAGS, "-shared", "-o", tmp, *[os.path.join(td, s + ".o") for s in SOURCES]], verbose)
            if check:
                for s in KERNEL_SOURCES:
                    with open(os.path.join(td, s + ".s")) as f:
                        check_device_asm(f.read(), s)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
