"""Builds libigc.so (HIP, gfx950) in-tree: implicit_gemm_conv_amd/libigc.so.

Each tile configuration listed in csrc/tile_configs.hpp is compiled as its own
object from csrc/instances.hip (in parallel), then linked with the host-side
C ABI (csrc/igc_lib.hip, csrc/registry.hip), the split-K reduction
(csrc/split_reduce.hip) and the measurement probes (csrc/probes.hip).
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libigc.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I" + os.path.join(ROOT, "include"),
         # packed fp32 VALU ops are disabled for all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def tile_configs():
    text = open(os.path.join(CSRC, "tile_configs.hpp")).read()
    return [tuple(int(v) for v in m)
            for m in re.findall(r"X\((\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)\)", text)]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{out}")
    return out


def build(jobs=None, verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    units = []
    for (bm, bn, bk, d, w, mi, h, lw) in tile_configs():
        obj = os.path.join(OBJ_DIR, f"inst_{bm}x{bn}x{bk}x{d}x{w}x{mi}x{h}x{lw}.o")
        units.append([HIPCC, *FLAGS, f"-DIGC_BM={bm}", f"-DIGC_BN={bn}", f"-DIGC_BK={bk}", f"-DIGC_D={d}", f"-DIGC_W={w}",
                      f"-DIGC_MI={mi}", f"-DIGC_HALF={h}", f"-DIGC_LW={lw}", "-c", os.path.join(CSRC, "instances.hip"),
                      "-o", obj])
    for name in ("igc_lib", "registry", "split_reduce", "probes"):
        units.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, name + ".hip"),
                      "-o", os.path.join(OBJ_DIR, name + ".o")])
    jobs = jobs or min(len(units), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, units):
            if verbose and out.strip():
                print(out)
    objs = [u[u.index("-o") + 1] for u in units]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
