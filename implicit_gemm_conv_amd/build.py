"""Builds the HIP libraries (gfx950) in-tree:

  implicit_gemm_conv_amd/libigc.so         the GEMM / convolution C ABI (include/igc.h)
  implicit_gemm_conv_amd/libigc_probes.so  measurement probes (include/igc_probes.h)

Each tile configuration listed in csrc/tile_configs.hpp is compiled from
csrc/instances.hip as one object per operation family (bf16 GEMM, fp16 GEMM,
forward convolution, data gradient, filter gradient; study-only
configurations build the bf16 and fp16 GEMM and the bf16 forward convolution,
forward-convolution configurations the study GEMMs and the complete forward
convolution), all in parallel, then linked with the host-side C ABI (csrc/igc_lib.hip,
csrc/registry.hip) and the split-K reduction (csrc/split_reduce.hip).
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
PROBES_LIB = os.path.join(PKG, "libigc_probes.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I" + os.path.join(ROOT, "include"),
         # packed fp32 VALU ops are disabled for all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

FAMILIES_FULL = (0, 1, 2, 3, 4)   # bf16 GEMM, fp16 GEMM, forward conv, data gradient, filter gradient
FAMILIES_STUDY = (0, 1, 2)        # bf16 and fp16 GEMM (row-major A), bf16 forward conv


def tile_configs():
    """(bm, bn, bk, depth, waves, mfma, half, loaders, sync, scope) per X(...) line of tile_configs.hpp."""
    text = open(os.path.join(CSRC, "tile_configs.hpp")).read()
    rows = re.findall(r"^\s*X\(([\d,\s]+)\)", text, re.M)
    out = []
    for r in rows:
        vals = tuple(int(v) for v in r.split(","))
        if len(vals) != 10:
            raise ValueError(f"tile_configs.hpp: expected 10 fields, got {r}")
        out.append(vals)
    return out


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{out}")
    return out


def instance_units(configs=None):
    units = []
    # IGC_BUILD_ONLY="256x256x32x4x8x16x0x4x0,..." builds a subset of the configurations (a quick partial build
    # while working on one tile; the others then report IGC_ERR_UNSUPPORTED)
    only = [c for c in os.environ.get("IGC_BUILD_ONLY", "").split(",") if c]
    for (bm, bn, bk, d, w, mi, h, lw, sy, scope) in (configs or tile_configs()):
        if only and f"{bm}x{bn}x{bk}x{d}x{w}x{mi}x{h}x{lw}x{sy}" not in only:
            continue
        full, sk, conv = scope & 1, (scope >> 1) & 1, (scope >> 2) & 1
        fams = [(f, full) for f in (FAMILIES_FULL if full else FAMILIES_STUDY)]
        if conv and not full:  # the study GEMMs, and the forward convolution complete
            fams = [(0, 0), (1, 0), (2, 1)]
        for fam, fam_full in fams:
            obj = os.path.join(OBJ_DIR, f"inst_{bm}x{bn}x{bk}x{d}x{w}x{mi}x{h}x{lw}x{sy}_f{fam}.o")
            units.append([HIPCC, *FLAGS, f"-DIGC_BM={bm}", f"-DIGC_BN={bn}", f"-DIGC_BK={bk}", f"-DIGC_D={d}",
                          f"-DIGC_W={w}", f"-DIGC_MI={mi}", f"-DIGC_HALF={h}", f"-DIGC_LW={lw}", f"-DIGC_SYNC={sy}",
                          f"-DIGC_FULL={fam_full}", f"-DIGC_SK={sk}", f"-DIGC_FAMILY={fam}", "-c",
                          os.path.join(CSRC, "instances.hip"),
                          "-o", obj])
    return units


def host_unit(name):
    return [HIPCC, *FLAGS, "-c", os.path.join(CSRC, name + ".hip"), "-o", os.path.join(OBJ_DIR, name + ".o")]


def build(jobs=None, verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    units = instance_units() + [host_unit(n) for n in ("igc_lib", "registry", "split_reduce", "probes")]
    # longest first: the instance objects dominate
    jobs = jobs or min(len(units), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, units):
            if verbose and out.strip():
                print(out)
    objs = [u[u.index("-o") + 1] for u in units]
    probe_obj = [o for o in objs if o.endswith("probes.o")]
    lib_objs = [o for o in objs if not o.endswith("probes.o")]
    for target, parts in ((LIB, lib_objs), (PROBES_LIB, probe_obj)):
        tmp = target + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts])
        os.replace(tmp, target)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
