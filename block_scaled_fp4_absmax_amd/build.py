"""Build libfp4.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4.so")
SOURCES = ["quant.hip", "rotate_mx.hip", "rotate_int.hip", "rotate_nv.hip", "rotate_mat.hip",
           "unrotate_mx.hip", "unrotate_int.hip", "unrotate_nv.hip", "unrotate_mat.hip", "givens.hip", "gemm.hip", "gemm_nv.hip", "api.cpp", "perm.cpp", "calib.cpp", "device.cpp"]
HEADERS = ["fp4_device.hpp", "launch.hpp", "rotation.hpp", "rotate_kernels.hpp",
           "unrotate_kernels.hpp", "split_k.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # exact IEEE fp32 arithmetic as written: no contraction, no fast-math
    "-ffp-contract=off", "-fno-fast-math",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs (no copies out of accumulation registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


# Sources whose MFMA accumulators may live in the accumulation registers: the
# GEMMs' 256 accumulators per lane do not fit the ordinary VGPRs.
ACC_REGISTER_SOURCES = {"gemm.hip", "gemm_nv.hip"}


def _source_flags(src, flags):
    if src not in ACC_REGISTER_SOURCES:
        return flags
    out, skip = [], False
    for i, f in enumerate(flags):
        if skip:
            skip = False
            continue
        if f == "-mllvm" and i + 1 < len(flags) and flags[i + 1] == "-amdgpu-mfma-vgpr-form":
            skip = True
            continue
        out.append(f)
    return out


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    """Compile every HIP/C++ source (in parallel, one object each) and link
    them into ``out`` (always recompiles)."""
    common = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="fp4build") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [_source_flags(s, [c for c in common if c != "-shared"]) +
                ["-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            errs = list(ex.map(_run, cmds))
        tmp = out + ".tmp%d" % os.getpid()
        errs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
    err = "\n".join(e for e in errs if e)
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def is_stale(out=LIB) -> bool:
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    srcs = [os.path.join(CSRC, s) for s in SOURCES + HEADERS]
    srcs.append(os.path.join(ROOT, "include", "fp4.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


if __name__ == "__main__":
    print(build(verbose=True))
