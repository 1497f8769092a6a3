"""Build libox.so, the gfx950 HIP library, in-tree.

Every *.hip unit is compiled with hipcc for gfx950 only (in parallel), the
host-only units (*.cpp: the C-ABI front end and kernel planners) with g++, and the objects are linked by hipcc into
conv_implicit_gemm_amd/libox.so.  Packed-fp32 instruction selection is
disabled for the device code (-target-feature -packed-fp32-ops).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libox.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + CSRC, "-I" + INCLUDE]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-ffp-contract=off",
             "-I" + CSRC, "-I" + INCLUDE]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every kernel unit and the front end; link libox.so; return its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    hips = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cmds = []
    objs = []
    for f in hips:
        o = os.path.join(OBJDIR, f[:-4] + ".o")
        objs.append(o)
        cmds.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
    for f in sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp")):
        o = os.path.join(OBJDIR, f[:-4] + ".o")
        objs.append(o)
        cmds.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
