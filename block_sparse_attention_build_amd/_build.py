"""Build libbsa.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Every .hip file directly under csrc/ is compiled to an object in parallel,
then linked into block_sparse_attention_build_amd/libbsa.so.  The C ABI
layer (bsa_abi.hip) is compiled a second time with BSA_CHECKED=1 and linked
with the same kernel objects into libbsa_checked.so, the build that verifies
device-side contracts on the host.  The benchmark's read-bandwidth probe
(csrc/probe/) is linked on its own into libbsa_probe.so.  Objects go to
_build/ at the repository root.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")
CHECKED_LIB = os.path.join(PKG, "libbsa_checked.so")
ABI_SRC = "bsa_abi.hip"
PROBE_LIB = os.path.join(PKG, "libbsa_probe.so")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, verbose, defines=()):
    tag = "".join("." + d.split("=")[0].lower() for d in defines)
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = ["hipcc", *CXXFLAGS, *(f"-D{d}" for d in defines), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: that warning is noise
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    abi = os.path.join(CSRC, ABI_SRC)
    jobs = [(src, ()) for src in srcs + probe] + [(abi, ("BSA_CHECKED=1",))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    lib_objs = objs[:len(srcs)]
    _link(lib_objs, LIB, verbose)
    kernels = [o for o, src in zip(lib_objs, srcs) if os.path.basename(src) != ABI_SRC]
    _link(kernels + [objs[-1]], CHECKED_LIB, verbose)
    _link(objs[len(srcs):len(srcs) + len(probe)], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
