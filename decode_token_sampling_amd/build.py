"""Build libvs.so (the HIP sampling library) in-tree for gfx950 with hipcc.

Every translation unit is compiled to an object in parallel, then linked into
``decode_token_sampling_amd/libvs.so``. Flags that matter for the numerics:
``-ffp-contract=off`` (no fused multiply-add unless written), correctly
rounded fp32 division (hipcc's default, no fast-math), fp32 denormals kept,
and packed-fp32 instruction selection switched off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvs.so")
# a test aid with the device exponential alone (never linked into libvs.so)
SELFTEST_LIB = os.path.join(HERE, "libvs_selftest.so")
SELFTEST_SOURCES = ["selftest.hip"]
SOURCES = ["vs_api.hip", "k_select.hip", "k_row.hip", "k_full.hip", "k_state.hip", "k_gumbel.hip",
           "k_penalize.hip"]
ARCH = os.environ.get("VS_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; keep other warnings visible
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (the device
# code is built as usual; the flags apply to the host pass only). Load the
# result with clang's ASan runtime preloaded.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """libvs.so with sanitised host code, written to ``out_dir`` (the in-tree
    library is left alone)."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *HOST_SANITIZE]
        r = subprocess.run(["hipcc", *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libvs.so")
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC",
                        *HOST_SANITIZE[:4], *objs, "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return lib


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + SELFTEST_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], SELFTEST_LIB)
    if verbose:
        print(f"built {LIB} and {SELFTEST_LIB}")
    return LIB


if __name__ == "__main__":
    build()
