"""Build libbinv.so in-tree with hipcc for gfx950.

Every HIP source is compiled with the same flags: no fast-math, no floating
point contraction (so shared arithmetic compiles identically in every kernel),
and packed fp32 instructions disabled.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbinv.so")
SOURCES = ["abi.cpp", "rmsnorm.hip", "gemm.hip", "gemm_packed.hip", "attention.hip",
           "attention_tuned.hip", "glue.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build_library(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# test-only HIP code (kernels that check a device function of the library on
# every input); built beside the tests, never linked into libbinv
TEST_SUPPORT = os.path.join(ROOT, "tests", "gpu_support")
TEST_LIBS = {"libconvcheck.so": ["conv_check.hip"]}


def build_test_support(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    out = []
    for lib, srcs in TEST_LIBS.items():
        objs = []
        for src in srcs:
            obj = os.path.join(BUILD, "test_" + src + ".o")
            cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(TEST_SUPPORT, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
            objs.append(obj)
        path = os.path.join(TEST_SUPPORT, lib)
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", path + ".tmp"]
                       + objs, check=True)
        os.replace(path + ".tmp", path)
        out.append(path)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_test_support(verbose=True))
