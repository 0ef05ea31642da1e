"""fp64 CPU oracle for the batch-invariant kernels.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library never calls it and it never calls the HIP library:
the two share no code.  Inputs are plain numpy arrays (decoded from bf16 /
fp32 by the caller); every result is fp64.

The arithmetic lives in ``oracle.c`` (plain C, fp64, reductions in ascending
index order) and is loaded with ctypes; ``build()`` compiles it with gcc.
``tiny.py`` is a second implementation of the same definitions, pure Python
with exactly rounded sums and nothing shared with ``oracle.c``, against which
the tests check this one on tiny inputs.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose=False):
    """Compile oracle.c into liboracle.so (gcc, -O2, no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.POINTER(ctypes.c_double)
    PI = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_bf16_array.argtypes = [P, P, i64]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rmsnorm.argtypes = [P, i64, P, P, i64, i64, i64, ctypes.c_double]
    lib.oracle_gemm.restype = None
    lib.oracle_gemm.argtypes = [P, i64, P, i64, P, i64, i64, i64, i64]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [P, PI, P, P, i64, i64, i64, i64, i64, ctypes.c_double, P]
    lib.oracle_attention_chunked.restype = ctypes.c_int
    lib.oracle_attention_chunked.argtypes = [P, PI, P, P, i64, i64, i64, i64, i64,
                                             ctypes.c_double, i64, i64, P]
    lib.oracle_chunk_partition.restype = i64
    lib.oracle_chunk_partition.argtypes = [i64, i64, PI]
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads():
    """OpenMP threads the oracle's row loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n):
    """Threads for the oracle's row loops from now on (results do not change)."""
    _load().oracle_set_num_threads(int(n))


def round_bf16(x):
    """Round fp64 values to the nearest bf16 value (ties to even); returns fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_round_bf16_array(_p(x), _p(y), x.size)
    return y


def split_bf16x3(x):
    """The three bf16 parts of fp32 values, for contracting fp32 activations on
    bf16 matrix cores (fp32-activation mitigation: devpress.csdn.net explainer of
    "Defeating Nondeterminism in LLM Inference", sections 2 and 6 -- weights stay
    bf16, activations fp32).  hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi
    - mid), nearest-even; the differences are formed in fp64, where they are
    exact.  Returns (hi, mid, lo) as fp64 arrays."""
    x = _f64(x)
    hi = round_bf16(x)
    mid = round_bf16(x - hi)
    lo = round_bf16(x - hi - mid)
    return hi, mid, lo


def rmsnorm(x, gamma, eps):
    """y = x / sqrt(mean(x^2) + eps) * gamma, row by row.  x [M, d], gamma [d]."""
    x = _f64(x)
    gamma = _f64(gamma)
    M, d = x.shape
    y = np.empty_like(x)
    _load().oracle_rmsnorm(_p(x), d, _p(gamma), _p(y), d, M, d, float(eps))
    return y


def gemm(a, w):
    """C = A @ W with A [M, K], W [K, N]; every C[i, j] summed over ascending k."""
    a = _f64(a)
    w = _f64(w)
    M, K = a.shape
    K2, N = w.shape
    assert K == K2
    c = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm(_p(a), K, _p(w), N, _p(c), N, M, N, K)
    return c


def _attn_args(q, pos, k, v):
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    nq, Hq, D = q.shape
    L, Hkv, D2 = k.shape
    assert D == D2 and v.shape == k.shape and pos.shape == (nq,)
    assert Hq % Hkv == 0
    return q, pos, k, v, nq, Hq, D, L, Hkv


def attention(q, pos, k, v, scale):
    """Causal GQA attention of one sequence.

    q [nq, Hq, D] at absolute positions pos [nq]; k, v [L, Hkv, D] in logical
    token order.  Row i attends to keys 0..pos[i].  Returns out [nq, Hq, D].
    """
    q, pos, k, v, nq, Hq, D, L, Hkv = _attn_args(q, pos, k, v)
    out = np.empty((nq, Hq, D), dtype=np.float64)
    rc = _load().oracle_attention(_p(q), pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  _p(k), _p(v), nq, L, Hq, Hkv, D, float(scale), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_attention failed ({rc})")
    return out


def attention_chunked(q, pos, k, v, scale, chunk=256, depth=9):
    """The same attention as the method evaluates it: fixed-size chunks counted
    from absolute position 0, per-chunk (m, l, o) partials, and a binary merge
    tree padded to 2**depth leaves.  fp64 throughout."""
    q, pos, k, v, nq, Hq, D, L, Hkv = _attn_args(q, pos, k, v)
    out = np.empty((nq, Hq, D), dtype=np.float64)
    rc = _load().oracle_attention_chunked(
        _p(q), pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(k), _p(v),
        nq, L, Hq, Hkv, D, float(scale), int(chunk), int(depth), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_attention_chunked failed ({rc})")
    return out


def chunk_partition(n_keys, chunk=256):
    """Valid-key counts of the fixed-size chunks covering keys 0..n_keys-1."""
    counts = np.zeros(max(1, (n_keys + chunk - 1) // chunk), dtype=np.int64)
    n = _load().oracle_chunk_partition(int(n_keys), int(chunk),
                                       counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return [int(c) for c in counts[:n]]
