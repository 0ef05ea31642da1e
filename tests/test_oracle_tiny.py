"""The C oracle against oracle/tiny.py, an independent pure-Python brute force
written from the same definitions (math.fsum sums, plain loops), on random
inputs with every size at most 32: agreement to 1e-12, and exact agreement of
the chunk partition and of the bf16 rounding."""
import struct

import numpy as np
import pytest

import oracle
from oracle import tiny

TOL = 1e-12


def max_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(float(np.max(np.abs(ref))), 1e-300)
    return float(np.max(np.abs(got - ref))) / scale


@pytest.mark.parametrize("seed", range(8))
def test_rmsnorm_and_gemm_match_brute_force(seed):
    r = np.random.default_rng(100 + seed)
    M, N, K, d = (int(v) for v in r.integers(1, 33, 4))
    x = r.normal(0.0, 3.0, (M, d))
    g = r.uniform(0.5, 1.5, d)
    assert max_rel(oracle.rmsnorm(x, g, 1e-6), tiny.rmsnorm(x.tolist(), g.tolist(), 1e-6)) <= TOL
    a = r.normal(0.0, 1.0, (M, K))
    w = r.normal(0.0, 1.0, (K, N))
    assert max_rel(oracle.gemm(a, w), tiny.gemm(a.tolist(), w.tolist())) <= TOL


@pytest.mark.parametrize("seed", range(8))
def test_attention_plain_and_chunked_match_brute_force(seed):
    r = np.random.default_rng(200 + seed)
    L = int(r.integers(1, 33))
    Hkv = int(r.choice([1, 2]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    D = int(r.choice([4, 8, 16]))
    nq = int(r.integers(1, min(L, 6) + 1))
    pos = np.sort(r.choice(L, nq, replace=False)).astype(np.int64)
    q = r.normal(0.0, 1.0, (nq, Hq, D))
    k = r.normal(0.0, 1.0, (L, Hkv, D))
    v = r.normal(0.0, 1.0, (L, Hkv, D))
    scale = 1.0 / np.sqrt(D)
    ref = tiny.attention(q.tolist(), pos.tolist(), k.tolist(), v.tolist(), scale)
    assert max_rel(oracle.attention(q, pos, k, v, scale), ref) <= TOL
    for chunk in (1, 3, 4, 8):
        n_chunks = (L + chunk - 1) // chunk
        depth = max(1, int(np.ceil(np.log2(n_chunks)))) + 1      # one level of padding more
        got = oracle.attention_chunked(q, pos, k, v, scale, chunk=chunk, depth=depth)
        brute = tiny.attention_chunked(q.tolist(), pos.tolist(), k.tolist(), v.tolist(), scale,
                                       chunk, depth)
        assert max_rel(got, brute) <= TOL, chunk
        # the merge tree reaches the plain softmax up to rounding
        assert max_rel(brute, ref) <= TOL, chunk


def test_chunk_partition_matches_brute_force():
    for chunk in (1, 4, 7, 16, 256):
        for n in range(0, 70):
            assert oracle.chunk_partition(n, chunk) == tiny.chunk_partition(n, chunk), (n, chunk)
    assert tiny.chunk_partition(500, 256) == [256, 244]
    assert tiny.chunk_partition(1000, 256) == [256, 256, 256, 232]


def _bits(x):
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def test_round_bf16_matches_brute_force_exactly():
    r = np.random.default_rng(7)
    vals = list(r.normal(0.0, 1.0, 2000) * np.exp2(r.integers(-140, 128, 2000)))
    # exact halfway points between neighbouring bf16 values (ties go to the
    # even significand), the subnormal range, the largest values and signed zeros
    for m in range(256, 512, 7):
        for e in (-133, -126, -1, 0, 5, 119):
            vals.append((m + 0.5) * 2.0 ** e)
            vals.append(-(m + 0.5) * 2.0 ** e)
    vals += [255 * 2.0 ** 120, 255.5 * 2.0 ** 120, 255.25 * 2.0 ** 120, 2.0 ** -134,
             1.5 * 2.0 ** -134, 2.0 ** -135, 0.0, -0.0, 1e300, -1e300]
    got = oracle.round_bf16(np.array(vals, dtype=np.float64))
    for x, y in zip(vals, got):
        assert _bits(float(y)) == _bits(tiny.round_bf16(float(x))), x
