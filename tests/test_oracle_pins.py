"""Pins for the fp64 oracle: closed forms, hand-worked cases, invariants,
exact (integer / rational) brute force and the pages' worked examples.

Each pin is chosen so a plausible slip in the oracle (dropped eps or scale,
mean over d-1, transposed operand, wrong GQA head, off-by-one causal mask,
no max subtraction, a wrong merge formula) fails at least one test.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


# ------------------------------------------------------------------ bf16 rounding
def test_round_bf16_known_values():
    # ties go to the even 8-bit significand
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([-3.140625]))[0] == -3.140625
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.round_bf16(np.array([big]))[0] == big
    assert np.isinf(oracle.round_bf16(np.array([big * (1 + 2.0 ** -8)]))[0])
    assert oracle.round_bf16(np.array([2.0 ** -133]))[0] == 2.0 ** -133     # smallest subnormal
    assert oracle.round_bf16(np.array([0.0]))[0] == 0.0


def test_round_bf16_matches_torch_on_fp32_values():
    # On fp32-representable inputs RNE to bf16 is also what torch's cast does.
    g = torch.Generator().manual_seed(5)
    x = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 8)
    bits = x.view(torch.int32)
    ties = (bits & ~0xFFFF) | 0x8000                      # exact halfway cases
    x = torch.cat([x, ties.view(torch.float32)])
    want = x.to(torch.bfloat16).double().numpy()
    got = oracle.round_bf16(x.double().numpy())
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------------ fp32 -> three bf16 parts
def test_split_bf16x3_reconstructs_fp32_exactly():
    # fp32 has a 24-bit significand and each bf16 part carries 8 bits, so the
    # three parts must add back to x exactly (parts in the normal range); a
    # dropped part, a sign slip in a difference or a truncating rounding fails
    g = torch.Generator().manual_seed(11)
    x = torch.randn(50000, generator=g) * torch.exp(torch.randn(50000, generator=g) * 6)
    x = torch.cat([x, torch.tensor([0.0, -0.0, 1.0, -1.0, 3.0e38, -1e-30, 1 + 2.0 ** -23])])
    xd = x.double().numpy()
    hi, mid, lo = oracle.split_bf16x3(xd)
    np.testing.assert_array_equal(hi + mid + lo, xd)
    for part in (hi, mid, lo):                                 # each part is a bf16 value
        np.testing.assert_array_equal(oracle.round_bf16(part), part)
    nz = hi != 0
    assert np.all(np.abs(mid[nz]) <= np.abs(hi[nz]) * 2.0 ** -8)   # |mid| <= half an ulp of hi
    # by hand: 1 + 2^-23 -> hi = 1, and the residual 2^-23 is itself a bf16 value
    h1, m1, l1 = oracle.split_bf16x3(np.array([1 + 2.0 ** -23]))
    assert (h1[0], m1[0], l1[0]) == (1.0, 2.0 ** -23, 0.0)
    # 1 + 2^-8 + 2^-16 + 2^-23 lies above the midpoint 1 + 2^-8, so hi = 1 + 2^-7;
    # the residual -2^-8 + 2^-16 + 2^-23 rounds (spacing 2^-16 there) to
    # mid = -2^-8 + 2^-16, leaving lo = 2^-23
    h2, m2, l2 = oracle.split_bf16x3(np.array([1 + 2.0 ** -8 + 2.0 ** -16 + 2.0 ** -23]))
    assert (h2[0], m2[0], l2[0]) == (1.0 + 2.0 ** -7, -(2.0 ** -8) + 2.0 ** -16, 2.0 ** -23)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_hand_worked_golden():
    for row in read_golden("rmsnorm_hand_worked.txt"):
        x0, x1, g0, g1, eps = map(float, row[0].split())
        y0, y1 = map(float, row[1].split())
        tol = float(row[2])
        y = oracle.rmsnorm(np.array([[x0, x1]]), np.array([g0, g1]), eps)
        assert abs(y[0, 0] - y0) < tol and abs(y[0, 1] - y1) < tol


def test_rmsnorm_zero_row_is_zero():
    y = oracle.rmsnorm(np.zeros((2, 64)), np.full(64, 1.7), 1e-6)
    assert np.all(y == 0.0) and not np.any(np.isnan(y))


def test_rmsnorm_constant_and_one_hot_rows():
    d, eps = 64, 1e-6
    g = np.linspace(0.5, 1.5, d)
    c = 2.5
    y = oracle.rmsnorm(np.full((1, d), c), g, eps)
    np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * g, rtol=1e-15)
    a, j = -7.0, 13
    x = np.zeros((1, d)); x[0, j] = a
    y = oracle.rmsnorm(x, g, eps)
    want = np.zeros(d); want[j] = a / math.sqrt(a * a / d + eps) * g[j]
    np.testing.assert_allclose(y[0], want, rtol=1e-15, atol=0)


def test_rmsnorm_unit_mean_square_invariant():
    # with gamma = 1: mean(y^2) = ms / (ms + eps) exactly in reals (divides by d, not d-1)
    r = np.random.default_rng(1)
    x = r.normal(size=(5, 96)) * np.array([[1e-4], [1e-2], [1.0], [10.0], [300.0]])
    eps = 1e-6
    y = oracle.rmsnorm(x, np.ones(96), eps)
    ms = (x * x).mean(axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-13)


def test_rmsnorm_gamma_is_per_feature():
    r = np.random.default_rng(2)
    x = r.normal(size=(3, 32))
    g = r.uniform(0.5, 1.5, size=32)
    y1 = oracle.rmsnorm(x, np.ones(32), 1e-6)
    y2 = oracle.rmsnorm(x, g, 1e-6)
    np.testing.assert_allclose(y2, y1 * g[None, :], rtol=1e-15)


# ------------------------------------------------------------------ GEMM
def test_gemm_integer_brute_force_exact():
    # exact integer arithmetic (Python ints) -- fp64 is exact for these magnitudes
    r = np.random.default_rng(3)
    M, K, N = 5, 7, 4
    A = r.integers(-4, 5, size=(M, K))
    W = r.integers(-4, 5, size=(K, N))
    want = [[sum(int(A[i, k]) * int(W[k, j]) for k in range(K)) for j in range(N)] for i in range(M)]
    got = oracle.gemm(A, W)
    assert got.tolist() == want


def test_gemm_rational_error_bound():
    # exact rational product vs fp64: |err| <= K * u * sum|a||w| (u = 2^-53), per element
    r = np.random.default_rng(4)
    M, K, N = 3, 40, 6
    A = r.normal(size=(M, K))
    W = r.normal(size=(K, N))
    got = oracle.gemm(A, W)
    u = 2.0 ** -53
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(A[i, k]) * Fraction(W[k, j]) for k in range(K))
            bound = K * u * sum(abs(A[i, k] * W[k, j]) for k in range(K)) * 1.01
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(bound)


def test_gemm_identity_and_permutation():
    r = np.random.default_rng(5)
    K, N = 16, 24
    W = r.normal(size=(K, N))
    np.testing.assert_array_equal(oracle.gemm(np.eye(K), W), W)
    perm = r.permutation(K)
    P = np.eye(K)[perm]                       # row i selects W[perm[i]]
    np.testing.assert_array_equal(oracle.gemm(P, W), W[perm])


def test_gemm_all_ones_row_gives_column_sums():
    K, N = 10, 3
    W = np.arange(K * N, dtype=np.float64).reshape(K, N)   # W[k, j] = 3k + j, not symmetric
    c = oracle.gemm(np.ones((1, K)), W)[0]
    np.testing.assert_array_equal(c, [3 * K * (K - 1) / 2 + j * K for j in range(N)])


# ------------------------------------------------------------------ attention
def _one_hot_v(L, D):
    v = np.zeros((L, 1, D))
    for j in range(L):
        v[j, 0, j] = 1.0
    return v


def test_attention_single_key_returns_v0_exactly():
    r = np.random.default_rng(6)
    q = r.normal(size=(1, 2, 8))
    k = r.normal(size=(1, 1, 8))
    v = r.normal(size=(1, 1, 8))
    out = oracle.attention(q, [0], k, v, 0.3)
    np.testing.assert_array_equal(out[0, 0], v[0, 0])
    np.testing.assert_array_equal(out[0, 1], v[0, 0])


def test_attention_closed_form_softmax_weights():
    # q = 2 e0, scale 0.5 -> s_j = k_j[0]; scores [0, ln2, ln3] -> weights [1, 2, 3] / 6
    D = 4
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 2.0
    k = np.zeros((3, 1, D)); k[:, 0, 0] = [0.0, math.log(2), math.log(3)]
    out = oracle.attention(q, [2], k, _one_hot_v(3, D), 0.5)
    np.testing.assert_allclose(out[0, 0], [1 / 6, 2 / 6, 3 / 6, 0.0], rtol=1e-14, atol=1e-16)


def test_attention_large_scores_need_max_subtraction():
    D = 2
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, D)); k[:, 0, 0] = [1000.0, 1000.0 + math.log(3)]
    out = oracle.attention(q, [1], k, _one_hot_v(2, D), 1.0)
    np.testing.assert_allclose(out[0, 0], [0.25, 0.75], rtol=1e-12)


def test_attention_two_token_logistic_case():
    # D = 64 so scale = 1/8; q = e0, k0 = 0, k1 = 8 e0: scores [0, 1]
    D = 64
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, D)); k[1, 0, 0] = 8.0
    out = oracle.attention(q, [1], k, _one_hot_v(2, D), 1 / 8)
    w1 = 1 / (1 + math.exp(-1))
    np.testing.assert_allclose(out[0, 0, :2], [1 - w1, w1], rtol=1e-14)
    assert abs(out[0, 0, 0] - 0.268941421) < 1e-9


def test_attention_causal_mask_counts_keys_0_to_pos():
    # zero keys -> equal scores -> uniform weights over exactly keys 0..pos
    L, D = 9, 9
    q = np.random.default_rng(7).normal(size=(4, 1, D))
    pos = [0, 3, 4, 8]
    out = oracle.attention(q, pos, np.zeros((L, 1, D)), _one_hot_v(L, D), 0.7)
    for i, p in enumerate(pos):
        want = np.zeros(D); want[: p + 1] = 1.0 / (p + 1)
        np.testing.assert_allclose(out[i, 0], want, rtol=1e-14, atol=1e-17)


def test_attention_all_keys_equal_gives_mean_of_v():
    r = np.random.default_rng(8)
    L, D = 37, 16
    k = np.repeat(r.normal(size=(1, 1, D)), L, axis=0)
    v = r.normal(size=(L, 1, D))
    out = oracle.attention(r.normal(size=(1, 1, D)), [L - 1], k, v, 0.25)
    np.testing.assert_allclose(out[0, 0], v[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_gqa_head_mapping():
    # heads 0,1 read KV head 0 (values 1), heads 2,3 read KV head 1 (values 2)
    r = np.random.default_rng(9)
    L, D = 5, 8
    k = r.normal(size=(L, 2, D))
    v = np.empty((L, 2, D)); v[:, 0] = 1.0; v[:, 1] = 2.0
    out = oracle.attention(r.normal(size=(2, 4, D)), [3, 4], k, v, 0.3)
    np.testing.assert_allclose(out[:, :2], 1.0, rtol=1e-15)
    np.testing.assert_allclose(out[:, 2:], 2.0, rtol=1e-15)
    # and it equals MHA with each KV head repeated for its group of query heads
    qq = r.normal(size=(2, 4, D))
    vv = r.normal(size=(L, 2, D))
    gqa = oracle.attention(qq, [2, 4], k, vv, 0.3)
    mha = oracle.attention(qq, [2, 4], np.repeat(k, 2, axis=1), np.repeat(vv, 2, axis=1), 0.3)
    np.testing.assert_allclose(gqa, mha, rtol=1e-15)


def test_attention_score_shift_invariance():
    # an extra feature adds the same constant c to every score of a row: no change
    r = np.random.default_rng(10)
    L, D, scale, c = 20, 8, 0.2, 5.0
    q = r.normal(size=(1, 1, D)); k = r.normal(size=(L, 1, D)); v = r.normal(size=(L, 1, D))
    base = oracle.attention(q, [L - 1], k, v, scale)
    q2 = np.concatenate([q, np.full((1, 1, 1), c / scale)], axis=2)
    k2 = np.concatenate([k, np.ones((L, 1, 1))], axis=2)
    v2 = np.concatenate([v, np.zeros((L, 1, 1))], axis=2)
    shifted = oracle.attention(q2, [L - 1], k2, v2, scale)
    np.testing.assert_allclose(shifted[..., :D], base, rtol=1e-13)


def test_attention_scale_enters_scores():
    # scale s with q, or scale 1 with s*q: same scores
    r = np.random.default_rng(11)
    q = r.normal(size=(1, 1, 8)); k = r.normal(size=(6, 1, 8)); v = r.normal(size=(6, 1, 8))
    a = oracle.attention(q, [5], k, v, 0.37)
    b = oracle.attention(q * 0.37, [5], k, v, 1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    c = oracle.attention(q, [5], k, v, 1.0)
    assert np.max(np.abs(a - c)) > 1e-3


# ------------------------------------------------------------------ chunked form
@pytest.mark.parametrize("L", [1, 255, 256, 257, 700, 1300])
def test_chunked_attention_equals_plain(L):
    r = np.random.default_rng(100 + L)
    Hq, Hkv, D = 4, 2, 16
    k = r.normal(size=(L, Hkv, D)); v = r.normal(size=(L, Hkv, D))
    pos = sorted(set([0, L // 3, L // 2, L - 1]))
    q = r.normal(size=(len(pos), Hq, D))
    plain = oracle.attention(q, pos, k, v, 0.25)
    chunked = oracle.attention_chunked(q, pos, k, v, 0.25, chunk=256, depth=9)
    np.testing.assert_allclose(chunked, plain, rtol=1e-12, atol=1e-14)


def test_chunked_attention_depth_padding_is_exact():
    # identity leaves are exact no-ops: depth 3 and depth 9 give the same bits
    r = np.random.default_rng(12)
    L, D = 1500, 8
    k = r.normal(size=(L, 1, D)); v = r.normal(size=(L, 1, D))
    q = r.normal(size=(3, 1, D))
    pos = [L - 1, 1024, 300]
    a = oracle.attention_chunked(q, pos, k, v, 0.3, chunk=256, depth=3)
    b = oracle.attention_chunked(q, pos, k, v, 0.3, chunk=256, depth=9)
    np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.attention_chunked(q[:1], [L - 1], k, v, 0.3, chunk=256, depth=2)


def test_chunk_partition_golden_fixed256():
    for row in read_golden("chunk_partition_fixed256.txt"):
        L = int(row[0])
        counts = [int(c) for c in row[1].split()]
        token_chunk = int(row[2])
        assert oracle.chunk_partition(L, 256) == counts
        assert 300 // 256 == token_chunk
        # the chunk holding token 300 is a full 256-token chunk in both examples
        assert counts[token_chunk] == 256 or L == 500


def test_block32_counterexample_golden():
    rows = {r[0]: [int(x) for x in r[1].split()] for r in read_golden("block32_counterexample.txt")}
    separate = oracle.chunk_partition(80, 32) + oracle.chunk_partition(48, 32)
    assert separate == rows["separate_cache_80_new_48"]
    assert oracle.chunk_partition(128, 32) == rows["one_shot_128"]
    # a single partition from absolute position 0 is the same whatever the split
    # between cached and new tokens
    assert oracle.chunk_partition(80 + 48, 32) == rows["one_shot_128"]
