"""binv_gemm_bf16 on the GPU: exact integer parity, identity, oracle parity at
the GEMM shapes, bitwise invariance of a target row to M and to its position
in the tile, run-to-run determinism, and the shape-tuned comparator."""
import numpy as np
import pytest
import torch

import invariant_deterministic_fixed_amd as binv
import oracle
from invariant_deterministic_fixed_amd import synth
from helpers import TOL_BF16, TOL_F32_LOGITS, assert_bitwise_equal, bits, f64, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M_SWEEP = [1, 2, 7, 16, 64, 256, 1024, 2048, 8192]


def ints(shape, seed, lo=-4, hi=4):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.integers(lo, hi + 1, size=shape).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (7, 136, 264), (16, 24, 200), (33, 4104, 136),
                                   (64, 8, 72), (130, 256, 512), (257, 392, 1032)])
def test_integer_inputs_exact(M, N, K):
    # |sum| <= K * 16 < 2^24: every fp32 partial sum is exact in any order
    A, W = ints((M, K), 1 + M), ints((K, N), 2 + N)
    exact = oracle.gemm(f64(A), f64(W))
    c32 = binv.gemm(A.to(DEV), W.to(DEV), out_dtype=torch.float32)
    np.testing.assert_array_equal(f64(c32), exact)
    c16 = binv.gemm(A.to(DEV), W.to(DEV))
    np.testing.assert_array_equal(f64(c16), oracle.round_bf16(exact))


def test_identity_and_permutation_rows():
    K, N = 256, 384
    W = synth.normal((K, N), 0.02, 5)
    I = torch.eye(K, dtype=torch.bfloat16)
    c = binv.gemm(I.to(DEV), W.to(DEV), out_dtype=torch.float32)
    np.testing.assert_array_equal(f64(c), f64(W))
    perm = np.random.default_rng(3).permutation(K)[:100]
    P = torch.zeros((100, K), dtype=torch.bfloat16)
    P[np.arange(100), perm] = 1
    c = binv.gemm(P.to(DEV), W.to(DEV))
    np.testing.assert_array_equal(f64(c), f64(W)[perm])


def test_k_zero_writes_zeros():
    A = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((0, 16), dtype=torch.bfloat16, device=DEV)
    out = torch.full((5, 16), 7.0, device=DEV)
    # K = 0: lda/ldw are not meaningful; pass through the raw ABI with ld = 8
    st = binv.lib().binv_gemm_bf16(A.data_ptr() or (1 << 20), 8, W.data_ptr() or (1 << 20), 16,
                                   out.data_ptr(), 0, 16, 5, 16, 0, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_parity_tiny_layer():
    A = synth.normal((8, 256), 1.0, synth.seed_for(1))
    W = synth.normal((256, 256), 0.02, synth.seed_for(1) + 1)
    c = binv.gemm(A.to(DEV), W.to(DEV))
    assert row_rel_err(f64(c), oracle.gemm(f64(A), f64(W))).max() <= TOL_BF16


@pytest.mark.parametrize("N,K", [(4096, 4096), (14336, 4096), (4096, 14336)])
def test_parity_layer_shapes_sampled_rows(N, K):
    M = 256
    A = synth.normal((M, K), 1.0, synth.seed_for(2) + N + K)
    W = synth.normal((K, N), 0.02, synth.seed_for(2) + 7)
    c16 = binv.gemm(A.to(DEV), W.to(DEV)).cpu()
    c32 = binv.gemm(A.to(DEV), W.to(DEV), out_dtype=torch.float32).cpu()
    rows = [0, 1, 37, 128, 255]
    ref = oracle.gemm(f64(A[rows]), f64(W))
    assert row_rel_err(f64(c16[rows]), ref).max() <= TOL_BF16
    assert row_rel_err(f64(c32[rows]), ref).max() <= 1e-5


def test_parity_lm_head_fp32_logits():
    K, N = 4096, 128256
    A = synth.normal((3, K), 1.0, synth.seed_for(5))
    W = synth.normal((K, N), 0.02, synth.seed_for(5) + 1)
    c = binv.gemm(A.to(DEV), W.to(DEV), out_dtype=torch.float32).cpu()
    ref = oracle.gemm(f64(A), f64(W))
    assert row_rel_err(f64(c), ref).max() <= TOL_F32_LOGITS


@pytest.mark.parametrize("N,K", [(4096, 4096), (14336, 4096), (4096, 14336)])
def test_row0_bitwise_invariant_over_M(N, K):
    W = synth.normal((K, N), 0.02, synth.seed_for(2) + 7).to(DEV)
    target = synth.normal((1, K), 1.0, synth.TARGET_SEED)
    ref16 = ref32 = None
    sweep = M_SWEEP if N * K <= 4096 * 4096 else [1, 7, 256, 1024, 4096]
    for M in sweep:
        A = synth.normal((M, K), 1.0, synth.seed_for(2, trial=M))
        A[0] = target[0]
        Ad = A.to(DEV)
        c16 = binv.gemm(Ad, W)[:1]
        c32 = binv.gemm(Ad, W, out_dtype=torch.float32)[:1]
        if ref16 is None:
            ref16, ref32 = c16.clone(), c32.clone()
        assert_bitwise_equal(c16, ref16, f"bf16 M={M}")
        assert_bitwise_equal(c32, ref32, f"fp32 M={M}")


@pytest.mark.parametrize("N,K", [(24, 72), (4104, 200), (4096, 4160), (136, 4096), (6152, 200),
                                 (14344, 136), (14336, 4096), (4096, 14336)])
def test_kernels_chosen_by_shape_agree_bitwise(N, K):
    # M <= 64 runs on strips of 16, 32 or 64 columns (by N), mid-size M on
    # 64 x 64, 128 x 128 or 256 x 128 tiles and large M x N on 256 x 256 tiles (the
    # two-group schedule for tiles inside C with K a multiple of 64, the
    # one-group schedule on the edges); every element must come out with the
    # same bits on all of them, ragged N and K, zero and negative-zero rows
    # against an all-negative column included, over the whole M sweep of the
    # GEMM workload at the FFN shapes
    W = synth.normal((K, N), 0.02, 41 + N)
    W[:, 3] = -W[:, 3].abs() - 0.01
    W = W.to(DEV)
    big_m = 8192 if N >= 4096 else 130                  # 256 x 256 tiles when N allows
    A = synth.normal((big_m, K), 1.0, 43 + K)
    A[5] = 0.0
    A[6] = -0.0
    Ad = A.to(DEV)
    ref32 = binv.gemm(Ad, W, out_dtype=torch.float32)
    ref16 = binv.gemm(Ad, W)
    ms = [1, 7, 16, 17, 32, 33, 64, 65, 130, 300]
    if big_m == 8192:
        ms += [2, 256, 512, 600, 1024, 2048, 4097]
    for M in ms:
        assert_bitwise_equal(binv.gemm(Ad[:M], W, out_dtype=torch.float32), ref32[:M], f"fp32 M={M}")
        assert_bitwise_equal(binv.gemm(Ad[:M], W), ref16[:M], f"bf16 M={M}")


@pytest.mark.parametrize("N,K", [(4096, 4096), (6144, 4096), (4096, 14336), (200, 72),
                                 (1000, 4104), (24, 8)])
def test_packed_weights_give_the_plain_entry_points_bits(N, K):
    # decode batches over weights packed per 16-column strip: every row equals
    # binv_gemm_bf16's bitwise (bf16 and fp32 out) for M over 1..64, with N and
    # K that leave partial strips and a partial 64-wide K-tile
    A = synth.normal((64, K), 1.0, 41, DEV)
    W = synth.normal((K, N), 0.02, 42, DEV)
    wp = binv.gemm_pack(W)
    assert wp.data.numel() == binv.lib().binv_gemm_bf16_packed_bytes(N, K)
    for M in (1, 2, 5, 15, 16, 17, 31, 32, 33, 48, 63, 64):
        for dt in (torch.bfloat16, torch.float32):
            plain = binv.gemm(A[:M], W, out_dtype=dt)
            packed = binv.gemm_packed(A[:M], wp, out_dtype=dt)
            assert_bitwise_equal(packed, plain, f"M={M} {dt}")
    # strided A rows, an output with a leading dimension past N
    Ab = synth.normal((7, K + 64), 1.0, 43, DEV)
    out = torch.full((7, N + 8), float("nan"), dtype=torch.float32, device=DEV)
    binv.gemm_packed(Ab[:, :K], wp, out=out[:, :N])
    assert_bitwise_equal(out[:, :N], binv.gemm(Ab[:, :K], W, out_dtype=torch.float32), "strided")
    assert bool(torch.isnan(out[:, N:]).all())


def test_packed_weights_exact_integers_and_limits():
    # exact against the oracle on integer inputs; K = 0 writes zeros; M > 64
    # is rejected without a launch
    M, N, K = 9, 136, 264
    A, W = ints((M, K), 51), ints((K, N), 52)
    wp = binv.gemm_pack(W.to(DEV))
    c32 = binv.gemm_packed(A.to(DEV), wp, out_dtype=torch.float32)
    np.testing.assert_array_equal(f64(c32), oracle.gemm(f64(A), f64(W)))
    wz = binv.gemm_pack(torch.empty((0, 16), dtype=torch.bfloat16, device=DEV))
    z = torch.full((3, 16), 7.0, dtype=torch.float32, device=DEV)
    binv.gemm_packed(torch.empty((3, 0), dtype=torch.bfloat16, device=DEV), wz, out=z)
    assert bool((z == 0).all())
    with pytest.raises(binv.BinvError):
        binv.gemm_packed(torch.zeros((65, K), dtype=torch.bfloat16, device=DEV), wp)


def test_target_row_at_every_tile_position():
    # the target lands at every row of a 128-row tile and in several tiles:
    # all copies must carry identical bits
    K, N = 4096, 4096
    W = synth.normal((K, N), 0.02, 9).to(DEV)
    target = synth.normal((1, K), 1.0, synth.TARGET_SEED)
    A = synth.normal((520, K), 1.0, 123)
    rows = list(range(128)) + [128 + 5, 256 + 64, 384 + 127, 512, 519]
    for r in rows:
        A[r] = target[0]
    c = binv.gemm(A.to(DEV), W, out_dtype=torch.float32).cpu()
    alone = binv.gemm(target.to(DEV), W, out_dtype=torch.float32).cpu()
    for r in rows:
        assert_bitwise_equal(c[r:r + 1], alone, f"row {r}")


def test_run_to_run_deterministic():
    A = synth.normal((2048, 2048), 1.0, 31).to(DEV)
    W = synth.normal((2048, 2048), 0.02, 32).to(DEV)
    a = binv.gemm(A, W, out_dtype=torch.float32)
    b = binv.gemm(A, W, out_dtype=torch.float32)
    assert_bitwise_equal(a, b, "repeat")


def test_tuned_comparator_parity_and_positive_control():
    K, N = 4096, 4096
    W = synth.normal((K, N), 0.02, synth.seed_for(2) + 7).to(DEV)
    target = synth.normal((1, K), 1.0, synth.TARGET_SEED)
    ref = oracle.gemm(f64(target), f64(W))
    outs = []
    for M in [1, 64, 8192]:
        A = synth.normal((M, K), 1.0, synth.seed_for(2, trial=M))
        A[0] = target[0]
        c = binv.gemm(A.to(DEV), W, out_dtype=torch.float32, tuned=True)[:1]
        assert row_rel_err(f64(c), ref).max() <= 1e-5
        outs.append(bits(c))
    assert any(not np.array_equal(outs[0], o) for o in outs[1:]), \
        "tuned GEMM gave identical bits for every M: the sweep is not sensitive"


def test_batch_composition_probe_on_torch_mm():
    # the pages' probe: mm(a[:1], b) vs mm(a, b)[:1] with linspace inputs.
    # Reported only: whether the vendor GEMM differs is not ours to gate.
    B, D = 2048, 4096
    a = torch.linspace(-1000, 1000, B * D, device=DEV).reshape(B, D)
    b = torch.linspace(-1000, 1000, D * D, device=DEV).reshape(D, D)
    diff = (torch.mm(a[:1], b) - torch.mm(a, b)[:1]).abs().max().item()
    print(f"torch.mm batch-composition max abs diff: {diff}")
    ab, bb = a.to(torch.bfloat16), b.to(torch.bfloat16)
    ours = (binv.gemm(ab[:1], bb, out_dtype=torch.float32)
            - binv.gemm(ab, bb, out_dtype=torch.float32)[:1]).abs().max().item()
    assert ours == 0.0
