"""binv_rmsnorm on the GPU: parity with the fp64 oracle, closed forms,
bitwise invariance to M and batch position, run-to-run determinism, and a
positive control on the shape-tuned comparator."""
import numpy as np
import pytest
import torch

import invariant_deterministic_fixed_amd as binv
import oracle
from invariant_deterministic_fixed_amd import synth
from helpers import TOL_BF16, assert_bitwise_equal, bits, f64, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6
M_SWEEP = [1, 2, 3, 7, 16, 33, 64, 255, 256, 1024, 4097, 8192, 16384]


def rms_case(M, d, seed, x_dtype=torch.bfloat16, std=3.0, outliers=True):
    x = synth.normal((M, d), std, seed, dtype=torch.float32)
    if outliers:
        x = synth.with_outliers(x, 0.01, 50.0, seed + 1)
    x = x.to(x_dtype)
    g = synth.uniform((d,), 0.5, 1.5, seed + 2)
    return x, g


def oracle_rms(x, g):
    return oracle.rmsnorm(f64(x), f64(g), EPS)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_parity_tiny_layer_fp32_input(M):
    # fp32 activations x ~ N(0,1), hidden 256, bf16 gamma ~ U(0.5, 1.5)
    x, g = rms_case(M, 256, synth.seed_for(1), torch.float32, std=1.0, outliers=False)
    y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS)
    err = row_rel_err(f64(y), oracle_rms(x, g))
    assert err.max() <= TOL_BF16, err.max()
    yf = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
    assert row_rel_err(f64(yf), oracle_rms(x, g)).max() <= 1e-5


@pytest.mark.parametrize("d", [4096, 5120])
@pytest.mark.parametrize("M", [1, 7, 33, 257])
def test_parity_bf16_rows_with_outliers(M, d):
    x, g = rms_case(M, d, synth.seed_for(3) + M)
    y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS)
    ref = oracle_rms(x, g)
    assert row_rel_err(f64(y), ref).max() <= TOL_BF16
    yf = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
    assert row_rel_err(f64(yf), ref).max() <= 1e-5


@pytest.mark.parametrize("x_dtype,d", [(torch.bfloat16, 8), (torch.bfloat16, 16384),
                                       (torch.float32, 4), (torch.float32, 8192)])
def test_parity_smallest_and_largest_feature_size(x_dtype, d):
    # the feature sizes at the ends of the supported range (d a multiple of 8
    # for bf16 rows, of 4 for fp32, up to 16384 / 8192): against the oracle,
    # and a row's bits the same alone and in a batch of 300
    M = 300
    x, g = rms_case(M, d, synth.seed_for(3) + d, x_dtype)
    y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
    assert row_rel_err(f64(y), oracle_rms(x, g)).max() <= 1e-5
    for r in (0, 151, M - 1):
        alone = binv.rmsnorm(x[r:r + 1].to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
        assert_bitwise_equal(alone, y[r:r + 1], f"row {r} alone vs in the batch, d = {d}")


def test_parity_full_size_sampled_rows():
    M, d = 16384, 4096
    x, g = rms_case(M, d, synth.seed_for(3))
    y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
    rows = np.random.default_rng(0).choice(M, 64, replace=False)
    ref = oracle.rmsnorm(f64(x[rows]), f64(g), EPS)
    assert row_rel_err(f64(y.cpu()[rows]), ref).max() <= 1e-5


def test_zero_rows_and_constant_rows():
    d = 4096
    x = torch.zeros((3, d), dtype=torch.bfloat16)
    x[1] = 2.5
    x[2, 17] = -7.0
    g = torch.ones(d, dtype=torch.bfloat16)
    y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32).cpu()
    assert torch.all(y[0] == 0) and not torch.isnan(y).any()
    ref = oracle_rms(x, g)
    assert row_rel_err(f64(y), ref).max() <= 1e-6


def test_invariance_to_batch_size_and_position():
    d = 4096
    tx, g = rms_case(1, d, synth.TARGET_SEED)
    gd = g.to(DEV)
    alone = binv.rmsnorm(tx.to(DEV), gd, EPS)
    alone32 = binv.rmsnorm(tx.to(DEV), gd, EPS, out_dtype=torch.float32)
    rng = np.random.default_rng(7)
    for M in M_SWEEP:
        x, _ = rms_case(M, d, synth.seed_for(3, trial=M))
        p = int(rng.integers(0, M))
        x[p] = tx[0]
        xd = x.to(DEV)
        y = binv.rmsnorm(xd, gd, EPS)
        assert_bitwise_equal(y[p:p + 1], alone, f"bf16 out, M={M}, row {p}")
        y32 = binv.rmsnorm(xd, gd, EPS, out_dtype=torch.float32)
        assert_bitwise_equal(y32[p:p + 1], alone32, f"fp32 out, M={M}, row {p}")


def test_invariance_d5120_and_fp32_input():
    for d, xdt in [(5120, torch.bfloat16), (256, torch.float32)]:
        tx, g = rms_case(1, d, synth.TARGET_SEED, xdt)
        alone = binv.rmsnorm(tx.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
        for M in [2, 64, 4097]:
            x, _ = rms_case(M, d, synth.seed_for(3, trial=M), xdt)
            x[M - 1] = tx[0]
            y = binv.rmsnorm(x.to(DEV), g.to(DEV), EPS, out_dtype=torch.float32)
            assert_bitwise_equal(y[M - 1:], alone, f"d={d} M={M}")


def test_run_to_run_deterministic():
    x, g = rms_case(4096, 4096, 11)
    xd, gd = x.to(DEV), g.to(DEV)
    a = binv.rmsnorm(xd, gd, EPS, out_dtype=torch.float32)
    b = binv.rmsnorm(xd, gd, EPS, out_dtype=torch.float32)
    assert_bitwise_equal(a, b, "repeat")


def test_tuned_comparator_parity_and_positive_control():
    d = 4096
    tx, g = rms_case(1, d, synth.TARGET_SEED)
    gd = g.to(DEV)
    outs = []
    for M in [1, 256, 8192]:
        x, _ = rms_case(M, d, synth.seed_for(3, trial=M))
        x[0] = tx[0]
        y = binv.rmsnorm(x.to(DEV), gd, EPS, out_dtype=torch.float32, tuned=True)
        assert row_rel_err(f64(y[:1]), oracle_rms(tx, g)).max() <= 1e-5
        outs.append(bits(y[:1]))
    # different M -> different block size -> different reduction tree -> some bit differs
    assert any(not np.array_equal(outs[0], o) for o in outs[1:]), \
        "tuned RMSNorm gave identical bits for every M: the sweep is not sensitive"


def test_ragged_leading_dimension():
    d, ld = 4096, 4096 + 64
    base, g = rms_case(5, ld, 21)
    xd = base.to(DEV)[:, :d]
    out = torch.zeros((5, ld), dtype=torch.float32, device=DEV)
    binv.rmsnorm(xd, g[:d].to(DEV), EPS, out=out[:, :d])
    ref = oracle.rmsnorm(f64(base[:, :d]), f64(g[:d]), EPS)
    assert row_rel_err(f64(out[:, :d]), ref).max() <= 1e-5
    assert torch.all(out[:, d:] == 0)
