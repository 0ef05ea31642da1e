"""Decoder glue kernels on the GPU against the fp64 reference pieces."""
import numpy as np
import pytest
import torch

import invariant_deterministic_fixed_amd as binv
import oracle
from invariant_deterministic_fixed_amd import synth
from oracle import decoder as od
from helpers import TOL_BF16, assert_bitwise_equal, f64, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_embed_exact_and_out_of_range_rows_zero():
    table = synth.normal((1000, 256), 0.02, 1, DEV)
    ids = torch.tensor([0, 999, 17, -1, 1000, 17], dtype=torch.int32, device=DEV)
    out = binv.embed(ids, table).cpu()
    ref = np.zeros((6, 256))
    for i, t in enumerate([0, 999, 17, None, None, 17]):
        if t is not None:
            ref[i] = f64(table[t])
    np.testing.assert_array_equal(out.double().numpy(), ref)


def test_residual_add_is_the_rounded_fp32_sum():
    h = synth.normal((37, 4096), 1.0, 2, DEV, dtype=torch.float32)
    x = synth.normal((37, 4096), 1.0, 3, DEV)
    want = (f64(h) + f64(x)).astype(np.float32)
    binv.residual_add(h, x)
    np.testing.assert_array_equal(h.cpu().numpy(), want)


@pytest.mark.parametrize("M,d", [(1, 4096), (37, 4096), (300, 256), (5, 8192)])
@pytest.mark.parametrize("g_dt,y_dt", [(torch.bfloat16, torch.bfloat16),
                                       (torch.float32, torch.float32)])
def test_add_rmsnorm_is_residual_add_then_rmsnorm(M, d, g_dt, y_dt):
    # the fused launch gives the bits of the two separate calls, in h and in y
    h0 = synth.normal((M, d), 1.0, 11, DEV, dtype=torch.float32)
    a = synth.normal((M, d), 3.0, 12, DEV)
    gamma = synth.uniform((d,), 0.5, 1.5, 13, DEV).to(g_dt)
    h1, h2 = h0.clone(), h0.clone()
    binv.residual_add(h1, a)
    want = binv.rmsnorm(h1, gamma, 1e-6, out_dtype=y_dt)
    got = binv.add_rmsnorm(h2, a, gamma, 1e-6, out_dtype=y_dt)
    assert_bitwise_equal(h2, h1, "updated residual")
    assert_bitwise_equal(got, want, "norm output")
    # and the norm is the fp64 RMSNorm of the updated rows, to bf16/fp32 rounding
    ref = oracle.rmsnorm(f64(h1), f64(gamma), 1e-6)
    assert row_rel_err(f64(got), ref).max() <= TOL_BF16


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 4, 2)])
def test_rope_and_kv_write(D, Hq, Hkv):
    T = 300
    qkv = synth.normal((T, (Hq + 2 * Hkv) * D), 1.0, 4, DEV)
    pos = np.random.default_rng(5).choice(5000, T, replace=False).astype(np.int32)
    n_pages = 5000 // 16 + 1
    pt = torch.randperm(n_pages, device=DEV).to(torch.int32).view(1, -1)
    kc = torch.zeros((n_pages, Hkv, 16, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((n_pages, Hkv, D, 16), dtype=torch.bfloat16, device=DEV)
    seq = torch.zeros(T, dtype=torch.int32, device=DEV)
    q = binv.rope_kv_write(qkv, seq, torch.from_numpy(pos).to(DEV), Hq, Hkv, D, 5e5, kc, vc, pt)
    x = f64(qkv)
    q_ref = od.rope(x[:, :Hq * D].reshape(T, Hq, D), pos, 5e5)
    k_ref = od.rope(x[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D), pos, 5e5)
    v_ref = x[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    assert row_rel_err(f64(q), q_ref).max() <= TOL_BF16
    # gather back out of the pages in the documented layout
    page = pt[0].cpu().numpy()[pos // 16]
    slot = pos % 16
    kg = kc.cpu()[torch.as_tensor(page.astype(np.int64)), :, torch.as_tensor(slot.astype(np.int64)), :]
    vg = vc.cpu()[torch.as_tensor(page.astype(np.int64)), :, :, torch.as_tensor(slot.astype(np.int64))]
    assert row_rel_err(kg.double().numpy(), k_ref).max() <= TOL_BF16
    np.testing.assert_array_equal(vg.double().numpy(), v_ref)          # v is copied bit for bit
    # bits depend only on (token, position): the same row at another batch slot
    q2 = binv.rope_kv_write(qkv[[7, 3]].contiguous(), seq[:2],
                            torch.from_numpy(pos[[7, 3]]).to(DEV), Hq, Hkv, D, 5e5, kc, vc, pt)
    assert_bitwise_equal(q2[0], q[7], "rope row 7")
    assert_bitwise_equal(q2[1], q[3], "rope row 3")


def test_swiglu_against_fp64():
    gu = synth.normal((64, 2 * 1000), 2.0, 6, DEV)
    out = binv.swiglu(gu)
    g = f64(gu)
    ref = od.silu(g[:, :1000]) * g[:, 1000:]
    assert row_rel_err(f64(out), ref).max() <= TOL_BF16


def test_gather_rows_bit_copy():
    src = synth.normal((50, 4096), 1.0, 7, DEV, dtype=torch.float32)
    idx = torch.tensor([49, 0, 7, 7], dtype=torch.int32, device=DEV)
    out = binv.gather_rows(src, idx)
    assert_bitwise_equal(out, src[[49, 0, 7, 7]], "gather")


def test_topk_exact_with_ties_and_nan():
    x = synth.normal((9, 128256), 3.0, 8, DEV, dtype=torch.float32)
    x[1, 100:140] = 50.0                       # a block of ties above everything else
    x[2, 5] = float("nan")
    x[3, :] = -1.0                             # every entry tied
    # distinct values that all share one exponent: more same-bucket entries than
    # the kernel gathers, so it falls back to radix passes over the whole row
    x[5] = 1.0 + torch.rand(128256, generator=torch.Generator(device=DEV).manual_seed(3),
                            device=DEV)
    # the 20th place falls inside a tie: 10 entries at 100, 30 tied at 99
    x[6, 1000:1010] = 100.0
    x[6, 5000:5030] = 99.0
    # 15 clear winners, then the 20th place inside a tie of scattered entries:
    # 100 of them (picked by index among the gathered entries) and 300 (more
    # than that path ranks; the row falls back to the full radix passes)
    perm = np.random.default_rng(9).permutation(128256)
    for r, n_tie in [(7, 100), (8, 300)]:
        x[r, torch.as_tensor(perm[:15], device=DEV)] = 200.0
        x[r, torch.as_tensor(perm[15:15 + n_tie], device=DEV)] = 150.0
    ids, vals = binv.topk(x, 20)
    xc = x.cpu().numpy()
    for r in range(9):
        row = np.where(np.isnan(xc[r]), -np.inf, xc[r])
        want_ids, want_vals = od.topk(row, 20)
        np.testing.assert_array_equal(ids[r].cpu().numpy(), want_ids)
        np.testing.assert_array_equal(vals[r].cpu().numpy(), want_vals.astype(np.float32))
    assert ids[1].tolist() == list(range(100, 120))
    assert ids[3].tolist() == list(range(20))
    assert ids[6].tolist() == list(range(1000, 1010)) + list(range(5000, 5010))
    for r, n_tie in [(7, 100), (8, 300)]:
        assert ids[r].tolist() == sorted(perm[:15].tolist()) + sorted(perm[15:15 + n_tie].tolist())[:5]


@pytest.mark.parametrize("n,ldx", [(128256, 128256), (50001, 50003), (4099, 4101)])
def test_topk_matches_oracle_across_paths(n, ldx):
    # rows that take each path of the kernel: a thin first bucket (normal
    # logits), a crowded one (uniform values; many share the top 11 key bits),
    # a crowded one with a few exact ties at the 20th place, and rows whose
    # starts are not 16-byte aligned (odd ldx) or whose length is not a
    # multiple of 4
    g = torch.Generator(device=DEV).manual_seed(n)
    x = torch.empty((6, ldx), device=DEV)
    x[0] = torch.randn(ldx, generator=g, device=DEV) * 3.0
    x[1] = torch.randn(ldx, generator=g, device=DEV) * 2.0
    x[2] = torch.rand(ldx, generator=g, device=DEV) * 2 - 1
    x[3] = torch.rand(ldx, generator=g, device=DEV) * 2 - 1
    x[3, 7::97] = 0.99990234375                # every 97th entry: exact ties at the top
    x[4] = torch.rand(ldx, generator=g, device=DEV) * 2 - 1
    x[4, n // 3] = 5.0
    x[5] = -torch.rand(ldx, generator=g, device=DEV)          # all negative
    flat = x.reshape(-1)[: 5 * ldx + n]
    xs = torch.as_strided(flat, (6, n), (ldx, 1))
    ids, vals = binv.topk(xs, 20)
    xc = xs.cpu().numpy()
    for r in range(6):
        want_ids, want_vals = od.topk(xc[r].astype(np.float64), 20)
        np.testing.assert_array_equal(ids[r].cpu().numpy(), want_ids, err_msg=f"row {r}")
        np.testing.assert_array_equal(vals[r].cpu().numpy(), want_vals.astype(np.float32))


def test_topk_long_rows_prefix_then_rest():
    # Rows longer than the kernel's 16384-entry prefix: the prefix's winners and
    # the later entries above their K-th key decide, except where the kernel
    # must fall back to the whole row -- every such case against the oracle.
    n, K, P = 128256, 20, 16384
    g = torch.Generator(device=DEV).manual_seed(77)
    x = torch.randn((7, n), generator=g, device=DEV)
    x[0, P + 5:P + 25] = 50.0                # all 20 winners past the prefix
    x[1, :P] = float("nan")                  # prefix without K valid entries
    x[2] = torch.arange(n, device=DEV, dtype=torch.float32)   # rising: too many candidates
    x[3, :P] = 0.0                           # 300 ties past the prefix at the K-th key
    x[3, 100:120] = 1.0
    x[3, P:] = 0.0
    perm = np.random.default_rng(5).permutation(n - P)[:300] + P
    x[3, torch.as_tensor(perm, device=DEV)] = 2.0
    x[4, :] = 0.0                            # the K-th key of the prefix, again later
    x[4, 3:28] = 7.0
    x[4, P + 1000:P + 1100] = 7.0
    x[5, 17] = 9.0                           # one winner in the prefix, the rest later
    x[5, P + 17::4000] = 8.0
    x[6, n - 1] = 100.0                      # the last entry wins
    ids, vals = binv.topk(x, K)
    xc = x.cpu().numpy()
    for r in range(7):
        row = np.where(np.isnan(xc[r]), -np.inf, xc[r])
        want_ids, want_vals = od.topk(row, K)
        np.testing.assert_array_equal(ids[r].cpu().numpy(), want_ids, err_msg=f"row {r}")
        np.testing.assert_array_equal(vals[r].cpu().numpy(), want_vals.astype(np.float32))
    assert ids[0].tolist() == list(range(P + 5, P + 25))
    assert ids[3].tolist() == sorted(perm.tolist())[:K]
    assert ids[4].tolist() == list(range(3, 23))


def test_topk_signed_zero_and_short_rows():
    x = torch.full((2, 64), float("nan"), device=DEV)
    x[0, :5] = torch.tensor([0.0, -0.0, 1.0, -0.0, 0.0], device=DEV)
    ids, vals = binv.topk(x, 8)
    # five real entries: 1.0 first, then the zeros in index order, then padding
    assert ids[0].tolist() == [2, 0, 1, 3, 4, -1, -1, -1]
    assert torch.isinf(vals[0, 5:]).all() and (vals[0, 5:] < 0).all()
    assert ids[1].tolist() == [-1] * 8
