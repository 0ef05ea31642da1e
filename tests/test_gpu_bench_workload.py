"""The benchmark's own workload, at full size and in the launch configuration
bench.py times: sampled outputs against the fp64 oracle, and two runs of the
step bitwise equal."""
import numpy as np
import pytest
import torch

import bench
import oracle
from helpers import TOL_BF16, assert_bitwise_equal, f64, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def workload():
    w = bench.build_workload("cuda:0")
    bench.run_step(w)
    torch.cuda.synchronize()
    outs = {k: w[k].clone() for k in ["y", "C", "dec_out", "pf_out"]}
    yield w, outs
    del w
    torch.cuda.empty_cache()


def test_step_is_run_to_run_bitwise(workload):
    w, outs = workload
    bench.run_step(w)
    torch.cuda.synchronize()
    for k in outs:
        assert_bitwise_equal(w[k], outs[k], k)


def test_rmsnorm_and_gemm_sampled_rows(workload):
    w, outs = workload
    rows = np.random.default_rng(1).choice(bench.GEMM_M, 24, replace=False)
    rows = np.concatenate([[0, bench.GEMM_M - 1], rows])
    x = f64(w["x"][rows])
    y_ref = oracle.rmsnorm(x, f64(w["gamma"]), 1e-6)
    assert row_rel_err(f64(outs["y"][rows]), y_ref).max() <= TOL_BF16
    c_ref = oracle.gemm(oracle.round_bf16(y_ref), f64(w["W"]))
    assert row_rel_err(f64(outs["C"][rows]), c_ref).max() <= TOL_BF16


def test_decode_sampled_sequences(workload):
    w, outs = workload
    lens = w["dec_lens"]
    picks = [int(np.argmax(lens)), int(np.argmin(lens)), 0, 100, 255]
    q = f64(w["dec_q"])
    for b in picks:
        k, v = w["dec_cache"].logical(b)
        ref = oracle.attention(q[b:b + 1], [int(lens[b]) - 1], f64(k), f64(v), w["scale"])
        assert row_rel_err(f64(outs["dec_out"][b:b + 1]), ref).max() <= TOL_BF16, b


def test_prefill_sampled_rows(workload):
    w, outs = workload
    k, v = w["pf_kv"]
    rows = [0, 1, 255, 256, 2047, 4095]
    ref = oracle.attention(f64(w["pf_q"][rows]), rows, f64(k), f64(v), w["scale"])
    assert row_rel_err(f64(outs["pf_out"][rows]), ref).max() <= TOL_BF16


def test_glue_leg_sampled(workload):
    # the decoder-glue leg as bench.py runs it: RoPE'd queries, SwiGLU rows and
    # the top-20 selection against the fp64 pieces; the gathered rows are exact
    from oracle import decoder as od
    w, _ = workload
    rows = [0, 1000, 4095]
    x = f64(w["qkv"][rows])
    q_ref = od.rope(x[:, :bench.HQ * bench.HD].reshape(3, bench.HQ, bench.HD), rows, bench.THETA)
    assert row_rel_err(f64(w["rope_q"][rows]), q_ref).max() <= TOL_BF16
    g = f64(w["gu"][rows])
    s_ref = od.silu(g[:, :bench.FFN]) * g[:, bench.FFN:]
    assert row_rel_err(f64(w["swi"][rows]), s_ref).max() <= TOL_BF16
    import invariant_deterministic_fixed_amd as binv
    ids, _ = binv.topk(w["logits"], 20)
    lg = w["logits"].cpu().numpy()
    for r in [0, 255]:
        np.testing.assert_array_equal(ids[r].cpu().numpy(), od.topk(lg[r], 20)[0])
    assert_bitwise_equal(w["hl"], w["h"][w["rows"].long()], "gathered rows")
