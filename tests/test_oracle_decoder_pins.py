"""Pins for the fp64 reference decoder's own steps (RoPE, SiLU, top-k, the
layer wiring), each against a closed form, an identity or a hand-worked case."""
import math

import numpy as np

import oracle
from oracle import decoder as od


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).normal(size=(1, 3, 8))
    np.testing.assert_array_equal(od.rope(x, [0], 5e5), x)


def test_rope_two_dim_closed_form():
    # D = 2: one pair, frequency theta^0 = 1, angle = position
    out = od.rope(np.array([[[1.0, 0.0]]]), [1], 5e5)
    np.testing.assert_allclose(out[0, 0], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    out = od.rope(np.array([[[0.0, 1.0]]]), [2], 5e5)
    np.testing.assert_allclose(out[0, 0], [-math.sin(2.0), math.cos(2.0)], rtol=1e-15)


def test_rope_preserves_pair_norms_and_uses_relative_positions():
    r = np.random.default_rng(1)
    D = 16
    q, k = r.normal(size=(1, 1, D)), r.normal(size=(1, 1, D))
    qa = od.rope(q, [7], 10000.0)
    n0 = q[0, 0, :8] ** 2 + q[0, 0, 8:] ** 2
    n1 = qa[0, 0, :8] ** 2 + qa[0, 0, 8:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)
    d1 = np.dot(od.rope(q, [9], 10000.0)[0, 0], od.rope(k, [4], 10000.0)[0, 0])
    d2 = np.dot(od.rope(q, [105], 10000.0)[0, 0], od.rope(k, [100], 10000.0)[0, 0])
    assert abs(d1 - d2) < 1e-12 * max(1.0, abs(d1))


def test_silu_identities():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(od.silu(x) - od.silu(-x), x, atol=1e-12)
    assert od.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(od.silu(np.array([40.0]))[0], 40.0, rtol=1e-15)
    np.testing.assert_allclose(od.silu(np.array([1.0]))[0], 1 / (1 + math.exp(-1)), rtol=1e-15)


def test_topk_hand_worked_ties():
    ids, vals = od.topk([1.0, 3.0, 3.0, 2.0, -1.0], 4)
    assert ids.tolist() == [1, 2, 3, 0] and vals.tolist() == [3.0, 3.0, 2.0, 1.0]


def _tiny(seed, zero_mixers=False):
    r = np.random.default_rng(seed)
    cfg = dict(hidden=32, n_heads=4, n_kv=2, head_dim=8, ffn=48, vocab=50, theta=5e5, eps=1e-6)
    H, D, F, V = 32, 8, 48, 50
    bf = lambda a: oracle.round_bf16(a)  # noqa: E731
    layers = []
    for _ in range(2):
        layers.append(dict(wqkv=bf(r.normal(size=(H, (4 + 2 * 2) * D)) * 0.2),
                           wo=np.zeros((4 * D, H)) if zero_mixers else bf(r.normal(size=(4 * D, H)) * 0.2),
                           wgu=bf(r.normal(size=(H, 2 * F)) * 0.2),
                           wd=np.zeros((F, H)) if zero_mixers else bf(r.normal(size=(F, H)) * 0.2)))
    w = dict(embed=bf(r.normal(size=(V, H))), lm_head=bf(r.normal(size=(H, V)) * 0.2), layers=layers)
    return w, cfg


def test_forward_without_mixers_is_norm_then_head():
    # attention and FFN outputs projected by zero matrices leave the residual
    # stream equal to the embedding: logits = bf16(rmsnorm(embed[ids])) @ Wlm
    w, cfg = _tiny(2, zero_mixers=True)
    ids = [3, 7, 7, 49, 0]
    got = od.forward(w, cfg, ids)
    x = oracle.round_bf16(oracle.rmsnorm(w["embed"][ids], np.ones(32), 1e-6))
    np.testing.assert_allclose(got, x @ w["lm_head"], rtol=1e-12, atol=1e-12)


def test_forward_is_causal():
    w, cfg = _tiny(3)
    a = od.forward(w, cfg, [1, 2, 3, 4, 5, 6])
    b = od.forward(w, cfg, [1, 2, 3, 9, 9, 9])
    np.testing.assert_array_equal(a[:3], b[:3])
    assert np.max(np.abs(a[3:] - b[3:])) > 1e-6
