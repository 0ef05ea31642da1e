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


# ---------------------------------------------------------------------------
# Layer wiring against an independent implementation of the same architecture:
# the Llama decoder of the transformers library (pre-norm RMSNorm, rotate-half
# RoPE, grouped-query attention with query head h reading KV head h // G,
# SwiGLU silu(gate) * up, untied LM head), in fp64 on the CPU with the same
# weights.  Nothing of the oracle is shared with it.

HF_CFG = dict(layers=2, hidden=64, n_heads=4, n_kv=2, head_dim=16, ffn=96, vocab=50, theta=5e5,
              eps=1e-6)


def _hf_weights(seed):
    r = np.random.default_rng(seed)
    c = HF_CFG
    H, Hq, Hkv, D, F, V = c["hidden"], c["n_heads"], c["n_kv"], c["head_dim"], c["ffn"], c["vocab"]
    bf = oracle.round_bf16
    layers = [dict(wqkv=bf(r.normal(size=(H, (Hq + 2 * Hkv) * D)) * 0.2),
                   wo=bf(r.normal(size=(Hq * D, H)) * 0.2),
                   wgu=bf(r.normal(size=(H, 2 * F)) * 0.2),
                   wd=bf(r.normal(size=(F, H)) * 0.2)) for _ in range(c["layers"])]
    return dict(embed=bf(r.normal(size=(V, H))), lm_head=bf(r.normal(size=(H, V)) * 0.2),
                layers=layers)


def _hf_model(w, monkeypatch=None, rnd=None):
    """transformers' LlamaForCausalLM holding the weights `w` (fp64).  With
    `rnd`, forward hooks round to bf16 at the boundaries the GPU decoder stores
    in bf16 (RMSNorm outputs, projection outputs, rotated q / k, the attention
    output, the SwiGLU product), and RMSNorm and the rotary angles are
    evaluated in fp64 instead of the library's fp32."""
    import torch
    from transformers import LlamaConfig, LlamaForCausalLM
    from transformers.models.llama import modeling_llama as ml

    c = HF_CFG
    H, Hq, Hkv, D, F = c["hidden"], c["n_heads"], c["n_kv"], c["head_dim"], c["ffn"]
    cfg = LlamaConfig(vocab_size=c["vocab"], hidden_size=H, intermediate_size=F,
                      num_hidden_layers=c["layers"], num_attention_heads=Hq,
                      num_key_value_heads=Hkv, head_dim=D, rms_norm_eps=c["eps"],
                      rope_theta=c["theta"], tie_word_embeddings=False, attention_bias=False,
                      mlp_bias=False, max_position_embeddings=64, attn_implementation="sdpa")
    torch.manual_seed(0)
    m = LlamaForCausalLM(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(w["embed"]))
        m.lm_head.weight.copy_(t(w["lm_head"].T))
        m.model.norm.weight.fill_(1.0)
        for lw, L in zip(w["layers"], m.model.layers):
            a = L.self_attn
            a.q_proj.weight.copy_(t(lw["wqkv"][:, :Hq * D].T))
            a.k_proj.weight.copy_(t(lw["wqkv"][:, Hq * D:(Hq + Hkv) * D].T))
            a.v_proj.weight.copy_(t(lw["wqkv"][:, (Hq + Hkv) * D:].T))
            a.o_proj.weight.copy_(t(lw["wo"].T))
            L.mlp.gate_proj.weight.copy_(t(lw["wgu"][:, :F].T))
            L.mlp.up_proj.weight.copy_(t(lw["wgu"][:, F:].T))
            L.mlp.down_proj.weight.copy_(t(lw["wd"].T))
            L.input_layernorm.weight.fill_(1.0)
            L.post_attention_layernorm.weight.fill_(1.0)
    if rnd is None:
        return m

    def r(x):
        return torch.from_numpy(rnd(x.detach().numpy()))

    def out_hook(mod, inp, out):
        return r(out)

    def in_hook(mod, inp):
        return (r(inp[0]),) + tuple(inp[1:])

    def norm64(self, hidden_states):        # the library's expression, without its fp32 cast
        variance = hidden_states.pow(2).mean(-1, keepdim=True)
        return self.weight * (hidden_states * torch.rsqrt(variance + self.variance_epsilon))

    def rope64(x, position_ids):             # the library's angles, in fp64
        base, dim = c["theta"], D
        inv = 1.0 / (base ** (torch.arange(0, dim, 2, dtype=torch.float64) / dim))
        freqs = position_ids[:, :, None].double() * inv[None, None, :]
        emb = torch.cat((freqs, freqs), dim=-1)
        return emb.cos(), emb.sin()

    plain_rope = ml.apply_rotary_pos_emb

    def rope_rounded(q, k, cos, sin, unsqueeze_dim=1):
        qe, ke = plain_rope(q, k, cos, sin, unsqueeze_dim)
        return r(qe), r(ke)

    monkeypatch.setattr(ml.LlamaRMSNorm, "forward", norm64)
    monkeypatch.setattr(ml, "apply_rotary_pos_emb", rope_rounded)
    m.model.rotary_emb.forward = rope64
    for L in m.model.layers:
        for mod in (L.input_layernorm, L.post_attention_layernorm, L.self_attn.q_proj,
                    L.self_attn.k_proj, L.self_attn.v_proj, L.self_attn.o_proj,
                    L.mlp.gate_proj, L.mlp.up_proj, L.mlp.down_proj):
            mod.register_forward_hook(out_hook)
        L.self_attn.o_proj.register_forward_pre_hook(in_hook)      # attention output
        L.mlp.down_proj.register_forward_pre_hook(in_hook)         # silu(gate) * up
    m.model.norm.register_forward_hook(out_hook)
    return m


def _hf_logits(m, ids):
    import torch
    with torch.no_grad():
        return m(torch.tensor([ids])).logits[0].double().numpy()


def _rel(a, b):
    return float(np.max(np.max(np.abs(a - b), axis=1) / np.max(np.abs(b), axis=1)))


IDS = [3, 17, 17, 42, 0, 9, 31, 8, 49, 22, 5]


def test_forward_wiring_equals_transformers_llama_unrounded():
    # with every bf16 rounding switched off the oracle is a plain fp64 Llama
    # decoder; the library evaluates RMSNorm and the rotary angles in fp32, so
    # agreement is to ~1e-6, while a wiring mistake (RoPE on v, gate and up
    # swapped, a wrong q / k / v column split or GQA head map) moves the
    # logits by 1e-1 or more
    w = _hf_weights(11)
    got = od.forward(w, HF_CFG, IDS, rnd=lambda x, tag: x)
    ref = _hf_logits(_hf_model(w), IDS)
    err = _rel(got, ref)
    assert err < 2e-5, err
    # planted mistakes in the weights handed to the oracle are caught
    F, D, Hq, Hkv = HF_CFG["ffn"], HF_CFG["head_dim"], HF_CFG["n_heads"], HF_CFG["n_kv"]
    swapped = dict(w, layers=[dict(l, wgu=np.concatenate([l["wgu"][:, F:], l["wgu"][:, :F]], 1))
                              for l in w["layers"]])
    assert _rel(od.forward(swapped, HF_CFG, IDS, rnd=lambda x, tag: x), ref) > 1e-2
    kv = (Hq + Hkv) * D
    kv_swapped = dict(w, layers=[dict(l, wqkv=np.concatenate(
        [l["wqkv"][:, :Hq * D], l["wqkv"][:, kv:], l["wqkv"][:, Hq * D:kv]], 1))
        for l in w["layers"]])
    assert _rel(od.forward(kv_swapped, HF_CFG, IDS, rnd=lambda x, tag: x), ref) > 1e-2


def test_forward_rounding_points_equal_transformers_llama_with_bf16_hooks(monkeypatch):
    # the same library model with bf16 rounding hooked in at the tensors the
    # GPU decoder stores in bf16, and fp64 arithmetic everywhere else: the
    # oracle must agree to fp64 rounding; skipping any one of its roundings
    # (a moved rounding point) must not
    w = _hf_weights(12)
    ref = _hf_logits(_hf_model(w, monkeypatch, rnd=oracle.round_bf16), IDS)
    got = od.forward(w, HF_CFG, IDS)
    assert _rel(got, ref) < 1e-9, _rel(got, ref)
    unrounded = od.forward(w, HF_CFG, IDS, rnd=lambda x, tag: x)
    assert _rel(unrounded, ref) > 1e-4
    for skip in od.ROUNDED_IN_LAYER + od.ROUNDED_AT_END:
        mutated = od.forward(w, HF_CFG, IDS,
                             rnd=lambda x, tag, skip=skip: x if tag == skip else oracle.round_bf16(x))
        assert _rel(mutated, ref) > 1e-4, f"skipping the rounding of {skip} went unnoticed"


def test_forward_rounds_exactly_the_listed_tensors_in_order():
    w, cfg = _tiny(4)
    cfg = dict(cfg, layers=2)
    seen = []

    def rec(x, tag):
        seen.append((tag, x.shape))
        return oracle.round_bf16(x)

    od.forward(w, cfg, [1, 2, 3], rnd=rec)
    tags = [t for t, _ in seen]
    assert tags == list(od.ROUNDED_IN_LAYER) * 2 + list(od.ROUNDED_AT_END)
    shapes = dict(seen)
    assert shapes["qkv"] == (3, (4 + 2 * 2) * 8) and shapes["q_rope"] == (3, 4, 8)
    assert shapes["k_rope"] == (3, 2, 8) and shapes["attn"] == (3, 4, 8)
    assert shapes["gate_up"] == (3, 96) and shapes["swiglu"] == (3, 48)
    assert shapes["x_final"] == (3, 32)


def test_layer_of_one_token_returns_v_through_wo():
    # position 0 sees one key, so attention returns that token's v exactly
    # (per query head, the v of its KV head); RoPE at position 0 is the
    # identity.  With the FFN weights zero, the layer adds bf16(a @ Wo) with
    # a = [v of KV head h // 2 for query heads h = 0..3]
    w, cfg = _tiny(5)
    lw = dict(w["layers"][0], wd=np.zeros((48, 32)))
    h = w["embed"][[7]]
    x = oracle.round_bf16(oracle.rmsnorm(h, np.ones(32), 1e-6))
    qkv = oracle.round_bf16(x @ lw["wqkv"])
    v = qkv[0, (4 + 2) * 8:].reshape(2, 8)
    a = np.concatenate([v[0], v[0], v[1], v[1]])[None, :]
    expect = h + oracle.round_bf16(a @ lw["wo"])
    np.testing.assert_array_equal(od.layer(lw, cfg, h), expect)
