"""fp64 reference decoder (pre-norm, Llama-style) for the end-to-end check.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Shares no code with the
HIP library.  Inputs are numpy arrays holding the bf16 weight values decoded to
fp64.

What it computes, per the decoder workload (random-init dense decoder with
grouped-query attention, SwiGLU FFN and RoPE) and the pages' point that every
reduction in it is one of RMSNorm / matmul / attention (devpress.csdn.net
explainer of "Defeating Nondeterminism in LLM Inference", section 3):

  h = embedding[ids]                                   (residual stream, fp64)
  per layer:
    x  = bf16(rmsnorm(h))            qkv = bf16(x @ Wqkv)
    q, k = bf16(rope(q)), bf16(rope(k))   (rotate-half, angle p * theta^(-2i/D))
    a  = bf16(causal GQA attention(q, k, v))
    h  = h + bf16(a @ Wo)
    x  = bf16(rmsnorm(h))            gu = bf16(x @ Wgu)
    h  = h + bf16( bf16(silu(g) * u) @ Wd )
  logits = bf16(rmsnorm(h)) @ Wlm                      (fp64, not rounded)

bf16(.) rounds to bf16 exactly where the GPU path stores bf16 (the tensors
named in ROUNDED_IN_LAYER and ROUNDED_AT_END); everything else is fp64.  RMSNorm
weights are 1.  The model is a pure function of the token list: logits at
position p use tokens 0..p only (no cache, no batching).  `layer` is one
decoder layer on its own, so a test can feed it the GPU's own residual stream
(teacher forcing) and compare one layer at a time.
"""
import math

import numpy as np

from . import attention, gemm, rmsnorm, round_bf16


def rope(x, pos, theta):
    """Rotate-half rotary embedding.  x [n, H, D] at positions pos [n]:
    x'[i] = x[i] cos a - x[i + D/2] sin a,  x'[i + D/2] = x[i + D/2] cos a + x[i] sin a,
    a = pos * theta^(-2i/D), i < D/2."""
    x = np.asarray(x, dtype=np.float64)
    n, H, D = x.shape
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]          # [n, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(g):
    """g * sigmoid(g) = g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def topk(row, k):
    """The k largest entries, by value descending, equal values by index ascending."""
    row = np.asarray(row)
    order = sorted(range(len(row)), key=lambda i: (-row[i], i))[:k]
    return np.array(order, dtype=np.int64), row[order]


# The tensors the GPU decoder stores in bf16, in the order one layer forms
# them (then the final norm's output): bf16(.) is applied to exactly these.
ROUNDED_IN_LAYER = ("x_attn", "qkv", "q_rope", "k_rope", "attn", "o_proj",
                    "x_mlp", "gate_up", "swiglu", "down_proj")
ROUNDED_AT_END = ("x_final",)


def _bf16(x, tag):
    return round_bf16(x)


def layer(lw, cfg, h, rnd=_bf16):
    """One decoder layer over the tokens at positions 0 .. n-1 of one sequence
    (a prefill of the whole list: each token attends to itself and the tokens
    before it).  h: residual stream [n, H] (fp64); returns the new residual.
    rnd(x, tag) rounds the tensor named `tag` (ROUNDED_IN_LAYER) to bf16."""
    n = h.shape[0]
    H, Hq, Hkv, D, F = cfg["hidden"], cfg["n_heads"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    eps, theta = cfg["eps"], cfg["theta"]
    ones = np.ones(H)
    pos = np.arange(n)
    x = rnd(rmsnorm(h, ones, eps), "x_attn")
    qkv = rnd(gemm(x, lw["wqkv"]), "qkv")
    q = qkv[:, :Hq * D].reshape(n, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    q = rnd(rope(q, pos, theta), "q_rope")
    k = rnd(rope(k, pos, theta), "k_rope")
    a = rnd(attention(q, pos, k, v, 1.0 / math.sqrt(D)), "attn")
    h = h + rnd(gemm(a.reshape(n, Hq * D), lw["wo"]), "o_proj")
    x = rnd(rmsnorm(h, ones, eps), "x_mlp")
    gu = rnd(gemm(x, lw["wgu"]), "gate_up")
    s = rnd(silu(gu[:, :F]) * gu[:, F:], "swiglu")
    return h + rnd(gemm(s, lw["wd"]), "down_proj")


def logits_of(weights, cfg, h, rnd=_bf16):
    """Final RMSNorm of the residual rows h [n, H], then the LM head (fp64, not rounded)."""
    x = rnd(rmsnorm(h, np.ones(cfg["hidden"]), cfg["eps"]), "x_final")
    return gemm(x, weights["lm_head"])


def forward(weights, cfg, ids, rnd=_bf16, last=None):
    """Logits [n, V] at every position of the token list `ids` (fp64); with
    last = m only those of the last m positions.  weights["layers"] may be a
    list, or a callable i -> layer weights (to hold one layer at a time)."""
    ids = np.asarray(ids, dtype=np.int64)
    h = np.asarray(weights["embed"][ids], dtype=np.float64)
    layers = weights["layers"]
    n_layers = cfg.get("layers", None) if callable(layers) else len(layers)
    for i in range(n_layers):
        lw = layers(i) if callable(layers) else layers[i]
        h = layer(lw, cfg, h, rnd)
    if last is not None:
        h = h[-int(last):]
    return logits_of(weights, cfg, h, rnd)
