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

bf16(.) rounds to bf16 exactly where the GPU path stores bf16; everything else
is fp64.  RMSNorm weights are 1.  The model is a pure function of the token
list: logits at position p use tokens 0..p only (no cache, no batching).
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


def forward(weights, cfg, ids):
    """Logits [n, V] at every position of the token list `ids` (fp64)."""
    ids = np.asarray(ids, dtype=np.int64)
    n = len(ids)
    H, Hq, Hkv, D, F = cfg["hidden"], cfg["n_heads"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    eps, theta = cfg["eps"], cfg["theta"]
    ones = np.ones(H)
    pos = np.arange(n)
    h = weights["embed"][ids].astype(np.float64)
    for layer in weights["layers"]:
        x = round_bf16(rmsnorm(h, ones, eps))
        qkv = round_bf16(gemm(x, layer["wqkv"]))
        q = qkv[:, :Hq * D].reshape(n, Hq, D)
        k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
        q = round_bf16(rope(q, pos, theta))
        k = round_bf16(rope(k, pos, theta))
        a = round_bf16(attention(q, pos, k, v, 1.0 / math.sqrt(D)))
        h = h + round_bf16(gemm(a.reshape(n, Hq * D), layer["wo"]))
        x = round_bf16(rmsnorm(h, ones, eps))
        gu = round_bf16(gemm(x, layer["wgu"]))
        s = round_bf16(silu(gu[:, :F]) * gu[:, F:])
        h = h + round_bf16(gemm(s, layer["wd"]))
    x = round_bf16(rmsnorm(h, ones, eps))
    return gemm(x, weights["lm_head"])
