"""Layer chains with bf16 or fp32 activations: the fp32-activation mitigation.

The devpress.csdn.net explainer of "Defeating Nondeterminism in LLM Inference"
(sections 2 and 6) names a second remedy beside batch-invariant kernels: keep
the weights in bf16 but carry the activations in fp32.  A reduction-order
change then perturbs results at fp32 granularity instead of flipping bf16
roundings; it narrows the differences without making them zero.

``chain`` applies x <- rmsnorm(x) @ W_l for the given weights, either way:
  "bf16": rmsnorm writes bf16, the GEMM reads it and writes bf16 (activations
          rounded at every tensor boundary, as in the decoder);
  "fp32": rmsnorm reads and writes fp32; ``split_bf16x3`` turns the fp32
          activations into [hi | mid | lo] bf16 parts that add back to them
          exactly, and the GEMM contracts those against [W; W; W] with fp32
          output: exact products, one fp32 accumulator per element (3x the
          matrix-core work of the bf16 chain).
Either way the kernels are the batch-invariant ones, or with ``tuned`` the
shape-tuned comparators, whose reduction order follows the batch.
"""
import torch

from . import binding as B


def stack3(w):
    """[W; W; W] for a bf16 weight W [K, N], the operand of the fp32 chain."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2
    return torch.cat([w, w, w], dim=0).contiguous()


def chain(x, weights, gamma, mode="bf16", tuned=False, eps=1e-6, weights3=None):
    """Final activations of the chain for the rows of x (fp32 or bf16 [M, d]).

    weights: bf16 [d, d] each (used by "bf16"); weights3: their ``stack3``
    (used by "fp32", computed here when not given).  gamma: RMSNorm weight [d].
    Returns bf16 ("bf16") or fp32 ("fp32") [M, d]."""
    if mode == "bf16":
        h = x.to(torch.bfloat16).contiguous()
        for w in weights:
            y = B.rmsnorm(h, gamma, eps, out_dtype=torch.bfloat16, tuned=tuned)
            h = B.gemm(y, w, out_dtype=torch.bfloat16, tuned=tuned)
        return h
    if mode == "fp32":
        if weights3 is None:
            weights3 = [stack3(w) for w in weights]
        h = x.to(torch.float32).contiguous()
        for w3 in weights3:
            y = B.rmsnorm(h, gamma, eps, out_dtype=torch.float32, tuned=tuned)
            h = B.gemm(B.split_bf16x3(y), w3, out_dtype=torch.float32, tuned=tuned)
        return h
    raise ValueError(f"mode must be 'bf16' or 'fp32', not {mode!r}")
