"""libbinv: batch-invariant RMSNorm, GEMM and paged attention for MI355X (gfx950).

The kernels are hand-written HIP in ``csrc/`` behind the C ABI of
``include/binv.h``; ``binding`` marshals torch tensors into those calls.
"""
from .binding import (BINV_BF16, BINV_F32, BinvError, PackedWeight,  # noqa: F401
                      add_rmsnorm, attn_decode, attn_decode_noalloc, attn_prefill,
                      attn_prefill_workspace_bytes, attn_workspace_bytes, embed, gather_rows,
                      gemm, gemm_pack, gemm_packed, lib, residual_add, rmsnorm, rope_kv_write,
                      split_bf16x3, status_str, swiglu, topk, version)
