"""The two fp32 -> bf16 conversions the kernels use are round to nearest even
on every input.

The GEMM, RMSNorm, glue and attention outputs round with f32_to_bf16 (one
value); every attention kernel rounds its softmax weights with p_pack (a pair,
gfx950's v_cvt_pk_bf16_f32).  Decode and prefill form the same intermediates
only with the same rounding everywhere (tom-jerr.github.io "Batch-Invariant
Kernel", Flash Attention: prefill and decode intermediates bit-identical), and
the oracle rounds to nearest even.  A test-only kernel
(tests/gpu_support/conv_check.hip, built by the package build) runs both, and
the round-to-nearest-even rule written out from the format's definition, over
all 2^32 bit patterns, NaNs included."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_support", "libconvcheck.so")


def test_bf16_conversions_agree_on_all_2_32_inputs():
    assert os.path.exists(LIB), "tests/gpu_support/libconvcheck.so missing: run the package build"
    lib = ctypes.CDLL(LIB)
    lib.conv_check_all_inputs.restype = ctypes.c_int
    lib.conv_check_all_inputs.argtypes = [ctypes.c_void_p] * 3
    counts = torch.full((3 * 65536,), 0xFFFF, dtype=torch.int32, device="cuda:0")
    first = torch.zeros(65536, dtype=torch.int32, device="cuda:0")
    st = lib.conv_check_all_inputs(ctypes.c_void_p(counts.data_ptr()),
                                   ctypes.c_void_p(first.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    c = counts.cpu().numpy().astype(np.int64).reshape(-1, 3)
    pair_vs_scalar, scalar_vs_rule, pair_hi_vs_rule = (int(x) for x in c.sum(axis=0))
    f = first.cpu().numpy().view(np.uint32)
    bad = f[f != 0xFFFFFFFF]
    print(f"mismatches over 2^32 inputs: pair (low half) vs scalar {pair_vs_scalar}, scalar vs "
          f"rule {scalar_vs_rule}, pair (high half) vs rule {pair_hi_vs_rule}", flush=True)
    assert (pair_vs_scalar, scalar_vs_rule, pair_hi_vs_rule) == (0, 0, 0), \
        f"first differing inputs: {[hex(int(x)) for x in bad[:8]]}"
