"""binv_attn_decode_paged_noalloc (decode through the library's fixed partials
buffer, for callers that cannot allocate) against binv_attn_decode_paged on
the same inputs: the outputs must be bitwise equal, on two calls in a row,
the second one smaller, with the output poisoned before each call."""
import math

import pytest
import torch

import invariant_deterministic_fixed_amd as binv
from invariant_deterministic_fixed_amd import binding, synth
from helpers import assert_bitwise_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, Hq, Hkv, D, lo, hi, seed):
    lens = synth.log_uniform_lengths(B, lo, hi, seed)
    seqs = [synth.random_kv(int(L), Hkv, D, seed + 31 * i, DEV) for i, L in enumerate(lens)]
    cache = synth.PagedKV(seqs, Hkv, D, seed + 5, device=DEV)
    q = synth.normal((B, Hq, D), 1.0, seed + 6, DEV)
    return cache, q, int(lens.max())


@pytest.mark.parametrize("shape", [(32, 8, 128), (4, 4, 64)])
def test_noalloc_decode_equals_workspace_decode(shape):
    Hq, Hkv, D = shape
    scale = 1.0 / math.sqrt(D)
    # first call larger than the second, so the second finds the first call's
    # partials in the shared array
    for B, lo, hi, seed in [(24, 128, 20000, 900), (5, 1, 3000, 901)]:
        cache, q, max_kv = _case(B, Hq, Hkv, D, lo, hi, seed)
        print(f"noalloc decode: Hq={Hq} Hkv={Hkv} D={D} B={B} max_kv_len={max_kv}", flush=True)
        ref = binv.attn_decode(q, cache.k_cache, cache.v_cache, cache.page_table, cache.kv_lens,
                               max_kv, scale)
        out = torch.full_like(q, float("nan"))
        binv.attn_decode_noalloc(q, cache.k_cache, cache.v_cache, cache.page_table,
                                 cache.kv_lens, max_kv, scale, out)
        torch.cuda.synchronize()
        assert_bitwise_equal(out, ref, f"B={B}")
        # the same call again on the same array: same bits
        out2 = torch.full_like(q, float("nan"))
        binv.attn_decode_noalloc(q, cache.k_cache, cache.v_cache, cache.page_table,
                                 cache.kv_lens, max_kv, scale, out2)
        torch.cuda.synchronize()
        assert_bitwise_equal(out2, ref, f"B={B}, repeated")


def test_noalloc_decode_rejects_calls_beyond_the_scratch():
    cache, q, _ = _case(2, 32, 8, 128, 128, 256, 902)
    out = torch.empty_like(q)
    with pytest.raises(binding.BinvError, match="SCRATCH"):
        # 2 sequences at the library's longest KV length need 2 x 512 slots of
        # 32 x 130 floats = 34 MB: fits; 64 sequences at 32768 need 136 MB: does not
        big_q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=DEV)
        big_lens = torch.full((64,), 256, dtype=torch.int32, device=DEV)
        big_pt = torch.zeros((64, cache.page_table.shape[1]), dtype=torch.int32, device=DEV)
        binv.attn_decode_noalloc(big_q, cache.k_cache, cache.v_cache, big_pt, big_lens, 32768,
                                 1.0 / math.sqrt(128), torch.empty_like(big_q))
    # a call within the limit still works after the rejected one
    binv.attn_decode_noalloc(q, cache.k_cache, cache.v_cache, cache.page_table, cache.kv_lens,
                             256, 1.0 / math.sqrt(128), out)
    ref = binv.attn_decode(q, cache.k_cache, cache.v_cache, cache.page_table, cache.kv_lens, 256,
                           1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    assert_bitwise_equal(out, ref, "after a rejected call")
