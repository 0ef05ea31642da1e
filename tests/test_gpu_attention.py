"""Paged decode / prefill attention on the GPU: parity with the fp64 oracle,
closed forms, bitwise invariance of a target sequence to its batch
neighbours, batch position and page placement, and bitwise equality of
one-shot prefill, chunked prefill and decode."""
import math

import numpy as np
import pytest
import torch

import invariant_deterministic_fixed_amd as binv
import invariant_deterministic_fixed_amd.binding as bd
import oracle
from invariant_deterministic_fixed_amd import synth
from helpers import TOL_BF16, assert_bitwise_equal, f64, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make_cache(lens, Hkv, D, seed, device=DEV, seqs=None, pt_stride=None):
    if seqs is None:
        seqs = [synth.random_kv(int(L), Hkv, D, seed + 17 * i, device) for i, L in enumerate(lens)]
    return synth.PagedKV(seqs, Hkv, D, seed, device=device, pt_stride=pt_stride), seqs


def decode(cache, q, scale, max_kv_len=None, **kw):
    mkl = int(max_kv_len or max(int(x) for x in cache.lens))
    return binv.attn_decode(q, cache.k_cache, cache.v_cache, cache.page_table, cache.kv_lens,
                            mkl, scale, **kw)


def oracle_decode(q, seqs, lens, scale):
    outs = []
    for b, (k, v) in enumerate(seqs):
        L = int(lens[b])
        outs.append(oracle.attention(f64(q[b:b + 1]), [L - 1], f64(k), f64(v), scale)[0])
    return np.stack(outs)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_decode_parity_tiny(B):
    Hq = Hkv = 4
    D = 64
    lens = synth.uniform_int_lengths(B, 1, 300, synth.seed_for(1) + B)
    cache, seqs = make_cache(lens, Hkv, D, synth.seed_for(1) + B)
    q = synth.normal((B, Hq, D), 1.0, 77 + B, DEV)
    scale = 1 / math.sqrt(D)
    out = decode(cache, q, scale)
    ref = oracle_decode(q, seqs, lens, scale)
    err = row_rel_err(f64(out), ref)
    assert err.max() <= TOL_BF16, err.max()


@pytest.mark.parametrize("lens", [[1, 255, 256, 257], [1000, 5000, 16, 4096], [32768]])
def test_decode_parity_gqa_shape(lens):
    Hq, Hkv, D = 32, 8, 128
    cache, seqs = make_cache(lens, Hkv, D, synth.seed_for(4) + len(lens))
    q = synth.normal((len(lens), Hq, D), 1.0, 5, DEV)
    scale = 1 / math.sqrt(D)
    out = decode(cache, q, scale)
    assert torch.isfinite(out.float()).all()
    ref = oracle_decode(q, seqs, lens, scale)
    err = row_rel_err(f64(out), ref)
    assert err.max() <= TOL_BF16, err.max()


def test_decode_single_key_returns_v0_bitwise():
    Hq, Hkv, D = 8, 2, 128
    cache, seqs = make_cache([1, 1, 1], Hkv, D, 3)
    q = synth.normal((3, Hq, D), 1.0, 4, DEV)
    out = decode(cache, q, 0.1).cpu()
    for b in range(3):
        v0 = seqs[b][1][0].cpu()                       # [Hkv, D]
        for h in range(Hq):
            assert_bitwise_equal(out[b, h], v0[h // (Hq // Hkv)], f"b={b} h={h}")


def test_decode_two_token_closed_form():
    # D = 64, scale = 1/8: q = e0, k0 = 0, k1 = 8 e0 -> scores [0, 1] -> weights
    # [1 - s(1), s(1)] with s the logistic function; v0 = e0, v1 = e1
    D, Hq, Hkv = 64, 1, 1
    k = torch.zeros((2, 1, D), dtype=torch.bfloat16); k[1, 0, 0] = 8.0
    v = torch.zeros((2, 1, D), dtype=torch.bfloat16); v[0, 0, 0] = 1.0; v[1, 0, 1] = 1.0
    cache, _ = make_cache([2], Hkv, D, 1, seqs=[(k.to(DEV), v.to(DEV))])
    q = torch.zeros((1, Hq, D), dtype=torch.bfloat16, device=DEV); q[0, 0, 0] = 1.0
    out = f64(decode(cache, q, 1 / 8))[0, 0]
    w1 = 1 / (1 + math.exp(-1))
    assert abs(out[0] - (1 - w1)) < 4e-3 and abs(out[1] - w1) < 4e-3
    assert np.all(out[2:] == 0)


def test_decode_all_keys_equal_gives_mean_of_v():
    Hq, Hkv, D, L = 4, 1, 128, 700
    k = synth.normal((1, Hkv, D), 1.0, 8).expand(L, Hkv, D).contiguous()
    v = synth.normal((L, Hkv, D), 1.0, 9)
    cache, _ = make_cache([L], Hkv, D, 2, seqs=[(k.to(DEV), v.to(DEV))])
    q = synth.normal((1, Hq, D), 1.0, 10, DEV)
    out = f64(decode(cache, q, 0.09))[0]
    mean = f64(v)[:, 0].mean(axis=0)
    assert row_rel_err(out, np.broadcast_to(mean, out.shape)).max() <= 1e-2


def test_decode_invariance_to_neighbours_position_and_pages():
    Hq, Hkv, D = 32, 8, 128
    scale = 1 / math.sqrt(D)
    L_t = 3000
    tk, tv = synth.random_kv(L_t, Hkv, D, synth.TARGET_SEED, DEV)
    tq = synth.normal((1, Hq, D), 1.0, synth.TARGET_SEED + 1, DEV)
    cache, _ = make_cache([L_t], Hkv, D, 1, seqs=[(tk, tv)])
    alone = decode(cache, tq, scale)
    ref = oracle_decode(tq, [(tk, tv)], [L_t], scale)
    assert row_rel_err(f64(alone), ref).max() <= TOL_BF16
    rng = np.random.default_rng(2024)
    plan = [(1, 32768), (7, 32768), (31, 32768), (255, 32768), (int(rng.integers(2, 200)), 4096)]
    for trial, (n, hi) in enumerate(plan):
        lens = synth.log_uniform_lengths(n, 128, hi, synth.seed_for(4, trial))
        pos = int(rng.integers(0, n + 1))
        seqs = [synth.random_kv(int(L), Hkv, D, synth.seed_for(4, trial) + 31 * i, DEV)
                for i, L in enumerate(lens)]
        seqs.insert(pos, (tk, tv))
        all_lens = [int(k.shape[0]) for k, _ in seqs]
        cache, _ = make_cache(all_lens, Hkv, D, synth.seed_for(4, trial) + 5, seqs=seqs)
        q = synth.normal((n + 1, Hq, D), 1.0, synth.seed_for(4, trial) + 6, DEV)
        q[pos] = tq[0]
        out = decode(cache, q, scale, max_kv_len=max(all_lens) + 100)
        assert_bitwise_equal(out[pos:pos + 1], alone, f"trial {trial}: {n} neighbours, pos {pos}")
        assert torch.isfinite(out.float()).all()
        del cache, seqs, out
        torch.cuda.empty_cache()


def test_decode_run_to_run_deterministic():
    lens = [4000, 200, 9000]
    cache, _ = make_cache(lens, 8, 128, 44)
    q = synth.normal((3, 32, 128), 1.0, 45, DEV)
    a = decode(cache, q, 0.088)
    b = decode(cache, q, 0.088)
    assert_bitwise_equal(a, b, "repeat")


def _prefill(cache, q, cu_q, kv_lens, max_q_len, max_kv_len, scale):
    return binv.attn_prefill(q, torch.as_tensor(cu_q, dtype=torch.int32, device=DEV),
                             cache.k_cache, cache.v_cache, cache.page_table,
                             torch.as_tensor(kv_lens, dtype=torch.int32, device=DEV),
                             max_q_len, max_kv_len, scale)


def test_prefill_parity_ragged_batch():
    Hq, Hkv, D = 8, 2, 128
    lens = [300, 17, 1000, 600]
    qlens = [300, 5, 33, 1]          # one-shot, tails of cached sequences, single token
    cache, seqs = make_cache(lens, Hkv, D, 61)
    T = sum(qlens)
    q = synth.normal((T, Hq, D), 1.0, 62, DEV)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    scale = 1 / math.sqrt(D)
    out = _prefill(cache, q, cu, lens, max(qlens), max(lens), scale)
    for b in range(len(lens)):
        k, v = seqs[b]
        pos = [lens[b] - qlens[b] + i for i in range(qlens[b])]
        ref = oracle.attention(f64(q[cu[b]:cu[b + 1]]), pos, f64(k), f64(v), scale)
        err = row_rel_err(f64(out[cu[b]:cu[b + 1]]), ref)
        assert err.max() <= TOL_BF16, (b, err.max())


def test_prefill_chunked_and_decode_bitwise_equal():
    Hq, Hkv, D, L = 32, 8, 128, 4096
    scale = 1 / math.sqrt(D)
    k, v = synth.random_kv(L, Hkv, D, synth.seed_for(4), DEV)
    cache, _ = make_cache([L], Hkv, D, 9, seqs=[(k, v)])
    q = synth.normal((L, Hq, D), 1.0, synth.seed_for(4) + 1, DEV)
    one_shot = _prefill(cache, q, [0, L], [L], L, L, scale)
    for step in [256, 512, 2048]:
        parts = []
        for s in range(0, L, step):
            e = min(L, s + step)
            parts.append(_prefill(cache, q[s:e].contiguous(), [0, e - s], [e], e - s, L, scale))
        assert_bitwise_equal(torch.cat(parts), one_shot, f"chunked prefill, chunk {step}")
    # decode of every position at once: 4096 "sequences" sharing the one page table
    pt = cache.page_table[:1].expand(L, -1).contiguous()
    kv_lens = torch.arange(1, L + 1, dtype=torch.int32, device=DEV)
    dec = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt, kv_lens, L, scale)
    assert_bitwise_equal(dec, one_shot, "decode vs prefill")
    # sampled oracle parity
    rows = [0, 1, 255, 256, 257, 1000, 2048, 4095]
    ref = oracle.attention(f64(q[rows]), rows, f64(k), f64(v), scale)
    assert row_rel_err(f64(one_shot[rows]), ref).max() <= TOL_BF16


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (4, 4, 64), (3, 3, 128), (5, 5, 64)])
def test_decode_tree_levels_equal_prefill_leaves(Hq, Hkv, D):
    # Decode hands a row's partials to the merge kernel as nodes of one, two or
    # four chunks depending on its chunk count; prefill always hands over
    # leaves.  Every decode position must equal the one-shot prefill of the
    # same position bit for bit.  The merge puts 2 (D = 128) or 4 (D = 64)
    # (token, head) rows in one wave: with an odd head count those rows belong
    # to different tokens with different node counts.
    L = 34 * 256 - 100
    scale = 1 / math.sqrt(D)
    k, v = synth.random_kv(L, Hkv, D, 91, DEV)
    cache, _ = make_cache([L], Hkv, D, 92, seqs=[(k, v)])
    q = synth.normal((L, Hq, D), 1.0, 93, DEV)
    one_shot = _prefill(cache, q, [0, L], [L], L, L, scale)
    rng = np.random.default_rng(94)
    edges = [0, 1, 255, 256, 4095, 4096, 4351, 4352, 4607, 8191, 8192, 8447, 8448, L - 1]
    rows = np.unique(np.concatenate([edges, rng.integers(0, L, 200)])).astype(np.int64)
    pt = cache.page_table[:1].expand(len(rows), -1).contiguous()
    kv_lens = torch.as_tensor(rows + 1, dtype=torch.int32, device=DEV)
    qr = q[torch.as_tensor(rows, device=DEV)].contiguous()
    dec = binv.attn_decode(qr, cache.k_cache, cache.v_cache, pt, kv_lens, L, scale)
    assert_bitwise_equal(dec, one_shot[torch.as_tensor(rows, device=DEV)], "decode vs prefill")
    sample = [0, 4096, 8447, L - 1]
    ref = oracle.attention(f64(q[sample]), sample, f64(k), f64(v), scale)
    assert row_rel_err(f64(one_shot[sample]), ref).max() <= TOL_BF16


def test_decode_long_rows_every_node_level_equal_leaves():
    # Rows of 1 .. 130 chunks: decode hands them over as leaves, pairs or
    # nodes of four chunks (the level follows the row's chunk count); the
    # same rows as one-token prefill sequences are merged from leaves.  Both
    # must give the same bits; a few rows against the oracle.
    Hq, Hkv, D = 32, 8, 128
    L = 130 * 256 - 100
    scale = 1 / math.sqrt(D)
    k, v = synth.random_kv(L, Hkv, D, 95, DEV)
    cache, _ = make_cache([L], Hkv, D, 96, seqs=[(k, v)])
    rng = np.random.default_rng(97)
    edges = [0, 255, 256] + [256 * n + d for n in (16, 32, 48, 64, 96, 112, 128) for d in (-1, 0)]
    rows = np.unique(np.concatenate([edges, rng.integers(0, L, 100), [L - 1]])).astype(np.int64)
    n = len(rows)
    qr = synth.normal((n, Hq, D), 1.0, 98, DEV)
    pt = cache.page_table[:1].expand(n, -1).contiguous()
    kv_lens = torch.as_tensor(rows + 1, dtype=torch.int32, device=DEV)
    dec = binv.attn_decode(qr, cache.k_cache, cache.v_cache, pt, kv_lens, L, scale)
    leaves = binv.attn_prefill(qr, torch.arange(n + 1, dtype=torch.int32, device=DEV),
                               cache.k_cache, cache.v_cache, pt, kv_lens, 1, L, scale)
    assert_bitwise_equal(dec, leaves, "decode nodes vs prefill leaves")
    for i in [0, int(np.searchsorted(rows, 256 * 97)), n - 1]:
        p = int(rows[i])
        ref = oracle.attention(f64(qr[i:i + 1]), [p], f64(k), f64(v), scale)
        assert row_rel_err(f64(dec[i:i + 1]), ref).max() <= TOL_BF16, p


def test_longest_rows_and_max_kv_len_bound_change_no_bits():
    # max_kv_len only sizes the grid and the workspace: rows of up to 70000
    # keys (274 chunks, so the merge's binary counter uses nine slots) give
    # the same bits under three bounds -- the longest row, 300 chunks and the
    # library's maximum -- through decode (nodes of up to four chunks) and
    # through one-token prefill (leaves); two rows against the oracle.
    Hq, Hkv, D = 32, 8, 128
    L = 70000
    scale = 1 / math.sqrt(D)
    k, v = synth.random_kv(L, Hkv, D, 131, DEV)
    cache, _ = make_cache([L], Hkv, D, 132, seqs=[(k, v)])
    rows = np.array([0, 255, 256, 40000, 65279, 65280, 65535, L - 1], dtype=np.int64)
    n = len(rows)
    qr = synth.normal((n, Hq, D), 1.0, 133, DEV)
    pt = cache.page_table[:1].expand(n, -1).contiguous()
    kv_lens = torch.as_tensor(rows + 1, dtype=torch.int32, device=DEV)
    cu = torch.arange(n + 1, dtype=torch.int32, device=DEV)
    outs = []
    for bound in (L, 300 * 256, bd.MAX_KV_LEN):
        outs.append(binv.attn_decode(qr, cache.k_cache, cache.v_cache, pt, kv_lens, bound, scale))
        outs.append(binv.attn_prefill(qr, cu, cache.k_cache, cache.v_cache, pt, kv_lens, 1,
                                      bound, scale))
    for i, o in enumerate(outs[1:], 1):
        assert_bitwise_equal(o, outs[0], f"output {i} vs decode under the tightest bound")
    for i in (3, n - 1):
        p = int(rows[i])
        ref = oracle.attention(f64(qr[i:i + 1]), [p], f64(k), f64(v), scale)
        assert row_rel_err(f64(outs[0][i:i + 1]), ref).max() <= TOL_BF16, p


def test_decode_at_the_maximum_batch():
    # B = 65535, the largest batch the decode entry point takes: 48 distinct
    # sequences of 1 .. 48 keys, each shared by the page-table rows of ~1365
    # batch rows.  Sampled rows against the oracle, and against the same row
    # decoded alone, bit for bit.
    Hq, Hkv, D = 32, 8, 128
    B = 65535
    base_lens = list(range(1, 49))
    cache, seqs = make_cache(base_lens, Hkv, D, 151)
    s_of = np.arange(B) % len(base_lens)
    pt = cache.page_table[torch.as_tensor(s_of, device=DEV)].contiguous()
    kv = torch.as_tensor(np.array(base_lens)[s_of], dtype=torch.int32, device=DEV)
    q = synth.normal((B, Hq, D), 1.0, 152, DEV)
    scale = 1 / math.sqrt(D)
    out = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt, kv, 48, scale)
    for b in (0, 1, 47, 48, 12345, 40000, B - 2, B - 1):
        s = int(s_of[b])
        k, v = seqs[s]
        ref = oracle.attention(f64(q[b:b + 1]), [base_lens[s] - 1], f64(k), f64(v), scale)
        assert row_rel_err(f64(out[b:b + 1]), ref).max() <= TOL_BF16, b
        alone = binv.attn_decode(q[b:b + 1].contiguous(), cache.k_cache, cache.v_cache,
                                 pt[b:b + 1].contiguous(), kv[b:b + 1].contiguous(), 48, scale)
        assert_bitwise_equal(alone, out[b:b + 1], f"row {b} alone vs in the batch")


def test_rows_at_the_maximum_kv_length():
    # A sequence of the library's maximum length fills all 512 leaves of the
    # merge tree.  Its last 128 positions as one prefill run (block kernel,
    # the deepest stack of pending subtrees) and as decode rows (nodes of up
    # to four chunks, then the merge over every level) give the same bits;
    # a middle row and the last row of the run against the oracle.
    Hq, Hkv, D = 32, 8, 128
    L = bd.MAX_KV_LEN
    scale = 1 / math.sqrt(D)
    k, v = synth.random_kv(L, Hkv, D, 141, DEV)
    cache, _ = make_cache([L], Hkv, D, 142, seqs=[(k, v)])
    n = 128
    q = synth.normal((n, Hq, D), 1.0, 143, DEV)
    pre = _prefill(cache, q, np.array([0, n], dtype=np.int32), [L], n, L, scale)
    pos = np.arange(L - n, L, dtype=np.int64)
    pt = cache.page_table[:1].expand(n, -1).contiguous()
    kv = torch.as_tensor(pos + 1, dtype=torch.int32, device=DEV)
    dec = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt, kv, L, scale)
    assert_bitwise_equal(dec, pre, "decode vs prefill at the maximum length")
    kd, vd = f64(k), f64(v)
    for i in (n // 2, n - 1):
        ref = oracle.attention(f64(q[i:i + 1]), [int(pos[i])], kd, vd, scale)
        assert row_rel_err(f64(pre[i:i + 1]), ref).max() <= TOL_BF16, i


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (32, 2)])
def test_prefill_head_groups_parity_and_decode_bitwise(Hq, Hkv):
    # D = 128 prefill blocks hold 128 / G tokens: G = 1, 8 and 16 besides the
    # G = 4 of the other tests; ragged batch with cached prefixes
    D = 128
    lens = [300, 17, 1000, 600]
    qlens = [300, 5, 133, 1]
    cache, seqs = make_cache(lens, Hkv, D, 71 + Hq)
    T = sum(qlens)
    q = synth.normal((T, Hq, D), 1.0, 72 + Hq, DEV)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    scale = 1 / math.sqrt(D)
    out = _prefill(cache, q, cu, lens, max(qlens), max(lens), scale)
    for b, (k, v) in enumerate(seqs):
        pos = [lens[b] - qlens[b] + i for i in range(qlens[b])]
        ref = oracle.attention(f64(q[cu[b]:cu[b + 1]]), pos, f64(k), f64(v), scale)
        assert row_rel_err(f64(out[cu[b]:cu[b + 1]]), ref).max() <= TOL_BF16, b
    # every prefill row equals the decode of the same position, bit for bit
    b_of = np.repeat(np.arange(len(lens)), qlens)
    pos_of = np.concatenate([[lens[b] - qlens[b] + i for i in range(qlens[b])] for b in range(len(lens))])
    pt = cache.page_table[torch.as_tensor(b_of, device=DEV)].contiguous()
    kv = torch.as_tensor(pos_of + 1, dtype=torch.int32, device=DEV)
    dec = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt, kv, max(lens), scale)
    assert_bitwise_equal(dec, out, "decode vs prefill")


@pytest.mark.parametrize("lens,qlens", [
    ([2000], [700]),                            # one sequence: pending subtrees only
    ([3000], [300]),                            # one sequence, few blocks: chunk-pair nodes
    ([700], [700]),                             # the same with a lone last chunk
    ([20000], [500]),                           # few blocks over 79 chunks: stacks again
    ([1500, 900, 300], [400, 7, 300]),          # leaves of short runs indexed per sequence
    ([1024] * 40, [100] + [1] * 39),            # leaves indexed per token, stacks among them
])
def test_prefill_workspace_layouts(lens, qlens):
    # The workspace of a prefill call is laid out by its shape: stacks of the
    # merge tree's pending subtrees for rows of long runs, one leaf per chunk
    # for rows of short runs.  With a workspace of exactly the reported size,
    # filled with NaN, every row equals the decode of its position bit for bit
    # (a slot read before it is written would carry the NaN into the output).
    Hq, Hkv, D = 32, 8, 128
    cache, seqs = make_cache(lens, Hkv, D, 91 + len(lens))
    T = sum(qlens)
    q = synth.normal((T, Hq, D), 1.0, 92 + len(lens), DEV)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    scale = 1 / math.sqrt(D)
    need = binv.attn_prefill_workspace_bytes(len(lens), T, max(qlens), max(lens), Hq, Hkv, D)
    assert 0 < need <= binv.attn_workspace_bytes(T, Hq, D, max(lens))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    out = binv.attn_prefill(q, torch.as_tensor(cu, dtype=torch.int32, device=DEV), cache.k_cache,
                            cache.v_cache, cache.page_table,
                            torch.as_tensor(lens, dtype=torch.int32, device=DEV), max(qlens),
                            max(lens), scale, workspace=ws)
    assert bool(torch.isfinite(out.float()).all())
    b_of = np.repeat(np.arange(len(lens)), qlens)
    pos_of = np.concatenate([[lens[b] - qlens[b] + i for i in range(qlens[b])]
                             for b in range(len(lens))])
    pt = cache.page_table[torch.as_tensor(b_of, device=DEV)].contiguous()
    kv = torch.as_tensor(pos_of + 1, dtype=torch.int32, device=DEV)
    dec = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt, kv, max(lens), scale)
    assert_bitwise_equal(dec, out, "decode vs prefill")
    # sampled rows against the oracle: first, last and a middle row of each run
    for b, (k, v) in enumerate(seqs[:3]):
        n = qlens[b]
        for i in sorted({0, n // 2, n - 1}):
            r = int(cu[b]) + i
            ref = oracle.attention(f64(q[r:r + 1]), [lens[b] - n + i], f64(k), f64(v), scale)
            assert row_rel_err(f64(out[r:r + 1]), ref).max() <= TOL_BF16, (b, i)


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (32, 2)])
def test_prefill_short_and_long_query_runs_bitwise_equal(Hq, Hkv):
    # At D = 128 a prefill call whose longest new-token run fills less than
    # half a 128-row block (an engine's decode steps, a few-token tail) runs
    # on the looping one-tile chunk kernel, a longer one on the block kernel.
    # The last rows of a long-run call must equal the same rows from short-run
    # calls (one token each, and the longest run just below the threshold).
    D = 128
    G = Hq // Hkv
    lens = [300, 17, 1000, 600, 4100]
    cache, seqs = make_cache(lens, Hkv, D, 81 + Hq)
    scale = 1 / math.sqrt(D)
    long_q = [160, 5, 333, 1, 260]
    T = sum(long_q)
    q = synth.normal((T, Hq, D), 1.0, 82 + Hq, DEV)
    cu = np.concatenate([[0], np.cumsum(long_q)]).astype(np.int32)
    assert max(long_q) * G >= 64
    out_long = _prefill(cache, q, cu, lens, max(long_q), max(lens), scale)
    # one token per sequence: each sequence's last position
    last = torch.as_tensor(cu[1:] - 1, dtype=torch.long, device=DEV)
    q1 = q[last].contiguous()
    out_one = _prefill(cache, q1, np.arange(len(lens) + 1, dtype=np.int32), lens, 1,
                       max(lens), scale)
    assert_bitwise_equal(out_one, out_long[last], "one-token prefill vs block prefill")
    # the longest run just below the threshold: the last k tokens of each sequence
    k_run = max(1, (64 - 1) // G)
    assert k_run * G < 64
    short_q = [min(k_run, n) for n in long_q]
    idx = np.concatenate([np.arange(cu[b + 1] - short_q[b], cu[b + 1]) for b in range(len(lens))])
    idx_t = torch.as_tensor(idx, dtype=torch.long, device=DEV)
    cu_s = np.concatenate([[0], np.cumsum(short_q)]).astype(np.int32)
    out_short = _prefill(cache, q[idx_t].contiguous(), cu_s, lens, max(short_q), max(lens), scale)
    assert_bitwise_equal(out_short, out_long[idx_t], "short-run prefill vs block prefill")
    # a call whose max_q_len overstates its runs (one sequence, 5 new tokens,
    # bound 200): the short run is still computed, by the chunk kernel
    b4 = 4
    rows5 = torch.arange(int(cu[b4 + 1]) - 5, int(cu[b4 + 1]), device=DEV)
    cache4, _ = make_cache([lens[b4]], Hkv, D, 0, seqs=[seqs[b4]])
    out5 = _prefill(cache4, q[rows5].contiguous(), [0, 5], [lens[b4]], 200, max(lens), scale)
    assert_bitwise_equal(out5, out_long[rows5], "overstated max_q_len")
    # sequences with no new tokens in a long-run call: the others' rows unchanged
    zq = [long_q[0], 0, long_q[2], 0, long_q[4]]
    keep = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in (0, 2, 4)])
    keep_t = torch.as_tensor(keep, dtype=torch.long, device=DEV)
    cu_z = np.concatenate([[0], np.cumsum(zq)]).astype(np.int32)
    out_z = _prefill(cache, q[keep_t].contiguous(), cu_z, lens, max(zq), max(lens), scale)
    assert_bitwise_equal(out_z, out_long[keep_t], "zero-length runs in a mixed call")
    # and the oracle on the one-token rows
    for b, (kk, vv) in enumerate(seqs):
        ref = oracle.attention(f64(q1[b:b + 1]), [lens[b] - 1], f64(kk), f64(vv), scale)
        assert row_rel_err(f64(out_one[b:b + 1]), ref).max() <= TOL_BF16, b


def test_prefill_tile_positions_do_not_change_bits():
    # the same tokens prefilled at different offsets inside the 16-row tiles
    Hq, Hkv, D, L = 32, 8, 128, 777
    scale = 0.09
    k, v = synth.random_kv(L, Hkv, D, 12, DEV)
    cache, _ = make_cache([L], Hkv, D, 13, seqs=[(k, v)])
    q = synth.normal((L, Hq, D), 1.0, 14, DEV)
    ref = _prefill(cache, q, [0, L], [L], L, L, scale)
    for s in [1, 2, 3, 5, 333]:
        part = _prefill(cache, q[s:].contiguous(), [0, L - s], [L], L - s, L, scale)
        assert_bitwise_equal(part, ref[s:], f"offset {s}")


def test_mha_tiny_head_dim_64_prefill_and_decode():
    Hq = Hkv = 4
    D, L = 64, 300
    k, v = synth.random_kv(L, Hkv, D, 15, DEV)
    cache, _ = make_cache([L], Hkv, D, 16, seqs=[(k, v)])
    q = synth.normal((L, Hq, D), 1.0, 17, DEV)
    pf = _prefill(cache, q, [0, L], [L], L, L, 0.125)
    pt = cache.page_table[:1].expand(L, -1).contiguous()
    dec = binv.attn_decode(q, cache.k_cache, cache.v_cache, pt,
                           torch.arange(1, L + 1, dtype=torch.int32, device=DEV), L, 0.125)
    assert_bitwise_equal(dec, pf, "decode vs prefill, D=64")
    ref = oracle.attention(f64(q), list(range(L)), f64(k), f64(v), 0.125)
    assert row_rel_err(f64(pf), ref).max() <= TOL_BF16


def test_tuned_decode_parity_and_positive_control():
    # the shape-tuned comparator must be right (oracle) and must NOT be
    # invariant: a long target's bits change with the batch size
    Hq, Hkv, D = 32, 8, 128
    scale = 1 / math.sqrt(D)
    L_t = 20000
    tk, tv = synth.random_kv(L_t, Hkv, D, synth.TARGET_SEED, DEV)
    tq = synth.normal((1, Hq, D), 1.0, synth.TARGET_SEED + 1, DEV)
    cache, _ = make_cache([L_t], Hkv, D, 1, seqs=[(tk, tv)])
    alone = decode(cache, tq, scale, tuned=True)
    ref = oracle_decode(tq, [(tk, tv)], [L_t], scale)
    assert row_rel_err(f64(alone), ref).max() <= TOL_BF16
    lens = synth.log_uniform_lengths(255, 128, 4096, 77)
    seqs = [synth.random_kv(int(L), Hkv, D, 500 + i, DEV) for i, L in enumerate(lens)] + [(tk, tv)]
    cache, _ = make_cache([int(k.shape[0]) for k, _ in seqs], Hkv, D, 3, seqs=seqs)
    q = synth.normal((256, Hq, D), 1.0, 9, DEV)
    q[255] = tq[0]
    out = decode(cache, q, scale, max_kv_len=L_t, tuned=True)
    inv = decode(cache, q, scale, max_kv_len=L_t)
    for b in [0, 100, 255]:
        k, v = seqs[b]
        r = oracle_decode(q[b:b + 1], [(k, v)], [int(k.shape[0])], scale)
        assert row_rel_err(f64(out[b:b + 1]), r).max() <= TOL_BF16
    # same sequences in batches of 8: the tuned split count changes with B, and
    # over ~1M bf16 outputs some bits must move (one sequence's 4096 outputs
    # usually hide a 1-ulp fp32 change under bf16 rounding)
    sub = []
    for b0 in range(0, 256, 8):
        part = make_cache([int(k.shape[0]) for k, _ in seqs[b0:b0 + 8]], Hkv, D, 11 + b0,
                          seqs=seqs[b0:b0 + 8])[0]
        sub.append(decode(part, q[b0:b0 + 8].contiguous(), scale, max_kv_len=L_t, tuned=True))
    sub = torch.cat(sub)
    assert not torch.equal(sub.view(torch.int16), out.view(torch.int16)), \
        "tuned decode gave identical bits for B=8 and B=256: the probe is not sensitive"
    inv_alone = decode(make_cache([L_t], Hkv, D, 1, seqs=[(tk, tv)])[0], tq, scale)
    assert_bitwise_equal(inv[255:], inv_alone, "invariant decode, same probe")
