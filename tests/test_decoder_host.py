"""Host-side logic of the decoder's paged KV pool (no GPU): page hand-out,
prefix sharing with reference counts, release."""
import pytest

from invariant_deterministic_fixed_amd import decoder as dec
from invariant_deterministic_fixed_amd.synth import PAGE_SIZE

CFG = dict(layers=1, n_kv=1, head_dim=64)


def pool(num_pages=8, max_seqs=4, max_len=64):
    return dec.KVPool(CFG, num_pages=num_pages, max_seqs=max_seqs, max_len=max_len, seed=1,
                      device="cpu")


def test_pages_come_from_a_shuffled_free_list_and_return():
    p = pool()
    a = p.alloc()
    p.ensure(a, 3 * PAGE_SIZE + 1)
    assert len(p.pages[a]) == 4 and len(set(p.pages[a])) == 4
    assert list(p.table[a, :4]) == p.pages[a]
    assert len(p.free) == 4
    p.release(a)
    assert len(p.free) == 8 and not p.used[a] and not p.pages[a]


def test_shared_prefix_pages_are_freed_by_the_last_owner():
    p = pool()
    a, b = p.alloc(), p.alloc()
    p.ensure(a, 2 * PAGE_SIZE + 5)                      # 3 pages
    p.share_prefix(a, b, 2 * PAGE_SIZE)                 # b shares a's first 2 pages
    assert p.pages[b] == p.pages[a][:2]
    assert list(p.table[b, :2]) == p.pages[a][:2]
    p.ensure(b, 2 * PAGE_SIZE + 1)                      # b's next token gets a page of its own
    assert p.pages[b][2] not in p.pages[a]
    shared = p.pages[a][:2]
    p.release(a)
    assert not any(s in p.free for s in shared)         # still held by b
    assert p.pages[a] == [] and len(p.free) == 8 - 2 - 1
    p.release(b)
    assert sorted(p.free) == list(range(8))


def test_share_prefix_rejects_partial_pages_and_nonempty_targets():
    p = pool()
    a, b = p.alloc(), p.alloc()
    p.ensure(a, 2 * PAGE_SIZE)
    with pytest.raises(ValueError):
        p.share_prefix(a, b, PAGE_SIZE + 3)            # not a whole number of pages
    with pytest.raises(ValueError):
        p.share_prefix(a, b, 3 * PAGE_SIZE)            # more than a holds
    p.ensure(b, 1)
    with pytest.raises(ValueError):
        p.share_prefix(a, b, PAGE_SIZE)                # b already holds pages


def test_pool_exhaustion_is_an_error():
    p = pool(num_pages=2)
    a = p.alloc()
    with pytest.raises(RuntimeError):
        p.ensure(a, 3 * PAGE_SIZE)
