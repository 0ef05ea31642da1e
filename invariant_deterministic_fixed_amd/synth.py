"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds data generation and data layout only -- none of the
arithmetic of the kernels or of the oracle.  Values are drawn in fp32 and
stored as bf16 with round-to-nearest-even (torch's conversion), so the GPU
path and the oracle read exactly the same numbers (the oracle decodes them
to fp64).

Seeds: a target row / sequence uses seed 42; neighbour trial t uses 1000 + t;
workload k offsets every seed by 100000 * k.
"""
import math

import numpy as np
import torch

TARGET_SEED = 42
PAGE_SIZE = 16


def seed_for(workload, trial=None):
    base = 100000 * int(workload)
    return base + (TARGET_SEED if trial is None else 1000 + int(trial))


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, device="cpu", dtype=torch.bfloat16):
    """N(0, std^2) samples drawn in fp32, stored as `dtype`."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, lo, hi, seed, device="cpu", dtype=torch.bfloat16):
    g = _gen(seed, device)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(hi - lo).add_(lo)
    return x.to(dtype)


def with_outliers(x, frac, value, seed):
    """Replace each element independently with probability `frac` by +-value (fair sign)."""
    g = _gen(seed, x.device.type)
    u = torch.rand(x.shape, generator=g, device=x.device)
    s = torch.rand(x.shape, generator=g, device=x.device)
    out = x.clone()
    mask = u < frac
    out[mask] = torch.where(s[mask] < 0.5, -value, value).to(x.dtype)
    return out


def log_uniform_lengths(n, lo, hi, seed):
    """round(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    r = np.random.default_rng(int(seed))
    v = np.exp(r.uniform(math.log(lo), math.log(hi), size=int(n)))
    return np.clip(np.rint(v), lo, hi).astype(np.int64)


def uniform_int_lengths(n, lo, hi, seed):
    r = np.random.default_rng(int(seed))
    return r.integers(lo, hi + 1, size=int(n)).astype(np.int64)


# --------------------------------------------------------------------------
# Paged KV cache layout (as declared in include/binv.h):
#   k_cache  [num_pages, Hkv, PAGE_SIZE, D]   token slot, then feature
#   v_cache  [num_pages, Hkv, D, PAGE_SIZE]   feature, then token slot
# logical token t of sequence b lives in page page_table[b, t // PAGE_SIZE],
# slot t % PAGE_SIZE.
# --------------------------------------------------------------------------
class PagedKV:
    """A paged KV cache filled with the given sequences.

    Pages are handed out from a shuffled free list, so physical placement
    changes with `seed`.  Slots past a sequence's length, unused pages and
    unused page-table entries point at NaN-filled memory: any read of them
    that is not masked shows up as NaN in the output.
    """

    def __init__(self, seqs, Hkv, D, seed, spare_pages=3, device="cpu", pt_stride=None):
        self.Hkv, self.D = Hkv, D
        self.lens = np.array([int(k.shape[0]) for k, _ in seqs], dtype=np.int64)
        n_pages = [max(1, -(-int(L) // PAGE_SIZE)) for L in self.lens]
        total = sum(n_pages) + spare_pages + 1           # +1 poison page
        r = np.random.default_rng(int(seed))
        free = r.permutation(total)
        poison = int(free[-1])
        self.num_pages = total
        need = max(n_pages) if n_pages else 1
        self.pt_stride = int(pt_stride) if pt_stride is not None else need + 1
        assert self.pt_stride >= need
        B = len(seqs)
        pt = np.full((max(B, 1), self.pt_stride), poison, dtype=np.int32)
        kc = torch.full((total, Hkv, PAGE_SIZE, D), float("nan"), dtype=torch.bfloat16, device=device)
        vc = torch.full((total, Hkv, D, PAGE_SIZE), float("nan"), dtype=torch.bfloat16, device=device)
        cursor = 0
        for b, (k, v) in enumerate(seqs):
            L = int(k.shape[0])
            n = n_pages[b]
            pages = free[cursor:cursor + n]
            cursor += n
            pt[b, :n] = pages
            if L == 0:
                continue
            pad = n * PAGE_SIZE - L
            kk = k.to(device=device, dtype=torch.bfloat16)
            vv = v.to(device=device, dtype=torch.bfloat16)
            if pad:
                nan_pad = torch.full((pad, Hkv, D), float("nan"), dtype=torch.bfloat16, device=device)
                kk = torch.cat([kk, nan_pad])
                vv = torch.cat([vv, nan_pad])
            idx = torch.as_tensor(pages.astype(np.int64), device=device)
            kc[idx] = kk.view(n, PAGE_SIZE, Hkv, D).permute(0, 2, 1, 3).contiguous()
            vc[idx] = vv.view(n, PAGE_SIZE, Hkv, D).permute(0, 2, 3, 1).contiguous()
        self.k_cache, self.v_cache = kc, vc
        self.page_table = torch.as_tensor(pt, device=device)
        self.kv_lens = torch.as_tensor(self.lens.astype(np.int32), device=device)
        self.poison_page = poison

    def logical(self, b):
        """The sequence's K, V as [L, Hkv, D] tensors, gathered back out of the pages."""
        L = int(self.lens[b])
        n = -(-L // PAGE_SIZE)
        pages = self.page_table[b, :n].long()
        k = self.k_cache[pages].permute(0, 2, 1, 3).reshape(n * PAGE_SIZE, self.Hkv, self.D)[:L]
        v = self.v_cache[pages].permute(0, 3, 1, 2).reshape(n * PAGE_SIZE, self.Hkv, self.D)[:L]
        return k, v

    def to(self, device):
        self.k_cache = self.k_cache.to(device)
        self.v_cache = self.v_cache.to(device)
        self.page_table = self.page_table.to(device)
        self.kv_lens = self.kv_lens.to(device)
        return self


def random_kv(L, Hkv, D, seed, device="cpu", std=1.0):
    k = normal((L, Hkv, D), std, seed, device)
    v = normal((L, Hkv, D), std, seed + 7919, device)
    return k, v
