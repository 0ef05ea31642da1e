"""A dense pre-norm decoder whose every numeric step runs in libbinv.

Host side only: weight allocation, page allocation from a shuffled free list,
the per-step token / position arrays, and the order of library calls.  One
`Decoder.step` runs all layers over a ragged batch of sequences, each
contributing a run of new tokens (a prefill chunk, or one decode token), and
returns the fp32 logits and the exact top-20 of each sequence's last token.

Per layer (residual stream h in fp32; the ops of the pages' three reductions
plus the pointwise glue, devpress.csdn.net explainer of "Defeating
Nondeterminism in LLM Inference", section 3):
    x = rmsnorm(h) -> bf16;  qkv = x @ Wqkv -> bf16
    RoPE on q, k; k and v written into the paged cache
    a = attention over cached + new keys (the unified prefill entry point;
        a decode token is a run of length 1)
    h += a @ Wo;  x = rmsnorm(h);  h += swiglu(x @ Wgu) @ Wd
then logits = rmsnorm(h_last) @ Wlm (fp32) and top-20 by value, ties by index.
RMSNorm weights are 1 (the workload fixes none).
"""
import math

import numpy as np
import torch

from . import binding as B
from .synth import PAGE_SIZE

CONFIG5 = dict(layers=32, hidden=4096, n_heads=32, n_kv=8, head_dim=128, ffn=14336,
               vocab=128256, theta=5e5, eps=1e-6)


def random_weights(cfg, seed, device, std=0.02):
    """bf16 weights ~ N(0, std^2), drawn in fp32 from a seeded generator."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    H, Hq, Hkv, D, F, V = (cfg["hidden"], cfg["n_heads"], cfg["n_kv"], cfg["head_dim"],
                           cfg["ffn"], cfg["vocab"])

    def mk(*shape):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for i in range(0, shape[0], 1024):          # draw in slabs to bound fp32 scratch
            rows = min(1024, shape[0] - i)
            t[i:i + rows] = (torch.randn((rows,) + shape[1:], generator=g, device=device,
                                         dtype=torch.float32) * std).to(torch.bfloat16)
        return t

    w = {"embed": mk(V, H), "layers": []}
    for _ in range(cfg["layers"]):
        w["layers"].append({"wqkv": mk(H, (Hq + 2 * Hkv) * D), "wo": mk(Hq * D, H),
                            "wgu": mk(H, 2 * F), "wd": mk(F, H)})
    w["lm_head"] = mk(H, V)
    w["norm"] = torch.ones(H, dtype=torch.bfloat16, device=device)
    return w


# Rows up to which an invariant product reads the packed copy of a weight
# (measured per shape: the packed product is faster up to 64 rows for the
# QKV, output and down projections, up to 16 for the 28672-wide gate-up
# projection and the LM head, whose many strips favour the row-major kernels
# beyond that).  The bits are the same either way.
PACKED_ROWS = {"wqkv": 64, "wo": 64, "wd": 64, "wgu": 16, "lm_head": 16}


def pack_weights(w):
    """Strip-packed copies (binv_gemm_bf16_pack) of every projection and of the
    LM head, keyed by the row-major tensor's id, for Decoder(packed=...):
    invariant products of up to PACKED_ROWS[name] rows then read them, with
    the bits of the row-major product (the packed entry point runs the same
    per-element chain) at a higher weight stream rate, for one more copy of
    those weights in HBM."""
    ws = [("lm_head", w["lm_head"])] + [(n, lw[n]) for lw in w["layers"]
                                        for n in ("wqkv", "wo", "wgu", "wd")]
    return {id(t): (t, B.gemm_pack(t), PACKED_ROWS[n]) for n, t in ws}


class KVPool:
    """Per-layer paged K/V caches and one host page table shared by all layers.

    Pages are handed out from a free list shuffled by `seed`, so where a
    sequence's pages sit changes from run to run.  A page may belong to several
    sequences (a shared prompt prefix, `share_prefix`); it returns to the free
    list when the last of them is released."""

    def __init__(self, cfg, num_pages, max_seqs, max_len, seed, device):
        Hkv, D = cfg["n_kv"], cfg["head_dim"]
        self.device = device
        self.k = [torch.zeros((num_pages, Hkv, PAGE_SIZE, D), dtype=torch.bfloat16, device=device)
                  for _ in range(cfg["layers"])]
        self.v = [torch.zeros((num_pages, Hkv, D, PAGE_SIZE), dtype=torch.bfloat16, device=device)
                  for _ in range(cfg["layers"])]
        self.free = list(np.random.default_rng(int(seed)).permutation(num_pages))
        self.refs = np.zeros(num_pages, dtype=np.int64)
        self.pps = -(-int(max_len) // PAGE_SIZE)
        self.table = np.zeros((max_seqs, self.pps), dtype=np.int32)
        self.pages = [[] for _ in range(max_seqs)]
        self.used = [False] * max_seqs

    def alloc(self):
        s = self.used.index(False)
        self.used[s] = True
        return s

    def ensure(self, slot, length):
        need = -(-int(length) // PAGE_SIZE)
        if need > self.pps:
            raise ValueError("sequence longer than the pool's max_len")
        while len(self.pages[slot]) < need:
            if not self.free:
                raise RuntimeError("KV pool out of pages")
            p = int(self.free.pop())
            self.refs[p] = 1
            self.table[slot, len(self.pages[slot])] = p
            self.pages[slot].append(p)

    def share_prefix(self, src, dst, n_tokens):
        """Give the empty sequence `dst` the pages that hold tokens [0, n_tokens)
        of `src`, without copying.  n_tokens must be a whole number of pages:
        `dst` then writes its own tokens into pages of its own."""
        n_tokens = int(n_tokens)
        if n_tokens % PAGE_SIZE or n_tokens // PAGE_SIZE > len(self.pages[src]):
            raise ValueError("a shared prefix must cover whole pages that src holds")
        if self.pages[dst]:
            raise ValueError("dst must hold no pages")
        for i, p in enumerate(self.pages[src][:n_tokens // PAGE_SIZE]):
            self.refs[p] += 1
            self.table[dst, i] = p
            self.pages[dst].append(p)

    def release(self, slot):
        for p in self.pages[slot]:
            self.refs[p] -= 1
            if self.refs[p] == 0:
                self.free.append(p)
        self.pages[slot] = []
        self.table[slot] = 0
        self.used[slot] = False


class Decoder:
    """tuned=True swaps in the shape-tuned comparators (not batch-invariant):
    split-K GEMM and block-size-by-M RMSNorm everywhere, and the split-by-batch
    decode attention on steps where every sequence brings one token; prefill
    steps keep the invariant attention, the only prefill kernel there is.  It
    exists to measure what invariance costs.

    step(items, protected=slots) is selective locking (the BlockLock post's
    per-request locking, BlockLock modes): the rows of the protected sequences
    run through the invariant RMSNorm and GEMM, every other row through the
    tuned comparators, and attention stays invariant for all.  A protected
    sequence's bits are then those of an all-invariant run; the others'
    are not batch-invariant.

    packed: pack_weights(weights), or None for row-major weights only; the
    bits are the same either way (products of more than a weight's
    PACKED_ROWS rows read the row-major weights)."""

    def __init__(self, weights, cfg, pool, max_tokens, max_seqs, max_kv_len, topk=20,
                 tuned=False, packed=None):
        self.w, self.cfg, self.pool, self.topk, self.tuned = weights, cfg, pool, topk, tuned
        dev = pool.device
        H, Hq, Hkv, D, F = (cfg["hidden"], cfg["n_heads"], cfg["n_kv"], cfg["head_dim"],
                            cfg["ffn"])
        T = int(max_tokens)
        bf = torch.bfloat16
        self.h = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.x = torch.empty((T, H), dtype=bf, device=dev)
        self.qkv = torch.empty((T, (Hq + 2 * Hkv) * D), dtype=bf, device=dev)
        self.q = torch.empty((T, Hq, D), dtype=bf, device=dev)
        self.a = torch.empty((T, Hq, D), dtype=bf, device=dev)
        self.o = torch.empty((T, H), dtype=bf, device=dev)
        self.gu = torch.empty((T, 2 * F), dtype=bf, device=dev)
        self.s = torch.empty((T, F), dtype=bf, device=dev)
        self.max_kv_len = int(max_kv_len)
        self.ws = torch.empty(B.attn_workspace_bytes(T, Hq, D, self.max_kv_len),
                              dtype=torch.uint8, device=dev)
        self.hl = torch.empty((max_seqs, H), dtype=torch.float32, device=dev)
        self.xl = torch.empty((max_seqs, H), dtype=bf, device=dev)
        self.logits = torch.empty((max_seqs, cfg["vocab"]), dtype=torch.float32, device=dev)
        self.max_tokens, self.max_seqs = T, max_seqs
        self._graphs = {}
        self._packed = packed if packed is not None else {}

    def step(self, items, protected=None, on_layer=None, graph=False):
        """items: list of (slot, new token ids, start position).  Returns
        (logits fp32 [n, V], top ids int32 [n, k], top values fp32 [n, k]) for
        the last token of each item, as device tensors, in item order.
        protected: a set of slots to run locked (see the class note).
        on_layer(i, h): called with the residual stream h [T, H] (fp32, device,
        the step's tokens in item order) before layer i and, with i = the
        layer count, after the last layer -- for tests that check one layer at
        a time.  After the call, self.hl / self.xl hold the last tokens'
        residual rows and their final-norm output (bf16), rows in item order
        unless `protected` reordered them.
        graph: run a decode step (one new token per item) as a HIP graph: the
        step's kernels are captured once per batch signature (sequence count,
        locked rows) and replayed with the step's inputs copied into the
        graph's own input buffer; the same kernels with the same arguments,
        so the same bits as the eager step, without the per-launch host work.
        The returned tensors then belong to the graph and are overwritten by
        its next replay."""
        prep = self._prepare(items, protected)
        if graph and on_layer is None and prep["max_q"] == 1:
            out = self._replay(prep)
        else:
            dv = torch.from_numpy(prep["host"]).to(self.pool.device)
            out = self._launch(dv, prep, on_layer)
        order = prep["order"]
        if order is not None:                     # back to the caller's item order
            inv = torch.as_tensor(np.argsort(order), device=self.pool.device)
            return tuple(t[inv] for t in out)
        return out

    def _prepare(self, items, protected):
        """Host side of a step: page allocation and the step's int32 inputs
        (token ids, token -> sequence, positions, cu, KV lengths, last-token
        rows, page-table rows) as one array."""
        pool = self.pool
        order, n_prot, t_prot = None, 0, 0
        if protected is not None:
            # protected sequences first, so their rows form one leading block
            order = sorted(range(len(items)), key=lambda i: items[i][0] not in protected)
            items = [items[i] for i in order]
            n_prot = sum(1 for slot, _, _ in items if slot in protected)
            t_prot = sum(len(t) for _, t, _ in items[:n_prot])
        # sequence b of this step reads row b of the step's page table: the
        # attention entry points and the KV write both address pages by the
        # sequence's index in the call, not by its pool slot
        ids, tseq, tpos, cu, lens = [], [], [], [0], []
        for b, (slot, toks, start) in enumerate(items):
            pool.ensure(slot, start + len(toks))
            ids.extend(int(t) for t in toks)
            tseq.extend([b] * len(toks))
            tpos.extend(range(start, start + len(toks)))
            cu.append(cu[-1] + len(toks))
            lens.append(start + len(toks))
        T, nb = len(ids), len(items)
        if T > self.max_tokens or nb > self.max_seqs or max(lens) > self.max_kv_len:
            raise ValueError("step larger than the decoder was sized for")
        rows = pool.table[[slot for slot, _, _ in items]]
        host = np.concatenate([np.array(ids + tseq + tpos + cu + lens + [c - 1 for c in cu[1:]],
                                        dtype=np.int32), rows.reshape(-1)])
        return dict(host=host, T=T, nb=nb, max_q=max(len(t) for _, t, _ in items),
                    order=order, locked=protected is not None, n_prot=n_prot, t_prot=t_prot)

    def _launch(self, dv, prep, on_layer=None):
        """Every kernel of a step, on the current stream, reading the step's
        inputs from the device array dv (laid out as _prepare's host array)."""
        cfg, pool = self.cfg, self.pool
        T, nb, max_q = prep["T"], prep["nb"], prep["max_q"]
        locked, n_prot, t_prot = prep["locked"], prep["n_prot"], prep["t_prot"]
        H, Hq, Hkv, D, F = (cfg["hidden"], cfg["n_heads"], cfg["n_kv"], cfg["head_dim"],
                            cfg["ffn"])
        ids_d, tseq_d, tpos_d = dv[:T], dv[T:2 * T], dv[2 * T:3 * T]
        cu_d = dv[3 * T:3 * T + nb + 1]
        lens_d = dv[3 * T + nb + 1:3 * T + 2 * nb + 1]
        last_d = dv[3 * T + 2 * nb + 1:3 * T + 3 * nb + 1]
        table = dv[3 * T + 3 * nb + 1:].view(nb, pool.pps)
        h, x, qkv, q, a, o, gu, s = (t[:T] for t in (self.h, self.x, self.qkv, self.q, self.a,
                                                     self.o, self.gu, self.s))
        scale = 1.0 / math.sqrt(D)
        tn = self.tuned
        decode_only = tn and max_q == 1

        def split(n_lead):
            # (rows, tuned) blocks: leading protected rows invariant, the rest tuned
            if not locked:
                return [(slice(0, None), tn)]
            return [(sl, t) for sl, t, n in ((slice(0, n_lead), False, n_lead),
                                             (slice(n_lead, None), True, 1)) if n > 0]

        rows_tok = split(t_prot if locked else 0)

        def norm(src, dst, blocks):
            for sl, t in blocks:
                if src[sl].shape[0]:
                    B.rmsnorm(src[sl], self.w["norm"], cfg["eps"], out=dst[sl], tuned=t)

        def mm(src, wt, dst, blocks):
            pk = self._packed.get(id(wt))
            for sl, t in blocks:
                n = src[sl].shape[0]
                if n and pk is not None and not t and n <= pk[2]:
                    B.gemm_packed(src[sl], pk[1], out=dst[sl])
                elif n:
                    B.gemm(src[sl], wt, out=dst[sl], tuned=t)

        def add_norm(dst, blocks):
            # h += o, then dst = norm(h): one fused launch when every row is
            # invariant (the bits of the two separate calls)
            if len(blocks) == 1 and not blocks[0][1]:
                B.add_rmsnorm(h, o, self.w["norm"], cfg["eps"], out=dst)
            else:
                B.residual_add(h, o)
                norm(h, dst, blocks)

        B.embed(ids_d, self.w["embed"], out=h)
        n_layers = len(self.w["layers"])
        for li, lw in enumerate(self.w["layers"]):
            if on_layer is not None:
                on_layer(li, h)
            if li == 0:
                norm(h, x, rows_tok)
            mm(x, lw["wqkv"], qkv, rows_tok)
            B.rope_kv_write(qkv, tseq_d, tpos_d, Hq, Hkv, D, cfg["theta"], pool.k[li], pool.v[li],
                            table, q_out=q)
            if decode_only:
                B.attn_decode(q, pool.k[li], pool.v[li], table, lens_d, self.max_kv_len, scale,
                              out=a, tuned=True)
            else:
                B.attn_prefill(q, cu_d, pool.k[li], pool.v[li], table, lens_d, max_q,
                               self.max_kv_len, scale, out=a, workspace=self.ws)
            mm(a.view(T, Hq * D), lw["wo"], o, rows_tok)
            add_norm(x, rows_tok)
            mm(x, lw["wgu"], gu, rows_tok)
            B.swiglu(gu, out=s)
            mm(s, lw["wd"], o, rows_tok)
            if li + 1 < n_layers:
                add_norm(x, rows_tok)            # and the next layer's input norm
            else:
                B.residual_add(h, o)
        if on_layer is not None:
            on_layer(len(self.w["layers"]), h)
        hl, xl, logits = self.hl[:nb], self.xl[:nb], self.logits[:nb]
        rows_seq = split(n_prot if locked else 0)
        B.gather_rows(h, last_d, out=hl)
        norm(hl, xl, rows_seq)
        mm(xl, self.w["lm_head"], logits, rows_seq)
        top_ids, top_vals = B.topk(logits, self.topk)
        return logits, top_ids, top_vals

    def _replay(self, prep):
        """A decode step as a HIP graph: captured on the first step of its
        signature (sequence count and locked block; the inputs' layout then
        has a fixed size), replayed after the step's inputs are copied into
        the graph's input array."""
        key = (prep["nb"], prep["locked"], prep["n_prot"], prep["t_prot"])
        host = torch.from_numpy(prep["host"])
        g = self._graphs.get(key)
        if g is None:
            dv = torch.empty(host.shape, dtype=torch.int32, device=self.pool.device)
            dv.copy_(host)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):             # one eager run first (lazy set-up)
                self._launch(dv, prep)
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                outs = self._launch(dv, prep)
            g = self._graphs[key] = (graph, dv, outs,
                                     torch.empty(host.shape, dtype=torch.int32).pin_memory())
        graph, dv, outs, pinned = g
        # the previous replay has read the pinned array before it is refilled
        torch.cuda.current_stream().synchronize()
        pinned.copy_(host)
        dv.copy_(pinned, non_blocking=True)
        graph.replay()
        return outs
