"""Invariance harness: run a target request alone and inside batches of
random neighbours, and record what must come out bit for bit the same.

The schedule imitates continuous batching with chunked prefill (the serving
setting the pages blame for nondeterminism: devpress.csdn.net explainer of
"Defeating Nondeterminism in LLM Inference", sections 2.3 and 3.3;
tom-jerr.github.io "Batch-Invariant Kernel", Motivation): every engine step
carries each decoding sequence's next token plus prefill chunks of the
sequences still reading their prompts, up to a token budget, in a shuffled
order.  The target's record per generated token is its greedy token and its
top-20 (ids, fp32 values) -- the acceptance test of the zhaixingw.cn BlockLock
post.
"""
import numpy as np
import torch


class Seq:
    def __init__(self, slot, prompt, max_new):
        self.slot, self.prompt, self.max_new = slot, list(prompt), max_new
        self.done_prefill = 0          # prompt tokens already in the cache
        self.generated = []
        self.next_tok = None           # token to feed in the next decode step

    def finished(self):
        return len(self.generated) >= self.max_new


def run(decoder, pool, target_prompt, n_new, neighbours=(), budget=None, seed=0,
        record_logits=False, lock_target=False, record_neighbours=False):
    """Greedy-decode `n_new` tokens of the target (slot order and batch order
    randomised by `seed`).  neighbours: list of prompts, each decoded greedily
    alongside.  budget: max prompt tokens per step (None: whole prompts at once).
    lock_target: run the target locked and everyone else on the tuned
    comparators (Decoder.step's selective locking).
    Returns a dict with the target's tokens, top-20 ids / values per token
    (host tensors) and, if asked, the full logits rows; with record_neighbours
    also "neighbours": per neighbour (in the order given) its generated tokens
    and the logits row that chose each."""
    rng = np.random.default_rng(int(seed))
    # slots are taken in a shuffled order so the target's page-table row moves too
    seqs = []
    order = list(range(len(neighbours) + 1))
    rng.shuffle(order)
    prompts = [target_prompt] + list(neighbours)
    slots = {}
    for i in order:
        slots[i] = pool.alloc()
    for i, p in enumerate(prompts):
        seqs.append(Seq(slots[i], p, n_new if i == 0 else 10 ** 9))
    target = seqs[0]
    out = {"tokens": [], "top_ids": [], "top_vals": [], "logits": []}
    nb_rec = {id(s): {"tokens": [], "logits": []} for s in seqs[1:]}
    while not target.finished():
        items, owners = [], []
        left = budget if budget is not None else float("inf")
        for s in seqs:
            if s.done_prefill < len(s.prompt):
                if left <= 0:
                    continue
                n = int(min(len(s.prompt) - s.done_prefill, left))
                items.append((s.slot, s.prompt[s.done_prefill:s.done_prefill + n], s.done_prefill))
                owners.append((s, "prefill", n))
                left -= n
            elif s is target or not s.finished():
                start = len(s.prompt) + len(s.generated) - 1
                items.append((s.slot, [s.generated[-1]], start))
                owners.append((s, "decode", 1))
        perm = rng.permutation(len(items))
        items = [items[i] for i in perm]
        owners = [owners[i] for i in perm]
        logits, top_ids, top_vals = decoder.step(
            items, protected={target.slot} if lock_target else None)
        ids_h = top_ids.cpu()
        for k, (s, kind, n) in enumerate(owners):
            if kind == "prefill":
                s.done_prefill += n
                if s.done_prefill < len(s.prompt):
                    continue                      # mid-prompt chunk: nothing generated yet
            s.generated.append(int(ids_h[k, 0]))
            if record_neighbours and s is not target:
                nb_rec[id(s)]["tokens"].append(int(ids_h[k, 0]))
                nb_rec[id(s)]["logits"].append(logits[k].cpu().clone())
            if s is target:
                out["tokens"].append(int(ids_h[k, 0]))
                out["top_ids"].append(ids_h[k].clone())
                out["top_vals"].append(top_vals[k].cpu().clone())
                if record_logits:
                    out["logits"].append(logits[k].cpu().clone())
    for s in seqs:
        pool.release(s.slot)
    out["top_ids"] = torch.stack(out["top_ids"])
    out["top_vals"] = torch.stack(out["top_vals"])
    if record_logits:
        out["logits"] = torch.stack(out["logits"])
    if record_neighbours:
        out["neighbours"] = [nb_rec[id(s)] for s in seqs[1:]]
    return out


def same_bits(a, b):
    """True if two runs produced identical tokens and top-20 ids / value bits."""
    return (a["tokens"] == b["tokens"] and torch.equal(a["top_ids"], b["top_ids"])
            and torch.equal(a["top_vals"].view(torch.int32), b["top_vals"].view(torch.int32)))
