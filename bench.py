#!/usr/bin/env python3
"""Benchmark of the batch-invariant hot path on one MI355X.

One step = one pass of every hot-path kernel over one batch of synthetic input:
  1. RMSNorm      x bf16 [8192, 4096] (N(0,3), 1% outliers at +-50) -> y bf16
  2. GEMM         y [8192, 4096] x W bf16 [4096, 4096] (N(0,0.02)) -> C bf16
  3. decode attn  paged, 32 query / 8 KV heads of 128, B = 256 sequences with
                  KV lengths log-uniform in [128, 32768], pages shuffled
  4. prefill attn one 4096-token sequence, same head shape, one shot
  5. decoder glue embedding of 8192 tokens into an fp32 residual stream,
                  residual add of the GEMM output, RoPE + paged KV write of a
                  4096-token fused q/k/v projection [4096, 6144], SwiGLU on a
                  [4096, 2 x 14336] gate/up block, row gather and exact top-20
                  of 256 rows of 128256 fp32 logits
Inputs are resident in HBM before the timed region.  The GPU's clocks ramp up
over the first second or so of sustained load, so before the W warmup steps
the step is run untimed for --ramp-seconds (default 1 s).  Each leg is bracketed by
HIP events recorded on the stream the kernels are launched on (torch's current
stream).  The decode leg streams ~6 GB of KV, far more than the 256 MB
last-level cache, so every leg starts from a cache the other legs have
flushed.

`value` is the GEMM leg in TFLOP/s (2*M*N*K per launch / mean launch time);
`rmsnorm_vs_device_copy` times a plain device copy of the RMSNorm leg's bytes
in the same cache state (right after a full step), the practical ceiling of
that HBM-bound leg;
the decode-attention GB/s (algorithmic bytes: K, V, q, out, page table) is
reported beside it with its own roofline.  `cpu_baseline` times the fp64
oracle on a bounded sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--ramp-seconds S] [--no-cpu-baseline]
       python bench.py --sweep   (per-shape figures of every workload family, invariant
                                  kernels beside the shape-tuned comparators, one JSON line
                                  per case)
       [--profile-copy]   (adds one 1 GiB device copy, the calibration kernel
                           for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
       python bench.py --gemm M,N,K [--gemm ...] [--reps R] [--packed]
                          (the invariant GEMM alone on the given shapes, cold
                           operands, one JSON line per shape: for per-shape
                           kernel traces and counters; --packed through the
                           packed-weight entry point)
       python bench.py --decoder B [--steps K]
                          (the 8B-class decoder's decode steps at batch B alone:
                           invariant kernels, packed weights, HIP graphs)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "batch-invariant GEMM TFLOP/s + decode-attn GB/s (% roofline), bitwise-invariant"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E

RMS_M, HIDDEN = 8192, 4096
GEMM_M, GEMM_N, GEMM_K = 8192, 4096, 4096
DEC_B, HQ, HKV, HD = 256, 32, 8, 128
DEC_LMIN, DEC_LMAX = 128, 32768
PREFILL_T = 4096
FFN, VOCAB, LOGIT_ROWS, THETA = 14336, 128256, 256, 5e5
WORKLOAD = (f"rmsnorm {RMS_M}x{HIDDEN} bf16 -> gemm {GEMM_M}x{GEMM_N}x{GEMM_K} bf16 -> "
            f"paged decode attn B={DEC_B} Hq={HQ} Hkv={HKV} D={HD} L~logU[{DEC_LMIN},{DEC_LMAX}] "
            f"-> prefill attn T={PREFILL_T} -> decoder glue (embed, residual add, RoPE+KV write, "
            f"SwiGLU F={FFN}, top-20 of {LOGIT_ROWS}x{VOCAB})")


def build_workload(device="cuda:0", seed_base=0):
    """All inputs of one step, resident on `device`."""
    import torch

    from invariant_deterministic_fixed_amd import synth
    import invariant_deterministic_fixed_amd as binv

    w = {}
    s3, s2, s4 = synth.seed_for(3), synth.seed_for(2), synth.seed_for(4)
    x = synth.normal((RMS_M, HIDDEN), 3.0, s3 + seed_base, device, dtype=torch.float32)
    w["x"] = synth.with_outliers(x, 0.01, 50.0, s3 + 1 + seed_base).to(torch.bfloat16)
    del x
    w["gamma"] = synth.uniform((HIDDEN,), 0.5, 1.5, s3 + 2, device)
    w["y"] = torch.empty((RMS_M, HIDDEN), dtype=torch.bfloat16, device=device)
    w["W"] = synth.normal((GEMM_K, GEMM_N), 0.02, s2 + 7, device)
    w["C"] = torch.empty((GEMM_M, GEMM_N), dtype=torch.bfloat16, device=device)

    lens = synth.log_uniform_lengths(DEC_B, DEC_LMIN, DEC_LMAX, s4 + seed_base)
    seqs = [synth.random_kv(int(L), HKV, HD, s4 + 100 + 31 * i, device) for i, L in enumerate(lens)]
    w["dec_cache"] = synth.PagedKV(seqs, HKV, HD, s4 + 5, device=device)
    del seqs
    w["dec_lens"] = lens
    w["dec_max_kv"] = int(lens.max())
    w["dec_q"] = synth.normal((DEC_B, HQ, HD), 1.0, s4 + 6, device)
    w["dec_out"] = torch.empty_like(w["dec_q"])
    w["dec_ws"] = torch.empty(binv.attn_workspace_bytes(DEC_B, HQ, HD, w["dec_max_kv"]),
                              dtype=torch.uint8, device=device)

    pk, pv = synth.random_kv(PREFILL_T, HKV, HD, s4 + 9, device)
    w["pf_kv"] = (pk, pv)
    w["pf_cache"] = synth.PagedKV([(pk, pv)], HKV, HD, s4 + 10, device=device)
    w["pf_q"] = synth.normal((PREFILL_T, HQ, HD), 1.0, s4 + 11, device)
    w["pf_cu"] = torch.tensor([0, PREFILL_T], dtype=torch.int32, device=device)
    w["pf_out"] = torch.empty_like(w["pf_q"])
    w["pf_ws"] = torch.empty(binv.attn_prefill_workspace_bytes(1, PREFILL_T, PREFILL_T, PREFILL_T,
                                                               HQ, HKV, HD),
                             dtype=torch.uint8, device=device)
    w["scale"] = 1.0 / math.sqrt(HD)

    # decoder glue
    g = torch.Generator(device=device)
    g.manual_seed(s4 + 20)
    w["ids"] = torch.randint(0, VOCAB, (GEMM_M,), generator=g, device=device, dtype=torch.int32)
    w["embed"] = synth.normal((VOCAB, HIDDEN), 0.02, s4 + 21, device)
    w["h"] = torch.empty((GEMM_M, HIDDEN), dtype=torch.float32, device=device)
    w["qkv"] = synth.normal((PREFILL_T, (HQ + 2 * HKV) * HD), 1.0, s4 + 22, device)
    w["rope_q"] = torch.empty((PREFILL_T, HQ, HD), dtype=torch.bfloat16, device=device)
    n_pages = PREFILL_T // 16
    w["rope_k"] = torch.zeros((n_pages, HKV, 16, HD), dtype=torch.bfloat16, device=device)
    w["rope_v"] = torch.zeros((n_pages, HKV, HD, 16), dtype=torch.bfloat16, device=device)
    w["rope_pt"] = torch.randperm(n_pages, generator=g, device=device).to(torch.int32).view(1, -1)
    w["rope_seq"] = torch.zeros(PREFILL_T, dtype=torch.int32, device=device)
    w["rope_pos"] = torch.arange(PREFILL_T, dtype=torch.int32, device=device)
    w["gu"] = synth.normal((PREFILL_T, 2 * FFN), 1.0, s4 + 23, device)
    w["swi"] = torch.empty((PREFILL_T, FFN), dtype=torch.bfloat16, device=device)
    w["logits"] = synth.normal((LOGIT_ROWS, VOCAB), 3.0, s4 + 24, device, dtype=torch.float32)
    w["rows"] = torch.randperm(GEMM_M, generator=g, device=device)[:LOGIT_ROWS].to(torch.int32)
    w["hl"] = torch.empty((LOGIT_ROWS, HIDDEN), dtype=torch.float32, device=device)
    return w


def run_step(w, events=None):
    """One pass of the hot path; if `events` (6 torch.cuda.Event) is given the
    legs are bracketed by them."""
    import invariant_deterministic_fixed_amd as binv

    ev = events or [None] * 6
    rec = (lambda e: e.record()) if events else (lambda e: None)
    rec(ev[0])
    binv.rmsnorm(w["x"], w["gamma"], 1e-6, out=w["y"])
    rec(ev[1])
    binv.gemm(w["y"], w["W"], out=w["C"])
    rec(ev[2])
    c = w["dec_cache"]
    binv.attn_decode(w["dec_q"], c.k_cache, c.v_cache, c.page_table, c.kv_lens, w["dec_max_kv"],
                     w["scale"], out=w["dec_out"], workspace=w["dec_ws"])
    rec(ev[3])
    p = w["pf_cache"]
    binv.attn_prefill(w["pf_q"], w["pf_cu"], p.k_cache, p.v_cache, p.page_table, p.kv_lens,
                      PREFILL_T, PREFILL_T, w["scale"], out=w["pf_out"], workspace=w["pf_ws"])
    rec(ev[4])
    binv.embed(w["ids"], w["embed"], out=w["h"])
    binv.residual_add(w["h"], w["C"])
    binv.rope_kv_write(w["qkv"], w["rope_seq"], w["rope_pos"], HQ, HKV, HD, THETA, w["rope_k"],
                       w["rope_v"], w["rope_pt"], q_out=w["rope_q"])
    binv.swiglu(w["gu"], out=w["swi"])
    binv.gather_rows(w["h"], w["rows"], out=w["hl"])
    binv.topk(w["logits"], 20)
    rec(ev[5])


def side_measurements(w, reps):
    """Figures beside the step, each on operands rotated over copies larger
    than the last-level cache: RMSNorm alone as back-to-back launches at the
    step's shape and at the largest RMSNorm workload (16384 rows), and the
    GEMM against hipBLASLt (torch.mm as a black box) and against the
    library's shape-tuned split-K comparator, on the same operands."""
    import torch
    import invariant_deterministic_fixed_amd as binv
    from invariant_deterministic_fixed_amd import synth

    dev = w["x"].device
    res = {}
    b2b = {}
    for M in (RMS_M, 16384):
        n = _copies(4 * M * HIDDEN, floor=600 << 20)
        xs = [synth.normal((M, HIDDEN), 3.0, 31 + i, dev).to(torch.bfloat16) for i in range(n)]
        y = torch.empty_like(xs[0])
        for x in xs:
            binv.rmsnorm(x, w["gamma"], 1e-6, out=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        launches = max(reps, 4 * n)
        e0.record()
        for k in range(launches):
            binv.rmsnorm(xs[k % n], w["gamma"], 1e-6, out=y)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / launches * 1e-3
        nbytes = 4 * M * HIDDEN + 2 * HIDDEN
        b2b[f"{M}x{HIDDEN}"] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                                "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4),
                                "launches": launches, "input_copies": n}
        del xs, y
    res["rmsnorm_back_to_back"] = b2b

    nW = _copies(2 * GEMM_K * GEMM_N, floor=600 << 20)
    Ws = [w["W"]] + [w["W"].clone() for _ in range(nW - 1)]
    C2 = torch.empty_like(w["C"])
    ws = torch.empty(binv.lib().binv_gemm_bf16_tuned_workspace_bytes(GEMM_M, GEMM_N, GEMM_K),
                     dtype=torch.uint8, device=dev)
    y = w["y"]
    t_inv = _cold_ms([lambda W=W: binv.gemm(y, W, out=C2) for W in Ws], reps=max(20, reps))
    t_mm = _cold_ms([lambda W=W: torch.mm(y, W, out=C2) for W in Ws], reps=max(20, reps))
    t_tun = _cold_ms([lambda W=W: binv.gemm(y, W, out=C2, tuned=True, workspace=ws) for W in Ws],
                     reps=max(20, reps))
    fl = 2.0 * GEMM_M * GEMM_N * GEMM_K
    res["gemm_vs_hipblaslt"] = {
        "invariant_TFLOPs": round(fl / t_inv / 1e9, 1),
        "hipblaslt_torch_mm_TFLOPs": round(fl / t_mm / 1e9, 1),
        "tuned_splitk_TFLOPs": round(fl / t_tun / 1e9, 1),
        "invariant_over_hipblaslt_speed": round(t_mm / t_inv, 3),
        "invariant_over_tuned_speed": round(t_tun / t_inv, 3)}
    del Ws, C2, ws
    torch.cuda.empty_cache()
    return res


def algorithmic(w):
    """Algorithmic work per launch of each leg (what the method must move / compute)."""
    lens = w["dec_lens"]
    sum_l = int(lens.sum())
    dec_bytes = (sum_l * HKV * HD * 2 * 2                   # K and V, bf16
                 + 2 * DEC_B * HQ * HD * 2                   # q in, out
                 + int(sum(-(-int(L) // 16) for L in lens)) * 4 + DEC_B * 4)   # page table, lens
    return {
        "rmsnorm_bytes": 2 * RMS_M * HIDDEN * 2 + HIDDEN * 2,
        "gemm_flops": 2 * GEMM_M * GEMM_N * GEMM_K,
        "gemm_bytes": 2 * (GEMM_M * GEMM_K + GEMM_K * GEMM_N + GEMM_M * GEMM_N),
        "decode_bytes": dec_bytes,
        "decode_sum_kv": sum_l,
        "prefill_flops": 4 * HQ * HD * (PREFILL_T * (PREFILL_T + 1) // 2),
        "glue_bytes": (GEMM_M * 4 + GEMM_M * HIDDEN * (2 + 4)          # embed: ids, rows in, h out
                       + GEMM_M * HIDDEN * (4 + 2 + 4)                  # residual add
                       + PREFILL_T * ((HQ + 2 * HKV) * HD * 2 + HQ * HD * 2 + 2 * HKV * HD * 2 + 8)
                       + PREFILL_T * (2 * FFN * 2 + FFN * 2)            # swiglu
                       + LOGIT_ROWS * (4 + 2 * HIDDEN * 4)              # gather
                       + LOGIT_ROWS * (VOCAB * 4 + 20 * 8)),            # top-20
    }


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel_key):
    """Measured HBM bytes per launch from the committed rocprofv3 counter summary,
    or None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    pinned = dict(rec.get("also", {}))
    pinned[rec["source"]] = rec["source_sha256"]
    for rel, digest in pinned.items():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or _sha(src) != digest:
            return None
    return rec["hbm_bytes_per_launch"]


def tiny_oracle_ms():
    """The oracle on the whole tiny single-layer workload (RMSNorm of 8 fp32
    rows of 256, the 256 x 256 GEMM, decode attention of 8 sequences with 4
    heads of 64 and lengths U[1, 300]), on one thread and on every core."""
    import oracle
    from invariant_deterministic_fixed_amd import synth

    x = synth.normal((8, 256), 1.0, synth.seed_for(1), dtype=torch_f32()).double().numpy()
    g = synth.uniform((256,), 0.5, 1.5, synth.seed_for(1) + 2).double().numpy()
    W = synth.normal((256, 256), 0.02, synth.seed_for(1) + 3).double().numpy()
    lens = synth.uniform_int_lengths(8, 1, 300, synth.seed_for(1) + 1)
    kv = [synth.random_kv(int(L), 4, 64, synth.seed_for(1) + 10 + i) for i, L in enumerate(lens)]
    kv = [(k.double().numpy(), v.double().numpy()) for k, v in kv]

    def run():
        y = oracle.round_bf16(oracle.rmsnorm(x, g, 1e-6))
        q = oracle.round_bf16(oracle.gemm(y, W)).reshape(8, 4, 64)
        for b, (k, v) in enumerate(kv):
            oracle.attention(q[b:b + 1], [int(lens[b]) - 1], k, v, 0.125)

    full = oracle.num_threads()
    out = {}
    for n in (1, full):
        oracle.set_num_threads(n)
        run()
        t0 = time.perf_counter()
        for _ in range(5):
            run()
        out[f"threads_{n}"] = round((time.perf_counter() - t0) / 5 * 1e3, 3)
    oracle.set_num_threads(full)
    return out


def torch_f32():
    import torch
    return torch.float32


def cpu_baseline(w, gemm_rows=GEMM_M, max_seqs=DEC_B, prefill_rows=512):
    """The fp64 oracle on a bounded sample of the same workload (the very same
    input values, copied from HBM to the host), on the host cores."""
    import oracle

    xd = w["x"][:gemm_rows].double().cpu().numpy()
    gd = w["gamma"].double().cpu().numpy()
    Wd = w["W"].double().cpu().numpy()
    t0 = time.perf_counter()
    y = oracle.round_bf16(oracle.rmsnorm(xd, gd, 1e-6))
    oracle.gemm(y, Wd)
    t_gemm = time.perf_counter() - t0
    gemm_tflops = 2.0 * gemm_rows * GEMM_N * GEMM_K / t_gemm / 1e12

    lens = w["dec_lens"]
    q = w["dec_q"].double().cpu().numpy()
    n_seq, nbytes, t_att = 0, 0, 0.0
    for b in range(min(DEC_B, max_seqs)):
        k, v = w["dec_cache"].logical(b)
        kd, vd = k.double().cpu().numpy(), v.double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.attention(q[b:b + 1], [int(lens[b]) - 1], kd, vd, w["scale"])
        t_att += time.perf_counter() - t0
        n_seq += 1
        nbytes += int(lens[b]) * HKV * HD * 2 * 2 + 2 * HQ * HD * 2
    pk, pv = w["pf_kv"]
    rows = list(range(0, PREFILL_T, PREFILL_T // prefill_rows))
    pq = w["pf_q"][rows].double().cpu().numpy()
    kd, vd = pk.double().cpu().numpy(), pv.double().cpu().numpy()
    t0 = time.perf_counter()
    oracle.attention(pq, rows, kd, vd, w["scale"])
    t_pf = time.perf_counter() - t0
    pf_flops = 4 * HQ * HD * sum(r + 1 for r in rows)
    tiny = tiny_oracle_ms()
    return {
        "value": gemm_tflops,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "tiny_layer_ms": tiny,
        "kind": "oracle",
        "sample": (f"fp64 RMSNorm + GEMM of {gemm_rows} of the {GEMM_M} rows ({t_gemm:.1f} s); "
                   f"fp64 decode attention of {n_seq} of the {DEC_B} sequences "
                   f"({t_att:.1f} s, {nbytes / t_att / 1e9:.3f} GB/s); fp64 prefill attention of "
                   f"{len(rows)} of the {PREFILL_T} rows ({t_pf:.1f} s, "
                   f"{pf_flops / t_pf / 1e12:.4f} TFLOP/s)"),
        "decode_attn_GBps": nbytes / t_att / 1e9,
        "prefill_attn_TFLOPs": pf_flops / t_pf / 1e12,
    }


# ---------------------------------------------------------------- sweep mode
def _cold_ms(fns, reps=20):
    """Mean ms of one call, cycling over `fns` (each bound to its own copy of
    the inputs, together larger than the 256 MB last-level cache, so no call
    finds its operands cached), events around each call."""
    import torch
    for f in fns[:2]:
        f()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for k in range(reps):
        evs[k][0].record()
        fns[k % len(fns)]()
        evs[k][1].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def _copies(nbytes, floor=640 << 20):
    return max(1, min(64, -(-floor // max(1, nbytes))))


def sweep(dev="cuda:0"):
    """Per-shape figures of every workload family, invariant kernels beside
    the shape-tuned comparators (and torch.mm, i.e. hipBLASLt, for the GEMM):
    one JSON object per line."""
    import numpy as np
    import torch
    import invariant_deterministic_fixed_amd as binv
    from invariant_deterministic_fixed_amd import synth, decoder as dec

    def paged(lens, seed):
        seqs = [synth.random_kv(int(L), HKV, HD, seed + 31 * i, dev) for i, L in enumerate(lens)]
        return synth.PagedKV(seqs, HKV, HD, seed + 5, device=dev)

    def emit(**kv):
        print(json.dumps(kv), flush=True)

    # clock ramp
    a = torch.randn((8192, 4096), device=dev).to(torch.bfloat16)
    b = torch.randn((4096, 4096), device=dev).to(torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        binv.gemm(a, b)
        torch.cuda.synchronize()
    del a, b

    # GEMM: invariant vs tuned vs torch.mm, per M and weight shape; up to 64
    # rows also the invariant product over strip-packed weights
    for (N, K, c32) in [(4096, 4096, False), (14336, 4096, False), (4096, 14336, False),
                        (128256, 4096, True)]:
        nw = _copies(2 * N * K)
        Ws = [synth.normal((K, N), 0.02, 7 + i, dev) for i in range(nw)]
        Wps = [binv.gemm_pack(W) for W in Ws]
        for M in [1, 2, 7, 16, 64, 256, 1024, 2048, 8192]:
            if c32 and M > 256:
                continue
            A = synth.normal((M, K), 1.0, 3, dev)
            od = torch.float32 if c32 else torch.bfloat16
            C = torch.empty((M, N), dtype=od, device=dev)
            ws = torch.empty(binv.lib().binv_gemm_bf16_tuned_workspace_bytes(M, N, K),
                             dtype=torch.uint8, device=dev)
            t_inv = _cold_ms([lambda W=W: binv.gemm(A, W, out=C) for W in Ws])
            t_tun = _cold_ms([lambda W=W: binv.gemm(A, W, out=C, tuned=True, workspace=ws)
                              for W in Ws])
            t_mm = t_pk = None
            if not c32:
                t_mm = _cold_ms([lambda W=W: torch.mm(A, W, out=C) for W in Ws])
            if M <= 64:
                t_pk = _cold_ms([lambda W=W: binv.gemm_packed(A, W, out=C) for W in Wps])
            flops = 2.0 * M * N * K
            nbytes = 2 * (M * K + K * N) + (4 if c32 else 2) * M * N
            roof_ms = max(flops / PEAK_BF16_TFLOPS / 1e9, nbytes / PEAK_HBM_GBPS / 1e6)
            emit(sweep="gemm", M=M, N=N, K=K, out="fp32" if c32 else "bf16",
                 invariant_TFLOPs=round(flops / t_inv / 1e9, 2),
                 tuned_TFLOPs=round(flops / t_tun / 1e9, 2),
                 torch_mm_TFLOPs=None if t_mm is None else round(flops / t_mm / 1e9, 2),
                 packed_TFLOPs=None if t_pk is None else round(flops / t_pk / 1e9, 2),
                 packed_weight_GBps=None if t_pk is None else round(2 * N * K / t_pk / 1e6, 1),
                 roofline_frac=round(roof_ms / t_inv, 4),
                 slowdown_vs_tuned=round(t_inv / t_tun, 3))
            del A, C, ws
        del Ws, Wps
        torch.cuda.empty_cache()

    # RMSNorm: invariant vs tuned, per M and d
    for d in [4096, 5120]:
        g = synth.uniform((d,), 0.5, 1.5, 5, dev).to(torch.bfloat16)
        for M in [1, 64, 1024, 4096, 8192, 16384]:
            n = _copies(4 * M * d)
            xs = [synth.normal((M, d), 3.0, 11 + i, dev).to(torch.bfloat16) for i in range(n)]
            y = torch.empty_like(xs[0])
            t_inv = _cold_ms([lambda x=x: binv.rmsnorm(x, g, 1e-6, out=y) for x in xs])
            t_tun = _cold_ms([lambda x=x: binv.rmsnorm(x, g, 1e-6, out=y, tuned=True) for x in xs])
            nbytes = 4 * M * d + 2 * d
            emit(sweep="rmsnorm", M=M, d=d, invariant_GBps=round(nbytes / t_inv / 1e6, 1),
                 tuned_GBps=round(nbytes / t_tun / 1e6, 1),
                 roofline_frac=round(nbytes / t_inv / 1e6 / PEAK_HBM_GBPS, 4),
                 slowdown_vs_tuned=round(t_inv / t_tun, 3))
            del xs, y
        torch.cuda.empty_cache()

    # decode attention: invariant vs tuned, per batch size (log-uniform lengths)
    for B in [1, 4, 16, 64, 256]:
        lens = synth.log_uniform_lengths(B, DEC_LMIN, DEC_LMAX, synth.seed_for(4) + B)
        kv_bytes = int(lens.sum()) * HKV * HD * 4
        caches = [paged(lens, synth.seed_for(4) + 1000 * i) for i in range(_copies(kv_bytes))]
        q = synth.normal((B, HQ, HD), 1.0, 9, dev)
        out = torch.empty_like(q)
        ws = torch.empty(binv.attn_workspace_bytes(B, HQ, HD, DEC_LMAX), dtype=torch.uint8,
                         device=dev)
        wst = torch.empty(binv.lib().binv_attn_decode_tuned_workspace_bytes(B, HQ, HD, DEC_LMAX),
                          dtype=torch.uint8, device=dev)
        scale = 1.0 / math.sqrt(HD)
        t_inv = _cold_ms([lambda c=c: binv.attn_decode(q, c.k_cache, c.v_cache, c.page_table,
                                                        c.kv_lens, DEC_LMAX, scale, out=out,
                                                        workspace=ws) for c in caches])
        t_tun = _cold_ms([lambda c=c: binv.attn_decode(q, c.k_cache, c.v_cache, c.page_table,
                                                        c.kv_lens, DEC_LMAX, scale, out=out,
                                                        workspace=wst, tuned=True)
                          for c in caches])
        nbytes = kv_bytes + 4 * B * HQ * HD + 4 * sum(-(-int(L) // 16) for L in lens)
        emit(sweep="decode_attn", B=B, sum_kv_tokens=int(lens.sum()),
             invariant_GBps=round(nbytes / t_inv / 1e6, 1), tuned_GBps=round(nbytes / t_tun / 1e6, 1),
             roofline_frac=round(nbytes / t_inv / 1e6 / PEAK_HBM_GBPS, 4),
             slowdown_vs_tuned=round(t_inv / t_tun, 3))
        del caches, q, out, ws, wst
        torch.cuda.empty_cache()

    # prefill attention: one 4096-token sequence, one shot and in chunks
    T = PREFILL_T
    c = paged([T], synth.seed_for(4) + 3)
    q = synth.normal((T, HQ, HD), 1.0, 13, dev)
    out = torch.empty_like(q)
    # sized for the largest piece; every smaller piece needs less
    ws = torch.empty(binv.attn_prefill_workspace_bytes(1, T, T, T, HQ, HKV, HD), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / math.sqrt(HD)
    for chunk in [T, 2048, 512, 256]:
        parts = []
        for s0 in range(0, T, chunk):
            n = min(chunk, T - s0)
            parts.append((s0, n, torch.tensor([0, n], dtype=torch.int32, device=dev),
                          torch.tensor([s0 + n], dtype=torch.int32, device=dev)))

        def run(parts=parts):
            for s0, n, cu, kvl in parts:
                binv.attn_prefill(q[s0:s0 + n], cu, c.k_cache, c.v_cache, c.page_table, kvl, n, T,
                                  scale, out=out[s0:s0 + n], workspace=ws)
        t = _cold_ms([run], reps=5)
        flops = 4.0 * HQ * HD * sum(p + 1 for p in range(T))
        emit(sweep="prefill_attn", T=T, chunk=chunk, TFLOPs=round(flops / t / 1e9, 2))
    del c, q, out, ws
    torch.cuda.empty_cache()

    # mixed engine step through the prefill entry point: one sequence runs a
    # prompt chunk, the others one decode token each, every context ctx long
    for (B, run_len, ctx) in [(64, 1, 1024), (64, 512, 1024), (256, 256, 2048), (16, 2048, 4096)]:
        qlens = [run_len] + [1] * (B - 1)
        c = paged([ctx] * B, synth.seed_for(4) + 7)
        T = sum(qlens)
        q = synth.normal((T, HQ, HD), 1.0, 17, dev)
        out = torch.empty_like(q)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32, device=dev)
        kvl = torch.full((B,), ctx, dtype=torch.int32, device=dev)
        ws = torch.empty(binv.attn_prefill_workspace_bytes(B, T, run_len, ctx, HQ, HKV, HD),
                         dtype=torch.uint8, device=dev)
        t = _cold_ms([lambda: binv.attn_prefill(q, cu, c.k_cache, c.v_cache, c.page_table, kvl,
                                                run_len, ctx, 1.0 / math.sqrt(HD), out=out,
                                                workspace=ws)], reps=5)
        kv_bytes = B * ctx * HKV * HD * 2 * 2
        emit(sweep="prefill_mixed", B=B, run=run_len, context=ctx, us=round(t * 1e3, 1),
             kv_GBps=round(kv_bytes / t / 1e6, 1))
        del c, q, out, ws
        torch.cuda.empty_cache()

    # 8B-class decoder: decode tokens/s at batch B with 1024-token contexts, all
    # invariant, all tuned, and one locked request among tuned neighbours; each
    # step replayed as a HIP graph (the serving configuration) and issued
    # eagerly (every kernel launched from Python).  The invariant decode-size
    # products read strip-packed weights (decoder.PACKED_ROWS; same bits)
    cfg = dec.CONFIG5
    w = dec.random_weights(cfg, 5, dev)
    packed = dec.pack_weights(w)
    for B in [1, 16, 64]:
        res = {}
        for mode in ("invariant", "tuned", "locked"):
            if mode == "locked" and B == 1:
                continue
            for graph in (True, False):
                res[(mode, graph)] = decoder_tokens_per_s(w, packed, B, mode, graph, 8, dev)
        emit(sweep="decoder_8b_decode", B=B, context=1024,
             invariant_tokens_per_s=round(res[("invariant", True)], 1),
             tuned_tokens_per_s=round(res[("tuned", True)], 1),
             locked_one_tokens_per_s=(round(res[("locked", True)], 1)
                                      if ("locked", True) in res else None),
             slowdown_vs_tuned=round(res[("tuned", True)] / res[("invariant", True)], 3),
             eager_invariant_tokens_per_s=round(res[("invariant", False)], 1),
             eager_tuned_tokens_per_s=round(res[("tuned", False)], 1),
             eager_locked_one_tokens_per_s=(round(res[("locked", False)], 1)
                                            if ("locked", False) in res else None))
    del w, packed
    torch.cuda.empty_cache()

    # fp32-activation mitigation: six RMSNorm -> GEMM blocks at d = 4096 with
    # bf16 or fp32 activations, invariant or tuned kernels; the target row's
    # output drift over batch sizes 1 / 64 / 256 / 1024 and the chain's time
    from invariant_deterministic_fixed_amd import fp32act
    d, layers = 4096, 6
    ws = [synth.normal((d, d), 1.0 / 64, 300 + l, dev) for l in range(layers)]
    ws3 = [fp32act.stack3(x) for x in ws]
    gamma = torch.ones(d, dtype=torch.bfloat16, device=dev)
    target = synth.normal((1, d), 1.0, 299, dev)
    r = np.random.default_rng(298)
    for mode in ("bf16", "fp32"):
        for tuned in (False, True):
            outs, ms = {}, {}
            for B in (1, 64, 256, 1024):
                X = synth.normal((B, d), 1.0, 400 + B, dev)
                p = int(r.integers(0, B))
                X[p] = target[0]
                outs[B] = fp32act.chain(X, ws, gamma, mode, tuned, weights3=ws3)[p].double().cpu()
                ms[B] = _cold_ms([lambda: fp32act.chain(X, ws, gamma, mode, tuned, weights3=ws3)],
                                 reps=10)
            base = outs[1]
            drift = max(float((outs[B] - base).abs().max()) for B in outs) / float(base.abs().max())
            moved = max(int((outs[B] != base).sum()) for B in outs)
            emit(sweep="fp32act_chain", activations=mode,
                 kernels="tuned" if tuned else "invariant", d=d, layers=layers,
                 drift_rel=drift, elements_moved=moved,
                 ms_B1=round(ms[1], 4), ms_B64=round(ms[64], 4), ms_B1024=round(ms[1024], 4))


def decoder_tokens_per_s(w, packed, B, mode, graph, steps, dev="cuda:0"):
    """8B-class decoder: B sequences prefilled with 1024 random tokens each
    (untimed), one untimed decode step (a graph's capture), then `steps` timed
    decode steps of one token per sequence; returns tokens/s.  mode: invariant,
    tuned (the comparators), or locked (sequence 0 invariant among tuned ones);
    invariant decode-size products read `packed` (not with tuned)."""
    import numpy as np
    import torch
    from invariant_deterministic_fixed_amd import decoder as dec

    cfg = dec.CONFIG5
    pool = dec.KVPool(cfg, num_pages=B * (1024 + 64) // 16 + B, max_seqs=B,
                      max_len=1024 + 64, seed=11, device=dev)
    d = dec.Decoder(w, cfg, pool, max_tokens=max(1024, B), max_seqs=B,
                    max_kv_len=1024 + 64, tuned=(mode == "tuned"),
                    packed=None if mode == "tuned" else packed)
    r = np.random.default_rng(42)
    slots = [pool.alloc() for _ in range(B)]
    prot = {slots[0]} if mode == "locked" else None
    toks = {}
    for sl in slots:
        _, ids, _ = d.step([(sl, r.integers(0, cfg["vocab"], 1024).tolist(), 0)])
        toks[sl] = int(ids[0, 0])
    _, ids, _ = d.step([(sl, [toks[sl]], 1024) for sl in slots], protected=prot, graph=graph)
    ids = ids.cpu()
    for i, sl in enumerate(slots):
        toks[sl] = int(ids[i, 0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        _, ids, _ = d.step([(sl, [toks[sl]], 1025 + k) for sl in slots], protected=prot,
                           graph=graph)
        ids = ids.cpu()
        for i, sl in enumerate(slots):
            toks[sl] = int(ids[i, 0])
    torch.cuda.synchronize()
    tps = B * steps / (time.perf_counter() - t0)
    del d, pool
    torch.cuda.empty_cache()
    return tps


def decoder_only(B, steps, dev="cuda:0"):
    """The 8B-class decoder's decode steps alone (invariant, packed weights,
    HIP graphs): one JSON line, for traces of a decode step."""
    from invariant_deterministic_fixed_amd import decoder as dec

    w = dec.random_weights(dec.CONFIG5, 5, dev)
    packed = dec.pack_weights(w)
    tps = decoder_tokens_per_s(w, packed, B, "invariant", True, steps, dev)
    print(json.dumps({"decoder_8b_decode": {"B": B, "context": 1024, "steps": steps,
                                            "tokens_per_s": round(tps, 1),
                                            "ms_per_step": round(B / tps * 1e3, 3)}}),
          flush=True)


def gemm_shapes(shapes, reps, dev="cuda:0", packed=False):
    """The invariant GEMM alone, per shape (M, N, K): weights rotated over
    enough copies to exceed the last-level cache, R timed launches.  packed:
    through binv_gemm_bf16_packed on strip-packed copies (M <= 64)."""
    import torch
    import invariant_deterministic_fixed_amd as binv
    from invariant_deterministic_fixed_amd import synth

    a = torch.randn((8192, 4096), device=dev).to(torch.bfloat16)
    b = torch.randn((4096, 4096), device=dev).to(torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:                  # clock ramp
        binv.gemm(a, b)
        torch.cuda.synchronize()
    del a, b
    for (M, N, K) in shapes:
        Ws = [synth.normal((K, N), 0.02, 7 + i, dev) for i in range(_copies(2 * N * K))]
        A = synth.normal((M, K), 1.0, 3, dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if packed:
            Ws = [binv.gemm_pack(W) for W in Ws]
            t = _cold_ms([lambda W=W: binv.gemm_packed(A, W, out=C) for W in Ws], reps=reps)
        else:
            t = _cold_ms([lambda W=W: binv.gemm(A, W, out=C) for W in Ws], reps=reps)
        flops = 2.0 * M * N * K
        nbytes = 2 * (M * K + K * N + M * N)
        roof_ms = max(flops / PEAK_BF16_TFLOPS / 1e9, nbytes / PEAK_HBM_GBPS / 1e6)
        print(json.dumps({"gemm": [M, N, K], "packed": packed, "us": round(t * 1e3, 2),
                          "TFLOPs": round(flops / t / 1e9, 2), "GBps": round(nbytes / t / 1e6, 1),
                          "roofline_frac": round(roof_ms / t, 4)}), flush=True)
        del Ws, A, C
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-seconds", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-copy", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="per-shape figures (one JSON line per case) instead of the bench line")
    ap.add_argument("--gemm", action="append", default=[],
                    help="M,N,K: time the invariant GEMM alone on this shape (repeatable)")
    ap.add_argument("--packed", action="store_true",
                    help="with --gemm: the packed-weight entry point (M <= 64)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--decoder", type=int, default=0, metavar="B",
                    help="time the 8B-class decoder's decode steps at batch B alone "
                         "(--steps of them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(dev)
        return
    if args.decoder:
        decoder_only(args.decoder, args.steps, dev)
        return
    if args.gemm:
        gemm_shapes([tuple(int(v) for v in g.split(",")) for g in args.gemm], args.reps, dev,
                    packed=args.packed)
        return
    w = build_workload(dev)
    work = algorithmic(w)
    torch.cuda.synchronize()

    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:   # clock ramp, untimed
        run_step(w)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step(w)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(w, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    legs = ["rmsnorm", "gemm", "decode_attn", "prefill_attn", "decoder_glue"]
    per = {n: sorted(e[i].elapsed_time(e[i + 1]) for e in evs) for i, n in enumerate(legs)}
    ms = {n: sum(v) / len(v) for n, v in per.items()}

    def pct(v, q):
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    s = {n: ms[n] * 1e-3 for n in legs}
    gemm_tflops = work["gemm_flops"] / s["gemm"] / 1e12
    dec_gbps = work["decode_bytes"] / s["decode_attn"] / 1e9
    rms_gbps = work["rmsnorm_bytes"] / s["rmsnorm"] / 1e9
    pf_tflops = work["prefill_flops"] / s["prefill_attn"] / 1e12
    glue_gbps = work["glue_bytes"] / s["decoder_glue"] / 1e9

    # reference for the HBM-bound RMSNorm leg: a plain device copy of the same
    # bytes (x -> y, no arithmetic), timed in the same cache state, i.e. right
    # after a full step, where the next step's RMSNorm would start
    cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    for k in range(args.steps):
        run_step(w)
        cevs[k][0].record()
        w["y"].copy_(w["x"])
        cevs[k][1].record()
    torch.cuda.synchronize()
    copy_s = sum(a.elapsed_time(b) for a, b in cevs) / args.steps * 1e-3
    copy_gbps = work["rmsnorm_bytes"] / copy_s / 1e9

    if args.profile_copy:
        # calibration for the HBM byte counters: one elementwise kernel that
        # reads 1 GiB and writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    extra = side_measurements(w, args.steps)

    gemm_traffic = traffic_for("gemm_bf16_kernel")
    dec_traffic = traffic_for("attn_decode")
    out = {
        "metric": METRIC,
        "value": round(gemm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "gemm": [GEMM_M, GEMM_N, GEMM_K],
                   "rmsnorm": [RMS_M, HIDDEN], "decode_B": DEC_B,
                   "decode_sum_kv_tokens": work["decode_sum_kv"], "prefill_T": PREFILL_T,
                   "heads": [HQ, HKV, HD], "page_size": 16, "split_kv_chunk": 256},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": gemm_traffic, "kernel": "gemm_bf16_kernel",
                     "per_launch": {"flops": work["gemm_flops"], "bytes": work["gemm_bytes"]}},
        "decode_attn": {"value": round(dec_gbps, 1), "unit": "GB/s",
                        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1),
                                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                     "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                     "traffic": dec_traffic,
                                     "kernel": "attn_chunk_kernel + attn_merge_kernel",
                                     "per_launch": {"bytes": work["decode_bytes"]}}},
        "legs_ms": {n: round(ms[n], 4) for n in legs},
        "legs_ms_median": {n: round(pct(per[n], 0.5), 4) for n in legs},
        "legs_ms_p10": {n: round(pct(per[n], 0.1), 4) for n in legs},
        "legs_ms_p90": {n: round(pct(per[n], 0.9), 4) for n in legs},
        "rmsnorm_GBps": round(rms_gbps, 1),
        "rmsnorm_frac_hbm": round(rms_gbps / PEAK_HBM_GBPS, 4),
        "rmsnorm_vs_device_copy": {"copy_GBps": round(copy_gbps, 1),
                                   "ratio": round(rms_gbps / copy_gbps, 3)},
        "prefill_attn_TFLOPs": round(pf_tflops, 2),
        "decoder_glue_GBps": round(glue_gbps, 1),
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
