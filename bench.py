#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X (gfx950).

Default run (N = 1):
  * headline: causal MSA prefill of one 131072-token sequence, bf16, 8 KV heads x 8
    query heads per group, head_dim 128, index dim 128, 128-token blocks, top_k 16
    (index scores -> top-k -> sparse attention, timed as one step);
  * decode: one MSA decode step of 8 sequences against 1,048,576-token bf16 caches with
    the same heads (index scan -> top-k -> split-K sparse attention + combine).
Each is timed with HIP events on the stream the kernels run on, after W untimed
warmup steps; the dominant kernel of each is also timed launch by launch for its
roofline fraction. The CPU oracle is then timed on a bounded sample of the same
inputs (and the sampled rows are checked against the GPU result).
Then the other workloads of the same metric run as extra legs with their own settings
(EXTRA_LEGS): the 1,048,576-token prefill with its dense GQA baseline, the 4096-token fp32
prefill (every row checked against the oracle) and the 4 x 131072 decode step.

One JSON line goes to stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA prefill tok/s @128K & decode µs/tok @1M; % MFMA peak / % HBM BW"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
BLOCK = 128

WORKLOADS = {
    "prefill_128k": dict(kind="prefill", T=131072, G=8, Hpg=8, d_idx=128, top_k=16, planted=8,
                         dtype="bf16", chunk=131072),
    "prefill_1m": dict(kind="prefill", T=1 << 20, G=8, Hpg=8, d_idx=128, top_k=16, planted=16,
                       dtype="bf16", chunk=131072),
    "prefill_4k_f32": dict(kind="prefill", T=4096, G=2, Hpg=3, d_idx=64, top_k=4, planted=0,
                           dtype="f32", chunk=4096),
    "decode_1m": dict(kind="decode", B=8, L=1 << 20, G=8, Hpg=8, d_idx=128, top_k=16, planted=16,
                      dtype="bf16"),
    "decode_128k": dict(kind="decode", B=4, L=131072, G=8, Hpg=8, d_idx=128, top_k=16,
                        planted=16, dtype="bf16"),
}

# Settings of the legs that run after the two headline legs (the other workloads of the
# same metric). The 1M prefill keeps its step count small (about a second a step) and runs
# its dense baseline once; the small workloads check every row against the oracle.
EXTRA_LEGS = {
    "prefill_1m": dict(steps=2, warmup=1, kl=0, gemm_calibration=0, dense_reps=1,
                       dense_warm=False, cpu_seconds=10.0, paged=0),
    "prefill_4k_f32": dict(kl=0, gemm_calibration=0, dense_reps=5, oracle_all_rows=True),
    "decode_128k": dict(dense_reps=5),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work (what the method must do; not the dense work it avoids) ---------

def prefill_index_flops(T, G, d_idx, top_k):
    nblk = (T + BLOCK - 1) // BLOCK
    s = sum(b for b in range(top_k, nblk))
    # rows of local block b score b full blocks, only when b >= top_k
    tokens_per_block = [min(BLOCK, T - b * BLOCK) for b in range(nblk)]
    return sum(2.0 * d_idx * G * BLOCK * b * tokens_per_block[b] for b in range(top_k, nblk))


def prefill_attn_flops(T, Hq, D, top_k):
    tot = 0
    for t_block in range((T + BLOCK - 1) // BLOCK):
        n_in = min(BLOCK, T - t_block * BLOCK)
        kept = min(top_k, t_block + 1) - 1           # full non-local blocks
        # sum over the block's tokens of visible keys: 128*kept + (t mod 128) + 1
        tot += n_in * BLOCK * kept + n_in * (n_in + 1) // 2
    return 4.0 * D * Hq * tot


def kl_pairs(T, top_k):
    """Visible kept (row, key) pairs per group of a causal prefill with full selections."""
    tot = 0
    for t_block in range((T + BLOCK - 1) // BLOCK):
        n_in = min(BLOCK, T - t_block * BLOCK)
        kept = min(top_k, t_block + 1) - 1
        tot += n_in * BLOCK * kept + n_in * (n_in + 1) // 2
    return tot


def kl_flops(T, G, Hpg, D, d_idx, top_k):
    """Index-branch KL loss + gradients: per visible kept pair, the main logits of the
    group's heads (2 Hpg D), the index logit (2 d), and its share of dq_idx and dk_idx
    (2 d each). The second pass's recomputation of the logits is not counted."""
    return float(G * kl_pairs(T, top_k)) * (2.0 * Hpg * D + 6.0 * d_idx)


def dense_prefill_flops(T, Hq, D):
    """Causal dense attention: 4 D FLOPs per (head, query t, visible key j <= t)."""
    return 4.0 * D * Hq * T * (T + 1) / 2


def dense_decode_bytes(lens, G, Hpg, D, esize):
    """Whole-cache decode: every visible K and V row of each group once, plus q and out."""
    return sum(2 * G * L * D * esize + 2 * G * Hpg * D * esize for L in lens)


def time_reps(torch, fn, reps, warm=True):
    """Mean milliseconds of fn() over reps runs, after one untimed run when warm (HIP
    events)."""
    if warm:
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def decode_bytes(lens, G, Hpg, D, d_idx, top_k, esize):
    tot = 0
    for L in lens:
        b = (L - 1) // BLOCK
        scan = b * BLOCK if b >= top_k else 0
        if b + 1 <= top_k:
            n = L
        else:
            n = BLOCK * (top_k - 1) + (L - 1) % BLOCK + 1
        tot += scan * d_idx * esize + 2 * esize * D * G * n + esize * (2 * G * Hpg * D + G * d_idx)
    return tot


def decode_scan_bytes(lens, d_idx, top_k, esize):
    tot = 0
    for L in lens:
        b = (L - 1) // BLOCK
        if b >= top_k:
            tot += b * BLOCK * d_idx * esize
    return tot


# ---- timing helpers -----------------------------------------------------------------------

class KernelTimer:
    """HIP events around one entry point's launches, on the stream they run on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        s = self.torch.cuda.current_stream()
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.a.record(s)
        return self

    def __exit__(self, *exc):
        s = self.torch.cuda.current_stream()
        b = self.torch.cuda.Event(enable_timing=True)
        b.record(s)
        self.pairs.append((self.a, b))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def measured_traffic(kernel_fragment, kind, launch):
    """HBM bytes per launch of a kernel from profiles/traffic.json (two rocprofv3 --pmc
    runs, scaled by a plain copy), or None when absent, when the kernel's source has
    changed since the counters were taken, or when they were taken on another workload or
    launch configuration (`launch`, this run's description of the `kind` leg)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        from block_sparse_long_05_amd.profiling import source_hash
        t = json.load(open(path))
        if t.get("launches", {}).get(kind) != launch:
            return None
        for name, v in t["kernels"].items():
            if kernel_fragment in name:
                h = source_hash(name)
                if h is None or v.get("source_hash") != h:
                    return None
                if v.get("read_bytes") is None or v.get("write_bytes") is None:
                    return None
                return v["read_bytes"] + v["write_bytes"]
    except Exception:
        return None
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ---- prefill --------------------------------------------------------------------------------

def run_prefill(name, cfg, args, torch, msa, synth):
    T, G, Hpg, d_idx, top_k = cfg["T"], cfg["G"], cfg["Hpg"], cfg["d_idx"], cfg["top_k"]
    chunk = min(args.chunk or cfg["chunk"], T)
    log(f"[{name}] generating inputs T={T} G={G} Hpg={Hpg} d_idx={d_idx} k={top_k}")
    x = synth.prefill_inputs(T, G, Hpg, 128, d_idx, dtype=cfg["dtype"], seed=1000 + T,
                             planted_per_group=cfg["planted"], device="cuda")
    torch.cuda.synchronize()
    q = x["q"]
    out = torch.empty_like(q)
    chunks = [(c0, min(chunk, T - c0)) for c0 in range(0, T, chunk)]
    probs = [msa.Problem(dtype=cfg["dtype"], mode="prefill", num_groups=G, heads_per_group=Hpg,
                         index_dim=d_idx, top_k=top_k, seq_len=T, q_begin=c0, q_count=n,
                         algo=args.algo) for c0, n in chunks]
    fused = args.index == "fused" and all(msa.index_topk_supported(p) for p in probs)
    # the fused index branch needs no workspace, so it can take more rows per launch than
    # the attention (default: the whole sequence in one launch, one tail instead of one
    # per chunk)
    ichunk = min(args.index_chunk or T, T) if fused else chunk
    ichunks = [(c0, min(ichunk, T - c0)) for c0 in range(0, T, ichunk)]
    iprobs = [msa.Problem(dtype=cfg["dtype"], mode="prefill", num_groups=G, heads_per_group=Hpg,
                          index_dim=d_idx, top_k=top_k, seq_len=T, q_begin=c0, q_count=n)
              for c0, n in ichunks] if fused else None
    bs = None if fused else torch.empty((chunk, G, probs[0].nblk), dtype=torch.float32,
                                        device="cuda")
    idx_full = torch.empty((T, G, top_k), dtype=torch.int32, device="cuda")
    ws_bytes = max(msa.msa_workspace_size(p, "sparse_attn_prefill") for p in probs)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None

    timers = {}

    def step(timed):
        if fused:
            for p, (c0, n) in zip(iprobs, ichunks):
                if timed:
                    with timers.setdefault("index_topk", KernelTimer(torch)):
                        msa.msa_index_topk(p, x["q_idx"], x["k_idx"], idx_full[c0:c0 + n])
                else:
                    msa.msa_index_topk(p, x["q_idx"], x["k_idx"], idx_full[c0:c0 + n])
        for p, (c0, n) in zip(probs, chunks):
            idx = idx_full[c0:c0 + n]
            if not timed:
                if not fused:
                    msa.msa_index_scores(p, x["q_idx"], x["k_idx"], bs)
                    msa.msa_block_topk(p, bs, idx)
                msa.msa_sparse_attn_prefill(p, q, x["k"], x["v"], idx, out, ws)
                continue
            if not fused:
                with timers.setdefault("index_scores", KernelTimer(torch)):
                    msa.msa_index_scores(p, x["q_idx"], x["k_idx"], bs)
                with timers.setdefault("block_topk", KernelTimer(torch)):
                    msa.msa_block_topk(p, bs, idx)
            with timers.setdefault("sparse_attn", KernelTimer(torch)):
                msa.msa_sparse_attn_prefill(p, q, x["k"], x["v"], idx, out, ws)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    # the step time, with nothing between the launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        step(False)
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel durations: events around every launch of each entry point
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    per_kernel = {k: v.mean_ms() * (len(ichunks) if k == "index_topk" else len(chunks))
                  for k, v in timers.items()}

    idx_flops = prefill_index_flops(T, G, d_idx, top_k)
    att_flops = prefill_attn_flops(T, G * Hpg, 128, top_k)
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_F32_TFLOPS
    idx_name = "index_topk" if fused else "index_scores"
    idx_ms_launch = timers[idx_name].mean_ms()
    n_idx_launch = len(ichunks) if fused else len(chunks)
    idx_tflops = idx_flops / n_idx_launch / (idx_ms_launch * 1e-3) / 1e12
    total_tflops = (idx_flops + att_flops) / (ms * 1e-3) / 1e12
    # the workload and launch configuration (what the stored HBM counters must match)
    launch = (f"{name} chunk={chunk} index_rows={ichunk} algo={args.algo} "
              f"index={'fused' if fused else 'separate'}")
    res = dict(
        workload=name, launch=launch, T=T, G=G, Hpg=Hpg, d_idx=d_idx, top_k=top_k,
        dtype=cfg["dtype"], chunk=chunk, index_launch_rows=ichunk, algo=args.algo,
        index_branch="fused" if fused else "separate",
        ms_per_step=ms, wall_s=wall, tok_per_s=T / (ms * 1e-3),
        kernel_ms_per_step=per_kernel,
        flops=dict(index=idx_flops, attention=att_flops),
        path_tflops=total_tflops, path_frac_of_peak=total_tflops / peak,
        roofline=dict(bound="mfma",
                      kernel="index_topk_prefill" if fused else "index_scores_prefill",
                      achieved=idx_tflops, peak=peak, unit="TFLOP/s", frac=idx_tflops / peak,
                      traffic=measured_traffic("index_topk_prefill" if fused
                                               else "index_scores_prefill", "prefill", launch),
                      work_per_launch=idx_flops / n_idx_launch, launch_ms=idx_ms_launch),
    )
    log(f"[{name}] {ms:.3f} ms/step  {res['tok_per_s']:.4g} tok/s  kernels {per_kernel}  "
        f"path {total_tflops:.1f} TFLOP/s ({res['path_frac_of_peak']*100:.1f}% of peak)  "
        f"index {idx_tflops:.1f} TFLOP/s")
    if args.kl and cfg["dtype"] == "bf16" and d_idx == 128:
        res["kl"] = run_kl(name, cfg, args, torch, msa, x, idx_full, chunks, T, G, Hpg, d_idx,
                           top_k, peak)
    if cfg["dtype"] == "bf16" and args.gemm_calibration:
        # The card's practical bf16 MFMA rate on the same kind of data, outside the timed
        # region: the vendor GEMM (torch.matmul -> hipBLASLt) on N(0,1) operands. The spec
        # peak is not sustained on random data (the clock drops under dense MFMA load).
        n = 16384
        ga = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        gb = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        gemm_ms = time_reps(torch, lambda: torch.matmul(ga, gb), 5)
        del ga, gb
        gemm_tflops = 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
        res["measured_bf16_gemm_tflops"] = gemm_tflops
        res["path_frac_of_measured_gemm"] = total_tflops / gemm_tflops
        res["roofline"]["frac_of_measured_gemm"] = idx_tflops / gemm_tflops
        log(f"[{name}] vendor bf16 GEMM {n}^3 on N(0,1) data: {gemm_tflops:.0f} TFLOP/s; path "
            f"{res['path_frac_of_measured_gemm'] * 100:.1f}% of it, index kernel "
            f"{res['roofline']['frac_of_measured_gemm'] * 100:.1f}%")
    if args.dense_reps > 0:
        # dense causal GQA attention over the same rows (the speedup context): same chunks
        dout = torch.empty_like(q)  # its own output: `out` is checked against the oracle below

        def dense_step():
            for p in probs:
                msa.msa_dense_gqa_attn(p, q, x["k"], x["v"], dout)
        dense_ms = time_reps(torch, dense_step, args.dense_reps,
                             warm=getattr(args, "dense_warm", True))
        del dout
        dense_flops = dense_prefill_flops(T, G * Hpg, 128)
        res["dense"] = dict(ms=dense_ms, tflops=dense_flops / (dense_ms * 1e-3) / 1e12,
                            frac_of_peak=dense_flops / (dense_ms * 1e-3) / 1e12 / peak,
                            speedup=dense_ms / ms, reps=args.dense_reps)
        log(f"[{name}] dense GQA {dense_ms:.1f} ms ({res['dense']['tflops']:.0f} TFLOP/s); "
            f"MSA speedup {res['dense']['speedup']:.1f}x")
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["parity"] = prefill_oracle_sample(name, cfg, x, out, idx_full,
                                                                   args)
    del x, out, bs, idx_full, ws
    torch.cuda.empty_cache()
    return res


def prefill_oracle_sample(name, cfg, x, out, idx_full, args):
    """Time the oracle on 32-token slices of evenly spaced query blocks until about
    args.cpu_seconds have passed, and compare those rows with the GPU's."""
    import numpy as np
    from oracle import msa_oracle as orc
    from tests import parity

    T, top_k = cfg["T"], cfg["top_k"]
    host = {k: x[k].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    nblk = (T + BLOCK - 1) // BLOCK
    all_rows = getattr(args, "oracle_all_rows", False)
    if all_rows:   # every row, one query block at a time, latest first
        slices = [np.arange(b * BLOCK, min(b * BLOCK + BLOCK, T)) for b in range(nblk - 1, -1, -1)]
    else:          # 32-token slices of evenly spaced query blocks, latest first
        order = np.linspace(nblk - 1, 0, num=min(nblk, 64)).astype(int)
        slices = [np.arange(int(b) * BLOCK + (j % 4) * 32, min(int(b) * BLOCK + (j % 4) * 32 + 32, T))
                  for j, b in enumerate(order)]
    done, secs, worst, ties, differ, nsl = 0, 0.0, 0.0, 0, 0, 0
    for rows in slices:
        if len(rows) == 0:
            continue
        t0 = time.perf_counter()
        res = orc.prefill(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], top_k,
                          rows=rows)
        secs += time.perf_counter() - t0
        done += len(rows)
        nsl += 1
        got_out = out[rows[0]:rows[-1] + 1].float().cpu().numpy()
        got_idx = idx_full[rows[0]:rows[-1] + 1].cpu().numpy()
        info = parity.check_prefill(host, rows, got_out, got_idx, None, res, top_k,
                                    q_begin=int(rows[0]), out_offset=int(rows[0]), label=name)
        worst = max(worst, info["err"])
        ties += info["near_ties"]
        differ += info["differ"]
        if secs >= args.cpu_seconds and not all_rows:
            break
    cores = blas_threads()
    sample = (f"all {T} query tokens x {cfg['G']} groups of the input (whole rows: index scores "
              f"over all earlier keys, top-k, attention)" if all_rows else
              f"{done} query tokens x {cfg['G']} groups in {nsl} slices of 32 tokens "
              f"from evenly spaced query blocks of the same {T}-token input, latest "
              f"first (whole rows: index scores over all earlier keys, top-k, "
              f"attention)")
    base = dict(value=done / secs, unit="tok/s", cores=cores, kind="oracle", sample=sample,
                seconds=secs, cpu=cpu_model())
    par = dict(rows_checked=done, max_abs_err=worst, near_tie_rows=ties,
               near_tie_selection_differences=differ, ok=True)
    log(f"[{name}] oracle {base['value']:.3g} tok/s on {cores} threads; parity {par}")
    return base, par


def run_kl(name, cfg, args, torch, msa, x, idx_full, chunks, T, G, Hpg, d_idx, top_k, peak):
    """The index-branch KL loss and gradients over the selection the index branch just
    made (training side; not part of the prefill step above)."""
    scale = 1.0 / d_idx ** 0.5
    kprobs = [msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                          index_dim=d_idx, top_k=top_k, seq_len=T, q_begin=c0, q_count=n)
              for c0, n in chunks]
    kws = torch.empty(max(msa.msa_workspace_size(p, "index_kl") for p in kprobs),
                      dtype=torch.uint8, device="cuda")
    loss = torch.empty((T, G), dtype=torch.float32, device="cuda")
    dq = torch.empty((T, G, d_idx), dtype=torch.float32, device="cuda")
    dk = torch.zeros((T, d_idx), dtype=torch.float32, device="cuda")

    def kl_step():
        dk.zero_()
        for p, (c0, n) in zip(kprobs, chunks):
            msa.msa_index_kl_prefill(p, x["q"], x["k"], x["q_idx"], x["k_idx"],
                                     idx_full[c0:c0 + n], scale, loss[c0:c0 + n], dq[c0:c0 + n],
                                     dk, kws)
    kl_ms = time_reps(torch, kl_step, max(1, args.steps // 2))
    fl = kl_flops(T, G, Hpg, 128, d_idx, top_k)
    tf = fl / (kl_ms * 1e-3) / 1e12
    # the same with the main heads' normalisers from the forward attention's lse output
    # (what a training step has anyway); the attention itself is not timed here
    main_lse = torch.empty((T, G * Hpg), dtype=torch.float32, device="cuda")
    aprobs = [msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                          index_dim=d_idx, top_k=top_k, seq_len=T, q_begin=c0, q_count=n)
              for c0, n in chunks]
    aws = torch.empty(max(msa.msa_workspace_size(p, "sparse_attn_prefill") for p in aprobs),
                      dtype=torch.uint8, device="cuda")
    aout = torch.empty_like(x["q"])
    for p, (c0, n) in zip(aprobs, chunks):
        msa.msa_sparse_attn_prefill(p, x["q"], x["k"], x["v"], idx_full[c0:c0 + n], aout, aws,
                                    lse=main_lse)
    del aws, aout
    loss_ref = loss.clone()

    def kl_step_lse():
        dk.zero_()
        for p, (c0, n) in zip(kprobs, chunks):
            msa.msa_index_kl_prefill(p, x["q"], x["k"], x["q_idx"], x["k_idx"],
                                     idx_full[c0:c0 + n], scale, loss[c0:c0 + n], dq[c0:c0 + n],
                                     dk, kws, main_lse=main_lse)
    kl_lse_ms = time_reps(torch, kl_step_lse, max(1, args.steps // 2))
    tf_lse = fl / (kl_lse_ms * 1e-3) / 1e12
    lse_loss_diff = float((loss - loss_ref).abs().max())
    del main_lse
    # identities of the gradients at full size (fp64 on the device): each row's score
    # gradients sum to zero, and sum_j dk[j] . k_idx[j] = sum_(t,g) dq[t,g] . q_idx[t,g]
    dk64 = dk.double()
    lhs = float((dk64 * x["k_idx"].double()).sum())
    rhs = float((dq.double() * x["q_idx"].double()).sum())
    zero_rel = float(dk64.sum(0).abs().max() / dk64.abs().sum(0).max())
    out = dict(ms=kl_ms, tflops=tf, frac_of_peak=tf / peak, flops=fl, index_scale=scale,
               with_main_lse=dict(ms=kl_lse_ms, tflops=tf_lse, frac_of_peak=tf_lse / peak,
                                  max_loss_diff_vs_standalone=lse_loss_diff),
               loss_mean=float(loss.double().mean()), dk_sum_rel=zero_rel,
               identity_rel=abs(lhs - rhs) / max(abs(lhs), abs(rhs), 1e-30))
    log(f"[{name}] index KL loss+grad {kl_ms:.2f} ms ({tf:.0f} TFLOP/s, "
        f"{tf / peak * 100:.1f}% of peak); with the attention's lse {kl_lse_ms:.2f} ms "
        f"({tf_lse:.0f} TFLOP/s, loss diff {lse_loss_diff:.1e})  mean loss {out['loss_mean']:.4f}  "
        f"sum dk rel {zero_rel:.2e}  identity rel {out['identity_rel']:.2e}")
    del kws, loss, dq, dk
    torch.cuda.empty_cache()
    return out


# ---- decode ------------------------------------------------------------------------------

def run_decode(name, cfg, args, torch, msa, synth):
    B, L, G, Hpg, d_idx, top_k = cfg["B"], cfg["L"], cfg["G"], cfg["Hpg"], cfg["d_idx"], cfg["top_k"]
    log(f"[{name}] generating inputs B={B} L={L} G={G} Hpg={Hpg} k={top_k}")
    x = synth.decode_inputs(B, L, G, Hpg, 128, d_idx, dtype=cfg["dtype"], seed=2000 + B,
                            planted_per_group=cfg["planted"], device="cuda")
    torch.cuda.synchronize()
    p = msa.decode_problem(x, top_k)
    out = torch.empty_like(x["q"])
    bs = msa.alloc_block_scores(p)
    idx = msa.alloc_block_idx(p)
    ws = msa.alloc_workspace(p, "sparse_attn_decode")

    timers = {}

    # the step: index scan, then selection + attention + combine in one call (the selection
    # runs inside the attention launch where that is faster)
    def step(timed):
        if not timed:
            msa.msa_index_scores(p, x["q_idx"], x["k_idx"], bs)
            msa.msa_sparse_attn_decode_topk(p, x["q"], x["k_cache"], x["v_cache"], bs, idx, out,
                                            ws)
            return
        with timers.setdefault("index_scan", KernelTimer(torch)):
            msa.msa_index_scores(p, x["q_idx"], x["k_idx"], bs)
        with timers.setdefault("topk_sparse_attn", KernelTimer(torch)):
            msa.msa_sparse_attn_decode_topk(p, x["q"], x["k_cache"], x["v_cache"], bs, idx, out,
                                            ws)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        step(True)
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    # untimed-by-kernel loop: the step time without per-kernel events in between
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(s)
    for _ in range(args.steps):
        step(False)
    e3.record(s)
    torch.cuda.synchronize()
    ms_plain = e2.elapsed_time(e3) / args.steps
    lens = [L] * B
    esize = 2 if cfg["dtype"] == "bf16" else 4
    tot_bytes = decode_bytes(lens, G, Hpg, 128, d_idx, top_k, esize)
    scan_bytes = decode_scan_bytes(lens, d_idx, top_k, esize)
    scan_ms = timers["index_scan"].mean_ms()
    scan_gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    res = dict(
        workload=name, launch=name, B=B, L=L, G=G, Hpg=Hpg, d_idx=d_idx, top_k=top_k,
        dtype=cfg["dtype"], us_per_step=ms_plain * 1e3, us_per_token=ms_plain * 1e3 / B,
        us_per_step_with_kernel_events=ms * 1e3, wall_s=wall,
        kernel_us={k: v.mean_ms() * 1e3 for k, v in timers.items()},
        bytes_per_step=tot_bytes, path_gbs=tot_bytes / (ms_plain * 1e-3) / 1e9,
        path_frac_of_hbm=tot_bytes / (ms_plain * 1e-3) / 1e9 / PEAK_HBM_GBS,
        roofline=dict(bound="hbm", kernel="index_scores_decode", achieved=scan_gbs,
                      peak=PEAK_HBM_GBS, unit="GB/s", frac=scan_gbs / PEAK_HBM_GBS,
                      traffic=measured_traffic("index_scores_decode", "decode", name),
                      work_per_launch=scan_bytes, launch_ms=scan_ms),
    )
    if args.paged:
        # the same step on a paged copy of the caches (pages at seeded random ids)
        pgd = synth.to_paged(x, seed=B)
        pout = torch.empty_like(out)
        pidx = torch.empty_like(idx)

        def paged_step():
            msa.msa_index_scores_paged(p, x["q_idx"], pgd["k_idx_pages"], pgd["block_table"], bs)
            msa.msa_sparse_attn_decode_topk_paged(p, x["q"], pgd["k_pages"], pgd["v_pages"],
                                                  pgd["block_table"], bs, pidx, pout, ws)
        paged_ms = time_reps(torch, paged_step, args.steps)
        res["paged"] = dict(us_per_step=paged_ms * 1e3, us_per_token=paged_ms * 1e3 / B,
                            vs_contiguous=paged_ms / ms_plain,
                            same_output=bool(torch.equal(pout, out) and torch.equal(pidx, idx)))
        del pgd, pout, pidx
        torch.cuda.empty_cache()
    if args.dense_reps > 0:
        dws = msa.alloc_workspace(p, "dense_gqa_attn")
        dout = torch.empty_like(out)  # `out` is checked against the oracle below
        dense_ms = time_reps(torch, lambda: msa.msa_dense_gqa_attn(p, x["q"], x["k_cache"],
                                                                    x["v_cache"], dout, dws),
                             max(3, args.dense_reps))
        dense_bytes = dense_decode_bytes(lens, G, Hpg, 128, esize)
        res["dense"] = dict(us_per_step=dense_ms * 1e3, gbs=dense_bytes / (dense_ms * 1e-3) / 1e9,
                            frac_of_hbm=dense_bytes / (dense_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            speedup=dense_ms / ms_plain,
                            kernel="decode_dense_bf16" if cfg["dtype"] == "bf16"
                            else "gather_attn (dense decode)")
        del dws, dout
    log(f"[{name}] {res['us_per_step']:.1f} us/step {res['us_per_token']:.2f} us/token  "
        f"kernels {res['kernel_us']}  path {res['path_gbs']:.0f} GB/s "
        f"({res['path_frac_of_hbm']*100:.1f}% of HBM)  scan {scan_gbs:.0f} GB/s"
        + (f"  dense {res['dense']['us_per_step']:.0f} us/step, MSA speedup "
           f"{res['dense']['speedup']:.1f}x" if "dense" in res else "")
        + (f"  paged {res['paged']['us_per_step']:.1f} us/step (same output: "
           f"{res['paged']['same_output']})" if "paged" in res else ""))
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["parity"] = decode_oracle_sample(name, cfg, x, out, idx, args,
                                                                  torch)
    del x, out, bs, idx, ws
    torch.cuda.empty_cache()
    return res


def decode_oracle_sample(name, cfg, x, out, idx, args, torch):
    import numpy as np
    from oracle import msa_oracle as orc
    from tests import parity

    B, top_k = cfg["B"], cfg["top_k"]
    done, secs, worst, ties, differ = 0, 0.0, 0.0, 0, 0
    for b in range(B):
        hx = {k: x[k][b:b + 1].cpu() for k in ("q", "q_idx", "k_idx", "seq_lens")}
        hx["k_cache"] = x["k_cache"][b:b + 1].cpu()
        hx["v_cache"] = x["v_cache"][b:b + 1].cpu()
        t0 = time.perf_counter()
        res = orc.decode(hx["q"], hx["k_cache"], hx["v_cache"], hx["q_idx"], hx["k_idx"],
                         hx["seq_lens"], top_k)
        secs += time.perf_counter() - t0
        done += 1
        info = parity.check_decode(hx, out[b:b + 1].float().cpu().numpy(),
                                   idx[b:b + 1].cpu().numpy(), None, res, top_k, label=name)
        worst = max(worst, info["err"])
        ties += info["near_ties"]
        differ += info["differ"]
        del hx
        if secs >= args.cpu_seconds:
            break
    cores = blas_threads()
    base = dict(value=secs / done * 1e6, unit="us/token", cores=cores, kind="oracle",
                sample=f"{done} of the {B} sequences of the same decode step (whole rows: index "
                       f"scan over all {cfg['L']} cached keys, top-k, attention)",
                seconds=secs, cpu=cpu_model())
    par = dict(sequences_checked=done, max_abs_err=worst, near_tie_rows=ties,
               near_tie_selection_differences=differ, ok=True)
    log(f"[{name}] oracle {base['value']:.4g} us/token on {cores} threads; parity {par}")
    return base, par


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill", default="prefill_128k", help="prefill workload ('none' to skip)")
    ap.add_argument("--decode", default="decode_1m", help="decode workload ('none' to skip)")
    ap.add_argument("--algo", default="auto", choices=["auto", "query_centric", "kv_centric"])
    ap.add_argument("--index", default="fused", choices=["fused", "separate"],
                    help="prefill index branch: one fused index->top-k kernel (when built for "
                         "the problem) or index scores then top-k")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (the reference "
                         "dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="prefill query rows per call (0 = the workload's default)")
    ap.add_argument("--index-chunk", type=int, default=0,
                    help="query rows per fused index launch (0: the whole sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kl", type=int, default=1,
                    help="also time the index-branch KL loss + gradients on the prefill's "
                         "selection (1/0)")
    ap.add_argument("--paged", type=int, default=1,
                    help="also time the decode step on a paged copy of the caches (1/0)")
    ap.add_argument("--dense-reps", type=int, default=1,
                    help="timed runs of the dense GQA entry point on the same workload "
                         "(speedup context; 0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--gemm-calibration", type=int, default=1,
                    help="also time the vendor bf16 GEMM (16384^3, N(0,1) operands) and report "
                         "the prefill path against it (1/0)")
    ap.add_argument("--extra", default=",".join(EXTRA_LEGS),
                    help="comma-separated workloads run after the two headline legs, each with "
                         "its own settings (EXTRA_LEGS); 'none' to skip")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the MSA hot path here has no multi-GPU "
              "path (no sharding, no collectives). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_05_amd import msa, synth
    msa.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pre = dec = None
    if args.prefill != "none":
        pre = run_prefill(args.prefill, WORKLOADS[args.prefill], args, torch, msa, synth)
    if args.decode != "none":
        dec = run_decode(args.decode, WORKLOADS[args.decode], args, torch, msa, synth)

    extra = {}
    for name in ([] if args.extra in ("", "none") else args.extra.split(",")):
        if name in (args.prefill, args.decode):
            continue
        leg = argparse.Namespace(**vars(args))
        for k, v in EXTRA_LEGS.get(name, {}).items():
            setattr(leg, k, v)
        runner = run_prefill if WORKLOADS[name]["kind"] == "prefill" else run_decode
        extra[name] = runner(name, WORKLOADS[name], leg, torch, msa, synth)

    if pre is None and dec is None:
        return
    head = pre if pre is not None else dec
    if pre is not None:
        value, unit, hib, ms = pre["tok_per_s"], "tok/s", True, pre["ms_per_step"]
        config = {"workload": f"MSA causal prefill, 1 sequence x {pre['T']} tokens, {pre['dtype']}, "
                              f"{pre['G']} KV heads x {pre['Hpg']} q heads/group, head_dim 128, "
                              f"index dim {pre['d_idx']}, block 128, top_k {pre['top_k']}",
                  "name": pre["workload"], "global_batch": 1, "seq_len": pre["T"],
                  "parallelism": "single GPU"}
    else:
        value, unit, hib, ms = dec["us_per_token"], "us/token", False, dec["us_per_step"] / 1e3
        config = {"workload": f"MSA decode step, batch {dec['B']}, cache {dec['L']} tokens",
                  "name": dec["workload"], "global_batch": dec["B"], "seq_len": dec["L"],
                  "parallelism": "single GPU"}
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": hib, "scaling": "weak",
        "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic: seeded N(0,1) inputs with planted index blocks",
        "config": config, "roofline": dict(head["roofline"]),
        "cpu_baseline": head.get("cpu_baseline"),
    }
    # The roofline object is the dominant kernel's (its algorithmic work per launch over its
    # launch time); the whole step against the same peak sits beside it as `path`, with the
    # target fraction for the step.
    if pre is not None:
        line["roofline"]["path"] = dict(
            achieved=pre["path_tflops"], peak=line["roofline"]["peak"], unit="TFLOP/s",
            frac=pre["path_frac_of_peak"], target_frac=0.5,
            target_met=pre["path_frac_of_peak"] >= 0.5,
            what="index + attention FLOPs of the whole prefill step / step time")
        line["path_frac_of_peak"] = pre["path_frac_of_peak"]
    else:
        line["roofline"]["path"] = dict(
            achieved=dec["path_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
            frac=dec["path_frac_of_hbm"], target_frac=0.6,
            target_met=dec["path_frac_of_hbm"] >= 0.6,
            what="algorithmic bytes of the whole decode step / step time")
    if pre is not None:
        line["prefill"] = pre
    if dec is not None:
        dec["roofline"] = dict(dec["roofline"], path=dict(
            achieved=dec["path_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
            frac=dec["path_frac_of_hbm"], target_frac=0.6,
            target_met=dec["path_frac_of_hbm"] >= 0.6,
            what="algorithmic bytes of the whole decode step / step time"))
        line["decode"] = dec
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
