"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on outputs the oracle can compute one by one (sampled query rows / sequences).

Workloads: decode of 4 sequences x 131072 cached tokens (all rows checked), decode of
8 x 1,048,576 (two sequences checked), causal prefill of 131072 tokens (sampled
32-token slices) and of 1,048,576 tokens (sampled 8-token slices), the index-branch KL
loss at 131072 tokens, and the tail rows of a 2,097,152-token sequence, long enough that the
reverse index takes its per-entry atomic form. All bf16 with 8 KV heads x 8 query heads per group, head_dim 128,
index dim 128, 128-token blocks, top_k 16, planted blocks as in the benchmark (the 2M tail:
one KV head with one query head, to keep its inputs small).
"""

import numpy as np
import pytest
import torch

from block_sparse_long_05_amd import msa, synth
from oracle import msa_oracle as orc
from tests import parity

pytestmark = pytest.mark.gpu


def _decode_case(B, L, seed, check):
    x = synth.decode_inputs(B, L, 8, 8, 128, 128, dtype="bf16", seed=seed, planted_per_group=16,
                            device="cuda")
    out, idx, _ = msa.decode(x, 16)
    torch.cuda.synchronize()
    print(f"decode B={B} L={L} ran", flush=True)
    for b in check:
        hx = {k: x[k][b:b + 1].cpu() for k in ("q", "q_idx", "k_idx", "seq_lens", "k_cache",
                                               "v_cache")}
        res = orc.decode(hx["q"], hx["k_cache"], hx["v_cache"], hx["q_idx"], hx["k_idx"],
                         hx["seq_lens"], 16)
        info = parity.check_decode(hx, out[b:b + 1].float().cpu().numpy(),
                                   idx[b:b + 1].cpu().numpy(), None, res, 16, label=f"seq {b}")
        print(b, info, flush=True)
        del hx


def test_decode_128k_all_sequences():
    _decode_case(4, 131072, seed=2004, check=range(4))


def test_decode_1m_sampled_sequences():
    _decode_case(8, 1 << 20, seed=2008, check=[0, 7])


def test_prefill_128k_sampled_rows():
    T = 131072
    x = synth.prefill_inputs(T, 8, 8, 128, 128, dtype="bf16", seed=1000 + T,
                             planted_per_group=8, device="cuda")
    out, idx, _ = msa.prefill(x, 16)
    # the fused index branch (the launch bench.py times) selects exactly the same blocks
    p = msa.Problem(dtype="bf16", mode="prefill", num_groups=8, heads_per_group=8,
                    index_dim=128, top_k=16, seq_len=T, q_begin=0, q_count=T)
    fused = msa.alloc_block_idx(p)
    msa.msa_index_topk(p, x["q_idx"], x["k_idx"], fused)
    torch.cuda.synchronize()
    assert torch.equal(fused, idx)
    host = {k: x[k].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    for lo in (0, 2048 + 17, 65536 - 16, T - 32):
        rows = np.arange(lo, min(lo + 32, T))
        res = orc.prefill(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], 16,
                          rows=rows)
        got_out = out[rows[0]:rows[-1] + 1].float().cpu().numpy()
        got_idx = idx[rows[0]:rows[-1] + 1].cpu().numpy()
        info = parity.check_prefill(host, rows, got_out, got_idx, None, res, 16,
                                    q_begin=int(rows[0]), out_offset=int(rows[0]),
                                    label=f"rows {lo}")
        print(lo, info, flush=True)


def test_index_kl_128k_sampled_rows():
    """Index-branch KL loss and gradients at 131072 tokens on the fused index branch's own
    selection (the launch bench.py times), standalone and with the attention's lse:
    sampled rows' loss and dq_idx against the oracle (on the oracle's selection, which
    must agree), and dk_idx through identities that hold at any size."""
    T, G, Hpg, k = 131072, 8, 8, 16
    scale = 1.0 / 128 ** 0.5
    x = synth.prefill_inputs(T, G, Hpg, 128, 128, dtype="bf16", seed=1000 + T,
                             planted_per_group=8, device="cuda")
    p = msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                    index_dim=128, top_k=k, seq_len=T, q_begin=0, q_count=T)
    idx = msa.alloc_block_idx(p)
    msa.msa_index_topk(p, x["q_idx"], x["k_idx"], idx)
    lse = torch.empty((T, G * Hpg), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_prefill(p, x["q"], x["k"], x["v"], idx, torch.empty_like(x["q"]),
                                msa.alloc_workspace(p, "sparse_attn_prefill"), lse=lse)
    loss, dq, dk = msa.index_kl(x, idx, k, scale)
    loss2, dq2, dk2 = msa.index_kl(x, idx, k, scale, main_lse=lse)
    torch.cuda.synchronize()
    print("kl 128k ran", flush=True)
    # gradient identities (fp64 on the device): row score gradients sum to zero over each
    # row's keys; and the loss depends on q_idx, k_idx only through their dot products
    for d_k, d_q, label in ((dk, dq, "standalone"), (dk2, dq2, "main lse")):
        d64 = d_k.double()
        zero_rel = float(d64.sum(0).abs().max() / d64.abs().sum(0).max())
        lhs = float((d64 * x["k_idx"].double()).sum())
        rhs = float((d_q.double() * x["q_idx"].double()).sum())
        assert zero_rel < 1e-4, (label, zero_rel)
        assert abs(lhs - rhs) <= 1e-4 * max(abs(lhs), abs(rhs)), (label, lhs, rhs)
    assert float((loss - loss2).abs().max()) <= 1e-4 * (1.0 + float(loss.abs().max()))
    host = {kk: x[kk].cpu() for kk in ("q", "k", "v", "q_idx", "k_idx")}
    for lo in (2048 + 5, 65536 - 8, T - 16):
        rows = np.arange(lo, lo + 16)
        res = orc.prefill(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], k,
                          rows=rows)
        gidx = idx[lo:lo + 16].cpu().numpy()
        differ = parity.check_selection(gidx, res, k, rows // orc.BLOCK, label=f"rows {lo}")
        ref = orc.index_kl(host["q"], host["k"], host["q_idx"], host["k_idx"],
                           orc.selection_array(res["sel"], k), scale, q_begin=lo)
        keep = np.array([not any((i, g) in differ for g in range(G)) for i in range(16)])
        sub = {kk: (v[keep] if kk in ("loss", "dq_idx", "dq_abs", "mass_abs", "loss_abs") else v)
               for kk, v in ref.items()}
        for lo_l, lo_q, label in ((loss, dq, "standalone"), (loss2, dq2, "main lse")):
            got_l = parity.np32(lo_l[lo:lo + 16])[keep]
            got_q = parity.np32(lo_q[lo:lo + 16])[keep]
            print(lo, label, parity.check_kl(got_l, got_q, sub, np.arange(int(keep.sum())),
                                             label=f"rows {lo} {label}"), flush=True)


def test_prefill_1m_sampled_rows():
    """Causal prefill of 1,048,576 tokens as the benchmark runs it (the fused index branch over
    all rows in one launch, the attention in chunks of 131072 rows sharing one workspace):
    sampled query rows against the oracle."""
    T, G, Hpg, k, chunk = 1 << 20, 8, 8, 16, 131072
    x = synth.prefill_inputs(T, G, Hpg, 128, 128, dtype="bf16", seed=1000 + T,
                             planted_per_group=16, device="cuda")
    p_all = msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                        index_dim=128, top_k=k, seq_len=T, q_begin=0, q_count=T)
    idx = msa.alloc_block_idx(p_all)
    msa.msa_index_topk(p_all, x["q_idx"], x["k_idx"], idx)
    out = torch.empty_like(x["q"])
    probs = [msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                         index_dim=128, top_k=k, seq_len=T, q_begin=c0, q_count=chunk)
             for c0 in range(0, T, chunk)]
    ws = msa.alloc_workspace(probs[-1], "sparse_attn_prefill")
    for p in probs:
        msa.msa_sparse_attn_prefill(p, x["q"], x["k"], x["v"], idx[p.q_begin:p.q_begin + chunk],
                                    out, ws)
    torch.cuda.synchronize()
    print("prefill 1M ran", flush=True)
    del ws
    host = {kk: x[kk].cpu() for kk in ("q", "k", "v", "q_idx", "k_idx")}
    for lo in (chunk - 4, 600000, T - 8):
        rows = np.arange(lo, lo + 8)
        res = orc.prefill(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], k,
                          rows=rows)
        got_out = out[lo:lo + 8].float().cpu().numpy()
        got_idx = idx[lo:lo + 8].cpu().numpy()
        info = parity.check_prefill(host, rows, got_out, got_idx, None, res, k, q_begin=lo,
                                    out_offset=lo, label=f"1M rows {lo}")
        print(lo, info, flush=True)


def test_prefill_reverse_index_beyond_lds_counters():
    """A 2,097,152-token sequence (16384 blocks): the per-block counters of the reverse index and a
    chunk's shared lists no longer fit in 64 KiB of LDS, so the attention sorts its rare entries
    with one device-scope atomic per entry. The last 1000 query rows (a ragged query tile at one
    head per group) run the fused index branch and the attention; sampled rows against the oracle."""
    T, G, Hpg, k = 1 << 21, 1, 1, 16
    q_count = 1000
    q_begin = T - q_count
    # 8 planted blocks (shared by the query tiles) + the local block + 7 independent choices
    # per row (the rare entries that go through the reverse index)
    x = synth.prefill_inputs(T, G, Hpg, 128, 128, dtype="bf16", seed=77, planted_per_group=8,
                             device="cuda")
    p = msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                    index_dim=128, top_k=k, seq_len=T, q_begin=q_begin, q_count=q_count)
    assert p.nblk * 4 >= 64 * 1024  # the per-block counters alone fill 64 KiB
    idx = msa.alloc_block_idx(p)
    msa.msa_index_topk(p, x["q_idx"], x["k_idx"], idx)
    out = torch.empty_like(x["q"])
    ws = msa.alloc_workspace(p, "sparse_attn_prefill")
    msa.msa_sparse_attn_prefill(p, x["q"], x["k"], x["v"], idx, out, ws)
    torch.cuda.synchronize()
    print("prefill 2M tail ran", flush=True)
    del ws
    host = {kk: x[kk].cpu() for kk in ("q", "k", "v", "q_idx", "k_idx")}
    for lo in (q_begin, q_begin + 509, T - 8):
        rows = np.arange(lo, lo + 8)
        res = orc.prefill(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], k,
                          rows=rows)
        got_out = out[lo:lo + 8].float().cpu().numpy()
        got_idx = idx[lo - q_begin:lo - q_begin + 8].cpu().numpy()
        info = parity.check_prefill(host, rows, got_out, got_idx, None, res, k, q_begin=lo,
                                    out_offset=lo, label=f"2M rows {lo}")
        print(lo, info, flush=True)
