"""The hot path under HIP graph capture: a decode step and a prefill, each captured once
through the C ABI (torch.cuda.graph) and replayed with new inputs written in place between
the replays, with eager library work and synchronizations in between. Every replay must
give exactly the eager result for the same inputs (the library records no memset and
allocates nothing inside its calls; all scratch comes from the caller's workspace)."""

import pytest
import torch

from block_sparse_long_05_amd import msa, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # first run outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return g


def test_decode_step_graph_replays():
    """Index scan + selection/attention/combine captured once; replays with new queries,
    new caches and grown sequence lengths match eager calls bit for bit."""
    B, L, G, Hpg, top_k = 3, 5000, 4, 8, 8
    x = synth.decode_inputs(B, L, G, Hpg, 128, 128, dtype="bf16", seed=31, planted_per_group=2,
                            seq_lens=[4000, 2500, 700], device=DEV)
    p = msa.decode_problem(x, top_k)
    bs = msa.alloc_block_scores(p)
    idx = msa.alloc_block_idx(p)
    out = torch.empty_like(x["q"])
    ws = msa.alloc_workspace(p, "sparse_attn_decode")

    def step():
        msa.msa_index_scores(p, x["q_idx"], x["k_idx"], bs)
        msa.msa_sparse_attn_decode_topk(p, x["q"], x["k_cache"], x["v_cache"], bs, idx, out, ws)

    g = _capture(step)
    gen = torch.Generator(device=DEV).manual_seed(7)
    for rep in range(4):
        print(f"decode graph replay {rep}", flush=True)
        for name in ("q", "q_idx"):
            x[name].copy_(torch.randn(x[name].shape, generator=gen, device=DEV))
        x["k_cache"][:, :, 64 * rep:64 * rep + 64].normal_(generator=gen)
        x["seq_lens"].copy_(torch.tensor([4000 + 300 * rep, 2500 + 7 * rep, 700 + 128 * rep],
                                         dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        got_out, got_idx = out.clone(), idx.clone()
        ref_out, ref_idx, _ = msa.decode(x, top_k)  # eager, separate selection, new buffers
        torch.cuda.synchronize()
        assert torch.equal(got_idx, ref_idx), rep
        assert torch.equal(got_out, ref_out), rep


def test_prefill_graph_replays():
    """Fused index branch + hybrid sparse attention (with lse) captured once; replays with
    new inputs match eager calls bit for bit."""
    T, G, Hpg, top_k = 3000, 2, 8, 8
    x = synth.prefill_inputs(T, G, Hpg, 128, 128, dtype="bf16", seed=32, planted_per_group=3,
                             device=DEV)
    p = msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                    index_dim=128, top_k=top_k, seq_len=T, q_begin=0, q_count=T)
    idx = msa.alloc_block_idx(p)
    out = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:2], dtype=torch.float32, device=DEV)
    ws = msa.alloc_workspace(p, "sparse_attn_prefill")

    def step():
        msa.msa_index_topk(p, x["q_idx"], x["k_idx"], idx)
        msa.msa_sparse_attn_prefill(p, x["q"], x["k"], x["v"], idx, out, ws, lse=lse)

    g = _capture(step)
    gen = torch.Generator(device=DEV).manual_seed(8)
    for rep in range(3):
        print(f"prefill graph replay {rep}", flush=True)
        for name in ("q", "q_idx", "k_idx", "v"):
            x[name].copy_(torch.randn(x[name].shape, generator=gen, device=DEV))
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), idx.clone(), lse.clone())
        ref_lse = torch.empty_like(lse)
        ref_out, ref_idx, _ = msa.prefill(x, top_k, index="fused", lse=ref_lse)
        torch.cuda.synchronize()
        assert torch.equal(got[1], ref_idx), rep
        assert torch.equal(got[0], ref_out), rep
        assert torch.equal(got[2], ref_lse), rep
