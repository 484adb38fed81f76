"""The allocation-free decode entry (msa_sparse_attn_decode_noalloc) against the regular
msa_sparse_attn_decode on the same data: bit-identical outputs, on two calls in a row
whose second problem is smaller (the scratch keeps the first call's contents), for bf16
and fp32, and the oracle's tolerance on the first case."""

import numpy as np
import pytest
import torch

from block_sparse_long_05_amd import msa, synth
from oracle import msa_oracle as orc
from tests import parity

pytestmark = pytest.mark.gpu


def _case(B, L, G, Hpg, top_k, dtype, lens, seed):
    x = synth.decode_inputs(B, L, G, Hpg, 128, 128, dtype=dtype, seed=seed,
                            planted_per_group=4, seq_lens=lens)
    xd = {k: v.cuda() for k, v in x.items()}
    p = msa.decode_problem(xd, top_k)
    bs = msa.alloc_block_scores(p)
    idx = msa.alloc_block_idx(p)
    msa.msa_index_scores(p, xd["q_idx"], xd["k_idx"], bs)
    msa.msa_block_topk(p, bs, idx)
    ref = torch.zeros_like(xd["q"])
    ws = msa.alloc_workspace(p, "sparse_attn_decode")
    msa.msa_sparse_attn_decode(p, xd["q"], xd["k_cache"], xd["v_cache"], idx, ref, ws)
    torch.cuda.synchronize()
    return x, xd, p, idx, bs, ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_regular_entry(dtype):
    big = _case(6, 5000, 8, 8, 16, dtype, [5000, 4097, 3000, 129, 1, 4500], seed=31)
    small = _case(2, 3000, 4, 3, 6, dtype, [3000, 700], seed=32)
    for label, (x, xd, p, idx, bs, ref) in (("first", big), ("second, smaller", small)):
        print(f"noalloc decode {dtype} {label}: B={p.batch} G={p.num_groups} "
              f"Hpg={p.heads_per_group} k={p.top_k}", flush=True)
        out = torch.full_like(xd["q"], float("nan"))
        msa.msa_sparse_attn_decode_noalloc(p, xd["q"], xd["k_cache"], xd["v_cache"], idx, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), label
    # the first case against the oracle as well (same bar as the regular decode tests)
    x, xd, p, idx, bs, ref = big
    out = torch.zeros_like(xd["q"])
    msa.msa_sparse_attn_decode_noalloc(p, xd["q"], xd["k_cache"], xd["v_cache"], idx, out)
    torch.cuda.synchronize()
    res = orc.decode(x["q"], x["k_cache"], x["v_cache"], x["q_idx"], x["k_idx"], x["seq_lens"],
                     p.top_k)
    print(parity.check_decode(x, parity.np32(out), idx.cpu().numpy(), parity.np32(bs), res,
                              p.top_k, label="noalloc"))


def test_noalloc_decode_rejects_too_large():
    """A problem beyond the fixed scratch is refused before any launch."""
    x = synth.decode_inputs(64, 256, 8, 8, 128, 128, dtype="bf16", seed=3)
    xd = {k: v.cuda() for k, v in x.items()}
    p = msa.decode_problem(xd, 16)
    assert msa.msa_workspace_size(p, "sparse_attn_decode") > msa.NOALLOC_SCRATCH_BYTES
    idx = msa.alloc_block_idx(p)
    out = torch.zeros_like(xd["q"])
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_attn_decode_noalloc(p, xd["q"], xd["k_cache"], xd["v_cache"], idx, out)
    assert e.value.status == msa.MSA_ERR_TOO_LARGE
