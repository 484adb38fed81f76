"""GPU parity of the index-branch KL loss and gradients (msa_index_kl_prefill, through the
C ABI) against the CPU oracle, on seeded random selections: several workgroup units per
block (blocks that every row keeps), ragged tails, chunked calls that accumulate the key
gradient, padding and invisible ids."""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_05_amd import msa, synth
from oracle import msa_oracle as orc
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(T, G, Hpg, seed):
    return synth.prefill_inputs(T, G, Hpg, 128, 128, dtype="bf16", seed=seed)


def _dev(x):
    return {k: v.to(DEV) for k, v in x.items() if k in ("q", "k", "q_idx", "k_idx")}


_ORACLE = {}


def _oracle_cached(key, x, sel, scale):
    if key not in _ORACLE:
        _ORACLE[key] = orc.index_kl(x["q"], x["k"], x["q_idx"], x["k_idx"], sel, scale)
    return _ORACLE[key]


def _oracle(x, sel, scale, q_begin=0, rows=None):
    return orc.index_kl(x["q"], x["k"], x["q_idx"], x["k_idx"], sel, scale, q_begin=q_begin,
                        rows=rows)


CASES = [
    # T, G, Hpg, top_k, popular blocks per group, index_scale, seed
    (700, 2, 3, 3, 1, 0.2, 1),
    (2100, 8, 8, 16, 4, 1.0 / math.sqrt(128), 2),   # 16 blocks x 128 tokens, 8 x 8 heads
    (100, 1, 1, 1, 0, 0.05, 3),                      # one partial block
    (1333, 4, 2, 6, 2, 0.3, 4),
    (600, 1, 16, 3, 1, 0.3, 5),                      # 16 heads per group (the maximum)
    (1500, 2, 4, 24, 2, 0.15, 6),                    # top_k 24 > blocks: padded rows
]


@pytest.mark.parametrize("T,G,Hpg,top_k,popular,scale,seed", CASES)
def test_index_kl_matches_oracle(T, G, Hpg, top_k, popular, scale, seed):
    print(f"index kl T={T} G={G} Hpg={Hpg} k={top_k} scale={scale:.4f}", flush=True)
    x = _inputs(T, G, Hpg, seed)
    sel = synth.random_selection(T, G, top_k, seed=seed, popular_per_group=popular)
    loss, dq, dk = msa.index_kl(_dev(x), sel.to(DEV), top_k, scale)
    torch.cuda.synchronize()
    ref = _oracle_cached((T, G, Hpg, top_k, popular, scale, seed), x, sel.numpy(), scale)
    print(parity.check_kl(parity.np32(loss), parity.np32(dq), ref, np.arange(T),
                          parity.np32(dk), label=f"T={T}"))


def test_index_kl_chunks_accumulate_and_repeat():
    """Two chunked calls add their key gradients into one buffer; loss and dq_idx rows are
    chunk-relative; a second run gives bit-identical loss and dq_idx."""
    T, G, Hpg, top_k, scale = 1500, 4, 2, 5, 0.25
    print(f"index kl chunks T={T}", flush=True)
    x = _inputs(T, G, Hpg, 7)
    xd = _dev(x)
    sel = synth.random_selection(T, G, top_k, seed=7, popular_per_group=2)
    seld = sel.to(DEV)
    dk = torch.zeros((T, 128), dtype=torch.float32, device=DEV)
    l0, q0, _ = msa.index_kl(xd, seld[:700].contiguous(), top_k, scale, 0, 700, dk_idx=dk)
    l1, q1, _ = msa.index_kl(xd, seld[700:].contiguous(), top_k, scale, 700, 800, dk_idx=dk)
    l1b, q1b, _ = msa.index_kl(xd, seld[700:].contiguous(), top_k, scale, 700, 800,
                               dk_idx=torch.zeros_like(dk))
    torch.cuda.synchronize()
    assert torch.equal(l1, l1b) and torch.equal(q1, q1b)
    ref = _oracle(x, sel.numpy(), scale)
    loss = np.concatenate([parity.np32(l0), parity.np32(l1)])
    dq = np.concatenate([parity.np32(q0), parity.np32(q1)])
    parity.check_kl(loss, dq, ref, np.arange(T), parity.np32(dk), label="chunks")


def test_index_kl_padding_and_invisible_ids():
    """Rows whose ids are all padding get loss 0 and zero dq_idx; ids above a row's local
    block are ignored like padding."""
    T, G, Hpg, top_k, scale = 900, 2, 2, 4, 0.3
    print("index kl padding", flush=True)
    x = _inputs(T, G, Hpg, 11)
    sel = synth.random_selection(T, G, top_k, seed=11, popular_per_group=1).clone()
    sel[100:140] = -1
    sel[600, 0, 0] = 6                        # token 600 is in block 4: block 6 is invisible
    sel[601, 1, :] = torch.tensor([0, 4, 5, 6], dtype=torch.int32)
    loss, dq, dk = msa.index_kl(_dev(x), sel.to(DEV), top_k, scale)
    torch.cuda.synchronize()
    assert (parity.np32(loss)[100:140] == 0).all() and (parity.np32(dq)[100:140] == 0).all()
    ref = _oracle(x, sel.numpy(), scale)
    parity.check_kl(parity.np32(loss), parity.np32(dq), ref, np.arange(T), parity.np32(dk),
                    label="padding")


@pytest.mark.parametrize("algo", ["auto", "query_centric"])
def test_index_kl_with_main_lse(algo):
    """With the main heads' normalisers taken from msa_sparse_attn_prefill's lse output (same
    selection), the loss and gradients still match the oracle and the standalone call."""
    T, G, Hpg, top_k, scale = 2100, 8, 8, 16, 1.0 / math.sqrt(128)
    print(f"index kl with main lse ({algo})", flush=True)
    x = _inputs(T, G, Hpg, 2)
    xd = _dev(x)
    xd["v"] = x["v"].to(DEV)
    sel = synth.random_selection(T, G, top_k, seed=2, popular_per_group=4)
    seld = sel.to(DEV)
    p = msa.Problem(dtype="bf16", mode="prefill", num_groups=G, heads_per_group=Hpg,
                    index_dim=128, top_k=top_k, seq_len=T, q_begin=0, q_count=T, algo=algo)
    lse = torch.empty((T, G * Hpg), dtype=torch.float32, device=DEV)
    msa.msa_sparse_attn_prefill(p, xd["q"], xd["k"], xd["v"], seld, torch.empty_like(xd["q"]),
                                msa.alloc_workspace(p, "sparse_attn_prefill"), lse=lse)
    loss, dq, dk = msa.index_kl(xd, seld, top_k, scale, main_lse=lse)
    loss0, dq0, dk0 = msa.index_kl(xd, seld, top_k, scale)
    torch.cuda.synchronize()
    ref = _oracle_cached((T, G, Hpg, top_k, 4, scale, 2), x, sel.numpy(), scale)
    print(parity.check_kl(parity.np32(loss), parity.np32(dq), ref, np.arange(T),
                          parity.np32(dk), label="main lse"))
    assert float((loss - loss0).abs().max()) < 1e-4
