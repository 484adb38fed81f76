"""CPU checks of the comparison helpers the GPU parity tests use (tests/parity.py)."""

import numpy as np
import pytest

from block_sparse_long_05_amd import synth
from oracle import msa_oracle as orc
from tests import parity


def _fp32_block_scores(q_row, k_rows, b, order):
    """fp32 token scores summed term by term in a given order (a stand-in for a device's
    fp32 accumulation), max-pooled per block."""
    q = orc.as_f64(orc.host(q_row)).astype(np.float32)
    k = orc.as_f64(orc.host(k_rows[: b * orc.BLOCK])).astype(np.float32)
    terms = (k * q[None, :])[:, order]              # fp32 products
    acc = np.zeros(len(k), dtype=np.float32)
    for i in range(terms.shape[1]):
        acc = acc + terms[:, i]                      # one fp32 rounding per add
    return acc.reshape(b, orc.BLOCK).max(axis=1).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_score_bound_covers_fp32_accumulation(dtype):
    """Planted index keys make small scores out of large terms (cancellation): an fp32 sum
    in any order stays within block_score_bounds of the fp64 oracle, while the error can
    exceed 2e-5 of the score itself (the relative tolerance this bound replaced). A block
    score taken from the wrong block fails the check."""
    B, L, G = 2, 4000, 8
    x = synth.decode_inputs(B, L, G, 8, 128, 128, dtype=dtype, seed=31, planted_per_group=4)
    res = orc.decode(x["q"], x["k_cache"], x["v_cache"], x["q_idx"], x["k_idx"],
                     x["seq_lens"], 16)
    rng = np.random.default_rng(0)
    nblk = L // 128
    bs = np.zeros((B, G, nblk), dtype=np.float32)
    worst_rel = 0.0
    for (i, g), ref in res["block_scores"].items():
        b = len(ref)
        got = _fp32_block_scores(x["q_idx"][i, g], x["k_idx"][i], b, rng.permutation(128))
        bs[i, g, :b] = got
        worst_rel = max(worst_rel, float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))))
    ops = lambda i, g: (x["q_idx"][i, g], x["k_idx"][i])
    ratio = parity.check_block_scores(bs, res["block_scores"], lambda i: i, ops)
    assert 0.0 < ratio <= 1.0
    if dtype == "f32":
        assert worst_rel > 2e-6      # errors well beyond one rounding of the score
    wrong = bs.copy()
    wrong[1, 3, 5] = wrong[1, 3, 6]
    with pytest.raises(AssertionError):
        parity.check_block_scores(wrong, res["block_scores"], lambda i: i, ops)
    off = bs.copy()
    off[0, 2, 7] += 0.05
    with pytest.raises(AssertionError):
        parity.check_block_scores(off, res["block_scores"], lambda i: i, ops)
