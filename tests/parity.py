"""Comparison helpers for the GPU parity tests: HIP results vs the CPU oracle.

Tolerances (outputs, max abs): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with fp32
accumulation. Selected block sets must match bit for bit except on rows the oracle
declares near ties (relative gap < 1e-5 between the last selected and the first
unselected block score, computed in fp64); such rows are counted, and their outputs
are checked against the oracle's attention over the GPU's own selection.
"""

import numpy as np
import torch

from oracle import msa_oracle as orc

OUT_TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
# Softmax normalisers ln sum exp(s / sqrt(D)): fp32 logits of exact products (bf16) or fp32
# MFMA (fp32), fp32 sums of fp32 exponentials; absolute errors are ~1e-6 on values ~10.
LSE_TOL = 1e-4
# Block scores: fp32 accumulation of the d_idx products of a token score. Whatever the
# summation order, |fl(sum_i x_i) - sum_i x_i| <= gamma * sum_i |x_i| with gamma ~ n u
# (u = 2^-24; bf16 products are exact in fp32, fp32 products add one rounding each), and a
# block maximum moves by at most the largest error of its tokens. So a block score may be
# off by SCORE_GAMMA_PER_DIM * d * A_c, where A_c = max_{j in block c} sum_i |q_i k_ji|:
# a bound that follows the cancellation inside each dot product (a small score made of
# large terms), which a tolerance relative to the score itself does not.
SCORE_GAMMA_PER_DIM = 1.01 * 2.0 ** -24


def np32(x):
    return x.detach().float().cpu().numpy()


def block_score_bounds(q_row, k_rows, b):
    """Per-block error bounds of the device's fp32 block scores of one index-query row:
    q_row [d], k_rows [>= 128 b, d] (host tensors or arrays)."""
    q = np.abs(orc.as_f64(orc.host(q_row)))
    k = np.abs(orc.as_f64(orc.host(k_rows[: b * orc.BLOCK])))
    a = (k @ q).reshape(b, orc.BLOCK).max(axis=1)
    return (len(q) + 2) * SCORE_GAMMA_PER_DIM * a


def check_block_scores(bs_gpu, oracle_scores, row_map, operands, label=""):
    """oracle_scores {(i, g): fp64 scores of blocks 0..b-1}; row_map i -> gpu row;
    operands(i, g) -> (index query row, index key rows) of that oracle row. Returns the
    worst ratio of error to bound."""
    worst = 0.0
    for (i, g), ref in oracle_scores.items():
        if not len(ref):
            continue
        got = bs_gpu[row_map(i), g, : len(ref)].astype(np.float64)
        bound = block_score_bounds(*operands(i, g), len(ref)) + 1e-30
        ratio = float(np.max(np.abs(got - ref) / bound))
        assert ratio <= 1.0, (
            f"{label} block score of row {i} group {g}: error {np.max(np.abs(got - ref))} "
            f"beyond the fp32 accumulation bound (ratio {ratio})")
        worst = max(worst, ratio)
    return worst


def validate_tie_selection(sel_row, scores, b, top_k, label=""):
    """A device selection on a row the oracle declares a near tie must still be a valid
    selection under the rule (researchpapers.dev summary, "Mechanism": the local block is
    always kept; the others are the best-scoring earlier blocks), with only blocks whose
    fp64 scores sit within the near-tie gap of the cut allowed to trade places:
      * ids ascending and distinct, the local block b last, the others in [0, b), exactly
        min(top_k, b + 1) of them, -1 after;
      * every chosen earlier block scores >= r_k - gap and every unchosen earlier block
        <= r_{k-1} + gap, where r_{k-1} >= r_k are the (k-1)-th and k-th best earlier
        scores (the oracle's last kept and first dropped) and gap = 1e-5 * max(|r_{k-1}|,
        |r_k|), the near-tie threshold."""
    sel_row = np.asarray(sel_row).astype(np.int64)
    n = min(top_k, b + 1)
    ids, pad = sel_row[:n], sel_row[n:]
    assert np.all(pad == -1), f"{label}: padding {pad.tolist()}"
    assert np.all(np.diff(ids) > 0), f"{label}: ids not ascending/distinct {ids.tolist()}"
    assert ids[-1] == b, f"{label}: local block {b} missing from {ids.tolist()}"
    others = ids[:-1]
    assert len(others) == 0 or (others.min() >= 0 and others.max() < b), (
        f"{label}: ids outside [0, {b}) in {ids.tolist()}")
    if b + 1 <= top_k:
        return
    scores = np.asarray(scores, dtype=np.float64)[:b] + 0.0
    ranked = np.sort(scores)[::-1]
    r_last, r_next = ranked[top_k - 2], ranked[top_k - 1]
    gap = orc.NEAR_TIE_REL * max(abs(r_last), abs(r_next))
    chosen = np.zeros(b, dtype=bool)
    chosen[others] = True
    assert np.all(scores[chosen] >= r_next - gap), (
        f"{label}: a kept block scores {scores[chosen].min()} < cut {r_next}")
    if (~chosen).any():
        assert np.all(scores[~chosen] <= r_last + gap), (
            f"{label}: a dropped block scores {scores[~chosen].max()} > cut {r_last}")


def check_selection(idx_gpu, res, top_k, local_blocks, label=""):
    """idx_gpu [R, G, top_k]: the device's ids for the R oracle rows of `res` (an oracle
    prefill/decode result), local_blocks [R] the rows' local blocks. Rows must match the
    oracle bit for bit unless the oracle declares a near tie; on such rows the device's
    set must pass validate_tie_selection against the oracle's fp64 block scores.
    Returns the set of (i, g) rows whose selection differs."""
    ref = orc.selection_array(res["sel"], top_k)
    diff = np.any(idx_gpu != ref, axis=2)
    bad = diff & ~res["near_tie"]
    assert not bad.any(), (
        f"{label}: {int(bad.sum())} rows differ without a near tie, first "
        f"{np.argwhere(bad)[:5].tolist()}")
    differ = {tuple(x) for x in np.argwhere(diff).tolist()}
    for (i, g) in differ:
        b = int(local_blocks[i])
        validate_tie_selection(idx_gpu[i, g], res["block_scores"][(i, g)], b, top_k,
                               label=f"{label} row {i} group {g}")
    return differ


def check_prefill(x, rows, out_gpu, idx_gpu, bs_gpu, res, top_k, q_begin=0, out_offset=0,
                  label="", lse_gpu=None):
    """Compare a prefill run for oracle rows `rows` (absolute token ids). idx_gpu and
    bs_gpu start at row q_begin, out_gpu at row out_offset."""
    dtype = x["q"].dtype
    tol = OUT_TOL[dtype]
    G = x["k"].shape[0]
    Hpg = x["q"].shape[1] // G
    rows = np.asarray(rows)
    idx_rows = idx_gpu[rows - q_begin]
    differ = check_selection(idx_rows, res, top_k, rows // orc.BLOCK, label)
    if bs_gpu is not None:
        check_block_scores(bs_gpu, res["block_scores"], lambda i: rows[i] - q_begin,
                           lambda i, g: (x["q_idx"][int(rows[i]), g], x["k_idx"]), label)
    got = out_gpu[rows - out_offset].astype(np.float64)
    ref = res["out"].copy()
    for (i, g) in differ:
        t = int(rows[i])
        hs = slice(g * Hpg, (g + 1) * Hpg)
        ref[i, hs] = orc.attend_on_selection(x["q"][t, hs], x["k"][g], x["v"][g],
                                             idx_rows[i, g], t)
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, f"{label}: max abs err {err} > {tol}"
    info = dict(err=err, near_ties=int(res["near_tie"].sum()), differ=len(differ))
    if lse_gpu is not None:  # rows whose selection differs (near ties) are left out
        keep = np.ones((len(rows), G), dtype=bool)
        for (i, g) in differ:
            keep[i, g] = False
        keep = np.repeat(keep, Hpg, axis=1)
        lerr = np.abs(lse_gpu[rows - out_offset].astype(np.float64) - res["lse"])[keep]
        info["lse_err"] = float(lerr.max()) if lerr.size else 0.0
        assert info["lse_err"] <= LSE_TOL, f"{label}: lse max abs err {info['lse_err']}"
    return info


def check_decode(x, out_gpu, idx_gpu, bs_gpu, res, top_k, label=""):
    dtype = x["q"].dtype
    tol = OUT_TOL[dtype]
    G = x["k_cache"].shape[1]
    Hpg = x["q"].shape[1] // G
    lens = x["seq_lens"].cpu().numpy()
    differ = check_selection(idx_gpu, res, top_k, (lens - 1) // orc.BLOCK, label)
    if bs_gpu is not None:
        check_block_scores(bs_gpu, res["block_scores"], lambda i: i,
                           lambda i, g: (x["q_idx"][i, g], x["k_idx"][i]), label)
    got = out_gpu.astype(np.float64)
    ref = res["out"].copy()
    for (b, g) in differ:
        hs = slice(g * Hpg, (g + 1) * Hpg)
        ref[b, hs] = orc.attend_on_selection(x["q"][b, hs], x["k_cache"][b, g],
                                             x["v_cache"][b, g], idx_gpu[b, g], int(lens[b]) - 1)
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, f"{label}: max abs err {err} > {tol}"
    return dict(err=err, near_ties=int(res["near_tie"].sum()), differ=len(differ))


# ---- index-branch KL loss ---------------------------------------------------------------
# The device keeps P and I in fp32 (relative errors ~1e-6: fp32 accumulation of exact bf16
# products, the hardware exp2) and rounds W = index_scale (I - P) to bf16 for the two
# gradient products. bf16 holds 8 significant bits, so that rounding moves each term by at
# most 2^-8 of itself, and |err| <= 2^-8 sum_j |W_j| |x_j| is the worst case (x the other
# operand: k_idx rows for dq, q_idx rows for dk); measured errors reach 0.6-0.8 of it, and
# match a bf16-W emulation of the oracle to ~1e-8. Per element:
#   loss:   |err| <= KL_LOSS_REL * (1 + sum_j P_j |ln P_j - ln I_j|)     (measured < 1e-6)
#   dq, dk: |err| <= 2 * 2^-8 * sum_j |W_j| |x_j|
#                    + KL_MASS_REL * index_scale * sum_j (P_j + I_j) |x_j|
# the last term covering the fp32 errors of P and I where W cancels (I ~ P).
KL_LOSS_REL = 2e-5
KL_W_REL = 2.0 ** -7
KL_MASS_REL = 1e-5


def check_kl(loss, dq, ref, rows_gpu, dk=None, label=""):
    """loss [n, G], dq [n, G, d] of the device rows rows_gpu vs the oracle dict `ref` of the
    same rows; dk (the whole [T, d] gradient) vs ref["dk_idx"] when given."""
    got_l = loss[rows_gpu].astype(np.float64)
    tol_l = KL_LOSS_REL * (1.0 + ref["loss_abs"])
    err_l = np.abs(got_l - ref["loss"])
    assert (err_l <= tol_l).all(), (
        f"{label} loss: {int((err_l > tol_l).sum())} rows off, worst {float(err_l.max())}")
    got_q = dq[rows_gpu].astype(np.float64)
    tol_q = KL_W_REL * ref["dq_abs"] + KL_MASS_REL * ref["mass_abs"] + 1e-7
    err_q = np.abs(got_q - ref["dq_idx"])
    assert (err_q <= tol_q).all(), (
        f"{label} dq_idx: {int((err_q > tol_q).sum())} values off, worst ratio "
        f"{float((err_q / tol_q).max())}")
    out = dict(loss_max_err=float(err_l.max()), dq_worst_ratio=float((err_q / tol_q).max()))
    if dk is not None:
        tol_k = KL_W_REL * ref["dk_abs"] + KL_MASS_REL * ref["dk_mass"] + 1e-7
        err_k = np.abs(dk.astype(np.float64) - ref["dk_idx"])
        assert (err_k <= tol_k).all(), (
            f"{label} dk_idx: {int((err_k > tol_k).sum())} values off, worst ratio "
            f"{float((err_k / tol_k).max())}")
        out["dk_worst_ratio"] = float((err_k / tol_k).max())
    return out
