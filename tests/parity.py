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
# Block scores: fp32 accumulation of d_idx products against the fp64 oracle.
SCORE_RTOL = 2e-5


def np32(x):
    return x.detach().float().cpu().numpy()


def check_block_scores(bs_gpu, oracle_scores, row_map, label=""):
    """oracle_scores {(i, g): fp64 scores of blocks 0..b-1}; row_map i -> gpu row."""
    worst = 0.0
    for (i, g), ref in oracle_scores.items():
        got = bs_gpu[row_map(i), g, : len(ref)].astype(np.float64)
        scale = np.maximum(1.0, np.abs(ref))
        err = float(np.max(np.abs(got - ref) / scale)) if len(ref) else 0.0
        worst = max(worst, err)
    assert worst <= SCORE_RTOL, f"{label} block score rel err {worst}"
    return worst


def check_selection(idx_gpu, oracle_sel, near_tie, top_k, label=""):
    """Returns the set of (i, g) rows whose selection differs (all near ties)."""
    ref = orc.selection_array(oracle_sel, top_k)
    diff = np.any(idx_gpu != ref, axis=2)
    bad = diff & ~near_tie
    assert not bad.any(), (
        f"{label}: {int(bad.sum())} rows differ without a near tie, first "
        f"{np.argwhere(bad)[:5].tolist()}")
    return {tuple(x) for x in np.argwhere(diff).tolist()}


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
    differ = check_selection(idx_rows, res["sel"], res["near_tie"], top_k, label)
    if bs_gpu is not None:
        check_block_scores(bs_gpu, res["block_scores"], lambda i: rows[i] - q_begin, label)
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
    differ = check_selection(idx_gpu, res["sel"], res["near_tie"], top_k, label)
    if bs_gpu is not None:
        check_block_scores(bs_gpu, res["block_scores"], lambda i: i, label)
    got = out_gpu.astype(np.float64)
    ref = res["out"].copy()
    lens = x["seq_lens"].cpu().numpy()
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
