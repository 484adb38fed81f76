"""Plain CPU oracle of the MiniMax Sparse Attention (MSA) hot path, in NumPy float64.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this module:
only the test suite, the package smoke check and the benchmark's CPU-baseline leg use
it. It shares no code, table or helper with the HIP kernels.

What it computes, and where the pages say so:

* Index branch (mlqm.cn blog on the MiniMax M3 sparse attention, section 2.1;
  researchpapers.dev MSA summary, "Mechanism"): one index query per GQA group is
  dotted with the single shared index-key head, s_j = Q_idx[t, g] . K_idx[j]; the
  token scores are reduced to one score per 128-token block by max pooling; per
  (query, group) the top-k blocks are kept and the most recent (local) block is
  always kept. Only visible tokens are scored.
* Main branch (same blog, section 2.2, the gather + flash-attention pseudo-code;
  researchpapers.dev summary, "Mechanism": exact softmax attention on the selected
  blocks): every query head of the group attends, with exact softmax, to the keys of
  the selected blocks that are causally visible, O = softmax(q K^T / sqrt(d)) V
  (the scaled dot-product formula of the Lightning-attention explainer, section 2.1).
* Budget: 16 blocks of 128 tokens per query group (researchpapers.dev summary,
  "2048 KV tokens").

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):
  R1 index score = raw dot product, no scale (any positive scale keeps the ranking);
  R2 block c covers tokens [128c, 128c + 127];
  R3 causal: query t sees j <= t; local block b = t // 128; blocks > b are never chosen;
  R4 top_k counts the local block: Sel = {b} + the (top_k - 1) best of blocks [0, b);
  R5 when b + 1 <= top_k every visible block is selected;
  R6 ranking: higher block score first, then lower block index (-0.0 == +0.0);
  R7 near tie: last selected vs first unselected non-local score, relative gap < 1e-5;
  R8 head h belongs to group h // Hpg;
  R9 attention scale 1 / sqrt(head_dim);
  R11 decode: a cache of L tokens holds the current token, whose position is L - 1.

The inputs may be NumPy arrays or torch tensors (fp32 / bf16); each slice a row
uses is widened exactly to float64 when it is used.
"""

from __future__ import annotations

import math

import numpy as np
import scipy.sparse

BLOCK = 128
NEAR_TIE_REL = 1e-5


class BF16Bits:
    """bf16 data held as its raw 16-bit patterns (a NumPy uint16 array), so that slicing
    stays in NumPy and widening is exact: the pattern is the top half of an fp32."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, i):
        return BF16Bits(self.bits[i])

    def __len__(self):
        return len(self.bits)


def host(x):
    """Zero-copy NumPy view of an input (torch CPU tensor or NumPy array)."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach()
        if x.device.type != "cpu":
            x = x.cpu()
        if x.dtype == torch.bfloat16:
            return BF16Bits(x.view(torch.int16).numpy().view(np.uint16))
        return x.numpy()
    return x


_WIDEN_AT_ENTRY = 1 << 24  # inputs up to this many elements are widened once, up front


def host_small_f64(x):
    """host(x), already widened to float64 when it is small."""
    x = host(x)
    n = int(np.prod(x.shape)) if len(x.shape) else 1
    return as_f64(x) if n <= _WIDEN_AT_ENTRY else x


def as_f64(x) -> np.ndarray:
    """Exact widening of fp32 / bf16 / fp64 data to float64."""
    if hasattr(x, "detach"):
        x = host(x)
    if isinstance(x, BF16Bits):
        return (x.bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------
# Index branch
# ----------------------------------------------------------------------------------

def index_block_scores(q_idx_rows: np.ndarray, k_idx: np.ndarray, b: int,
                       block: int = BLOCK) -> np.ndarray:
    """Block scores of blocks 0..b-1 for index-query rows that share local block b.

    q_idx_rows [R, d_idx]; k_idx [>= b*block, d_idx]. Token scores are the matrix
    product Q_idx . K_idx^T over the keys of the fully visible blocks (blog section
    2.1), and a block's score is the max over its 128 token scores (block max
    pooling, same section). Returns [R, b].
    """
    keys = k_idx[: b * block]
    s = q_idx_rows @ keys.T                      # [R, b*block] token scores
    return s.reshape(s.shape[0], b, block).max(axis=2)


def select_blocks(block_scores: np.ndarray, b: int, top_k: int):
    """Blocks kept for one (query, group) row whose local block is b.

    block_scores holds the scores of blocks 0..b-1 (the local block is not scored:
    it is always kept, researchpapers.dev summary, "Mechanism"). Returns
    (ascending block ids, near_tie flag).
    """
    if b + 1 <= top_k:                           # R5: everything visible fits
        return np.arange(b + 1, dtype=np.int64), False
    scores = np.asarray(block_scores, dtype=np.float64)[:b] + 0.0   # -0.0 -> +0.0
    # R6: sort by score descending, then block index ascending.
    order = np.lexsort((np.arange(b), -scores))
    chosen = order[: top_k - 1]
    sel = np.sort(np.concatenate([chosen, [b]])).astype(np.int64)
    tie = False
    if top_k >= 2:
        hi = scores[order[top_k - 2]]            # last selected non-local score
        lo = scores[order[top_k - 1]]            # first unselected score
        den = max(abs(hi), abs(lo))
        tie = True if den == 0.0 else bool((hi - lo) / den < NEAR_TIE_REL)
    return sel, tie


# ----------------------------------------------------------------------------------
# Main branch
# ----------------------------------------------------------------------------------

def attend(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray,
           scale: float) -> np.ndarray:
    """Exact softmax attention of q_heads [H, D] over keys/values [n, D]."""
    logits = (q_heads @ keys.T) * scale
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ values) / p.sum(axis=1, keepdims=True)


def attend_lse(q_heads: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """Natural-log normaliser of each head's softmax: ln sum_j exp(q . k_j * scale), [H]."""
    logits = (q_heads @ keys.T) * scale
    m = logits.max(axis=1)
    return m + np.log(np.exp(logits - m[:, None]).sum(axis=1))


def visible_keys(sel, t: int, block: int = BLOCK) -> np.ndarray:
    """Token ids of the selected blocks that query position t can see (j <= t)."""
    parts = [np.arange(c * block, min(c * block + block, t + 1)) for c in sel]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _row(q_t, k_g, v_g, q_idx_tg, k_idx, t, top_k, block, scale, bs=None):
    """One (query, group): selection and attention. K/V rows are widened to float64
    only for the tokens the selection reaches."""
    b = t // block
    if b + 1 <= top_k:
        sel, tie = np.arange(b + 1, dtype=np.int64), False
    else:
        if bs is None:
            bs = index_block_scores(as_f64(q_idx_tg)[None, :], as_f64(k_idx[: b * block]), b,
                                    block)[0]
        sel, tie = select_blocks(bs, b, top_k)
    j = visible_keys(sel, t, block)
    qh, kk = as_f64(q_t), as_f64(k_g[j])
    return attend(qh, kk, as_f64(v_g[j]), scale), sel, tie, bs, attend_lse(qh, kk, scale)


def prefill(q, k, v, q_idx, k_idx, top_k: int, block: int = BLOCK, rows=None) -> dict:
    """Causal MSA prefill for the query positions `rows` (default: all).

    q [T, G*Hpg, D]; k, v [G, T, D]; q_idx [T, G, d_idx]; k_idx [T, d_idx].
    Returns dict(out [R, Hq, D], lse [R, Hq] (ln of each head's softmax normaliser),
    sel [R][G] -> ascending ids, near_tie [R, G] bool,
    block_scores {(i, g): array of b scores} for rows that were scored, rows [R]).
    Inputs are widened to float64 slice by slice, as each row needs them.
    """
    q, k, v = host_small_f64(q), host_small_f64(k), host_small_f64(v)
    q_idx, k_idx = host_small_f64(q_idx), host_small_f64(k_idx)
    T, Hq, D = q.shape
    G = k.shape[0]
    Hpg = Hq // G
    scale = 1.0 / math.sqrt(D)                   # R9
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, D))
    lse = np.zeros((len(rows), Hq))
    sel_all = [[None] * G for _ in rows]
    tie = np.zeros((len(rows), G), dtype=bool)
    scores = {}
    # Rows sharing a local block b see the same keys, so their block scores come
    # from one matrix product Q_idx . K_idx^T.
    by_block = {}
    for i, t in enumerate(rows.tolist()):
        by_block.setdefault(t // block, []).append(i)
    for b, idxs in by_block.items():
        bs_rows = None
        if b + 1 > top_k:
            qi = as_f64(q_idx[rows[idxs]]).reshape(len(idxs) * G, -1)
            bs_rows = index_block_scores(qi, as_f64(k_idx[: b * block]), b, block)
            bs_rows = bs_rows.reshape(len(idxs), G, b)
        for n, i in enumerate(idxs):
            t = int(rows[i])
            for g in range(G):
                hs = slice(g * Hpg, (g + 1) * Hpg)   # R8
                bs = None if bs_rows is None else bs_rows[n, g]
                o, sel, tg, bs, ls = _row(q[t, hs], k[g], v[g], q_idx[t, g], k_idx, t, top_k,
                                          block, scale, bs)
                out[i, hs] = o
                lse[i, hs] = ls
                sel_all[i][g] = sel
                tie[i, g] = tg
                if bs is not None:
                    scores[(i, g)] = bs
    return dict(out=out, lse=lse, sel=sel_all, near_tie=tie, block_scores=scores, rows=rows)


def decode(q, k_cache, v_cache, q_idx, k_idx, seq_lens, top_k: int,
           block: int = BLOCK) -> dict:
    """One MSA decode step for B sequences.

    q [B, G*Hpg, D]; k_cache, v_cache [B, G, Lmax, D]; q_idx [B, G, d_idx];
    k_idx [B, Lmax, d_idx]; seq_lens [B]. The query sits at position L_b - 1 (R11).
    """
    lens = [int(x) for x in np.asarray(as_f64(seq_lens)).tolist()]
    q, k_cache, v_cache = host_small_f64(q), host_small_f64(k_cache), host_small_f64(v_cache)
    q_idx, k_idx = host_small_f64(q_idx), host_small_f64(k_idx)
    B, Hq, D = q.shape
    G = k_cache.shape[1]
    Hpg = Hq // G
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D))
    sel_all = [[None] * G for _ in range(B)]
    tie = np.zeros((B, G), dtype=bool)
    scores = {}
    for bi in range(B):
        t = lens[bi] - 1
        b = t // block
        bs_all = None
        if b + 1 > top_k:                        # all G index queries in one product
            bs_all = index_block_scores(as_f64(q_idx[bi]), as_f64(k_idx[bi][: b * block]), b,
                                        block)
        for g in range(G):
            hs = slice(g * Hpg, (g + 1) * Hpg)
            bs = None if bs_all is None else bs_all[g]
            o, sel, tg, bs, _ = _row(q[bi, hs], k_cache[bi, g], v_cache[bi, g], q_idx[bi, g],
                                  k_idx[bi], t, top_k, block, scale, bs)
            out[bi, hs] = o
            sel_all[bi][g] = sel
            tie[bi, g] = tg
            if bs is not None:
                scores[(bi, g)] = bs
    return dict(out=out, sel=sel_all, near_tie=tie, block_scores=scores)


# ----------------------------------------------------------------------------------
# Index-branch KL loss (training side)
#
# researchpapers.dev summary, "Mechanism": the Index Branch is trained with a KL loss
# towards the Main Branch's distribution on the selected blocks, and the gradient from
# the index path into the main attention is cut. Readings (the pages give no formula):
#   K1 the target P of a (query t, group g) row is the main branch's token-level
#      attention distribution over the visible tokens of the selected blocks, averaged
#      over the Hpg heads of the group (one index query serves the whole group);
#   K2 the index distribution I is a softmax of index_scale * q_idx[t, g] . k_idx[j]
#      over the same tokens (index_scale is the caller's temperature; selection is
#      unaffected by it);
#   K3 loss = KL(P || I) = sum_j P_j (ln P_j - ln I_j), with 0 ln 0 = 0;
#   K4 P is a constant (stop-gradient): gradients flow only into q_idx and k_idx,
#      and they are the gradients of the sum of the per-row losses;
#   K5 a row with no visible selected token has loss 0 and zero gradient.
# ----------------------------------------------------------------------------------

def kl_row(q_t, k_g, q_idx_tg, k_idx, sel, t: int, index_scale: float,
           block: int = BLOCK) -> dict:
    """KL(P || I) of one (query, group) row and its gradient.

    q_t [Hpg, D] the group's query heads at position t; k_g [T, D] the group's keys;
    q_idx_tg [d]; k_idx [T, d]; sel the selected block ids (ids < 0 ignored).
    Returns dict(loss, dq [d], keys (token ids), gx (d loss / d index score of each
    token, already times index_scale), p_plus_i (P_j + I_j), and the magnitude sums the device
    comparison uses: dq_abs = sum_j |gx_j| |k_idx[j]|, mass_abs = index_scale *
    sum_j (P_j + I_j) |k_idx[j]|, loss_abs = sum_j P_j |ln P_j - ln I_j|)."""
    q_t = as_f64(q_t)
    qi = as_f64(q_idx_tg)
    d = qi.shape[-1]
    sel = [int(c) for c in np.asarray(sel).ravel().tolist() if int(c) >= 0]
    keys = visible_keys(sel, t, block)
    if len(keys) == 0:                           # K5
        z = np.zeros(d)
        return dict(loss=0.0, dq=z, keys=keys, gx=np.zeros(0), p_plus_i=np.zeros(0),
                    dq_abs=z, mass_abs=z, loss_abs=0.0)
    D = q_t.shape[-1]
    kk = as_f64(k_g[keys])
    ki = as_f64(k_idx[keys])
    # main branch distribution per head (R9 scale), then the mean over the group (K1)
    logits = (q_t @ kk.T) / math.sqrt(D)
    logits = logits - logits.max(axis=1, keepdims=True)
    ph = np.exp(logits)
    ph = ph / ph.sum(axis=1, keepdims=True)
    P = ph.mean(axis=0)
    # index distribution (K2), kept in log form
    x = index_scale * (ki @ qi)
    xm = x.max()
    log_i = x - (xm + math.log(np.exp(x - xm).sum()))
    I = np.exp(log_i)
    pos = P > 0.0                                # K3: 0 ln 0 = 0
    diff = np.zeros_like(P)
    diff[pos] = np.log(P[pos]) - log_i[pos]
    loss = float((P * diff).sum())
    gx = index_scale * (I - P)                   # d loss / d (q_idx . k_idx[j])
    return dict(loss=loss, dq=gx @ ki, keys=keys, gx=gx, p_plus_i=P + I,
                dq_abs=np.abs(gx) @ np.abs(ki),
                mass_abs=index_scale * ((P + I) @ np.abs(ki)),
                loss_abs=float((P * np.abs(diff)).sum()))


def index_kl(q, k, q_idx, k_idx, block_idx, index_scale: float, q_begin: int = 0,
             rows=None, block: int = BLOCK) -> dict:
    """Index-branch KL loss and gradients for chunk rows `rows` (default: all).

    q [T, G*Hpg, D]; k [G, T, D]; q_idx [T, G, d]; k_idx [T, d];
    block_idx [R, G, top_k]: row i is token q_begin + i. Returns dict(loss [n, G],
    dq_idx [n, G, d], dk_idx [T, d] (the sum over the given rows of each row's
    gradient with respect to the index keys), dq_abs [n, G, d], mass_abs [n, G, d],
    loss_abs [n, G], dk_abs [T, d] = sum |gx_j| |q_idx|, dk_mass [T, d] =
    index_scale * sum (P_j + I_j) |q_idx|, rows)."""
    q, k = host_small_f64(q), host_small_f64(k)
    q_idx, k_idx = host_small_f64(q_idx), host_small_f64(k_idx)
    bi = np.asarray(host(block_idx))
    T, Hq, _ = q.shape
    G = k.shape[0]
    Hpg = Hq // G
    d = q_idx.shape[-1]
    rows = np.arange(bi.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    loss = np.zeros((n, G))
    loss_abs = np.zeros((n, G))
    dq = np.zeros((n, G, d))
    dq_abs = np.zeros((n, G, d))
    mass_abs = np.zeros((n, G, d))
    # dk_idx[j] = sum over rows of gx_row[j] q_idx_row: the rows' token gradients are
    # collected as a sparse [rows, T] matrix W and dk_idx = W^T . Q_idx (one product).
    w_rows, w_keys, w_val, w_pi, qi_rows = [], [], [], [], []
    for a, i in enumerate(rows.tolist()):
        t = q_begin + i
        for g in range(G):
            qi = as_f64(q_idx[t, g])
            r = kl_row(q[t, g * Hpg:(g + 1) * Hpg], k[g], qi, k_idx, bi[i, g], t, index_scale,
                       block)
            loss[a, g], dq[a, g] = r["loss"], r["dq"]
            dq_abs[a, g], mass_abs[a, g], loss_abs[a, g] = r["dq_abs"], r["mass_abs"], r["loss_abs"]
            w_rows.append(np.full(len(r["keys"]), len(qi_rows)))
            w_keys.append(r["keys"])
            w_val.append(r["gx"])
            w_pi.append(r["p_plus_i"])
            qi_rows.append(qi)
    if qi_rows:
        shape = (len(qi_rows), T)
        ij = (np.concatenate(w_rows), np.concatenate(w_keys))
        W = scipy.sparse.csr_matrix((np.concatenate(w_val), ij), shape=shape)
        S = scipy.sparse.csr_matrix((np.concatenate(w_pi), ij), shape=shape)
        QI = np.stack(qi_rows)
        dk = np.asarray(W.T @ QI)
        dk_abs = np.asarray(abs(W).T @ np.abs(QI))
        dk_mass = index_scale * np.asarray(S.T @ np.abs(QI))
    else:
        dk = dk_abs = dk_mass = np.zeros((T, d))
    return dict(loss=loss, dq_idx=dq, dk_idx=dk, dq_abs=dq_abs, mass_abs=mass_abs,
                loss_abs=loss_abs, dk_abs=dk_abs, dk_mass=dk_mass, rows=rows)


# ----------------------------------------------------------------------------------
# Dense GQA attention (the comparison baseline of the researchpapers.dev summary,
# "Key results": MSA against dense GQA with the same heads)
# ----------------------------------------------------------------------------------

def dense_prefill(q, k, v, rows=None) -> np.ndarray:
    """Causal softmax attention of every head over all keys j <= t of its group."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    T, Hq, D = q.shape
    G = k.shape[0]
    Hpg = Hq // G
    scale = 1.0 / math.sqrt(D)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, D))
    for i, t in enumerate(rows.tolist()):
        for g in range(G):
            hs = slice(g * Hpg, (g + 1) * Hpg)
            out[i, hs] = attend(q[t, hs], k[g, : t + 1], v[g, : t + 1], scale)
    return out


def dense_decode(q, k_cache, v_cache, seq_lens) -> np.ndarray:
    """Softmax attention of each sequence's query over its whole cache."""
    q, kc, vc = as_f64(q), as_f64(k_cache), as_f64(v_cache)
    lens = [int(x) for x in np.asarray(as_f64(seq_lens)).tolist()]
    B, Hq, D = q.shape
    G = kc.shape[1]
    Hpg = Hq // G
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D))
    for bi in range(B):
        L = lens[bi]
        for g in range(G):
            hs = slice(g * Hpg, (g + 1) * Hpg)
            out[bi, hs] = attend(q[bi, hs], kc[bi, g, :L], vc[bi, g, :L], scale)
    return out


# ----------------------------------------------------------------------------------
# Helpers for comparing against a device result
# ----------------------------------------------------------------------------------

def selection_array(sel, top_k: int) -> np.ndarray:
    """Pack a [R][G] list of ascending id arrays as [R, G, top_k] int32, -1 padded."""
    R, G = len(sel), len(sel[0])
    a = np.full((R, G, top_k), -1, dtype=np.int32)
    for i in range(R):
        for g in range(G):
            s = sel[i][g]
            a[i, g, : len(s)] = s
    return a


def attend_on_selection(q_t, k_g, v_g, sel, t, block: int = BLOCK) -> np.ndarray:
    """Attention of one token's group heads over a given selection (for rows where
    a device picked a different set on a declared near tie). Ids < 0 are padding; the
    others must be distinct (a repeated id would count its block twice)."""
    q_t, k_g, v_g = as_f64(q_t), host(k_g), host(v_g)
    sel = [int(c) for c in sel if int(c) >= 0]
    assert len(set(sel)) == len(sel), f"repeated block id in {sel}"
    j = visible_keys(sel, t, block)
    return attend(q_t, as_f64(k_g[j]), as_f64(v_g[j]), 1.0 / math.sqrt(q_t.shape[-1]))
