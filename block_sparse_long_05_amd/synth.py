"""Seeded synthetic inputs for the MSA hot path.

This module only draws data. It holds no step of the method (no scoring, pooling,
selection or attention), so both the CPU oracle and the HIP path can take their
inputs from it without sharing any of the method's arithmetic.

Shapes follow the workloads of the MiniMax Sparse Attention pages (researchpapers.dev
summary, "Key results": 16 blocks x 128 tokens per query group; mlqm.cn blog, section 2.1:
one index query per GQA group and one shared index-key head):

prefill
    q      [T, G*Hpg, D]     query heads, head h belongs to group h // Hpg
    k, v   [G, T, D]         one K/V head per GQA group
    q_idx  [T, G, d_idx]     one index query per token and group
    k_idx  [T, d_idx]        the single shared index-key head
decode
    q       [B, G*Hpg, D]
    k_cache [B, G, Lmax, D], v_cache likewise
    q_idx   [B, G, d_idx]
    k_idx   [B, Lmax, d_idx]
    seq_lens [B] int32 (cache length per sequence, the current token included)

Values are i.i.d. N(0, 1) drawn in fp32 from a seeded torch generator and, for bf16
workloads, rounded once to bf16 (round to nearest even). Both sides consume exactly
the same rounded tensors.

Planted blocks make the index branch's choice clear-cut on part of the rows:
prefill: per group a direction u_g ~ N(0, I) is added to every index query of that
    group, and 4*u_g to the index keys of `planted_per_group` random whole blocks.
decode: per (sequence, group) `planted_per_group` random blocks get 4*q_idx[b, g]
    added to their index keys.
"""

from __future__ import annotations

import torch

BLOCK = 128
_CHUNK_ROWS = 1 << 16


def _dtype(name: str) -> torch.dtype:
    if name in ("bf16", "bfloat16"):
        return torch.bfloat16
    if name in ("f32", "fp32", "float32"):
        return torch.float32
    raise ValueError(f"unknown dtype {name!r}")


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + tensor_id * 7919) & ((1 << 62) - 1))
    return g


def _randn_into(out: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    """Fill `out` with N(0,1) drawn in fp32, chunked along dim 0 to bound temporaries."""
    flat = out.view(out.shape[0], -1)
    rows_per = max(1, (_CHUNK_ROWS * 128) // max(1, flat.shape[1]))
    for r0 in range(0, flat.shape[0], rows_per):
        r1 = min(flat.shape[0], r0 + rows_per)
        tmp = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=out.device,
                          dtype=torch.float32)
        flat[r0:r1].copy_(tmp)
    return out


def _randn(shape, dtype, device, gen):
    return _randn_into(torch.empty(shape, dtype=dtype, device=device), gen)


def _distinct_blocks(n_pick: int, n_blocks: int, gen: torch.Generator, device) -> torch.Tensor:
    """n_pick distinct block ids from [0, n_blocks), padded with -1 when there are fewer."""
    perm = torch.randperm(n_blocks, generator=gen, device=device)[:n_pick].to("cpu")
    pad = torch.full((n_pick - perm.numel(),), -1, dtype=perm.dtype)
    return torch.cat([perm, pad])


def prefill_inputs(T: int, G: int, Hpg: int, D: int = 128, d_idx: int = 128,
                   dtype: str = "bf16", seed: int = 0, planted_per_group: int = 0,
                   plant_scale: float = 4.0, device="cpu") -> dict:
    """Inputs of one causal prefill over T tokens (see module docstring)."""
    dt = _dtype(dtype)
    dev = torch.device(device)
    q = _randn((T, G * Hpg, D), dt, dev, _gen(dev, seed, 1))
    k = _randn((G, T, D), dt, dev, _gen(dev, seed, 2))
    v = _randn((G, T, D), dt, dev, _gen(dev, seed, 3))
    planted = torch.empty((G, 0), dtype=torch.int64)
    n_full = T // BLOCK
    if planted_per_group > 0 and n_full > 0:
        gen_p = _gen(dev, seed, 6)
        u = torch.randn((G, d_idx), generator=gen_p, device=dev, dtype=torch.float32)
        q_idx = torch.empty((T, G, d_idx), dtype=dt, device=dev)
        gq = _gen(dev, seed, 4)
        for t0 in range(0, T, _CHUNK_ROWS):
            t1 = min(T, t0 + _CHUNK_ROWS)
            z = torch.randn((t1 - t0, G, d_idx), generator=gq, device=dev, dtype=torch.float32)
            q_idx[t0:t1].copy_(z + u[None])
        k_idx32 = torch.empty((T, d_idx), dtype=torch.float32, device=dev)
        _randn_into(k_idx32, _gen(dev, seed, 5))
        rows = []
        for g in range(G):
            blocks = _distinct_blocks(planted_per_group, n_full, gen_p, dev)
            rows.append(blocks)
            for c in blocks.tolist():
                if c >= 0:
                    k_idx32[c * BLOCK:(c + 1) * BLOCK] += plant_scale * u[g]
        planted = torch.stack(rows)
        k_idx = k_idx32.to(dt)
        del k_idx32
    else:
        q_idx = _randn((T, G, d_idx), dt, dev, _gen(dev, seed, 4))
        k_idx = _randn((T, d_idx), dt, dev, _gen(dev, seed, 5))
    return dict(q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx, planted=planted)


def decode_inputs(B: int, max_len: int, G: int, Hpg: int, D: int = 128, d_idx: int = 128,
                  dtype: str = "bf16", seed: int = 0, planted_per_group: int = 0,
                  plant_scale: float = 4.0, seq_lens=None, device="cpu") -> dict:
    """Inputs of one decode step of B sequences against a KV cache of capacity max_len.

    seq_lens defaults to max_len for every sequence; a list gives ragged lengths.
    """
    dt = _dtype(dtype)
    dev = torch.device(device)
    if seq_lens is None:
        seq_lens = [max_len] * B
    seq_lens = [int(x) for x in seq_lens]
    if len(seq_lens) != B or min(seq_lens) < 1 or max(seq_lens) > max_len:
        raise ValueError("seq_lens must hold B lengths in [1, max_len]")
    q = _randn((B, G * Hpg, D), dt, dev, _gen(dev, seed, 11))
    k_cache = torch.empty((B, G, max_len, D), dtype=dt, device=dev)
    v_cache = torch.empty((B, G, max_len, D), dtype=dt, device=dev)
    gk, gv = _gen(dev, seed, 12), _gen(dev, seed, 13)
    for b in range(B):
        for g in range(G):
            _randn_into(k_cache[b, g], gk)
            _randn_into(v_cache[b, g], gv)
    q_idx = _randn((B, G, d_idx), dt, dev, _gen(dev, seed, 14))
    k_idx = torch.empty((B, max_len, d_idx), dtype=dt, device=dev)
    gki = _gen(dev, seed, 15)
    planted = torch.empty((B, G, 0), dtype=torch.int64)
    if planted_per_group > 0:
        gen_p = _gen(dev, seed, 16)
        q_idx32 = q_idx.to(torch.float32)
        per_b = []
        for b in range(B):
            kb = torch.empty((max_len, d_idx), dtype=torch.float32, device=dev)
            _randn_into(kb, gki)
            n_blk = (seq_lens[b] + BLOCK - 1) // BLOCK
            per_g = []
            for g in range(G):
                blocks = _distinct_blocks(planted_per_group, n_blk, gen_p, dev)
                per_g.append(blocks)
                for c in blocks.tolist():
                    if c >= 0:
                        kb[c * BLOCK:min((c + 1) * BLOCK, max_len)] += plant_scale * q_idx32[b, g]
            per_b.append(torch.stack(per_g))
            k_idx[b].copy_(kb)
            del kb
        planted = torch.stack(per_b)
    else:
        for b in range(B):
            _randn_into(k_idx[b], gki)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device=dev)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, q_idx=q_idx, k_idx=k_idx,
                seq_lens=lens, planted=planted)


def random_selection(q_count: int, G: int, top_k: int, q_begin: int = 0, seed: int = 0,
                     popular_per_group: int = 0) -> torch.Tensor:
    """A valid block selection drawn at random, int32 [q_count, G, top_k] on the CPU: row i
    (token t = q_begin + i, local block b = t // 128) holds b and top_k - 1 distinct blocks
    of [0, b) (every block 0..b when b + 1 <= top_k), ascending, padded with -1. Each group
    has popular_per_group blocks that every row able to see them picks first, so blocks
    are kept by long runs of rows as well as by single rows. No scores are involved."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed((int(seed) * 7919 + 104729) & ((1 << 62) - 1))
    t = q_begin + torch.arange(q_count)
    b = t // BLOCK
    nblk = int(b.max().item()) + 1 if q_count > 0 else 1
    r = torch.rand((q_count, G, nblk), generator=gen)
    if popular_per_group > 0:
        for g in range(G):
            pop = torch.randperm(nblk, generator=gen)[:popular_per_group]
            r[:, g, pop] -= 2.0
    c = torch.arange(nblk)
    big = 1e9
    r = torch.where(c[None, None, :] < b[:, None, None], r, torch.full_like(r, big))
    r = torch.where(c[None, None, :] == b[:, None, None], torch.full_like(r, -big), r)
    kk = min(top_k, nblk)
    val, pick = torch.topk(r, kk, dim=2, largest=False)
    pick = torch.where(val < big, pick, torch.full_like(pick, 1 << 30))
    pick, _ = torch.sort(pick, dim=2)
    out = torch.full((q_count, G, top_k), -1, dtype=torch.int32)
    out[:, :, :kk] = torch.where(pick < (1 << 30), pick, torch.full_like(pick, -1)).to(torch.int32)
    return out


def to_paged(x: dict, seed: int = 0, spare_pages: int = 3) -> dict:
    """The decode caches of `x` (from decode_inputs) laid out in 128-token pages placed at
    seeded random page ids, as a paged KV cache would hold them:
        k_idx_pages [P, 128, d_idx]   k_pages, v_pages [P, G, 128, D]
        block_table [B, max_len / 128] int32 (page of logical block c of sequence b)
    P = B * max_len / 128 + spare_pages; the spare pages hold zeros. Only data moves."""
    kc, vc, ki = x["k_cache"], x["v_cache"], x["k_idx"]
    B, G, L, D = kc.shape
    if L % BLOCK:
        raise ValueError("max_len must be a multiple of 128 for a paged layout")
    nb = L // BLOCK
    d_idx = ki.shape[-1]
    P = B * nb + spare_pages
    gen = torch.Generator(device="cpu")
    gen.manual_seed((int(seed) * 1_000_003 + 99991) & ((1 << 62) - 1))
    perm = torch.randperm(P, generator=gen)[:B * nb].to(kc.device)
    k_pages = torch.zeros((P, G, BLOCK, D), dtype=kc.dtype, device=kc.device)
    v_pages = torch.zeros_like(k_pages)
    k_idx_pages = torch.zeros((P, BLOCK, d_idx), dtype=ki.dtype, device=ki.device)
    k_pages[perm] = kc.view(B, G, nb, BLOCK, D).permute(0, 2, 1, 3, 4).reshape(B * nb, G, BLOCK, D)
    v_pages[perm] = vc.view(B, G, nb, BLOCK, D).permute(0, 2, 1, 3, 4).reshape(B * nb, G, BLOCK, D)
    k_idx_pages[perm] = ki.view(B * nb, BLOCK, d_idx)
    table = perm.view(B, nb).to(torch.int32).contiguous()
    return dict(k_pages=k_pages, v_pages=v_pages, k_idx_pages=k_idx_pages, block_table=table)
