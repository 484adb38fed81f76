"""Thin ctypes binding of libmsa.so (include/msa.h).

Argument marshalling only: torch tensors become raw device pointers and the current
HIP stream; every step of the hot path runs in the library's kernels. There is no
fallback: if libmsa.so is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARGUMENT = 1
MSA_ERR_UNSUPPORTED = 2
MSA_ERR_WORKSPACE_TOO_SMALL = 3
MSA_ERR_HIP = 4
MSA_ERR_TOO_LARGE = 5
NOALLOC_SCRATCH_BYTES = 32 << 20  # MSA_NOALLOC_SCRATCH_BYTES

DTYPE = {"f32": 0, "bf16": 1}
MODE = {"prefill": 0, "decode": 1}
ENTRY = {"index_scores": 0, "block_topk": 1, "sparse_attn_prefill": 2,
         "sparse_attn_decode": 3, "dense_gqa_attn": 4, "index_topk": 5, "index_kl": 6}
ALGO = {"auto": 0, "query_centric": 1, "kv_centric": 2}

BLOCK = 128

# Every symbol include/msa.h declares.
EXPORTED = ["msa_index_scores", "msa_block_topk", "msa_index_topk", "msa_sparse_attn_prefill",
            "msa_sparse_attn_decode", "msa_sparse_attn_decode_topk",
            "msa_sparse_attn_decode_noalloc", "msa_index_scores_paged", "msa_sparse_attn_decode_paged",
            "msa_sparse_attn_decode_topk_paged",
            "msa_index_kl_prefill", "msa_dense_gqa_attn", "msa_workspace_size",
            "msa_status_string", "msa_abi_version"]


class CProblem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("num_groups", ctypes.c_int32),
        ("heads_per_group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("seq_len", ctypes.c_int64), ("q_begin", ctypes.c_int64), ("q_count", ctypes.c_int64),
        ("batch", ctypes.c_int32), ("algo", ctypes.c_int32), ("max_len", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p),
    ]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmsa.so (built by build.py / __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m block_sparse_long_05_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(CProblem)
    lib.msa_index_scores.argtypes = [pp, vp, vp, vp, vp]
    lib.msa_block_topk.argtypes = [pp, vp, vp, vp]
    lib.msa_index_topk.argtypes = [pp, vp, vp, vp, vp]
    lib.msa_sparse_attn_prefill.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_decode.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_decode_topk.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_decode_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp]
    lib.msa_dense_gqa_attn.argtypes = [pp, vp, vp, vp, vp, vp, sz, vp]
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.msa_index_scores_paged.argtypes = [pp, vp, vp, vp, i32, i64, vp, vp]
    lib.msa_sparse_attn_decode_paged.argtypes = [pp, vp, vp, vp, vp, i32, i64, vp, vp, vp, sz, vp]
    lib.msa_sparse_attn_decode_topk_paged.argtypes = [pp, vp, vp, vp, vp, i32, i64, vp, vp, vp,
                                                      vp, sz, vp]
    lib.msa_index_kl_prefill.argtypes = [pp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                         vp, sz, vp]
    lib.msa_workspace_size.argtypes = [pp, ctypes.c_int32, ctypes.POINTER(sz)]
    lib.msa_status_string.argtypes = [ctypes.c_int]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_abi_version.argtypes = []
    for name in ("msa_index_scores", "msa_block_topk", "msa_index_topk", "msa_sparse_attn_prefill",
                 "msa_index_scores_paged", "msa_sparse_attn_decode_paged",
                 "msa_sparse_attn_decode_topk_paged", "msa_sparse_attn_decode", "msa_sparse_attn_decode_topk",
                 "msa_sparse_attn_decode_noalloc", "msa_dense_gqa_attn", "msa_workspace_size",
                 "msa_index_kl_prefill",
                 "msa_abi_version"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().msa_status_string(int(status)).decode()


@dataclass
class Problem:
    """Python mirror of msa_problem (see include/msa.h for every field)."""
    dtype: str
    mode: str
    num_groups: int
    heads_per_group: int
    index_dim: int
    top_k: int
    head_dim: int = 128
    block_size: int = BLOCK
    seq_len: int = 0
    q_begin: int = 0
    q_count: int = 0
    batch: int = 0
    algo: str = "auto"
    max_len: int = 0
    seq_lens: Optional[torch.Tensor] = None  # device int32 [B]
    _c: Optional[CProblem] = None

    def c(self) -> CProblem:
        sl = self.seq_lens
        self._c = CProblem(DTYPE[self.dtype], MODE[self.mode], self.num_groups,
                           self.heads_per_group, self.head_dim, self.index_dim, self.block_size,
                           self.top_k, self.seq_len, self.q_begin, self.q_count, self.batch,
                           ALGO[self.algo], self.max_len, 0 if sl is None else sl.data_ptr())
        return self._c

    @property
    def nblk(self) -> int:
        n = self.seq_len if self.mode == "prefill" else self.max_len
        return (n + BLOCK - 1) // BLOCK

    @property
    def rows(self) -> int:
        return self.q_count if self.mode == "prefill" else self.batch


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if x.device.type != "cuda":
            raise ValueError("MSA tensors must live in device memory")
        if not x.is_contiguous():
            raise ValueError("MSA tensors must be contiguous")
        return x.data_ptr()
    raise TypeError(type(x))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MSA_OK:
        raise MsaError(status, where)


def msa_workspace_size(p: Problem, entry: str) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_workspace_size(ctypes.byref(p.c()), ENTRY[entry], ctypes.byref(n)),
           "msa_workspace_size")
    return int(n.value)


def msa_index_scores(p: Problem, q_idx, k_idx, block_scores, stream=None):
    _check(load_library().msa_index_scores(ctypes.byref(p.c()), _ptr(q_idx), _ptr(k_idx),
                                           _ptr(block_scores), _stream(stream)),
           "msa_index_scores")


def msa_block_topk(p: Problem, block_scores, block_idx, stream=None):
    _check(load_library().msa_block_topk(ctypes.byref(p.c()), _ptr(block_scores), _ptr(block_idx),
                                         _stream(stream)), "msa_block_topk")


def msa_index_topk(p: Problem, q_idx, k_idx, block_idx, stream=None):
    _check(load_library().msa_index_topk(ctypes.byref(p.c()), _ptr(q_idx), _ptr(k_idx),
                                         _ptr(block_idx), _stream(stream)), "msa_index_topk")


def msa_index_scores_paged(p: Problem, q_idx, k_idx_pages, block_table, block_scores,
                           stream=None):
    """Decode index scan over a paged index-key cache (see include/msa.h)."""
    _check(load_library().msa_index_scores_paged(
        ctypes.byref(p.c()), _ptr(q_idx), _ptr(k_idx_pages), _ptr(block_table),
        int(block_table.shape[1]), int(k_idx_pages.shape[0]), _ptr(block_scores),
        _stream(stream)), "msa_index_scores_paged")


def msa_sparse_attn_decode_paged(p: Problem, q, k_pages, v_pages, block_table, block_idx, out,
                                 workspace=None, stream=None):
    """Decode sparse attention reading each kept block from its page (see include/msa.h)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_sparse_attn_decode_paged(
        ctypes.byref(p.c()), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
        int(block_table.shape[1]), int(k_pages.shape[0]), _ptr(block_idx), _ptr(out),
        _ptr(workspace), ws_bytes, _stream(stream)), "msa_sparse_attn_decode_paged")


def msa_sparse_attn_decode_topk_paged(p: Problem, q, k_pages, v_pages, block_table, block_scores,
                                      block_idx, out, workspace=None, stream=None):
    """msa_sparse_attn_decode_topk on paged caches (see include/msa.h)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_sparse_attn_decode_topk_paged(
        ctypes.byref(p.c()), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
        int(block_table.shape[1]), int(k_pages.shape[0]), _ptr(block_scores), _ptr(block_idx),
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)), "msa_sparse_attn_decode_topk_paged")


def index_topk_supported(p: Problem) -> bool:
    """Whether msa_index_topk (the fused index branch) is built for this problem."""
    return p.mode == "prefill" and p.dtype == "bf16" and p.top_k <= 16


def msa_sparse_attn_prefill(p: Problem, q, k, v, block_idx, out, workspace=None, stream=None,
                            lse=None):
    """lse (optional, fp32 [T, Hq]) receives each row's and head's ln softmax normaliser."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_sparse_attn_prefill(
        ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)), "msa_sparse_attn_prefill")


def msa_sparse_attn_decode(p: Problem, q, k_cache, v_cache, block_idx, out, workspace=None,
                           stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_sparse_attn_decode(
        ctypes.byref(p.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_idx), _ptr(out),
        _ptr(workspace), ws_bytes, _stream(stream)), "msa_sparse_attn_decode")


def msa_sparse_attn_decode_topk(p: Problem, q, k_cache, v_cache, block_scores, block_idx, out,
                                workspace=None, stream=None):
    """msa_block_topk and msa_sparse_attn_decode in one call (the selection inside the
    attention launch where that is faster): block_idx and out as the two calls write them."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_sparse_attn_decode_topk(
        ctypes.byref(p.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_scores),
        _ptr(block_idx), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
        "msa_sparse_attn_decode_topk")


def msa_sparse_attn_decode_noalloc(p: Problem, q, k_cache, v_cache, block_idx, out,
                                   stream=None):
    """msa_sparse_attn_decode without a workspace: the library's fixed per-GPU scratch holds
    the split partials (see include/msa.h). The stream must belong to the current device."""
    _check(load_library().msa_sparse_attn_decode_noalloc(
        ctypes.byref(p.c()), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_idx), _ptr(out),
        _stream(stream)), "msa_sparse_attn_decode_noalloc")


def msa_index_kl_prefill(p: Problem, q, k, q_idx, k_idx, block_idx, index_scale: float, loss,
                         dq_idx, dk_idx, workspace=None, stream=None, main_lse=None):
    """Index-branch KL loss (loss [q_count, G], dq_idx [q_count, G, 128] written) and its
    index-key gradient (ADDED into dk_idx [T, 128]); all three fp32. main_lse: the lse that
    msa_sparse_attn_prefill wrote for the same selection (optional)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_index_kl_prefill(
        ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
        _ptr(main_lse), float(index_scale), _ptr(loss), _ptr(dq_idx), _ptr(dk_idx),
        _ptr(workspace), ws_bytes, _stream(stream)), "msa_index_kl_prefill")


def msa_dense_gqa_attn(p: Problem, q, k, v, out, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().msa_dense_gqa_attn(
        ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace), ws_bytes,
        _stream(stream)), "msa_dense_gqa_attn")


# ---- buffer helpers (allocation stays with the caller, i.e. torch) -----------------------

def alloc_workspace(p: Problem, entry: str, device="cuda") -> Optional[torch.Tensor]:
    n = msa_workspace_size(p, entry)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def alloc_block_scores(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty((p.rows, p.num_groups, p.nblk), dtype=torch.float32, device=device)


def alloc_block_idx(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty((p.rows, p.num_groups, p.top_k), dtype=torch.int32, device=device)


# ---- input checks of the high-level helpers ---------------------------------------------
# The C ABI sees only pointers, so it cannot tell a mismatched shape or dtype from a valid
# one; the helpers below check what their arguments imply before any launch.

_DT = {torch.float32: "f32", torch.bfloat16: "bf16"}


def _expect(t, name, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def check_prefill_inputs(x: dict) -> tuple:
    """Validates q [T, Hq, 128], k, v [G, T, 128], q_idx [T, G, d], k_idx [T, d] (one dtype,
    fp32 or bf16, Hq divisible by G); returns (T, G, Hpg, d, dtype name)."""
    q = x["q"]
    if q.dim() != 3 or q.dtype not in _DT:
        raise ValueError("q must be [T, Hq, D] fp32 or bf16")
    T, Hq, D = q.shape
    if x["k"].dim() != 3:
        raise ValueError("k must be [G, T, D]")
    G = x["k"].shape[0]
    if G < 1 or Hq % G != 0:
        raise ValueError(f"Hq = {Hq} query heads are not a multiple of G = {G} groups")
    d = x["q_idx"].shape[-1]
    _expect(x["k"], "k", (G, T, D), q.dtype)
    _expect(x["v"], "v", (G, T, D), q.dtype)
    _expect(x["q_idx"], "q_idx", (T, G, d), q.dtype)
    _expect(x["k_idx"], "k_idx", (T, d), q.dtype)
    return T, G, Hq // G, d, _DT[q.dtype]


def check_decode_inputs(x: dict) -> tuple:
    """Validates q [B, Hq, 128], k_cache, v_cache [B, G, max_len, 128], q_idx [B, G, d],
    k_idx [B, max_len, d] (one dtype), seq_lens int32 [B]; returns (B, G, Hpg, d, max_len,
    dtype name)."""
    q = x["q"]
    if q.dim() != 3 or q.dtype not in _DT:
        raise ValueError("q must be [B, Hq, D] fp32 or bf16")
    B, Hq, D = q.shape
    if x["k_cache"].dim() != 4:
        raise ValueError("k_cache must be [B, G, max_len, D]")
    G, L = x["k_cache"].shape[1], x["k_cache"].shape[2]
    if G < 1 or Hq % G != 0:
        raise ValueError(f"Hq = {Hq} query heads are not a multiple of G = {G} groups")
    d = x["q_idx"].shape[-1]
    _expect(x["k_cache"], "k_cache", (B, G, L, D), q.dtype)
    _expect(x["v_cache"], "v_cache", (B, G, L, D), q.dtype)
    _expect(x["q_idx"], "q_idx", (B, G, d), q.dtype)
    _expect(x["k_idx"], "k_idx", (B, L, d), q.dtype)
    _expect(x["seq_lens"], "seq_lens", (B,), torch.int32)
    return B, G, Hq // G, d, L, _DT[q.dtype]


def _check_out(t, name, shape, dtype):
    if t is not None:
        _expect(t, name, shape, dtype)


# ---- the whole hot path, as a chain of the C calls ------------------------------------------

def prefill(x: dict, top_k: int, q_begin: int = 0, q_count: Optional[int] = None,
            algo: str = "auto", out=None, block_scores=None, block_idx=None, workspace=None,
            stream=None, index: str = "separate", lse=None):
    """MSA prefill of query rows [q_begin, q_begin + q_count): index scores -> top-k ->
    sparse attention. x holds q, k, v, q_idx, k_idx on the device; lse (fp32 [T, Hq]), when
    given, receives the rows' softmax normalisers. index="fused" runs the
    index branch as msa_index_topk (no block scores; block_scores is returned as None).
    Returns (out, block_idx, block_scores)."""
    q = x["q"]
    T, G, Hpg, d, dt = check_prefill_inputs(x)
    if q_count is None:
        q_count = T - q_begin
    p = Problem(dtype=dt, mode="prefill", num_groups=G, heads_per_group=Hpg, index_dim=d,
                top_k=top_k, head_dim=q.shape[2], seq_len=T, q_begin=q_begin, q_count=q_count,
                algo=algo)
    if index not in ("separate", "fused"):
        raise ValueError(f"index must be 'separate' or 'fused', not {index!r}")
    _check_out(out, "out", q.shape, q.dtype)
    _check_out(lse, "lse", q.shape[:2], torch.float32)
    _check_out(block_idx, "block_idx", (q_count, G, top_k), torch.int32)
    _check_out(block_scores, "block_scores", (q_count, G, p.nblk), torch.float32)
    if out is None:
        out = torch.empty_like(q)
    if block_idx is None:
        block_idx = alloc_block_idx(p, q.device)
    if workspace is None:
        workspace = alloc_workspace(p, "sparse_attn_prefill", q.device)
    if index == "fused":
        msa_index_topk(p, x["q_idx"], x["k_idx"], block_idx, stream)
        block_scores = None
    else:
        if block_scores is None:
            block_scores = alloc_block_scores(p, q.device)
        msa_index_scores(p, x["q_idx"], x["k_idx"], block_scores, stream)
        msa_block_topk(p, block_scores, block_idx, stream)
    msa_sparse_attn_prefill(p, q, x["k"], x["v"], block_idx, out, workspace, stream, lse=lse)
    return out, block_idx, block_scores


def index_kl(x: dict, block_idx, top_k: int, index_scale: float, q_begin: int = 0,
             q_count: Optional[int] = None, dk_idx=None, workspace=None, stream=None,
             main_lse=None):
    """Index-branch KL loss and gradients for query rows [q_begin, q_begin + q_count) on the
    selection block_idx [q_count, G, top_k]. x holds q, k, q_idx, k_idx (bf16) on the device.
    dk_idx (fp32 [T, 128]) is accumulated into; a zeroed one is made when it is None.
    Returns (loss [q_count, G], dq_idx [q_count, G, 128], dk_idx)."""
    q = x["q"]
    T, G, Hpg, d, dt = check_prefill_inputs(dict(x, v=x["k"]))
    if q_count is None:
        q_count = T - q_begin
    p = Problem(dtype=dt, mode="prefill", num_groups=G, heads_per_group=Hpg, index_dim=d,
                top_k=top_k, head_dim=q.shape[2], seq_len=T, q_begin=q_begin, q_count=q_count)
    _expect(block_idx, "block_idx", (q_count, G, top_k), torch.int32)
    _check_out(dk_idx, "dk_idx", (T, d), torch.float32)
    _check_out(main_lse, "main_lse", q.shape[:2], torch.float32)
    loss = torch.empty((q_count, G), dtype=torch.float32, device=q.device)
    dq = torch.empty((q_count, G, x["q_idx"].shape[-1]), dtype=torch.float32, device=q.device)
    if dk_idx is None:
        dk_idx = torch.zeros((T, x["k_idx"].shape[-1]), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(p, "index_kl", q.device)
    msa_index_kl_prefill(p, q, x["k"], x["q_idx"], x["k_idx"], block_idx, index_scale, loss, dq,
                         dk_idx, workspace, stream, main_lse=main_lse)
    return loss, dq, dk_idx


def decode_problem(x: dict, top_k: int) -> Problem:
    q = x["q"]
    B, G, Hpg, d, L, dt = check_decode_inputs(x)
    return Problem(dtype=dt, mode="decode", num_groups=G, heads_per_group=Hpg, index_dim=d,
                   top_k=top_k, head_dim=q.shape[2], batch=B, max_len=L, seq_lens=x["seq_lens"])


def decode(x: dict, top_k: int, out=None, block_scores=None, block_idx=None, workspace=None,
           stream=None, topk: str = "separate"):
    """One MSA decode step: index scan -> top-k -> split-K sparse attention + combine.
    topk="fused" selects inside the attention launch (msa_sparse_attn_decode_topk).
    Returns (out, block_idx, block_scores)."""
    if topk not in ("separate", "fused"):
        raise ValueError(f"topk must be 'separate' or 'fused', not {topk!r}")
    p = decode_problem(x, top_k)
    _check_out(out, "out", x["q"].shape, x["q"].dtype)
    _check_out(block_scores, "block_scores", (p.batch, p.num_groups, p.nblk), torch.float32)
    _check_out(block_idx, "block_idx", (p.batch, p.num_groups, top_k), torch.int32)
    if out is None:
        out = torch.empty_like(x["q"])
    if block_scores is None:
        block_scores = alloc_block_scores(p, x["q"].device)
    if block_idx is None:
        block_idx = alloc_block_idx(p, x["q"].device)
    if workspace is None:
        workspace = alloc_workspace(p, "sparse_attn_decode", x["q"].device)
    msa_index_scores(p, x["q_idx"], x["k_idx"], block_scores, stream)
    if topk == "fused":
        msa_sparse_attn_decode_topk(p, x["q"], x["k_cache"], x["v_cache"], block_scores,
                                    block_idx, out, workspace, stream)
        return out, block_idx, block_scores
    msa_block_topk(p, block_scores, block_idx, stream)
    msa_sparse_attn_decode(p, x["q"], x["k_cache"], x["v_cache"], block_idx, out, workspace,
                           stream)
    return out, block_idx, block_scores
