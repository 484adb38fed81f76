"""Host-only checks of the C ABI: the library loads, exports every function that
include/msa.h declares, and rejects bad arguments on the host before any launch.
No call here reaches a kernel, so these run without a GPU."""

import ctypes
import os
import re

import pytest

from block_sparse_long_05_amd import msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(msa.LIB_PATH),
                                reason="libmsa.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(msa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(msa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = msa.load_library()
    assert lib.msa_abi_version() == 4
    for s in range(5):
        assert msa.status_string(s).startswith("MSA_")


def _prefill(**kw):
    base = dict(dtype="bf16", mode="prefill", num_groups=8, heads_per_group=8, index_dim=128,
                top_k=16, seq_len=4096, q_begin=0, q_count=4096)
    base.update(kw)
    return msa.Problem(**base)


def _call_index(p):
    return msa.load_library().msa_index_scores(ctypes.byref(p.c()), FAKE, FAKE, FAKE, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(index_dim=96), msa.MSA_ERR_UNSUPPORTED),
    (dict(block_size=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(heads_per_group=17), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_groups=65), msa.MSA_ERR_UNSUPPORTED),
    (dict(top_k=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(top_k=65), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_groups=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(q_begin=4000, q_count=200), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(q_begin=-1), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(seq_len=0, q_count=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(seq_len=(1 << 30) + 1, q_count=1), msa.MSA_ERR_INVALID_ARGUMENT),
])
def test_prefill_validation(kw, code):
    assert _call_index(_prefill(**kw)) == code


def test_bad_enums_and_null_pointers():
    lib = msa.load_library()
    p = _prefill()
    c = p.c()
    c.dtype = 7
    assert lib.msa_index_scores(ctypes.byref(c), FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    c = p.c()
    c.mode = 3
    assert lib.msa_block_topk(ctypes.byref(c), FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    c = p.c()
    c.algo = 9
    assert lib.msa_sparse_attn_prefill(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_index_scores(None, FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    c = p.c()
    assert lib.msa_index_scores(ctypes.byref(c), 0, FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_index_scores(ctypes.byref(c), FAKE + 2, FAKE, FAKE, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_sparse_attn_prefill(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 0, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    # lse is optional, but when given it must be 4-byte aligned
    assert lib.msa_sparse_attn_prefill(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 0,
                                       0, 0) == msa.MSA_ERR_INVALID_ARGUMENT


def test_mode_mismatch_rejected():
    lib = msa.load_library()
    c = _prefill().c()
    assert lib.msa_sparse_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                      0) == msa.MSA_ERR_INVALID_ARGUMENT


def _decode(**kw):
    base = dict(dtype="bf16", mode="decode", num_groups=8, heads_per_group=8, index_dim=128,
                top_k=16, batch=4, max_len=131072)
    base.update(kw)
    p = msa.Problem(**base)
    c = p.c()
    c.seq_lens = FAKE
    return c


def test_decode_validation_and_workspace():
    lib = msa.load_library()
    n = ctypes.c_size_t(0)
    c = _decode()
    assert lib.msa_workspace_size(ctypes.byref(c), msa.ENTRY["sparse_attn_decode"],
                                  ctypes.byref(n)) == msa.MSA_OK
    # bf16: B * G * (top_k block splits) * Hpg heads * (128 + 2) floats, each part
    # 256-byte aligned
    units = 4 * 8 * 16 * 8
    assert n.value == units * 128 * 4 + ((units * 2 * 4 + 255) // 256) * 256
    # fp32: two half-block splits per kept block
    n32 = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(_decode(dtype="f32")),
                                  msa.ENTRY["sparse_attn_decode"], ctypes.byref(n32)) == msa.MSA_OK
    units32 = 4 * 8 * 32 * 8
    assert n32.value == units32 * 128 * 4 + ((units32 * 2 * 4 + 255) // 256) * 256
    # too small a workspace is refused before launching
    assert lib.msa_sparse_attn_decode(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      n.value - 1, 0) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    bad = _decode()
    bad.seq_lens = 0
    assert lib.msa_block_topk(ctypes.byref(bad), FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    for kw in (dict(batch=0), dict(max_len=0), dict(batch=70000)):
        c = _decode(**kw)
        assert lib.msa_block_topk(ctypes.byref(c), FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_workspace_size(ctypes.byref(_decode()), 99, ctypes.byref(n)) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_workspace_size(ctypes.byref(_decode()), 0, None) == msa.MSA_ERR_INVALID_ARGUMENT


def test_empty_chunk_is_a_no_op():
    """q_count == 0 returns MSA_OK without launching (safe without a device)."""
    lib = msa.load_library()
    c = _prefill(q_begin=4096, q_count=0).c()
    assert lib.msa_index_scores(ctypes.byref(c), FAKE, FAKE, FAKE, 0) == msa.MSA_OK
    assert lib.msa_block_topk(ctypes.byref(c), FAKE, FAKE, 0) == msa.MSA_OK
    assert lib.msa_sparse_attn_prefill(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 0) \
        == msa.MSA_OK


def test_index_topk_rejections():
    """The fused index branch is built for bf16 prefill with top_k <= 16 only; anything
    else is refused on the host (MSA_ERR_UNSUPPORTED), as are misaligned pointers."""
    lib = msa.load_library()
    ok = _prefill(top_k=16)
    assert msa.index_topk_supported(ok)
    for p in (_prefill(dtype="f32"), _prefill(top_k=17)):
        assert not msa.index_topk_supported(p)
        assert lib.msa_index_topk(ctypes.byref(p.c()), FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_topk(ctypes.byref(_decode()), FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_topk(ctypes.byref(ok.c()), FAKE + 4, FAKE, FAKE, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_index_topk(ctypes.byref(_prefill(q_begin=4096, q_count=0).c()), FAKE, FAKE,
                              FAKE, 0) == msa.MSA_OK
    n = ctypes.c_size_t(7)
    assert lib.msa_workspace_size(ctypes.byref(ok.c()), msa.ENTRY["index_topk"],
                                  ctypes.byref(n)) == msa.MSA_OK and n.value == 0


def test_paged_decode_validation():
    """The paged entries check mode, table pointer, page counts and that max_len equals
    pages_per_seq * 128 on the host, before any launch."""
    lib = msa.load_library()
    c = _decode(max_len=4096)   # 32 pages per sequence
    bad_mode = _prefill().c()
    ok_args = (FAKE, FAKE, FAKE, 32, 100, FAKE, 0)
    assert lib.msa_index_scores_paged(ctypes.byref(bad_mode), *ok_args) == msa.MSA_ERR_INVALID_ARGUMENT
    for args in ((FAKE, FAKE, 0, 32, 100, FAKE, 0),        # null table
                 (FAKE, FAKE, FAKE + 2, 32, 100, FAKE, 0),  # misaligned table
                 (FAKE, FAKE, FAKE, 31, 100, FAKE, 0),      # max_len != pages_per_seq * 128
                 (FAKE, FAKE, FAKE, 0, 100, FAKE, 0),
                 (FAKE, FAKE, FAKE, 32, 0, FAKE, 0),        # no pages
                 (FAKE + 4, FAKE, FAKE, 32, 100, FAKE, 0)):  # misaligned q_idx
        assert lib.msa_index_scores_paged(ctypes.byref(c), *args) == msa.MSA_ERR_INVALID_ARGUMENT
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(c), msa.ENTRY["sparse_attn_decode"],
                                  ctypes.byref(n)) == msa.MSA_OK
    assert lib.msa_sparse_attn_decode_paged(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 31, 100,
                                            FAKE, FAKE, FAKE, n.value, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT
    assert lib.msa_sparse_attn_decode_paged(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 32, 100,
                                            FAKE, FAKE, FAKE, n.value - 1, 0) \
        == msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_index_kl_validation():
    """The KL entry is built for bf16 prefill with index_dim 128; it checks the temperature,
    pointer alignment and workspace size on the host, before any launch."""
    lib = msa.load_library()
    ok = _prefill()
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(ok.c()), msa.ENTRY["index_kl"],
                                  ctypes.byref(n)) == msa.MSA_OK and n.value > 0
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)

    def call(p, scale=0.1, ws=n.value, loss=FAKE, main_lse=0):
        return lib.msa_index_kl_prefill(ctypes.byref(p.c()), *args, main_lse, ctypes.c_float(scale),
                                        loss, FAKE, FAKE, FAKE, ws, 0)

    for p in (_prefill(dtype="f32"), _prefill(index_dim=64)):
        assert call(p) == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_kl_prefill(ctypes.byref(_decode()), *args, 0, ctypes.c_float(0.1), FAKE,
                                    FAKE, FAKE, FAKE, n.value, 0) == msa.MSA_ERR_UNSUPPORTED
    assert call(ok, main_lse=FAKE + 2) == msa.MSA_ERR_INVALID_ARGUMENT
    for scale in (0.0, -1.0, float("inf"), float("nan")):
        assert call(ok, scale) == msa.MSA_ERR_INVALID_ARGUMENT
    assert call(ok, loss=FAKE + 4) == msa.MSA_ERR_INVALID_ARGUMENT
    assert call(ok, ws=n.value - 1) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert call(_prefill(q_begin=4096, q_count=0), ws=0) == msa.MSA_OK
    m = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(_decode()), msa.ENTRY["index_kl"],
                                  ctypes.byref(m)) == msa.MSA_ERR_INVALID_ARGUMENT


def test_entry_count_limit_of_the_reverse_index():
    """The KV-centric prefill and the KL loss sort a chunk's q_count * G * top_k kept entries
    by 32-bit id: from 2^31 entries on, the KV-centric algo and the KL entry refuse the call
    (before any launch) and the default algo needs no workspace (it runs query-centric)."""
    lib = msa.load_library()
    big = dict(seq_len=1 << 30, q_begin=0, q_count=1 << 30, num_groups=64, top_k=64)
    n = ctypes.c_size_t(7)
    assert lib.msa_workspace_size(ctypes.byref(_prefill(**big).c()), msa.ENTRY["index_kl"],
                                  ctypes.byref(n)) == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_workspace_size(ctypes.byref(_prefill(algo="kv_centric", **big).c()),
                                  msa.ENTRY["sparse_attn_prefill"],
                                  ctypes.byref(n)) == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_workspace_size(ctypes.byref(_prefill(**big).c()),
                                  msa.ENTRY["sparse_attn_prefill"], ctypes.byref(n)) == msa.MSA_OK
    assert n.value == 0
    assert lib.msa_sparse_attn_prefill(ctypes.byref(_prefill(algo="kv_centric", **big).c()),
                                       FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, 0) \
        == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_kl_prefill(ctypes.byref(_prefill(**big).c()), FAKE, FAKE, FAKE, FAKE,
                                    FAKE, 0, ctypes.c_float(0.1), FAKE, FAKE, FAKE, FAKE,
                                    1 << 40, 0) == msa.MSA_ERR_UNSUPPORTED
    # just under the limit the KV-centric workspace is sized as usual
    under = dict(seq_len=1 << 22, q_begin=0, q_count=(1 << 31) // (64 * 64) - 1, num_groups=64,
                 top_k=64)
    assert lib.msa_workspace_size(ctypes.byref(_prefill(algo="kv_centric", **under).c()),
                                  msa.ENTRY["sparse_attn_prefill"], ctypes.byref(n)) == msa.MSA_OK
    assert n.value > 0


def test_python_helpers_reject_mismatched_inputs():
    """The C ABI cannot see buffer sizes, so the high-level helpers check shapes and dtypes
    before any launch: a mixed dtype, a head count that is not a multiple of the groups, or
    a wrongly shaped tensor raises ValueError (the tensors here never reach the device)."""
    import torch
    T, G, Hpg, d = 256, 2, 3, 64

    def pre(dtype=torch.bfloat16, **over):
        x = dict(q=torch.zeros(T, G * Hpg, 128, dtype=dtype),
                 k=torch.zeros(G, T, 128, dtype=dtype), v=torch.zeros(G, T, 128, dtype=dtype),
                 q_idx=torch.zeros(T, G, d, dtype=dtype), k_idx=torch.zeros(T, d, dtype=dtype))
        x.update(over)
        return x

    assert msa.check_prefill_inputs(pre()) == (T, G, Hpg, d, "bf16")
    bad = [pre(k=torch.zeros(G, T, 128, dtype=torch.float32)),            # mixed dtype
           pre(q=torch.zeros(T, 7, 128, dtype=torch.bfloat16)),             # 7 heads, 2 groups
           pre(v=torch.zeros(G, T - 1, 128, dtype=torch.bfloat16)),         # short v
           pre(q_idx=torch.zeros(T, G + 1, d, dtype=torch.bfloat16)),       # wrong groups
           pre(k_idx=torch.zeros(T, 128, dtype=torch.bfloat16)),            # wrong index dim
           pre(dtype=torch.float16)]                                         # unsupported dtype
    for x in bad:
        with pytest.raises(ValueError):
            msa.prefill(x, 4)
    with pytest.raises(ValueError):   # an output buffer of the wrong shape
        msa.prefill(pre(), 4, block_idx=torch.zeros(T, G, 5, dtype=torch.int32))
    B, L = 2, 512

    def dec(**over):
        dt = torch.bfloat16
        x = dict(q=torch.zeros(B, G * Hpg, 128, dtype=dt),
                 k_cache=torch.zeros(B, G, L, 128, dtype=dt),
                 v_cache=torch.zeros(B, G, L, 128, dtype=dt),
                 q_idx=torch.zeros(B, G, d, dtype=dt), k_idx=torch.zeros(B, L, d, dtype=dt),
                 seq_lens=torch.full((B,), L, dtype=torch.int32))
        x.update(over)
        return x

    assert msa.check_decode_inputs(dec()) == (B, G, Hpg, d, L, "bf16")
    for x in [dec(k_idx=torch.zeros(B, L, d, dtype=torch.float32)),
              dec(v_cache=torch.zeros(B, G, L // 2, 128, dtype=torch.bfloat16)),
              dec(seq_lens=torch.full((B,), L, dtype=torch.int64)),
              dec(q=torch.zeros(B, 5, 128, dtype=torch.bfloat16))]:
        with pytest.raises(ValueError):
            msa.decode(x, 4)


def test_noalloc_decode_validation():
    """The allocation-free decode entry refuses, on the host, what does not fit its fixed
    scratch (MSA_ERR_TOO_LARGE) and what the regular entry refuses; nothing reaches the
    device."""
    lib = msa.load_library()
    call = lib.msa_sparse_attn_decode_noalloc
    assert msa.NOALLOC_SCRATCH_BYTES == 32 << 20
    # bf16, G = Hpg = 8, top_k = 16: 1024 head-blocks per sequence, 520 bytes each
    n = ctypes.c_size_t(0)
    for B, fits in ((63, True), (64, False), (65535, False)):
        c = _decode(batch=B)
        assert lib.msa_workspace_size(ctypes.byref(c), msa.ENTRY["sparse_attn_decode"],
                                      ctypes.byref(n)) == msa.MSA_OK
        assert (n.value <= msa.NOALLOC_SCRATCH_BYTES) == fits
        if not fits:
            assert call(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_TOO_LARGE
    c32 = _decode(batch=32, dtype="f32")   # fp32 splits blocks in two: 65536 head-halves
    assert call(ctypes.byref(c32), FAKE, FAKE, FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_TOO_LARGE
    c = _decode(batch=4)
    assert call(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE + 4, 0) == \
        msa.MSA_ERR_INVALID_ARGUMENT                                  # misaligned out
    assert call(ctypes.byref(c), 0, FAKE, FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(_prefill().c()), FAKE, FAKE, FAKE, FAKE, FAKE, 0) == \
        msa.MSA_ERR_INVALID_ARGUMENT                                  # prefill problem
    assert call(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == msa.MSA_ERR_INVALID_ARGUMENT
    assert "scratch" in msa.status_string(msa.MSA_ERR_TOO_LARGE)


def test_decode_topk_rejections():
    """The decode attention with the selection folded in checks mode, alignment and the
    workspace on the host, before any launch."""
    lib = msa.load_library()
    c = _decode()
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(c), msa.ENTRY["sparse_attn_decode"],
                                  ctypes.byref(n)) == msa.MSA_OK and n.value > 0

    def call(cp, ws=n.value, scores=FAKE, idx=FAKE):
        return lib.msa_sparse_attn_decode_topk(ctypes.byref(cp), FAKE, FAKE, FAKE, scores, idx,
                                               FAKE, FAKE, ws, 0)

    assert call(_prefill().c()) == msa.MSA_ERR_INVALID_ARGUMENT
    assert call(c, scores=FAKE + 4) == msa.MSA_ERR_INVALID_ARGUMENT
    cp = _decode(max_len=4096)
    assert lib.msa_sparse_attn_decode_topk_paged(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, 31, 100,
                                                 FAKE, FAKE, FAKE, FAKE, n.value, 0) \
        == msa.MSA_ERR_INVALID_ARGUMENT  # max_len != pages_per_seq * 128
    assert lib.msa_sparse_attn_decode_topk_paged(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, 32, 100,
                                                 FAKE, FAKE, FAKE, FAKE, 0, 0) \
        == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert call(c, idx=FAKE + 8) == msa.MSA_ERR_INVALID_ARGUMENT
    assert call(c, ws=n.value - 1) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
