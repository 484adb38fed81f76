/*
 * msa.h - C ABI of the MiniMax Sparse Attention (MSA) hot path on AMD gfx950 (MI355X).
 *
 * The method (researchpapers.dev summary "MiniMax Sparse Attention", section
 * "Mechanism"; mlqm.cn blog on the MiniMax M3 sparse attention, sections 2.1-2.2):
 *   Index branch - one index query per GQA group is dotted with a single shared
 *     index-key head; token scores are max-pooled per 128-token block; per (query,
 *     group) the top-k blocks are kept, the query's own (local) block always
 *     included and future blocks never.
 *   Main branch - every query head of the group runs exact softmax attention over
 *     the keys of the kept blocks only (16 blocks x 128 tokens in the pages'
 *     configuration), both for causal prefill and for single-token decode.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous,
 *     row-major and 16-byte aligned. The library never allocates, frees, copies to
 *     the host or synchronises; work is enqueued in order on `stream` (a
 *     hipStream_t; NULL = the default stream). Calls are stateless and re-entrant,
 *     except msa_sparse_attn_decode_noalloc, whose fixed per-GPU scratch is shared by
 *     all of its calls on that GPU (see there).
 *   - All argument checks run on the host before any launch, so every error return
 *     below happens without touching the device. A failed launch returns
 *     MSA_ERR_HIP; faults inside kernels surface at the caller's next sync.
 *   - Float tensors other than block scores have the element type `dtype`
 *     (fp32 or bf16); arithmetic accumulates in fp32; outputs round to nearest even.
 *   - Shapes (G = num_groups, Hpg = heads_per_group, Hq = G*Hpg, D = head_dim,
 *     d = index_dim, nblk = ceil(len / 128), head h belongs to group h / Hpg):
 *       prefill  q [T, Hq, D]   k, v [G, T, D]   q_idx [T, G, d]   k_idx [T, d]
 *                out [T, Hq, D]
 *       decode   q [B, Hq, D]   k_cache, v_cache [B, G, max_len, D]
 *                q_idx [B, G, d]   k_idx [B, max_len, d]   seq_lens [B] (int32)
 *                out [B, Hq, D]
 *     Full tensors are always passed whole; prefill calls work on query rows
 *     [q_begin, q_begin + q_count) and the per-call intermediates (block scores,
 *     block ids) hold only those rows ("chunk-relative").
 *   - Inputs must be finite. NaN/Inf inputs give unspecified results (no fault).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 4
#define MSA_BLOCK_SIZE 128
#define MSA_HEAD_DIM 128
#define MSA_MAX_TOPK 64
#define MSA_MAX_GROUPS 64
#define MSA_MAX_HEADS_PER_GROUP 16

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad range, bad enum */
  MSA_ERR_UNSUPPORTED = 2,         /* valid but not built: head_dim, index_dim, block size, ... */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < msa_workspace_size(...) */
  MSA_ERR_HIP = 4,                 /* a kernel launch (or a runtime query) failed */
  MSA_ERR_TOO_LARGE = 5            /* needs more than the fixed scratch of an allocation-free
                                      entry point (MSA_NOALLOC_SCRATCH_BYTES) */
} msa_status;

typedef enum { MSA_DTYPE_F32 = 0, MSA_DTYPE_BF16 = 1 } msa_dtype;
typedef enum { MSA_MODE_PREFILL = 0, MSA_MODE_DECODE = 1 } msa_mode;

/* Which entry point a workspace size is asked for. */
typedef enum {
  MSA_ENTRY_INDEX_SCORES = 0,
  MSA_ENTRY_BLOCK_TOPK = 1,
  MSA_ENTRY_SPARSE_ATTN_PREFILL = 2,
  MSA_ENTRY_SPARSE_ATTN_DECODE = 3,
  MSA_ENTRY_DENSE_GQA_ATTN = 4,
  MSA_ENTRY_INDEX_TOPK = 5,
  MSA_ENTRY_INDEX_KL = 6
} msa_entry;

/* Prefill main-branch algorithm. Both give the same result up to fp32 rounding. */
typedef enum {
  MSA_ALGO_AUTO = 0,           /* library choice (KV-centric when the workspace allows) */
  MSA_ALGO_QUERY_CENTRIC = 1,  /* one wave per (token, group); no workspace */
  MSA_ALGO_KV_CENTRIC = 2      /* reverse index: each kept block staged once for all its queries */
} msa_algo;

typedef struct msa_problem {
  int32_t dtype;           /* msa_dtype of q, k, v, q_idx, k_idx, caches and out */
  int32_t mode;            /* msa_mode */
  int32_t num_groups;      /* G: GQA groups = KV heads = index queries per token, 1..64 */
  int32_t heads_per_group; /* Hpg: query heads per group, 1..16 */
  int32_t head_dim;        /* D: 128 */
  int32_t index_dim;       /* d: 64 or 128 */
  int32_t block_size;      /* 128 (selection and pooling granularity) */
  int32_t top_k;           /* blocks kept per (query, group), local block included, 1..64 */
  int64_t seq_len;         /* prefill: T, tokens in the sequence, 1..2^30 */
  int64_t q_begin;         /* prefill: first query row of this call */
  int64_t q_count;         /* prefill: query rows of this call (0 = nothing to do) */
  int32_t batch;           /* decode: B, 1..65535 */
  int32_t algo;            /* msa_algo (prefill sparse attention only) */
  int64_t max_len;         /* decode: cache capacity in tokens, 1..2^30 */
  const int32_t* seq_lens; /* decode: device int32[B]; each must be in [1, max_len]
                              (values outside are clamped into that range) */
} msa_problem;

/*
 * Index branch, step 1+2: token scores Q_idx . K_idx^T fused with 128-token block max
 * pooling (mlqm.cn blog, section 2.1: single shared index key, block max pooling).
 *   prefill: for chunk row i (token t = q_begin + i, local block b = t / 128) and
 *     group g, writes block_scores[i, g, c] = max_{j in block c} q_idx[t, g] . k_idx[j]
 *     for c < b, only when b >= top_k (otherwise every visible block is kept and no
 *     score is needed). block_scores is fp32 [q_count, G, nblk], nblk = ceil(T/128).
 *   decode: the same for the query at position L_b - 1 of sequence b, over
 *     k_idx[b, :, :]; block_scores is fp32 [B, G, ceil(max_len/128)].
 *   Entries not named above are left untouched. The token scores never reach memory.
 */
msa_status msa_index_scores(const msa_problem* p, const void* q_idx, const void* k_idx,
                            float* block_scores, void* stream);

/*
 * Index branch, step 3: block selection (researchpapers.dev summary, "Mechanism":
 * top-k blocks per query and group with the local block always kept).
 * For each row: if b + 1 <= top_k, blocks 0..b; otherwise b plus the top_k - 1 best
 * of blocks 0..b-1, ranked by score (higher first) then block index (lower first),
 * with -0.0 equal to +0.0. block_idx is int32 [rows, G, top_k] (rows = q_count for
 * prefill, B for decode), ascending, padded with -1. Reads only the block_scores
 * entries that msa_index_scores writes.
 */
msa_status msa_block_topk(const msa_problem* p, const float* block_scores, int32_t* block_idx,
                          void* stream);

/*
 * Index branch, steps 1-3 fused (prefill): writes block_idx for query rows
 * [q_begin, q_begin + q_count) exactly as msa_index_scores followed by msa_block_topk
 * would, but the block scores never reach memory: each query row keeps a running
 * top-(k-1) of its block maxima while the key blocks stream past (researchpapers.dev
 * summary "Mechanism"; mlqm.cn blog, section 2.1). Same ranking, padding and layout as
 * msa_block_topk. Built for dtype bf16, top_k <= 16 and prefill; any other problem returns
 * MSA_ERR_UNSUPPORTED (the two separate calls cover it). No workspace.
 */
msa_status msa_index_topk(const msa_problem* p, const void* q_idx, const void* k_idx,
                          int32_t* block_idx, void* stream);

/*
 * Main branch, prefill (mlqm.cn blog, section 2.2: gather the kept K/V blocks, then
 * attention; every head of a group shares the group's selection): for chunk row i
 * (token t = q_begin + i) and head h of group g,
 *   out[t, h] = sum_j softmax_j(q[t, h] . k[g, j] / sqrt(D)) v[g, j]
 * over the tokens j <= t of the blocks listed in block_idx[i, g, :]. Ids < 0 are
 * padding; ids above the query's local block are ignored. Writes out rows
 * [q_begin, q_begin + q_count). lse may be NULL; otherwise it is fp32 [T, Hq] (4-byte
 * aligned) and receives, for the same rows, lse[t, h] = ln sum_j exp(q[t, h] . k[g, j] /
 * sqrt(D)) over the same tokens (the softmax normaliser a backward pass or the index-branch
 * KL loss needs; -inf for a row with no visible kept token). workspace may be NULL when
 * msa_workspace_size(p, MSA_ENTRY_SPARSE_ATTN_PREFILL) is 0 for the chosen algo. The
 * KV-centric algo sorts the chunk's q_count * G * top_k kept entries by 32-bit id: with
 * 2^31 or more of them MSA_ALGO_AUTO runs the query-centric path and MSA_ALGO_KV_CENTRIC
 * returns MSA_ERR_UNSUPPORTED (call it on smaller row chunks).
 */
msa_status msa_sparse_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                   const void* v, const int32_t* block_idx, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Main branch, decode: the same attention for the single query of each sequence
 * (position L_b - 1) over the kept blocks of its cache, split over the kept blocks
 * and merged with a log-sum-exp combine in a fixed order.
 */
msa_status msa_sparse_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_idx, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Index branch step 3 and the main branch, decode, in one call: the block selection of
 * msa_block_topk (researchpapers.dev summary, "Mechanism": the local block plus the top_k - 1
 * best earlier blocks, same ranking and layout) with msa_sparse_attn_decode (mlqm.cn blog,
 * section 2.2: gather the kept blocks, then attention). block_scores is what
 * msa_index_scores (decode) wrote, fp32 [B, G, ceil(max_len/128)]; the call writes block_idx
 * (int32 [B, G, top_k]) with exactly the values msa_block_topk gives, and out bit for bit as
 * msa_block_topk followed by msa_sparse_attn_decode. For bf16 rows of up to 1024 blocks, or
 * up to 8192 blocks when B * G * top_k <= 2 * (the device's CU count), each attention
 * workgroup selects its (sequence, group)'s blocks from the scores itself and takes the one
 * of its slot, so the selection costs no launch of its own; otherwise the two kernels run
 * one after the other. Workspace: msa_workspace_size(p, MSA_ENTRY_SPARSE_ATTN_DECODE) (else
 * MSA_ERR_WORKSPACE_TOO_SMALL); mode must be MSA_MODE_DECODE (else MSA_ERR_INVALID_ARGUMENT).
 */
msa_status msa_sparse_attn_decode_topk(const msa_problem* p, const void* q, const void* k_cache,
                                       const void* v_cache, const float* block_scores,
                                       int32_t* block_idx, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of msa_sparse_attn_decode, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results (bit for bit) as msa_sparse_attn_decode,
 * minus the workspace: the split partials live in a fixed scratch array of
 * MSA_NOALLOC_SCRATCH_BYTES that the library holds once per GPU, from that GPU's first call
 * until the process ends. Neither this call nor its kernels allocate or free anything.
 *   - A problem whose msa_workspace_size(p, MSA_ENTRY_SPARSE_ATTN_DECODE) exceeds
 *     MSA_NOALLOC_SCRATCH_BYTES returns MSA_ERR_TOO_LARGE before anything else runs
 *     (32 MiB holds bf16 problems with B * G * Hpg * top_k <= 64512, e.g. 63 sequences of
 *     8 groups x 8 heads x 16 blocks; fp32 splits each block in two and holds half that).
 *   - `stream` must belong to the calling thread's current device (hipSetDevice): the
 *     scratch used is that device's copy.
 *   - Every call on one GPU shares that GPU's scratch, and each call overwrites what the
 *     previous one left there (nothing in it needs to start at zero). Calls whose work
 *     overlaps on one GPU (the same stream is fine; different streams, or different host
 *     threads, without ordering between them, are not) race and give unspecified results.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
msa_status msa_sparse_attn_decode_noalloc(const msa_problem* p, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_idx, void* out, void* stream);

/*
 * Paged decode (the GQA KV cache as a server keeps it, reused as is: researchpapers.dev
 * summary "Mechanism" and mlqm.cn blog section 3.1). The caches hold pages of 128 tokens,
 * one selection block per page, in any order:
 *   k_idx_pages [num_pages, 128, d]    k_pages, v_pages [num_pages, G, 128, D]
 *   block_table int32 [B, pages_per_seq]: page of logical block c of sequence b
 * with p->max_len == pages_per_seq * 128 (the per-sequence capacity); seq_lens as for
 * decode. Table entries of blocks after a sequence's local block (L - 1) / 128 are not
 * read. Page ids must lie in [0, num_pages); any other id reads page 0 (unspecified
 * values, no fault). The results equal those of the contiguous calls on the same data:
 * msa_index_scores_paged writes block_scores like msa_index_scores (decode), and
 * msa_block_topk then works unchanged on logical block ids; msa_sparse_attn_decode_paged
 * is msa_sparse_attn_decode reading each kept block from its page (same workspace size).
 * mode must be MSA_MODE_DECODE (else MSA_ERR_INVALID_ARGUMENT).
 */
msa_status msa_index_scores_paged(const msa_problem* p, const void* q_idx, const void* k_idx_pages,
                                  const int32_t* block_table, int32_t pages_per_seq,
                                  int64_t num_pages, float* block_scores, void* stream);
msa_status msa_sparse_attn_decode_paged(const msa_problem* p, const void* q, const void* k_pages,
                                        const void* v_pages, const int32_t* block_table,
                                        int32_t pages_per_seq, int64_t num_pages,
                                        const int32_t* block_idx, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);
/* msa_sparse_attn_decode_topk on the paged caches above (same arguments as
 * msa_sparse_attn_decode_paged, with block_scores in, block_idx out). */
msa_status msa_sparse_attn_decode_topk_paged(const msa_problem* p, const void* q,
                                             const void* k_pages, const void* v_pages,
                                             const int32_t* block_table, int32_t pages_per_seq,
                                             int64_t num_pages, const float* block_scores,
                                             int32_t* block_idx, void* out, void* workspace,
                                             size_t workspace_bytes, void* stream);

/*
 * Index-branch KL loss and its gradient, prefill (the training side of the index branch:
 * researchpapers.dev summary, "Mechanism": the index branch learns the main branch's
 * distribution on the selected blocks through a KL loss, and no gradient flows from it into
 * the main attention). For chunk row i (token t = q_begin + i) and group g, over the tokens
 * j <= t of the blocks listed in block_idx[i, g, :] (ids < 0 are padding, ids above the
 * local block are ignored, listed ids must be distinct):
 *   P_j = (1 / Hpg) sum over the group's heads h of softmax_j(q[t, h] . k[g, j] / sqrt(D))
 *   I_j = softmax_j(index_scale * q_idx[t, g] . k_idx[j])
 *   loss[i, g] = sum_j P_j (ln P_j - ln I_j)                        (0 ln 0 = 0)
 *   dq_idx[i, g, :] = sum_j index_scale (I_j - P_j) k_idx[j]
 *   dk_idx[j, :] += sum over the chunk's rows of index_scale (I_j - P_j) q_idx[t, g]
 * P is a constant: these are the gradients of sum(loss) with respect to q_idx and k_idx
 * only. A row with no visible kept token gets loss 0 and a zero gradient.
 * Layouts: q [T, G*Hpg, 128], k [G, T, 128], q_idx [T, G, 128], k_idx [T, 128] (bf16, full
 * tensors as for msa_sparse_attn_prefill); block_idx int32 [q_count, G, top_k]; loss fp32
 * [q_count, G] and dq_idx fp32 [q_count, G, 128] are written; dk_idx fp32 [T, 128] is
 * ADDED to (the caller zeroes it once, so the chunks of one sequence accumulate).
 * Built for dtype bf16, index_dim 128 and mode prefill, with fewer than 2^31 kept entries
 * q_count * G * top_k per call (else MSA_ERR_UNSUPPORTED: call it on smaller row chunks);
 * index_scale must be finite and > 0 (else MSA_ERR_INVALID_ARGUMENT). Loss and dq_idx are
 * bit-identical from run to run; dk_idx sums each block's entries in the order the
 * reverse index places them, which may vary from run to run at the level of fp32 rounding.
 * main_lse may be NULL; otherwise it is the fp32 [T, Hq] lse that msa_sparse_attn_prefill
 * wrote for the same rows and block_idx (ln of each head's softmax normaliser), and the main
 * heads' normalisers are taken from it instead of being recomputed (4-byte aligned).
 * Workspace: msa_workspace_size(p, MSA_ENTRY_INDEX_KL).
 */
msa_status msa_index_kl_prefill(const msa_problem* p, const void* q, const void* k,
                                const void* q_idx, const void* k_idx, const int32_t* block_idx,
                                const float* main_lse, float index_scale, float* loss,
                                float* dq_idx, float* dk_idx, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Dense GQA attention with the same heads (the baseline the researchpapers.dev summary
 * compares MSA against, "Key results"). Prefill: causal attention of query rows
 * [q_begin, q_begin + q_count) over keys j <= t. Decode: each sequence's query over
 * its whole cache of L_b tokens. Used for speedup context only.
 */
msa_status msa_dense_gqa_attn(const msa_problem* p, const void* q, const void* k, const void* v,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that `entry` needs for problem p (0 if none). */
msa_status msa_workspace_size(const msa_problem* p, int32_t entry, size_t* bytes);

/* Static description of a status code. */
const char* msa_status_string(msa_status s);

/* MSA_ABI_VERSION of the built library. */
int32_t msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
