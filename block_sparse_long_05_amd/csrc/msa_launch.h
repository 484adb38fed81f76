// Host-side launchers of the MSA kernels (internal; the public ABI is include/msa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// All launchers enqueue on `stream` and return hipGetLastError() of their launches.
hipError_t launch_index_scores_prefill(int bf16, int index_dim, const void* q_idx,
                                       const void* k_idx, float* block_scores, int64_t q_begin,
                                       int64_t q_count, int G, int top_k, int nblk,
                                       hipStream_t stream);

// Paged caches: logical block c of sequence b lives in page table[b * pps + c] (a page
// holds one 128-token block); table == nullptr means the contiguous per-sequence layout.
// Page ids outside [0, num_pages) read page 0 instead (unspecified values, no fault).
struct PageMap {
  const int32_t* table;
  int pps;            // pages per sequence (table row length)
  int64_t num_pages;
  int64_t page_elems; // elements per page of the tensor being addressed (per group for K/V)
  // Start of block c of sequence b: `contig` is sequence b's base in the contiguous layout;
  // `base` the paged tensor; `block_elems` the elements of one block in either layout.
  template <class T>
  __host__ __device__ const T* block(const T* base, const T* contig, int64_t b, int c,
                                     int64_t block_elems) const {
    if (table == nullptr) return contig + (int64_t)c * block_elems;
    int64_t pg = table[b * pps + c];
    if (pg < 0 || pg >= num_pages) pg = 0;
    return base + pg * page_elems;
  }
};

hipError_t launch_index_scores_decode(int bf16, int index_dim, const void* q_idx,
                                      const void* k_idx, float* block_scores,
                                      const int32_t* seq_lens, int B, int64_t max_len, int G,
                                      int top_k, int nblk, PageMap pm, hipStream_t stream);

// Fused prefill index scores + block max + top-k (bf16, top_k <= 16).
hipError_t launch_index_topk_prefill(int index_dim, const void* q_idx, const void* k_idx,
                                     int32_t* block_idx, int64_t q_begin, int64_t q_count, int G,
                                     int top_k, hipStream_t stream);

hipError_t launch_block_topk(const float* block_scores, int32_t* block_idx, int64_t rows, int G,
                             int nblk, int top_k, int decode, int64_t q_begin,
                             const int32_t* seq_lens, int64_t max_len, hipStream_t stream);

// Gather attention: one wave per (query, group[, split]); see attn_gather.hip.
enum GatherMode { kPrefillSparse = 0, kPrefillDense = 1, kDecodeSparse = 2, kDecodeDense = 3 };

struct GatherParams {
  int mode;
  int bf16;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_idx;  // sparse modes
  void* out;                 // prefill: final output
  float* lse;                // sparse prefill: per (row, head) ln of the softmax normaliser, or null
  float* part_o;             // decode: [units][Hpg][128] unnormalised partial outputs
  float* part_ml;            // decode: [units][Hpg][2] (running max in log2 units, sum)
  int G, Hpg, top_k;
  int64_t q_begin, q_count, seq_len;  // prefill
  const int32_t* seq_lens;            // decode
  int B;
  int64_t max_len;
  int nsplit;            // decode: splits per (sequence, group)
  int blocks_per_split;  // decode
  int half_blocks;       // decode: each split covers one half (64 keys) of one listed block
  PageMap pages;         // decode: paged K/V caches (pages.table == nullptr: contiguous)
};

hipError_t launch_gather_attn(const GatherParams& p, hipStream_t stream);

// Longest decode row (blocks) that a workgroup selects from (msa_select.h: kRowMax).
constexpr int kSelectMaxBlocks = 8192;

// Sparse decode attention, bf16 (decode_attn.hip): one partial per (sequence, group, kept
// block) into part_o [B * G * top_k][Hpg][128] / part_ml [..][Hpg][2]. With block_scores
// (fp32 [B, G, nblk], nblk <= kRowMax) the kernel selects the blocks itself and writes
// them to idx_out; block_idx is then not read.
hipError_t launch_decode_attn_bf16(const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, const int32_t* seq_lens, int B,
                                   int64_t max_len, int G, int Hpg, int top_k, PageMap pm,
                                   float* part_o, float* part_ml, hipStream_t st,
                                   const float* block_scores = nullptr, int32_t* idx_out = nullptr,
                                   int nblk = 0);

// Dense decode attention, bf16 (decode_attn.hip): one partial per (sequence, group, split of
// keys_per_split cache keys), nsplit splits per (sequence, group), as dense_decode_plan sets.
void dense_decode_plan(int B, int G, int64_t max_len, int* nsplit, int64_t* keys_per_split);
hipError_t launch_decode_dense_bf16(const void* q, const void* k, const void* v,
                                    const int32_t* seq_lens, int B, int64_t max_len, int G,
                                    int Hpg, float* part_o, float* part_ml, hipStream_t st);

// Fixed-order log-sum-exp merge of decode partials into out [B, Hq, 128].
hipError_t launch_decode_combine(int bf16, const float* part_o, const float* part_ml, void* out,
                                 int B, int G, int Hpg, int nsplit, hipStream_t stream);

// KV-centric sparse prefill attention (attn_tile.hip): reverse index, per-block tiles,
// log-sum-exp merge. `workspace` must hold kv_workspace_bytes(...) bytes.
size_t kv_workspace_bytes(int bf16, int64_t q_count, int G, int Hpg, int top_k, int nblk);
// Dense causal GQA prefill (bf16, flash-style) for query rows [q_begin, q_begin + q_count).
hipError_t launch_dense_prefill_bf16(const void* q, const void* k, const void* v, void* out, int G,
                                     int Hpg, int64_t q_begin, int64_t q_count, int64_t seq_len,
                                     hipStream_t stream);

// Reverse index (attn_tile.hip): counting sort of the visible kept entries (those not in
// `shared`, when given) by bucket g * nblk + c; offset[nb] = number sorted. count and cursor
// hold kStripes * nb counters each, offset nb + 1.
constexpr int kStripes = 16;
void launch_reverse_index(const int32_t* block_idx, int64_t n_entries, int G, int top_k,
                          int64_t q_begin, int nblk, const int32_t* shared, int QT,
                          int32_t* count, int32_t* cursor, int32_t* offset, int32_t* sorted,
                          hipStream_t st);
// In-place exclusive scan of a[0 .. n) with the total written to a[n] (one workgroup).
void launch_exclusive_scan(int32_t* a, int64_t n, hipStream_t st);

// Index-branch KL loss and gradients (index_kl.hip), bf16, D = d_idx = 128.
size_t kl_workspace_bytes(int64_t q_count, int G, int Hpg, int top_k, int nblk);
hipError_t launch_index_kl_prefill(const void* q, const void* k, const void* q_idx,
                                   const void* k_idx, const int32_t* block_idx,
                                   const float* main_lse, float index_scale,
                                   float* loss, float* dq_idx, float* dk_idx, void* workspace,
                                   int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count,
                                   int64_t seq_len, int nblk, hipStream_t st);

hipError_t launch_kv_prefill(int bf16, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, void* out, float* lse, void* workspace,
                             int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count,
                             int64_t seq_len, int nblk, hipStream_t stream);

}  // namespace msa
