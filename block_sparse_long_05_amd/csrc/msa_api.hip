// Host side of the MSA C ABI (include/msa.h): argument validation, workspace sizing
// and launch configuration. Every check runs before any HIP call, so a rejected call
// never touches the device. The library keeps no state and never allocates or syncs.
#include "msa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "msa_launch.h"

using namespace msa;

namespace {

constexpr int64_t kMaxLen = int64_t(1) << 30;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* ptr) { return ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

msa_status check_problem(const msa_problem* p) {
  if (p == nullptr) return MSA_ERR_INVALID_ARGUMENT;
  if (p->dtype != MSA_DTYPE_F32 && p->dtype != MSA_DTYPE_BF16) return MSA_ERR_INVALID_ARGUMENT;
  if (p->mode != MSA_MODE_PREFILL && p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
  if (p->num_groups < 1 || p->heads_per_group < 1 || p->head_dim < 1 || p->index_dim < 1 ||
      p->block_size < 1 || p->top_k < 1)
    return MSA_ERR_INVALID_ARGUMENT;
  if (p->num_groups > MSA_MAX_GROUPS || p->heads_per_group > MSA_MAX_HEADS_PER_GROUP)
    return MSA_ERR_UNSUPPORTED;
  if (p->head_dim != MSA_HEAD_DIM || p->block_size != MSA_BLOCK_SIZE) return MSA_ERR_UNSUPPORTED;
  if (p->index_dim != 64 && p->index_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (p->top_k > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARGUMENT;
  if (p->mode == MSA_MODE_PREFILL) {
    if (p->seq_len < 1 || p->seq_len > kMaxLen) return MSA_ERR_INVALID_ARGUMENT;
    if (p->q_begin < 0 || p->q_count < 0 || p->q_begin + p->q_count > p->seq_len)
      return MSA_ERR_INVALID_ARGUMENT;
    if (p->algo < MSA_ALGO_AUTO || p->algo > MSA_ALGO_KV_CENTRIC) return MSA_ERR_INVALID_ARGUMENT;
  } else {
    if (p->batch < 1 || p->batch > 65535) return MSA_ERR_INVALID_ARGUMENT;
    if (p->max_len < 1 || p->max_len > kMaxLen) return MSA_ERR_INVALID_ARGUMENT;
    if (p->seq_lens == nullptr || (reinterpret_cast<uintptr_t>(p->seq_lens) & 3u) != 0)
      return MSA_ERR_INVALID_ARGUMENT;
  }
  return MSA_OK;
}

int64_t nblk_of(const msa_problem* p) {
  return ceil_div(p->mode == MSA_MODE_PREFILL ? p->seq_len : p->max_len, MSA_BLOCK_SIZE);
}

// Decode split-K plan: sparse bf16 uses one kept block per split (the block kernel of
// decode_attn.hip), sparse fp32 one half (64 keys) of one kept block per split; dense
// spreads the cache blocks so that the launch has a few thousand waves.
bool decode_block_kernel(const msa_problem* p, bool dense) {
  return !dense && p->dtype == MSA_DTYPE_BF16;
}

// Dense bf16 decode streams each (sequence, group) cache in a few long splits.
bool decode_dense_stream_kernel(const msa_problem* p, bool dense) {
  return dense && p->dtype == MSA_DTYPE_BF16;
}

void decode_split(const msa_problem* p, bool dense, int* nsplit, int* bps) {
  if (!dense) {
    *nsplit = decode_block_kernel(p, dense) ? p->top_k : 2 * p->top_k;
    *bps = 1;
    return;
  }
  if (decode_dense_stream_kernel(p, dense)) {
    int64_t kps;
    dense_decode_plan(p->batch, p->num_groups, p->max_len, nsplit, &kps);
    *bps = 0;
    return;
  }
  const int64_t nblk = nblk_of(p);
  int64_t per = ceil_div((int64_t)p->batch * p->num_groups * nblk, 4096);
  if (per < 1) per = 1;
  *bps = (int)per;
  *nsplit = (int)ceil_div(nblk, per);
}

size_t decode_ws_bytes(const msa_problem* p, bool dense) {
  int nsplit, bps;
  decode_split(p, dense, &nsplit, &bps);
  const size_t units = (size_t)p->batch * p->num_groups * nsplit * p->heads_per_group;
  return align_up(units * MSA_HEAD_DIM * sizeof(float)) + align_up(units * 2 * sizeof(float));
}

// The KV-centric prefill and the KL loss sort the kept entries (row, group, slot) by 32-bit
// entry id: the chunk must hold fewer than 2^31 of them.
bool entries_fit_int32(const msa_problem* p) {
  return (int64_t)p->q_count * p->num_groups * p->top_k < (int64_t(1) << 31);
}

size_t prefill_kv_ws_bytes(const msa_problem* p) {
  return kv_workspace_bytes(p->dtype == MSA_DTYPE_BF16, p->q_count, p->num_groups,
                            p->heads_per_group, p->top_k, (int)nblk_of(p));
}

size_t kl_ws_bytes(const msa_problem* p) {
  return kl_workspace_bytes(p->q_count, p->num_groups, p->heads_per_group, p->top_k,
                            (int)nblk_of(p));
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

// Scratch of the allocation-free decode entry point. Each GPU that runs the library holds
// its own copy from the module's load until the process ends. In host code `scratch`
// names only a host-side stand-in: its device address comes from hipGetSymbolAddress, once
// per device, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (looked up on the device's first call).
msa_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return MSA_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MSA_OK;
}

// Compute units of the current device (queried on the device's first call, then cached).
std::atomic<int> g_cu_count[kMaxDevices];

msa_status device_cu_count(int* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return MSA_ERR_HIP;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return MSA_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

msa_status run_decode_attention(const msa_problem* p, bool dense, const void* q, const void* k,
                                const void* v, const int32_t* block_idx, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t st,
                                PageMap pm = PageMap{}, const float* block_scores = nullptr,
                                int32_t* idx_out = nullptr) {
  const size_t need = decode_ws_bytes(p, dense);
  if (workspace_bytes < need) return MSA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return MSA_ERR_INVALID_ARGUMENT;
  int nsplit, bps;
  decode_split(p, dense, &nsplit, &bps);
  const size_t units = (size_t)p->batch * p->num_groups * nsplit * p->heads_per_group;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            align_up(units * MSA_HEAD_DIM * sizeof(float)));
  const int bf16 = p->dtype == MSA_DTYPE_BF16;
  if (decode_dense_stream_kernel(p, dense)) {
    hipError_t e = launch_decode_dense_bf16(q, k, v, p->seq_lens, p->batch, p->max_len,
                                            p->num_groups, p->heads_per_group, part_o, part_ml,
                                            st);
    if (e != hipSuccess) return MSA_ERR_HIP;
    return hip_status(launch_decode_combine(bf16, part_o, part_ml, out, p->batch,
                                            p->num_groups, p->heads_per_group, nsplit, st));
  }
  if (decode_block_kernel(p, dense)) {
    hipError_t e = launch_decode_attn_bf16(q, k, v, block_idx, p->seq_lens, p->batch,
                                           p->max_len, p->num_groups, p->heads_per_group,
                                           p->top_k, pm, part_o, part_ml, st, block_scores,
                                           idx_out, (int)nblk_of(p));
    if (e != hipSuccess) return MSA_ERR_HIP;
    return hip_status(launch_decode_combine(bf16, part_o, part_ml, out, p->batch,
                                            p->num_groups, p->heads_per_group, nsplit, st));
  }
  GatherParams gp = {};
  gp.mode = dense ? kDecodeDense : kDecodeSparse;
  gp.bf16 = bf16;
  gp.q = q;
  gp.k = k;
  gp.v = v;
  gp.block_idx = block_idx;
  gp.part_o = part_o;
  gp.part_ml = part_ml;
  gp.G = p->num_groups;
  gp.Hpg = p->heads_per_group;
  gp.top_k = p->top_k;
  gp.seq_lens = p->seq_lens;
  gp.B = p->batch;
  gp.max_len = p->max_len;
  gp.nsplit = nsplit;
  gp.blocks_per_split = bps;
  gp.half_blocks = dense ? 0 : 1;
  gp.pages = pm;
  hipError_t e = launch_gather_attn(gp, st);
  if (e != hipSuccess) return MSA_ERR_HIP;
  return hip_status(launch_decode_combine(gp.bf16, part_o, part_ml, out, p->batch, p->num_groups,
                                          p->heads_per_group, nsplit, st));
}

// msa_block_topk + the decode attention, or the attention workgroups selecting their own
// blocks: when each of them reads a short row (<= 1024 blocks) or when every workgroup is
// resident at once (one per (sequence, group, slot), two per CU). Otherwise the selection's
// reads, repeated by every workgroup of a row, cost more than the top-k launch they save.
msa_status run_decode_topk_attention(const msa_problem* p, const void* q, const void* k,
                                     const void* v, const float* block_scores,
                                     int32_t* block_idx, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t st, PageMap pm) {
  if (!aligned16(block_scores) || !aligned16(block_idx) || !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < decode_ws_bytes(p, false)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  const int64_t nblk = nblk_of(p);
  const int64_t units = (int64_t)p->batch * p->num_groups * p->top_k;
  int cus = 0;
  const msa_status sc = device_cu_count(&cus);
  if (sc != MSA_OK) return sc;
  if (decode_block_kernel(p, false) && nblk <= kSelectMaxBlocks &&
      (nblk <= 1024 || units <= 2 * (int64_t)cus))
    return run_decode_attention(p, false, q, k, v, nullptr, out, workspace, workspace_bytes, st,
                                pm, block_scores, block_idx);
  hipError_t e = launch_block_topk(block_scores, block_idx, (int64_t)p->batch * p->num_groups,
                                   p->num_groups, (int)nblk, p->top_k, 1, 0, p->seq_lens,
                                   p->max_len, st);
  if (e != hipSuccess) return MSA_ERR_HIP;
  return run_decode_attention(p, false, q, k, v, block_idx, out, workspace, workspace_bytes, st,
                              pm);
}

}  // namespace

extern "C" {

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARGUMENT: return "MSA_ERR_INVALID_ARGUMENT: bad pointer, range or enum";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: dimension or option not built";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL: see msa_workspace_size";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: a kernel launch or runtime query failed";
    case MSA_ERR_TOO_LARGE:
      return "MSA_ERR_TOO_LARGE: the problem exceeds the fixed scratch of an allocation-free "
             "entry point";
  }
  return "MSA_ERR_UNKNOWN";
}

msa_status msa_workspace_size(const msa_problem* p, int32_t entry, size_t* bytes) {
  if (bytes == nullptr) return MSA_ERR_INVALID_ARGUMENT;
  *bytes = 0;
  const msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  switch (entry) {
    case MSA_ENTRY_INDEX_SCORES:
    case MSA_ENTRY_BLOCK_TOPK:
    case MSA_ENTRY_INDEX_TOPK:
      return MSA_OK;
    case MSA_ENTRY_SPARSE_ATTN_PREFILL:
      if (p->mode != MSA_MODE_PREFILL) return MSA_ERR_INVALID_ARGUMENT;
      if (p->algo == MSA_ALGO_KV_CENTRIC && !entries_fit_int32(p)) return MSA_ERR_UNSUPPORTED;
      if (p->algo != MSA_ALGO_QUERY_CENTRIC && entries_fit_int32(p))
        *bytes = prefill_kv_ws_bytes(p);
      return MSA_OK;
    case MSA_ENTRY_SPARSE_ATTN_DECODE:
      if (p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
      *bytes = decode_ws_bytes(p, false);
      return MSA_OK;
    case MSA_ENTRY_DENSE_GQA_ATTN:
      if (p->mode == MSA_MODE_DECODE) *bytes = decode_ws_bytes(p, true);
      return MSA_OK;
    case MSA_ENTRY_INDEX_KL:
      if (p->mode != MSA_MODE_PREFILL) return MSA_ERR_INVALID_ARGUMENT;
      if (!entries_fit_int32(p)) return MSA_ERR_UNSUPPORTED;
      *bytes = kl_ws_bytes(p);
      return MSA_OK;
    default:
      return MSA_ERR_INVALID_ARGUMENT;
  }
}

msa_status msa_index_scores(const msa_problem* p, const void* q_idx, const void* k_idx,
                            float* block_scores, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_scores))
    return MSA_ERR_INVALID_ARGUMENT;
  const int bf16 = p->dtype == MSA_DTYPE_BF16;
  const int nblk = (int)nblk_of(p);
  if (p->mode == MSA_MODE_PREFILL) {
    if (p->q_count == 0) return MSA_OK;
    return hip_status(launch_index_scores_prefill(bf16, p->index_dim, q_idx, k_idx, block_scores,
                                                  p->q_begin, p->q_count, p->num_groups,
                                                  p->top_k, nblk, as_stream(stream)));
  }
  return hip_status(launch_index_scores_decode(bf16, p->index_dim, q_idx, k_idx, block_scores,
                                               p->seq_lens, p->batch, p->max_len,
                                               p->num_groups, p->top_k, nblk, PageMap{},
                                               as_stream(stream)));
}

msa_status msa_block_topk(const msa_problem* p, const float* block_scores, int32_t* block_idx,
                          void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!aligned16(block_scores) || !aligned16(block_idx)) return MSA_ERR_INVALID_ARGUMENT;
  const bool decode = p->mode == MSA_MODE_DECODE;
  const int64_t rows = (decode ? (int64_t)p->batch : p->q_count) * p->num_groups;
  if (rows == 0) return MSA_OK;
  return hip_status(launch_block_topk(block_scores, block_idx, rows, p->num_groups,
                                      (int)nblk_of(p), p->top_k, decode ? 1 : 0, p->q_begin,
                                      p->seq_lens, p->max_len, as_stream(stream)));
}

msa_status msa_index_topk(const msa_problem* p, const void* q_idx, const void* k_idx,
                          int32_t* block_idx, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_PREFILL || p->dtype != MSA_DTYPE_BF16 || p->top_k > 16)
    return MSA_ERR_UNSUPPORTED;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_idx))
    return MSA_ERR_INVALID_ARGUMENT;
  if (p->q_count == 0) return MSA_OK;
  return hip_status(launch_index_topk_prefill(p->index_dim, q_idx, k_idx, block_idx, p->q_begin,
                                              p->q_count, p->num_groups, p->top_k,
                                              as_stream(stream)));
}

msa_status msa_sparse_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                   const void* v, const int32_t* block_idx, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_PREFILL) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) || !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return MSA_ERR_INVALID_ARGUMENT;
  if (p->q_count == 0) return MSA_OK;
  // KV-centric when asked for, or by default when the caller's workspace can hold it (and
  // the chunk's kept entries fit 32-bit ids; otherwise the query-centric path runs).
  bool kv = p->algo == MSA_ALGO_KV_CENTRIC;
  if (kv && !entries_fit_int32(p)) return MSA_ERR_UNSUPPORTED;
  if (p->algo != MSA_ALGO_QUERY_CENTRIC && entries_fit_int32(p)) {
    const size_t need = prefill_kv_ws_bytes(p);
    const bool fits = workspace != nullptr && workspace_bytes >= need;
    if (kv && !fits) return workspace == nullptr && workspace_bytes >= need
                                ? MSA_ERR_INVALID_ARGUMENT
                                : MSA_ERR_WORKSPACE_TOO_SMALL;
    kv = fits;
  }
  if (kv) {
    if (!aligned16(workspace)) return MSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_kv_prefill(p->dtype == MSA_DTYPE_BF16, q, k, v, block_idx, out, lse,
                                        workspace, p->num_groups, p->heads_per_group, p->top_k,
                                        p->q_begin, p->q_count, p->seq_len, (int)nblk_of(p),
                                        as_stream(stream)));
  }
  GatherParams gp = {};
  gp.mode = kPrefillSparse;
  gp.bf16 = p->dtype == MSA_DTYPE_BF16;
  gp.q = q;
  gp.k = k;
  gp.v = v;
  gp.block_idx = block_idx;
  gp.out = out;
  gp.lse = lse;
  gp.G = p->num_groups;
  gp.Hpg = p->heads_per_group;
  gp.top_k = p->top_k;
  gp.q_begin = p->q_begin;
  gp.q_count = p->q_count;
  gp.seq_len = p->seq_len;
  return hip_status(launch_gather_attn(gp, as_stream(stream)));
}

msa_status msa_index_kl_prefill(const msa_problem* p, const void* q, const void* k,
                                const void* q_idx, const void* k_idx, const int32_t* block_idx,
                                const float* main_lse, float index_scale, float* loss,
                                float* dq_idx, float* dk_idx, void* workspace,
                                size_t workspace_bytes, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_PREFILL || p->dtype != MSA_DTYPE_BF16 || p->index_dim != 128)
    return MSA_ERR_UNSUPPORTED;
  if (!(index_scale > 0.f) || !(index_scale < 3.0e38f)) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) ||
      !aligned16(block_idx) || !aligned16(loss) || !aligned16(dq_idx) || !aligned16(dk_idx))
    return MSA_ERR_INVALID_ARGUMENT;
  if (main_lse != nullptr && (reinterpret_cast<uintptr_t>(main_lse) & 3u) != 0)
    return MSA_ERR_INVALID_ARGUMENT;
  if (p->q_count == 0) return MSA_OK;
  if (!entries_fit_int32(p)) return MSA_ERR_UNSUPPORTED;  // chunk the rows
  if (workspace_bytes < kl_ws_bytes(p)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return MSA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_index_kl_prefill(q, k, q_idx, k_idx, block_idx, main_lse, index_scale,
                                            loss,
                                            dq_idx, dk_idx, workspace, p->num_groups,
                                            p->heads_per_group, p->top_k, p->q_begin, p->q_count,
                                            p->seq_len, (int)nblk_of(p), as_stream(stream)));
}

msa_status msa_sparse_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_idx, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(block_idx) ||
      !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  return run_decode_attention(p, false, q, k_cache, v_cache, block_idx, out, workspace,
                              workspace_bytes, as_stream(stream));
}

msa_status msa_sparse_attn_decode_topk(const msa_problem* p, const void* q, const void* k_cache,
                                       const void* v_cache, const float* block_scores,
                                       int32_t* block_idx, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return MSA_ERR_INVALID_ARGUMENT;
  return run_decode_topk_attention(p, q, k_cache, v_cache, block_scores, block_idx, out,
                                   workspace, workspace_bytes, as_stream(stream), PageMap{});
}

msa_status msa_sparse_attn_decode_noalloc(const msa_problem* p, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_idx, void* out, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(block_idx) ||
      !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  if (decode_ws_bytes(p, false) > MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != MSA_OK) return st;
  return run_decode_attention(p, false, q, k_cache, v_cache, block_idx, out, ws,
                              MSA_NOALLOC_SCRATCH_BYTES, as_stream(stream));
}

namespace {
// Host checks shared by the paged entry points.
msa_status check_paged(const msa_problem* p, const int32_t* block_table, int32_t pages_per_seq,
                       int64_t num_pages) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->mode != MSA_MODE_DECODE) return MSA_ERR_INVALID_ARGUMENT;
  if (block_table == nullptr || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
    return MSA_ERR_INVALID_ARGUMENT;
  if (pages_per_seq < 1 || num_pages < 1) return MSA_ERR_INVALID_ARGUMENT;
  if (p->max_len != (int64_t)pages_per_seq * MSA_BLOCK_SIZE) return MSA_ERR_INVALID_ARGUMENT;
  return MSA_OK;
}
}  // namespace

msa_status msa_index_scores_paged(const msa_problem* p, const void* q_idx, const void* k_idx_pages,
                                  const int32_t* block_table, int32_t pages_per_seq,
                                  int64_t num_pages, float* block_scores, void* stream) {
  msa_status st = check_paged(p, block_table, pages_per_seq, num_pages);
  if (st != MSA_OK) return st;
  if (!aligned16(q_idx) || !aligned16(k_idx_pages) || !aligned16(block_scores))
    return MSA_ERR_INVALID_ARGUMENT;
  const PageMap pm{block_table, pages_per_seq, num_pages,
                   (int64_t)MSA_BLOCK_SIZE * p->index_dim};
  return hip_status(launch_index_scores_decode(p->dtype == MSA_DTYPE_BF16, p->index_dim, q_idx,
                                               k_idx_pages, block_scores, p->seq_lens, p->batch,
                                               p->max_len, p->num_groups, p->top_k,
                                               (int)nblk_of(p), pm, as_stream(stream)));
}

msa_status msa_sparse_attn_decode_paged(const msa_problem* p, const void* q, const void* k_pages,
                                        const void* v_pages, const int32_t* block_table,
                                        int32_t pages_per_seq, int64_t num_pages,
                                        const int32_t* block_idx, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  msa_status st = check_paged(p, block_table, pages_per_seq, num_pages);
  if (st != MSA_OK) return st;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(block_idx) ||
      !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  const PageMap pm{block_table, pages_per_seq, num_pages,
                   (int64_t)p->num_groups * MSA_BLOCK_SIZE * MSA_HEAD_DIM};
  return run_decode_attention(p, false, q, k_pages, v_pages, block_idx, out, workspace,
                              workspace_bytes, as_stream(stream), pm);
}

msa_status msa_sparse_attn_decode_topk_paged(const msa_problem* p, const void* q,
                                             const void* k_pages, const void* v_pages,
                                             const int32_t* block_table, int32_t pages_per_seq,
                                             int64_t num_pages, const float* block_scores,
                                             int32_t* block_idx, void* out, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  msa_status st = check_paged(p, block_table, pages_per_seq, num_pages);
  if (st != MSA_OK) return st;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages)) return MSA_ERR_INVALID_ARGUMENT;
  const PageMap pm{block_table, pages_per_seq, num_pages,
                   (int64_t)p->num_groups * MSA_BLOCK_SIZE * MSA_HEAD_DIM};
  return run_decode_topk_attention(p, q, k_pages, v_pages, block_scores, block_idx, out,
                                   workspace, workspace_bytes, as_stream(stream), pm);
}

msa_status msa_dense_gqa_attn(const msa_problem* p, const void* q, const void* k, const void* v,
                              void* out, void* workspace, size_t workspace_bytes, void* stream) {
  msa_status st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return MSA_ERR_INVALID_ARGUMENT;
  if (p->mode == MSA_MODE_DECODE)
    return run_decode_attention(p, true, q, k, v, nullptr, out, workspace, workspace_bytes,
                                as_stream(stream));
  if (p->q_count == 0) return MSA_OK;
  if (p->dtype == MSA_DTYPE_BF16)
    return hip_status(launch_dense_prefill_bf16(q, k, v, out, p->num_groups, p->heads_per_group,
                                                p->q_begin, p->q_count, p->seq_len,
                                                as_stream(stream)));
  GatherParams gp = {};
  gp.mode = kPrefillDense;
  gp.bf16 = p->dtype == MSA_DTYPE_BF16;
  gp.q = q;
  gp.k = k;
  gp.v = v;
  gp.out = out;
  gp.G = p->num_groups;
  gp.Hpg = p->heads_per_group;
  gp.top_k = p->top_k;
  gp.q_begin = p->q_begin;
  gp.q_count = p->q_count;
  gp.seq_len = p->seq_len;
  return hip_status(launch_gather_attn(gp, as_stream(stream)));
}

}  // extern "C"
