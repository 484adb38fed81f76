// Index branch of MSA, block selection: per (query, group) keep the local block and the
// top_k - 1 best earlier blocks (researchpapers.dev summary "MiniMax Sparse Attention",
// "Mechanism"; mlqm.cn blog, section 2.2: topk_block_selection). Ranking: higher
// score first, then lower block index; -0.0 == +0.0.
//
// One wave per row. Exact selection without sorting:
//   1. every lane reduces its strided scores to one maximum; the K-th largest of the 64
//      lane maxima (K = top_k - 1) is a lower bound LB of the K-th largest score,
//      because K lanes each hold a score >= LB;
//   2. the scores >= LB are compacted into LDS in ascending block order (ballot
//      prefix sums); with ordinary data that is a few dozen candidates;
//   3. the K-th largest key tau among the candidates comes from a most-significant-bit
//      first search on 32-bit order-preserving keys, counting with the whole wave;
//   4. blocks with key > tau are kept, and of those with key == tau the lowest indices,
//      emitted in ascending block order.
// If the candidates overflow the LDS buffer (heavily tied rows), steps 3-4 run over
// the row in global memory instead, with the same result.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kTopkWaves = 4;
constexpr int kCandCap = 512;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Steps 3-4 over n items get(i) -> (key, block id), items in ascending block order.
template <class Get>
__device__ __forceinline__ void select_exact(Get get, int n, int K, int32_t* out, int lane) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
    for (int i = lane; i < n; i += 64) cnt += get(i).x >= cand ? 1 : 0;
    cnt = wave_sum_int(cnt);
    if (cnt >= K) tau = cand;
  }
  int gt = 0;
  for (int i = lane; i < n; i += 64) gt += get(i).x > tau ? 1 : 0;
  gt = wave_sum_int(gt);
  const int need_eq = K - gt;
  int eq_base = 0, sel_base = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    uint2 e = make_uint2(0u, 0u);
    if (i < n) e = get(i);
    const bool valid = i < n;
    const bool is_gt = valid && e.x > tau;
    const bool is_eq = valid && e.x == tau;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = eq_base + __popcll(eqm & lanemask_lt(lane));
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) out[sel_base + __popcll(selm & lanemask_lt(lane))] = (int32_t)e.y;
    eq_base += __popcll(eqm);
    sel_base += __popcll(selm);
  }
}

__global__ __launch_bounds__(64 * kTopkWaves) void block_topk_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ out, int64_t rows, int G, int nblk,
    int top_k, int decode, int64_t q_begin, const int32_t* __restrict__ seq_lens,
    int64_t max_len) {
  __shared__ uint32_t cand_key[kTopkWaves][kCandCap];
  __shared__ int32_t cand_idx[kTopkWaves][kCandCap];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kTopkWaves + wave;
  if (row >= rows) return;
  int b;
  if (decode) {
    int64_t L = seq_lens[row / G];
    L = L < 1 ? 1 : (L > max_len ? max_len : L);
    b = (int)((L - 1) / kBlock);
  } else {
    b = (int)((q_begin + row / G) / kBlock);
  }
  int32_t* o = out + row * top_k;
  if (b + 1 <= top_k) {  // every visible block fits
    for (int i = lane; i < top_k; i += 64) o[i] = i <= b ? i : -1;
    return;
  }
  const int K = top_k - 1;
  if (lane == 0) o[K] = b;  // the local block is the largest kept id
  if (K == 0) return;
  const float* s = scores + row * (int64_t)nblk;

  // 1. lower bound from the lane maxima.
  uint32_t lmax = 0;  // below the key of every finite float
  for (int c = lane; c < b; c += 64) lmax = max(lmax, ordered_key(s[c]));
  uint32_t lb = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = lb | (1u << bit);
    if (__popcll(__ballot(lmax >= cand)) >= K) lb = cand;
  }
  // 2. compact the candidates (ascending block order).
  uint32_t* ck = cand_key[wave];
  int32_t* ci = cand_idx[wave];
  int n = 0;
  for (int c0 = 0; c0 < b; c0 += 64) {
    const int c = c0 + lane;
    uint32_t key = 0;
    if (c < b) key = ordered_key(s[c]);
    const bool take = c < b && key >= lb;
    const uint64_t m = __ballot(take);
    const int pos = n + __popcll(m & lanemask_lt(lane));
    if (take && pos < kCandCap) {
      ck[pos] = key;
      ci[pos] = c;
    }
    n += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (n <= kCandCap) {
    select_exact([&](int i) { return make_uint2(ck[i], (uint32_t)ci[i]); }, n, K, o, lane);
  } else {
    select_exact([&](int i) { return make_uint2(ordered_key(s[i]), (uint32_t)i); }, b, K, o,
                 lane);
  }
}

hipError_t launch_block_topk(const float* block_scores, int32_t* block_idx, int64_t rows, int G,
                             int nblk, int top_k, int decode, int64_t q_begin,
                             const int32_t* seq_lens, int64_t max_len, hipStream_t stream) {
  const int64_t grid = (rows + kTopkWaves - 1) / kTopkWaves;
  hipLaunchKernelGGL(block_topk_kernel, dim3((unsigned)grid), dim3(64 * kTopkWaves), 0, stream,
                     block_scores, block_idx, rows, G, nblk, top_k, decode, q_begin, seq_lens,
                     max_len);
  return hipGetLastError();
}

}  // namespace msa
