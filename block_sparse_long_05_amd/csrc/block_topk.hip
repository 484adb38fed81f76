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
#include "msa_select.h"

namespace msa {

constexpr int kTopkWaves = 4;
constexpr int kCandCap = 512;

// Steps 3-4 over n items get(i) -> (key, block id), items in ascending block order.
// Counting uses popcount(ballot(...)) (one scalar op per 64 items) rather than
// shuffle reductions; up to 64 * kHeldSel items are read once into registers.
constexpr int kHeldSel = 8;

template <class Get>
__device__ __forceinline__ void select_exact(Get get, int n, int K, int32_t* out, int lane) {
  if (n <= 64 * kHeldSel) {
    uint32_t key[kHeldSel];
    int32_t idx[kHeldSel];
#pragma unroll
    for (int j = 0; j < kHeldSel; ++j) {
      const int i = 64 * j + lane;
      uint2 e = make_uint2(0u, 0u);
      if (i < n) e = get(i);
      key[j] = e.x;
      idx[j] = (int32_t)e.y;
    }
    const int nj = (n + 63) / 64;
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kHeldSel; ++j)
        if (j < nj) cnt += __popcll(__ballot(64 * j + lane < n && key[j] >= cand));
      if (cnt >= K) tau = cand;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < kHeldSel; ++j)
      if (j < nj) gt += __popcll(__ballot(64 * j + lane < n && key[j] > tau));
    const int need_eq = K - gt;
    int eq_base = 0, sel_base = 0;
#pragma unroll
    for (int j = 0; j < kHeldSel; ++j) {
      if (j < nj) {
        const bool valid = 64 * j + lane < n;
        const bool is_gt = valid && key[j] > tau;
        const bool is_eq = valid && key[j] == tau;
        const uint64_t eqm = __ballot(is_eq);
        const int eq_rank = eq_base + __popcll(eqm & lanemask_lt(lane));
        const bool sel = is_gt || (is_eq && eq_rank < need_eq);
        const uint64_t selm = __ballot(sel);
        if (sel) out[sel_base + __popcll(selm & lanemask_lt(lane))] = idx[j];
        eq_base += __popcll(eqm);
        sel_base += __popcll(selm);
      }
    }
    return;
  }
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      cnt += __popcll(__ballot(i < n && get(i).x >= cand));
    }
    if (cnt >= K) tau = cand;
  }
  int gt = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    gt += __popcll(__ballot(i < n && get(i).x > tau));
  }
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
  __shared__ int32_t kept_w[kTopkWaves][64];
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
  uint32_t* ck = cand_key[wave];
  int32_t* ci = cand_idx[wave];

  // Rows of up to 2048 blocks: the row is read once into registers (16-byte loads when
  // rows start 16-byte aligned), all loads in flight together; the candidates >= LB are
  // ranked as distinct 64-bit values (key << 32) | ~block, which encode the tie rule, so
  // their order in LDS does not matter.
  constexpr int kWaveHeld = 32;
  if (b <= 64 * kWaveHeld) {
    uint32_t key[kWaveHeld];
    const bool vec = (nblk & 3) == 0;
    auto blk = [&](int j) { return vec ? 4 * lane + 256 * (j >> 2) + (j & 3) : lane + 64 * j; };
    if (vec) {
#pragma unroll
      for (int j4 = 0; j4 < kWaveHeld / 4; ++j4) {
        const int c0 = 4 * lane + 256 * j4;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c0 < b) f = *reinterpret_cast<const float4*>(s + c0);
        key[4 * j4 + 0] = c0 + 0 < b ? ordered_key(f.x) : 0u;
        key[4 * j4 + 1] = c0 + 1 < b ? ordered_key(f.y) : 0u;
        key[4 * j4 + 2] = c0 + 2 < b ? ordered_key(f.z) : 0u;
        key[4 * j4 + 3] = c0 + 3 < b ? ordered_key(f.w) : 0u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kWaveHeld; ++j) {
        const int c = lane + 64 * j;
        key[j] = c < b ? ordered_key(s[c]) : 0u;
      }
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int j = 0; j < kWaveHeld; ++j) lmax = max(lmax, key[j]);
    uint32_t lb = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = lb | (1u << bit);
      if ((int)__popcll(__ballot(lmax >= cand)) >= K) lb = cand;
    }
    lb = max(lb, 1u);  // padding keys (0) never pass
    int n = 0;
#pragma unroll
    for (int j = 0; j < kWaveHeld; ++j) {
      const bool take = key[j] >= lb;
      const uint64_t m = __ballot(take);
      const int pos = n + __popcll(m & lanemask_lt(lane));
      if (take && pos < kCandCap) {
        ck[pos] = key[j];
        ci[pos] = blk(j);
      }
      n += __popcll(m);
    }
    if (n > 128) {
      // Ties at the bound (an all-equal row: every key). Keys above it all go; of the keys
      // equal to it the row keeps at most the K with the lowest ids, so only those are
      // offered, ranked by block id: (slab, lane, position) for 16-byte rows, else (j, lane).
      n = 0;
#pragma unroll
      for (int j = 0; j < kWaveHeld; ++j) {
        const bool take = key[j] > lb;
        const uint64_t m = __ballot(take);
        const int pos = n + __popcll(m & lanemask_lt(lane));
        if (take && pos < kCandCap) {
          ck[pos] = key[j];
          ci[pos] = blk(j);
        }
        n += __popcll(m);
      }
      int r0 = 0;  // equal keys in lower ids
      if (vec) {
#pragma unroll
        for (int j4 = 0; j4 < kWaveHeld / 4; ++j4) {
          if (r0 >= K) break;
          int cnt = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) cnt += key[4 * j4 + i] == lb ? 1 : 0;
          int incl = cnt;  // inclusive prefix over the lanes
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
          }
          int r = r0 + incl - cnt;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (key[4 * j4 + i] == lb) {
              if (r < K && n + r < kCandCap) {
                ck[n + r] = lb;
                ci[n + r] = blk(4 * j4 + i);
              }
              ++r;
            }
          }
          r0 += __shfl(incl, 63, 64);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kWaveHeld; ++j) {
          if (r0 >= K) break;
          const bool eq = key[j] == lb;
          const uint64_t m = __ballot(eq);
          const int r = r0 + __popcll(m & lanemask_lt(lane));
          if (eq && r < K && n + r < kCandCap) {
            ck[n + r] = lb;
            ci[n + r] = blk(j);
          }
          r0 += __popcll(m);
        }
      }
      n += min(r0, K);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (n <= kCandCap) {
      int base = 0;
      for (int i0 = 0; i0 < n; i0 += 64) {
        const bool valid = i0 + lane < n;
        const uint64_t v =
            valid ? ((uint64_t)ck[i0 + lane] << 32) | (0xFFFFFFFFu - (uint32_t)ci[i0 + lane]) : 0ull;
        int above = 0;
        for (int jj = 0; jj < n; ++jj)
          above += (((uint64_t)ck[jj] << 32) | (0xFFFFFFFFu - (uint32_t)ci[jj])) > v ? 1 : 0;
        const bool kept = valid && above < K;
        const uint64_t m = __ballot(kept);
        if (kept) kept_w[wave][base + __popcll(m & lanemask_lt(lane))] = ci[i0 + lane];
        base += __popcll(m);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < K) {  // ascending block order: each lane ranks one kept block
        const int c = kept_w[wave][lane];
        int rank = 0;
        for (int i = 0; i < K; ++i) rank += kept_w[wave][i] < c ? 1 : 0;
        o[rank] = c;
      }
      return;
    }
    // more candidates than LDS holds (heavily tied rows): the general path below
  }

  // 1. lower bound from the lane maxima.
  uint32_t lmax = 0;  // below the key of every finite float
  for (int c = lane; c < b; c += 64) lmax = max(lmax, ordered_key(s[c]));
  uint32_t lb = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = lb | (1u << bit);
    if ((int)__popcll(__ballot(lmax >= cand)) >= K) lb = cand;
  }
  lb = max(lb, 1u);
  // 2. compact the candidates (ascending block order): every key above the bound, and of the
  //    keys equal to it only the first K (the row keeps at most the K lowest-id ones of those)
  int n = 0, neq = 0;
  for (int c0 = 0; c0 < b; c0 += 64) {
    const int c = c0 + lane;
    uint32_t key = 0;
    if (c < b) key = ordered_key(s[c]);
    const bool eq = c < b && key == lb;
    const uint64_t me = __ballot(eq);
    const bool take = (c < b && key > lb) || (eq && neq + __popcll(me & lanemask_lt(lane)) < K);
    neq += __popcll(me);
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

// Long rows (decode: every cache block is a candidate): one workgroup of 16 waves per
// row. Wave w takes the exact top-K of its contiguous segment of blocks; because any
// block of the row's top-K is in the top-K of its own segment under the same order,
// wave 0 then finishes with an exact selection over the <= 16*K segment winners,
// which lie in ascending block order segment after segment.
constexpr int kLongWaves = 16;

__global__ __launch_bounds__(64 * kLongWaves) void block_topk_long_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ out, int G, int nblk, int top_k,
    int decode, int64_t q_begin, const int32_t* __restrict__ seq_lens, int64_t max_len) {
  __shared__ uint32_t win_key[kLongWaves * 64];
  __shared__ int32_t win_idx[kLongWaves * 64];
  __shared__ int32_t win_n[kLongWaves];
  __shared__ uint32_t seg_key[kLongWaves][kCandCap];
  __shared__ int32_t seg_idx[kLongWaves][kCandCap];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  int b;
  if (decode) {
    int64_t L = seq_lens[row / G];
    L = L < 1 ? 1 : (L > max_len ? max_len : L);
    b = (int)((L - 1) / kBlock);
  } else {
    b = (int)((q_begin + row / G) / kBlock);
  }
  int32_t* o = out + row * top_k;
  if (b + 1 <= top_k) {
    if (wave == 0)
      for (int i = lane; i < top_k; i += 64) o[i] = i <= b ? i : -1;
    return;
  }
  const int K = top_k - 1;
  if (wave == 0 && lane == 0) o[K] = b;
  if (K == 0) return;
  const float* s = scores + row * (int64_t)nblk;
  // segment of this wave: [lo, hi), 64-aligned
  const int per = ((b + kLongWaves - 1) / kLongWaves + 63) / 64 * 64;
  const int lo = min(b, wave * per), hi = min(b, lo + per);
  const int n = hi - lo;
  int32_t* wi = &win_idx[wave * 64];
  uint32_t* wk = &win_key[wave * 64];
  if (n <= K) {  // the whole segment goes through
    for (int i = lane; i < n; i += 64) {
      wi[i] = lo + i;
      wk[i] = ordered_key(s[lo + i]);
    }
    if (lane == 0) win_n[wave] = n;
  } else {
    // lower bound from lane maxima, candidates to LDS, exact selection. Segments of up
    // to 64 * kHeld blocks keep each lane's keys in registers (loaded once).
    constexpr int kHeld = 16;
    uint32_t held[kHeld];
    const bool in_regs = n <= 64 * kHeld;
    uint32_t lmax = 0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kHeld; ++j) {
        const int c = lo + 64 * j + lane;
        held[j] = c < hi ? ordered_key(s[c]) : 0u;
        lmax = max(lmax, held[j]);
      }
    } else {
      for (int c = lo + lane; c < hi; c += 64) lmax = max(lmax, ordered_key(s[c]));
    }
    uint32_t lb = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = lb | (1u << bit);
      if ((int)__popcll(__ballot(lmax >= cand)) >= K) lb = cand;
    }
    lb = max(lb, 1u);
    uint32_t* ck = seg_key[wave];
    int32_t* ci = seg_idx[wave];
    // every key above the bound; of the keys equal to it only the first K in block order (the
    // segment keeps at most the K lowest-id ones of those)
    int nc = 0, neq = 0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kHeld; ++j) {
        const int c = lo + 64 * j + lane;
        const bool eq = c < hi && held[j] == lb;
        const uint64_t me = __ballot(eq);
        const bool take =
            (c < hi && held[j] > lb) || (eq && neq + __popcll(me & lanemask_lt(lane)) < K);
        neq += __popcll(me);
        const uint64_t m = __ballot(take);
        const int pos = nc + __popcll(m & lanemask_lt(lane));
        if (take && pos < kCandCap) {
          ck[pos] = held[j];
          ci[pos] = c;
        }
        nc += __popcll(m);
      }
    } else {
      for (int c0 = lo; c0 < hi; c0 += 64) {
        const int c = c0 + lane;
        uint32_t key = 0;
        if (c < hi) key = ordered_key(s[c]);
        const bool eq = c < hi && key == lb;
        const uint64_t me = __ballot(eq);
        const bool take = (c < hi && key > lb) || (eq && neq + __popcll(me & lanemask_lt(lane)) < K);
        neq += __popcll(me);
        const uint64_t m = __ballot(take);
        const int pos = nc + __popcll(m & lanemask_lt(lane));
        if (take && pos < kCandCap) {
          ck[pos] = key;
          ci[pos] = c;
        }
        nc += __popcll(m);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (nc <= kCandCap)
      select_exact([&](int i) { return make_uint2(ck[i], (uint32_t)ci[i]); }, nc, K, wi, lane);
    else
      select_exact([&](int i) { return make_uint2(ordered_key(s[lo + i]), (uint32_t)(lo + i)); }, n,
                   K, wi, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < K; i += 64) wk[i] = ordered_key(s[wi[i]]);
    if (lane == 0) win_n[wave] = K;
  }
  __syncthreads();
  if (wave != 0) return;
  // Concatenate the winners (ascending block order; at most 16 * 63 of them, stored
  // flat over the segment buffers) and select exactly.
  uint32_t* all_key = &seg_key[0][0];
  int32_t* all_idx = &seg_idx[0][0];
  int tot = 0;
  for (int w = 0; w < kLongWaves; ++w) {
    const int m = win_n[w];
    for (int i = lane; i < m; i += 64) {
      all_key[tot + i] = win_key[w * 64 + i];
      all_idx[tot + i] = win_idx[w * 64 + i];
    }
    tot += m;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  select_exact([&](int i) { return make_uint2(all_key[i], (uint32_t)all_idx[i]); }, tot, K, o,
               lane);
}

// Decode rows (few rows, up to 8192 blocks each): one workgroup of 256 threads per row
// selects with row_select_wg (the whole row in registers, every load in flight at once),
// then writes the kept blocks in ascending order and the local block last.
__global__ __launch_bounds__(kRowThreads) void block_topk_row_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ out, int G, int nblk, int top_k,
    int decode, int64_t q_begin, const int32_t* __restrict__ seq_lens, int64_t max_len) {
  __shared__ uint64_t cand[kRowMax];
  __shared__ RowSelectShared sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
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
    if (tid < top_k) o[tid] = tid <= b ? tid : -1;
    return;
  }
  const int K = top_k - 1;
  if (tid == 0) o[K] = b;  // the local block is the largest kept id
  if (K == 0) return;
  row_select_wg(scores + row * (int64_t)nblk, (nblk & 3) == 0, b, K, cand, sh, tid);
  // the K kept blocks in ascending order: each thread ranks one of them among the others
  if (tid < K) {
    const int c = sh.sel[tid];
    o[sel_rank(sh.sel, K, c)] = c;
  }
}

hipError_t launch_block_topk(const float* block_scores, int32_t* block_idx, int64_t rows, int G,
                             int nblk, int top_k, int decode, int64_t q_begin,
                             const int32_t* seq_lens, int64_t max_len, hipStream_t stream) {
  if (decode && nblk <= kRowMax) {
    hipLaunchKernelGGL(block_topk_row_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream,
                       block_scores, block_idx, G, nblk, top_k, decode, q_begin, seq_lens, max_len);
    return hipGetLastError();
  }
  if (nblk > 2048 && rows <= 8192) {
    hipLaunchKernelGGL(block_topk_long_kernel, dim3((unsigned)rows), dim3(64 * kLongWaves), 0,
                       stream, block_scores, block_idx, G, nblk, top_k, decode, q_begin, seq_lens,
                       max_len);
    return hipGetLastError();
  }
  const int64_t grid = (rows + kTopkWaves - 1) / kTopkWaves;
  hipLaunchKernelGGL(block_topk_kernel, dim3((unsigned)grid), dim3(64 * kTopkWaves), 0, stream,
                     block_scores, block_idx, rows, G, nblk, top_k, decode, q_begin, seq_lens,
                     max_len);
  return hipGetLastError();
}

}  // namespace msa
