// Block selection of one decode row by a workgroup (researchpapers.dev summary "MiniMax
// Sparse Attention", "Mechanism": the local block plus the top_k - 1 best earlier blocks;
// mlqm.cn blog, section 2.2: topk_block_selection). Ranking: higher score first, then lower
// block index; -0.0 == +0.0. Shared by the decode top-k kernel and the decode attention
// kernel that selects its own block, so the two give the same ids by construction.
//
// 256 threads, rows of up to 8192 blocks, the whole row in registers so that every load is
// in flight at once and no step waits on global memory twice:
//   1. thread i holds the keys of blocks 4i .. 4i + 3, 4i + 1024 .. (16-byte loads; blocks
//      i, i + 256, ... when rows are not 16-byte aligned) and their maximum;
//   2. every wave takes the same lower bound LB of the row's K-th largest key: the K-th
//      largest of 64 group maxima (group l = threads l, l + 64, l + 128, l + 192; K groups
//      each hold a distinct key >= LB), or of the 256 thread maxima when K > 16 (a tighter
//      bound keeps the candidates few), and at least 1 so that padding keys (0) never pass;
//   3. each wave writes its keys >= LB to its own LDS region as 64-bit values
//      (key << 32) | ~block, which are distinct and order the row exactly by the rule (when
//      ties make those many, the keys > LB and only its K lowest-id keys == LB);
//   4. one wave keeps the K largest of those values (up to 256 candidates: each is kept
//      when fewer than K others are larger; more, in heavily tied rows: the K-th largest
//      from a most-significant-bit-first search).
#pragma once

#include <type_traits>

#include "msa_device.h"

namespace msa {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

constexpr int kRowThreads = 256;
constexpr int kRowPer = 32;
constexpr int kRowMax = kRowThreads * kRowPer;  // longest row a workgroup selects from

struct RowSelectShared {
  uint32_t tmax[kRowThreads];
  int32_t sel[64];
  int wcount[4];
  int slot_id;  // free for the caller
};
constexpr int kWaveCand = kRowMax / 4;  // LDS candidates per wave (64 lanes x kRowPer keys)

// Selects the K = top_k - 1 best of blocks 0 .. b - 1 of the row s (b > K >= 1). cand is an
// LDS array of kRowMax entries. Every thread of the workgroup calls it; on return (after a
// workgroup barrier) sh.sel[0 .. K) holds the kept blocks, in no particular order.
__device__ __forceinline__ void row_select_wg(const float* __restrict__ s, bool vec, int b, int K,
                                               uint64_t* cand, RowSelectShared& sh, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t key[kRowPer];
  auto blk = [&](int j) {
    return vec ? 4 * tid + kRowThreads * 4 * (j >> 2) + (j & 3) : tid + kRowThreads * j;
  };
  if (vec) {
#pragma unroll
    for (int j4 = 0; j4 < kRowPer / 4; ++j4) {
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (kRowThreads * 4 * j4 < b) {  // uniform: the slab holds a visible block
        const int c0 = 4 * tid + kRowThreads * 4 * j4;
        f = *reinterpret_cast<const float4*>(s + min(c0, (b - 1) & ~3));
      }
      const int c0 = 4 * tid + kRowThreads * 4 * j4;
      key[4 * j4 + 0] = c0 + 0 < b ? ordered_key(f.x) : 0u;
      key[4 * j4 + 1] = c0 + 1 < b ? ordered_key(f.y) : 0u;
      key[4 * j4 + 2] = c0 + 2 < b ? ordered_key(f.z) : 0u;
      key[4 * j4 + 3] = c0 + 3 < b ? ordered_key(f.w) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      float f = 0.f;
      if (kRowThreads * j < b) f = s[min(tid + kRowThreads * j, b - 1)];
      key[j] = tid + kRowThreads * j < b ? ordered_key(f) : 0u;
    }
  }
  uint32_t tmax = 0;
#pragma unroll
  for (int j = 0; j < kRowPer; ++j) tmax = max(tmax, key[j]);
  sh.tmax[tid] = tmax;
  __syncthreads();
  // every wave the same lower bound, so no barrier is needed to share it
  uint32_t lb = 0;
  if (K <= 16) {
    // 64 group maxima (group l = threads l, l + 64, l + 128, l + 192): one ballot a step
    const uint32_t gm = max(max(sh.tmax[lane], sh.tmax[lane + 64]),
                            max(sh.tmax[lane + 128], sh.tmax[lane + 192]));
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = lb | (1u << bit);
      if ((int)__popcll(__ballot(gm >= c)) >= K) lb = c;
    }
  } else {  // larger K: the 256 thread maxima keep the candidates few
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = sh.tmax[lane + 64 * i];
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = lb | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(v[i] >= c));
      if (cnt >= K) lb = c;
    }
  }
  lb = max(lb, 1u);  // padding keys (0) never pass
  // this wave's candidates, in its own region of cand
  uint64_t* cw = cand + wave * kWaveCand;
  auto cval = [&](int j) {
    return ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)blk(j));
  };
  int n = 0;
#pragma unroll
  for (int j = 0; j < kRowPer; ++j) {
    const bool take = key[j] >= lb;
    const uint64_t m = __ballot(take);
    if (m == 0) continue;
    if (take) cw[n + __popcll(m & lanemask_lt(lane))] = cval(j);
    n += __popcll(m);
  }
  if (n > 64) {
    n = 0;  // the region is written again
    // Many keys at or above the bound, i.e. ties at it (an all-equal row: every key). Keys
    // above the bound all go; of the keys equal to it the row can keep only the K with the
    // lowest block ids, and those are among the K lowest of their own wave, so the wave offers
    // just those: ranked by block id, i.e. by (slab, lane, position) for 16-byte rows and by
    // (j, lane) otherwise.
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const bool take = key[j] > lb;
      const uint64_t m = __ballot(take);
      if (m == 0) continue;
      if (take) cw[n + __popcll(m & lanemask_lt(lane))] = cval(j);
      n += __popcll(m);
    }
    int r0 = 0;  // the wave's equal keys in lower ids
    if (vec) {
#pragma unroll
      for (int j4 = 0; j4 < kRowPer / 4; ++j4) {
        if (r0 >= K) break;
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt += key[4 * j4 + i] == lb ? 1 : 0;
        int incl = cnt;  // inclusive prefix over the wave's lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        int r = r0 + incl - cnt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (key[4 * j4 + i] == lb) {
            if (r < K) cw[n + r] = cval(4 * j4 + i);
            ++r;
          }
        }
        r0 += __shfl(incl, 63, 64);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRowPer; ++j) {
        if (r0 >= K) break;
        const bool eq = key[j] == lb;
        const uint64_t m = __ballot(eq);
        const int r = r0 + __popcll(m & lanemask_lt(lane));
        if (eq && r < K) cw[n + r] = cval(j);
        r0 += __popcll(m);
      }
    }
    n += min(r0, K);
  }
  if (lane == 0) sh.wcount[wave] = n;
  __syncthreads();
  if (wave == 0) {
    const int n0 = sh.wcount[0], n1 = sh.wcount[1], n2 = sh.wcount[2], n3 = sh.wcount[3];
    const int p1 = n0, p2 = n0 + n1, p3 = n0 + n1 + n2, nt = p3 + n3;
    auto at = [&](int i) {
      const int w = (i >= p1) + (i >= p2) + (i >= p3);
      const int pw = w == 0 ? 0 : (w == 1 ? p1 : (w == 2 ? p2 : p3));
      return cand[w * kWaveCand + i - pw];
    };
    // above[i] = number of candidates larger than v[i] (values are distinct)
    auto count_above = [&](auto& v, auto& above, auto held) {
      constexpr int H = decltype(held)::value;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint64_t* c = cand + w * kWaveCand;
        const int nw = w == 0 ? n0 : (w == 1 ? n1 : (w == 2 ? n2 : n3));
#pragma unroll 4
        for (int j = 0; j < nw; ++j) {
          const uint64_t x = c[j];
#pragma unroll
          for (int i = 0; i < H; ++i) above[i] += x > v[i] ? 1 : 0;
        }
      }
    };
    if (nt <= 64) {
      uint64_t v[1] = {lane < nt ? at(lane) : 0ull};
      int above[1] = {0};
      count_above(v, above, std::integral_constant<int, 1>{});
      const bool kept = lane < nt && above[0] < K;
      const uint64_t m = __ballot(kept);
      if (kept) sh.sel[__popcll(m & lanemask_lt(lane))] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[0]);
    } else if (nt <= 256) {
      uint64_t v[4];
      int above[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = lane + 64 * i < nt ? at(lane + 64 * i) : 0ull;
        above[i] = 0;
      }
      count_above(v, above, std::integral_constant<int, 4>{});
      int base = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool kept = lane + 64 * i < nt && above[i] < K;
        const uint64_t m = __ballot(kept);
        if (kept) sh.sel[base + __popcll(m & lanemask_lt(lane))] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[i]);
        base += __popcll(m);
      }
    } else {  // heavily tied rows: a most-significant-bit-first search over the candidates
      const int nw[4] = {n0, n1, n2, n3};
      auto count_ge = [&](uint64_t c) {
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          for (int i0 = 0; i0 < nw[w]; i0 += 64)
            cnt += __popcll(__ballot(i0 + lane < nw[w] && cand[w * kWaveCand + i0 + lane] >= c));
        return cnt;
      };
      uint64_t tau = 0;
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t c = tau | (1ull << bit);
        if (count_ge(c) >= K) tau = c;
      }
      int base = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        for (int i0 = 0; i0 < nw[w]; i0 += 64) {
          const uint64_t v = i0 + lane < nw[w] ? cand[w * kWaveCand + i0 + lane] : 0ull;
          const bool kept = v >= tau && v != 0ull;
          const uint64_t m = __ballot(kept);
          if (kept) sh.sel[base + __popcll(m & lanemask_lt(lane))] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
          base += __popcll(m);
        }
    }
  }
  __syncthreads();
}

// Position of kept block c in ascending order among sel[0 .. K).
__device__ __forceinline__ int sel_rank(const int32_t* sel, int K, int c) {
  int rank = 0;
  for (int i = 0; i < K; ++i) rank += sel[i] < c ? 1 : 0;
  return rank;
}

}  // namespace msa
