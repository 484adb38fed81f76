// Index-branch KL loss and its gradient (the training side of the index branch).
//
// The researchpapers.dev summary of the MSA paper ("Mechanism") trains the Index Branch with
// a KL loss towards the Main Branch's distribution on the selected blocks and cuts the
// gradient from the index path into the main attention. For a (query t, group g) row with
// visible selected tokens j:
//   P_j = mean over the group's heads h of softmax_j(q[t, h] . k[g, j] / sqrt(D))   (constant)
//   I_j = softmax_j(index_scale * q_idx[t, g] . k_idx[j])
//   loss = sum_j P_j (ln P_j - ln I_j)
//   W_j  = index_scale * (I_j - P_j)
//   dq_idx[t, g] = sum_j W_j k_idx[j]        dk_idx[j] += sum over rows W_j q_idx[t, g]
//
// The work is organised on the KV side, like the reverse-index half of the main branch:
// all kept entries are counting-sorted by (g, block), each bucket is cut into units of at
// most 256 entries (a unit never spans two blocks), and one workgroup per unit stages the
// block's K (row swizzle) and index keys (V swizzle) in LDS once. Two passes over the units:
//   pass 0: per entry, a partial (max, sum of exponentials) for each head and for the
//           index scores over the block's visible keys; a fold turns a row's partials into
//           log-sum-exps (log2 units) in slot order. When the caller passes the main heads'
//           log-sum-exps (the forward attention computes them anyway), only the index
//           scores are reduced here;
//   pass 1: per entry, P (head mean, from the row's log-sum-exps) and I for the block's
//           keys, the entry's loss term, its dq_idx partial (K_idx^T . W^T, the transpose
//           read of the main branch's PV product) and, per unit, the dk_idx partial of the
//           block (wave w owns keys 32 w .. 32 w + 31; the waves' W and q_idx tiles are
//           exchanged through LDS and read back transposed).
// Folds then sum a row's loss and dq_idx partials in slot order, and a block's dk_idx
// partials over groups and units in order, adding into dk_idx.
#include <algorithm>
#include <math.h>

#include "msa_device.h"
#include "msa_launch.h"
#include "msa_tile.h"

namespace msa {

constexpr int kUnit = 256;                        // sorted entries per unit at most
constexpr int kRowBytes = kHeadDim * 2;           // one bf16 row of 128 values
constexpr int kWaveTile = 32 * kRowBytes;         // 32 rows (one wave's entries)

__global__ void kl_unit_count_kernel(const int32_t* __restrict__ offset, int64_t nb,
                                     int32_t* __restrict__ unit_off) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < nb;
       k += (int64_t)gridDim.x * blockDim.x)
    unit_off[k] = (offset[k + 1] - offset[k] + kUnit - 1) / kUnit;
}

__global__ void kl_unit_fill_kernel(const int32_t* __restrict__ unit_off, int64_t nb,
                                    int32_t* __restrict__ unit_bucket) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < nb;
       k += (int64_t)gridDim.x * blockDim.x)
    for (int32_t u = unit_off[k]; u < unit_off[k + 1]; ++u) unit_bucket[u] = (int32_t)k;
}

// One MFMA operand row of 128 bf16 values. The loads are unconditional: a lane without an
// entry addresses the chunk's first row and has every key masked (its causal limit is -1024),
// and a load behind a lane mask would make the compiler wait for every access in flight.
__device__ __forceinline__ void load_row_op(u32x4* op, const uint16_t* row, int q) {
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s)
    op[s] = *reinterpret_cast<const u32x4*>(row + 16 * s + 8 * q);
}

// Pass 0 (kGrad false) or pass 1 (kGrad true) over one unit. kIndexOnly: pass 0 with the
// main heads' log-sum-exps given by the caller, so only the index scores are reduced.
// Pass 0 over one unit: per entry, (max, sum of exponentials) of each main head's scores and
// of the index scores over the block's visible keys. kIndexOnly: the main heads'
// log-sum-exps are given by the caller, so only the index scores are reduced. Four waves
// take the unit's 32-entry groups in turn; two workgroups share a CU (65 KiB of LDS).
template <bool kIndexOnly>
__global__ __launch_bounds__(256, 2) void kl_stats_unit_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ QI, const uint16_t* __restrict__ KI,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ unit_off, const int32_t* __restrict__ unit_bucket, int64_t nb,
    int nblk, int G, int Hpg, int top_k, int64_t q_begin, int64_t seq_len, float index_scale,
    float* __restrict__ part_stats) {
  __shared__ __align__(16) uint8_t Kb[kIndexOnly ? 16 : kBlock * kRowBytes];
  __shared__ __align__(16) uint8_t KIb[kBlock * kRowBytes];
  __shared__ int32_t ids[kUnit];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  if (u >= unit_off[nb]) return;
  const int k = __builtin_amdgcn_readfirstlane(unit_bucket[u]);
  const int g = k / nblk;
  const int c = k - g * nblk;
  const int e0 = offset[k] + kUnit * (u - unit_off[k]);
  const int n = min(kUnit, offset[k + 1] - e0);
  if (tid < n) ids[tid] = sorted[e0 + tid];
  if constexpr (!kIndexOnly) k_block_dma<256>(K, g, c, seq_len, Kb, tid);
  k_block_dma<256, true>(KI, 0, c, seq_len, KIb, tid);
  MSA_WAIT_VMCNT(0);
  __syncthreads();

  const int n32 = lane & 31, q = lane >> 5;
  const float c_main = kLog2e / sqrtf((float)kHeadDim);
  const float c_idx = kLog2e * index_scale;
  const int Hq = G * Hpg;
  const int ngroups = (n + 31) / 32;

  for (int grp = wave; grp < ngroups; grp += 4) {
    const int ent = 32 * grp + n32;
    const bool ok = ent < n;
    const int32_t id = ok ? ids[ent] : 0;
    const int64_t rowg = id / top_k;                 // chunk row * G + g
    const int64_t t = q_begin + rowg / G;
    // last visible key offset in the block, folded with the lane's key offset 4q
    const int lim = min(max((int)t - c * kBlock, -1), kBlock - 1);
    const int limq = ok ? lim - 4 * q : -1024;  // no key is visible to a lane without entry
    const uint16_t* qrow = Q + (t * Hq + (int64_t)g * Hpg) * kHeadDim;
    u32x4 qiop[kHeadDim / 16];
    load_row_op(qiop, QI + (t * G + g) * kHeadDim, q);
    // (max, sum) of head h's scores (h < Hpg, from the rows in qop) or of the index scores
    // only entries of the block's own tokens see part of it: a wave with none of those skips
    // the per-score causal compares (a lane without entry has limit -1024)
    const bool cut = __ballot(limq < kBlock - 1 - 4 * q) != 0;
    auto stat = [&](int h, const u32x4* qop, bool main) __attribute__((always_inline)) {
      const float sc = main ? c_main : c_idx;
      f32x16 sv[4];
      float mx = -INFINITY;
      int lq = limq;
      asm volatile("" : "+v"(lq));
      if (main) s_tiles4_swz(Kb, n32, qop, q, sv);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if (!main) sv[kt] = s_tile_vswz(KIb, 32 * kt + n32, qiop, q);
        if (cut) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = 32 * kt + 8 * (r >> 2) + (r & 3) <= lq ? sv[kt][r] * sc : -INFINITY;
            sv[kt][r] = x;
            mx = fmaxf(mx, x);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sv[kt][r] *= sc;
            mx = fmaxf(mx, sv[kt][r]);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float l = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) l += fast_exp2(sv[kt][r] - mx);
      l += __shfl_xor(l, 32, 64);
      if (ok && q == 0)
        *reinterpret_cast<float2*>(part_stats + ((int64_t)id * (Hpg + 1) + h) * 2) =
            make_float2(mx, l);
    };
    if constexpr (!kIndexOnly) {
      // the next head's query rows are loaded while this head's products run (two buffers;
      // past the last head the last one is loaded again: every load is unconditional)
      const int hl = Hpg - 1;
      u32x4 qa[kHeadDim / 16], qb[kHeadDim / 16];
      load_row_op(qa, qrow, q);
      for (int h = 0; h < Hpg; h += 2) {
        load_row_op(qb, qrow + min(h + 1, hl) * kHeadDim, q);
        stat(h, qa, true);
        if (h + 1 >= Hpg) break;
        load_row_op(qa, qrow + min(h + 2, hl) * kHeadDim, q);
        stat(h + 1, qb, true);
      }
    }
    stat(Hpg, qiop, false);
  }
}

// Pass 1 over one unit: per entry, P (head mean, from the row's log-sum-exps) and I for the
// block's keys, the entry's loss term, W = index_scale (I - P) and its dq_idx partial
// (K_idx^T . W^T, the transpose read of the main branch's PV product); per unit, the block's
// dk_idx partial W^T . q_idx. Eight waves (two per SIMD): wave w takes entries
// 32 w .. 32 w + 31, so a unit of at most 256 entries is a single round. W is rounded to
// bf16 once and serves both products. The block's key gradient is split over the waves
// (wave w: keys 32 (w % 4) + 0..31, dims 64 (w / 4) + 0..63); the waves' W and q_idx tiles
// reach it through LDS in two halves (waves 0-3, then 4-7) sharing one exchange area, in the
// unit's entry order.
__global__ __launch_bounds__(512, 2) void kl_grad_unit_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ QI, const uint16_t* __restrict__ KI,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ unit_off, const int32_t* __restrict__ unit_bucket, int64_t nb,
    int nblk, int G, int Hpg, int top_k, int64_t q_begin, int64_t seq_len, float index_scale,
    const float* __restrict__ lse, float* __restrict__ part_loss, float* __restrict__ part_dq,
    float* __restrict__ part_dk) {
  __shared__ __align__(16) uint8_t Kb[kBlock * kRowBytes];
  __shared__ __align__(16) uint8_t KIb[kBlock * kRowBytes];
  __shared__ __align__(16) uint8_t Wb[4 * kWaveTile];   // per publishing wave: W tile
  __shared__ __align__(16) uint8_t QIb[4 * kWaveTile];  // per publishing wave: q_idx rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  if (u >= unit_off[nb]) return;
  const int k = __builtin_amdgcn_readfirstlane(unit_bucket[u]);
  const int g = k / nblk;
  const int c = k - g * nblk;
  const int e0 = offset[k] + kUnit * (u - unit_off[k]);
  const int n = min(kUnit, offset[k + 1] - e0);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  k_block_dma_s<512>(K, g, c, seq_len, Kb, wv, dma_lane_off<false>(lane), tid);
  k_block_dma_s<512, true>(KI, 0, c, seq_len, KIb, wv, dma_lane_off<true>(lane), tid);

  const int n32 = lane & 31, q = lane >> 5;
  const int ent = 32 * wave + n32;
  const bool ok = ent < n;
  const int32_t id = ok ? sorted[e0 + ent] : 0;
  MSA_WAIT_VMCNT(0);
  __syncthreads();

  const float c_main = kLog2e / sqrtf((float)kHeadDim);
  const float c_idx = kLog2e * index_scale;
  const int Hq = G * Hpg;
  const int ngroups = (n + 31) / 32;
  const bool active = wave < ngroups;  // wave-uniform
  uint32_t wp[4][8];                   // W (bf16 pairs) of the lane's 64 keys
  u32x4 qiop[kHeadDim / 16];
  if (active) {
    const int64_t rowg = id / top_k;  // chunk row * G + g
    const int64_t t = q_begin + rowg / G;
    const int lim = min(max((int)t - c * kBlock, -1), kBlock - 1);
    const int limq = ok ? lim - 4 * q : -1024;  // no key is visible to a lane without entry
    const uint16_t* qrow = Q + (t * Hq + (int64_t)g * Hpg) * kHeadDim;
    const float* lrow = lse + rowg * (Hpg + 1);
    float w[4][16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w[kt][r] = 0.f;
    // P: mean over the group's heads of each head's probabilities. The next head's query
    // rows and log-sum-exp are loaded while this head's products run (two buffers; past the
    // last head the last one is loaded again, so every load is unconditional and the compiler
    // waits only for the buffer it reads).
    // Only entries of the block's own tokens see part of it (their local block); a wave with
    // none of those skips the per-score causal compares (one uniform test per wave). A lane
    // without entry has every key masked: its limit is -1024.
    const bool cut = __ballot(limq < kBlock - 1 - 4 * q) != 0;
    auto head_p = [&](const u32x4* qop, float lh) __attribute__((always_inline)) {
      // the causal compares are redone per head (two VALU ops per score) rather than
      // kept as 64 hoisted lane masks, which the compiler would spill
      int lq = limq;
      asm volatile("" : "+v"(lq));
      f32x16 acc4[4];
      s_tiles4_swz(Kb, n32, qop, q, acc4);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 sv = acc4[kt];
        if (cut) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(sv[r], c_main, -lh));
            w[kt][r] += 32 * kt + 8 * (r >> 2) + (r & 3) <= lq ? e : 0.f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) w[kt][r] += fast_exp2(fmaf(sv[r], c_main, -lh));
        }
      }
    };
    {
      const int hl = Hpg - 1;
      u32x4 qa[kHeadDim / 16], qb[kHeadDim / 16];
      load_row_op(qa, qrow, q);
      float la = lrow[0];  // a lane without entry reads row 0 (all its keys masked)
      for (int h = 0; h < Hpg; h += 2) {
        load_row_op(qb, qrow + min(h + 1, hl) * kHeadDim, q);
        const float lb = lrow[min(h + 1, hl)];
        head_p(qa, la);
        if (h + 1 >= Hpg) break;
        load_row_op(qa, qrow + min(h + 2, hl) * kHeadDim, q);
        la = lrow[min(h + 2, hl)];
        head_p(qb, lb);
      }
    }
    load_row_op(qiop, QI + (t * G + g) * kHeadDim, q);
    const float inv_h = 1.f / (float)Hpg;
    const float li = lrow[Hpg];
    float lsum = 0.f;
    int lq = limq;
    asm volatile("" : "+v"(lq));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const f32x16 xv = s_tile_vswz(KIb, 32 * kt + n32, qiop, q);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = w[kt][r] * inv_h;             // 0 for keys the row cannot see
        const float z = fmaf(xv[r], c_idx, -li);      // log2 I
        const float iv = fast_exp2(z);
        // P ln(P / I) in log2 units; p = 0 gives 0 (the clamp only keeps the log finite)
        lsum += p * (__builtin_amdgcn_logf(fmaxf(p, 1e-30f)) - z);
        w[kt][r] = index_scale * (iv - p);
      }
      if (cut) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          w[kt][r] = 32 * kt + 8 * (r >> 2) + (r & 3) <= lq ? w[kt][r] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) wp[kt][i] = pack_bf16x2(w[kt][2 * i], w[kt][2 * i + 1]);
    }
    lsum += __shfl_xor(lsum, 32, 64);
    if (ok && q == 0) part_loss[id] = lsum * kLn2;
    // dq^T = K_idx^T . W^T over the block's two 64-key halves
    f32x16 o[4] = {};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 pb[4];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const uint32_t* pr = &wp[2 * half + (uu >> 1)][4 * (uu & 1)];
        pb[uu] = u32x4{pr[0], pr[1], pr[2], pr[3]};
      }
      pv_half_tr(o, pb, KIb, lane, half);
    }
    if (ok) {
      float* dst = part_dq + (int64_t)id * kHeadDim + 4 * q;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * j) =
              f32x4{o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
    }
  }
  // dk (keys 32 (wave % 4) + C rows, dims 64 (wave / 4) + 32 dn + column) += W^T . q_idx
  f32x16 dk[2] = {};
  const int kq = wave & 3, dq0 = 2 * (wave >> 2);
#pragma unroll
  for (int hx = 0; hx < 2; ++hx) {
    if (hx == 1) __syncthreads();  // every wave is done reading the first half's tiles
    if ((wave >> 2) == hx && active) {
      // this wave's W (32 entries x 128 keys) and q_idx rows into its slot, V swizzle
      uint8_t* wrow = Wb + kq * kWaveTile + n32 * kRowBytes;
      const int sw = v_swz(n32);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x2*>(wrow + (((4 * kt + j) ^ sw) * 16) + 8 * q) =
              u32x2{wp[kt][2 * j], wp[kt][2 * j + 1]};
      uint8_t* qrow_l = QIb + kq * kWaveTile + n32 * kRowBytes;
#pragma unroll
      for (int s = 0; s < kHeadDim / 16; ++s)
        *reinterpret_cast<u32x4*>(qrow_l + ((2 * s + q) ^ sw) * 16) = qiop[s];
    }
    __syncthreads();
    for (int src = 0; src < 4; ++src) {
      if (4 * hx + src >= ngroups) break;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 a = tr_operand(Wb + src * kWaveTile, 16 * ks, kq, lane);
#pragma unroll
        for (int dn = 0; dn < 2; ++dn)
          dk[dn] = mfma32(a, tr_operand(QIb + src * kWaveTile, 16 * ks, dq0 + dn, lane), dk[dn]);
      }
    }
  }
  float* dst = part_dk + (int64_t)u * kBlock * kHeadDim;
#pragma unroll
  for (int dn = 0; dn < 2; ++dn)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kq + 8 * (r >> 2) + 4 * q + (r & 3);
      dst[key * kHeadDim + 32 * (dq0 + dn) + n32] = dk[dn][r];
    }
}

// Row log-sum-exps (log2 units) of the main heads and the index scores from the partials of
// the row's visible entries, combined in slot order. -inf for a row without any.
// With main_lse (ln units, [T, G * Hpg]) the main heads' values are taken from it.
__global__ void kl_stats_fold_kernel(const int32_t* __restrict__ block_idx,
                                     const float* __restrict__ part_stats,
                                     const float* __restrict__ main_lse, float* __restrict__ lse,
                                     int64_t rows_g, int G, int Hpg, int top_k, int64_t q_begin) {
  const int H1 = Hpg + 1;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < rows_g * H1;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rg = x / H1;
    const int h = (int)(x - rg * H1);
    if (main_lse != nullptr && h < Hpg) {
      const int64_t t = q_begin + rg / G;
      const int g = (int)(rg % G);
      lse[rg * H1 + h] = main_lse[(t * G + g) * Hpg + h] * kLog2e;
      continue;
    }
    const int64_t b = (q_begin + rg / G) / kBlock;
    float m = -INFINITY;
    for (int s = 0; s < top_k; ++s) {
      const int cb = block_idx[rg * top_k + s];
      if (cb < 0 || cb > b) continue;
      m = fmaxf(m, part_stats[((rg * top_k + s) * H1 + h) * 2]);
    }
    float l = 0.f;
    for (int s = 0; s < top_k; ++s) {
      const int cb = block_idx[rg * top_k + s];
      if (cb < 0 || cb > b) continue;
      const float* ps = part_stats + ((rg * top_k + s) * H1 + h) * 2;
      l += ps[1] * exp2f(ps[0] - m);
    }
    lse[rg * H1 + h] = l > 0.f ? m + log2f(l) : -INFINITY;
  }
}

// A row's loss and dq_idx: its visible entries' partials summed in slot order (32 threads
// per row, 4 gradient values each).
__global__ void kl_grad_fold_kernel(const int32_t* __restrict__ block_idx,
                                    const float* __restrict__ part_loss,
                                    const float* __restrict__ part_dq, float* __restrict__ loss,
                                    float* __restrict__ dq, int64_t rows_g, int G, int top_k,
                                    int64_t q_begin) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < rows_g * 32;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rg = x >> 5;
    const int j = (int)(x & 31);
    const int64_t b = (q_begin + rg / G) / kBlock;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float ls = 0.f;
    // every slot's partial is loaded (four slots in flight) and the invisible ones, never
    // written, are dropped by a select rather than skipped by a branch
#pragma unroll 4
    for (int s = 0; s < top_k; ++s) {
      const int cb = block_idx[rg * top_k + s];
      const bool vis = cb >= 0 && cb <= b;
      const int64_t e = rg * top_k + s;
      const f32x4 x = *reinterpret_cast<const f32x4*>(part_dq + e * kHeadDim + 4 * j);
      const float xl = part_loss[e];
      acc = vis ? acc + x : acc;
      ls = vis ? ls + xl : ls;
    }
    *reinterpret_cast<f32x4*>(dq + rg * kHeadDim + 4 * j) = acc;
    if (j == 0) loss[rg] = ls;
  }
}

// dk_idx[key] += the key's block partials over groups, then units, in order.
__global__ void kl_dk_fold_kernel(const int32_t* __restrict__ unit_off,
                                  const float* __restrict__ part_dk, float* __restrict__ dk,
                                  int nblk, int G, int64_t seq_len) {
  const int64_t total = (int64_t)nblk * kBlock * 32;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(x / (kBlock * 32));
    const int j = (int)((x >> 5) & (kBlock - 1));
    const int v = (int)(x & 31);
    const int64_t key = (int64_t)c * kBlock + j;
    if (key >= seq_len) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bool any = false;
    for (int g = 0; g < G; ++g) {
      const int64_t kb = (int64_t)g * nblk + c;
      const int32_t u0 = unit_off[kb], u1 = unit_off[kb + 1];
      any = any || u1 > u0;
      // the bucket's units in groups of four (four partial rows in flight), summed in order
      int32_t uu = u0;
      for (; uu + 4 <= u1; uu += 4) {
        f32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[i] = *reinterpret_cast<const f32x4*>(
              part_dk + ((int64_t)(uu + i) * kBlock + j) * kHeadDim + 4 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += x[i];
      }
      for (; uu < u1; ++uu)
        acc += *reinterpret_cast<const f32x4*>(part_dk + ((int64_t)uu * kBlock + j) * kHeadDim + 4 * v);
    }
    if (any) {
      f32x4* d = reinterpret_cast<f32x4*>(dk + key * kHeadDim + 4 * v);
      *d = *d + acc;
    }
  }
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t kl_max_units(int64_t n_entries, int64_t nb) { return (n_entries + kUnit - 1) / kUnit + nb; }

size_t kl_workspace_bytes(int64_t q_count, int G, int Hpg, int top_k, int nblk) {
  const int64_t nb = (int64_t)G * nblk;
  const int64_t E = q_count * G * top_k;
  const int64_t U = kl_max_units(E, nb);
  return al256((size_t)nb * kStripes * 4) * 2 + al256((size_t)(nb + 1) * 4) * 2 +
         al256((size_t)E * 4) + al256((size_t)U * 4) + al256((size_t)E * (Hpg + 1) * 2 * 4) +
         al256((size_t)q_count * G * (Hpg + 1) * 4) + al256((size_t)E * 4) +
         al256((size_t)E * kHeadDim * 4) + al256((size_t)U * kBlock * kHeadDim * 4);
}

hipError_t launch_index_kl_prefill(const void* q, const void* k, const void* q_idx,
                                   const void* k_idx, const int32_t* block_idx,
                                   const float* main_lse, float index_scale,
                                   float* loss, float* dq_idx, float* dk_idx, void* workspace,
                                   int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count,
                                   int64_t seq_len, int nblk, hipStream_t st) {
  const int64_t nb = (int64_t)G * nblk;
  const int64_t E = q_count * G * top_k;
  const int64_t U = kl_max_units(E, nb);
  char* w = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) {
    char* p = w;
    w += al256(bytes);
    return p;
  };
  int32_t* count = reinterpret_cast<int32_t*>(take((size_t)nb * kStripes * 4));
  int32_t* cursor = reinterpret_cast<int32_t*>(take((size_t)nb * kStripes * 4));
  int32_t* offset = reinterpret_cast<int32_t*>(take((size_t)(nb + 1) * 4));
  int32_t* unit_off = reinterpret_cast<int32_t*>(take((size_t)(nb + 1) * 4));
  int32_t* sorted = reinterpret_cast<int32_t*>(take((size_t)E * 4));
  int32_t* unit_bucket = reinterpret_cast<int32_t*>(take((size_t)U * 4));
  float* part_stats = reinterpret_cast<float*>(take((size_t)E * (Hpg + 1) * 2 * 4));
  float* lse = reinterpret_cast<float*>(take((size_t)q_count * G * (Hpg + 1) * 4));
  float* part_loss = reinterpret_cast<float*>(take((size_t)E * 4));
  float* part_dq = reinterpret_cast<float*>(take((size_t)E * kHeadDim * 4));
  float* part_dk = reinterpret_cast<float*>(take((size_t)U * kBlock * kHeadDim * 4));

  launch_reverse_index(block_idx, E, G, top_k, q_begin, nblk, nullptr, 1, count, cursor, offset,
                       sorted, st);
  const unsigned grid_b = (unsigned)std::min<int64_t>((nb + 255) / 256, 65536);
  hipLaunchKernelGGL(kl_unit_count_kernel, dim3(grid_b), dim3(256), 0, st, offset, nb, unit_off);
  launch_exclusive_scan(unit_off, nb, st);
  hipLaunchKernelGGL(kl_unit_fill_kernel, dim3(grid_b), dim3(256), 0, st, unit_off, nb,
                     unit_bucket);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* QI = static_cast<const uint16_t*>(q_idx);
  const uint16_t* KI = static_cast<const uint16_t*>(k_idx);
  if (main_lse != nullptr)
    hipLaunchKernelGGL((kl_stats_unit_kernel<true>), dim3((unsigned)U), dim3(256), 0, st, Q, K,
                       QI, KI, sorted, offset, unit_off, unit_bucket, nb, nblk, G, Hpg, top_k,
                       q_begin, seq_len, index_scale, part_stats);
  else
    hipLaunchKernelGGL((kl_stats_unit_kernel<false>), dim3((unsigned)U), dim3(256), 0, st, Q, K,
                       QI, KI, sorted, offset, unit_off, unit_bucket, nb, nblk, G, Hpg, top_k,
                       q_begin, seq_len, index_scale, part_stats);
  const int64_t rows_g = q_count * G;
  const unsigned grid_s = (unsigned)std::min<int64_t>((rows_g * (Hpg + 1) + 255) / 256, 65536);
  hipLaunchKernelGGL(kl_stats_fold_kernel, dim3(grid_s), dim3(256), 0, st, block_idx, part_stats,
                     main_lse, lse, rows_g, G, Hpg, top_k, q_begin);
  hipLaunchKernelGGL(kl_grad_unit_kernel, dim3((unsigned)U), dim3(512), 0, st, Q, K, QI, KI,
                     sorted, offset, unit_off, unit_bucket, nb, nblk, G, Hpg, top_k, q_begin,
                     seq_len, index_scale, lse, part_loss, part_dq, part_dk);
  const unsigned grid_g = (unsigned)std::min<int64_t>((rows_g * 32 + 255) / 256, 65536);
  hipLaunchKernelGGL(kl_grad_fold_kernel, dim3(grid_g), dim3(256), 0, st, block_idx, part_loss,
                     part_dq, loss, dq_idx, rows_g, G, top_k, q_begin);
  const unsigned grid_k = (unsigned)std::min<int64_t>(((int64_t)nblk * kBlock * 32 + 255) / 256, 65536);
  hipLaunchKernelGGL(kl_dk_fold_kernel, dim3(grid_k), dim3(256), 0, st, unit_off, part_dk,
                     dk_idx, nblk, G, seq_len);
  return hipGetLastError();
}

}  // namespace msa
