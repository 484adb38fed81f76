// Main branch of MSA for decode, bf16: exact softmax attention of one token's query heads
// over the kept blocks of its sequence (the blocks the index branch selected for the
// token's group), split by block so the blocks of a sequence are read in parallel.
//
// One workgroup of four waves per (sequence, group, kept block); wave w takes keys
// 32 w .. 32 w + 31 of the block. Each wave stages its 32 K rows (row swizzle) and V rows
// (V swizzle) in LDS by direct global->LDS loads and runs the same products as the prefill
// tile kernels on 32x32x16 bf16 MFMAs, with the group's query heads as the MFMA columns
// (Hpg <= 16 of 32, the rest read a valid head and are never stored):
//   S^T = K . Q^T (32 keys x 32 columns), softmax statistics over the wave's keys,
//   O^T += V^T . P^T (128 dims x 32 columns) with V read through the LDS transpose read.
// The four waves' (max, sum, output) are merged in LDS into the block's partial, which the
// decode combine then merges over the kept blocks in slot order (fixed order: the result is
// bit-identical from run to run).
#include "msa_device.h"
#include "msa_launch.h"
#include "msa_select.h"
#include "msa_tile.h"

namespace msa {

static_assert(kSelectMaxBlocks == kRowMax, "the host's row limit is the selection's");

// Rows row0 .. row0 + 31 of a block (rows at or past nvalid repeat row nvalid - 1, which
// the caller masks) into a 32-row LDS buffer: load i covers buffer rows 4 i .. 4 i + 3, a
// quarter-wave per row; chunk x of buffer row r at position x ^ (r % 16) (row swizzle) or
// x ^ v_swz(r) (V swizzle).
template <bool kVSwz>
__device__ __forceinline__ void rows32_dma(const uint16_t* blk, int row0, int nvalid,
                                           uint8_t* buf, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ (kVSwz ? v_swz(r) : (r & 15));
    const int rr = min(row0 + r, nvalid - 1);
    __builtin_amdgcn_global_load_lds((const void*)(blk + rr * kHeadDim + chunk * 8),
                                     (__attribute__((address_space(3))) void*)(buf + i * 1024),
                                     16, 0, kLoadOnce);
  }
}

// kSelect: the workgroup first selects its (sequence, group)'s blocks from the block scores
// itself (row_select_wg, the code of the decode top-k kernel: the same ids), takes the one
// of its slot and writes it to block_idx; otherwise it reads its block from block_idx.
template <bool kSelect>
__global__ __launch_bounds__(256, 2) void decode_attn_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ block_idx,
    const float* __restrict__ block_scores, int32_t* __restrict__ idx_out, int nblk,
    const int32_t* __restrict__ seq_lens, int64_t max_len, int G, int Hpg, int top_k,
    PageMap pm, float* __restrict__ part_o, float* __restrict__ part_ml) {
  // staging: per wave 8 KiB of K then 8 KiB of V; reused for the merge (4 x 16 KiB) and,
  // before the staging, for the selection's candidates
  __shared__ __align__(16) uint8_t lds[4 * 2 * 32 * 256];
  __shared__ float2 mls[4][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.x;        // (bg, slot j): one partial
  const int64_t bg = u / top_k;        // sequence * G + group
  const int64_t bseq = bg / G;
  const int g = (int)(bg - bseq * G);
  int64_t L = seq_lens[bseq];
  L = L < 1 ? 1 : (L > max_len ? max_len : L);
  const int blocal = (int)((L - 1) / kBlock);
  // B operand of S^T: column n = head n of the group (columns >= Hpg read head Hpg - 1);
  // loaded first, so that the loads run under the selection or the block id's load
  const int n32 = lane & 31, q = lane >> 5;
  const int Hq = G * Hpg;
  const uint16_t* qrow = Q + (bseq * Hq + (int64_t)g * Hpg + min(n32, Hpg - 1)) * kHeadDim;
  u32x4 qop[kHeadDim / 16];
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s)
    qop[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * q);
  int c;
  if constexpr (kSelect) {
    static_assert(sizeof(lds) >= kRowMax * sizeof(uint64_t), "candidates must fit the staging");
    __shared__ RowSelectShared sh;
    const int j = (int)(u - bg * top_k);
    if (blocal + 1 <= top_k) {  // every visible block is kept
      c = j <= blocal ? j : -1;
    } else if (j == top_k - 1) {  // the local block is the largest kept id
      c = blocal;
    } else {
      const int Ksel = top_k - 1;
      row_select_wg(block_scores + bg * nblk, (nblk & 3) == 0, blocal, Ksel,
                    reinterpret_cast<uint64_t*>(lds), sh, tid);
      if (tid < Ksel) {
        const int cc = sh.sel[tid];
        if (sel_rank(sh.sel, Ksel, cc) == j) sh.slot_id = cc;
      }
      __syncthreads();  // also: every candidate read is done before the staging reuses lds
      c = sh.slot_id;
    }
    if (tid == 0) idx_out[u] = c;
  } else {
    c = block_idx[u];
  }
  float* po = part_o + u * Hpg * kHeadDim;
  if (c < 0 || c > blocal) {  // padding or an invisible id: an empty partial
    for (int x = tid; x < Hpg * kHeadDim; x += 256) po[x] = 0.f;
    if (tid < Hpg)
      reinterpret_cast<float2*>(part_ml)[u * Hpg + tid] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int64_t key0 = (int64_t)c * kBlock;
  const int nvalid = (int)min((int64_t)kBlock, L - key0);
  const int64_t bstride = (int64_t)kBlock * kHeadDim;
  const uint16_t* kblk = K + (bg * max_len + key0) * kHeadDim;
  const uint16_t* vblk = V + (bg * max_len + key0) * kHeadDim;
  if (pm.table != nullptr) {  // the block's page; group g's rows inside it
    kblk = pm.block(K, K, bseq, c, bstride) + (int64_t)g * bstride;
    vblk = pm.block(V, V, bseq, c, bstride) + (int64_t)g * bstride;
  }
  uint8_t* Kw = lds + wave * 2 * 32 * 256;
  uint8_t* Vw = Kw + 32 * 256;
  rows32_dma<false>(kblk, 32 * wave, nvalid, Kw, lane);
  rows32_dma<true>(vblk, 32 * wave, nvalid, Vw, lane);

  MSA_WAIT_VMCNT(0);
  __builtin_amdgcn_wave_barrier();  // this wave's rows have landed (only this wave reads them)

  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const f32x16 sv = s_tile_swz(Kw, n32, qop, q);
  // lane (column n, half q) holds keys 32 w + 8 (r / 4) + 4 q + r % 4
  const int lim = nvalid - 1 - 32 * wave - 4 * q;
  float p[16];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = 8 * (r >> 2) + (r & 3) <= lim ? sv[r] : -INFINITY;
    mx = fmaxf(mx, p[r]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_w = mx * qk_scale;  // -inf when none of the wave's keys is valid
  const float mneg = m_w == -INFINITY ? 0.f : -m_w;
  float l_w = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = fast_exp2(fmaf(p[r], qk_scale, mneg));
    l_w += p[r];
  }
  l_w += __shfl_xor(l_w, 32, 64);
  f32x16 o[4] = {};
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const float* pr = p + 8 * uu;
    const u32x4 pb = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                           pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(tr_operand(Vw, 16 * uu, dt, lane), pb, o[dt]);
  }

  // merge the four waves: wave w then combines dims 32 w .. 32 w + 31 of every column
  __syncthreads();  // every wave is done with the staged rows
  float* ob = reinterpret_cast<float*>(lds);  // [wave][dt][r][lane]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ob[((wave * 4 + dt) * 16 + r) * 64 + lane] = o[dt][r];
  if (q == 0) mls[wave][n32] = make_float2(m_w, l_w);
  __syncthreads();
  float2 st[4];
  float M = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    st[w2] = mls[w2][n32];
    M = fmaxf(M, st[w2].x);
  }
  float wt[4], Lsum = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    wt[w2] = st[w2].x == -INFINITY ? 0.f : fast_exp2(st[w2].x - M);
    Lsum += wt[w2] * st[w2].y;
  }
  const int dt = wave;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float a = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) a = fmaf(wt[w2], ob[((w2 * 4 + dt) * 16 + r) * 64 + lane], a);
    acc[r] = a;
  }
  if (n32 < Hpg) {
    // column n32 = head, dims 32 dt + 8 (r / 4) + 4 q + r % 4
    float* dst = po + n32 * kHeadDim + 32 * dt + 4 * q;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      *reinterpret_cast<f32x4*>(dst + 8 * rr) =
          f32x4{acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
    if (wave == 0 && q == 0)
      reinterpret_cast<float2*>(part_ml)[u * Hpg + n32] = make_float2(M, Lsum);
  }
}

// ------------------------------------------------------------------------------------
// Dense decode, bf16 (the whole-cache baseline the pages compare MSA against: dense GQA
// attention with the same heads, researchpapers.dev summary, "Key results").
// One wave per (sequence, group, split of the cache): the wave streams its keys in steps of
// 32 through a private ring of kDenseRing LDS stages (K rows in the row swizzle, V rows in
// the V swizzle, 16 KiB a stage) filled by direct global->LDS loads, with kDenseRing - 1
// stages in flight while one is consumed, and keeps an online softmax (running maximum,
// rescaled sum and output) over its keys. The partials go to the same fixed-order combine
// as the sparse decode.
constexpr int kDenseRing = 3;
constexpr int kDenseStage = 2 * 32 * 256;

// Rows row0 .. row0 + 31 of one (sequence, group) cache into a 32-row LDS buffer (rows at or
// past `len` repeat row len - 1, which the caller masks); chunk x of buffer row r at position
// x ^ (r % 16) (row swizzle) or x ^ v_swz(r) (V swizzle).
template <bool kVSwz>
__device__ __forceinline__ void rows32_dma_seq(const uint16_t* base, int64_t row0, int64_t len,
                                               uint8_t* buf, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ (kVSwz ? v_swz(r) : (r & 15));
    const int64_t rr = min(row0 + r, len - 1);
    __builtin_amdgcn_global_load_lds((const void*)(base + rr * kHeadDim + chunk * 8),
                                     (__attribute__((address_space(3))) void*)(buf + i * 1024),
                                     16, 0, kLoadOnce);
  }
}

__global__ __launch_bounds__(64) void decode_dense_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ seq_lens, int64_t max_len,
    int G, int Hpg, int nsplit, int64_t keys_per_split, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  __shared__ __align__(16) uint8_t lds[kDenseRing][kDenseStage];
  const int lane = threadIdx.x;
  const int64_t u = blockIdx.x;  // (sequence * G + group, split): one partial
  const int64_t bg = u / nsplit;
  const int64_t split = u - bg * nsplit;
  const int64_t bseq = bg / G;
  const int g = (int)(bg - bseq * G);
  int64_t L = seq_lens[bseq];
  L = L < 1 ? 1 : (L > max_len ? max_len : L);
  const int64_t k_begin = split * keys_per_split;
  const int64_t k_end = min(k_begin + keys_per_split, L);
  float* po = part_o + u * Hpg * kHeadDim;
  if (k_begin >= k_end) {  // a split past the sequence's end: an empty partial
    for (int x = lane; x < Hpg * kHeadDim; x += 64) po[x] = 0.f;
    if (lane < Hpg)
      reinterpret_cast<float2*>(part_ml)[u * Hpg + lane] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int nsteps = (int)((k_end - k_begin + 31) / 32);
  const uint16_t* kb = K + bg * max_len * kHeadDim;
  const uint16_t* vb = V + bg * max_len * kHeadDim;
  auto issue = [&](int st) {
    uint8_t* buf = lds[st % kDenseRing];
    rows32_dma_seq<false>(kb, k_begin + 32 * st, L, buf, lane);
    rows32_dma_seq<true>(vb, k_begin + 32 * st, L, buf + 32 * 256, lane);
  };
  for (int st = 0; st < kDenseRing - 1 && st < nsteps; ++st) issue(st);

  // B operand of S^T: column n = head n of the group (columns >= Hpg read head Hpg - 1)
  const int n32 = lane & 31, q = lane >> 5;
  const int Hq = G * Hpg;
  const uint16_t* qrow = Q + (bseq * Hq + (int64_t)g * Hpg + min(n32, Hpg - 1)) * kHeadDim;
  u32x4 qop[kHeadDim / 16];
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s)
    qop[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * q);

  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  float m_run = -INFINITY;  // running maximum of this lane's column, log2 units
  float l_run = 0.f;
  f32x16 o[4] = {};
  for (int st = 0; st < nsteps; ++st) {
    if (st + kDenseRing - 1 < nsteps) issue(st + kDenseRing - 1);
    // 16 loads per stage; wait until only the stages issued after this one remain
    const int later = min(kDenseRing - 1, nsteps - 1 - st);
    if (later >= 2) MSA_WAIT_VMCNT(32);
    else if (later == 1) MSA_WAIT_VMCNT(16);
    else MSA_WAIT_VMCNT(0);
    __builtin_amdgcn_wave_barrier();
    const uint8_t* Ks = lds[st % kDenseRing];
    const uint8_t* Vs = Ks + 32 * 256;
    const f32x16 sv = s_tile_swz(Ks, n32, qop, q);
    // lane (column n, half q) holds keys 8 (r / 4) + 4 q + r % 4 of the step
    const int64_t key0 = k_begin + 32 * (int64_t)st;
    const int lim = (int)min((int64_t)31, k_end - 1 - key0) - 4 * q;
    float p[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = 8 * (r >> 2) + (r & 3) <= lim ? sv[r] : -INFINITY;
      mx = fmaxf(mx, p[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // every step holds a visible key, so the new maximum is finite
    const float m_new = fmaxf(m_run, mx * qk_scale);
    const float alpha = fast_exp2(m_run - m_new);  // 0 on the first step
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(p[r], qk_scale, -m_new));
      ls += p[r];
    }
    ls += __shfl_xor(ls, 32, 64);
    l_run = fmaf(l_run, alpha, ls);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const float* pr = p + 8 * uu;
      const u32x4 pb = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                             pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(tr_operand(Vs, 16 * uu, dt, lane), pb, o[dt]);
    }
    // this stage's reads are done before it is refilled kDenseRing - 1 steps on
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  }
  if (n32 < Hpg) {
    // column n32 = head, dims 32 dt + 8 (r / 4) + 4 q + r % 4
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      float* dst = po + n32 * kHeadDim + 32 * dt + 4 * q;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<f32x4*>(dst + 8 * rr) =
            f32x4{o[dt][4 * rr], o[dt][4 * rr + 1], o[dt][4 * rr + 2], o[dt][4 * rr + 3]};
    }
    if (q == 0) reinterpret_cast<float2*>(part_ml)[u * Hpg + n32] = make_float2(m_run, l_run);
  }
}

void dense_decode_plan(int B, int G, int64_t max_len, int* nsplit, int64_t* keys_per_split) {
  // about six rounds of the chip's resident waves (three per CU at 48 KiB of LDS each)
  const int64_t target = 6 * 3 * 256;
  int64_t per_bg = (target + (int64_t)B * G - 1) / ((int64_t)B * G);
  if (per_bg < 1) per_bg = 1;
  int64_t kps = (max_len + per_bg - 1) / per_bg;
  kps = (kps + 31) / 32 * 32;
  *keys_per_split = kps;
  *nsplit = (int)((max_len + kps - 1) / kps);
}

hipError_t launch_decode_dense_bf16(const void* q, const void* k, const void* v,
                                    const int32_t* seq_lens, int B, int64_t max_len, int G,
                                    int Hpg, float* part_o, float* part_ml, hipStream_t st) {
  int nsplit;
  int64_t kps;
  dense_decode_plan(B, G, max_len, &nsplit, &kps);
  const int64_t units = (int64_t)B * G * nsplit;
  hipLaunchKernelGGL(decode_dense_bf16_kernel, dim3((unsigned)units), dim3(64), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, seq_lens,
                     max_len, G, Hpg, nsplit, kps, part_o, part_ml);
  return hipGetLastError();
}

hipError_t launch_decode_attn_bf16(const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, const int32_t* seq_lens, int B,
                                   int64_t max_len, int G, int Hpg, int top_k, PageMap pm,
                                   float* part_o, float* part_ml, hipStream_t st,
                                   const float* block_scores, int32_t* idx_out, int nblk) {
  const int64_t units = (int64_t)B * G * top_k;
  if (block_scores != nullptr) {
    hipLaunchKernelGGL(decode_attn_bf16_kernel<true>, dim3((unsigned)units), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, nullptr,
                       block_scores, idx_out, nblk, seq_lens, max_len, G, Hpg, top_k, pm,
                       part_o, part_ml);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_attn_bf16_kernel<false>, dim3((unsigned)units), dim3(256), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, block_idx,
                     nullptr, nullptr, 0, seq_lens, max_len, G, Hpg, top_k, pm, part_o,
                     part_ml);
  return hipGetLastError();
}

}  // namespace msa
