// Main branch of MSA, one wave per (query, group [, split]): exact softmax attention of
// the group's query heads over the keys of a list of 128-token blocks (mlqm.cn blog,
// section 2.2: gather the kept K/V blocks, then flash attention; all heads of a GQA
// group share one selection, so one pass over the blocks serves every head).
//
// Per block: S^T = K . Q^T on 16x16 MFMAs (K operands straight from global memory,
// 16 B per lane; the <= 16 heads of the group are the 16 MFMA columns), an online
// softmax per head across blocks (running max in log2 units, running sum), then
// O += P . V on the vector ALUs: P goes to LDS once and is read back as broadcasts,
// and each lane owns two of the 128 output dims, so every V row is one coalesced
// 256-byte read by the wave.
//
// Modes: prefill over block_idx (query-centric path), prefill over all visible
// blocks (dense reference), decode split-K over block_idx or over the whole cache;
// decode writes unnormalised partials that decode_combine_kernel merges in a fixed
// split order.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

template <class E>
struct KOp;
template <>
struct KOp<BF16> {
  typedef u32x4 type;
  static constexpr int kStep = 32;  // dims per 16x16x32 MFMA
  static __device__ __forceinline__ type load(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ type zero() { return u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ float2 load2(const uint16_t* p) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(bf16_bits_to_f32(w & 0xffffu), bf16_bits_to_f32(w >> 16));
  }
  static __device__ __forceinline__ void store2(uint16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  }
};
template <>
struct KOp<F32> {
  typedef float type;
  static constexpr int kStep = 4;  // dims per 16x16x4 fp32 MFMA
  static __device__ __forceinline__ type load(const float* p) { return *p; }
  static __device__ __forceinline__ type zero() { return 0.f; }
  static __device__ __forceinline__ float2 load2(const float* p) {
    return *reinterpret_cast<const float2*>(p);
  }
  static __device__ __forceinline__ void store2(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

constexpr int kPRow = kBlock + 4;  // LDS row stride of P (floats)

template <class E, int HMAX>
__global__ __launch_bounds__(64) void gather_attn_kernel(GatherParams p) {
  typedef typename E::elem elem;
  typedef KOp<E> O;
  constexpr int kNStep = kHeadDim / O::kStep;
  __shared__ __align__(16) float Ps[16 * kPRow];
  __shared__ float alpha_s[16];
  __shared__ float lsum_s[16];

  const int lane = threadIdx.x;
  const int hcol = lane & 15;   // head of this lane in the S^T tiles
  const int kgrp = lane >> 4;   // k-group of this lane in the MFMA operands
  const int Hpg = p.Hpg;
  const int Hq = p.G * Hpg;
  const int64_t u = blockIdx.x;
  const bool decode = p.mode >= kDecodeSparse;
  const bool sparse = p.mode == kPrefillSparse || p.mode == kDecodeSparse;

  const elem *kbase, *vbase, *qrow;
  int64_t limit;  // keys j < limit are visible
  int jbeg, jend; // range of list positions (sparse) or block ids (dense)
  int koff = 0, kspan = kBlock;  // keys [koff, koff + kspan) of each block
  const int32_t* list = nullptr;
  int64_t bseq = 0, i = 0;
  int g;
  int sp = 0;
  if (!decode) {
    i = u / p.G;
    g = (int)(u % p.G);
    const int64_t t = p.q_begin + i;
    limit = t + 1;
    kbase = (const elem*)p.k + (int64_t)g * p.seq_len * kHeadDim;
    vbase = (const elem*)p.v + (int64_t)g * p.seq_len * kHeadDim;
    qrow = (const elem*)p.q + (t * Hq + (int64_t)g * Hpg) * kHeadDim;
    if (sparse) {
      list = p.block_idx + (i * p.G + g) * p.top_k;
      jbeg = 0;
      jend = p.top_k;
    } else {
      jbeg = 0;
      jend = (int)(t / kBlock) + 1;
    }
  } else {
    const int64_t bg = u / p.nsplit;
    sp = (int)(u % p.nsplit);
    bseq = bg / p.G;
    g = (int)(bg % p.G);
    int64_t L = p.seq_lens[bseq];
    L = L < 1 ? 1 : (L > p.max_len ? p.max_len : L);
    limit = L;
    kbase = (const elem*)p.k + bg * p.max_len * kHeadDim;
    vbase = (const elem*)p.v + bg * p.max_len * kHeadDim;
    qrow = (const elem*)p.q + (bseq * Hq + (int64_t)g * Hpg) * kHeadDim;
    const int nlist = sparse ? p.top_k : (int)((L - 1) / kBlock) + 1;
    if (sparse) list = p.block_idx + bg * p.top_k;
    if (p.half_blocks) {
      jbeg = sp >> 1;
      jend = min(jbeg + 1, nlist);
      koff = (sp & 1) * (kBlock / 2);
      kspan = kBlock / 2;
    } else {
      jbeg = sp * p.blocks_per_split;
      jend = min(jbeg + p.blocks_per_split, nlist);
    }
  }
  const int blocal = (int)((limit - 1) / kBlock);
  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);

  typename O::type qop[kNStep];
  {
    const bool ok = hcol < Hpg;
    const elem* qp = qrow + (ok ? hcol : 0) * kHeadDim + kgrp * E::kPerLane;
#pragma unroll
    for (int s = 0; s < kNStep; ++s) qop[s] = ok ? O::load(qp + s * O::kStep) : O::zero();
  }

  float acc[HMAX][2];
#pragma unroll
  for (int h = 0; h < HMAX; ++h) acc[h][0] = acc[h][1] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int jj = jbeg; jj < jend; ++jj) {
    const int c = list ? list[jj] : jj;
    if (c < 0 || c > blocal) continue;
    const int64_t key0 = (int64_t)c * kBlock + koff;
    const int nvalid = (int)min((int64_t)kspan, limit - key0);
    if (nvalid <= 0) continue;
    // rows koff .. of block c: contiguous caches, or the block's page (decode)
    const elem* kblk = kbase + key0 * kHeadDim;
    const elem* vblk = vbase + key0 * kHeadDim;
    if (decode && p.pages.table != nullptr) {
      const int64_t in_page = ((int64_t)g * kBlock + koff) * kHeadDim;
      kblk = p.pages.block((const elem*)p.k, kbase, bseq, c, (int64_t)kBlock * kHeadDim) + in_page;
      vblk = p.pages.block((const elem*)p.v, vbase, bseq, c, (int64_t)kBlock * kHeadDim) + in_page;
    }

    // Half-block (64-key) bf16 units issue their V rows together with the K rows, so
    // the wave pays one memory round trip for both.
    constexpr bool kPreV = E::is_bf16;
    uint32_t vpre[kPreV ? 64 : 1];
    if constexpr (kPreV) {
      if (kspan == 64) {
        const elem* vp0 = vblk + 2 * lane;
        // unconditional loads (rows past the valid keys read row 0, then zeroed), so that
        // no load sits behind a branch and waits alone
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vp0 + (int64_t)(j < nvalid ? j : 0) * kHeadDim);
          vpre[j] = j < nvalid ? w : 0u;
        }
      }
    }
    // S^T = K . Q^T for the 16-key tiles (8 per block, 4 per half block).
    f32x4 s4[8];
    const int ntiles = kspan / 16;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      if (kt < ntiles) {
        const int kk = 16 * kt + hcol;
        const bool ok = kk < nvalid;
        const elem* kp = kblk + (ok ? kk : 0) * kHeadDim + kgrp * E::kPerLane;
#pragma unroll
        for (int s = 0; s < kNStep; ++s) {
          const typename O::type w = O::load(kp + s * O::kStep);
          a = mfma16(ok ? w : O::zero(), qop[s], a);
        }
      }
      s4[kt] = a;
    }
    // Scale, mask, block max per head.
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kt + 4 * kgrp + r;
        const float x = kk < nvalid ? s4[kt][r] * qk_scale : -INFINITY;
        s4[kt][r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = wave_max_xor(mloc, 16);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 pv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = m_new == -INFINITY ? 0.f : fast_exp2(s4[kt][r] - m_new);
        pv[r] = e;
        psum += e;
      }
      *reinterpret_cast<f32x4*>(&Ps[hcol * kPRow + 16 * kt + 4 * kgrp]) = pv;
    }
    psum = wave_sum_xor(psum, 16);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (lane < 16) alpha_s[lane] = alpha;
    __syncthreads();

    // O = O * alpha + P . V ; this lane owns dims 2*lane, 2*lane + 1.
#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
      const float a = alpha_s[h];
      acc[h][0] *= a;
      acc[h][1] *= a;
    }
    if (kPreV && kspan == 64) {
#pragma unroll
      for (int j4 = 0; j4 < 64; j4 += 4) {
        float2 vv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          vv[q] = make_float2(bf16_bits_to_f32(vpre[j4 + q] & 0xffffu), bf16_bits_to_f32(vpre[j4 + q] >> 16));
#pragma unroll
        for (int h = 0; h < HMAX; ++h) {
          if (h < Hpg) {
            const f32x4 pp = *reinterpret_cast<const f32x4*>(&Ps[h * kPRow + j4]);
            acc[h][0] += pp[0] * vv[0].x + pp[1] * vv[1].x + pp[2] * vv[2].x + pp[3] * vv[3].x;
            acc[h][1] += pp[0] * vv[0].y + pp[1] * vv[1].y + pp[2] * vv[2].y + pp[3] * vv[3].y;
          }
        }
      }
    } else {
      const elem* vp = vblk + 2 * lane;
      // V rows in batches of 16 so that many loads are in flight per wave.
      for (int j0 = 0; j0 < nvalid; j0 += 16) {
        float2 vv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          vv[q] = (j0 + q < nvalid) ? O::load2(vp + (int64_t)(j0 + q) * kHeadDim) : make_float2(0.f, 0.f);
#pragma unroll
        for (int q4 = 0; q4 < 16; q4 += 4) {
#pragma unroll
          for (int h = 0; h < HMAX; ++h) {
            if (h < Hpg) {
              const f32x4 pp = *reinterpret_cast<const f32x4*>(&Ps[h * kPRow + j0 + q4]);
              acc[h][0] += pp[0] * vv[q4].x + pp[1] * vv[q4 + 1].x + pp[2] * vv[q4 + 2].x + pp[3] * vv[q4 + 3].x;
              acc[h][1] += pp[0] * vv[q4].y + pp[1] * vv[q4 + 1].y + pp[2] * vv[q4 + 2].y + pp[3] * vv[q4 + 3].y;
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if (!decode) {
    if (lane < 16) lsum_s[lane] = l_run;
    // lanes h < 16 hold head h's running maximum (log2 units) and sum
    if (sparse && p.lse != nullptr && lane < Hpg)
      p.lse[(p.q_begin + i) * Hq + (int64_t)g * Hpg + lane] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    __syncthreads();
    elem* orow = (elem*)p.out + ((p.q_begin + i) * Hq + (int64_t)g * Hpg) * kHeadDim + 2 * lane;
#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
      if (h < Hpg) {
        const float inv = 1.f / lsum_s[h];
        O::store2(orow + h * kHeadDim, acc[h][0] * inv, acc[h][1] * inv);
      }
    }
  } else {
    float* po = p.part_o + (u * Hpg) * kHeadDim + 2 * lane;
#pragma unroll
    for (int h = 0; h < HMAX; ++h)
      if (h < Hpg) *reinterpret_cast<float2*>(po + h * kHeadDim) = make_float2(acc[h][0], acc[h][1]);
    if (lane < Hpg) {
      p.part_ml[(u * Hpg + lane) * 2 + 0] = m_run;
      p.part_ml[(u * Hpg + lane) * 2 + 1] = l_run;
    }
  }
}

// One wave per (sequence, head). Lanes hold the (m, l) of 64 splits at a time (all
// loaded at once): pass 1 reduces the global max, pass 2 forms each split's weight in
// its lane and broadcasts it while every lane streams its two dims of the partials (up to
// 32 splits: all partials requested up front instead). The
// order of the sum is fixed, so the result is deterministic.
template <class E>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            typename E::elem* __restrict__ out,
                                                            int Hpg, int nsplit) {
  const int lane = threadIdx.x;
  const int64_t bg = blockIdx.x / Hpg;
  const int h = blockIdx.x % Hpg;
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  constexpr int kFew = 32;
  if (nsplit <= kFew) {
    // up to 32 splits (top_k <= 16): every partial and every (m, l) is requested at once,
    // so the wave waits for memory once
    float2 o[kFew];
#pragma unroll
    for (int k = 0; k < kFew; ++k)
      o[k] = k < nsplit ? *reinterpret_cast<const float2*>(
                              part_o + ((bg * nsplit + k) * Hpg + h) * kHeadDim + 2 * lane)
                        : make_float2(0.f, 0.f);
    const float2 v = lane < nsplit ? ml[(bg * nsplit + lane) * Hpg + h] : make_float2(-INFINITY, 0.f);
    const float Mf = wave_max_xor(v.x, 1);
    const float w = v.x == -INFINITY ? 0.f : fast_exp2(v.x - Mf);
    const float Lf = wave_sum_xor(w * v.y, 1);
    float b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int k = 0; k < kFew; ++k) {
      if (k < nsplit) {
        const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
        b0 += wk * o[k].x;
        b1 += wk * o[k].y;
      }
    }
    const float invf = Lf > 0.f ? 1.f / Lf : 0.f;
    KOp<E>::store2(out + (bg * Hpg + h) * kHeadDim + 2 * lane, b0 * invf, b1 * invf);
    return;
  }
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int sp = s0 + lane;
    if (sp < nsplit) M = fmaxf(M, ml[(bg * nsplit + sp) * Hpg + h].x);
  }
  M = wave_max_xor(M, 1);
  float a0 = 0.f, a1 = 0.f, L = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int sp = s0 + lane;
    float w = 0.f, l = 0.f;
    if (sp < nsplit) {
      const float2 v = ml[(bg * nsplit + sp) * Hpg + h];
      w = (v.x == -INFINITY) ? 0.f : fast_exp2(v.x - M);
      l = v.y;
    }
    L += wave_sum_xor(w * l, 1);
    const int cnt = min(64, nsplit - s0);
    // 32 partials requested at a time (one wait per 32, not one per partial)
    for (int k0 = 0; k0 < cnt; k0 += kFew) {
      float2 o[kFew];
#pragma unroll
      for (int k = 0; k < kFew; ++k)
        o[k] = k0 + k < cnt ? *reinterpret_cast<const float2*>(
                                  part_o + ((bg * nsplit + s0 + k0 + k) * Hpg + h) * kHeadDim +
                                  2 * lane)
                            : make_float2(0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kFew; ++k) {
        if (k0 + k < cnt) {
          const float wk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k0 + k));
          a0 += wk * o[k].x;
          a1 += wk * o[k].y;
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  KOp<E>::store2(out + (bg * Hpg + h) * kHeadDim + 2 * lane, a0 * inv, a1 * inv);
}

template <class E>
static hipError_t launch_gather_t(const GatherParams& p, hipStream_t st) {
  int64_t units;
  if (p.mode == kPrefillSparse || p.mode == kPrefillDense)
    units = p.q_count * p.G;
  else
    units = (int64_t)p.B * p.G * p.nsplit;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)units);
  if (p.Hpg <= 4)
    hipLaunchKernelGGL((gather_attn_kernel<E, 4>), grid, dim3(64), 0, st, p);
  else if (p.Hpg <= 8)
    hipLaunchKernelGGL((gather_attn_kernel<E, 8>), grid, dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((gather_attn_kernel<E, 16>), grid, dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gather_attn(const GatherParams& p, hipStream_t stream) {
  return p.bf16 ? launch_gather_t<BF16>(p, stream) : launch_gather_t<F32>(p, stream);
}

hipError_t launch_decode_combine(int bf16, const float* part_o, const float* part_ml, void* out,
                                 int B, int G, int Hpg, int nsplit, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)B * G * Hpg);
  if (bf16)
    hipLaunchKernelGGL(decode_combine_kernel<BF16>, dim3(grid), dim3(64), 0, stream, part_o,
                       part_ml, (uint16_t*)out, Hpg, nsplit);
  else
    hipLaunchKernelGGL(decode_combine_kernel<F32>, dim3(grid), dim3(64), 0, stream, part_o,
                       part_ml, (float*)out, Hpg, nsplit);
  return hipGetLastError();
}

}  // namespace msa
