// Main branch of MSA for prefill, KV-centric ("reverse index") form.
//
// The researchpapers.dev summary of the MSA paper ("What it means for inference
// teams") names the real costs of a sparse prefill kernel: index construction, top-k,
// query gathering, reverse indexing and load balancing; the baguaai.com note on MSA
// describes the kernel as aggregating queries on the KV side. This file implements
// that data flow for gfx950:
//
//   1. reverse index: a counting sort of every kept (token, group, slot) entry of
//      block_idx by its KV block (group g, block c) - count, exclusive scan, scatter;
//   2. kv_attn_kernel: the sorted entries are cut into fixed tiles of 128 entries
//      (load balance independent of how popular a block is). Each tile walks its runs
//      of equal (g, c): the block's K (row-major) and V (transposed) are staged in LDS
//      once and every query of the run attends to it with 32x32x16 bf16 MFMAs,
//      rows = (entry, head) pairs gathered from Q. A row sees one block, so its softmax
//      is exact within the block; it writes a partial (o / l, m, l);
//   3. kv_merge_kernel: per (token, group) the <= top_k partials are merged with a
//      log-sum-exp combine in slot order (deterministic; no atomics touch values).
//
// MFMA orientation: S^T = K . Q^T so that a lane owns one query row and holds 16 of
// its keys per 32-key tile; the softmax reductions are in-lane plus one exchange
// with the other half-wave, and P^T in the same registers is already the B operand
// of O^T = V^T . P^T.
#include <algorithm>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kTile = 128;                 // sorted entries per workgroup
constexpr int kKRow = kHeadDim + 8;        // LDS row stride of K (elements)
constexpr int kVRow = kBlock + 4;          // LDS row stride of V^T (elements)

// ---- reverse index --------------------------------------------------------------------
__global__ void kv_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

__device__ __forceinline__ int64_t entry_bucket(const int32_t* block_idx, int64_t id, int G,
                                                int top_k, int64_t q_begin, int nblk) {
  const int c = block_idx[id];
  const int64_t rowg = id / top_k;
  const int g = (int)(rowg % G);
  const int64_t t = q_begin + rowg / G;
  if (c < 0 || (int64_t)c > t / kBlock) return -1;
  return (int64_t)g * nblk + c;
}

__global__ void kv_count_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                int top_k, int64_t q_begin, int nblk, int32_t* __restrict__ count) {
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk);
    if (k >= 0) atomicAdd(&count[k], 1);
  }
}

// Exclusive scan of count[0..n) into offset[0..n] (offset[n] = total) and cursor[0..n).
__global__ __launch_bounds__(1024) void kv_scan_kernel(const int32_t* __restrict__ count,
                                                       int64_t n, int32_t* __restrict__ offset,
                                                       int32_t* __restrict__ cursor) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = min(n, tid * per), hi = min(n, lo + per);
  int32_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += count[i];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;  // exclusive prefix of this thread's range
  for (int64_t i = lo; i < hi; ++i) {
    offset[i] = run;
    cursor[i] = run;
    run += count[i];
  }
  if (tid == 1023) offset[n] = part[1023];
}

__global__ void kv_scatter_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                  int top_k, int64_t q_begin, int nblk,
                                  int32_t* __restrict__ cursor, int32_t* __restrict__ sorted) {
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk);
    if (k >= 0) sorted[atomicAdd(&cursor[k], 1)] = (int32_t)id;
  }
}

// ---- the tile kernel ---------------------------------------------------------------------
template <class E>
struct TileOps;

template <>
struct TileOps<BF16> {
  typedef uint16_t elem;
  // Q^T operand of k-step s (16 dims): lane group q holds dims 16s + 8q .. +8.
  static constexpr int kQSteps = kHeadDim / 16;
  typedef u32x4 qop_t;
  static __device__ __forceinline__ void load_q(qop_t* op, const elem* row, int q, bool ok) {
#pragma unroll
    for (int s = 0; s < kQSteps; ++s)
      op[s] = ok ? *reinterpret_cast<const u32x4*>(row + 16 * s + 8 * q) : u32x4{0u, 0u, 0u, 0u};
  }
  // S^T tile (32 keys from `krow0`, the lane's key row in LDS)
  static __device__ __forceinline__ f32x16 s_tile(const elem* krow, const qop_t* op, int q) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kQSteps; ++s)
      acc = mfma32(*reinterpret_cast<const u32x4*>(krow + 16 * s + 8 * q), op[s], acc);
    return acc;
  }
  // P^T operands: chunk u (16 keys) = regs p[u/2][8(u%2) .. +8] of the S^T tiles as bf16,
  // packed right after the exponentials so that only 32 registers stay live.
  typedef u32x4 pop_t;
  static constexpr int kPChunks = 8;
  static __device__ __forceinline__ void pack_p(pop_t* pb, const float (&p)[4][16]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* pr = &p[u >> 1][8 * (u & 1)];
      pb[u] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                    pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    }
  }
  // O^T += V^T . P^T over the 128 keys. The A operand of chunk u holds, for lane group q,
  // keys 16u + 4q + 0..3 and 16u + 8 + 4q + 0..3: the keys of the P^T registers.
  static __device__ __forceinline__ void pv(f32x16* o, const pop_t* pb, const elem* vt, int lane) {
    const int m = lane & 31, q = lane >> 5;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const elem* vr = vt + (32 * dt + m) * kVRow + 16 * u + 4 * q;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = mfma32(a, pb[u], o[dt]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep one chunk's operands live at a time
    }
  }
  static __device__ __forceinline__ void store4(elem* dst, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
};

template <>
struct TileOps<F32> {
  typedef float elem;
  static constexpr int kQSteps = kHeadDim / 2;  // 32x32x2 fp32: dim 2s + q
  typedef float qop_t;
  static __device__ __forceinline__ void load_q(qop_t* op, const elem* row, int q, bool ok) {
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) op[s] = ok ? row[2 * s + q] : 0.f;
  }
  static __device__ __forceinline__ f32x16 s_tile(const elem* krow, const qop_t* op, int q) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) acc = mfma32(krow[2 * s + q], op[s], acc);
    return acc;
  }
  // fp32 P^T operands: k-step (kt, r) takes, in lane group q, the probability of key
  // 32kt + 8(r/4) + 4q + r%4, which is register r of S^T tile kt.
  typedef float pop_t;
  static constexpr int kPChunks = 64;
  static __device__ __forceinline__ void pack_p(pop_t* pb, const float (&p)[4][16]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[16 * kt + r] = p[kt][r];
  }
  static __device__ __forceinline__ void pv(f32x16* o, const pop_t* pb, const elem* vt, int lane) {
    const int m = lane & 31, q = lane >> 5;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * q + (r & 3);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = mfma32(vt[(32 * dt + m) * kVRow + key], pb[16 * kt + r], o[dt]);
      }
  }
  static __device__ __forceinline__ void store4(elem* dst, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
};

template <class E>
__global__ __launch_bounds__(256, 2) void kv_attn_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offset_total,
    typename E::elem* __restrict__ part_o, float* __restrict__ part_ml, int G, int Hpg,
    int top_k, int64_t q_begin, int64_t seq_len) {
  typedef typename E::elem elem;
  typedef TileOps<E> T;
  __shared__ __align__(16) elem Ks[kBlock * kKRow];
  __shared__ __align__(16) elem Vt[kHeadDim * kVRow];
  __shared__ int32_t ids[kTile];
  __shared__ int32_t keys[kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t total = *offset_total;
  const int64_t e0 = (int64_t)blockIdx.x * kTile;
  if (e0 >= total) return;
  const int n = (int)min((int64_t)kTile, total - e0);
  const int Hq = G * Hpg;
  const int epr = 32 / Hpg;  // entries per 32-row tile
  if (tid < n) {
    const int32_t id = sorted[e0 + tid];
    ids[tid] = id;
    const int64_t rowg = id / top_k;
    keys[tid] = (int32_t)((rowg % G) << 24) | block_idx[id];  // (g, c): g < 64, c < 2^24
  }
  __syncthreads();
  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);

  int r0 = 0;
  while (r0 < n) {
    const int key = keys[r0];
    int r1 = r0 + 1;
    while (r1 < n && keys[r1] == key) ++r1;
    const int g = key >> 24;
    const int c = key & 0xffffff;
    // Stage K (row-major) and V (transposed) of block c of group g.
    {
      const int64_t key0 = (int64_t)c * kBlock;
      const int nk = (int)min((int64_t)kBlock, seq_len - key0);
      const elem* kg = K + ((int64_t)g * seq_len + key0) * kHeadDim;
      const elem* vg = V + ((int64_t)g * seq_len + key0) * kHeadDim;
      constexpr int kPer = 16 / sizeof(elem);  // elements per 16-byte chunk
      constexpr int kChunks = kBlock * kHeadDim / kPer;
      // K: consecutive lanes take consecutive 16-byte chunks of a row (row-major LDS).
      for (int ch = tid; ch < kChunks; ch += 256) {
        const int row = ch / (kHeadDim / kPer);
        const int col = (ch % (kHeadDim / kPer)) * kPer;
        u32x4 kv = {0u, 0u, 0u, 0u};
        if (row < nk) kv = *reinterpret_cast<const u32x4*>(kg + row * kHeadDim + col);
        *reinterpret_cast<u32x4*>(&Ks[row * kKRow + col]) = kv;
      }
      // V^T: consecutive lanes take consecutive key pairs of one 16-byte column chunk,
      // so each transposed write packs two keys and the lanes hit distinct banks.
      if constexpr (E::is_bf16) {
        for (int it = tid; it < (kBlock / 2) * (kHeadDim / 8); it += 256) {
          const int pr = it % (kBlock / 2);
          const int col = (it / (kBlock / 2)) * 8;
          const int r = 2 * pr;
          u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
          if (r < nk) a = *reinterpret_cast<const u32x4*>(vg + r * kHeadDim + col);
          if (r + 1 < nk) b = *reinterpret_cast<const u32x4*>(vg + (r + 1) * kHeadDim + col);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = (a[j] & 0xffffu) | (b[j] << 16);
            const uint32_t hi = (a[j] >> 16) | (b[j] & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(&Vt[(col + 2 * j) * kVRow + r]) = lo;
            *reinterpret_cast<uint32_t*>(&Vt[(col + 2 * j + 1) * kVRow + r]) = hi;
          }
        }
      } else {
        for (int it = tid; it < kBlock * (kHeadDim / kPer); it += 256) {
          const int row = it % kBlock;
          const int col = (it / kBlock) * kPer;
          u32x4 vv = {0u, 0u, 0u, 0u};
          if (row < nk) vv = *reinterpret_cast<const u32x4*>(vg + row * kHeadDim + col);
          const elem* ve = reinterpret_cast<const elem*>(&vv);
#pragma unroll
          for (int j = 0; j < kPer; ++j) Vt[(col + j) * kVRow + row] = ve[j];
        }
      }
    }
    __syncthreads();

    // Row tiles of this run, round-robin over the waves.
    const int nrt = (r1 - r0 + epr - 1) / epr;
    for (int rt = wave; rt < nrt; rt += 4) {
      const int n32 = lane & 31, q = lane >> 5;
      const int e = n32 / Hpg;
      const int h = n32 - e * Hpg;
      const int ent = r0 + rt * epr + e;
      const bool ok = e < epr && ent < r1;
      const int32_t id = ok ? ids[ent] : 0;
      const int64_t t = q_begin + (id / top_k) / G;
      typename T::qop_t qop[T::kQSteps];
      T::load_q(qop, Q + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, ok);
      // S^T for the 128 keys, scaled to log2 units and masked (causal in the local block).
      float p[4][16];
      float mx = -INFINITY;
      const int64_t lim = t - (int64_t)c * kBlock;  // keys kk <= lim are visible
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 s = T::s_tile(&Ks[(32 * kt + n32) * kKRow], qop, q);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * kt + 8 * (r >> 2) + 4 * q + (r & 3);
          const float x = kk <= lim ? s[r] * qk_scale : -INFINITY;
          p[kt][r] = x;
          mx = fmaxf(mx, x);
        }
        __builtin_amdgcn_sched_barrier(0);  // one key tile's K operands live at a time
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float l = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ev = exp2f(p[kt][r] - mx);
          p[kt][r] = ev;
          l += ev;
        }
      l += __shfl_xor(l, 32, 64);
      typename T::pop_t pb[T::kPChunks];
      T::pack_p(pb, p);
      f32x16 o[4] = {};
      T::pv(o, pb, Vt, lane);
      if (ok) {
        const float inv = 1.f / l;
        const int64_t prow = (int64_t)id * Hpg + h;
        elem* dst = part_o + prow * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            T::store4(dst + 32 * dt + 8 * j + 4 * q, o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv,
                      o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
        if (q == 0) *reinterpret_cast<float2*>(part_ml + prow * 2) = make_float2(mx, l);
      }
    }
    __syncthreads();
    r0 = r1;
  }
}

// ---- merge ----------------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(64) void kv_merge_kernel(const typename E::elem* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ block_idx,
                                                      typename E::elem* __restrict__ out, int G,
                                                      int Hpg, int top_k, int64_t q_begin) {
  typedef typename E::elem elem;
  const int lane = threadIdx.x;
  const int64_t rowg = blockIdx.x;  // (i, g)
  const int64_t i = rowg / G;
  const int g = (int)(rowg % G);
  const int64_t t = q_begin + i;
  const int blocal = (int)(t / kBlock);
  const int32_t* sel = block_idx + rowg * top_k;
  const int Hq = G * Hpg;
  for (int h = 0; h < Hpg; ++h) {
    float M = -INFINITY;
    for (int s = 0; s < top_k; ++s) {
      const int c = sel[s];
      if (c < 0 || c > blocal) continue;
      M = fmaxf(M, part_ml[((rowg * top_k + s) * Hpg + h) * 2]);
    }
    float a0 = 0.f, a1 = 0.f, L = 0.f;
    for (int s = 0; s < top_k; ++s) {
      const int c = sel[s];
      if (c < 0 || c > blocal) continue;
      const int64_t prow = (rowg * top_k + s) * Hpg + h;
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + prow * 2);
      const float w = ml.y * exp2f(ml.x - M);
      const elem* src = part_o + prow * kHeadDim + 2 * lane;
      float o0, o1;
      if constexpr (E::is_bf16) {
        const uint32_t wbits = *reinterpret_cast<const uint32_t*>(src);
        o0 = bf16_bits_to_f32(wbits & 0xffffu);
        o1 = bf16_bits_to_f32(wbits >> 16);
      } else {
        const float2 v = *reinterpret_cast<const float2*>(src);
        o0 = v.x;
        o1 = v.y;
      }
      a0 += w * o0;
      a1 += w * o1;
      L += w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    elem* dst = out + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim + 2 * lane;
    if constexpr (E::is_bf16) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(a0 * inv, a1 * inv);
    } else {
      *reinterpret_cast<float2*>(dst) = make_float2(a0 * inv, a1 * inv);
    }
  }
}

// ---- host side -------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

size_t kv_workspace_bytes(int bf16, int64_t q_count, int G, int Hpg, int top_k, int nblk) {
  const int64_t nb = (int64_t)G * nblk;
  const int64_t E = q_count * G * top_k;
  const size_t es = bf16 ? 2 : 4;
  return al256((size_t)(nb + 1) * 4) * 3 + al256((size_t)E * 4) + al256((size_t)E * Hpg * 2 * 4) +
         al256((size_t)E * Hpg * kHeadDim * es);
}

template <class E>
static hipError_t launch_kv_t(const void* q, const void* k, const void* v,
                              const int32_t* block_idx, void* out, void* ws, int G, int Hpg,
                              int top_k, int64_t q_begin, int64_t q_count, int64_t seq_len,
                              int nblk, hipStream_t st) {
  typedef typename E::elem elem;
  const int64_t nb = (int64_t)G * nblk;
  const int64_t n_entries = q_count * G * top_k;
  char* w = static_cast<char*>(ws);
  int32_t* count = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)(nb + 1) * 4);
  int32_t* offset = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)(nb + 1) * 4);
  int32_t* cursor = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)(nb + 1) * 4);
  int32_t* sorted = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)n_entries * 4);
  float* part_ml = reinterpret_cast<float*>(w);
  w += al256((size_t)n_entries * Hpg * 2 * 4);
  elem* part_o = reinterpret_cast<elem*>(w);

  const unsigned grid_e = (unsigned)std::min<int64_t>((n_entries + 255) / 256, 65536);
  hipLaunchKernelGGL(kv_zero_kernel, dim3((unsigned)std::min<int64_t>((nb + 255) / 256, 4096)),
                     dim3(256), 0, st, count, nb);
  hipLaunchKernelGGL(kv_count_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries, G,
                     top_k, q_begin, nblk, count);
  hipLaunchKernelGGL(kv_scan_kernel, dim3(1), dim3(1024), 0, st, count, nb, offset, cursor);
  hipLaunchKernelGGL(kv_scatter_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries, G,
                     top_k, q_begin, nblk, cursor, sorted);
  const unsigned tiles = (unsigned)((n_entries + kTile - 1) / kTile);
  hipLaunchKernelGGL((kv_attn_kernel<E>), dim3(tiles), dim3(256), 0, st, (const elem*)q,
                     (const elem*)k, (const elem*)v, block_idx, sorted, offset + nb, part_o,
                     part_ml, G, Hpg, top_k, q_begin, seq_len);
  hipLaunchKernelGGL((kv_merge_kernel<E>), dim3((unsigned)(q_count * G)), dim3(64), 0, st, part_o,
                     part_ml, block_idx, (elem*)out, G, Hpg, top_k, q_begin);
  return hipGetLastError();
}

hipError_t launch_kv_prefill(int bf16, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, void* out, void* workspace, int G, int Hpg,
                             int top_k, int64_t q_begin, int64_t q_count, int64_t seq_len,
                             int nblk, hipStream_t stream) {
  if (bf16)
    return launch_kv_t<BF16>(q, k, v, block_idx, out, workspace, G, Hpg, top_k, q_begin, q_count,
                             seq_len, nblk, stream);
  return launch_kv_t<F32>(q, k, v, block_idx, out, workspace, G, Hpg, top_k, q_begin, q_count,
                          seq_len, nblk, stream);
}

}  // namespace msa
