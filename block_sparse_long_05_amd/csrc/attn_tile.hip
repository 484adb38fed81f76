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

constexpr int kTile = 256;                 // sorted entries per workgroup
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

// Popular blocks (the local block, blocks most queries pick) would send every
// increment to one counter. Each bucket therefore has kStripes counters, picked by
// token, in separate cache lines: count[stripe * nbuckets + bucket]. The scan walks
// buckets in order and stripes within a bucket, so the sorted entries of one bucket
// stay contiguous.
constexpr int kStripes = 16;

__global__ void kv_count_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                int top_k, int64_t q_begin, int nblk, int32_t* __restrict__ count) {
  const int64_t nb = (int64_t)G * nblk;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk);
    const int stripe = (int)((id / ((int64_t)G * top_k)) % kStripes);
    if (k >= 0) atomicAdd(&count[stripe * nb + k], 1);
  }
}

// Exclusive scan over (bucket, stripe) in bucket-major order. Writes cursor[] (same
// layout as count[]) and bucket_off[0..nb] (start of each bucket; bucket_off[nb] = total).
__global__ __launch_bounds__(1024) void kv_scan_kernel(const int32_t* __restrict__ count,
                                                       int64_t nb, int32_t* __restrict__ cursor,
                                                       int32_t* __restrict__ bucket_off) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t lo = min(nb, tid * per), hi = min(nb, lo + per);
  int32_t s = 0;
  for (int64_t k = lo; k < hi; ++k)
    for (int st = 0; st < kStripes; ++st) s += count[st * nb + k];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;  // exclusive prefix of this thread's range
  for (int64_t k = lo; k < hi; ++k) {
    bucket_off[k] = run;
    for (int st = 0; st < kStripes; ++st) {
      cursor[st * nb + k] = run;
      run += count[st * nb + k];
    }
  }
  if (tid == 1023) bucket_off[nb] = part[1023];
}

__global__ void kv_scatter_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                  int top_k, int64_t q_begin, int nblk,
                                  int32_t* __restrict__ cursor, int32_t* __restrict__ sorted) {
  const int64_t nb = (int64_t)G * nblk;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk);
    const int stripe = (int)((id / ((int64_t)G * top_k)) % kStripes);
    if (k >= 0) sorted[atomicAdd(&cursor[stripe * nb + k], 1)] = (int32_t)id;
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

// One workgroup (4 waves, 512 registers each) per CU. Latency is hidden explicitly:
// the K/V block of the next run is loaded into registers while the current run computes
// and is then written to the other LDS buffer (bf16; fp32 single-buffers), and each
// wave gathers the queries of its next row tile while the current one finishes.
template <class E>
struct KvStage {
  typedef typename E::elem elem;
  static constexpr int kPer = 16 / sizeof(elem);                      // elements per chunk
  static constexpr int kKChunks = kBlock * kHeadDim / kPer / 256;     // K chunks per thread
  static constexpr int kVItems = E::is_bf16 ? (kBlock / 2) * (kHeadDim / 8) / 256
                                            : kBlock * (kHeadDim / kPer) / 256;
  static constexpr int kVRegs = E::is_bf16 ? 2 * kVItems : kVItems;
  u32x4 kr[kKChunks];
  u32x4 vr[kVRegs];

  __device__ __forceinline__ void load(const elem* K, const elem* V, int g, int c, int64_t seq_len,
                                       int tid) {
    const int64_t key0 = (int64_t)c * kBlock;
    const int nk = (int)min((int64_t)kBlock, seq_len - key0);
    const elem* kg = K + ((int64_t)g * seq_len + key0) * kHeadDim;
    const elem* vg = V + ((int64_t)g * seq_len + key0) * kHeadDim;
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      const int ch = tid + 256 * i;
      const int row = ch / (kHeadDim / kPer);
      const int col = (ch % (kHeadDim / kPer)) * kPer;
      kr[i] = row < nk ? *reinterpret_cast<const u32x4*>(kg + row * kHeadDim + col) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kVItems; ++i) {
      const int it = tid + 256 * i;
      if constexpr (E::is_bf16) {
        const int r = 2 * (it % (kBlock / 2));
        const int col = (it / (kBlock / 2)) * 8;
        vr[2 * i] = r < nk ? *reinterpret_cast<const u32x4*>(vg + r * kHeadDim + col) : u32x4{0u, 0u, 0u, 0u};
        vr[2 * i + 1] = r + 1 < nk ? *reinterpret_cast<const u32x4*>(vg + (r + 1) * kHeadDim + col)
                                   : u32x4{0u, 0u, 0u, 0u};
      } else {
        const int row = it % kBlock;
        const int col = (it / kBlock) * kPer;
        vr[i] = row < nk ? *reinterpret_cast<const u32x4*>(vg + row * kHeadDim + col) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // K row-major (consecutive lanes: consecutive 16-byte chunks of a row); V transposed
  // (consecutive lanes: consecutive key pairs, two keys packed per 4-byte write).
  __device__ __forceinline__ void store(elem* Ks, elem* Vt, int tid) const {
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      const int ch = tid + 256 * i;
      const int row = ch / (kHeadDim / kPer);
      const int col = (ch % (kHeadDim / kPer)) * kPer;
      *reinterpret_cast<u32x4*>(&Ks[row * kKRow + col]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < kVItems; ++i) {
      const int it = tid + 256 * i;
      if constexpr (E::is_bf16) {
        const int r = 2 * (it % (kBlock / 2));
        const int col = (it / (kBlock / 2)) * 8;
        const u32x4 a = vr[2 * i], b = vr[2 * i + 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *reinterpret_cast<uint32_t*>(&Vt[(col + 2 * j) * kVRow + r]) = (a[j] & 0xffffu) | (b[j] << 16);
          *reinterpret_cast<uint32_t*>(&Vt[(col + 2 * j + 1) * kVRow + r]) = (a[j] >> 16) | (b[j] & 0xffff0000u);
        }
      } else {
        const int row = it % kBlock;
        const int col = (it / kBlock) * kPer;
        const elem* ve = reinterpret_cast<const elem*>(&vr[i]);
#pragma unroll
        for (int j = 0; j < kPer; ++j) Vt[(col + j) * kVRow + row] = ve[j];
      }
    }
  }
};

template <class E>
__global__ __launch_bounds__(256, 1) void kv_attn_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offset_total,
    typename E::elem* __restrict__ part_o, float* __restrict__ part_ml, int G, int Hpg,
    int top_k, int64_t q_begin, int64_t seq_len) {
  typedef typename E::elem elem;
  typedef TileOps<E> T;
  constexpr int kBufs = E::is_bf16 ? 2 : 1;
  __shared__ __align__(16) elem Ks[kBufs][kBlock * kKRow];
  __shared__ __align__(16) elem Vt[kBufs][kHeadDim * kVRow];
  __shared__ int32_t ids[kTile];
  __shared__ int32_t keys[kTile];
  __shared__ int32_t run_start[kTile + 1];
  __shared__ uint64_t bmask[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t total = *offset_total;
  const int64_t e0 = (int64_t)blockIdx.x * kTile;
  if (e0 >= total) return;
  const int n = (int)min((int64_t)kTile, total - e0);
  const int Hq = G * Hpg;
  const int epr = 32 / Hpg;  // entries per 32-row tile
  int32_t mykey = -1;
  if (tid < n) {
    const int32_t id = sorted[e0 + tid];
    ids[tid] = id;
    mykey = (int32_t)(((id / top_k) % G) << 24) | block_idx[id];  // (g, c): g < 64, c < 2^24
    keys[tid] = mykey;
  }
  __syncthreads();
  // Runs of equal (g, c): boundary flags -> ballots -> run_start[] by prefix popcount.
  const bool boundary = tid < n && (tid == 0 || keys[tid - 1] != mykey);
  const uint64_t wm = __ballot(boundary);
  if (lane == 0) bmask[wave] = wm;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += __popcll(bmask[w]);
  const int nruns = __popcll(bmask[0]) + __popcll(bmask[1]) + __popcll(bmask[2]) + __popcll(bmask[3]);
  if (boundary) run_start[before + __popcll(wm & ((1ull << lane) - 1ull))] = tid;
  if (tid == 0) run_start[nruns] = n;
  __syncthreads();

  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const int n32 = lane & 31, q = lane >> 5;
  const int e = n32 / Hpg;
  const int h = n32 - e * Hpg;

  KvStage<E> st;
  {
    const int key = keys[0];
    st.load(K, V, key >> 24, key & 0xffffff, seq_len, tid);
    st.store(Ks[0], Vt[0], tid);
  }
  __syncthreads();

  for (int j = 0; j < nruns; ++j) {
    const int r0 = run_start[j], r1 = run_start[j + 1];
    const int key = keys[r0];
    const int g = key >> 24;
    const int c = key & 0xffffff;
    const int buf = kBufs == 2 ? (j & 1) : 0;
    const bool next = j + 1 < nruns;
    if (kBufs == 2 && next) {
      const int nkey = keys[r1];
      st.load(K, V, nkey >> 24, nkey & 0xffffff, seq_len, tid);
    }
    const elem* ks = Ks[buf];
    const elem* vt = Vt[buf];

    // Row tiles of this run, round-robin over the waves; the next row tile's queries
    // are gathered as soon as S^T has consumed the current ones.
    const int nrt = (r1 - r0 + epr - 1) / epr;
    auto row_of = [&](int rt, int32_t& id, int64_t& t) {
      const int ent = r0 + rt * epr + e;
      const bool ok = e < epr && ent < r1;
      id = ok ? ids[ent] : 0;
      t = q_begin + (id / top_k) / G;
      return ok;
    };
    typename T::qop_t qop[T::kQSteps];
    int32_t id = 0;
    int64_t t = 0;
    bool ok = false;
    if (wave < nrt) {
      ok = row_of(wave, id, t);
      T::load_q(qop, Q + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, ok);
    }
    for (int rt = wave; rt < nrt; rt += 4) {
      // S^T for the 128 keys. Only a row tile holding a local-block entry needs the
      // causal mask (keys kk <= lim visible); the scale goes into the exponent's FMA.
      float p[4][16];
      float mx = -INFINITY;
      const int64_t lim = t - (int64_t)c * kBlock;
      const bool masked = __ballot(ok && lim < kBlock - 1) != 0;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 s = T::s_tile(&ks[(32 * kt + n32) * kKRow], qop, q);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[r];
          if (masked) {
            const int kk = 32 * kt + 8 * (r >> 2) + 4 * q + (r & 3);
            x = kk <= lim ? x : -INFINITY;
          }
          p[kt][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      const int32_t cur_id = id;
      const bool cur_ok = ok;
      if (rt + 4 < nrt) {
        ok = row_of(rt + 4, id, t);
        T::load_q(qop, Q + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, ok);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxs = mx * qk_scale;  // row max in log2 units (finite: key 128c <= t)
      float l = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ev = fast_exp2(fmaf(p[kt][r], qk_scale, -mxs));
          p[kt][r] = ev;
          l += ev;
        }
      l += __shfl_xor(l, 32, 64);
      typename T::pop_t pb[T::kPChunks];
      T::pack_p(pb, p);
      f32x16 o[4] = {};
      T::pv(o, pb, vt, lane);
      if (cur_ok) {
        const float inv = 1.f / l;
        const int64_t prow = (int64_t)cur_id * Hpg + h;
        elem* dst = part_o + prow * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            T::store4(dst + 32 * dt + 8 * jj + 4 * q, o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv,
                      o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
        if (q == 0) *reinterpret_cast<float2*>(part_ml + prow * 2) = make_float2(mxs, l);
      }
    }
    if (next) {
      if constexpr (kBufs == 2) {
        st.store(Ks[buf ^ 1], Vt[buf ^ 1], tid);
      } else {
        __syncthreads();  // single buffer: everyone is done reading it
        const int nkey = keys[r1];
        st.load(K, V, nkey >> 24, nkey & 0xffffff, seq_len, tid);
        st.store(Ks[0], Vt[0], tid);
      }
    }
    __syncthreads();
  }
}

// ---- merge ----------------------------------------------------------------------------------
// One wave per (token, group). Lane = (head quarter hq = lane / 16, dims 8*(lane % 16) ..+8):
// every load moves 16 bytes of one head's partial and one instruction covers four heads.
// Pass 1 finds each head's maximum, pass 2 weights and sums the partials in slot order.
template <class E, int HMAX>
__global__ __launch_bounds__(64) void kv_merge_kernel(const typename E::elem* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ block_idx,
                                                      typename E::elem* __restrict__ out, int G,
                                                      int Hpg, int top_k, int64_t q_begin) {
  typedef typename E::elem elem;
  constexpr int HJ = HMAX / 4;  // heads per lane
  const int lane = threadIdx.x;
  const int hq = lane >> 4;
  const int d8 = (lane & 15) * 8;
  const int64_t rowg = blockIdx.x;  // (i, g)
  const int64_t i = rowg / G;
  const int g = (int)(rowg % G);
  const int64_t t = q_begin + i;
  const int blocal = (int)(t / kBlock);
  const int32_t* sel = block_idx + rowg * top_k;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + rowg * top_k * Hpg;
  const int Hq = G * Hpg;
  float M[HJ], L[HJ], acc[HJ][8];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    M[j] = -INFINITY;
    L[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  for (int s = 0; s < top_k; ++s) {
    const int c = sel[s];
    if (c < 0 || c > blocal) continue;
#pragma unroll
    for (int j = 0; j < HJ; ++j)
      if (hq + 4 * j < Hpg) M[j] = fmaxf(M[j], ml[s * Hpg + hq + 4 * j].x);
  }
  for (int s = 0; s < top_k; ++s) {
    const int c = sel[s];
    if (c < 0 || c > blocal) continue;
    const elem* src = part_o + ((rowg * top_k + s) * Hpg) * kHeadDim + d8;
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const int h = hq + 4 * j;
      if (h < Hpg) {
        const float2 p = ml[s * Hpg + h];
        const float w = p.y * fast_exp2(p.x - M[j]);
        L[j] += w;
        float o[8];
        if constexpr (E::is_bf16) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src + h * kHeadDim);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
            o[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
          }
        } else {
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + h * kHeadDim);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + h * kHeadDim + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = v0[e];
            o[4 + e] = v1[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += w * o[e];
      }
    }
  }
  elem* dst = out + (t * Hq + (int64_t)g * Hpg) * kHeadDim + d8;
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int h = hq + 4 * j;
    if (h < Hpg) {
      const float inv = L[j] > 0.f ? 1.f / L[j] : 0.f;
      if constexpr (E::is_bf16) {
        *reinterpret_cast<u32x4*>(dst + h * kHeadDim) =
            u32x4{pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv), pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv),
                  pack_bf16x2(acc[j][4] * inv, acc[j][5] * inv), pack_bf16x2(acc[j][6] * inv, acc[j][7] * inv)};
      } else {
        *reinterpret_cast<f32x4*>(dst + h * kHeadDim) =
            f32x4{acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv};
        *reinterpret_cast<f32x4*>(dst + h * kHeadDim + 4) =
            f32x4{acc[j][4] * inv, acc[j][5] * inv, acc[j][6] * inv, acc[j][7] * inv};
      }
    }
  }
}

// ---- host side -------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

size_t kv_workspace_bytes(int bf16, int64_t q_count, int G, int Hpg, int top_k, int nblk) {
  const int64_t nb = (int64_t)G * nblk;
  const int64_t E = q_count * G * top_k;
  const size_t es = bf16 ? 2 : 4;
  return al256((size_t)nb * kStripes * 4) * 2 + al256((size_t)(nb + 1) * 4) +
         al256((size_t)E * 4) + al256((size_t)E * Hpg * 2 * 4) +
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
  w += al256((size_t)nb * kStripes * 4);
  int32_t* cursor = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)nb * kStripes * 4);
  int32_t* offset = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)(nb + 1) * 4);
  int32_t* sorted = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)n_entries * 4);
  float* part_ml = reinterpret_cast<float*>(w);
  w += al256((size_t)n_entries * Hpg * 2 * 4);
  elem* part_o = reinterpret_cast<elem*>(w);

  const unsigned grid_e = (unsigned)std::min<int64_t>((n_entries + 255) / 256, 65536);
  const int64_t ncnt = nb * kStripes;
  hipLaunchKernelGGL(kv_zero_kernel, dim3((unsigned)std::min<int64_t>((ncnt + 255) / 256, 4096)),
                     dim3(256), 0, st, count, ncnt);
  hipLaunchKernelGGL(kv_count_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries, G,
                     top_k, q_begin, nblk, count);
  hipLaunchKernelGGL(kv_scan_kernel, dim3(1), dim3(1024), 0, st, count, nb, cursor, offset);
  hipLaunchKernelGGL(kv_scatter_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries, G,
                     top_k, q_begin, nblk, cursor, sorted);
  const unsigned tiles = (unsigned)((n_entries + kTile - 1) / kTile);
  hipLaunchKernelGGL((kv_attn_kernel<E>), dim3(tiles), dim3(256), 0, st, (const elem*)q,
                     (const elem*)k, (const elem*)v, block_idx, sorted, offset + nb, part_o,
                     part_ml, G, Hpg, top_k, q_begin, seq_len);
  const dim3 mgrid((unsigned)(q_count * G));
  if (Hpg <= 4)
    hipLaunchKernelGGL((kv_merge_kernel<E, 4>), mgrid, dim3(64), 0, st, part_o, part_ml,
                       block_idx, (elem*)out, G, Hpg, top_k, q_begin);
  else if (Hpg <= 8)
    hipLaunchKernelGGL((kv_merge_kernel<E, 8>), mgrid, dim3(64), 0, st, part_o, part_ml,
                       block_idx, (elem*)out, G, Hpg, top_k, q_begin);
  else
    hipLaunchKernelGGL((kv_merge_kernel<E, 16>), mgrid, dim3(64), 0, st, part_o, part_ml,
                       block_idx, (elem*)out, G, Hpg, top_k, q_begin);
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
