// Main branch of MSA for prefill: a hybrid of query-tile and KV-centric ("reverse index")
// attention.
//
// The researchpapers.dev summary of the MSA paper ("What it means for inference
// teams") names the real costs of a sparse prefill kernel: index construction, top-k,
// query gathering, reverse indexing and load balancing; the baguaai.com note on MSA
// describes the kernel as aggregating queries on the KV side. Neighbouring tokens tend to
// keep the same blocks (the local block always, blocks that score high for a whole
// stretch of text often), so the work is split by how widely a block is kept:
//
//   1. kv_classify_kernel: per query tile (a few consecutive tokens) and group, the
//      blocks kept by at least half of the tile's tokens form the tile's shared list;
//   2. reverse index of the other ("rare") kept entries: a counting sort by KV block
//      (group g, block c) - count, exclusive scan, scatter, with each chunk of rows
//      summing its per-block counts in LDS before one global atomic per block;
//   3. kv_attn_kernel: the sorted rare entries are cut into fixed tiles of 256 entries
//      (load balance independent of how popular a block is). Each tile walks its runs
//      of equal (g, c): the block's K and V (transposed) are staged in LDS once and
//      every query of the run attends to it with 32x32x16 bf16 MFMAs, rows = (entry,
//      head) pairs gathered from Q. A row sees one block, so its softmax is exact within
//      the block; it writes a partial (o / l, m, l);
//   4. qtile_attn kernels: per (query tile, group) the shared blocks are staged in LDS
//      one after another and every row of the tile runs an online softmax over those it
//      keeps (others masked); the row also folds in its rare partials with a log-sum-exp
//      combine in slot order (deterministic; no atomics touch values; the bf16 kernel
//      folds them first, while its first shared block is staged) and writes the output.
//
// MFMA orientation: S^T = K . Q^T so that a lane owns one query row and holds 16 of
// its keys per 32-key tile; the softmax reductions are in-lane plus one exchange
// with the other half-wave, and P^T in the same registers is already the B operand
// of O^T = V^T . P^T.
#include <algorithm>

#include "msa_device.h"
#include "msa_launch.h"
#include "msa_tile.h"

namespace msa {

constexpr int kTile = 256;                 // sorted entries per workgroup
// The bf16 reverse-index kernel takes 512 (two per thread): half as many block stagings and
// prologues (16.34 -> 16.26 ms for the attention at 131072 tokens).
constexpr int kKvTile = 2 * kTile;
constexpr int kTileF32 = 64;               // the same for the fp32 tile kernel
constexpr int kQtileWavesF32 = 4;          // row tiles (waves) of an fp32 query tile
constexpr int kKRow = kHeadDim + 8;        // LDS row stride of K (elements)
constexpr int kVRow = kBlock + 4;          // LDS row stride of V^T (elements)

// ---- reverse index --------------------------------------------------------------------
__global__ void kv_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Partials are stored in fragment order: value d = 32 dt + 8 jj + 4 q + r of a head's 128
// sits at 64 q + 16 dt + 4 jj + r, so the 64 values one lane holds are contiguous.
__device__ __forceinline__ int frag_pos(int dt, int jj, int q) { return 64 * q + 16 * dt + 4 * jj; }

// Query tiles: the rows of one 32-row MFMA tile are floor(32 / Hpg) tokens x Hpg heads,
// and a query tile is the row tiles of one workgroup: 8 for bf16, 4 for fp32 (whose
// problems are small: more workgroups fill the chip).
__host__ __device__ __forceinline__ int qtile_tokens(int Hpg, int bf16) {
  return (bf16 ? 8 : kQtileWavesF32) * (32 / Hpg);
}

// True when block c is in the tile's shared list (ascending, -1 padded).
__device__ __forceinline__ bool in_shared(const int32_t* slist, int top_k, int c) {
  for (int j = 0; j < top_k; ++j) {
    const int v = slist[j];
    if (v < 0 || v > c) return false;
    if (v == c) return true;
  }
  return false;
}

// Bucket (g * nblk + c) of a kept entry that goes through the reverse index, -1 for
// padding, invisible ids and entries of a shared block of the entry's query tile (no
// shared lists: every visible entry goes through).
__device__ __forceinline__ int64_t entry_bucket(const int32_t* block_idx, int64_t id, int G,
                                                int top_k, int64_t q_begin, int nblk,
                                                const int32_t* shared, int QT) {
  const int c = block_idx[id];
  const int64_t rowg = id / top_k;
  const int g = (int)(rowg % G);
  const int64_t i = rowg / G;
  const int64_t t = q_begin + i;
  if (c < 0 || (int64_t)c > t / kBlock) return -1;
  if (shared != nullptr && in_shared(shared + ((i / QT) * G + g) * top_k, top_k, c)) return -1;
  return (int64_t)g * nblk + c;
}

// One wave per (query tile, group): a block is shared when at least half of the tile's
// tokens keep it. Candidates are the blocks of the tile's last token (any block kept by
// half of the tokens is likely among them; the split only moves work between the two
// paths, every kept entry is still handled exactly once). The tile's ids are read once,
// 64 at a time, and each candidate's count comes from one ballot per 64 ids.
__global__ __launch_bounds__(256) void kv_classify_kernel(const int32_t* __restrict__ block_idx,
                                                          int32_t* __restrict__ shared, int G,
                                                          int top_k, int64_t q_begin,
                                                          int64_t q_count, int QT, int64_t npairs) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= npairs) return;
  const int64_t tile = pair / G;
  const int g = (int)(pair % G);
  const int64_t i0 = tile * QT;
  const int ntok = (int)min((int64_t)QT, q_count - i0);
  const int64_t t_last = q_begin + i0 + ntok - 1;
  int cand = -1;
  if (lane < top_k) {
    cand = block_idx[((i0 + ntok - 1) * G + g) * top_k + lane];
    if (cand < 0 || (int64_t)cand > t_last / kBlock) cand = -1;
  }
  int cnt = 0;  // lane j: how many of the tile's visible ids equal candidate j
  const int ne = ntok * top_k;
  for (int e0 = 0; e0 < ne; e0 += 64) {
    const int e = e0 + lane;
    int c = -1;
    if (e < ne) {
      const int tok = e / top_k;
      c = block_idx[((i0 + tok) * G + g) * top_k + (e - tok * top_k)];
      if ((int64_t)c > (q_begin + i0 + tok) / kBlock) c = -1;
    }
    for (int j = 0; j < top_k; ++j) {
      const int cj = __builtin_amdgcn_readlane(cand, j);
      if (cj < 0) continue;
      const int m = __popcll(__ballot(c == cj));
      cnt += lane == j ? m : 0;
    }
  }
  const bool keep = cand >= 0 && 2 * cnt >= ntok;
  const uint64_t m = __ballot(keep);
  const int pos = __popcll(m & ((1ull << lane) - 1ull));
  int32_t* out = shared + pair * top_k;
  if (keep) out[pos] = cand;
  const int nkeep = __popcll(m);
  for (int j = nkeep + lane; j < top_k; j += 64) out[j] = -1;
}

// Popular blocks (the local block, blocks most queries pick) would send every
// increment to one counter. Each bucket therefore has kStripes counters, picked by
// token, in separate cache lines: count[stripe * nbuckets + bucket]. The scan walks
// buckets in order and stripes within a bucket, so the sorted entries of one bucket
// stay contiguous.

__global__ void kv_count_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                int top_k, int64_t q_begin, int nblk, const int32_t* __restrict__ shared,
                                int QT, int32_t* __restrict__ count) {
  const int64_t nb = (int64_t)G * nblk;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk, shared, QT);
    const int stripe = (int)((id / ((int64_t)G * top_k)) % kStripes);
    if (k >= 0) atomicAdd(&count[stripe * nb + k], 1);
  }
}

// Exclusive scan over (bucket, stripe) in bucket-major order, in three passes that each
// read the counters coalesced (one thread per bucket): bucket totals into bucket_off[k],
// an in-place exclusive scan of the totals (bucket_off[nb] = total), then each stripe's
// cursor = its bucket's start + the counts of the earlier stripes of that bucket.
__global__ void kv_bucket_total_kernel(const int32_t* __restrict__ count, int64_t nb,
                                       int32_t* __restrict__ bucket_off) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < nb;
       k += (int64_t)gridDim.x * blockDim.x) {
    int32_t s = 0;
#pragma unroll
    for (int st = 0; st < kStripes; ++st) s += count[st * nb + k];
    bucket_off[k] = s;
  }
}

__global__ __launch_bounds__(1024) void kv_scan_kernel(int64_t nb, int32_t* __restrict__ bucket_off) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t lo = min(nb, tid * per), hi = min(nb, lo + per);
  int32_t s = 0;
  // unrolled so that several loads of the thread's range are in flight at once
#pragma unroll 8
  for (int64_t k = lo; k < hi; ++k) s += bucket_off[k];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;  // exclusive prefix of this thread's range
#pragma unroll 8
  for (int64_t k = lo; k < hi; ++k) {
    const int32_t c = bucket_off[k];
    bucket_off[k] = run;
    run += c;
  }
  if (tid == 1023) bucket_off[nb] = part[1023];
}

__global__ void kv_cursor_kernel(const int32_t* __restrict__ count, int64_t nb,
                                 const int32_t* __restrict__ bucket_off,
                                 int32_t* __restrict__ cursor) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < nb;
       k += (int64_t)gridDim.x * blockDim.x) {
    int32_t run = bucket_off[k];
#pragma unroll
    for (int st = 0; st < kStripes; ++st) {
      cursor[st * nb + k] = run;
      run += count[st * nb + k];
    }
  }
}

__global__ void kv_scatter_kernel(const int32_t* __restrict__ block_idx, int64_t n_entries, int G,
                                  int top_k, int64_t q_begin, int nblk,
                                  const int32_t* __restrict__ shared, int QT,
                                  int32_t* __restrict__ cursor, int32_t* __restrict__ sorted) {
  const int64_t nb = (int64_t)G * nblk;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < n_entries;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = entry_bucket(block_idx, id, G, top_k, q_begin, nblk, shared, QT);
    const int stripe = (int)((id / ((int64_t)G * top_k)) % kStripes);
    if (k >= 0) sorted[atomicAdd(&cursor[stripe * nb + k], 1)] = (int32_t)id;
  }
}

// The same count and scatter with the per-block sums taken in LDS first: one workgroup per
// (chunk of query rows, group) counts its entries per block with LDS atomics, then adds each
// nonzero count to the (stripe, bucket) counter with one global atomic (stripe = chunk), so
// a popular block costs one global atomic per chunk instead of one per entry. The scatter
// reserves each block's range the same way, then walks its entries again and takes each
// position from an LDS atomic on the reserved base. Used when the nblk counters and the
// chunk's shared lists fit in LDS; the order of entries inside a bucket is arbitrary, as
// with the kernels above. A chunk starts at a multiple of QT rows, so its tiles are whole.
constexpr int kRiThreads = 512;
constexpr int kRiLdsBytes = 64 * 1024;

template <bool kScatter>
__global__ __launch_bounds__(kRiThreads) void kv_index_lds_kernel(
    const int32_t* __restrict__ block_idx, int64_t q_count, int G, int top_k, int64_t q_begin,
    int nblk, const int32_t* __restrict__ shared, int QT, int rows, int32_t* __restrict__ ctr,
    int32_t* __restrict__ sorted) {
  extern __shared__ int32_t cnt[];  // nblk counters, then the shared lists of the chunk's tiles
  const int tid = threadIdx.x;
  // workgroups are dealt to the 8 XCDs in turn: renumber them so that the G groups of a chunk
  // (whose ids share cache lines) run on one XCD and share its L2
  unsigned wg = blockIdx.x;
  if ((gridDim.x & 7u) == 0) wg = (wg & 7u) * (gridDim.x >> 3) + (wg >> 3);
  const int g = (int)(wg % G);
  const int64_t chunk = wg / G;
  const int64_t i_lo = chunk * rows;
  const int ntok = (int)min((int64_t)rows, q_count - i_lo);
  const int64_t nb = (int64_t)G * nblk;
  int32_t* gctr = ctr + (chunk % kStripes) * nb + (int64_t)g * nblk;
  int32_t* sl = cnt + nblk;
  const int ntl = shared != nullptr ? (ntok + QT - 1) / QT : 0;
  for (int c = tid; c < nblk; c += kRiThreads) cnt[c] = 0;
  for (int x = tid; x < ntl * top_k; x += kRiThreads) {
    const int tl = x / top_k;
    sl[x] = shared[((i_lo / QT + tl) * G + g) * top_k + (x - tl * top_k)];
  }
  __syncthreads();
  const int ne = ntok * top_k;
  const int t_lo = (int)(q_begin + i_lo);  // < 2^30
  // block of entry e of the chunk, -1 when it does not go through the reverse index
  auto bucket = [&](int e, int64_t* id) {
    const int tok = e / top_k;
    *id = ((i_lo + tok) * G + g) * top_k + (e - tok * top_k);
    const int c = block_idx[*id];
    if (c < 0 || c > (t_lo + tok) / kBlock) return -1;
    if (shared != nullptr) {
      const int32_t* l = sl + (tok / QT) * top_k;  // ascending, -1 padded
      for (int j = 0; j < top_k; ++j) {
        const int v = l[j];
        if (v < 0 || v > c) break;
        if (v == c) return -1;
      }
    }
    return c;
  };
  for (int e = tid; e < ne; e += kRiThreads) {
    int64_t id;
    const int c = bucket(e, &id);
    if (c >= 0) atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  for (int c = tid; c < nblk; c += kRiThreads) {
    const int n = cnt[c];
    if (n > 0) {
      const int base = atomicAdd(&gctr[c], n);
      if (kScatter) cnt[c] = base;
    }
  }
  if (!kScatter) return;
  __syncthreads();
  for (int e = tid; e < ne; e += kRiThreads) {
    int64_t id;
    const int c = bucket(e, &id);
    if (c >= 0) sorted[atomicAdd(&cnt[c], 1)] = (int32_t)id;
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
template <class E, int NT = 256>
struct KvStage {
  typedef typename E::elem elem;
  static constexpr int kPer = 16 / sizeof(elem);                      // elements per chunk
  static constexpr int kKChunks = kBlock * kHeadDim / kPer / NT;      // K chunks per thread
  static constexpr int kVItems = E::is_bf16 ? (kBlock / 2) * (kHeadDim / 8) / NT
                                            : kBlock * (kHeadDim / kPer) / NT;
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
      const int ch = tid + NT * i;
      const int row = ch / (kHeadDim / kPer);
      const int col = (ch % (kHeadDim / kPer)) * kPer;
      kr[i] = row < nk ? *reinterpret_cast<const u32x4*>(kg + row * kHeadDim + col) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kVItems; ++i) {
      const int it = tid + NT * i;
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
      const int ch = tid + NT * i;
      const int row = ch / (kHeadDim / kPer);
      const int col = (ch % (kHeadDim / kPer)) * kPer;
      *reinterpret_cast<u32x4*>(&Ks[row * kKRow + col]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < kVItems; ++i) {
      const int it = tid + NT * i;
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

// TILE sorted entries per workgroup (the fp32 path takes small tiles: its problems are small,
// and more workgroups fill the chip).
template <class E, int TILE = kTile>
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
  __shared__ int32_t ids[TILE];
  __shared__ int32_t keys[TILE];
  __shared__ int32_t run_start[TILE + 1];
  __shared__ uint64_t bmask[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t total = *offset_total;
  const int64_t e0 = (int64_t)blockIdx.x * TILE;
  if (e0 >= total) return;
  const int n = (int)min((int64_t)TILE, total - e0);
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
      // 32-bit limit, clamped to [-1, 128], with the lane's key offset 4q folded in
      const int lim = min(max((int)t - c * kBlock, -1), kBlock);
      const int limq = lim - 4 * q;
      const bool masked = __ballot(ok && lim < kBlock - 1) != 0;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 s = T::s_tile(&ks[(32 * kt + n32) * kKRow], qop, q);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[r];
          if (masked) {
            x = 32 * kt + 8 * (r >> 2) + (r & 3) <= limq ? x : -INFINITY;
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
            T::store4(dst + frag_pos(dt, jj, q), o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv,
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


// ---- reverse-index tile attention, bf16 ----------------------------------------------------
// K and V of each run's block are staged row-major by direct global->LDS loads into one
// 64 KB buffer, so two workgroups share a CU and one's staging and query gathers overlap
// the other's MFMA work. A row tile sees one block: its four S tiles give the exact block
// maximum, then the exponentials and PV run per 64-key half. An entry's partial (Hpg heads x 128
// values, bf16) is one lane-interleaved block: the 16-byte chunk i (values
// 32 (i / 2) + 8 (i % 2) .. of the lane's fragment) of head h, lane group q sits at
// element i * 16 Hpg + 8 (h + Hpg q), so each store instruction writes whole cache lines.
// (m, l) = the row's reference maximum and sum go to part_ml.
__global__ __launch_bounds__(256, 2) void kv_attn_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offset_total,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int G, int Hpg, int top_k,
    int64_t q_begin, int64_t seq_len) {
  typedef TileOps<BF16> T;
  __shared__ __align__(16) uint8_t Kb[kBlock * 256];
  __shared__ __align__(16) uint8_t Vb[kBlock * 256];
  __shared__ int32_t ids[kKvTile];
  __shared__ int32_t keys[kKvTile];
  __shared__ int32_t run_start[kKvTile + 1];
  __shared__ uint64_t bmask[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t total = *offset_total;
  const int64_t e0 = (int64_t)blockIdx.x * kKvTile;
  if (e0 >= total) return;
  const int n = (int)min((int64_t)kKvTile, total - e0);
  const int Hq = G * Hpg;
  const int epr = 32 / Hpg;  // entries per 32-row tile
  int32_t mykey[2] = {-1, -1};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int i = tid + 256 * hf;
    if (i < n) {
      const int32_t id = sorted[e0 + i];
      ids[i] = id;
      mykey[hf] = (int32_t)(((id / top_k) % G) << 24) | block_idx[id];  // (g, c): c < 2^24
      keys[i] = mykey[hf];
    }
  }
  __syncthreads();
  // Runs of equal (g, c): boundary flags -> ballots -> run_start[] by prefix popcount.
  bool boundary[2];
  uint64_t wm[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int i = tid + 256 * hf;
    boundary[hf] = i < n && (i == 0 || keys[i - 1] != mykey[hf]);
    wm[hf] = __ballot(boundary[hf]);
    if (lane == 0) bmask[4 * hf + wave] = wm[hf];
  }
  __syncthreads();
  int nruns = 0;
  for (int w = 0; w < 8; ++w) nruns += __popcll(bmask[w]);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    int before = 0;
    for (int w = 0; w < 4 * hf + wave; ++w) before += __popcll(bmask[w]);
    if (boundary[hf])
      run_start[before + __popcll(wm[hf] & ((1ull << lane) - 1ull))] = tid + 256 * hf;
  }
  if (tid == 0) run_start[nruns] = n;
  __syncthreads();

  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const int n32 = lane & 31, q = lane >> 5;
  const int e = n32 / Hpg;
  const int h = n32 - e * Hpg;

  for (int j = 0; j < nruns; ++j) {
    // wave-uniform values in scalar registers (the staging addresses then use them)
    const int r0 = __builtin_amdgcn_readfirstlane(run_start[j]);
    const int r1 = __builtin_amdgcn_readfirstlane(run_start[j + 1]);
    const int key = __builtin_amdgcn_readfirstlane(keys[r0]);
    const int g = key >> 24;
    const int c = key & 0xffffff;
    if (j > 0) __syncthreads();  // every wave is done with the previous block
    // Lane-derived addresses are recomputed in each loop instead of being kept live
    // across it (the empty asm hides that the lane id does not change).
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    k_block_dma_s<256>(K, g, c, seq_len, Kb, wv, dma_lane_off<false>(tid_v & 63), tid_v);
    k_block_dma_s<256, true>(V, g, c, seq_len, Vb, wv, dma_lane_off<true>(tid_v & 63), tid_v);
    const int nrt = (r1 - r0 + epr - 1) / epr;
    auto row_of = [&](int rt, int32_t& id, int64_t& t) {
      const int ent = r0 + rt * epr + e;
      const bool ok = e < epr && ent < r1;
      id = ok ? ids[ent] : 0;
      t = q_begin + (id / top_k) / G;
      return ok;
    };
    // Row tiles alternate between two query-operand buffers: the queries of row tile
    // rt + 4 are requested as row tile rt starts, a whole row tile ahead of their use. The
    // loads are unconditional (a lane without entry reads the chunk's first row, whose
    // results it never stores): a load behind a lane mask would make the compiler wait for
    // every access in flight, the previous row tile's partial stores included.
    T::qop_t qa[T::kQSteps], qb[T::kQSteps];
    int32_t ida = 0, idb = 0;
    int64_t ta = 0, tb = 0;
    bool oka = false, okb = false;
    if (wave < nrt) {
      oka = row_of(wave, ida, ta);
      T::load_q(qa, Q + (ta * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, true);
    }
    MSA_WAIT_VMCNT(0);  // this wave's K and V loads have landed
    __syncthreads();
    auto row_tile = [&](int rt, const T::qop_t* qc, int32_t cur_id, int64_t tc, bool cur_ok,
                        T::qop_t* qn, int32_t& idn, int64_t& tn, bool& okn) {
      if (rt + 4 < nrt) {
        okn = row_of(rt + 4, idn, tn);
        T::load_q(qn, Q + (tn * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, true);
      }
      int lane_v = lane;
      asm volatile("" : "+v"(lane_v));
      const int n32v = lane_v & 31, qv = lane_v >> 5;
      const int lim = min(max((int)tc - c * kBlock, -1), kBlock);
      int limq = lim - 4 * q;  // the lane's key offset 4q folded into the limit
      asm volatile("" : "+v"(limq));
      const bool masked = __ballot(cur_ok && lim < kBlock - 1) != 0;
      f32x16 o[4] = {};
      // all four S^T tiles of the block and their maximum first: a row sees one block here,
      // so the maximum is exact and the accumulator is never rescaled
      float p[4][16];
      float mx = -INFINITY;
      f32x16 acc4[4];
      s_tiles4_swz(Kb, n32v, qc, qv, acc4);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 sv = acc4[kt];
        // the compare and select only where a row of the wave ends inside the block
        if (masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[kt][r] = 32 * kt + 8 * (r >> 2) + (r & 3) <= limq ? sv[r] : -INFINITY;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) p[kt][r] = sv[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, p[kt][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_run = mx * qk_scale;  // key 128c <= t: -inf only for a lane without entry
      const float mneg = m_run == -INFINITY ? 0.f : -m_run;
      float l_run = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 pb[4];
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          float* pr = p[2 * half + kk2];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[r] = fast_exp2(fmaf(pr[r], qk_scale, mneg));
            l_run += pr[r];
          }
          pb[2 * kk2] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                              pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
          pb[2 * kk2 + 1] = u32x4{pack_bf16x2(pr[8], pr[9]), pack_bf16x2(pr[10], pr[11]),
                                  pack_bf16x2(pr[12], pr[13]), pack_bf16x2(pr[14], pr[15])};
        }
        pv_half_tr(o, pb, Vb, lane_v, half);
      }
      l_run += __shfl_xor(l_run, 32, 64);
      if (cur_ok) {
        const float inv = 1.f / l_run;
        const int64_t prow = (int64_t)cur_id * Hpg + h;
        // lane-interleaved entry block: chunk i of lane (h, q) at i * 16 Hpg + 8 (h + Hpg q)
        uint16_t* dst = part_o + (int64_t)cur_id * Hpg * kHeadDim + 8 * (h + Hpg * q);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) {
            const int b0 = 8 * hp;
            *reinterpret_cast<u32x4*>(dst + (2 * dt + hp) * 16 * Hpg) =
                u32x4{pack_bf16x2(o[dt][b0] * inv, o[dt][b0 + 1] * inv),
                      pack_bf16x2(o[dt][b0 + 2] * inv, o[dt][b0 + 3] * inv),
                      pack_bf16x2(o[dt][b0 + 4] * inv, o[dt][b0 + 5] * inv),
                      pack_bf16x2(o[dt][b0 + 6] * inv, o[dt][b0 + 7] * inv)};
          }
        if (q == 0) *reinterpret_cast<float2*>(part_ml + prow * 2) = make_float2(m_run, l_run);
      }
    };
    for (int rt = wave; rt < nrt; rt += 8) {
      row_tile(rt, qa, ida, ta, oka, qb, idb, tb, okb);
      if (rt + 4 < nrt) row_tile(rt + 4, qb, idb, tb, okb, qa, ida, ta, oka);
    }
  }
}


// ---- query-tile attention over the shared blocks, folding in the rare partials ------------
// One workgroup (8 waves) per (query tile, group); wave w owns row tile w.
// For each shared block of the tile (staged once in LDS, the next one loaded while the
// current is used) every row runs an online softmax step - rows whose token did not keep
// the block are masked, the local block gets the causal mask. Then each row folds in
// the partials (o / l, m, l) of its rare entries, computed by the reverse-index path, in
// slot order, and the final output is written. No partial is stored for shared entries.
template <class E, int NW = 8>
__global__ __launch_bounds__(64 * NW, 1) void qtile_attn_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ shared, const typename E::elem* __restrict__ part_o,
    const float* __restrict__ part_ml, typename E::elem* __restrict__ out,
    float* __restrict__ lse, int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count,
    int64_t seq_len) {
  typedef typename E::elem elem;
  typedef TileOps<E> T;
  constexpr int kBufs = 1;  // fp32 path: one staged block
  __shared__ __align__(16) elem Ks[kBufs][kBlock * kKRow];
  __shared__ __align__(16) elem Vt[kBufs][kHeadDim * kVRow];
  __shared__ int32_t sl[64];
  __shared__ uint64_t selmask[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int epr = 32 / Hpg;
  const int QT = NW * epr;
  const int64_t tile = blockIdx.x / G;
  const int g = (int)(blockIdx.x % G);
  const int64_t i0 = tile * QT;
  const int ntok = (int)min((int64_t)QT, q_count - i0);
  const int Hq = G * Hpg;
  const int32_t* slist = shared + (tile * G + g) * top_k;
  if (tid < top_k) sl[tid] = slist[tid];
  __syncthreads();
  int ns = 0;
  while (ns < top_k && sl[ns] >= 0) ++ns;
  for (int tok = tid; tok < ntok; tok += 64 * NW) {
    const int32_t* tl = block_idx + ((i0 + tok) * G + g) * top_k;
    const int b = (int)((q_begin + i0 + tok) / kBlock);
    uint64_t mk = 0;
    for (int s2 = 0; s2 < top_k; ++s2) {
      const int c = tl[s2];
      if (c < 0 || c > b) continue;
      for (int j = 0; j < ns; ++j)
        if (sl[j] == c) mk |= 1ull << j;
    }
    selmask[tok] = mk;
  }
  __syncthreads();

  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const int n32 = lane & 31, q = lane >> 5;
  const int e = n32 / Hpg;
  const int h = n32 - e * Hpg;
  constexpr int rt = 0;  // one row tile per wave
  int tok_r[1];
  bool ok_r[1];
  int64_t t_r[1];
  uint64_t mask_r[1];
  tok_r[0] = wave * epr + e;
  ok_r[0] = e < epr && tok_r[0] < ntok;
  t_r[0] = q_begin + i0 + (ok_r[0] ? tok_r[0] : 0);
  mask_r[0] = ok_r[0] ? selmask[tok_r[0]] : 0ull;
  float m_r[1] = {-INFINITY}, l_r[1] = {0.f};
  f32x16 o[1][4] = {};

  KvStage<E, 64 * NW> st;
  if (ns > 0) {
    st.load(K, V, g, sl[0], seq_len, tid);
    st.store(Ks[0], Vt[0], tid);
  }
  __syncthreads();
  for (int j = 0; j < ns; ++j) {
    const int c = sl[j];
    const int buf = kBufs == 2 ? (j & 1) : 0;
    const bool next = j + 1 < ns;
    if (kBufs == 2 && next) st.load(K, V, g, sl[j + 1], seq_len, tid);
    const elem* ks = Ks[buf];
    const elem* vt = Vt[buf];
    do {
      const bool sel = ok_r[rt] && ((mask_r[rt] >> j) & 1ull);
      if (__ballot(sel) == 0) break;
      typename T::qop_t qop[T::kQSteps];
      T::load_q(qop, Q + (t_r[rt] * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, sel);
      const int lim =
          min(max((int)t_r[rt] - c * kBlock, -1), kBlock);
      const int limq = lim - 4 * q;
      const bool causal = __ballot(sel && lim < kBlock - 1) != 0;
      float p[4][16];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 sv = T::s_tile(&ks[(32 * kt + n32) * kKRow], qop, q);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sel ? sv[r] : -INFINITY;
          if (causal) {
            x = 32 * kt + 8 * (r >> 2) + (r & 3) <= limq ? x : -INFINITY;
          }
          p[kt][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_r[rt], mx * qk_scale);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_r[rt] - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ev = m_new == -INFINITY ? 0.f : fast_exp2(fmaf(p[kt][r], qk_scale, -m_new));
          p[kt][r] = ev;
          lsum += ev;
        }
      lsum += __shfl_xor(lsum, 32, 64);
      l_r[rt] = l_r[rt] * alpha + lsum;
      m_r[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rt][dt][r] *= alpha;
      typename T::pop_t pb[T::kPChunks];
      T::pack_p(pb, p);
      T::pv(o[rt], pb, vt, lane);
    } while (false);
    if (next) {
      if constexpr (kBufs == 2) {
        st.store(Ks[buf ^ 1], Vt[buf ^ 1], tid);
      } else {
        __syncthreads();
        st.load(K, V, g, sl[j + 1], seq_len, tid);
        st.store(Ks[0], Vt[0], tid);
      }
    }
    __syncthreads();
  }

  // Fold in the rare entries' partials (slot order), then normalise and store.
  {
    const int64_t irow = i0 + (ok_r[rt] ? tok_r[rt] : 0);
    const int32_t* tl = block_idx + (irow * G + g) * top_k;
    const int b = (int)(t_r[rt] / kBlock);
    for (int s2 = 0; s2 < top_k; ++s2) {
      const int c = ok_r[rt] ? tl[s2] : -1;
      bool rare = c >= 0 && c <= b;
      if (rare)
        for (int j = 0; j < ns; ++j)
          if (sl[j] == c) rare = false;
      if (__ballot(rare) == 0) continue;
      if (rare) {
        const int64_t prow = ((irow * G + g) * top_k + s2) * Hpg + h;
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + prow * 2);
        const float M = fmaxf(m_r[rt], ml.x);
        const float a = m_r[rt] == -INFINITY ? 0.f : fast_exp2(m_r[rt] - M);
        const float wgt = ml.y * fast_exp2(ml.x - M);
        const elem* src = part_o + prow * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float v4[4];
            const elem* sp = src + frag_pos(dt, jj, q);
            if constexpr (E::is_bf16) {
              const u32x2 w2 = *reinterpret_cast<const u32x2*>(sp);
              v4[0] = bf16_bits_to_f32(w2[0] & 0xffffu);
              v4[1] = bf16_bits_to_f32(w2[0] >> 16);
              v4[2] = bf16_bits_to_f32(w2[1] & 0xffffu);
              v4[3] = bf16_bits_to_f32(w2[1] >> 16);
            } else {
              const f32x4 w4 = *reinterpret_cast<const f32x4*>(sp);
              v4[0] = w4[0];
              v4[1] = w4[1];
              v4[2] = w4[2];
              v4[3] = w4[3];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) o[rt][dt][4 * jj + r] = o[rt][dt][4 * jj + r] * a + wgt * v4[r];
          }
        l_r[rt] = l_r[rt] * a + wgt;
        m_r[rt] = M;
      }
    }
    if (ok_r[rt]) {
      const float inv = l_r[rt] > 0.f ? 1.f / l_r[rt] : 0.f;
      if (lse != nullptr && q == 0)
        lse[t_r[rt] * Hq + (int64_t)g * Hpg + h] =
            l_r[rt] > 0.f ? (m_r[rt] + log2f(l_r[rt])) * kLn2 : -INFINITY;
      elem* dst = out + (t_r[rt] * Hq + (int64_t)g * Hpg + h) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          T::store4(dst + 32 * dt + 8 * jj + 4 * q, o[rt][dt][4 * jj] * inv,
                    o[rt][dt][4 * jj + 1] * inv, o[rt][dt][4 * jj + 2] * inv,
                    o[rt][dt][4 * jj + 3] * inv);
    }
  }
}

// ---- query-tile attention over the shared blocks, folding in the rare partials ------------
// One workgroup (8 waves) per (query tile, group); wave w owns row tile w.
// For each shared block of the tile (staged once in LDS, the next one loaded while the
// current is used) every row runs an online softmax step - rows whose token did not keep
// the block are masked, the local block gets the causal mask. Then each row folds in
// the partials (o / l, m, l) of its rare entries, computed by the reverse-index path, in
// slot order, and the final output is written. No partial is stored for shared entries.
// bf16 form: 8 waves with one row tile each (a query tile is 8 row tiles), one workgroup
// per CU with the shared blocks double-buffered in LDS: block j + 1 is loaded (K and V
// row-major, by direct global->LDS loads) while block j is used; PV reads V through the
// LDS transpose read. Q stays in registers across the shared blocks. A block's four S
// tiles and their maximum come first; a row's running maximum is raised only when that
// block maximum exceeds it by more than 8 (log2 units), so the accumulator is rescaled
// rarely and every exponential stays below 2^8; the final division by the row sum makes the
// result the same up to rounding. A block every row of a wave sees whole skips the per-score
// mask. The tile's kept entries are classified by all threads at once (LDS atomic ORs into
// per-token masks), and each lane folds in its own rare partials through buffer views,
// before the shared blocks, in one online pass with the same lazy maximum: their loads
// overlap the first block's staging.
// Launch bounds (512, 2): at least two waves per SIMD, i.e. 256 registers a lane; the 135 KiB
// of LDS let one workgroup occupy a CU.
template <int KMAX>
__global__ __launch_bounds__(512, 2) void qtile_attn_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ shared, const uint16_t* __restrict__ part_o,
    const float* __restrict__ part_ml, uint16_t* __restrict__ out, float* __restrict__ lse,
    int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count, int64_t seq_len) {
  typedef TileOps<BF16> T;
  // two buffers per operand: block j + 1 is staged while block j is read (the block loop is
  // unrolled by two, so every access names its buffer)
  __shared__ __align__(16) uint8_t Kb0[kBlock * 256];
  __shared__ __align__(16) uint8_t Kb1[kBlock * 256];
  __shared__ __align__(16) uint8_t Vb0[kBlock * 256];
  __shared__ __align__(16) uint8_t Vb1[kBlock * 256];
  __shared__ int32_t sl[64];
  __shared__ unsigned long long selmask[256];   // per token: which shared blocks it keeps
  __shared__ unsigned long long raremask[256];  // per token: which slots go through the partials

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int epr = 32 / Hpg;
  const int QT = 8 * epr;
  const int64_t tile = blockIdx.x / G;
  const int g = (int)(blockIdx.x % G);
  const int64_t i0 = tile * QT;
  const int ntok = (int)min((int64_t)QT, q_count - i0);
  const int Hq = G * Hpg;
  // The loads that depend only on the launch go out together and share one round trip: the
  // tile's shared list (ascending, -1 padded; each wave counts it from one load per lane),
  // this thread's first kept entry id and the lane's query row. The barriers below wait for
  // LDS only, so the query rows stay in flight across them. Every load is unconditional
  // (clamped indexes, results selected afterwards): loads behind lane conditions would leave
  // the compiler unable to count them, and it would then wait for all of them at the first
  // use of any.
  const int slv_raw = shared[(tile * G + g) * top_k + min(lane, top_k - 1)];
  const int ne = ntok * top_k;
  const int en0 = min(tid, ne - 1);
  const int c_first = block_idx[((i0 + en0 / top_k) * G + g) * top_k + en0 % top_k];
  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const int n32 = lane & 31, q = lane >> 5;
  const int e = n32 / Hpg;
  const int h = n32 - e * Hpg;
  const int tok = wave * epr + e;
  const bool ok = e < epr && tok < ntok;
  const int64_t irow = i0 + (ok ? tok : 0);
  const int64_t t = q_begin + irow;
  const int tq = (int)t;
  // a lane without a token reads its tile's first row: its results are never stored
  T::qop_t qop[T::kQSteps];
  T::load_q(qop, Q + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, true);
  const int slv = lane < top_k ? slv_raw : -1;
  const int ns = __popcll(__ballot(slv >= 0));
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // the first shared block (lane 0's list entry) is staged while the masks are built
  if (ns > 0) {
    const int c0 = __builtin_amdgcn_readfirstlane(slv);
    k_block_dma_asm<512>(K, g, c0, seq_len, Kb0, wv, dma_lane_off<false>(lane), tid);
    k_block_dma_asm<512, true>(V, g, c0, seq_len, Vb0, wv, dma_lane_off<true>(lane), tid);
  }
  if (tid < 64) sl[tid] = slv;  // -1 past the list
  if (tid < QT) {
    selmask[tid] = 0ull;
    raremask[tid] = 0ull;
  }
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    MSA_WAIT_VMCNT_LDS(63);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  lds_barrier();
  // Per token: bit j of selmask = it keeps shared block j, bit s of raremask = its slot s
  // is visible and not shared. One thread per kept entry (coalesced id loads).
  auto mark = [&](int en, int c) __attribute__((always_inline)) {
    const int tk = en / top_k;
    const int s2 = en - tk * top_k;
    const int b = (int)((q_begin + i0 + tk) / kBlock);
    if (c < 0 || c > b) return;
    int jm = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) jm = sl[j] == c ? j : jm;  // c >= 0 never meets the -1s
    if (jm >= 0)
      atomicOr(&selmask[tk], 1ull << jm);
    else
      atomicOr(&raremask[tk], 1ull << s2);
  };
  if (tid < ne) mark(tid, c_first);
  for (int en = tid + 512; en < ne; en += 512) mark(en, block_idx[((i0 + en / top_k) * G + g) * top_k + en % top_k]);
  lds_barrier();
  const uint64_t mymask = ok ? selmask[tok] : 0ull;
  const uint64_t myrare = ok ? raremask[tok] : 0ull;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4] = {};

  // Rare partials first, while the first shared block is being staged: one pass reads each
  // rare slot's (m, l) and partial (lane-interleaved entry blocks, as the tile kernel wrote
  // them: each load instruction covers whole cache lines) and merges it into the row's
  // online softmax, which the shared blocks then continue. Each lane walks only its own
  // rare slots, in slot order, so a wave iterates as often as its busiest token has rare
  // slots. The partials are read through buffer views of the tile's entries (group g, 32-bit
  // offsets); a lane with no slot left reads past the bound and gets zeros, so no load
  // sits behind a branch.
  if (__ballot(myrare != 0)) {
    const int64_t ebase = (i0 * G + g) * top_k;
    const uint32_t span = (uint32_t)((int64_t)(ntok - 1) * G * top_k + top_k);  // < 2^20
    const __amdgpu_buffer_rsrc_t v_ml = buffer_view(part_ml + ebase * Hpg * 2, span * Hpg * 8);
    const __amdgpu_buffer_rsrc_t v_o =
        buffer_view(part_o + ebase * Hpg * kHeadDim, span * Hpg * kHeadDim * 2);
    const uint32_t tok_e = (uint32_t)((ok ? tok : 0) * G * top_k);
    // slots whose (m, l) and partial loads are issued together
    constexpr int kPartPer = 3;
    const uint32_t lane_b = (uint32_t)(8 * (h + Hpg * q)) * 2;
    for (uint64_t rem = myrare; __ballot(rem != 0);) {
      float2 ml[kPartPer];
      u32x4 w4[kPartPer][8];
      bool hs[kPartPer];
#pragma unroll
      for (int k2 = 0; k2 < kPartPer; ++k2) {
        hs[k2] = rem != 0;
        const uint32_t ent = tok_e + (uint32_t)__builtin_ctzll(rem | (1ull << 63));
        rem &= rem - 1ull;
        ml[k2] = __builtin_bit_cast(
            float2, __builtin_amdgcn_raw_buffer_load_b64(
                        v_ml, hs[k2] ? (ent * Hpg + h) * 8 : kBufNone, 0, 0));
        const uint32_t ob = hs[k2] ? ent * Hpg * kHeadDim * 2 + lane_b : kBufNone;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w4[k2][i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(v_o, ob + i * 32 * Hpg, 0, 0));
      }
      // online merge with the lazy maximum of the block loop: the running maximum (-inf
      // before the lane's first slot) is raised only when a partial's maximum exceeds it by
      // more than 8, so every weight below stays under 2^8 times its l
      float mr = -INFINITY;
#pragma unroll
      for (int k2 = 0; k2 < kPartPer; ++k2) mr = hs[k2] ? fmaxf(mr, ml[k2].x) : mr;
      const bool raise = mr > m_run + 8.f;
      if (__ballot(raise)) {
        const float alpha = raise ? (m_run == -INFINITY ? 0.f : fast_exp2(m_run - mr)) : 1.f;
        m_run = raise ? mr : m_run;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
#pragma unroll
      for (int k2 = 0; k2 < kPartPer; ++k2) {
        const float w = hs[k2] ? ml[k2].y * fast_exp2(ml[k2].x - m_run) : 0.f;
        l_run += w;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j2 = 0; j2 < 8; ++j2) {
            const uint32_t bits =
                j2 & 1 ? w4[k2][i][j2 >> 1] >> 16 : w4[k2][i][j2 >> 1] & 0xffffu;
            const int r = 4 * (2 * (i & 1) + (j2 >> 2)) + (j2 & 3);
            o[i >> 1][r] = fmaf(w, bf16_bits_to_f32(bits), o[i >> 1][r]);
          }
      }
    }
  }
  auto shared_block = [&](int j, const uint8_t* Kc, const uint8_t* Vc, uint8_t* Kn, uint8_t* Vn) {
    const int c = __builtin_amdgcn_readfirstlane(sl[j]);  // uniform: scalar staging base
    // block j (loaded during block j - 1) has landed for every wave, and every wave is
    // done with block j - 1, whose buffer now takes block j + 1
    MSA_WAIT_VMCNT(0);
    __syncthreads();
    // lane-derived addresses are recomputed per block rather than kept live (the empty
    // asm hides that the thread id does not change)
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int lane_v = tid_v & 63;
    const int n32v = lane_v & 31, qv = lane_v >> 5;
    if (j + 1 < ns) {
      const int cn = __builtin_amdgcn_readfirstlane(sl[j + 1]);
      k_block_dma_asm<512>(K, g, cn, seq_len, Kn, wv, dma_lane_off<false>(lane_v), tid_v);
      k_block_dma_asm<512, true>(V, g, cn, seq_len, Vn, wv, dma_lane_off<true>(lane_v), tid_v);
    }
    const bool sel = (mymask >> j) & 1ull;
    if (__ballot(sel) == 0) return;
    // A row that did not keep the block (or has no token) joins the products but takes the
    // exponent offset -inf: its probabilities are all 0 and its maximum is ignored, with no
    // mask on its single scores. Only a block that reaches past a keeping row's own position
    // (the causal block of the query tile) masks single scores: one uniform test per block.
    // lim: last visible key offset in the block (int32: t < 2^31).
    const int lim = min(max(tq - c * kBlock, -1), kBlock - 1);
    const bool masked = __ballot(sel && lim < kBlock - 1) != 0;
    int limq = lim - 4 * qv;  // the lane's key offset 4q folded into the limit
    asm volatile("" : "+v"(limq));
    // the block's 128 keys: all four S^T tiles and their maximum first (one test of the lazy
    // maximum per block), then per 64-key half the exponentials, which the compiler can
    // interleave with the other half's PV products
    float p[4][16];
    float mx = -INFINITY;
    f32x16 acc4[4];
    s_tiles4_swz(Kc, n32v, qop, qv, acc4);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const f32x16 sv = acc4[kt];
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          p[kt][r] = 32 * kt + 8 * (r >> 2) + (r & 3) <= limq ? sv[r] : -INFINITY;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kt][r] = sv[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, p[kt][r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mxs = mx * qk_scale;
    const bool raise = sel && mxs > m_run + 8.f;
    if (__ballot(raise)) {
      const float alpha = raise ? fast_exp2(m_run - mxs) : 1.f;
      m_run = raise ? mxs : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    // masked scores and rows that skip the block give exp2(-inf) = 0
    const float mneg = !sel ? -INFINITY : m_run == -INFINITY ? 0.f : -m_run;
    float lsum = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 pb[4];
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        float* pr = p[2 * half + kk2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = fast_exp2(fmaf(pr[r], qk_scale, mneg));
          lsum += pr[r];
        }
        pb[2 * kk2] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                            pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
        pb[2 * kk2 + 1] = u32x4{pack_bf16x2(pr[8], pr[9]), pack_bf16x2(pr[10], pr[11]),
                                pack_bf16x2(pr[12], pr[13]), pack_bf16x2(pr[14], pr[15])};
      }
      pv_half_tr(o, pb, Vc, lane_v, half);
    }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run += lsum;
  };
#pragma unroll
  for (int s2 = 0; s2 < T::kQSteps; ++s2) asm volatile("" ::"v"(qop[s2]));
  for (int j = 0; j < ns; j += 2) {
    shared_block(j, Kb0, Vb0, Kb1, Vb1);
    if (j + 1 < ns) shared_block(j + 1, Kb1, Vb1, Kb0, Vb0);
  }
  MSA_WAIT_VMCNT(0);

  if (ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (lse != nullptr && q == 0)
      lse[t * Hq + (int64_t)g * Hpg + h] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    uint16_t* dst = out + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        T::store4(dst + 32 * dt + 8 * jj + 4 * q, o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv,
                  o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
  }
}

// ---- dense causal GQA prefill, bf16 (the dense baseline the sparse path is compared with) --
// Flash-style: one workgroup per (query tile of 4 row tiles, group); every visible block is
// streamed through LDS (K and V by direct global->LDS loads, PV through transpose reads),
// each row keeps an online softmax with the lazily raised maximum of the query-tile
// kernel, and the output is written once at the end. The latest (heaviest) tiles start
// first; two workgroups share a CU.
__global__ __launch_bounds__(256, 2) void dense_attn_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ out, int G, int Hpg,
    int64_t q_begin, int64_t q_count, int64_t seq_len) {
  typedef TileOps<BF16> T;
  __shared__ __align__(16) uint8_t Kb[kBlock * 256];
  __shared__ __align__(16) uint8_t Vb[kBlock * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int epr = 32 / Hpg;
  const int QT = 4 * epr;
  const int64_t ntiles = (q_count + QT - 1) / QT;
  const int64_t tile = ntiles - 1 - (int64_t)(blockIdx.x / G);
  const int g = (int)(blockIdx.x % G);
  const int64_t i0 = tile * QT;
  const int ntok = (int)min((int64_t)QT, q_count - i0);
  const int Hq = G * Hpg;
  const float qk_scale = kLog2e / sqrtf((float)kHeadDim);
  const int n32 = lane & 31, q = lane >> 5;
  const int e = n32 / Hpg;
  const int h = n32 - e * Hpg;
  const int tok = wave * epr + e;
  const bool ok = e < epr && tok < ntok;
  const int64_t t = q_begin + i0 + (ok ? tok : 0);
  T::qop_t qop[T::kQSteps];
  T::load_q(qop, Q + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim, q, ok);
  const int nb = (int)((q_begin + i0 + ntok - 1) / kBlock) + 1;  // blocks 0 .. local of the last
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4] = {};

  for (int c = 0; c < nb; ++c) {
    if (c > 0) __syncthreads();  // every wave is done with the previous block
    int tid_v = tid;  // lane-derived addresses are recomputed per block, not kept live
    asm volatile("" : "+v"(tid_v));
    const int lane_v = tid_v & 63;
    const int n32v = lane_v & 31, qv = lane_v >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    k_block_dma_s<256>(K, g, c, seq_len, Kb, wv, dma_lane_off<false>(lane_v), tid_v);
    k_block_dma_s<256, true>(V, g, c, seq_len, Vb, wv, dma_lane_off<true>(lane_v), tid_v);
    MSA_WAIT_VMCNT(0);
    __syncthreads();
    const int lim = min(max((int)t - c * kBlock, -1), kBlock);
    int limq = lim - 4 * qv;
    asm volatile("" : "+v"(limq));
    const bool causal = __ballot(lim < kBlock - 1) != 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float p[2][16];
      float mx = -INFINITY;
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const int kt = 2 * half + kk2;
        const f32x16 sv = s_tile_swz(Kb, 32 * kt + n32v, qop, qv);
        // the compare and select only on the diagonal blocks
        if (causal) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[kk2][r] = 32 * kt + 8 * (r >> 2) + (r & 3) <= limq ? sv[r] : -INFINITY;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) p[kk2][r] = sv[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, p[kk2][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxs = mx * qk_scale;
      const bool raise = mxs > m_run + 8.f;  // key 0 of block 0 is visible to every row
      if (__ballot(raise)) {
        const float alpha = raise ? fast_exp2(m_run - mxs) : 1.f;
        m_run = raise ? mxs : m_run;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      float lsum = 0.f;
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ev = fast_exp2(fmaf(p[kk2][r], qk_scale, -m_run));
          p[kk2][r] = ev;
          lsum += ev;
        }
      lsum += __shfl_xor(lsum, 32, 64);
      l_run += lsum;
      u32x4 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pr = &p[u >> 1][8 * (u & 1)];
        pb[u] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
      }
      pv_half_tr(o, pb, Vb, lane_v, half);
    }
  }
  if (ok) {
    const float inv = 1.f / l_run;
    uint16_t* dst = out + (t * Hq + (int64_t)g * Hpg + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        T::store4(dst + 32 * dt + 8 * jj + 4 * q, o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv,
                  o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
  }
}

hipError_t launch_dense_prefill_bf16(const void* q, const void* k, const void* v, void* out, int G,
                                     int Hpg, int64_t q_begin, int64_t q_count, int64_t seq_len,
                                     hipStream_t st) {
  const int QT = 4 * (32 / Hpg);  // the dense kernel's query tile: 4 row tiles
  const int64_t ntiles = (q_count + QT - 1) / QT;
  hipLaunchKernelGGL(dense_attn_bf16_kernel, dim3((unsigned)(ntiles * G)), dim3(256), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out,
                     G, Hpg, q_begin, q_count, seq_len);
  return hipGetLastError();
}

// ---- host side -------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

void launch_exclusive_scan(int32_t* a, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(kv_scan_kernel, dim3(1), dim3(1024), 0, st, n, a);
}

void launch_reverse_index(const int32_t* block_idx, int64_t n_entries, int G, int top_k,
                          int64_t q_begin, int nblk, const int32_t* shared, int QT,
                          int32_t* count, int32_t* cursor, int32_t* offset, int32_t* sorted,
                          hipStream_t st) {
  const int64_t nb = (int64_t)G * nblk;
  const unsigned grid_e = (unsigned)std::min<int64_t>((n_entries + 255) / 256, 65536);
  const int64_t ncnt = nb * kStripes;
  hipLaunchKernelGGL(kv_zero_kernel, dim3((unsigned)std::min<int64_t>((ncnt + 255) / 256, 4096)),
                     dim3(256), 0, st, count, ncnt);
  // LDS-aggregated form: about 512 workgroups, each over a whole number of query tiles, as
  // long as the nblk counters and the chunk's shared lists fit in LDS
  const int64_t q_count = n_entries / ((int64_t)G * top_k);
  const int64_t per_g = std::max<int64_t>(1, 512 / G);
  int64_t rows = ((q_count + per_g - 1) / per_g + QT - 1) / QT * QT;
  if (shared != nullptr)
    rows = std::min<int64_t>(rows, std::max<int64_t>(1, 4096 / top_k) * QT);
  const int64_t ntl = shared != nullptr ? rows / QT : 0;
  const size_t lds = (size_t)(nblk + ntl * top_k) * 4;
  const bool lds_path = q_count > 0 && lds <= (size_t)kRiLdsBytes && rows < (int64_t(1) << 30);
  const int64_t nchunk = lds_path ? (q_count + rows - 1) / rows : 0;
  if (lds_path)
    hipLaunchKernelGGL(kv_index_lds_kernel<false>, dim3((unsigned)(nchunk * G)),
                       dim3(kRiThreads), lds, st, block_idx, q_count, G, top_k, q_begin, nblk,
                       shared, QT, (int)rows, count, nullptr);
  else
    hipLaunchKernelGGL(kv_count_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries, G,
                       top_k, q_begin, nblk, shared, QT, count);
  const unsigned grid_b = (unsigned)std::min<int64_t>((nb + 255) / 256, 65536);
  hipLaunchKernelGGL(kv_bucket_total_kernel, dim3(grid_b), dim3(256), 0, st, count, nb, offset);
  launch_exclusive_scan(offset, nb, st);
  hipLaunchKernelGGL(kv_cursor_kernel, dim3(grid_b), dim3(256), 0, st, count, nb, offset, cursor);
  if (lds_path)
    hipLaunchKernelGGL(kv_index_lds_kernel<true>, dim3((unsigned)(nchunk * G)),
                       dim3(kRiThreads), lds, st, block_idx, q_count, G, top_k, q_begin, nblk,
                       shared, QT, (int)rows, cursor, sorted);
  else
    hipLaunchKernelGGL(kv_scatter_kernel, dim3(grid_e), dim3(256), 0, st, block_idx, n_entries,
                       G, top_k, q_begin, nblk, shared, QT, cursor, sorted);
}

size_t kv_workspace_bytes(int bf16, int64_t q_count, int G, int Hpg, int top_k, int nblk) {
  const int64_t nb = (int64_t)G * nblk;
  const int64_t E = q_count * G * top_k;
  const size_t es = bf16 ? 2 : 4;
  const int64_t ntiles = (q_count + qtile_tokens(Hpg, bf16) - 1) / qtile_tokens(Hpg, bf16);
  return al256((size_t)ntiles * G * top_k * 4) +
         al256((size_t)nb * kStripes * 4) * 2 + al256((size_t)(nb + 1) * 4) +
         al256((size_t)E * 4) + al256((size_t)E * Hpg * 2 * 4) +
         al256((size_t)E * Hpg * kHeadDim * es);
}

template <class E>
static hipError_t launch_kv_t(const void* q, const void* k, const void* v,
                              const int32_t* block_idx, void* out, float* lse, void* ws, int G,
                              int Hpg,
                              int top_k, int64_t q_begin, int64_t q_count, int64_t seq_len,
                              int nblk, hipStream_t st) {
  typedef typename E::elem elem;
  const int64_t nb = (int64_t)G * nblk;
  const int64_t n_entries = q_count * G * top_k;
  const int QT = qtile_tokens(Hpg, E::is_bf16 ? 1 : 0);
  const int64_t ntiles = (q_count + QT - 1) / QT;
  char* w = static_cast<char*>(ws);
  int32_t* shared = reinterpret_cast<int32_t*>(w);
  w += al256((size_t)ntiles * G * top_k * 4);
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

  const int64_t npairs = ntiles * G;
  hipLaunchKernelGGL(kv_classify_kernel, dim3((unsigned)((npairs + 3) / 4)), dim3(256), 0, st,
                     block_idx, shared, G, top_k, q_begin, q_count, QT, npairs);
  launch_reverse_index(block_idx, n_entries, G, top_k, q_begin, nblk, shared, QT, count, cursor,
                       offset, sorted, st);
  const unsigned tiles = (unsigned)((n_entries + kKvTile - 1) / kKvTile);
  if constexpr (E::is_bf16)
    hipLaunchKernelGGL(kv_attn_bf16_kernel, dim3(tiles), dim3(256), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, block_idx, sorted, offset + nb,
                       (uint16_t*)part_o, part_ml, G, Hpg, top_k, q_begin, seq_len);
  else
    hipLaunchKernelGGL((kv_attn_kernel<E, kTileF32>), dim3((unsigned)((n_entries + kTileF32 - 1) / kTileF32)),
                       dim3(256), 0, st, (const elem*)q, (const elem*)k, (const elem*)v, block_idx,
                       sorted, offset + nb, part_o, part_ml, G, Hpg, top_k, q_begin, seq_len);
  if constexpr (E::is_bf16) {
    if (top_k <= 16)
      hipLaunchKernelGGL((qtile_attn_bf16_kernel<16>), dim3((unsigned)npairs), dim3(512), 0, st,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, block_idx,
                         shared, (const uint16_t*)part_o, part_ml, (uint16_t*)out, lse, G, Hpg,
                         top_k,
                         q_begin, q_count, seq_len);
    else
      hipLaunchKernelGGL((qtile_attn_bf16_kernel<64>), dim3((unsigned)npairs), dim3(512), 0, st,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, block_idx,
                         shared, (const uint16_t*)part_o, part_ml, (uint16_t*)out, lse, G, Hpg,
                         top_k,
                         q_begin, q_count, seq_len);
  }
  if constexpr (!E::is_bf16)
    hipLaunchKernelGGL((qtile_attn_kernel<E, kQtileWavesF32>), dim3((unsigned)npairs),
                       dim3(64 * kQtileWavesF32), 0, st,
                       (const elem*)q, (const elem*)k, (const elem*)v, block_idx, shared,
                       (const elem*)part_o, part_ml, (elem*)out, lse, G, Hpg, top_k, q_begin,
                       q_count, seq_len);
  return hipGetLastError();
}

hipError_t launch_kv_prefill(int bf16, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, void* out, float* lse, void* workspace,
                             int G, int Hpg, int top_k, int64_t q_begin, int64_t q_count,
                             int64_t seq_len, int nblk, hipStream_t stream) {
  if (bf16)
    return launch_kv_t<BF16>(q, k, v, block_idx, out, lse, workspace, G, Hpg, top_k, q_begin,
                             q_count, seq_len, nblk, stream);
  return launch_kv_t<F32>(q, k, v, block_idx, out, lse, workspace, G, Hpg, top_k, q_begin,
                          q_count, seq_len, nblk, stream);
}

}  // namespace msa
