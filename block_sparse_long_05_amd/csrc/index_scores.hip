// Index branch of MSA: token scores Q_idx . K_idx^T fused with 128-token block max
// pooling (mlqm.cn blog on the MiniMax M3 sparse attention, section 2.1: one index
// query per GQA group, one shared index-key head, block max pooling).
//
// Prefill kernel: the index queries of all groups form one [rows = tokens*G, d] matrix
// and each workgroup owns 256 consecutive rows. It sweeps the key blocks
// 0..b-1 (b = local block of its last row) in order; each block of index keys is
// staged once in LDS (double-buffered) and shared by the 4 waves. The MFMA is
// oriented as S^T = K_idx . Q_idx^T so that the 32 keys of a tile sit in the
// accumulator registers of each lane (lane = query row): the block max is an
// in-lane max plus one cross-half exchange, and only the block maxima are written.
//
// Decode kernel: streams k_idx[b] once at HBM rate. Each wave scores whole 128-key
// blocks for up to 16 groups at a time on 16x16 MFMAs, K operands loaded straight
// from global memory into registers (16 B per lane, all 32 loads of a block issued
// before the first MFMA).
#include <algorithm>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

template <class E>
struct Operand;
template <>
struct Operand<BF16> {
  typedef u32x4 type;
  static __device__ __forceinline__ type load(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ type zero() { return u32x4{0u, 0u, 0u, 0u}; }
};
template <>
struct Operand<F32> {
  typedef float type;
  static __device__ __forceinline__ type load(const float* p) { return *p; }
  static __device__ __forceinline__ type zero() { return 0.f; }
};

// ------------------------------------------------------------------------------------
// Prefill
// ------------------------------------------------------------------------------------
template <class E, int DI>
struct PrefillCfg {
  typedef typename E::elem elem;
  static constexpr int kPad = E::is_bf16 ? 8 : 1;    // LDS row padding (elements)
  static constexpr int kRow = DI + kPad;             // LDS row stride (elements)
  static constexpr int kBuf = kBlock * kRow;         // one staged key block
  static constexpr int kStep = 2 * E::kPerLane;      // dims per 32x32 MFMA k-step
  static constexpr int kNStep = DI / kStep;
  static constexpr int kChunkElems = 16 / sizeof(elem);
  static constexpr int kChunks = kBlock * DI / kChunkElems;  // 16-byte chunks per block
  static constexpr int kChunksPerThread = kChunks / 256;
};

template <class E, int DI>
__global__ __launch_bounds__(256, 2) void index_scores_prefill_kernel(
    const typename E::elem* __restrict__ q_idx, const typename E::elem* __restrict__ k_idx,
    float* __restrict__ block_scores, int64_t q_begin, int64_t q_count, int G, int top_k,
    int nblk) {
  typedef PrefillCfg<E, DI> C;
  typedef typename E::elem elem;
  typedef typename Operand<E>::type op_t;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  elem* lds = reinterpret_cast<elem*>(smem_raw);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nrows = q_count * G;
  // Heaviest (latest) rows first: causal work grows with the row's position.
  const int64_t r0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * 256;
  const int64_t r_last = min(r0 + 255, nrows - 1);
  const int cmax_rows = (int)((q_begin + r_last / G) / kBlock);
  if (cmax_rows < top_k) return;  // every row keeps all its visible blocks: nothing to score
  // this workgroup's key blocks: chunk blockIdx.y of gridDim.y (block scores are independent,
  // so small problems spread a row tile's blocks over several workgroups)
  const int per = (cmax_rows + (int)gridDim.y - 1) / (int)gridDim.y;
  const int c_lo = (int)blockIdx.y * per;
  const int cmax = min(cmax_rows, c_lo + per);
  if (c_lo >= cmax) return;

  // This lane's B operands (index query rows), two 32-row tiles per wave.
  op_t qop[2][C::kNStep];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t R = r0 + 64 * wave + 32 * rt + (lane & 31);
    const bool ok = R < nrows;
    const elem* qp = q_idx + (q_begin * G + (ok ? R : 0)) * DI + (lane >> 5) * E::kPerLane;
#pragma unroll
    for (int s = 0; s < C::kNStep; ++s)
      qop[rt][s] = ok ? Operand<E>::load(qp + s * C::kStep) : Operand<E>::zero();
  }
  // The row this lane writes: lanes 0-31 tile 0, lanes 32-63 tile 1.
  const int64_t Rw = r0 + 64 * wave + lane;
  int bw = -1;
  if (Rw < nrows) bw = (int)((q_begin + Rw / G) / kBlock);
  const bool writes = bw >= top_k;
  float* out_row = block_scores + (Rw < nrows ? Rw : 0) * (int64_t)nblk;

  // Staging of one key block: thread-strided 16-byte chunks.
  u32x4 stage[C::kChunksPerThread];
  auto load_block = [&](int c) {
    const elem* src = k_idx + (int64_t)c * kBlock * DI;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int ch = threadIdx.x + 256 * i;
      stage[i] = *reinterpret_cast<const u32x4*>(src + ch * C::kChunkElems);
    }
  };
  auto store_block = [&](int buf) {
    elem* dst = lds + buf * C::kBuf;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int ch = threadIdx.x + 256 * i;
      const int row = ch / (DI / C::kChunkElems);
      const int col = (ch % (DI / C::kChunkElems)) * C::kChunkElems;
      if constexpr (E::is_bf16) {
        *reinterpret_cast<u32x4*>(dst + row * C::kRow + col) = stage[i];
      } else {
        float* d = reinterpret_cast<float*>(dst) + row * C::kRow + col;
        d[0] = __uint_as_float(stage[i][0]);
        d[1] = __uint_as_float(stage[i][1]);
        d[2] = __uint_as_float(stage[i][2]);
        d[3] = __uint_as_float(stage[i][3]);
      }
    }
  };

  load_block(c_lo);
  store_block(c_lo & 1);
  __syncthreads();
  for (int c = c_lo; c < cmax; ++c) {
    const bool has_next = c + 1 < cmax;
    if (has_next) load_block(c + 1);
    const elem* kb = lds + (c & 1) * C::kBuf + (lane & 31) * C::kRow + (lane >> 5) * E::kPerLane;
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; kt += 2) {
      f32x16 a00 = {}, a01 = {}, a10 = {}, a11 = {};
#pragma unroll
      for (int s = 0; s < C::kNStep; ++s) {
        const op_t ka = Operand<E>::load(kb + (kt * 32) * C::kRow + s * C::kStep);
        const op_t kc = Operand<E>::load(kb + (kt * 32 + 32) * C::kRow + s * C::kStep);
        a00 = mfma32(ka, qop[0][s], a00);
        a01 = mfma32(ka, qop[1][s], a01);
        a10 = mfma32(kc, qop[0][s], a10);
        a11 = mfma32(kc, qop[1][s], a11);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mx0 = fmaxf(mx0, fmaxf(a00[r], a10[r]));
        mx1 = fmaxf(mx1, fmaxf(a01[r], a11[r]));
      }
    }
    mx0 = fmaxf(mx0, __shfl_xor(mx0, 32, 64));
    mx1 = fmaxf(mx1, __shfl_xor(mx1, 32, 64));
    const float val = lane < 32 ? mx0 : mx1;
    if (writes && c < bw) out_row[c] = val;
    if (has_next) store_block((c + 1) & 1);
    __syncthreads();
  }
}

// Prefill, bf16: 4 waves x 128 index-query rows (4 row tiles of 32) per workgroup. The
// key block is staged by direct global->LDS loads into an unpadded, double-buffered
// LDS block whose 16-byte chunks are XOR-swizzled by row (position p of row r holds
// chunk p ^ (r % 16)): a quarter-wave loads one whole key row (coalesced) and the MFMA
// operand reads of 8 rows at a time fall in distinct banks. Each K operand read feeds
// the 4 row tiles. Block maxima are staged in LDS and written 8 blocks (32 contiguous bytes)
// per row.
template <int DI>
struct PrefillLds {
  static constexpr int kRowBytes = DI * 2;                 // one key row in LDS
  static constexpr int kChunks = DI / 8;                   // 16-byte chunks per row
  static constexpr int kBufBytes = kBlock * kRowBytes;     // one staged block
  static constexpr int kLoadsPerWave = kBufBytes / 1024 / 4;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one 1 KiB load covers
  static constexpr int kSteps = DI / 16;                   // 32x32x16 k-steps
};

template <int DI>
__device__ __forceinline__ void prefill_issue_block(const uint16_t* k_idx, int c, uint8_t* buf,
                                                    int wave, int lane) {
  typedef PrefillLds<DI> C;
  const uint16_t* src0 = k_idx + (int64_t)c * kBlock * DI;
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const int li = wave * C::kLoadsPerWave + i;            // 1 KiB load index in the block
    const int r = li * C::kRowsPerLoad + lane / C::kChunks;
    const int p = lane % C::kChunks;
    const int chunk = p ^ (r & (C::kChunks - 1));
    __builtin_amdgcn_global_load_lds((const void*)(src0 + (int64_t)r * DI + chunk * 8),
                                     (__attribute__((address_space(3))) void*)(buf + li * 1024),
                                     16, 0, 0);
  }
}

template <int DI>
__global__ __launch_bounds__(256, 2) void index_scores_prefill_lds_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    float* __restrict__ block_scores, int64_t q_begin, int64_t q_count, int G, int top_k,
    int nblk) {
  typedef PrefillLds<DI> C;
  constexpr int kBatch = 8;  // blocks whose maxima are written together (32 B per row)
  __shared__ __align__(16) uint8_t lds[2][C::kBufBytes];
  __shared__ __align__(16) float stage[4][128][kBatch];  // per wave: its rows x the batch
  constexpr int kRows = 512;  // rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nrows = q_count * G;
  const int64_t r0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * kRows;  // heaviest rows first
  const int64_t r_last = min(r0 + kRows - 1, nrows - 1);
  const int cmax = (int)((q_begin + r_last / G) / kBlock);
  if (cmax < top_k) return;

  // B operands: 4 row tiles of 32 rows; lane group q holds dims 16s + 8q .. +8.
  const int q = lane >> 5;
  u32x4 qop[4][C::kSteps];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t R = r0 + 128 * wave + 32 * rt + (lane & 31);
    const bool ok = R < nrows;
    const uint16_t* qp = q_idx + (q_begin * G + (ok ? R : 0)) * DI + 8 * q;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      qop[rt][s] = ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
  }
  const bool vec_ok = (nblk & 3) == 0;  // 16-byte row pieces of block_scores are aligned

  prefill_issue_block<DI>(k_idx, 0, lds[0], wave, lane);
  MSA_WAIT_VMCNT(0);
  __syncthreads();
  for (int cb = 0; cb < cmax; cb += kBatch) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = cb + j;
      if (c < cmax) {
        const bool has_next = c + 1 < cmax;
        if (has_next) prefill_issue_block<DI>(k_idx, c + 1, lds[(c + 1) & 1], wave, lane);
        const uint8_t* kb = lds[c & 1];
        float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int m = 32 * kt + (lane & 31);
          f32x16 acc[4] = {};
#pragma unroll
          for (int s = 0; s < C::kSteps; ++s) {
            const int pos = (2 * s + q) ^ (m & (C::kChunks - 1));
            const u32x4 a = *reinterpret_cast<const u32x4*>(kb + m * C::kRowBytes + pos * 16);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma32(a, qop[rt][s], acc[rt]);
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx[rt] = fmaxf(mx[rt], fmaxf(acc[rt][r], acc[rt][r + 1]));
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mx[rt] = fmaxf(mx[rt], __shfl_xor(mx[rt], 32, 64));
        // tiles 2q and 2q + 1 go to the stage from this half (column lane % 32)
        stage[wave][32 * (2 * q) + (lane & 31)][j] = q == 0 ? mx[0] : mx[2];
        stage[wave][32 * (2 * q + 1) + (lane & 31)][j] = q == 0 ? mx[1] : mx[3];
        if (has_next) MSA_WAIT_VMCNT(0);  // this wave's part of block c + 1 has landed
        __syncthreads();
      }
    }
    // The wave's 128 rows x kBatch maxima leave as 16-byte pieces (4 per lane), each row's
    // run contiguous; only blocks c < b(row) (and c < cmax) are written, and nothing for
    // rows that keep all their blocks.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int piece = 64 * it + lane;
      const int row = piece >> 1, hf = piece & 1;
      const int64_t R = r0 + 128 * wave + row;
      int lim = R < nrows ? (int)((q_begin + R / G) / kBlock) : 0;
      if (lim < top_k) lim = 0;
      lim = min(lim, cmax);
      const float4 v = *reinterpret_cast<const float4*>(&stage[wave][row][4 * hf]);
      const int c0 = cb + 4 * hf;
      float* dst = block_scores + (R < nrows ? R : 0) * (int64_t)nblk + c0;
      if (vec_ok && c0 + 3 < lim) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        if (c0 + 0 < lim) dst[0] = v.x;
        if (c0 + 1 < lim) dst[1] = v.y;
        if (c0 + 2 < lim) dst[2] = v.z;
        if (c0 + 3 < lim) dst[3] = v.w;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the stage reads are done before it is reused
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------------------------
// Fused index -> top-k (prefill, bf16, top_k <= 16)
// ------------------------------------------------------------------------------------
// The sweep of the prefill index kernel with 2 row tiles per wave, so that after the block
// maximum each lane owns one query row (row tile q, column lane % 32). The row keeps its
// running top-15 (order-preserving key, block id) sorted in registers, key descending and
// equal keys in arrival order, i.e. ascending id: a block enters only when its key beats
// the 15th strictly, since an equal key arrived earlier with a lower id and wins the tie.
// A row's top-(k-1) is contained in its top-15, so the first k-1 entries are its choice
// (researchpapers.dev summary "Mechanism"; mlqm.cn blog section 2.1). At the end the local
// block joins and the ids are written ascending. No block score reaches memory.
constexpr int kFuseK = 15;

template <int DI>
__global__ __launch_bounds__(256, 2) void index_topk_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    int32_t* __restrict__ block_idx, int64_t q_begin, int64_t q_count, int G, int top_k) {
  typedef PrefillLds<DI> C;
  constexpr int RT = 2;
  constexpr int kRows = 128 * RT;  // rows per workgroup
  __shared__ __align__(16) uint8_t lds0[C::kBufBytes];
  __shared__ __align__(16) uint8_t lds1[C::kBufBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 5;
  const int64_t nrows = q_count * G;
  const int64_t r0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * kRows;  // heaviest rows first
  const int64_t r_last = min(r0 + kRows - 1, nrows - 1);
  const int cmax = (int)((q_begin + r_last / G) / kBlock);  // blocks swept: 0 .. cmax - 1
  const int64_t R = r0 + 32 * RT * wave + 32 * q + (lane & 31);   // this lane's row
  const bool own = R < nrows;
  const int b = own ? (int)((q_begin + R / G) / kBlock) : 0;     // its local block

  uint32_t tk[kFuseK];
  int32_t ti[kFuseK];
#pragma unroll
  for (int i = 0; i < kFuseK; ++i) {
    tk[i] = 0u;  // below the key of every finite float
    ti[i] = -1;
  }
  if (cmax >= top_k && top_k > 1) {  // some row of the workgroup ranks blocks
    u32x4 qop[RT][C::kSteps];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t Rq = r0 + 32 * RT * wave + 32 * rt + (lane & 31);
      const bool ok = Rq < nrows;
      const uint16_t* qp = q_idx + (q_begin * G + (ok ? Rq : 0)) * DI + 8 * q;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s)
        qop[rt][s] = ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
    }
    prefill_issue_block<DI>(k_idx, 0, lds0, wave, lane);
    MSA_WAIT_VMCNT(0);
    __syncthreads();
    // unrolled by two so that every access names its buffer: the loads of block c + 1
    // then provably do not alias the reads of block c
    auto block = [&](int c, const uint8_t* cbuf, uint8_t* nbuf) {
      const bool has_next = c + 1 < cmax;
      if (has_next) prefill_issue_block<DI>(k_idx, c + 1, nbuf, wave, lane);
      const uint8_t* kb = cbuf;
      float mx[RT] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int m = 32 * kt + (lane & 31);
        f32x16 acc[RT] = {};
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
          const int pos = (2 * s + q) ^ (m & (C::kChunks - 1));
          const u32x4 a = *reinterpret_cast<const u32x4*>(kb + m * C::kRowBytes + pos * 16);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32(a, qop[rt][s], acc[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx[rt] = fmaxf(mx[rt], fmaxf(acc[rt][r], acc[rt][r + 1]));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) mx[rt] = fmaxf(mx[rt], __shfl_xor(mx[rt], 32, 64));
      const uint32_t key = ordered_key(q == 0 ? mx[0] : mx[1]);
      if (c < b && key > tk[kFuseK - 1]) {
        // sorted insert (old values are read before they are overwritten: i descends)
#pragma unroll
        for (int i = kFuseK - 1; i > 0; --i) {
          const bool up = key > tk[i - 1];
          const bool at = key > tk[i];
          tk[i] = up ? tk[i - 1] : (at ? key : tk[i]);
          ti[i] = up ? ti[i - 1] : (at ? c : ti[i]);
        }
        if (key > tk[0]) {
          tk[0] = key;
          ti[0] = c;
        }
      }
      if (has_next) MSA_WAIT_VMCNT(0);  // this wave's part of block c + 1 has landed
      __syncthreads();
    };
    for (int c = 0; c < cmax; c += 2) {
      block(c, lds0, lds1);
      if (c + 1 < cmax) block(c + 1, lds1, lds0);
    }
  }
  if (!own) return;
  int32_t* o = block_idx + R * top_k;
  if (b + 1 <= top_k) {  // every visible block is kept
    for (int i = 0; i < top_k; ++i) o[i] = i <= b ? i : -1;
    return;
  }
  // the first K = top_k - 1 entries, ascending (odd-even transposition sort), then b
  const int K = top_k - 1;
  int32_t sel[kFuseK];
#pragma unroll
  for (int i = 0; i < kFuseK; ++i) sel[i] = i < K ? ti[i] : 0x7fffffff;
#pragma unroll
  for (int round = 0; round < kFuseK; ++round)
#pragma unroll
    for (int i = round & 1; i + 1 < kFuseK; i += 2) {
      const int32_t lo = min(sel[i], sel[i + 1]), hi = max(sel[i], sel[i + 1]);
      sel[i] = lo;
      sel[i + 1] = hi;
    }
  for (int i = 0; i < K; ++i) o[i] = sel[i];
  o[K] = b;
}

hipError_t launch_index_topk_prefill(int index_dim, const void* q_idx, const void* k_idx,
                                     int32_t* block_idx, int64_t q_begin, int64_t q_count, int G,
                                     int top_k, hipStream_t st) {
  const int64_t grid = (q_count * G + 255) / 256;
  if (index_dim == 128)
    hipLaunchKernelGGL(index_topk_prefill_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st,
                       (const uint16_t*)q_idx, (const uint16_t*)k_idx, block_idx, q_begin,
                       q_count, G, top_k);
  else
    hipLaunchKernelGGL(index_topk_prefill_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st,
                       (const uint16_t*)q_idx, (const uint16_t*)k_idx, block_idx, q_begin,
                       q_count, G, top_k);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Decode
// ------------------------------------------------------------------------------------
template <class E, int DI>
__global__ __launch_bounds__(256) void index_scores_decode_kernel(
    const typename E::elem* __restrict__ q_idx, const typename E::elem* __restrict__ k_idx,
    float* __restrict__ block_scores, const int32_t* __restrict__ seq_lens, int64_t max_len,
    int G, int top_k, int nblk, int blocks_per_wg, PageMap pm) {
  typedef typename E::elem elem;
  typedef typename Operand<E>::type op_t;
  constexpr int kStep = 4 * E::kPerLane;  // dims per 16x16 MFMA k-step
  constexpr int kNStep = DI / kStep;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  int64_t L = seq_lens[b];
  L = L < 1 ? 1 : (L > max_len ? max_len : L);
  const int bl = (int)((L - 1) / kBlock);
  if (bl < top_k) return;
  const int c0 = blockIdx.x * blocks_per_wg;
  if (c0 >= bl) return;
  const int c1 = min(c0 + blocks_per_wg, bl);
  const elem* kbase = k_idx + (int64_t)b * max_len * DI;

  for (int g0 = 0; g0 < G; g0 += 16) {
    const int gq = g0 + (lane & 15);
    op_t qop[kNStep];
    {
      const bool ok = gq < G;
      const elem* qp = q_idx + ((int64_t)b * G + (ok ? gq : 0)) * DI + (lane >> 4) * E::kPerLane;
#pragma unroll
      for (int s = 0; s < kNStep; ++s)
        qop[s] = ok ? Operand<E>::load(qp + s * kStep) : Operand<E>::zero();
    }
    for (int c = c0 + wave; c < c1; c += 4) {
      const elem* kp = pm.block(k_idx, kbase, b, c, (int64_t)kBlock * DI) + (lane & 15) * DI +
                       (lane >> 4) * E::kPerLane;
      // bf16: the whole block's operands (32 x 16 B per lane) are in flight before the
      // first MFMA; fp32 (a correctness configuration) loads one 16-key tile at a time.
      constexpr int kGroup = E::is_bf16 ? 8 : 1;
      float mx = -INFINITY;
#pragma unroll
      for (int kg = 0; kg < 8; kg += kGroup) {
        op_t ka[kGroup][kNStep];
#pragma unroll
        for (int kt = 0; kt < kGroup; ++kt)
#pragma unroll
          for (int s = 0; s < kNStep; ++s)
            ka[kt][s] = Operand<E>::load(kp + (kg + kt) * 16 * DI + s * kStep);
#pragma unroll
        for (int kt = 0; kt < kGroup; ++kt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < kNStep; ++s) acc = mfma16(ka[kt][s], qop[s], acc);
          mx = fmaxf(mx, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 16 && gq < G) block_scores[((int64_t)b * G + gq) * nblk + c] = mx;
    }
  }
}

// Decode, bf16 with index dim 128 and up to 16 groups: each wave streams its blocks
// through a private ring of 2 LDS stages of 32 keys (8 KiB each) filled by direct
// global->LDS loads, one stage in flight while the other is consumed. With 64 KiB per
// workgroup two workgroups share a CU, which covers one's start and end with the other's
// stream (4 x 131072 keys: 25 -> 21 us; 8 x 1M stays at 311 us, 6.9 TB/s, with 2 to 5
// stages). A quarter-wave
// loads one whole 256-byte key row, so the reads are fully coalesced; the 16-byte
// chunks of row r are stored XOR-swizzled (position p holds chunk p ^ (r % 16)), so
// the MFMA operand reads - 16 rows, one chunk each per quarter-wave - fall in distinct
// LDS banks.
constexpr int kScanKeys = 32;                     // keys per stage
constexpr int kScanStage = kScanKeys * 256;       // bytes per stage (bf16, d = 128)
constexpr int kScanRing = 2;                      // stages per wave
constexpr int kScanLoads = kScanKeys / 4;         // 1 KiB loads per stage

__device__ __forceinline__ void scan_issue_stage(const uint16_t* rows, uint8_t* stage_lds,
                                                 int lane) {
  // load i covers key rows 4i .. 4i+3 of the stage
#pragma unroll
  for (int i = 0; i < kScanLoads; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int p = lane & 15;
    const int chunk = p ^ (r & 15);
    const uint16_t* src = rows + (int64_t)r * 128 + chunk * 8;
    __builtin_amdgcn_global_load_lds(
        (const void*)src, (__attribute__((address_space(3))) void*)(stage_lds + i * 1024), 16, 0,
        kLoadOnce);
  }
}


__global__ __launch_bounds__(256) void index_scores_decode_lds_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    float* __restrict__ block_scores, const int32_t* __restrict__ seq_lens, int64_t max_len,
    int G, int top_k, int nblk, int blocks_per_wg, PageMap pm) {
  __shared__ __align__(16) uint8_t lds[4][kScanRing][kScanStage];  // 64 KiB: two workgroups a CU
  constexpr int kPerBlock = kBlock / kScanKeys;                      // stages per block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  int64_t L = seq_lens[b];
  L = L < 1 ? 1 : (L > max_len ? max_len : L);
  const int bl = (int)((L - 1) / kBlock);
  if (bl < top_k) return;
  const int c0 = blockIdx.x * blocks_per_wg;
  if (c0 >= bl) return;
  const int c1 = min(c0 + blocks_per_wg, bl);
  const uint16_t* kbase = k_idx + (int64_t)b * max_len * 128;
  const int gq = lane & 15;
  const int q = lane >> 4;
  u32x4 qop[4];
  {
    const bool ok = gq < G;
    const uint16_t* qp = q_idx + ((int64_t)b * G + (ok ? gq : 0)) * 128 + 8 * q;
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = ok ? *reinterpret_cast<const u32x4*>(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
  }
  // This wave's blocks c0 + wave, c0 + wave + 4, ...: stages (block, quarter) in order.
  const int nb = (c1 - (c0 + wave) + 3) / 4;
  const int nstages = nb > 0 ? kPerBlock * nb : 0;
  // Paged caches: lane j holds the page of this wave's j-th block (at most 16 of them),
  // read once here. Looking the page up next to each block's loads would make the wait
  // for that lookup also wait for every stage already in flight.
  int my_page = 0;
  if (pm.table != nullptr && lane < nb) {
    int64_t pg = pm.table[(int64_t)b * pm.pps + c0 + wave + 4 * lane];
    my_page = (pg < 0 || pg >= pm.num_pages) ? 0 : (int)pg;
  }
  auto stage_rows = [&](int st) {
    const int j = st / kPerBlock;
    const uint16_t* blk =
        pm.table != nullptr
            ? k_idx + (int64_t)__builtin_amdgcn_readlane(my_page, j) * pm.page_elems
            : kbase + (int64_t)(c0 + wave + 4 * j) * (kBlock * 128);
    return blk + (st % kPerBlock) * kScanKeys * 128;
  };
  for (int st = 0; st < kScanRing - 1 && st < nstages; ++st)
    scan_issue_stage(stage_rows(st), lds[wave][st], lane);
  float mx = -INFINITY;
  for (int st = 0; st < nstages; ++st) {
    if (st + kScanRing - 1 < nstages)
      scan_issue_stage(stage_rows(st + kScanRing - 1), lds[wave][(st + kScanRing - 1) % kScanRing], lane);
    // stages issued after this one: min(3, nstages - 1 - st); wait until only those remain
    const int later = min(kScanRing - 1, nstages - 1 - st);
    if (later >= 3) MSA_WAIT_VMCNT(3 * kScanLoads);
    else if (later == 2) MSA_WAIT_VMCNT(2 * kScanLoads);
    else if (later == 1) MSA_WAIT_VMCNT(kScanLoads);
    else MSA_WAIT_VMCNT(0);
    __builtin_amdgcn_wave_barrier();
    const uint8_t* sl = lds[wave][st % kScanRing];
#pragma unroll
    for (int kt = 0; kt < kScanKeys / 16; ++kt) {
      const int m = 16 * kt + (lane & 15);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int pos = (4 * s + q) ^ (m & 15);
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + m * 256 + pos * 16);
        acc = mfma16(a, qop[s], acc);
      }
      mx = fmaxf(mx, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
    }
    // this buffer's reads are done before it is refilled kScanRing - 1 stages on
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (st % kPerBlock == kPerBlock - 1) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const int c = c0 + wave + 4 * (st / kPerBlock);
      if (lane < 16 && gq < G) block_scores[((int64_t)b * G + gq) * nblk + c] = mx;
      mx = -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
template <class E, int DI>
static hipError_t launch_prefill_t(const void* q_idx, const void* k_idx, float* bs,
                                   int64_t q_begin, int64_t q_count, int G, int top_k, int nblk,
                                   hipStream_t st) {
  typedef PrefillCfg<E, DI> C;
  const int64_t rows = q_count * G;
  if constexpr (E::is_bf16) {
    const int64_t grid = (rows + 511) / 512;
    hipLaunchKernelGGL(index_scores_prefill_lds_kernel<DI>, dim3((unsigned)grid), dim3(256), 0, st,
                       (const uint16_t*)q_idx, (const uint16_t*)k_idx, bs, q_begin, q_count, G,
                       top_k, nblk);
    return hipGetLastError();
  }
  const int64_t grid = (rows + 255) / 256;
  // enough workgroups for the chip (about 1024): the heaviest row tiles' blocks are split
  // into up to nblk / 2 chunks
  int64_t chunks = (1024 + grid - 1) / grid;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, (nblk + 1) / 2));
  const size_t lds = 2 * C::kBuf * sizeof(typename E::elem);
  hipLaunchKernelGGL((index_scores_prefill_kernel<E, DI>), dim3((unsigned)grid, (unsigned)chunks),
                     dim3(256), lds,
                     st, (const typename E::elem*)q_idx, (const typename E::elem*)k_idx, bs,
                     q_begin, q_count, G, top_k, nblk);
  return hipGetLastError();
}

hipError_t launch_index_scores_prefill(int bf16, int index_dim, const void* q_idx,
                                       const void* k_idx, float* block_scores, int64_t q_begin,
                                       int64_t q_count, int G, int top_k, int nblk,
                                       hipStream_t stream) {
  if (bf16) {
    if (index_dim == 128)
      return launch_prefill_t<BF16, 128>(q_idx, k_idx, block_scores, q_begin, q_count, G, top_k,
                                         nblk, stream);
    return launch_prefill_t<BF16, 64>(q_idx, k_idx, block_scores, q_begin, q_count, G, top_k,
                                      nblk, stream);
  }
  if (index_dim == 128)
    return launch_prefill_t<F32, 128>(q_idx, k_idx, block_scores, q_begin, q_count, G, top_k,
                                      nblk, stream);
  return launch_prefill_t<F32, 64>(q_idx, k_idx, block_scores, q_begin, q_count, G, top_k, nblk,
                                   stream);
}

template <class E, int DI>
static hipError_t launch_decode_t(const void* q_idx, const void* k_idx, float* bs,
                                  const int32_t* seq_lens, int B, int64_t max_len, int G,
                                  int top_k, int nblk, PageMap pm, hipStream_t st) {
  // Enough workgroups to cover the chip several times over at long contexts,
  // each sweeping a contiguous run of blocks (multiple of the 4 waves).
  const int64_t total = (int64_t)B * nblk;
  int64_t per = (total + 2047) / 2048;
  per = per < 4 ? 4 : (per > 64 ? 64 : per);
  per = (per + 3) / 4 * 4;
  const int gx = (int)((nblk + per - 1) / per);
  if constexpr (E::is_bf16 && DI == 128) {
    if (G <= 16) {
      hipLaunchKernelGGL(index_scores_decode_lds_kernel, dim3(gx, B), dim3(256), 0, st,
                         (const uint16_t*)q_idx, (const uint16_t*)k_idx, bs, seq_lens, max_len, G,
                         top_k, nblk, (int)per, pm);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((index_scores_decode_kernel<E, DI>), dim3(gx, B), dim3(256), 0, st,
                     (const typename E::elem*)q_idx, (const typename E::elem*)k_idx, bs, seq_lens,
                     max_len, G, top_k, nblk, (int)per, pm);
  return hipGetLastError();
}

hipError_t launch_index_scores_decode(int bf16, int index_dim, const void* q_idx,
                                      const void* k_idx, float* block_scores,
                                      const int32_t* seq_lens, int B, int64_t max_len, int G,
                                      int top_k, int nblk, PageMap pm, hipStream_t stream) {
  if (bf16) {
    if (index_dim == 128)
      return launch_decode_t<BF16, 128>(q_idx, k_idx, block_scores, seq_lens, B, max_len, G,
                                        top_k, nblk, pm, stream);
    return launch_decode_t<BF16, 64>(q_idx, k_idx, block_scores, seq_lens, B, max_len, G, top_k,
                                     nblk, pm, stream);
  }
  if (index_dim == 128)
    return launch_decode_t<F32, 128>(q_idx, k_idx, block_scores, seq_lens, B, max_len, G, top_k,
                                     nblk, pm, stream);
  return launch_decode_t<F32, 64>(q_idx, k_idx, block_scores, seq_lens, B, max_len, G, top_k,
                                  nblk, pm, stream);
}

}  // namespace msa
