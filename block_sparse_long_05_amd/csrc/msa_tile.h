// LDS staging of 128-token K / V / index-key blocks and the MFMA operand reads on them
// (gfx950, bf16, head dim 128), shared by the main-branch tile kernels and the index-branch
// KL kernels.
#pragma once

#include "msa_device.h"

namespace msa {

// ---- bf16 K staging by direct global->LDS loads (row-swizzled, unpadded) -----------------
// Row r of the staged block occupies 256 bytes; its 16-byte chunk x sits at position
// x ^ (r % 16), so a quarter-wave loads one whole row (coalesced) and the S^T operand reads
// of 8 rows at a time hit distinct banks.
// V blocks use another row swizzle (kVSwz): chunk x of row r sits at position
// x ^ (4 (r % 4) + (r / 4) % 4), which keeps the transpose reads of PV (4 rows x 4
// chunks per half-wave) on 16 distinct positions.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int NT, bool kVSwz = false>
__device__ __forceinline__ void k_block_dma(const uint16_t* K, int g, int c, int64_t seq_len,
                                            uint8_t* kbuf, int tid) {
  const int64_t key0 = (int64_t)c * kBlock;
  const int nk = (int)min((int64_t)kBlock, seq_len - key0);
  const uint16_t* kg = K + ((int64_t)g * seq_len + key0) * kHeadDim;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int kLoads = kBlock * 256 / 1024;  // 1 KiB loads per block
#pragma unroll
  for (int i = 0; i < kLoads / (NT / 64); ++i) {
    const int li = wave * (kLoads / (NT / 64)) + i;
    const int r = 4 * li + (lane >> 4);
    const int chunk = (lane & 15) ^ (kVSwz ? v_swz(r) : (r & 15));
    const int rr = r < nk ? r : nk - 1;  // rows past the sequence end repeat a valid row
    const uint32_t off = (uint32_t)(rr * kHeadDim + chunk * 8);  // 32-bit: uniform base + offset
    __builtin_amdgcn_global_load_lds((const void*)(kg + off),
                                     (__attribute__((address_space(3))) void*)(kbuf + li * 1024),
                                     16, 0, 0);
  }
}

// The same staging with the wave-uniform parts of every address in scalar registers.
// Wave w of NT / 64 loads rows 4 li + lane / 16 for li = w * P + i (P = loads per wave):
// row offset 256 (4 li) is uniform, and the swizzled chunk of lane (L = lane / 16,
// x = lane % 16) is x ^ (4 (i % 4) + L) (row swizzle) or x ^ (4 L + i % 4) (V swizzle),
// so a lane's byte offset within the 1 KiB of load li is dma_lane_off(lane) xor-ed with
// 64 (i % 4) or 16 (i % 4). `wave` must be wave-uniform. A block that ends before its
// 128th row (the sequence's last) takes the general path above.
template <bool kVSwz>
__device__ __forceinline__ uint32_t dma_lane_off(int lane) {
  const int L = (lane >> 4) & 3, x = lane & 15;
  return (uint32_t)(256 * L + 16 * (x ^ (kVSwz ? 4 * L : L)));
}

template <int NT, bool kVSwz = false>
__device__ __forceinline__ void k_block_dma_s(const uint16_t* K, int g, int c, int64_t seq_len,
                                              uint8_t* kbuf, int wave, uint32_t lane_off,
                                              int tid) {
  const int64_t key0 = (int64_t)c * kBlock;
  if (seq_len - key0 < kBlock) {
    k_block_dma<NT, kVSwz>(K, g, c, seq_len, kbuf, tid);
    return;
  }
  constexpr int kPer = kBlock * 256 / 1024 / (NT / 64);  // 1 KiB loads per wave
  const uint8_t* base = reinterpret_cast<const uint8_t*>(K + ((int64_t)g * seq_len + key0) * kHeadDim) +
                        (size_t)wave * kPer * 1024;
  uint8_t* lds = kbuf + wave * kPer * 1024;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t off = lane_off ^ (uint32_t)((kVSwz ? 16 : 64) * (i & 3));
    __builtin_amdgcn_global_load_lds((const void*)(base + 1024 * i + off),
                                     (__attribute__((address_space(3))) void*)(lds + 1024 * i),
                                     16, 0, 0);
  }
}

// ---- the same staging issued as inline assembly --------------------------------------------
// The compiler does not track these loads, so it adds no waits for them. (Its tracking of the
// direct-to-LDS builtin cannot tell the buffers of a ring apart: with a load into one buffer in
// flight it drains every pending load before LDS reads of another buffer, which serialises a
// double buffer.) The caller owns the synchronisation: MSA_WAIT_VMCNT on this wave's loads
// (kBlock * 256 / 1024 / (NT / 64) per block), then a barrier, before any wave reads the
// buffer, and no wave may still read a buffer when a load into it is issued. Loads issued
// before an ordinary load complete before it (vector memory loads return in order), so the
// compiler's own waits stay correct. M0 holds the wave-uniform LDS address of the 1 KiB row
// group (the load writes lane l's 16 bytes at M0 + 16 l).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
// `gbase` and `lds` must be wave-uniform; they are moved to scalar registers explicitly (the
// compiler cannot always prove a value uniform, and the instruction takes its base there).
__device__ __forceinline__ void lds_dma16(const uint8_t* gbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)gbase;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint8_t* sbase = (const uint8_t*)(uintptr_t)(lo | (hi << 32));
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0)
               : "memory");
}

template <int NT, bool kVSwz = false>
__device__ __forceinline__ void k_block_dma_asm(const uint16_t* K, int g, int c, int64_t seq_len,
                                                uint8_t* kbuf, int wave, uint32_t lane_off,
                                                int tid) {
  constexpr int kPer = kBlock * 256 / 1024 / (NT / 64);  // 1 KiB loads per wave
  const int64_t key0 = (int64_t)c * kBlock;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(K + ((int64_t)g * seq_len + key0) * kHeadDim);
  const uint32_t lds = lds_addr(kbuf) + (uint32_t)(wave * kPer * 1024);
  if (seq_len - key0 < kBlock) {
    // the sequence's last block: rows past its end repeat a valid row
    const int nk = (int)(seq_len - key0);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int li = wave * kPer + i;
      const int r = 4 * li + (lane >> 4);
      const int chunk = (lane & 15) ^ (kVSwz ? v_swz(r) : (r & 15));
      const int rr = r < nk ? r : nk - 1;
      lds_dma16(kg, (uint32_t)(rr * kHeadDim + chunk * 8) * 2u, lds + 1024 * i);
    }
    return;
  }
  const uint8_t* base = kg + (size_t)wave * kPer * 1024;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    lds_dma16(base, 1024u * i + (lane_off ^ (uint32_t)((kVSwz ? 16 : 64) * (i & 3))), lds + 1024 * i);
}

__device__ __forceinline__ f32x16 s_tile_swz(const uint8_t* kbuf, int m, const u32x4* qop, int q) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s) {
    const int pos = (2 * s + q) ^ (m & 15);
    acc = mfma32(*reinterpret_cast<const u32x4*>(kbuf + m * 256 + pos * 16), qop[s], acc);
  }
  return acc;
}

// The four S^T tiles of a 128-key block (keys 32 kt + m for lane column m) as four interleaved
// MFMA chains: each k-step's operand reads feed four independent accumulators, so the
// matrix core does not wait on one chain's results between tiles.
__device__ __forceinline__ void s_tiles4_swz(const uint8_t* kbuf, int m, const u32x4* qop, int q,
                                             f32x16 (&acc)[4]) {
  const uint8_t* kr = kbuf + m * 256;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x16{};
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s) {
    const int pos = (2 * s + q) ^ (m & 15);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      acc[kt] = mfma32(*reinterpret_cast<const u32x4*>(kr + kt * 32 * 256 + pos * 16), qop[s], acc[kt]);
  }
}

// O^T += V^T . P^T over one 64-key half of the block, V row-major in LDS in the V
// row swizzle of k_block_dma. The LDS transpose read (ds_read_b64_tr_b16) hands
// lane i of a 16-lane group column i % 4 of the 8-byte rows that lanes 4 j + i / 4
// (j = 0..3) address. Lane (m = lane % 32, q = lane / 32) needs D column 32 dt + m of
// keys 16 u + 4 q + 0..3 (then + 8): so lane r of its group addresses key row
// 16 u + 4 q + r / 4, columns 32 dt + 16 ((lane / 16) % 2) + 4 (r % 4) .. + 4.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void pv_half_tr(f32x16* o, const u32x4* pb, const uint8_t* vbuf,
                                           int lane, int half) {
  // Key row 16 u' + 4 q + j (+ 8 for the second read) holds chunk (4 dt + c0) at position
  // 4 (dt ^ j) + (c0 ^ q) (+ 2, xor, for the second read), with c0 = 2 hx + (r % 4) / 2.
  const int q = lane >> 5, hx = (lane >> 4) & 1, r = lane & 15;
  const int j = r >> 2;
  const int c0 = 2 * hx + ((r & 3) >> 1);
  const uint8_t* base = vbuf + (4 * q + j) * 256 + (r & 1) * 8;
  const uint8_t* lo_b[4];
  const uint8_t* hi_b[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    lo_b[dt] = base + 64 * (dt ^ j) + 16 * (c0 ^ q);
    hi_b[dt] = base + 8 * 256 + 64 * (dt ^ j) + 16 * (c0 ^ q ^ 2);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row0 = 64 * half + 16 * u;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const u32x2 lo = lds_read_tr16(lo_b[dt] + row0 * 256);
      const u32x2 hi = lds_read_tr16(hi_b[dt] + row0 * 256);
      o[dt] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[u], o[dt]);
    }
  }
}


// One 32x32x16 MFMA operand read with the transpose read from a buffer of 256-byte rows in
// the V swizzle: the 32 M (or N) indices are the buffer's columns 32 dt .. 32 dt + 31 (lane
// l % 32 takes column 32 dt + l % 32) and the 16 K indices its rows row0 .. row0 + 15 (row0 a
// multiple of 16), lane group q holding rows 4q + 0..3 and 8 + 4q + 0..3: the same order as
// the keys of the P^T registers of an S^T tile, so either operand of a product over those
// rows can be read this way.
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* buf, int row0, int dt, int lane) {
  const int q = lane >> 5, hx = (lane >> 4) & 1, r = lane & 15;
  const int j = r >> 2;
  const int c0 = 2 * hx + ((r & 3) >> 1);
  const uint8_t* base = buf + (row0 + 4 * q + j) * 256 + (r & 1) * 8;
  const u32x2 lo = lds_read_tr16(base + 64 * (dt ^ j) + 16 * (c0 ^ q));
  const u32x2 hi = lds_read_tr16(base + 8 * 256 + 64 * (dt ^ j) + 16 * (c0 ^ q ^ 2));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// S^T tile against a block staged in the V swizzle (row reads of 16-byte chunks).
__device__ __forceinline__ f32x16 s_tile_vswz(const uint8_t* kbuf, int m, const u32x4* qop, int q) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < kHeadDim / 16; ++s) {
    const int pos = (2 * s + q) ^ v_swz(m);
    acc = mfma32(*reinterpret_cast<const u32x4*>(kbuf + m * 256 + pos * 16), qop[s], acc);
  }
  return acc;
}

}  // namespace msa
