// ra_device.h -- gfx950 device helpers shared by the forward and backward
// kernels: vector types, the LDS tile layout with its swizzle, the LDS-DMA
// tile loader, cross-half lane exchanges, the transposed LDS read, and the
// mapping of a workgroup to its (batch, KV head, segment, row tile).
// Library-internal; included by .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_kernels.h"
#include "ra_sched.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// the exponent reference moves only when the running max passes it by more
// than this (log2 units): weights stay <= 2^kRescale
constexpr float kRescale = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kThreads = 256;  // workgroup size of the fp32 and elementwise kernels
// The elementwise kernels (merge, finalize, fills, delta, rotation) loop
// grid-stride but are launched with one workgroup per kThreads work items up
// to this many: a grid covering the whole array keeps far more loads in
// flight than a smaller grid looping over it (merge 4.5 -> 5.9 TB/s).
// The dispatch packet counts work items in 32 bits, so a grid holds at most
// 2^32 - 1 of them.
constexpr int64_t kMaxGridBlocks = int64_t(0xFFFFFFFF) / kThreads;
constexpr int kTK = 64;        // keys per tile
constexpr int kSlots = 4;      // LDS ring of K/V tiles; loads run kSlots-1 tiles ahead

// LDS layout of one K or V tile: 64 rows (keys) of D bf16, no padding. Each
// 16-byte chunk c of row r is stored at chunk position c ^ f(r) with
// f(r) = 4*(r%4) + (r/4)%4 (masked to the chunks of a row). The LDS has 64
// banks of 4 bytes, so a 256-byte row spans every bank once and a chunk's
// banks depend only on its position in the row. f is a bijection on any 16
// consecutive rows, so the 16-byte K operand reads (16 rows, one chunk, per
// bank cycle) are conflict-free; and f/4 differs across the 4 rows of a
// transposed V read, so its 4 rows x 4 adjacent chunks are too (measured:
// 200 and 148 bytes/clock per CU for the two patterns, against 120 and 115
// for a swizzle that only varies over 8 rows).
template <int D>
struct BfTile {
  static constexpr int DP = D < 32 ? 32 : D;       // head dims padded to the MFMA M of 32
  static constexpr int ROWB = D * 2;               // bytes per key row
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TB = kTK * ROWB;            // bytes per K (or V) tile
  static constexpr int SLOT = 2 * TB;              // K tile then V tile
  static constexpr int SEGS = TB / 1024;           // 1 KiB DMA segments per tile
  static constexpr int ROWS_PER_SEG = 1024 / ROWB;
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float max_xor32(float x) {
  // max with the value held by lane L^32 (one lane swap across the wave halves)
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float sum_xor32(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Work item of one workgroup. The grid is batch x hkv x (row tiles of every
// segment); within a segment the tiles run last-first, because under the
// causal rule later rows see more keys (heavy tiles start first).
struct TileRef {
  int b, g, tile;  // batch row, KV head, row tile within the segment
  int row0;        // first local query row of the segment
  int key0;        // first key of the segment in the block
  int rows;        // query rows of (segment, KV head): group * segment length
  int kv_len;      // keys of the segment
};

template <class Params>
__device__ __forceinline__ TileRef locate_tile(const Params& p) {
  TileRef t;
  int bid = blockIdx.x;
  const int per_b = p.hkv * p.tiles_total;
  t.b = bid / per_b;
  bid -= t.b * per_b;
  t.g = bid / p.tiles_total;
  const int tt = bid - t.g * p.tiles_total;
  int lo = 0, hi = p.seg.n;  // segment s with tile_off[s] <= tt < tile_off[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_off[mid] <= tt) lo = mid; else hi = mid;
  }
  t.tile = p.tile_off[lo + 1] - 1 - tt;
  t.row0 = p.seg.off[lo];
  const int len = p.seg.off[lo + 1] - t.row0;
  t.rows = len * p.group;
  t.key0 = p.packed ? t.row0 : 0;
  t.kv_len = p.packed ? len : p.kv_len;
  return t;
}

// One direct global -> LDS load (global_load_lds_dword / _dwordx4): lane l
// reads BYTES bytes at its own global address and writes them to
// dst + BYTES*l; dst is wave-uniform and goes to M0. Issued from inline
// assembly rather than through the compiler builtin: for the builtin the
// compiler also waits for every LDS load in flight (vmcnt(0)) before each
// transposed LDS read (ds_read_b64_tr_b16), which would drain the tiles the
// rings keep in flight on every step. The kernels order these loads
// themselves (s_waitcnt vmcnt(n) + s_barrier before a tile is read, and a
// slot is refilled only after the barrier that ends its last read). The
// s_nop covers the one wait state required between writing M0 and an LDS
// load that uses it.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* src, char* dst) {
  static_assert(BYTES == 4 || BYTES == 16, "global_load_lds moves 4 or 16 bytes per lane");
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)dst);
  if constexpr (BYTES == 16)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same with a wave-uniform base address (forced into scalar registers)
// and a 32-bit per-lane byte offset from it.
template <int BYTES>
__device__ __forceinline__ void lds_dma_off(const void* base, uint32_t off, char* dst) {
  static_assert(BYTES == 4 || BYTES == 16, "global_load_lds moves 4 or 16 bytes per lane");
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)dst);
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b64 >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
  const void* sbase = (const void*)(uintptr_t)sb;
  if constexpr (BYTES == 16)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(sbase), "{m0}"(m0) : "memory");
}

// Copies of K or V tiles (kTK keys x D) global -> LDS by global_load_lds_dwordx4
// (lane l of an instruction writes bytes [16l, 16l+16) of a 1 KiB LDS segment
// and reads any global address). A lane's row and chunk within a tile are
// fixed, so its byte offset from the tile's first key is too, and the tile
// base is a scalar. Key rows past kv_len re-read the last key (those keys are
// masked before the softmax); tiles past the last one that holds keys reload
// it (they are never read). Every wave issues LPW instructions per tile, so
// all waves have the same count of loads in flight. kv_len >= 1.
template <int D, int NW>
struct KvTileDma {
  using T = BfTile<D>;
  static constexpr int LPW = T::SEGS >= NW ? T::SEGS / NW : 1;
  uint32_t off[LPW], off_last[LPW];  // bytes from the tile base
  int seg[LPW];                       // LDS byte offset of the lane's segment
  int n_real;                         // tiles holding keys
  int64_t tile_elems;                 // elements from one tile base to the next

  __device__ __forceinline__ KvTileDma(int kv_len, int row_stride, int wave, int lane) {
    n_real = (kv_len + kTK - 1) / kTK;
    tile_elems = (int64_t)kTK * row_stride;
    const int last_row = kv_len - (n_real - 1) * kTK - 1;  // in the last real tile
    const int rin = lane / T::CPR, pc = lane % T::CPR;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int sg = (wave + j * NW) % T::SEGS;
      const int row = sg * T::ROWS_PER_SEG + rin;
      const int lc = pc ^ (swz(row) & (T::CPR - 1));
      seg[j] = sg * 1024;
      off[j] = (uint32_t)(row * row_stride + lc * 8) * 2u;
      off_last[j] = (uint32_t)(min(row, last_row) * row_stride + lc * 8) * 2u;
    }
  }
  // tile t of src into the LDS tile at dst
  __device__ __forceinline__ void issue(const uint16_t* src, int t, char* dst) const {
    const int te = min(t, n_real - 1);
    const bool last = te == n_real - 1;
    const uint16_t* base = src + te * tile_elems;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma_off<16>(base, last ? off_last[j] : off[j], dst + seg[j]);
  }
};


}  // namespace ra
