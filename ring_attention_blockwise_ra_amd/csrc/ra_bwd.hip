// ra_bwd.hip -- gfx950 kernels of the blockwise backward pass.
//
// Page (cited by title and section): troisinh.com "Ring Attention -- K/V
// truyen vong giua GPU, context trieu token", section "Blockwise Backward":
// the backward pass keeps no attention matrix; it recomputes the attention
// statistics, each device only on the K/V block visiting it.
//
// For the local queries against one block j, with the forward's saved
// lse (natural log) and D = rowsum(dO * O):
//   P  = exp(scale q k^T - lse)            (visible pairs; 0 elsewhere)
//   dP = dO v^T,   dS = P * (dP - D)
//   dq += scale dS k,   dk += scale dS^T q,   dv += P^T dO
// dq stays with the queries; dk and dv are this share's addends to block j's
// gradients (in a ring they travel with the block).
//
// Kernels
//   bwd_delta          D = rowsum(dO * O), one row per D/4 lanes.
//   bwd_dq_bf16<D,NW>  row tiles of 32*NW query rows (wave: 32 rows), K/V
//                      tiles of 64 keys streamed through LDS by DMA as in the
//                      forward kernel. Per 32 keys: S^T = K Q^T and
//                      dP^T = V dO^T (A from LDS, B = Q^T / dO^T fragments in
//                      registers), dS^T in registers, dQ^T += K^T dS^T (A =
//                      K^T by transposed LDS reads, B = dS^T from the
//                      accumulator layout, as P^T in the forward).
//   bwd_dkdv_bf16<D,NW> key tiles of 32*NW keys (wave: 32 keys, K and V in
//                      registers as B operands), query row tiles of 32 rows
//                      streamed through LDS by DMA. Per row tile:
//                      S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS),
//                      dV^T += dO^T P and dK^T += Q^T dS (A by transposed LDS
//                      reads, B = P / dS straight from the accumulators).
//   bwd_dq_f32<D>, bwd_dkdv_f32<D>  fp32 inputs, FMA, the same split.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "ra_device.h"
#include "ra_kernels.h"
#include "ra_sched.h"

namespace ra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_huge_valf();

// lse in natural units -> the exp2-domain subtrahend; a row that saw no key
// at all (lse = -inf) gets +inf, so its weights are exp2(-inf) = 0.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse == kNegInf ? kPosInf : lse * kLog2e;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
// A row's vpr = D/4 lanes are consecutive and vpr divides 64, so every row
// lies inside one wavefront and is reduced with lane exchanges.
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(int64_t rows, int vpr, const f32x4* out,
                                                              const void* dout, int is_bf16,
                                                              float* delta) {
  const int64_t total = rows * vpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const f32x4 o = out[i];
    float x0, x1, x2, x3;
    if (is_bf16) {
      const u32x2 w = reinterpret_cast<const u32x2*>(dout)[i];
      x0 = bf16_bits_to_float(w[0] & 0xffffu);
      x1 = bf16_bits_to_float(w[0] >> 16);
      x2 = bf16_bits_to_float(w[1] & 0xffffu);
      x3 = bf16_bits_to_float(w[1] >> 16);
    } else {
      const f32x4 w = reinterpret_cast<const f32x4*>(dout)[i];
      x0 = w[0];
      x1 = w[1];
      x2 = w[2];
      x3 = w[3];
    }
    float s = o[0] * x0 + o[1] * x1 + o[2] * x2 + o[3] * x3;
    for (int off = 1; off < vpr; off <<= 1) s += __shfl_xor(s, off);
    if ((i % vpr) == 0) delta[i / vpr] = s;
  }
}

// ---------------------------------------------------------------------------
// dq, bf16 MFMA
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_bf16(BwdParams p) {
  using T = BfTile<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = T::DP / 32;
  constexpr int LOADS_PER_TILE = 2 * KvTileDma<D, NW>::LPW;  // per wave: K and V
  constexpr int ROWS = 32 * NW;

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave values stay scalar
  const int half = lane >> 5;
  const int col = lane & 31;

  const TileRef tr = locate_tile(p);
  const int b = tr.b, g = tr.g;
  const int kv_len = tr.kv_len;
  const int rows_total = tr.rows;
  const int rho0 = tr.tile * ROWS;
  const int rho_last = min(rho0 + ROWS, rows_total) - 1;
  const int a_lo = rho0 / p.group;
  const int a_hi = rho_last / p.group;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int key_end = (int)ra::key_end(geom, a_hi, kv_len);
  const int full_end = (int)ra::key_end(geom, a_lo, kv_len);
  const int n_kt = (key_end + kTK - 1) / kTK;

  const int64_t q_off = (int64_t)b * p.q_bstride + (int64_t)tr.row0 * p.hq * D;
  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(p.q) + q_off;
  const uint16_t* __restrict__ og = reinterpret_cast<const uint16_t*>(p.dout) + q_off;
  const int kv_row_stride = p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)tr.key0 * kv_row_stride + (int64_t)g * D;
  const uint16_t* __restrict__ kg = reinterpret_cast<const uint16_t*>(p.k) + kv_base;
  const uint16_t* __restrict__ vg = reinterpret_cast<const uint16_t*>(p.v) + kv_base;

  const int rho = rho0 + wave * 32 + col;
  const bool row_ok = rho < rows_total;
  const int rr = row_ok ? rho : rows_total - 1;
  const int row_a = rr / p.group;
  const int row_h = g * p.group + (rr - row_a * p.group);
  const int lim = (int)ra::key_end(geom, row_a, kv_len) - 1;
  const int64_t r = ((int64_t)b * p.q_len + tr.row0 + row_a) * p.hq + row_h;
  const float lse2 = row_ok ? lse_to_log2(p.lse[r]) : kPosInf;
  const float dlt = row_ok ? p.delta[r] : 0.f;

  // Q^T and dO^T fragments (B operands): dims 16t + 8*half .. +8 of this row
  bf16x8 qf[KSTEPS], of[KSTEPS];
  {
    const int64_t off = ((int64_t)row_a * p.hq + row_h) * D + 8 * half;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qg + off + 16 * t);
      u32x4 y = *reinterpret_cast<const u32x4*>(og + off + 16 * t);
      if (!row_ok) x = y = u32x4{0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(bf16x8, x);
      of[t] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[db][i] = 0.f;
  const float sl2 = p.scale_log2;

  // LDS operand offsets, as in the forward kernel: row-major operand reads of
  // K / V (koff) and transposed reads of K (voff, voff8)
  int koff[KSTEPS];
  {
    const int fr = swz(col) & (T::CPR - 1);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) koff[t] = col * T::ROWB + (((2 * t + half) ^ fr) & (T::CPR - 1)) * 16;
  }
  int voff[DB], voff8[DB];
  {
    const int grp = lane >> 4, sl = lane & 15;
    const int rw = 4 * (grp >> 1) + (sl >> 2);
    const int lowc = 2 * (grp & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = (4 * db + lowc) & (T::CPR - 1);
      voff[db] = rw * T::ROWB + ((c ^ swz(rw)) & (T::CPR - 1)) * 16 + 8 * (sl & 1);
      voff8[db] = (rw + 8) * T::ROWB + ((c ^ swz(rw + 8)) & (T::CPR - 1)) * 16 + 8 * (sl & 1);
    }
  }

  auto slot_k = [&](int t) { return smem + (t & (kSlots - 1)) * T::SLOT; };
  auto slot_v = [&](int t) { return smem + (t & (kSlots - 1)) * T::SLOT + T::TB; };
  const KvTileDma<D, NW> kv_dma(kv_len, kv_row_stride, wave, lane);
  auto issue = [&](int t) {
    kv_dma.issue(kg, t, slot_k(t));
    kv_dma.issue(vg, t, slot_v(t));
  };
  // 32 keys: unit u is half u%2 of tile u/2
  auto unit = [&](int u) {
    const char* sK = slot_k(u >> 1) + (u & 1) * 32 * T::ROWB;
    const char* sV = slot_v(u >> 1) + (u & 1) * 32 * T::ROWB;
    f32x16 s, dp;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + koff[t]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], t == 0 ? f32x16{} : s, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + koff[t]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[t], t == 0 ? f32x16{} : dp, 0, 0, 0);
    }
    const int key0 = u * 32;
    const bool need_mask = key0 + 32 > full_end;
    const int rel = lim - key0 - 4 * half;
    bf16x8 dsb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x8 e8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = 8 * c + q;
        float pv = fast_exp2(__builtin_fmaf(s[i], sl2, -lse2));
        if (need_mask && 8 * (i >> 2) + (i & 3) > rel) pv = 0.f;
        e8[q] = pv * (dp[i] - dlt);
      }
      dsb[c] = __builtin_convertvector(e8, bf16x8);
    }
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int db = j >> 1, c = j & 1;
      const s16x4 lo = lds_read_tr16(sK + voff[db] + (c * 16) * T::ROWB);
      const s16x4 hi = lds_read_tr16(sK + voff8[db] + (c * 16) * T::ROWB);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[c], dqa[db], 0, 0, 0);
    }
    // scheduling hint: LDS operand reads interleaved with the MFMAs (as in
    // the forward kernel; about 1 % here)
    __builtin_amdgcn_iglp_opt(0);
  };

  if (n_kt > 0) {
    // Tiles live in a ring of kSlots LDS slots, loads kSlots-1 tiles ahead.
    // Step t first issues tile t+3 into the slot of tile t-1 (every wave read
    // it before the barrier that closed step t-1), runs the units of tile t,
    // then waits until tile t+1 has landed (at most two tiles of its own
    // loads in flight) and meets the other waves. Tiles past the end are
    // loaded with clamped rows and never read, so every wave's load count is
    // uniform.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    issue(0);
    issue(1);
    issue(2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
    const int n_u = (key_end + 31) / 32;
    for (int t = 0; t < n_kt; ++t) {
      issue(t + 3);
      unit(2 * t);
      if (2 * t + 1 < n_u) unit(2 * t + 1);
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if (row_ok) {
    float* drow = p.dq + r * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int d = db * 32 + 8 * u4 + 4 * half;
        if (d < D) {
          f32x4 o = *reinterpret_cast<const f32x4*>(drow + d);
          o[0] += sc * dqa[db][4 * u4];
          o[1] += sc * dqa[db][4 * u4 + 1];
          o[2] += sc * dqa[db][4 * u4 + 2];
          o[3] += sc * dqa[db][4 * u4 + 3];
          *reinterpret_cast<f32x4*>(drow + d) = o;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dk, dv, bf16 MFMA
// ---------------------------------------------------------------------------
// Work item: (batch, KV head, segment, key tile of 32*NW keys); key tiles run
// first-to-last, because under the causal rule earlier keys are seen by more
// rows (heavy tiles start first).
struct KeyTileRef {
  int b, g, kt;
  int row0, key0, rows, kv_len, len;
};

__device__ __forceinline__ KeyTileRef locate_key_tile(const BwdParams& p) {
  KeyTileRef t;
  int bid = blockIdx.x;
  const int per_b = p.hkv * p.tiles_total;
  t.b = bid / per_b;
  bid -= t.b * per_b;
  t.g = bid / p.tiles_total;
  const int tt = bid - t.g * p.tiles_total;
  int lo = 0, hi = p.seg.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_off[mid] <= tt) lo = mid; else hi = mid;
  }
  t.kt = tt - p.tile_off[lo];
  t.row0 = p.seg.off[lo];
  t.len = p.seg.off[lo + 1] - t.row0;
  t.rows = t.len * p.group;
  t.key0 = p.packed ? t.row0 : 0;
  t.kv_len = p.packed ? t.len : p.kv_len;
  return t;
}

// First local query index whose rows see any key >= k0 (e is nondecreasing).
__device__ __forceinline__ int first_row_seeing(BlockGeom geom, int k0, int n_rows_a, int kv_len) {
  int lo = 0, hi = n_rows_a;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key_end(geom, mid, kv_len) > k0) hi = mid; else lo = mid + 1;
  }
  return lo;
}

constexpr int kRT = 32;        // query rows per row tile of the dk/dv kernel
constexpr int kRowSlots = 4;   // LDS ring of row tiles; loads run 3 tiles ahead
constexpr int kRowSegP = 1040; // bytes per padded group of 4 rows (d = 128)

template <int D>
struct RowTile {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int TB = kRT * ROWB;          // bytes of one Q (or dO) row tile
  static constexpr int SEGS = TB / 1024;         // 1 KiB DMA segments
  static constexpr int ROWS_PER_SEG = 1024 / ROWB;
  static constexpr int SLOT = 2 * TB;            // Q tile then dO tile
};

// REG: the group size divides the row tile (every tile starts at a query
// index boundary), which lets the row loads use fixed per-lane offsets.
template <int D, int NW, bool REG>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_bf16(BwdParams p) {
  using T = BfTile<D>;
  using R = RowTile<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = T::DP / 32;
  constexpr int KEYS = 32 * NW;
  // d = 128: row tiles in the forward kernel's padded layout (rows in groups
  // of 4, one 1 KiB DMA instruction each, group j at j * kRowSegP bytes; the
  // 16-byte granule 16*(c/4) + 4*r + c%4 holds chunk c of row 4j + r), so
  // every Q / dO operand read is one base register plus an immediate offset
  // and stays bank-conflict free. Other head sizes: XOR-swizzled rows.
  constexpr bool PR = D == 128;
  constexpr int TBR = PR ? (kRT / 4) * kRowSegP : R::TB;  // bytes of one Q (or dO) row tile
  constexpr int SLOTR = 2 * TBR;
  constexpr int LPW = (R::SEGS + NW - 1) / NW;
  constexpr int LOADS_PER_TILE = 2 * LPW + 1;  // per wave: Q, dO and the row statistics

  // LDS: ring of (Q tile, dO tile); per wave a ring of row statistics
  // (lse[32] then delta[32], raw); per wave the key limit of each row
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave limits stay scalar
  const int half = lane >> 5;
  const int col = lane & 31;
  float* stats = reinterpret_cast<float*>(smem + kRowSlots * SLOTR) + wave * kRowSlots * 64;
  int* elim = reinterpret_cast<int*>(smem + kRowSlots * SLOTR + NW * kRowSlots * 64 * 4) + wave * 32;

  const KeyTileRef kr = locate_key_tile(p);
  const int b = kr.b, g = kr.g;
  const int kv_len = kr.kv_len;
  const int rows_total = kr.rows;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int k0 = kr.kt * KEYS;               // first key of the workgroup (segment-relative)
  const int kw_lo = k0 + 32 * wave;          // this wave's keys [kw_lo, kw_lo + 32)
  const int kmy = kw_lo + col;               // this lane's key (B column, output column)
  const bool key_ok = kmy < kv_len;

  const int kv_row_stride = p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)kr.key0 * kv_row_stride + (int64_t)g * D;
  // K and V fragments as B operands of S = Q K^T and dP = dO V^T: this lane's
  // key, dims 16t + 8*half .. +8
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const int kk = min(kmy, kv_len - 1);
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + kv_base + (int64_t)kk * kv_row_stride + 8 * half;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + kv_base + (int64_t)kk * kv_row_stride + 8 * half;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 x = *reinterpret_cast<const u32x4*>(kp + 16 * t);
      u32x4 y = *reinterpret_cast<const u32x4*>(vp + 16 * t);
      if (!key_ok) x = y = u32x4{0u, 0u, 0u, 0u};
      kf[t] = __builtin_bit_cast(bf16x8, x);
      vf[t] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[db][i] = dva[db][i] = 0.f;

  // rows that see any key of the workgroup start at query index a_start
  const int a_start = first_row_seeing(geom, k0, kr.len, kv_len);
  const int t_first = (a_start * p.group) / kRT;
  const int n_rt = (rows_total + kRT - 1) / kRT;

  const int64_t q_off = (int64_t)b * p.q_bstride + (int64_t)kr.row0 * p.hq * D;
  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(p.q) + q_off;
  const uint16_t* __restrict__ og = reinterpret_cast<const uint16_t*>(p.dout) + q_off;
  const int64_t st_off = (int64_t)b * p.q_len * p.hq + (int64_t)kr.row0 * p.hq;
  const int hbase = g * p.group;

  int qoff[KSTEPS];
  {
    const int fr = swz(col) & (R::CPR - 1);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) qoff[t] = col * R::ROWB + (((2 * t + half) ^ fr) & (R::CPR - 1)) * 16;
  }
  int voff[DB], voff8[DB];
  {
    const int grp = lane >> 4, sl = lane & 15;
    const int rw = 4 * (grp >> 1) + (sl >> 2);
    const int lowc = 2 * (grp & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = (4 * db + lowc) & (R::CPR - 1);
      voff[db] = rw * R::ROWB + ((c ^ swz(rw)) & (R::CPR - 1)) * 16 + 8 * (sl & 1);
      voff8[db] = (rw + 8) * R::ROWB + ((c ^ swz(rw + 8)) & (R::CPR - 1)) * 16 + 8 * (sl & 1);
    }
  }
  const float sl2 = p.scale_log2;

  auto slot_q = [&](int t) { return smem + (t & (kRowSlots - 1)) * SLOTR; };
  auto slot_o = [&](int t) { return smem + (t & (kRowSlots - 1)) * SLOTR + TBR; };
  // padded layout: S / dP step k reads qbase + 256*(k/2) + 32*(k%2); the
  // transposed read (db, chunk c) vbase + 4*kRowSegP*c + 256*db, its second
  // half two groups (8 rows) further
  int qbase = 0, vbase = 0;
  if constexpr (PR) {
    qbase = (col >> 2) * kRowSegP + 16 * (4 * (col & 3) + half);
    const int g16 = lane >> 4, sl = lane & 15;
    const int lowc = 2 * (g16 & 1) + ((sl >> 1) & 1);
    vbase = (g16 >> 1) * kRowSegP + 16 * (4 * (sl >> 2) + lowc) + 8 * (sl & 1);
  }
  auto slot_s = [&](int t) { return stats + (t & (kRowSlots - 1)) * 64; };

  // Row cursors of the DMA (groups that do not divide the row tile): row rho
  // of (segment, KV head) is query index rho / G, head rho % G. Tiles are
  // issued in order, so each cursor steps by 32 rows per issue (no division
  // in the loop); rows past the end read the last row (loaded, never used:
  // their weights are 0). dma_off / dma_lc (the LDS segment and swizzled
  // chunk of each lane) serve both forms.
  constexpr int LPW_R = (R::SEGS + NW - 1) / NW;
  const int grp = p.group;
  const int q32 = kRT / grp, r32 = kRT - q32 * grp;
  const int last = rows_total - 1, a_last = last / grp, h_last = last - a_last * grp;
  int c_rho[LPW_R + 1], c_a[LPW_R + 1], c_h[LPW_R + 1];
  int dma_off[LPW_R], dma_lc[LPW_R];
  {
    // padded: lane l writes granule l of its group, chunk 4*(l/16) + l%4 of row (l/4)%4
    const int rin = PR ? (lane >> 2) & 3 : lane / R::CPR, pc = lane % R::CPR;
#pragma unroll
    for (int j = 0; j < LPW_R; ++j) {
      const int seg = (wave + j * NW) % R::SEGS;
      const int row = seg * R::ROWS_PER_SEG + rin;
      dma_off[j] = seg * (PR ? kRowSegP : 1024);
      dma_lc[j] = PR ? (4 * (lane >> 4) + (lane & 3)) * 8 : (pc ^ (swz(row) & (R::CPR - 1))) * 8;
      c_rho[j] = t_first * kRT + row;
    }
    c_rho[LPW_R] = t_first * kRT + col;  // the statistics of row col
#pragma unroll
    for (int j = 0; j <= LPW_R; ++j) {
      c_a[j] = c_rho[j] / grp;
      c_h[j] = c_rho[j] - c_a[j] * grp;
    }
  }
  auto cursor_off = [&](int j) {  // (query index * hq + head) of cursor j, clamped
    const bool over = c_rho[j] > last;
    return (int64_t)(over ? a_last : c_a[j]) * p.hq + hbase + (over ? h_last : c_h[j]);
  };
  auto cursor_step = [&](int j) {
    c_rho[j] += kRT;
    c_a[j] += q32;
    c_h[j] += r32;
    if (c_h[j] >= grp) {
      c_h[j] -= grp;
      ++c_a[j];
    }
  };
  // lse (lanes 0-31) or delta (lanes 32-63): the pointer is chosen once and
  // kept in registers (otherwise the selection between the two parameters
  // becomes a per-lane load from the parameter block on every tile, with a
  // wait on all loads in flight)
  const float* stats_src = half == 0 ? p.lse : p.delta;
  asm volatile("" : "+v"(stats_src));
  // REG: tile t holds query indices [t*qpt, (t+1)*qpt) and each lane's row
  // sits at a fixed byte offset from the tile's first row (ro); in the last
  // tile rows past the end re-read its last valid row (ro_last).
  const int qpt = kRT / grp;
  const int vr = rows_total - (n_rt - 1) * kRT;  // valid rows of the last tile
  uint32_t ro[LPW_R + 1], ro_last[LPW_R + 1];
  if constexpr (REG) {
    const int rin = PR ? (lane >> 2) & 3 : lane / R::CPR;
#pragma unroll
    for (int j = 0; j <= LPW_R; ++j) {
      // Q / dO rows (j < LPW_R): bytes of the (query, head) row plus the
      // lane's chunk; the statistics (j = LPW_R): 4 bytes per (query, head)
      const int row = j < LPW_R ? ((wave + j * NW) % R::SEGS) * R::ROWS_PER_SEG + rin : col;
      const int rl = min(row, vr - 1);
      const int qh = (row / grp) * p.hq + hbase + row % grp;
      const int qhl = (rl / grp) * p.hq + hbase + rl % grp;
      if (j < LPW_R) {
        ro[j] = (uint32_t)(qh * D + dma_lc[j]) * 2u;
        ro_last[j] = (uint32_t)(qhl * D + dma_lc[j]) * 2u;
      } else {
        ro[j] = (uint32_t)qh * 4u;
        ro_last[j] = (uint32_t)qhl * 4u;
      }
    }
  }
  auto issue = [&](int t) {
    if constexpr (REG) {
      const int te = min(t, n_rt - 1);
      const bool lt = te == n_rt - 1;
      const int64_t tq = (int64_t)te * qpt * p.hq;  // first (query, head) index of the tile
#pragma unroll
      for (int j = 0; j < LPW_R; ++j) {
        const uint32_t off = lt ? ro_last[j] : ro[j];
        lds_dma_off<16>(qg + tq * D, off, slot_q(t) + dma_off[j]);
        lds_dma_off<16>(og + tq * D, off, slot_o(t) + dma_off[j]);
      }
      const char* src = reinterpret_cast<const char*>(stats_src + st_off + tq);
      lds_dma<4>(src + (lt ? ro_last[LPW_R] : ro[LPW_R]), reinterpret_cast<char*>(slot_s(t)));
      return;
    }
#pragma unroll
    for (int j = 0; j < LPW_R; ++j) {
      const int64_t off = cursor_off(j) * D + dma_lc[j];
      lds_dma<16>((const void*)(qg + off), slot_q(t) + dma_off[j]);
      lds_dma<16>((const void*)(og + off), slot_o(t) + dma_off[j]);
      cursor_step(j);
    }
    // lse (lanes 0-31) and delta (lanes 32-63) of rows 32t + col
    const float* src = stats_src + st_off + cursor_off(LPW_R);
    lds_dma<4>((const void*)src, reinterpret_cast<char*>(slot_s(t)));
    cursor_step(LPW_R);
  };

  // Per row tile: does any key of this wave meet a visible row (from tile
  // t_act on), and do some of its pairs need the element mask (before tile
  // t_full, and the ragged last tile). e is nondecreasing, so both are
  // thresholds, found once by bisection.
  auto a_hi_of = [&](int t) { return (min(t * kRT + kRT, rows_total) - 1) / grp; };
  int t_act, t_full;
  {
    int lo = t_first, hi = n_rt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kw_lo < (int)key_end(geom, a_hi_of(mid), kv_len)) hi = mid; else lo = mid + 1;
    }
    t_act = lo;
    lo = t_first;
    hi = n_rt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kw_lo + 31 < (int)key_end(geom, (mid * kRT) / grp, kv_len)) hi = mid; else lo = mid + 1;
    }
    t_full = lo;
  }
  const int t_ragged = (rows_total % kRT) ? n_rt - 1 : n_rt;
  auto active = [&](int t) { return t >= t_act; };
  auto needs_mask = [&](int t) { return t < t_full || t >= t_ragged; };
  // S = Q K^T and dP = dO V^T of row tile t (A operands: Q / dO rows in LDS)
  auto scores = [&](int t, f32x16& s, f32x16& dp) {
    const char* sQ = slot_q(t);
    const char* sO = slot_o(t);
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(PR ? sQ + qbase + 256 * (k >> 1) + 32 * (k & 1) : sQ + qoff[k]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[k], k == 0 ? f32x16{} : s, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(PR ? sO + qbase + 256 * (k >> 1) + 32 * (k & 1) : sO + qoff[k]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[k], k == 0 ? f32x16{} : dp, 0, 0, 0);
    }
  };
  // P and dS of row tile t as bf16 B operands; element i of this lane is
  // row 8*(i/4) + 4*half + i%4 of the tile. The masked form zeroes the
  // weights of keys at or past each row's limit (rows past the end have
  // limit 0); tiles before t_act are masked entirely that way.
  auto weights = [&](auto masked, int t, const f32x16& s, const f32x16& dp, bf16x8 (&pb)[2],
                     bf16x8 (&dsb)[2]) {
    constexpr bool MASK = decltype(masked)::value;
    if (MASK && half == 0) {
      const int rho = t * kRT + col;
      elim[col] = rho < rows_total ? (int)key_end(geom, rho / grp, kv_len) : 0;
    }
    float* st = slot_s(t);
    {  // lse -> exp2-domain subtrahend, once per row (lanes 0-31 own the lse slots)
      const float x = st[lane];
      st[lane] = half == 0 ? lse_to_log2(x) : x;  // a select keeps the step one block
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x8 p8, d8;
#pragma unroll
      for (int hq4 = 0; hq4 < 2; ++hq4) {
        const int rbase = 8 * (2 * c + hq4) + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + rbase);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 32 + rbase);
        u32x4 e4 = {0u, 0u, 0u, 0u};
        if constexpr (MASK) e4 = *reinterpret_cast<const u32x4*>(elim + rbase);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * c + 4 * hq4 + e;
          float pv = fast_exp2(__builtin_fmaf(s[i], sl2, -l4[e]));
          if constexpr (MASK) {
            if (kmy >= (int)e4[e]) pv = 0.f;
          }
          p8[4 * hq4 + e] = pv;
          d8[4 * hq4 + e] = pv * (dp[i] - d4[e]);
        }
      }
      pb[c] = __builtin_convertvector(p8, bf16x8);
      dsb[c] = __builtin_convertvector(d8, bf16x8);
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS (A operands by transposed LDS reads)
  auto accumulate = [&](int t, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) {
    const char* sQ = slot_q(t);
    const char* sO = slot_o(t);
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int db = j >> 1, c = j & 1;
      const int vlo = PR ? vbase + 4 * kRowSegP * c + 256 * db : voff[db] + (c * 16) * R::ROWB;
      const int vhi = PR ? vlo + 2 * kRowSegP : voff8[db] + (c * 16) * R::ROWB;
      const s16x4 olo = lds_read_tr16(sO + vlo);
      const s16x4 ohi = lds_read_tr16(sO + vhi);
      const bf16x8 ao = __builtin_bit_cast(bf16x8, __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7));
      dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[c], dva[db], 0, 0, 0);
      const s16x4 qlo = lds_read_tr16(sQ + vlo);
      const s16x4 qhi = lds_read_tr16(sQ + vhi);
      const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
      dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsb[c], dka[db], 0, 0, 0);
    }
  };
  // Step t: the weights of tile t (VALU) run beside the MFMAs of tile t+1's
  // scores, which do not depend on them; then tile t's accumulation.
  auto step = [&](int t, const f32x16& s_cur, const f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt) {
    issue(t + 3);
    bf16x8 pb[2], dsb[2];
    const bool act = active(t);
    if (act) {
      if (needs_mask(t))
        weights(std::true_type{}, t, s_cur, dp_cur, pb, dsb);
      else
        weights(std::false_type{}, t, s_cur, dp_cur, pb, dsb);
    }
    if (t + 1 < n_rt && active(t + 1)) scores(t + 1, s_nxt, dp_nxt);
    if (act) accumulate(t, pb, dsb);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
  };

  if (t_first < n_rt) {
    // Ring of kRowSlots row tiles, loads three tiles ahead. Step t reads
    // tiles t and t+1; it issues tile t+3 into the slot of tile t-1 (read
    // before the barrier closing step t-1) and ends once tile t+2 has landed
    // (one tile of its own loads in flight at most). Tiles past the end load
    // clamped rows and are never read.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    issue(t_first);
    issue(t_first + 1);
    issue(t_first + 2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
    f32x16 sA, dA, sB, dB;
    if (active(t_first)) scores(t_first, sA, dA);
    // Three phases: masked tiles before t_full, then the steady state (tile
    // t active and unmasked, a next tile exists) as one branch-free block per
    // step, so the scores of t+1 interleave with the weights of t; then the
    // ragged last tile. After an odd number of steps the score registers
    // swap roles once.
    auto fast_step = [&](int tt, const f32x16& s_cur, const f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt) {
      issue(tt + 3);
      bf16x8 pb[2], dsb[2];
      weights(std::false_type{}, tt, s_cur, dp_cur, pb, dsb);
      scores(tt + 1, s_nxt, dp_nxt);
      accumulate(tt, pb, dsb);
      // scheduling hint for the step's region (the compiler's second
      // interleave strategy; 1-4 % here, while the first one is 20 % slower)
      __builtin_amdgcn_iglp_opt(2);
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
    };
    const int e1 = max(t_first, min(t_full, n_rt));
    const int e2 = max(e1, min(n_rt - 1, t_ragged));
    int t = t_first;
    for (; t + 1 < e1; t += 2) {
      step(t, sA, dA, sB, dB);
      step(t + 1, sB, dB, sA, dA);
    }
    if (t < e1) {
      step(t, sA, dA, sB, dB);
      sA = sB;
      dA = dB;
      ++t;
    }
    for (; t + 1 < e2; t += 2) {
      fast_step(t, sA, dA, sB, dB);
      fast_step(t + 1, sB, dB, sA, dA);
    }
    if (t < e2) {
      fast_step(t, sA, dA, sB, dB);
      sA = sB;
      dA = dB;
      ++t;
    }
    for (; t + 1 < n_rt; t += 2) {
      step(t, sA, dA, sB, dB);
      step(t + 1, sB, dB, sA, dA);
    }
    if (t < n_rt) step(t, sA, dA, sB, dB);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if (key_ok && t_first < n_rt) {
    const int64_t o = kv_base + (int64_t)kmy * kv_row_stride;
    float* dkr = p.dk + o;
    float* dvr = p.dv + o;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int d = db * 32 + 8 * u4 + 4 * half;
        if (d < D) {
          f32x4 x = *reinterpret_cast<const f32x4*>(dkr + d);
          f32x4 y = *reinterpret_cast<const f32x4*>(dvr + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] += sc * dka[db][4 * u4 + e];
            y[e] += dva[db][4 * u4 + e];
          }
          *reinterpret_cast<f32x4*>(dkr + d) = x;
          *reinterpret_cast<f32x4*>(dvr + d) = y;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA backward (exact per-pair arithmetic)
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 32;

// dq: thread per (query row, 32-dim slice), keys streamed through LDS
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32(BwdParams p) {
  constexpr int DC = D < 32 ? D : 32;
  constexpr int TPR = D / DC;
  constexpr int ROWS = kThreads / TPR;
  __shared__ float sK[kF32Tile][D];
  __shared__ float sV[kF32Tile][D];
  const int tid = threadIdx.x;
  const TileRef tr = locate_tile(p);
  const int b = tr.b, g = tr.g, kv_len = tr.kv_len, rows_total = tr.rows;
  const int rho0 = tr.tile * ROWS;
  const int a_hi = (min(rho0 + ROWS, rows_total) - 1) / p.group;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int key_end = (int)ra::key_end(geom, a_hi, kv_len);
  const int rho = rho0 + tid / TPR, part = tid % TPR;
  const bool ok = rho < rows_total;
  const int rr = ok ? rho : rows_total - 1;
  const int a = rr / p.group;
  const int h = g * p.group + (rr - a * p.group);
  const int64_t r = ((int64_t)b * p.q_len + tr.row0 + a) * p.hq + h;
  const float lse2 = ok ? lse_to_log2(p.lse[r]) : kPosInf;
  const float dlt = ok ? p.delta[r] : 0.f;
  const int64_t kv_row_stride = (int64_t)p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)tr.key0 * kv_row_stride + (int64_t)g * D;
  const float* __restrict__ kgp = reinterpret_cast<const float*>(p.k) + kv_base;
  const float* __restrict__ vgp = reinterpret_cast<const float*>(p.v) + kv_base;
  float qv[DC], ov[DC], acc[DC];
  const float* qrow = reinterpret_cast<const float*>(p.q) + r * D + part * DC;
  const float* orow = reinterpret_cast<const float*>(p.dout) + r * D + part * DC;
#pragma unroll
  for (int i = 0; i < DC; ++i) {
    qv[i] = ok ? qrow[i] : 0.f;
    ov[i] = ok ? orow[i] : 0.f;
    acc[i] = 0.f;
  }
  const float sl2 = p.scale_log2;
  for (int key0 = 0; key0 < key_end; key0 += kF32Tile) {
    for (int e = tid; e < kF32Tile * D; e += kThreads) {
      const int kk = e / D, d = e % D, key = key0 + kk;
      sK[kk][d] = key < kv_len ? kgp[(int64_t)key * kv_row_stride + d] : 0.f;
      sV[kk][d] = key < kv_len ? vgp[(int64_t)key * kv_row_stride + d] : 0.f;
    }
    __syncthreads();
    const int nk = min(kF32Tile, key_end - key0);
    for (int kk = 0; kk < nk; ++kk) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < DC; ++i) {
        s = __builtin_fmaf(qv[i], sK[kk][part * DC + i], s);
        dp = __builtin_fmaf(ov[i], sV[kk][part * DC + i], dp);
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        s += __shfl_xor(s, o);
        dp += __shfl_xor(dp, o);
      }
      if (visible(geom, a, key0 + kk, kv_len)) {
        const float pw = fast_exp2(__builtin_fmaf(s, sl2, -lse2));
        const float ds = pw * (dp - dlt);
#pragma unroll
        for (int i = 0; i < DC; ++i) acc[i] = __builtin_fmaf(ds, sK[kk][part * DC + i], acc[i]);
      }
    }
    __syncthreads();
  }
  if (ok) {
    float* drow = p.dq + r * D + part * DC;
#pragma unroll
    for (int i = 0; i < DC; ++i) drow[i] += p.scale * acc[i];
  }
}

// dk, dv: thread per (key, 32-dim slice), query rows streamed through LDS
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32(BwdParams p) {
  constexpr int DC = D < 32 ? D : 32;
  constexpr int TPR = D / DC;
  constexpr int KEYS = kThreads / TPR;
  __shared__ float sQ[kF32Tile][D];
  __shared__ float sO[kF32Tile][D];
  __shared__ float sL[kF32Tile], sD[kF32Tile];
  __shared__ int sE[kF32Tile];
  const int tid = threadIdx.x;
  const KeyTileRef kr = locate_key_tile(p);
  const int b = kr.b, g = kr.g, kv_len = kr.kv_len, rows_total = kr.rows;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int k0 = kr.kt * KEYS;
  const int key = k0 + tid / TPR, part = tid % TPR;
  const bool key_ok = key < kv_len;
  const int64_t kv_row_stride = (int64_t)p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)kr.key0 * kv_row_stride + (int64_t)g * D;
  const int kk = min(key, kv_len - 1);
  const float* krow = reinterpret_cast<const float*>(p.k) + kv_base + (int64_t)kk * kv_row_stride + part * DC;
  const float* vrow = reinterpret_cast<const float*>(p.v) + kv_base + (int64_t)kk * kv_row_stride + part * DC;
  float kv_[DC], vv[DC], dk[DC], dv[DC];
#pragma unroll
  for (int i = 0; i < DC; ++i) {
    kv_[i] = key_ok ? krow[i] : 0.f;
    vv[i] = key_ok ? vrow[i] : 0.f;
    dk[i] = dv[i] = 0.f;
  }
  const int a_start = first_row_seeing(geom, k0, kr.len, kv_len);
  const int64_t q_off = (int64_t)b * p.q_bstride + (int64_t)kr.row0 * p.hq * D;
  const float* __restrict__ qg = reinterpret_cast<const float*>(p.q) + q_off;
  const float* __restrict__ og = reinterpret_cast<const float*>(p.dout) + q_off;
  const int64_t st_off = (int64_t)b * p.q_len * p.hq + (int64_t)kr.row0 * p.hq;
  const int hbase = g * p.group;
  const float sl2 = p.scale_log2;
  for (int rho0 = (a_start * p.group) / kF32Tile * kF32Tile; rho0 < rows_total; rho0 += kF32Tile) {
    for (int e = tid; e < kF32Tile * D; e += kThreads) {
      const int rr = e / D, d = e % D;
      const int rho = min(rho0 + rr, rows_total - 1);
      const int a = rho / p.group;
      const int64_t off = ((int64_t)a * p.hq + hbase + (rho - a * p.group)) * D + d;
      sQ[rr][d] = qg[off];
      sO[rr][d] = og[off];
    }
    if (tid < kF32Tile) {
      const int rho = rho0 + tid;
      const bool rok = rho < rows_total;
      const int rc = rok ? rho : rows_total - 1;
      const int a = rc / p.group;
      const int64_t sidx = st_off + (int64_t)a * p.hq + hbase + (rc - a * p.group);
      sL[tid] = rok ? lse_to_log2(p.lse[sidx]) : kPosInf;
      sD[tid] = rok ? p.delta[sidx] : 0.f;
      sE[tid] = rok ? (int)key_end(geom, a, kv_len) : 0;
    }
    __syncthreads();
    const int nr = min(kF32Tile, rows_total - rho0);
    for (int rr = 0; rr < nr; ++rr) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < DC; ++i) {
        s = __builtin_fmaf(sQ[rr][part * DC + i], kv_[i], s);
        dp = __builtin_fmaf(sO[rr][part * DC + i], vv[i], dp);
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        s += __shfl_xor(s, o);
        dp += __shfl_xor(dp, o);
      }
      if (key < sE[rr]) {
        const float pw = fast_exp2(__builtin_fmaf(s, sl2, -sL[rr]));
        const float ds = pw * (dp - sD[rr]);
#pragma unroll
        for (int i = 0; i < DC; ++i) {
          dv[i] = __builtin_fmaf(pw, sO[rr][part * DC + i], dv[i]);
          dk[i] = __builtin_fmaf(ds, sQ[rr][part * DC + i], dk[i]);
        }
      }
    }
    __syncthreads();
  }
  if (key_ok) {
    float* dkr = p.dk + kv_base + (int64_t)key * kv_row_stride + part * DC;
    float* dvr = p.dv + kv_base + (int64_t)key * kv_row_stride + part * DC;
#pragma unroll
    for (int i = 0; i < DC; ++i) {
      dkr[i] += p.scale * dk[i];
      dvr[i] += dv[i];
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int64_t set_tiles_bwd(BwdParams& p, int rows_per_tile, bool by_keys) {
  int64_t total = 0;
  for (int s = 0; s < p.seg.n; ++s) {
    p.tile_off[s] = (int32_t)total;
    const int64_t len = p.seg.off[s + 1] - p.seg.off[s];
    const int64_t n = by_keys ? (p.packed ? len : (s == 0 ? p.kv_len : 0)) : len * p.group;
    total += (n + rows_per_tile - 1) / rows_per_tile;
  }
  p.tile_off[p.seg.n] = (int32_t)total;
  p.tiles_total = (int32_t)total;
  return total;
}

constexpr int kDqWaves = 8;
constexpr int kKvWaves = 4;

template <int D>
static hipError_t launch_bwd_bf16(BwdParams p, hipStream_t stream) {
  {
    BwdParams q = p;
    const int64_t tiles = set_tiles_bwd(q, 32 * kDqWaves, false);
    const size_t smem = kSlots * BfTile<D>::SLOT;
    auto kern = bwd_dq_bf16<D, kDqWaves>;
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), smem);
    if (e != hipSuccess) return e;
    const int64_t grid = (int64_t)q.batch * q.hkv * tiles;
    if (grid > 0) hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDqWaves * 64), smem, stream, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    BwdParams q = p;
    const int64_t tiles = set_tiles_bwd(q, 32 * kKvWaves, true);
    const size_t rslot = D == 128 ? 2 * (kRT / 4) * kRowSegP : RowTile<D>::SLOT;  // padded rows at d = 128
    const size_t smem = kRowSlots * rslot + kKvWaves * (kRowSlots * 64 + 32) * 4;
    const bool reg = kRT % q.group == 0;
    auto kern = reg ? bwd_dkdv_bf16<D, kKvWaves, true> : bwd_dkdv_bf16<D, kKvWaves, false>;
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), smem);
    if (e != hipSuccess) return e;
    const int64_t grid = (int64_t)q.batch * q.hkv * tiles;
    if (grid > 0) hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kKvWaves * 64), smem, stream, q);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_f32(BwdParams p, hipStream_t stream) {
  constexpr int DC = D < 32 ? D : 32;
  constexpr int PER = kThreads / (D / DC);
  {
    BwdParams q = p;
    const int64_t grid = (int64_t)q.batch * q.hkv * set_tiles_bwd(q, PER, false);
    if (grid > 0) hipLaunchKernelGGL(bwd_dq_f32<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    BwdParams q = p;
    const int64_t grid = (int64_t)q.batch * q.hkv * set_tiles_bwd(q, PER, true);
    if (grid > 0) hipLaunchKernelGGL(bwd_dkdv_f32<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  }
  return hipGetLastError();
}

void bwd_tile_shapes(int is_bf16, int head_dim, TileShape out[2]) {
  if (is_bf16) {
    out[0] = TileShape{32 * kDqWaves, 64 * kDqWaves, 0};
    out[1] = TileShape{32 * kKvWaves, 64 * kKvWaves, 1};
    return;
  }
  const int dc = head_dim < 32 ? head_dim : 32;
  const int per = kThreads / (head_dim / dc);
  out[0] = TileShape{per, kThreads, 0};
  out[1] = TileShape{per, kThreads, 1};
}

hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t stream) {
  if (is_bf16) {
    switch (p.head_dim) {
      case 16: return launch_bwd_bf16<16>(p, stream);
      case 32: return launch_bwd_bf16<32>(p, stream);
      case 64: return launch_bwd_bf16<64>(p, stream);
      case 128: return launch_bwd_bf16<128>(p, stream);
    }
  } else {
    switch (p.head_dim) {
      case 16: return launch_bwd_f32<16>(p, stream);
      case 32: return launch_bwd_f32<32>(p, stream);
      case 64: return launch_bwd_f32<64>(p, stream);
      case 128: return launch_bwd_f32<128>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

__global__ __launch_bounds__(kThreads) void zero_kernel(int64_t n4, f32x4* x) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(int64_t n4, u32x4* x, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    x[i] = u32x4{value, value, value, value};
}

hipError_t launch_fill_u32(void* x, int64_t bytes, uint32_t value, hipStream_t stream) {
  const int64_t n4 = bytes / 16;  // callers pass multiples of 16 bytes
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, n4,
                     reinterpret_cast<u32x4*>(x), value);
  return hipGetLastError();
}

// dst_a <- src_a and dst_b <- src_b, n4 16-byte vectors each, in one launch
// (the two staging copies of a ring step)
__global__ __launch_bounds__(kThreads) void copy2_kernel(int64_t n4, const u32x4* __restrict__ sa,
                                                        u32x4* __restrict__ da,
                                                        const u32x4* __restrict__ sb,
                                                        u32x4* __restrict__ db) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n4; i += stride) {
    if (i < n4)
      da[i] = sa[i];
    else
      db[i - n4] = sb[i - n4];
  }
}

hipError_t launch_copy2(void* dst_a, const void* src_a, void* dst_b, const void* src_b,
                        int64_t bytes, hipStream_t stream) {
  const int64_t n4 = bytes / 16;  // callers pass multiples of 16 bytes
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (2 * n4 + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  hipLaunchKernelGGL(copy2_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, n4,
                     reinterpret_cast<const u32x4*>(src_a), reinterpret_cast<u32x4*>(dst_a),
                     reinterpret_cast<const u32x4*>(src_b), reinterpret_cast<u32x4*>(dst_b));
  return hipGetLastError();
}

hipError_t launch_zero(float* x, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;  // callers pass multiples of 4 (rows * head_dim)
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, n4,
                     reinterpret_cast<f32x4*>(x));
  return hipGetLastError();
}

hipError_t launch_bwd_delta(int64_t rows, int d, int is_bf16, const float* out, const void* dout,
                            float* delta, hipStream_t stream) {
  const int vpr = d / 4;
  int64_t blocks = (rows * vpr + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, rows, vpr,
                     reinterpret_cast<const f32x4*>(out), dout, is_bf16, delta);
  return hipGetLastError();
}

}  // namespace ra
