// ra_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the Ring Attention
// per-device step.
//
// Pages (cited by title and section):
//   [UL] Ultralytics glossary "Ring Attention", section "How ring attention
//        works": per step, attention of the local queries against the block
//        currently held; running sums of exponentiated scores and of
//        weighted values; the running maximum is subtracted before
//        exponentiating; one divide at the end.
//   [TS] troisinh.com "Ring Attention -- K/V truyen vong giua GPU, context
//        trieu token", section "Tai sao no hoat dong": the running max and
//        normaliser update, output rescaled the same way.
//
// Kernels
//   attn_bf16_mfma<D, NW>  one KV block against the local queries, bf16 in,
//                          fp32 accumulate, v_mfma_f32_32x32x16_bf16 for both
//                          contractions, K/V tiles staged through LDS,
//                          in-register online softmax (exp2 domain).
//   attn_f32_fma<D>        the same partial for fp32 inputs with fp32 FMA
//                          (exact per-key online update).
//   merge_partials         bandwidth-bound elementwise merge of two partials.
//   finalize               acc / l in place and lse = m + ln l.
//   fill_empty             the empty partial (-inf, 0, 0).
//   tile_classes           device form of the causal tile rule.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "ra_device.h"
#include "ra_kernels.h"
#include "ra_sched.h"

namespace ra {

// Online-softmax merge of two partials of one row ([TS] "Tai sao no hoat
// dong"): with running maxima x1, x2 (natural units), the merged maximum mm
// and the factors that bring each side's l and acc to it. An empty side
// (-inf) weighs 0. Used by the merge kernel and by the attention kernels when
// they merge their partial into the running state in place.
struct MergeCoef {
  float f1, f2, mm;
};
__device__ __forceinline__ MergeCoef merge_coef(float x1, float x2) {
  const float mm = fmaxf(x1, x2);
  return MergeCoef{(x1 == kNegInf) ? 0.f : expf(x1 - mm), (x2 == kNegInf) ? 0.f : expf(x2 - mm), mm};
}

// The final divide of one row ([UL] "How ring attention works"): the factor
// that turns acc into the output, and lse = m + ln l (-inf for l = 0), as
// finalize_kernel computes them.
__device__ __forceinline__ float finalize_inv(float l) { return l > 0.f ? 1.0f / l : 0.f; }
__device__ __forceinline__ float finalize_lse(float m, float l) {
  return l > 0.f ? m + logf(l) : kNegInf;
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention partial
// ---------------------------------------------------------------------------
//
// Work decomposition. For batch b and KV head g the G = hq/hkv query heads of
// the group share K/V; their rows are enumerated as rho = a*G + hh (a: local
// query index, hh: head within the group). A workgroup of NW waves owns 32*NW
// consecutive rows rho (wave w: rows [32w, 32w+32)) and streams block j's K/V
// of head g through LDS in tiles of 64 keys, double-buffered: the global
// loads of tile t+1 are in flight while tile t is computed. With NW = 8 two
// waves share each SIMD, so one wave's softmax (VALU) runs under the other's
// MFMAs.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand: lane L holds A[m = L%32][k = 8*(L/32) .. +8]
//   B operand: lane L holds B[k = 8*(L/32) .. +8][n = L%32]
//   C/D:       lane L, register i holds C[m = 8*(i/4) + 4*(L/32) + i%4][n = L%32]
// Scores are computed transposed, S^T = K Q^T (m = key, n = query), so each
// lane owns one query column: row max and row sum reduce over its own
// registers plus one exchange with lane L^32. The output is also transposed,
// O^T += V^T P^T (m = head dim, n = query): the rescale factor is per lane and
// the P^T operand comes straight from the S^T accumulator registers: within a
// 16-key chunk lane half h holds keys {4h..4h+3, 8+4h..8+4h+3}, which fixes
// the order of the reduction slots. K and V are stored row-major in LDS
// (head_dim contiguous). The K operand is one 16-byte read per lane. The V^T
// operand is gathered with two ds_read_b64_tr_b16 per MFMA: inside each group
// of 16 lanes that instruction hands output lane i, element j, the (i%4)-th
// 16-bit element of the 8 bytes addressed by source lane 4j + i/4. Source lane
// s therefore addresses V[k0 + s/4][d0 + 4(s%4)], and output lane i receives
// V[k0 .. k0+3][d0 + i]: four consecutive keys of one head dimension.
//
// LDS holds kSlots K tiles, then kSlots V tiles. For D = 128 with 8 waves a
// tile uses the padded layout below instead of the XOR-swizzled rows of
// BfTile: every operand read of a lane is then its one base address plus an
// immediate offset (no address arithmetic per read, 10 fewer VGPRs).

// D = 128 tile: rows in groups of 4 (one 1 KiB DMA instruction each), group j
// at j * SEGP bytes (64 bytes of padding per group). Inside a group the
// 16-byte granule 16*(c/4) + 4*r + c%4 holds chunk c (head dims 8c..8c+7) of
// row 4j + r. The padding of 4 granules rotates the banks by one granule per
// group, which keeps both operand reads conflict-free: a K read (16 lanes of
// 16 bytes, rows 0..15 of one chunk) and a transposed V read (32 lanes of 8
// bytes, 4 rows x 4 chunks) each cover all 64 banks once. Chunk c of row r
// lies at (r/4)*SEGP + 16*(16*(c/4) + 4*(r%4) + c%4), affine in c inside
// each run of 4 chunks, so the reads of successive MFMA steps differ by
// constants. Each group of 4 DMA lanes reads 64 contiguous bytes of one row.
struct KvTile128 {
  static constexpr int SEGP = 1040;
  static constexpr int TB = 16 * SEGP;   // 64 keys
  static constexpr int HALF = 8 * SEGP;  // 32 keys
};

// Global -> LDS copies of one tile in the KvTile128 layout (the same contract
// as KvTileDma: fixed per-lane offsets, the last key re-read past kv_len,
// tiles past the last one reload it, LPW loads per wave per tile).
template <int NW>
struct KvTileDma128 {
  static constexpr int LPW = 16 / NW;
  uint32_t off[LPW], off_last[LPW];
  int seg[LPW];
  int n_real;
  int64_t tile_elems;
  __device__ __forceinline__ KvTileDma128(int kv_len, int row_stride, int wave, int lane) {
    n_real = (kv_len + kTK - 1) / kTK;
    tile_elems = (int64_t)kTK * row_stride;
    const int last_row = kv_len - (n_real - 1) * kTK - 1;
    // lane l writes granule l of its group: chunk 4*(l/16) + l%4 of row (l/4)%4
    const int c = 4 * (lane >> 4) + (lane & 3), r4 = (lane >> 2) & 3;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int sg = (wave + j * NW) % 16;
      const int row = 4 * sg + r4;
      seg[j] = sg * KvTile128::SEGP;
      off[j] = (uint32_t)(row * row_stride + c * 8) * 2u;
      off_last[j] = (uint32_t)(min(row, last_row) * row_stride + c * 8) * 2u;
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* src, int t, char* dst) const {
    const int te = min(t, n_real - 1);
    const bool last = te == n_real - 1;
    const uint16_t* base = src + te * tile_elems;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma_off<16>(base, last ? off_last[j] : off[j], dst + seg[j]);
  }
};

template <int D, int NW>
constexpr bool kPadTile = D == 128 && (NW == 8 || NW == 4);

// K and V ring slots per workgroup: 4 + 4 with 8 waves (one workgroup per
// CU), 2 + 2 with 4 waves, so that two workgroups share a CU (each with its
// own rings, 65 KiB of LDS at d = 128).
template <int NW>
constexpr int kFwdSlots = NW == 4 ? 2 : kSlots;

// The kernel's dynamic LDS (K/V tile ring) is sized at launch, so the
// compiler cannot see that it limits the kernel to one workgroup per CU; with
// 8 waves that is two waves per SIMD, which is stated here so that the
// scheduler plans for up to 256 VGPRs rather than serialising operand reads
// to free registers for an occupancy the LDS never allows.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(kPadTile<D, NW> ? 2 : 1, kPadTile<D, NW> ? 2 : 8)))
void attn_bf16_mfma(AttnParams p) {
  using T = BfTile<D>;
  constexpr int ROWS = 32 * NW;
  constexpr int KSTEPS = D / 16;
  constexpr int KB = kTK / 32;   // 32-key blocks per tile
  constexpr int KC = kTK / 16;   // 16-key chunks per tile
  constexpr int DB = T::DP / 32; // 32-dim blocks of the output
  constexpr bool PAD = kPadTile<D, NW>;
  using Dma = std::conditional_t<PAD, KvTileDma128<NW>, KvTileDma<D, NW>>;
  constexpr int TBX = PAD ? KvTile128::TB : T::TB;                // bytes per K (or V) tile
  constexpr int HALFX = PAD ? KvTile128::HALF : 32 * T::ROWB;     // bytes per 32 keys

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

  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bstride +
                                    (int64_t)tr.row0 * p.hq * D;
  const int kv_row_stride = p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)tr.key0 * kv_row_stride + (int64_t)g * D;
  const uint16_t* __restrict__ kg = reinterpret_cast<const uint16_t*>(p.k) + kv_base;
  const uint16_t* __restrict__ vg = reinterpret_cast<const uint16_t*>(p.v) + kv_base;

  // this lane's query row
  const int rho = rho0 + wave * 32 + col;
  const bool row_ok = rho < rows_total;
  const int rr = row_ok ? rho : rows_total - 1;
  const int row_a = rr / p.group;
  const int row_h = g * p.group + (rr - row_a * p.group);
  // last key index visible to this row (keys past kv_len are never visible)
  const int lim = (int)ra::key_end(geom, row_a, kv_len) - 1;

  // Q^T fragments (B operand): lane holds dims 16t + 8*half .. +8 of its row
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = qg + ((int64_t)row_a * p.hq + row_h) * D + 8 * half;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * t);
      if (!row_ok) x = u32x4{0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Per-lane byte offsets of the LDS operand reads (swizzled chunk positions).
  // K operand, step t: row col (+32 per half tile), chunk 2t + half; f
  // depends on the row modulo 16, so the +32 row offset keeps it.
  int koff[KSTEPS];
  if constexpr (!PAD) {
    const int fr = swz(col) & (T::CPR - 1);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) koff[t] = col * T::ROWB + (((2 * t + half) ^ fr) & (T::CPR - 1)) * 16;
  }
  // V^T operand (transposed reads): rows r = 4*(grp/2) + sl/4 (+16 per chunk,
  // +32 per half tile) and r + 8 (the second read of an operand), head dims
  // db*32 + 16*(grp%2) + 4*(sl%4) .. +3, i.e. chunk 4 db + 2*(grp%2) + (sl/2)%2.
  int voff[DB], voff8[DB];
  if constexpr (!PAD) {
    const int grp = lane >> 4, sl = lane & 15;
    const int r = 4 * (grp >> 1) + (sl >> 2);
    const int lowc = 2 * (grp & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = (4 * db + lowc) & (T::CPR - 1);
      voff[db] = r * T::ROWB + ((c ^ swz(r)) & (T::CPR - 1)) * 16 + 8 * (sl & 1);
      voff8[db] = (r + 8) * T::ROWB + ((c ^ swz(r + 8)) & (T::CPR - 1)) * 16 + 8 * (sl & 1);
    }
  }

  // Lazy rescaling: P, l and O are kept relative to a per-row reference
  // `base` (log2 units) that only moves when the running max m_run exceeds
  // it by more than kRescale; the epilogue converts to the exact max. This
  // keeps the O rescale (a multiply per accumulator) off most units.
  float base = kNegInf;

  // Padded layout: K step t (chunk 2t + half of row col) at kbase + 256*(t/2)
  // + 32*(t%2); V^T read (db, chunk c) at vbase + 4*SEGP*c + 256*db, its second
  // half 8 rows (2 groups) further.
  int kbase = 0, vbase = 0;
  if constexpr (PAD) {
    kbase = (col >> 2) * KvTile128::SEGP + 16 * (4 * (col & 3) + half);
    const int grp = lane >> 4, sl = lane & 15;
    const int lowc = 2 * (grp & 1) + ((sl >> 1) & 1);
    vbase = (grp >> 1) * KvTile128::SEGP + 16 * (4 * (sl >> 2) + lowc) + 8 * (sl & 1);
  }

  // Two rings of kSlots 64-key tiles: K tile t in K slot t % kSlots, V tile t
  // in V slot t % kSlots.
  constexpr int SL = kFwdSlots<NW>;
  auto slot_k = [&](int t) { return smem + (t & (SL - 1)) * TBX; };
  auto slot_v = [&](int t) { return smem + (SL + (t & (SL - 1))) * TBX; };
  const Dma kv_dma(kv_len, kv_row_stride, wave, lane);
  auto issue_k = [&](int t) { kv_dma.issue(kg, t, slot_k(t)); };
  auto issue_v = [&](int t) { kv_dma.issue(vg, t, slot_v(t)); };
  // Work is done in units of 32 keys: unit u is half u%2 of tile u/2. S(u)
  // is one 32x32 MFMA tile (16 registers per lane), P(u) two bf16x8 operands.
  // ks / vs: the LDS slot holding tile u/2 (the caller knows it).
  auto qk = [&](f32x16& s_out, int u, int ks) {
    const char* sK = slot_k(ks) + (u & 1) * HALFX;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const char* pa = PAD ? sK + kbase + 256 * (t >> 1) + 32 * (t & 1) : sK + koff[t];
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(pa);
      s_out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], t == 0 ? f32x16{} : s_out, 0, 0, 0);
    }
  };
  auto pv = [&](const bf16x8 (&pf)[2], int u, int vs) {
    const char* sV = slot_v(vs) + (u & 1) * HALFX;
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int db = j >> 1, c = j & 1;
      const char* plo = PAD ? sV + vbase + 4 * KvTile128::SEGP * c + 256 * db : sV + voff[db] + (c * 16) * T::ROWB;
      const char* phi = PAD ? plo + 2 * KvTile128::SEGP : sV + voff8[db] + (c * 16) * T::ROWB;
      const s16x4 lo = lds_read_tr16(plo);
      const s16x4 hi = lds_read_tr16(phi);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], oacc[db], 0, 0, 0);
    }
  };
  // mask S(u) past the diagonal or the ragged tail, then move the reference
  // with its row max; returns the factor O must take after the PV of P(u-1)
  auto mask_and_ref = [&](f32x16& sc, int u) -> float {
    const int key0 = u * 32;
    if (key0 + 32 > full_end) {
      const int rel = lim - key0 - 4 * half;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (8 * (q >> 2) + (q & 3) > rel) sc[q] = kNegInf;
    }
    float mt = kNegInf;
#pragma unroll
    for (int q = 0; q < 16; ++q) mt = fmaxf(mt, sc[q]);
    m_run = fmaxf(m_run, max_xor32(mt) * sl2);
    const bool move = m_run > base + kRescale;
    const float nb = move ? m_run : base;
    const float alpha = move ? fast_exp2(base - nb) : 1.0f;  // 0 when base was -inf
    base = nb;
    l_run *= alpha;
    return alpha;
  };
  // P(u) = exp2(S(u) c - base) as bf16 operands; l += sum of the rounded
  // weights (the same ones the numerator uses)
  auto softmax_p = [&](const f32x16& sc, bf16x8 (&pf)[2]) {
    const float bexp = base == kNegInf ? 0.f : base;
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x8 e8;
#pragma unroll
      for (int q = 0; q < 8; ++q) e8[q] = fast_exp2(__builtin_fmaf(sc[8 * c + q], sl2, -bexp));
      const bf16x8 pb = __builtin_convertvector(e8, bf16x8);
      pf[c] = pb;
#pragma unroll
      for (int o = 0; o < 8; o += 2)
        ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[o], pb[o + 1]}, ones, ls, false);
    }
    l_run += ls;
  };
  auto rescale_o = [&](float alpha) {
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
  };
  // One unit u of the three-stage pipeline: with S(u) complete and P(u-1)
  // pending, issue S(u+1) = K(u+1) Q^T, compute P(u), and issue
  // O += V(u-1) P(u-1). None of these MFMAs depends on the exponentials of
  // the same unit, so the matrix core and the transcendental unit overlap.
  auto unit = [&](f32x16& sc, f32x16& sn, const bf16x8 (&pprev)[2], bf16x8 (&pcur)[2], int u,
                  bool has_next, bool has_prev, int ks, int vs) {
    const float alpha = mask_and_ref(sc, u);
    if (has_next) qk(sn, u + 1, ks);
    softmax_p(sc, pcur);
    if (has_prev) pv(pprev, u - 1, vs);
    // Scheduling hint for this unit's region: the compiler's "small GEMM"
    // interleave, which issues the LDS operand reads in pairs one MFMA ahead
    // of the MFMA that consumes them (measured 4 % faster than its default
    // order on a 131072-key block; the arithmetic is unchanged).
    __builtin_amdgcn_iglp_opt(0);
    rescale_o(alpha);
  };

  if (NW == 8 && n_kt > 0) {
    // Pipeline. Unit u reads K of tile (u+1)/2 (for S(u+1)) and V of tile
    // (u-1)/2 (for the P.V of P(u-1)). A step T runs units 4T+1 .. 4T+4, so
    // it reads K tiles 2T+1, 2T+2 and V tiles 2T, 2T+1. It first issues the
    // DMA of what step T+1 reads (K tiles 2T+3, 2T+4, V tiles 2T+2, 2T+3)
    // into the slots whose last reader was step T-1, and ends with each wave
    // waiting for its own loads and one barrier: the barrier makes the next
    // step's tiles visible to every wave and frees this step's slots. One
    // barrier per 128 keys, with the loads 128 keys ahead of their use.
    // Tiles past the last one are loaded (clamped rows) but never read.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // Q fragments
    issue_k(0);
    issue_k(1);
    issue_v(0);
    issue_v(1);
    issue_k(2);
    // K tile 0 (issued first) has landed once at most four tiles of this
    // wave's loads are in flight
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(4 * Dma::LPW) : "memory");

    const int n_u = (key_end + 31) / 32;  // units with any visible key
    f32x16 sA, sB;
    bf16x8 pA[2], pB[2];
    qk(sA, 0, 0);
    unit(sA, sB, pB, pA, 0, n_u > 1, false, 0, 0);  // S(1) -> sB, P(0) -> pA
    // the rest of the prologue's tiles have landed, and K slot 0 (read by
    // unit 0) is free for step 0's loads
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    // odd units keep S in sB and P in pB, even units S in sA and P in pA
    int T = 0;
    for (; 4 * T + 5 < n_u; ++T) {
      issue_k(2 * T + 3);
      issue_k(2 * T + 4);
      issue_v(2 * T + 2);
      issue_v(2 * T + 3);
      unit(sB, sA, pA, pB, 4 * T + 1, true, true, 2 * T + 1, 2 * T);
      unit(sA, sB, pB, pA, 4 * T + 2, true, true, 2 * T + 1, 2 * T);
      unit(sB, sA, pA, pB, 4 * T + 3, true, true, 2 * T + 2, 2 * T + 1);
      unit(sA, sB, pB, pA, 4 * T + 4, true, true, 2 * T + 2, 2 * T + 1);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // tail: units 4T+1 .. n_u-1 (at most four). Their K tiles (up to 2T+2) and
    // V tiles (up to 2T+1) are in place; the P.V of unit 4T+4 would read V
    // tile 2T+2, whose slot step T-1 freed.
    const int u0 = 4 * T + 1;
    if (u0 + 3 < n_u) {
      issue_v(2 * T + 2);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (u0 < n_u) {
      unit(sB, sA, pA, pB, u0, u0 + 1 < n_u, true, 2 * T + 1, 2 * T);
      if (u0 + 1 < n_u) {
        unit(sA, sB, pB, pA, u0 + 1, u0 + 2 < n_u, true, 2 * T + 1, 2 * T);
        if (u0 + 2 < n_u) {
          unit(sB, sA, pA, pB, u0 + 2, u0 + 3 < n_u, true, 2 * T + 2, 2 * T + 1);
          if (u0 + 3 < n_u) {
            unit(sA, sB, pB, pA, u0 + 3, false, true, 2 * T + 2, 2 * T + 1);
            pv(pA, u0 + 3, 2 * T + 2);
          } else {
            pv(pB, u0 + 2, 2 * T + 1);
          }
        } else {
          pv(pA, u0 + 1, 2 * T + 1);
        }
      } else {
        pv(pB, u0, 2 * T);
      }
    } else {
      pv(pA, u0 - 1, 2 * T);
    }
  }

  if (NW != 8 && n_kt > 0) {
    // Pipeline of a 4-wave workgroup (two per CU, 2 + 2 ring slots). A step t
    // runs units 2t+1, 2t+2: it reads K tile t+1 and V tile t, and first
    // issues K tile t+2 and V tile t+1 into the slots step t-1 read; it ends
    // with each wave waiting for its own loads and one barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // Q fragments
    issue_k(0);
    issue_k(1);
    issue_v(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * Dma::LPW) : "memory");
    const int n_u = (key_end + 31) / 32;
    f32x16 sA, sB;
    bf16x8 pA[2], pB[2];
    qk(sA, 0, 0);
    unit(sA, sB, pB, pA, 0, n_u > 1, false, 0, 0);
    // K tile 1 and V tile 0 have landed, and K slot 0 (read by unit 0) is free
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    int t = 0;
    for (; 2 * t + 3 < n_u; ++t) {
      issue_k(t + 2);
      issue_v(t + 1);
      unit(sB, sA, pA, pB, 2 * t + 1, true, true, t + 1, t);
      unit(sA, sB, pB, pA, 2 * t + 2, true, true, t + 1, t);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // tail: units 2t+1, 2t+2 (at most two) read K tile t+1 and V tile t; the
    // P.V of unit 2t+2 reads V tile t+1, whose slot step t-1 freed
    const int u0 = 2 * t + 1;
    if (u0 + 1 < n_u) {
      issue_v(t + 1);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (u0 < n_u) {
      unit(sB, sA, pA, pB, u0, u0 + 1 < n_u, true, t + 1, t);
      if (u0 + 1 < n_u) {
        unit(sA, sB, pB, pA, u0 + 1, false, true, t + 1, t);
        pv(pA, u0 + 1, t + 1);
      } else {
        pv(pB, u0, t);
      }
    } else {
      pv(pA, u0 - 1, t);
    }
  }

  // convert (l, O) from the reference `base` to the exact running max
  if (base != kNegInf) {
    const float f = fast_exp2(base - m_run);
    l_run *= f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= f;
  }

  // ---- epilogue: (m, l, acc) with m in natural units, written, or merged
  // into the running state (both lanes of a row read m and l before the
  // half-0 lane writes them); with finalize the divided output and lse
  const float lt = sum_xor32(l_run);
  if (row_ok) {
    const int64_t r = ((int64_t)b * p.q_len + tr.row0 + row_a) * p.hq + row_h;
    const float mp = (m_run == kNegInf) ? kNegInf : m_run * kLn2;
    float* arow = p.acc + r * D;
    float f1 = 0.f, f2 = 1.0f, mo = mp, lo = lt;
    if (p.accumulate) {
      const float l_old = p.l[r];
      const MergeCoef c = merge_coef(p.m[r], mp);
      f1 = c.f1;
      f2 = c.f2;
      mo = c.mm;
      lo = c.f1 * l_old + c.f2 * lt;
    }
    const float inv = p.finalize ? finalize_inv(lo) : 1.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * half;
        if (d < D) {
          f32x4 o;
          if (p.accumulate) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(arow + d);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = f1 * w[i] + f2 * oacc[db][4 * u + i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = oacc[db][4 * u + i];
          }
          if (p.finalize) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] *= inv;
          }
          *reinterpret_cast<f32x4*>(arow + d) = o;
        }
      }
    if (half == 0) {
      p.m[r] = mo;
      p.l[r] = lo;
      if (p.finalize && p.lse != nullptr) p.lse[r] = finalize_lse(mo, lo);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA attention partial (exact per-key online update)
// ---------------------------------------------------------------------------
constexpr int kF32TK = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_fma(AttnParams p) {
  constexpr int DC = D < 32 ? D : 32;     // dims per thread
  constexpr int TPR = D / DC;             // threads per row
  constexpr int ROWS = kThreads / TPR;    // rows per workgroup
  __shared__ float sK[kF32TK][D];
  __shared__ float sV[kF32TK][D];

  const int tid = threadIdx.x;
  const TileRef tr = locate_tile(p);
  const int b = tr.b, g = tr.g;
  const int kv_len = tr.kv_len;
  const int rows_total = tr.rows;
  const int rho0 = tr.tile * ROWS;
  const int rho_last = min(rho0 + ROWS, rows_total) - 1;
  const int a_hi = rho_last / p.group;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int key_end = (int)ra::key_end(geom, a_hi, kv_len);

  const int rho = rho0 + tid / TPR;
  const int part = tid % TPR;
  const bool ok = rho < rows_total;
  const int rr = ok ? rho : rows_total - 1;
  const int a = rr / p.group;
  const int h = g * p.group + (rr - a * p.group);

  const float* __restrict__ qg =
      reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_bstride + (int64_t)tr.row0 * p.hq * D;
  const int64_t kv_row_stride = (int64_t)p.hkv * D;
  const int64_t kv_base = (int64_t)b * p.kv_bstride + (int64_t)tr.key0 * kv_row_stride + (int64_t)g * D;
  const float* __restrict__ kgp = reinterpret_cast<const float*>(p.k) + kv_base;
  const float* __restrict__ vgp = reinterpret_cast<const float*>(p.v) + kv_base;

  float qv[DC], acc[DC];
  const float* qrow = qg + ((int64_t)a * p.hq + h) * D + part * DC;
#pragma unroll
  for (int i = 0; i < DC; ++i) {
    qv[i] = ok ? qrow[i] : 0.f;
    acc[i] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const float sl2 = p.scale_log2;

  for (int key0 = 0; key0 < key_end; key0 += kF32TK) {
    for (int e = tid; e < kF32TK * D; e += kThreads) {
      int kk = e / D, d = e % D;
      int key = key0 + kk;
      sK[kk][d] = key < kv_len ? kgp[(int64_t)key * kv_row_stride + d] : 0.f;
      sV[kk][d] = key < kv_len ? vgp[(int64_t)key * kv_row_stride + d] : 0.f;
    }
    __syncthreads();
    const int nk = min(kF32TK, key_end - key0);
    for (int kk = 0; kk < nk; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < DC; ++i) dot = __builtin_fmaf(qv[i], sK[kk][part * DC + i], dot);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) dot += __shfl_xor(dot, o);
      const int key = key0 + kk;
      if (visible(geom, a, key, kv_len)) {
        const float x = dot * sl2;
        const float m_new = fmaxf(m, x);
        const float alpha = fast_exp2(m - m_new);
        const float e = fast_exp2(x - m_new);
        l = l * alpha + e;
#pragma unroll
        for (int i = 0; i < DC; ++i) acc[i] = __builtin_fmaf(e, sV[kk][part * DC + i], acc[i] * alpha);
        m = m_new;
      }
    }
    __syncthreads();
  }

  if (ok) {
    const int64_t r = ((int64_t)b * p.q_len + tr.row0 + a) * p.hq + h;
    const float mp = (m == kNegInf) ? kNegInf : m * kLn2;
    float* arow = p.acc + r * D + part * DC;
    // the row's TPR threads share a wave: all read m and l before part 0 writes
    float f1 = 0.f, f2 = 1.0f, mo = mp, lo = l;
    if (p.accumulate) {
      const float l_old = p.l[r];
      const MergeCoef c = merge_coef(p.m[r], mp);
      f1 = c.f1;
      f2 = c.f2;
      mo = c.mm;
      lo = c.f1 * l_old + c.f2 * l;
    }
    const float inv = p.finalize ? finalize_inv(lo) : 1.0f;
#pragma unroll
    for (int i = 0; i < DC; i += 4) {
      f32x4 o;
      if (p.accumulate) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(arow + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f1 * w[e] + f2 * acc[i + e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[i + e];
      }
      if (p.finalize) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= inv;
      }
      *reinterpret_cast<f32x4*>(arow + i) = o;
    }
    if (part == 0) {
      p.m[r] = mo;
      p.l[r] = lo;
      if (p.finalize && p.lse != nullptr) p.lse[r] = finalize_lse(mo, lo);
    }
  }
}

// ---------------------------------------------------------------------------
// merge, finalize, fill, tile classes
// ---------------------------------------------------------------------------
// One thread per 4 consecutive accumulator elements. A row's D/4 threads are
// consecutive and D/4 divides 64, so every row lies inside one wavefront: all
// of its lanes read m/l before the lane that writes them (outputs may alias
// an input exactly).
__global__ __launch_bounds__(kThreads) void merge_partials_kernel(
    int64_t rows, int vec_per_row, const float* m1, const float* l1, const f32x4* a1,
    const float* m2, const float* l2, const f32x4* a2, float* mo, float* lo, f32x4* ao) {
  const int64_t total = rows * vec_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / vec_per_row;
    const MergeCoef c = merge_coef(m1[row], m2[row]);
    const f32x4 u = a1[i], w = a2[i];
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = c.f1 * u[e] + c.f2 * w[e];
    float nl = 0.f;
    const bool writer = (i - row * vec_per_row) == 0;
    if (writer) nl = c.f1 * l1[row] + c.f2 * l2[row];
    ao[i] = o;
    if (writer) {
      mo[row] = c.mm;
      lo[row] = nl;
    }
  }
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(int64_t rows, int vec_per_row,
                                                             const float* m, const float* l,
                                                             f32x4* acc, float* lse) {
  const int64_t total = rows * vec_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / vec_per_row;
    const float L = l[row];
    const float inv = finalize_inv(L);
    f32x4 x = acc[i];
    x[0] *= inv;
    x[1] *= inv;
    x[2] *= inv;
    x[3] *= inv;
    acc[i] = x;
    if (lse != nullptr && (i - row * vec_per_row) == 0)
      lse[row] = finalize_lse(m[row], L);
  }
}

__global__ __launch_bounds__(kThreads) void fill_empty_kernel(int64_t rows, int vec_per_row,
                                                               float* m, float* l, f32x4* acc) {
  const int64_t total = rows * vec_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / vec_per_row;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((i - row * vec_per_row) == 0) {
      m[row] = kNegInf;
      l[row] = 0.f;
    }
  }
}

__global__ __launch_bounds__(kThreads) void tile_classes_kernel(int kind, int delta, int64_t q_len,
                                                                 int64_t kv_len, int tq, int tk,
                                                                 int64_t nqt, int64_t nkt,
                                                                 int packed, SegTable seg,
                                                                 int8_t* out) {
  const int64_t total = nqt * nkt;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const BlockGeom geom{kind, delta};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t qt = i / nkt, kt = i - qt * nkt;
    const int64_t a_lo = qt * tq, a_hi = min(a_lo + tq, q_len) - 1;
    const int64_t b_lo = kt * tk, b_hi = min(b_lo + tk, kv_len) - 1;
    out[i] = (int8_t)(packed ? tile_class_packed(geom, seg, a_lo, a_hi, b_lo, b_hi)
                             : tile_class(geom, a_lo, a_hi, b_lo, b_hi, kv_len));
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int grid_for(int64_t total_threads) {
  int64_t blocks = (total_threads + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

// Row tiles of rows_per_tile rows per (segment, KV head); returns the total.
static int64_t set_tiles(AttnParams& p, int rows_per_tile) {
  int64_t total = 0;
  for (int s = 0; s < p.seg.n; ++s) {
    p.tile_off[s] = (int32_t)total;
    const int64_t rows = (int64_t)(p.seg.off[s + 1] - p.seg.off[s]) * p.group;
    total += (rows + rows_per_tile - 1) / rows_per_tile;
  }
  p.tile_off[p.seg.n] = (int32_t)total;
  p.tiles_total = (int32_t)total;
  return total;
}

// Kernels that use more than 64 KiB of dynamic LDS need the limit raised once
// per (kernel, device); the pairs already done are remembered.
hipError_t allow_dynamic_lds(const void* kern, size_t bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kern, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.insert({kern, dev});
  return e;
}

template <int D, int NW>
static hipError_t launch_bf16(AttnParams p, hipStream_t stream) {
  constexpr int ROWS = 32 * NW;
  const int64_t tiles = set_tiles(p, ROWS);
  // the K ring then the V ring
  const size_t smem = 2 * kFwdSlots<NW> * (size_t)(kPadTile<D, NW> ? KvTile128::TB : BfTile<D>::TB);
  auto kern = attn_bf16_mfma<D, NW>;
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), smem);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)p.batch * p.hkv * tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), smem, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(AttnParams p, hipStream_t stream) {
  constexpr int DC = D < 32 ? D : 32;
  constexpr int ROWS = kThreads / (D / DC);
  const int64_t grid = (int64_t)p.batch * p.hkv * set_tiles(p, ROWS);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_fma<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

TileShape fwd_tile_shape(int is_bf16, int head_dim, int waves) {
  if (is_bf16) return TileShape{32 * waves, 64 * waves, 0};
  const int dc = head_dim < 32 ? head_dim : 32;  // attn_f32_fma: one thread per (row, 32 dims)
  return TileShape{kThreads / (head_dim / dc), kThreads, 0};
}

hipError_t launch_attention(const AttnParams& p, int is_bf16, int waves, hipStream_t stream) {
  if (is_bf16) {
    if (waves == 4) {
      switch (p.head_dim) {
        case 16: return launch_bf16<16, 4>(p, stream);
        case 32: return launch_bf16<32, 4>(p, stream);
        case 64: return launch_bf16<64, 4>(p, stream);
        case 128: return launch_bf16<128, 4>(p, stream);
      }
    } else {
      switch (p.head_dim) {
        case 16: return launch_bf16<16, 8>(p, stream);
        case 32: return launch_bf16<32, 8>(p, stream);
        case 64: return launch_bf16<64, 8>(p, stream);
        case 128: return launch_bf16<128, 8>(p, stream);
      }
    }
  } else {
    switch (p.head_dim) {
      case 16: return launch_f32<16>(p, stream);
      case 32: return launch_f32<32>(p, stream);
      case 64: return launch_f32<64>(p, stream);
      case 128: return launch_f32<128>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int64_t rows, int d, const float* m1, const float* l1, const float* a1,
                        const float* m2, const float* l2, const float* a2, float* mo, float* lo,
                        float* ao, hipStream_t stream) {
  const int vpr = d / 4;
  hipLaunchKernelGGL(merge_partials_kernel, dim3(grid_for(rows * vpr)), dim3(kThreads), 0, stream,
                     rows, vpr, m1, l1, reinterpret_cast<const f32x4*>(a1), m2, l2,
                     reinterpret_cast<const f32x4*>(a2), mo, lo, reinterpret_cast<f32x4*>(ao));
  return hipGetLastError();
}

hipError_t launch_finalize(int64_t rows, int d, const float* m, const float* l, float* acc,
                           float* lse, hipStream_t stream) {
  const int vpr = d / 4;
  hipLaunchKernelGGL(finalize_kernel, dim3(grid_for(rows * vpr)), dim3(kThreads), 0, stream, rows,
                     vpr, m, l, reinterpret_cast<f32x4*>(acc), lse);
  return hipGetLastError();
}

hipError_t launch_fill_empty(int64_t rows, int d, float* m, float* l, float* acc,
                             hipStream_t stream) {
  const int vpr = d / 4;
  hipLaunchKernelGGL(fill_empty_kernel, dim3(grid_for(rows * vpr)), dim3(kThreads), 0, stream,
                     rows, vpr, m, l, reinterpret_cast<f32x4*>(acc));
  return hipGetLastError();
}

hipError_t launch_tile_classes(int kind, int delta, int64_t q_len, int64_t kv_len, int tq, int tk,
                               const SegTable* seg, int8_t* out, hipStream_t stream) {
  const int64_t nqt = (q_len + tq - 1) / tq, nkt = (kv_len + tk - 1) / tk;
  SegTable t{};
  if (seg) t = *seg;
  hipLaunchKernelGGL(tile_classes_kernel, dim3(grid_for(nqt * nkt)), dim3(kThreads), 0, stream,
                     kind, delta, q_len, kv_len, tq, tk, nqt, nkt, seg ? 1 : 0, t, out);
  return hipGetLastError();
}

}  // namespace ra
