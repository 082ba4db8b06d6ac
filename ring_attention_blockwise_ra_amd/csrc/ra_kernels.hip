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

#include "ra_kernels.h"
#include "ra_sched.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

constexpr int kThreads = 256;  // workgroup size of the fp32 and elementwise kernels
constexpr int kTK = 64;

template <int D>
struct BfTile {
  static constexpr int DP = D < 32 ? 32 : D;       // head dims padded to the MFMA M of 32
  static constexpr int KS = D + 8;                 // K row stride (bf16): 16-byte reads
                                                   // of 8 rows hit distinct banks
  static constexpr int VS = DP + 16;               // V row stride (bf16): the 4 rows of a
                                                   // transposed read hit distinct banks
  static constexpr int K_ELEMS = kTK * KS;
  static constexpr int V_ELEMS = kTK * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;    // one stage, bf16 elements
  static constexpr int CHUNKS = kTK * D / 8;       // 16-byte chunks of a K (or V) tile
};

template <int D, int NT>
struct KVRegs {
  static constexpr int IT = (BfTile<D>::CHUNKS + NT - 1) / NT;
  static constexpr bool EXACT = BfTile<D>::CHUNKS % NT == 0;
  u32x4 k[IT];
  u32x4 v[IT];
};

// Global -> registers without branches: key rows past kv_len re-read the last
// row. Those keys are masked to -inf before the softmax (their weight is 0),
// so what they hold never reaches the output.
template <int D, int NT>
__device__ __forceinline__ void load_kv_tile(KVRegs<D, NT>& r, const uint16_t* __restrict__ kp,
                                             const uint16_t* __restrict__ vp, int64_t row_stride,
                                             int key0, int kv_len, int tid) {
  using R = KVRegs<D, NT>;
#pragma unroll
  for (int it = 0; it < R::IT; ++it) {
    const int c = tid + it * NT;
    if (R::EXACT || c < BfTile<D>::CHUNKS) {
      const int key = min(key0 + c / (D / 8), kv_len - 1);
      const int64_t off = (int64_t)key * row_stride + (c % (D / 8)) * 8;
      r.k[it] = *reinterpret_cast<const u32x4*>(kp + off);
      r.v[it] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void store_kv_tile(const KVRegs<D, NT>& r, uint16_t* sbuf, int tid) {
  using T = BfTile<D>;
  using R = KVRegs<D, NT>;
#pragma unroll
  for (int it = 0; it < R::IT; ++it) {
    const int c = tid + it * NT;
    if (R::EXACT || c < T::CHUNKS) {
      const int key = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(sbuf + key * T::KS + col) = r.k[it];
      *reinterpret_cast<u32x4*>(sbuf + T::K_ELEMS + key * T::VS + col) = r.v[it];
    }
  }
}

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

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_mfma(AttnParams p) {
  using T = BfTile<D>;
  constexpr int NT = NW * 64;
  constexpr int ROWS = 32 * NW;
  constexpr int KSTEPS = D / 16;
  constexpr int KB = kTK / 32;   // 32-key blocks per tile
  constexpr int KC = kTK / 16;   // 16-key chunks per tile
  constexpr int DB = T::DP / 32; // 32-dim blocks of the output

  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // heavy tiles first (causal blocks: larger local index -> more keys)
  int bid = blockIdx.x;
  const int per_b = p.hkv * p.n_row_tiles;
  const int b = bid / per_b;
  bid -= b * per_b;
  const int g = bid / p.n_row_tiles;
  const int tile = p.n_row_tiles - 1 - (bid - g * p.n_row_tiles);

  const int rows_total = p.rows_per_bg;
  const int rho0 = tile * ROWS;
  const int rho_last = min(rho0 + ROWS, rows_total) - 1;
  const int a_lo = rho0 / p.group;
  const int a_hi = rho_last / p.group;

  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int key_end = (int)key_end_any(geom, a_hi, p.kv_len);
  const int full_end = (int)key_end_all(geom, a_lo, p.kv_len);
  const int n_kt = (key_end + kTK - 1) / kTK;

  const uint16_t* __restrict__ qg = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_bstride;
  const int64_t kv_row_stride = (int64_t)p.hkv * D;
  const uint16_t* __restrict__ kg =
      reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.kv_bstride + (int64_t)g * D;
  const uint16_t* __restrict__ vg =
      reinterpret_cast<const uint16_t*>(p.v) + (int64_t)b * p.kv_bstride + (int64_t)g * D;

  // this lane's query row
  const int rho = rho0 + wave * 32 + col;
  const bool row_ok = rho < rows_total;
  const int rr = row_ok ? rho : rows_total - 1;
  const int row_a = rr / p.group;
  const int row_h = g * p.group + (rr - row_a * p.group);
  // last key index visible to this row (keys past kv_len are never visible)
  const int lim = geom.kind == kAllVisible ? p.kv_len - 1
                : (geom.kind == kNoneVisible ? -1 : min(row_a - geom.delta, p.kv_len - 1));

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

  // per-lane offsets of the two LDS operand reads
  const int k_lane = col * T::KS + 8 * half;
  const int grp = lane >> 4, sl = lane & 15;
  const int v_lane = (4 * (grp >> 1) + (sl >> 2)) * T::VS + 16 * (grp & 1) + 4 * (sl & 3);

  if (n_kt > 0) {
    KVRegs<D, NT> regs;
    load_kv_tile<D, NT>(regs, kg, vg, kv_row_stride, 0, p.kv_len, tid);
    store_kv_tile<D, NT>(regs, smem, tid);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
      const uint16_t* sbuf = smem + (kt & 1) * T::BUF;
      const bool have_next = kt + 1 < n_kt;
      if (have_next) load_kv_tile<D, NT>(regs, kg, vg, kv_row_stride, (kt + 1) * kTK, p.kv_len, tid);

      // ---- S^T = K Q^T --------------------------------------------------
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          bf16x8 a = *reinterpret_cast<const bf16x8*>(sbuf + k_lane + kb * 32 * T::KS + 16 * t);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
        }
      }

      // ---- mask (tiles crossing the diagonal or the ragged tail) --------
      const int key0 = kt * kTK;
      if (key0 + kTK > full_end) {
        const int rel = lim - key0 - 4 * half;  // visible iff 8*(i/4) + i%4 + 32*kb <= rel
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + 8 * (i >> 2) + (i & 3) > rel) s[kb][i] = kNegInf;
      }

      // ---- online softmax (exp2 domain) --------------------------------
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      mt = max_xor32(mt);
      const float m_new = fmaxf(m_run, mt * sl2);
      const float base = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - base);
      m_run = m_new;
      bf16x8 pf[KC];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x8 e8;
#pragma unroll
          for (int j = 0; j < 8; ++j) e8[j] = fast_exp2(__builtin_fmaf(s[kb][8 * c2 + j], sl2, -base));
          const bf16x8 pb = __builtin_convertvector(e8, bf16x8);
          pf[kb * 2 + c2] = pb;
          // row sum of the rounded weights (the same ones the numerator uses)
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), ones, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), ones, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), ones, ls, false);
        }
      }
      l_run = alpha * l_run + ls;
      if (!__all(alpha == 1.0f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }

      // ---- O^T += V^T P^T ------------------------------------------------
      const uint16_t* sV = sbuf + T::K_ELEMS + v_lane;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const s16x4 lo = lds_read_tr16(sV + (c * 16) * T::VS + db * 32);
          const s16x4 hi = lds_read_tr16(sV + (c * 16 + 8) * T::VS + db * 32);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], oacc[db], 0, 0, 0);
        }
      }

      if (have_next) store_kv_tile<D, NT>(regs, smem + ((kt + 1) & 1) * T::BUF, tid);
      __syncthreads();
    }
  }

  // ---- epilogue: (m, l, acc) with m in natural units --------------------
  const float lt = sum_xor32(l_run);
  if (row_ok) {
    const int64_t r = ((int64_t)b * p.q_len + row_a) * p.hq + row_h;
    if (half == 0) {
      p.m[r] = (m_run == kNegInf) ? kNegInf : m_run * kLn2;
      p.l[r] = lt;
    }
    float* arow = p.acc + r * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + 8 * u + 4 * half;
        if (d < D) {
          f32x4 o = {oacc[db][4 * u], oacc[db][4 * u + 1], oacc[db][4 * u + 2], oacc[db][4 * u + 3]};
          *reinterpret_cast<f32x4*>(arow + d) = o;
        }
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
  int bid = blockIdx.x;
  const int per_b = p.hkv * p.n_row_tiles;
  const int b = bid / per_b;
  bid -= b * per_b;
  const int g = bid / p.n_row_tiles;
  const int tile = p.n_row_tiles - 1 - (bid - g * p.n_row_tiles);

  const int rows_total = p.rows_per_bg;
  const int rho0 = tile * ROWS;
  const int rho_last = min(rho0 + ROWS, rows_total) - 1;
  const int a_hi = rho_last / p.group;
  const BlockGeom geom{p.geom_kind, p.geom_delta};
  const int key_end = (int)key_end_any(geom, a_hi, p.kv_len);

  const int rho = rho0 + tid / TPR;
  const int part = tid % TPR;
  const bool ok = rho < rows_total;
  const int rr = ok ? rho : rows_total - 1;
  const int a = rr / p.group;
  const int h = g * p.group + (rr - a * p.group);

  const float* __restrict__ qg = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_bstride;
  const float* __restrict__ kgp =
      reinterpret_cast<const float*>(p.k) + (int64_t)b * p.kv_bstride + (int64_t)g * D;
  const float* __restrict__ vgp =
      reinterpret_cast<const float*>(p.v) + (int64_t)b * p.kv_bstride + (int64_t)g * D;
  const int64_t kv_row_stride = (int64_t)p.hkv * D;

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
      sK[kk][d] = key < p.kv_len ? kgp[(int64_t)key * kv_row_stride + d] : 0.f;
      sV[kk][d] = key < p.kv_len ? vgp[(int64_t)key * kv_row_stride + d] : 0.f;
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
      if (visible(geom, a, key)) {
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
    const int64_t r = ((int64_t)b * p.q_len + a) * p.hq + h;
    if (part == 0) {
      p.m[r] = (m == kNegInf) ? kNegInf : m * kLn2;
      p.l[r] = l;
    }
    float* arow = p.acc + r * D + part * DC;
#pragma unroll
    for (int i = 0; i < DC; i += 4) {
      f32x4 o = {acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
      *reinterpret_cast<f32x4*>(arow + i) = o;
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
    const float x1 = m1[row], x2 = m2[row];
    const float mm = fmaxf(x1, x2);
    const float f1 = (x1 == kNegInf) ? 0.f : expf(x1 - mm);
    const float f2 = (x2 == kNegInf) ? 0.f : expf(x2 - mm);
    const f32x4 u = a1[i], w = a2[i];
    f32x4 o;
    o[0] = f1 * u[0] + f2 * w[0];
    o[1] = f1 * u[1] + f2 * w[1];
    o[2] = f1 * u[2] + f2 * w[2];
    o[3] = f1 * u[3] + f2 * w[3];
    float nl = 0.f;
    const bool writer = (i - row * vec_per_row) == 0;
    if (writer) nl = f1 * l1[row] + f2 * l2[row];
    ao[i] = o;
    if (writer) {
      mo[row] = mm;
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
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    f32x4 x = acc[i];
    x[0] *= inv;
    x[1] *= inv;
    x[2] *= inv;
    x[3] *= inv;
    acc[i] = x;
    if (lse != nullptr && (i - row * vec_per_row) == 0)
      lse[row] = L > 0.f ? m[row] + logf(L) : kNegInf;
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
                                                                 int8_t* out) {
  const int64_t total = nqt * nkt;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const BlockGeom geom{kind, delta};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t qt = i / nkt, kt = i - qt * nkt;
    const int64_t a_lo = qt * tq, a_hi = min(a_lo + tq, q_len) - 1;
    const int64_t b_lo = kt * tk, b_hi = min(b_lo + tk, kv_len) - 1;
    out[i] = (int8_t)tile_class(geom, a_lo, a_hi, b_lo, b_hi);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int grid_for(int64_t total_threads) {
  int64_t blocks = (total_threads + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

template <int D, int NW>
static hipError_t launch_bf16(AttnParams p, hipStream_t stream) {
  constexpr int ROWS = 32 * NW;
  p.n_row_tiles = (p.rows_per_bg + ROWS - 1) / ROWS;
  const size_t smem = 2 * BfTile<D>::BUF * sizeof(uint16_t);
  auto kern = attn_bf16_mfma<D, NW>;
  static bool attr_set = false;  // per instantiation; benign race (idempotent)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t grid = (int64_t)p.batch * p.hkv * p.n_row_tiles;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), smem, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(AttnParams p, hipStream_t stream) {
  constexpr int DC = D < 32 ? D : 32;
  constexpr int ROWS = kThreads / (D / DC);
  p.n_row_tiles = (p.rows_per_bg + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)p.batch * p.hkv * p.n_row_tiles;
  hipLaunchKernelGGL(attn_f32_fma<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
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
                               int8_t* out, hipStream_t stream) {
  const int64_t nqt = (q_len + tq - 1) / tq, nkt = (kv_len + tk - 1) / tk;
  hipLaunchKernelGGL(tile_classes_kernel, dim3(grid_for(nqt * nkt)), dim3(kThreads), 0, stream,
                     kind, delta, q_len, kv_len, tq, tk, nqt, nkt, out);
  return hipGetLastError();
}

}  // namespace ra
