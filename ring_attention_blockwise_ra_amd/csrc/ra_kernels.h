// ra_kernels.h -- launch interface between the C ABI layer and the kernels
// (library-internal; not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_sched.h"

namespace ra {

struct AttnParams {
  const void* q;        // [batch, q_len, hq, D]
  const void* k;        // [batch, kv_len, hkv, D] (one block)
  const void* v;
  float* m;             // [batch, q_len, hq]
  float* l;
  float* acc;           // [batch, q_len, hq, D]
  int64_t q_bstride;    // elements per batch of q
  int64_t kv_bstride;   // elements per batch of k / v
  int32_t batch;
  int32_t q_len;
  int32_t kv_len;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  int32_t group;        // hq / hkv
  int32_t packed;       // 1: segment s also owns keys [off[s], off[s+1])
  int32_t accumulate;   // 1: merge the block's partial into (m, l, acc) in place
  int32_t finalize;     // 1: also divide: acc <- acc / l, lse <- m + ln l (lse may be null)
  float* lse;           // [batch, q_len, hq] when finalize
  int32_t tiles_total;  // set by the launcher: row tiles over all segments
  int32_t geom_kind;    // ra::BlockKind
  int32_t geom_delta;
  float scale_log2;     // scale * log2(e)
  SegTable seg;         // local row segments (one segment without packing)
  int32_t tile_off[kMaxSegs + 1];  // set by the launcher: first tile of each segment
};

// Backward pass of one block: dq += its dQ addend, dk/dv += its dK/dV addends.
struct BwdParams {
  const void* q;        // [batch, q_len, hq, D]
  const void* k;        // [batch, kv_len, hkv, D] (one block)
  const void* v;
  const void* dout;     // [batch, q_len, hq, D], same dtype as q
  const float* lse;     // [batch, q_len, hq], natural log
  const float* delta;   // [batch, q_len, hq]: rowsum(dout * out)
  float* dq;            // [batch, q_len, hq, D], accumulated
  float* dk;            // [batch, kv_len, hkv, D], accumulated
  float* dv;
  int64_t q_bstride;
  int64_t kv_bstride;
  int32_t batch;
  int32_t q_len;
  int32_t kv_len;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  int32_t group;
  int32_t packed;
  int32_t tiles_total;  // set by the launcher (row tiles or key tiles)
  int32_t geom_kind;
  int32_t geom_delta;
  float scale;          // natural units
  float scale_log2;     // scale * log2(e)
  SegTable seg;
  int32_t tile_off[kMaxSegs + 1];
};

// dq kernel then dk/dv kernel of one block, on one stream.
hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t stream);
// x[0 .. n) = 0 (n a multiple of 4), a kernel rather than a memset.
hipError_t launch_zero(float* x, int64_t n, hipStream_t stream);
// dst_a[0 .. bytes) = src_a and dst_b[0 .. bytes) = src_b in one kernel launch
// (bytes a multiple of 16; the regions must not overlap)
hipError_t launch_copy2(void* dst_a, const void* src_a, void* dst_b, const void* src_b,
                        int64_t bytes, hipStream_t stream);
// every 32-bit word of x[0 .. bytes) = value (bytes a multiple of 16), a kernel
hipError_t launch_fill_u32(void* x, int64_t bytes, uint32_t value, hipStream_t stream);
// delta[r] = sum_d dout[r, d] * out[r, d]; dout in the input dtype.
hipError_t launch_bwd_delta(int64_t rows, int d, int is_bf16, const float* out, const void* dout,
                            float* delta, hipStream_t stream);

// Rotary embedding of a block-shaped tensor [batch, len, heads, head_dim]:
// token a of block `block` at its global position (within its sequence when
// packed) turns head-dim pair (2i, 2i+1) by pos * inv_freq[i] (negated when
// inverse). y may equal x. accumulate: y += rotated x (float32 y only).
struct RopeParams {
  const void* x;
  void* y;
  int32_t in_bf16;
  int32_t out_bf16;
  int32_t accumulate;
  int32_t inverse;
  int32_t batch;
  int32_t len;
  int32_t heads;
  int32_t head_dim;
  int32_t layout;
  int32_t n_ring;
  int32_t block;
  int32_t packed;
  SegTable seg;
  double inv_freq[64];  // base^(-2i/head_dim), i < head_dim/2
};
hipError_t launch_rope(const RopeParams& p, hipStream_t stream);

// Raises the dynamic LDS limit of `kern` to `bytes` on the current device
// (once per kernel and device).
hipError_t allow_dynamic_lds(const void* kern, size_t bytes);

// waves: wavefronts per workgroup of the bf16 kernel (4 or 8; 32 rows each).
hipError_t launch_attention(const AttnParams& p, int is_bf16, int waves, hipStream_t stream);

// How a tiled kernel covers one (batch row, KV head): `per` query rows (the
// rows a*G + hh of the G grouped heads) or, with by_keys, `per` keys of the
// block per workgroup, with `threads` work items per workgroup; a packed
// share adds one partial tile per segment. The launchers tile with these
// numbers and the C ABI validates every launch's grid against them.
struct TileShape {
  int per;
  int threads;
  int by_keys;
};
TileShape fwd_tile_shape(int is_bf16, int head_dim, int waves);
// the backward's two launches: dq over query rows, then dk/dv over keys
void bwd_tile_shapes(int is_bf16, int head_dim, TileShape out[2]);

hipError_t launch_merge(int64_t rows, int d, const float* m1, const float* l1, const float* a1,
                        const float* m2, const float* l2, const float* a2, float* mo, float* lo,
                        float* ao, hipStream_t stream);
hipError_t launch_finalize(int64_t rows, int d, const float* m, const float* l, float* acc,
                           float* lse, hipStream_t stream);
hipError_t launch_fill_empty(int64_t rows, int d, float* m, float* l, float* acc,
                             hipStream_t stream);
// seg: NULL without packing
hipError_t launch_tile_classes(int kind, int delta, int64_t q_len, int64_t kv_len, int tq, int tk,
                               const SegTable* seg, int8_t* out, hipStream_t stream);

}  // namespace ra
