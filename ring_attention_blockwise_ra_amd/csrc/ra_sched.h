// ra_sched.h -- causal tile rule shared by the host mirror and the kernels.
//
// Global positions (troisinh "Ring Attention -- K/V truyen vong giua GPU",
// section "Y tuong cot loi" for contiguous chunks; Ultralytics "Ring
// Attention", section "How ring attention works", closing remark, for the
// striped assignment):
//   contiguous: query a of rank r sits at r*B + a, key b of block j at j*B + b
//   striped:    query a of rank r sits at a*N + r, key b of block j at b*N + j
// A key is visible iff its position <= the query's (autoregressive mask,
// troisinh section "Y nghia thuc te"). With q_len == kv_len == B this
// reduces to one of three block kinds:
//   contiguous: j < r every pair visible; j > r none; j == r visible iff b <= a
//   striped:    visible iff b <= a - delta with delta = (j > r)
// (b*N + j <= a*N + r  <=>  b <= a + (r - j)/N, and 0 <= |r - j| < N).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

enum BlockKind : int32_t { kAllVisible = 0, kNoneVisible = 1, kDiagonal = 2 };
enum TileClass : int32_t { kSkip = 0, kPartial = 1, kFull = 2 };

struct BlockGeom {
  int32_t kind;
  int32_t delta;  // only for kDiagonal: visible iff b <= a - delta
};

RA_HD BlockGeom block_geom(int32_t causal, int32_t layout, int32_t rank, int32_t j) {
  BlockGeom g{kAllVisible, 0};
  if (!causal) return g;
  if (layout == 0) {  // contiguous
    if (j < rank) return g;
    if (j > rank) { g.kind = kNoneVisible; return g; }
    g.kind = kDiagonal;
    return g;
  }
  g.kind = kDiagonal;  // striped
  g.delta = (j > rank) ? 1 : 0;
  return g;
}

// Class of query rows [a_lo, a_hi] x keys [b_lo, b_hi] (inclusive, in range).
RA_HD int32_t tile_class(BlockGeom g, int64_t a_lo, int64_t a_hi, int64_t b_lo, int64_t b_hi) {
  if (g.kind == kAllVisible) return kFull;
  if (g.kind == kNoneVisible) return kSkip;
  if (b_hi <= a_lo - g.delta) return kFull;
  if (b_lo > a_hi - g.delta) return kSkip;
  return kPartial;
}

// Number of leading keys [0, n) any of the rows <= a_hi can see.
RA_HD int64_t key_end_any(BlockGeom g, int64_t a_hi, int64_t kv_len) {
  if (g.kind == kAllVisible) return kv_len;
  if (g.kind == kNoneVisible) return 0;
  int64_t e = a_hi - g.delta + 1;
  return e < 0 ? 0 : (e > kv_len ? kv_len : e);
}

// Number of leading keys [0, n) every row >= a_lo can see.
RA_HD int64_t key_end_all(BlockGeom g, int64_t a_lo, int64_t kv_len) {
  return key_end_any(g, a_lo, kv_len);
}

// Element rule (used inside PARTIAL tiles).
RA_HD bool visible(BlockGeom g, int64_t a, int64_t b) {
  if (g.kind == kAllVisible) return true;
  if (g.kind == kNoneVisible) return false;
  return b <= a - g.delta;
}

}  // namespace ra
