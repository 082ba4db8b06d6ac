// ra_sched.h -- causal tile rule shared by the host mirror and the kernels.
//
// Global positions (troisinh "Ring Attention -- K/V truyen vong giua GPU",
// section "Y tuong cot loi" for contiguous chunks; Ultralytics "Ring
// Attention", section "How ring attention works", closing remark, for the
// striped assignment; AI Understanding "Sekvensparallellism och
// ringuppmarksamhet", section "Framtiden for sekvensparallellism och
// ringuppmarksamhet", for zigzag as a rebalancing variant):
//   contiguous: query a of rank r sits at r*B + a, key b of block j at j*B + b
//   striped:    query a of rank r sits at a*N + r, key b of block j at b*N + j
//   zigzag:     2N chunks of h = B/2 tokens; block i holds chunk i (local
//               0..h-1) then chunk 2N-1-i (local h..B-1)
// A key is visible iff its position <= the query's (autoregressive mask,
// troisinh section "Y nghia thuc te"). In every layout local order follows
// position order, so the keys a query row a sees form a prefix [0, e(a)) of
// the block, and e(a) never decreases with a. With q_len == kv_len == B the
// prefix length e(a) is one of five block kinds:
//   contiguous: j < r all; j > r none; j == r diagonal (e = a + 1)
//   striped:    diagonal with delta = (j > r): e = a + 1 - delta
//               (b*N + j <= a*N + r  <=>  b <= a + (r - j)/N, |r - j| < N)
//   zigzag:     j == r diagonal; j < r key prefix (every row sees exactly
//               chunk j, e = h); j > r row suffix (rows of chunk 2N-1-r see
//               the whole block, rows of chunk r see nothing)
// Packed sequences (troisinh section "Trade-off thuc te": sequences of
// different lengths) split every sequence over the blocks on its own; a
// block is the concatenation of the slices, so a segment of local rows sees
// only the same segment of keys, under the rule above with B = its length.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

enum BlockKind : int32_t {
  kAllVisible = 0,
  kNoneVisible = 1,
  kDiagonal = 2,   // e(a) = a + 1 - delta
  kKeyPrefix = 3,  // e(a) = kv_len / 2
  kRowSuffix = 4,  // e(a) = kv_len if a >= kv_len / 2 else 0
};
enum TileClass : int32_t { kSkip = 0, kPartial = 1, kFull = 2 };

constexpr int kMaxSegs = 256;  // packed sequences per launch

struct BlockGeom {
  int32_t kind;
  int32_t delta;  // only for kDiagonal
};

// Local row offsets of the packed segments: segment s is rows
// [off[s], off[s+1]); n = 1 and off = {0, q_len} without packing.
struct SegTable {
  int32_t n;
  int32_t off[kMaxSegs + 1];
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
  if (layout == 2) {  // zigzag
    g.kind = j == rank ? kDiagonal : (j < rank ? kKeyPrefix : kRowSuffix);
    return g;
  }
  g.kind = kDiagonal;  // striped
  g.delta = (j > rank) ? 1 : 0;
  return g;
}

// Number of leading keys [0, e) of the block that row a sees.
RA_HD int64_t key_end(BlockGeom g, int64_t a, int64_t kv_len) {
  switch (g.kind) {
    case kAllVisible: return kv_len;
    case kNoneVisible: return 0;
    case kKeyPrefix: return kv_len / 2;
    case kRowSuffix: return a >= kv_len / 2 ? kv_len : 0;
    default: {
      const int64_t e = a - g.delta + 1;
      return e < 0 ? 0 : (e > kv_len ? kv_len : e);
    }
  }
}

// Class of query rows [a_lo, a_hi] x keys [b_lo, b_hi] (inclusive, in range).
// e is nondecreasing, so the first row sees the fewest keys and the last row
// the most.
RA_HD int32_t tile_class(BlockGeom g, int64_t a_lo, int64_t a_hi, int64_t b_lo, int64_t b_hi,
                         int64_t kv_len) {
  if (b_hi < key_end(g, a_lo, kv_len)) return kFull;
  if (b_lo >= key_end(g, a_hi, kv_len)) return kSkip;
  return kPartial;
}

// Element rule (used inside PARTIAL tiles).
RA_HD bool visible(BlockGeom g, int64_t a, int64_t b, int64_t kv_len) {
  return b < key_end(g, a, kv_len);
}

// Global position of local token a of block j (len tokens per block, or
// per block slice of one packed sequence): the layouts above.
RA_HD int64_t token_position(int32_t layout, int32_t n_ring, int32_t j, int64_t len, int64_t a) {
  if (layout == 0) return (int64_t)j * len + a;
  if (layout == 1) return a * n_ring + j;
  const int64_t h = len / 2;  // zigzag
  return a < h ? (int64_t)j * h + a : (int64_t)(2 * n_ring - 1 - j) * h + (a - h);
}

// Segment holding local row a (the last one starting at or before a, so
// empty segments are passed over).
RA_HD int32_t segment_of(const SegTable& t, int64_t a) {
  int32_t lo = 0, hi = t.n;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (t.off[mid] <= a) lo = mid; else hi = mid;
  }
  return lo;
}

// Class of a tile of a packed share: every segment the rows touch is judged
// on its own (keys outside a row's segment are never visible to it).
RA_HD int32_t tile_class_packed(BlockGeom g, const SegTable& t, int64_t a_lo, int64_t a_hi,
                                int64_t b_lo, int64_t b_hi) {
  bool any = false, all = true;
  for (int32_t s = segment_of(t, a_lo); s < t.n && t.off[s] <= a_hi; ++s) {
    const int64_t s0 = t.off[s], s1 = t.off[s + 1];  // rows and keys [s0, s1)
    const int64_t r0 = a_lo > s0 ? a_lo : s0, r1 = a_hi < s1 - 1 ? a_hi : s1 - 1;
    if (r0 > r1) continue;
    const int64_t k0 = b_lo > s0 ? b_lo : s0, k1 = b_hi < s1 - 1 ? b_hi : s1 - 1;
    if (k0 > k1) { all = false; continue; }
    if (k0 != b_lo || k1 != b_hi) all = false;
    const int32_t c = tile_class(g, r0 - s0, r1 - s0, k0 - s0, k1 - s0, s1 - s0);
    if (c != kSkip) any = true;
    if (c != kFull) all = false;
  }
  return all ? kFull : (any ? kPartial : kSkip);
}

}  // namespace ra
