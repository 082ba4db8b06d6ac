// ra_api.hip -- the C ABI of include/ra.h: host-side validation, the causal
// tile scheduler's host mirror, and the one-GPU ring loop.
//
// Ring loop (Ultralytics "Ring Attention", section "How ring attention
// works"; jisaku "Ring Attention", sections on the processing flow and on
// overlapping communication with computation): step s uses block
// j = (rank - s) mod N; while step s computes, the block for step s+1 is
// brought in. On one GPU "bringing in" is a stream-ordered device-to-device
// copy on a side stream into one of two staging buffers; events order each
// copy after the last kernel that read its buffer (write-after-read) and each
// step's kernels after the copy that filled their buffer (read-after-write).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "ra.h"
#include "ra_kernels.h"
#include "ra_sched.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Debug switches, read at every call:
//   RA_DEBUG_SYNC=1   each entry point waits for its streams after its
//                     launches (the ring after every step) and reports the
//                     first error with the launch or step it came from;
//   RA_DEBUG_POISON=1 the ring fills each staging buffer with NaN right
//                     before the copy that refills it, so a kernel that reads
//                     a buffer before its copy has landed computes NaN
//                     instead of a stale block.
// Both are for eager calls: a stream cannot be waited on under graph capture.
bool debug_on(const char* name) {
  const char* e = getenv(name);
  return e && e[0] == '1' && e[1] == 0;
}

ra_status debug_sync(hipStream_t a, hipStream_t b, const char* what, int step) {
  if (!debug_on("RA_DEBUG_SYNC")) return RA_OK;
  hipError_t e = hipStreamSynchronize(a);
  if (e == hipSuccess && b != nullptr && b != a) e = hipStreamSynchronize(b);
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) return RA_OK;
  if (step >= 0)
    return fail(RA_ERR_HIP, "%s, step %d: %s", what, step, hipGetErrorString(e));
  return hip_fail(e, what);
}

// 0x7FC0 is a bf16 quiet NaN and 0x7FC07FC0 a float32 one
constexpr uint32_t kPoison = 0x7FC07FC0u;

struct Shape {
  int64_t rows;        // batch * q_len * hq
  int64_t q_elems;     // batch * q_len * hq * d
  int64_t kv_elems;    // batch * kv_len * hkv * d (one block)
  size_t elem;         // bytes per q/k/v element
  float scale;
  int32_t packed;      // packed sequences
  ra::SegTable seg;    // local row segments ({0, q_len} without packing)
};

static_assert(RA_MAX_SEQS == ra::kMaxSegs, "segment table size");

// Packed sequences: check cu_seqlens and fill the local segment table.
ra_status validate_packed(const ra_problem* p, Shape* s) {
  s->packed = p->n_seqs > 0;
  s->seg.n = 1;
  s->seg.off[0] = 0;
  s->seg.off[1] = (int32_t)p->q_len;
  if (p->n_seqs == 0) return RA_OK;
  if (p->n_seqs < 0 || p->n_seqs > RA_MAX_SEQS)
    return fail(RA_ERR_INVALID_ARG, "n_seqs %d out of [0, %d]", p->n_seqs, RA_MAX_SEQS);
  if (p->cu_seqlens == nullptr) return fail(RA_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (p->batch != 1) return fail(RA_ERR_INVALID_ARG, "packed sequences need batch == 1");
  if (p->q_len != p->kv_len)
    return fail(RA_ERR_INVALID_ARG, "packed sequences need q_len == kv_len");
  if (p->cu_seqlens[0] != 0) return fail(RA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  const int64_t mult = (int64_t)p->n_ring * (p->layout == RA_LAYOUT_ZIGZAG ? 2 : 1);
  for (int i = 0; i < p->n_seqs; ++i) {
    const int64_t len = p->cu_seqlens[i + 1] - p->cu_seqlens[i];
    if (len < 0) return fail(RA_ERR_INVALID_ARG, "cu_seqlens decreases at %d", i + 1);
    if (len % mult != 0)
      return fail(RA_ERR_INVALID_ARG, "sequence %d: length %lld is not a multiple of %lld", i,
                  (long long)len, (long long)mult);
  }
  if (p->cu_seqlens[p->n_seqs] != p->q_len * p->n_ring)
    return fail(RA_ERR_INVALID_ARG, "cu_seqlens[n_seqs] = %lld, expected q_len * n_ring = %lld",
                (long long)p->cu_seqlens[p->n_seqs], (long long)(p->q_len * p->n_ring));
  s->seg.n = p->n_seqs;
  for (int i = 0; i <= p->n_seqs; ++i) s->seg.off[i] = (int32_t)(p->cu_seqlens[i] / p->n_ring);
  return RA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ra_status validate_problem(const ra_problem* p, Shape* s) {
  if (p == nullptr) return fail(RA_ERR_INVALID_ARG, "problem is NULL");
  if (p->dtype != RA_F32 && p->dtype != RA_BF16)
    return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_F32 or RA_BF16", p->dtype);
  if (p->batch < 0) return fail(RA_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->hq < 1 || p->hkv < 1)
    return fail(RA_ERR_INVALID_ARG, "hq (%d) and hkv (%d) must be >= 1", p->hq, p->hkv);
  if (p->hq % p->hkv != 0)
    return fail(RA_ERR_INVALID_ARG, "hq (%d) is not a multiple of hkv (%d)", p->hq, p->hkv);
  if (p->head_dim <= 0) return fail(RA_ERR_INVALID_ARG, "head_dim %d <= 0", p->head_dim);
  if (p->head_dim != 16 && p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (16, 32, 64, 128)", p->head_dim);
  const int64_t kMaxLen = int64_t(1) << 30;
  if (p->q_len < 0 || p->q_len > kMaxLen)
    return fail(RA_ERR_INVALID_ARG, "q_len %lld out of [0, 2^30]", (long long)p->q_len);
  if (p->kv_len < 0 || p->kv_len > kMaxLen)
    return fail(RA_ERR_INVALID_ARG, "kv_len %lld out of [0, 2^30]", (long long)p->kv_len);
  if (p->n_ring < 1) return fail(RA_ERR_INVALID_ARG, "n_ring %d < 1", p->n_ring);
  if (p->rank < 0 || p->rank >= p->n_ring)
    return fail(RA_ERR_INVALID_ARG, "rank %d out of [0, n_ring=%d)", p->rank, p->n_ring);
  if (p->causal != 0 && p->causal != 1)
    return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", p->causal);
  if (p->layout != RA_LAYOUT_CONTIGUOUS && p->layout != RA_LAYOUT_STRIPED &&
      p->layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "layout %d unknown", p->layout);
  if (p->layout == RA_LAYOUT_ZIGZAG && p->n_seqs == 0 && (p->q_len % 2 || p->kv_len % 2))
    return fail(RA_ERR_INVALID_ARG, "zigzag needs even q_len and kv_len");
  if (p->causal && p->q_len != p->kv_len)
    return fail(RA_ERR_INVALID_ARG, "causal requires q_len == kv_len (%lld vs %lld)",
                (long long)p->q_len, (long long)p->kv_len);
  if (isnan(p->scale) || isinf(p->scale))
    return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  if (isnan(p->rope_theta) || isinf(p->rope_theta) || p->rope_theta < 0.f)
    return fail(RA_ERR_INVALID_ARG, "rope_theta must be finite and >= 0");
  // the kernels address one batch row of a KV block with 32-bit offsets
  if ((int64_t)p->kv_len * p->hkv * p->head_dim > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "kv_len*hkv*head_dim exceeds 2^31-1 elements");
  const int64_t group = p->hq / p->hkv;
  if (group * p->q_len > INT32_MAX)
    return fail(RA_ERR_INVALID_ARG, "(hq/hkv)*q_len exceeds 2^31-1");
  ra_status st = validate_packed(p, s);
  if (st != RA_OK) return st;
  s->rows = (int64_t)p->batch * p->q_len * p->hq;
  s->q_elems = s->rows * p->head_dim;
  s->kv_elems = (int64_t)p->batch * p->kv_len * p->hkv * p->head_dim;
  s->elem = p->dtype == RA_BF16 ? 2 : 4;
  s->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  return RA_OK;
}

// Workgroups of one tiled launch for one (batch row, KV head), counted as
// the launchers count them: row (or key) tiles of every segment.
int64_t tiles_per_head(const ra_problem* p, const Shape& s, ra::TileShape t) {
  int64_t total = 0;
  const int64_t group = p->hq / p->hkv;
  for (int i = 0; i < s.seg.n; ++i) {
    const int64_t len = (int64_t)s.seg.off[i + 1] - s.seg.off[i];
    const int64_t n = t.by_keys ? (s.packed ? len : (i == 0 ? p->kv_len : 0)) : len * group;
    total += (n + t.per - 1) / t.per;
  }
  return total;
}

// One launch of `t` over the problem must fit a dispatch: at most 2^31 - 1
// workgroups and 2^32 - 1 work items.
ra_status check_grid(const ra_problem* p, const Shape& s, ra::TileShape t, const char* kernel) {
  const int64_t heads = (int64_t)p->batch * p->hkv;
  int64_t blocks = 0, items = 0;
  if (__builtin_mul_overflow(heads, tiles_per_head(p, s, t), &blocks) || blocks > INT32_MAX ||
      __builtin_mul_overflow(blocks, (int64_t)t.threads, &items) || items > (int64_t)0xFFFFFFFF)
    return fail(RA_ERR_INVALID_ARG,
                "problem too large for one launch of the %s kernel (%d %s and %d work items per "
                "workgroup)", kernel, t.per, t.by_keys ? "keys" : "rows", t.threads);
  return RA_OK;
}

// Compute units of the GPU the launch shapes are chosen for (MI355X).
constexpr int64_t kGpuCus = 256;

// Waves per workgroup of the bf16 kernel: 8 (256 rows, one workgroup per CU,
// two waves per SIMD) unless the 8-wave grid of this share has fewer
// workgroups than the GPU has CUs; then 4 (128 rows, two workgroups per CU),
// which spreads a small share over twice as many CUs (+10 % on 1024-token
// blocks of 32 heads). RA_WAVES=4 or RA_WAVES=8 forces one (read at every
// call, so that validation and launch of one call agree).
int fwd_waves(const ra_problem* p, const Shape& s) {
  const char* e = getenv("RA_WAVES");
  if (e && (e[0] == '4' || e[0] == '8') && e[1] == 0) return e[0] - '0';
  if (p->dtype != RA_BF16) return 8;
  const int64_t wg8 = (int64_t)p->batch * p->hkv * tiles_per_head(p, s, ra::fwd_tile_shape(1, p->head_dim, 8));
  return wg8 < kGpuCus ? 4 : 8;
}

ra_status check_fwd_grid(const ra_problem* p, const Shape& s) {
  return check_grid(p, s, ra::fwd_tile_shape(p->dtype == RA_BF16, p->head_dim, fwd_waves(p, s)),
                    "attention");
}

ra_status check_bwd_grid(const ra_problem* p, const Shape& s) {
  ra::TileShape t[2];
  ra::bwd_tile_shapes(p->dtype == RA_BF16, p->head_dim, t);
  ra_status st = check_grid(p, s, t[0], "dq");
  return st != RA_OK ? st : check_grid(p, s, t[1], "dk/dv");
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0 || a == nullptr || b == nullptr) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

ra_status check_ptr(const void* p, size_t bytes, const char* name) {
  if (bytes == 0) return RA_OK;
  if (p == nullptr) return fail(RA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(RA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return RA_OK;
}

// Staging copies of fewer bytes per step than this (K and V of one block)
// run in order on the compute stream even when a copy stream is given. A
// second stream costs each step two cross-stream event waits that the GPU
// resolves on the critical path (about 10 us per step measured on MI355X);
// below this size the copies they would hide take less than that.
// RA_SIDE_STREAM_MIN_BYTES overrides it (0: always use the copy stream); it
// is read at every ring call.
size_t side_stream_min_bytes() {
  const char* e = getenv("RA_SIDE_STREAM_MIN_BYTES");
  if (e && *e) return (size_t)strtoull(e, nullptr, 10);
  return size_t(32) << 20;
}

ra::AttnParams make_params(const ra_problem* p, const Shape& s, int32_t j, const void* q,
                           const void* k, const void* v, float* m, float* l, float* acc) {
  ra::AttnParams a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.m = m;
  a.l = l;
  a.acc = acc;
  a.q_bstride = p->q_len * p->hq * p->head_dim;
  a.kv_bstride = p->kv_len * p->hkv * p->head_dim;
  a.batch = p->batch;
  a.q_len = (int32_t)p->q_len;
  a.kv_len = (int32_t)p->kv_len;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.head_dim = p->head_dim;
  a.group = p->hq / p->hkv;
  a.packed = s.packed;
  a.seg = s.seg;
  ra::BlockGeom g = ra::block_geom(p->causal, p->layout, p->rank, j);
  a.geom_kind = g.kind;
  a.geom_delta = g.delta;
  a.scale_log2 = s.scale * 1.4426950408889634f;
  return a;
}

// Enqueue one block's partial into (m, l, acc), or, with accumulate, merge
// it into the running state (m, l, acc) in place. Skipped-block semantics: a
// block with no visible pair (or no keys) yields the empty partial, which
// leaves a running state unchanged.
// finalize: the launch also divides, acc <- acc / l and lse <- m + ln l (the
// ring's last launch; lse may be null).
ra_status enqueue_partial(const ra_problem* p, const Shape& s, int32_t j, const void* q,
                          const void* k, const void* v, float* m, float* l, float* acc,
                          hipStream_t st, bool accumulate = false, bool finalize = false,
                          float* lse = nullptr) {
  ra::BlockGeom g = ra::block_geom(p->causal, p->layout, p->rank, j);
  hipError_t e;
  if (g.kind == ra::kNoneVisible || p->kv_len == 0) {
    if (accumulate) return RA_OK;
    e = ra::launch_fill_empty(s.rows, p->head_dim, m, l, acc, st);
    if (e != hipSuccess) return hip_fail(e, "fill_empty launch");
    return RA_OK;
  }
  ra::AttnParams a = make_params(p, s, j, q, k, v, m, l, acc);
  a.accumulate = accumulate ? 1 : 0;
  a.finalize = finalize ? 1 : 0;
  a.lse = lse;
  e = ra::launch_attention(a, p->dtype == RA_BF16, fwd_waves(p, s), st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return RA_OK;
}

ra::BwdParams make_bwd_params(const ra_problem* p, const Shape& s, int32_t j, const void* q,
                              const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, float* dq, float* dk, float* dv) {
  ra::BwdParams a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.q_bstride = p->q_len * p->hq * p->head_dim;
  a.kv_bstride = p->kv_len * p->hkv * p->head_dim;
  a.batch = p->batch;
  a.q_len = (int32_t)p->q_len;
  a.kv_len = (int32_t)p->kv_len;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.head_dim = p->head_dim;
  a.group = p->hq / p->hkv;
  a.packed = s.packed;
  a.seg = s.seg;
  ra::BlockGeom g = ra::block_geom(p->causal, p->layout, p->rank, j);
  a.geom_kind = g.kind;
  a.geom_delta = g.delta;
  a.scale = s.scale;
  a.scale_log2 = s.scale * 1.4426950408889634f;
  return a;
}

// Rotary embedding of block `block` (queries of the share when block ==
// rank and queries is set): tokens len, heads heads.
ra::RopeParams make_rope(const ra_problem* p, const Shape& s, bool queries, int32_t block,
                         int32_t heads, bool in_bf16, const void* x, bool out_bf16, void* y,
                         bool inverse, bool accumulate) {
  ra::RopeParams r{};
  r.x = x;
  r.y = y;
  r.in_bf16 = in_bf16;
  r.out_bf16 = out_bf16;
  r.accumulate = accumulate;
  r.inverse = inverse;
  r.batch = p->batch;
  r.len = (int32_t)(queries ? p->q_len : p->kv_len);
  r.heads = heads;
  r.head_dim = p->head_dim;
  r.layout = p->layout;
  r.n_ring = p->n_ring;
  r.block = block;
  r.packed = s.packed;
  r.seg = s.seg;
  for (int i = 0; i < p->head_dim / 2 && i < 64; ++i)
    r.inv_freq[i] = pow((double)p->rope_theta, -2.0 * i / p->head_dim);
  return r;
}

// Enqueue one block's backward addends (nothing for a block with no visible
// pair or no keys: its addends are zero).
ra_status enqueue_bwd(const ra_problem* p, const Shape& s, int32_t j, const void* q, const void* k,
                      const void* v, const void* dout, const float* lse, const float* delta,
                      float* dq, float* dk, float* dv, hipStream_t st) {
  ra::BlockGeom g = ra::block_geom(p->causal, p->layout, p->rank, j);
  if (g.kind == ra::kNoneVisible || p->kv_len == 0) return RA_OK;
  ra::BwdParams a = make_bwd_params(p, s, j, q, k, v, dout, lse, delta, dq, dk, dv);
  hipError_t e = ra::launch_bwd(a, p->dtype == RA_BF16, st);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return RA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct BwdWsLayout {
  size_t stage_k[2], stage_v[2], delta, qrot, dktmp, total;
};

BwdWsLayout bwd_ws_layout(const ra_problem* p, const Shape& s) {
  BwdWsLayout w{};
  const size_t blk = align256((size_t)s.kv_elems * s.elem);
  const bool rope = p->rope_theta > 0.f;
  const bool staged = p->n_ring > 1 || rope;
  size_t off = 0;
  for (int i = 0; i < 2; ++i) {
    w.stage_k[i] = off;
    off += staged ? blk : 0;
    w.stage_v[i] = off;
    off += staged ? blk : 0;
  }
  w.delta = off;
  off += align256((size_t)s.rows * 4);
  w.qrot = off;
  off += rope ? align256((size_t)s.q_elems * s.elem) : 0;
  w.dktmp = off;
  off += rope ? align256((size_t)s.kv_elems * 4) : 0;
  w.total = off;
  return w;
}

struct WsLayout {
  size_t stage_k[2], stage_v[2], rm, rl, qrot, total;
};

bool rope_on(const ra_problem* p) { return p->rope_theta > 0.f; }

WsLayout ws_layout(const ra_problem* p, const Shape& s) {
  WsLayout w{};
  const size_t blk = align256((size_t)s.kv_elems * s.elem);
  const size_t rowb = align256((size_t)s.rows * 4);
  size_t off = 0;
  const bool staged = p->n_ring > 1 || rope_on(p);
  for (int i = 0; i < 2; ++i) {
    w.stage_k[i] = off;
    off += staged ? blk : 0;
    w.stage_v[i] = off;
    off += staged ? blk : 0;
  }
  w.rm = off; off += rowb;
  w.rl = off; off += rowb;
  w.qrot = off; off += rope_on(p) ? align256((size_t)s.q_elems * s.elem) : 0;
  w.total = off;
  return w;
}

// Per-device event pool for the ring loop (timing disabled).
struct DeviceEvents {
  std::mutex mu;
  bool ready = false;
  hipEvent_t entry{}, copy_done[2]{}, compute_done[2]{};
};

std::mutex g_pool_mu;
std::vector<DeviceEvents*> g_pool;

ra_status get_events(DeviceEvents** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  DeviceEvents* de;
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if ((int)g_pool.size() <= dev) g_pool.resize(dev + 1, nullptr);
    if (g_pool[dev] == nullptr) g_pool[dev] = new DeviceEvents();
    de = g_pool[dev];
  }
  *out = de;
  return RA_OK;
}

ra_status init_events(DeviceEvents* de) {
  if (de->ready) return RA_OK;
  hipEvent_t* all[5] = {&de->entry, &de->copy_done[0], &de->copy_done[1], &de->compute_done[0],
                        &de->compute_done[1]};
  for (hipEvent_t* ev : all) {
    hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  de->ready = true;
  return RA_OK;
}

// The ring's K/V blocks on their way into the two staging buffers. Step s
// uses block (rank - s) mod N; it reads the block in place unless it is
// staged (every step s >= 1, and step 0 too with rotary embedding, which
// rotates K while copying it). Events order each copy after the last reader
// of its buffer and each step's kernels after the copy that filled theirs.
struct Stager {
  const ra_problem* p;
  const Shape* s;
  const char* kbase;
  const char* vbase;
  size_t blk;
  char* stage_k[2];
  char* stage_v[2];
  DeviceEvents* de;
  hipStream_t cs, xs;
  bool sep, rope;
  bool poison = debug_on("RA_DEBUG_POISON");

  int block_of(int step) const { return ((p->rank - step) % p->n_ring + p->n_ring) % p->n_ring; }
  bool staged(int step) const { return rope || step >= 1; }

  ra_status begin() {
    hipError_t e;
    if (!sep) return RA_OK;
    if ((e = hipEventRecord(de->entry, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(xs, de->entry, 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    return RA_OK;
  }
  ra_status stage(int step) {
    const int j = block_of(step), b = step % 2;
    hipStream_t on = sep ? xs : cs;
    hipError_t e;
    if (poison) {
      if ((e = ra::launch_fill_u32(stage_k[b], (int64_t)blk, kPoison, on)) != hipSuccess ||
          (e = ra::launch_fill_u32(stage_v[b], (int64_t)blk, kPoison, on)) != hipSuccess)
        return hip_fail(e, "poison fill");
    }
    if (rope) {
      ra::RopeParams r = make_rope(p, *s, false, j, p->hkv, p->dtype == RA_BF16,
                                   kbase + (size_t)j * blk, p->dtype == RA_BF16, stage_k[b],
                                   false, false);
      e = ra::launch_rope(r, on);
      if (e == hipSuccess)
        e = hipMemcpyAsync(stage_v[b], vbase + (size_t)j * blk, blk, hipMemcpyDeviceToDevice, on);
    } else {
      // K and V of the block in one copy kernel (one launch per step)
      e = ra::launch_copy2(stage_k[b], kbase + (size_t)j * blk, stage_v[b],
                           vbase + (size_t)j * blk, (int64_t)blk, on);
    }
    if (e != hipSuccess) return hip_fail(e, "staging copy");
    if (sep && (e = hipEventRecord(de->copy_done[b], xs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord");
    return RA_OK;
  }
  // before step `step` computes: bring in the block of step+1 (its buffer
  // was last read by step-1) and wait for this step's own block
  ra_status advance(int step, const void** k, const void** v) {
    hipError_t e;
    if (step >= 1 && step + 1 < p->n_ring) {
      if (sep && staged(step - 1) &&
          (e = hipStreamWaitEvent(xs, de->compute_done[(step - 1) % 2], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      ra_status st = stage(step + 1);
      if (st != RA_OK) return st;
    }
    const int j = block_of(step), b = step % 2;
    if (!staged(step)) {
      *k = kbase + (size_t)j * blk;
      *v = vbase + (size_t)j * blk;
      return RA_OK;
    }
    if (sep && (e = hipStreamWaitEvent(cs, de->copy_done[b], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    *k = stage_k[b];
    *v = stage_v[b];
    return RA_OK;
  }
  // after step `step`'s kernels are enqueued; step 1's block is brought in
  // once step 0's kernels are queued, so that its copy runs under them
  ra_status done(int step) {
    hipError_t e;
    if (sep && staged(step) && (e = hipEventRecord(de->compute_done[step % 2], cs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord");
    if (step == 0 && p->n_ring > 1) return stage(1);
    return RA_OK;
  }
  // the first copy: step 0's block when it is staged (rotary embedding)
  ra_status start() {
    ra_status st = begin();
    if (st == RA_OK && rope) st = stage(0);
    return st;
  }
};

// Workspace of ra_ring_fwd_noalloc: one file-scope device array per GPU,
// allocated with the code object when a device loads the library and held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address is resolved once per device with
// hipGetSymbolAddress and only that address is handed to kernels and copies.
constexpr size_t kScratchBytes = size_t(64) << 20;
static_assert(RA_NOALLOC_WORKSPACE_BYTES == kScratchBytes, "scratch size");
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch;  // device address of `scratch`, per device

// Set-up of the allocation-free entry point on the current device (its first
// call there): the array's device address and the ring's event pool, so
// that later calls create nothing.
ra_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(RA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    DeviceEvents* de = nullptr;
    ra_status st = get_events(&de);
    if (st != RA_OK) return st;
    {
      std::lock_guard<std::mutex> lk2(de->mu);
      if ((st = init_events(de)) != RA_OK) return st;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

const char* ra_last_error(void) { return g_err.c_str(); }

static ra_status block_partial_entry(const ra_problem* prob, int32_t kv_block_j, const void* q,
                                     const void* k, const void* v, float* m, float* l,
                                     float* acc, void* hip_stream, bool accumulate) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if (kv_block_j < 0 || kv_block_j >= prob->n_ring)
      return fail(RA_ERR_INVALID_ARG, "kv_block_j %d out of [0, n_ring=%d)", kv_block_j,
                  prob->n_ring);
    if ((st = check_fwd_grid(prob, s)) != RA_OK) return st;
    const size_t qb = s.q_elems * s.elem, kb = s.kv_elems * s.elem;
    const size_t rb = s.rows * 4, ab = s.q_elems * 4;
    if ((st = check_ptr(q, qb, "q")) || (st = check_ptr(k, kb, "k")) ||
        (st = check_ptr(v, kb, "v")) || (st = check_ptr(m, rb, "m")) ||
        (st = check_ptr(l, rb, "l")) || (st = check_ptr(acc, ab, "acc")))
      return st;
    const void* ins[3] = {q, k, v};
    const size_t insz[3] = {qb, kb, kb};
    const void* outs[3] = {m, l, acc};
    const size_t outsz[3] = {rb, rb, ab};
    for (int i = 0; i < 3; ++i)
      for (int o = 0; o < 3; ++o)
        if (overlap(ins[i], insz[i], outs[o], outsz[o]))
          return fail(RA_ERR_INVALID_ARG, "outputs must not overlap q, k or v");
    if (overlap(m, rb, l, rb) || overlap(m, rb, acc, ab) || overlap(l, rb, acc, ab))
      return fail(RA_ERR_INVALID_ARG, "m, l and acc must not overlap");
    if (s.rows == 0) return RA_OK;
    st = enqueue_partial(prob, s, kv_block_j, q, k, v, m, l, acc,
                         static_cast<hipStream_t>(hip_stream), accumulate);
    return st != RA_OK ? st
                       : debug_sync(static_cast<hipStream_t>(hip_stream), nullptr,
                                    accumulate ? "accumulate" : "partial", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_block_attn_partial(const ra_problem* prob, int32_t kv_block_j, const void* q,
                                const void* k, const void* v, float* m, float* l, float* acc,
                                void* hip_stream) {
  return block_partial_entry(prob, kv_block_j, q, k, v, m, l, acc, hip_stream, false);
}

ra_status ra_block_attn_accumulate(const ra_problem* prob, int32_t kv_block_j, const void* q,
                                   const void* k, const void* v, float* m, float* l, float* acc,
                                   void* hip_stream) {
  return block_partial_entry(prob, kv_block_j, q, k, v, m, l, acc, hip_stream, true);
}

static ra_status check_alias_exact(const void* out, const void* in1, const void* in2, size_t n,
                                   const char* name) {
  if ((out == in1) || (out == in2)) return RA_OK;
  if (overlap(out, n, in1, n) || overlap(out, n, in2, n))
    return fail(RA_ERR_INVALID_ARG, "%s partially overlaps an input", name);
  return RA_OK;
}

ra_status ra_merge_partials(int64_t rows, int32_t head_dim, const float* m1, const float* l1,
                            const float* acc1, const float* m2, const float* l2,
                            const float* acc2, float* m_out, float* l_out, float* acc_out,
                            void* hip_stream) {
  try {
    if (rows < 0) return fail(RA_ERR_INVALID_ARG, "rows %lld < 0", (long long)rows);
    if (head_dim <= 0) return fail(RA_ERR_INVALID_ARG, "head_dim %d <= 0", head_dim);
    if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
      return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (16, 32, 64, 128)", head_dim);
    if (rows > (int64_t(1) << 40)) return fail(RA_ERR_INVALID_ARG, "rows too large");
    const size_t rb = rows * 4, ab = rows * head_dim * 4;
    ra_status st;
    if ((st = check_ptr(m1, rb, "m1")) || (st = check_ptr(l1, rb, "l1")) ||
        (st = check_ptr(acc1, ab, "acc1")) || (st = check_ptr(m2, rb, "m2")) ||
        (st = check_ptr(l2, rb, "l2")) || (st = check_ptr(acc2, ab, "acc2")) ||
        (st = check_ptr(m_out, rb, "m_out")) || (st = check_ptr(l_out, rb, "l_out")) ||
        (st = check_ptr(acc_out, ab, "acc_out")))
      return st;
    if ((st = check_alias_exact(m_out, m1, m2, rb, "m_out")) ||
        (st = check_alias_exact(l_out, l1, l2, rb, "l_out")) ||
        (st = check_alias_exact(acc_out, acc1, acc2, ab, "acc_out")))
      return st;
    if (overlap(m_out, rb, l_out, rb) || overlap(m_out, rb, acc_out, ab) ||
        overlap(l_out, rb, acc_out, ab))
      return fail(RA_ERR_INVALID_ARG, "m_out, l_out and acc_out must not overlap");
    if (rows == 0) return RA_OK;
    hipError_t e = ra::launch_merge(rows, head_dim, m1, l1, acc1, m2, l2, acc2, m_out, l_out,
                                    acc_out, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "merge", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_finalize(int64_t rows, int32_t head_dim, const float* m, const float* l, float* acc,
                      float* lse, void* hip_stream) {
  try {
    if (rows < 0) return fail(RA_ERR_INVALID_ARG, "rows %lld < 0", (long long)rows);
    if (head_dim <= 0) return fail(RA_ERR_INVALID_ARG, "head_dim %d <= 0", head_dim);
    if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
      return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (16, 32, 64, 128)", head_dim);
    if (rows > (int64_t(1) << 40)) return fail(RA_ERR_INVALID_ARG, "rows too large");
    const size_t rb = rows * 4, ab = rows * head_dim * 4;
    ra_status st;
    if ((st = check_ptr(m, rb, "m")) || (st = check_ptr(l, rb, "l")) ||
        (st = check_ptr(acc, ab, "acc")))
      return st;
    if (lse != nullptr && (st = check_ptr(lse, rb, "lse"))) return st;
    if (lse != nullptr && (overlap(lse, rb, acc, ab) || overlap(lse, rb, m, rb) ||
                           overlap(lse, rb, l, rb)))
      return fail(RA_ERR_INVALID_ARG, "lse must not overlap m, l or acc");
    if (rows == 0) return RA_OK;
    hipError_t e =
        ra::launch_finalize(rows, head_dim, m, l, acc, lse, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "finalize launch");
    return debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "finalize", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

size_t ra_ring_workspace_bytes(const ra_problem* prob) {
  try {
    Shape s;
    if (validate_problem(prob, &s) != RA_OK) return 0;
    return ws_layout(prob, s).total;
  } catch (...) {
    return 0;
  }
}

// The ring's tensors apart from the workspace: pointers, alignment, block
// size (host-side only, before any HIP call).
static ra_status check_ring_fwd_tensors(const ra_problem* prob, const Shape& s, const void* q,
                                        const void* k, const void* v, const float* out,
                                        const float* lse) {
  ra_status st;
  const size_t blk = s.kv_elems * s.elem, kvb = blk * prob->n_ring;
  const size_t rb = s.rows * 4;
  if ((st = check_ptr(q, s.q_elems * s.elem, "q")) || (st = check_ptr(k, kvb, "k")) ||
      (st = check_ptr(v, kvb, "v")) || (st = check_ptr(out, s.q_elems * 4, "out")))
    return st;
  if (lse != nullptr && (st = check_ptr(lse, rb, "lse"))) return st;
  if (blk % 16 != 0 && prob->n_ring > 1)
    return fail(RA_ERR_INVALID_ARG, "one KV block (%zu bytes) must be a multiple of 16 bytes",
                blk);
  return RA_OK;
}

static ra_status ring_fwd_impl(const ra_problem* prob, const Shape& s, const void* q,
                               const void* k, const void* v, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* compute_stream,
                               void* copy_stream) {
  try {
    ra_status st;
    const int n = prob->n_ring;
    const size_t qb = s.q_elems * s.elem;
    const size_t blk = s.kv_elems * s.elem;
    const size_t kvb = blk * n;
    const size_t ob = s.q_elems * 4, rb = s.rows * 4;
    if ((st = check_ring_fwd_tensors(prob, s, q, k, v, out, lse)) != RA_OK) return st;
    const WsLayout w = ws_layout(prob, s);
    if (s.rows > 0) {
      if (workspace == nullptr || workspace_bytes < w.total)
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
      if (!aligned16(workspace))
        return fail(RA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    const void* ins[3] = {q, k, v};
    const size_t insz[3] = {qb, kvb, kvb};
    for (int i = 0; i < 3; ++i) {
      if (overlap(out, ob, ins[i], insz[i]))
        return fail(RA_ERR_INVALID_ARG, "out must not overlap q, k or v");
      if (lse && overlap(lse, rb, ins[i], insz[i]))
        return fail(RA_ERR_INVALID_ARG, "lse must not overlap q, k or v");
      if (s.rows > 0 && overlap(workspace, w.total, ins[i], insz[i]))
        return fail(RA_ERR_INVALID_ARG, "workspace must not overlap q, k or v");
    }
    if (lse && overlap(lse, rb, out, ob)) return fail(RA_ERR_INVALID_ARG, "lse overlaps out");
    if (s.rows > 0 && (overlap(workspace, w.total, out, ob) ||
                       (lse && overlap(workspace, w.total, lse, rb))))
      return fail(RA_ERR_INVALID_ARG, "workspace must not overlap out or lse");
    if (s.rows == 0) return RA_OK;

    // ---- enqueue -------------------------------------------------------
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    hipStream_t xs = static_cast<hipStream_t>(copy_stream);
    const bool sep = xs != nullptr && xs != cs && 2 * blk >= side_stream_min_bytes();
    DeviceEvents* de = nullptr;
    if ((st = get_events(&de)) != RA_OK) return st;
    std::lock_guard<std::mutex> lk(de->mu);
    if ((st = init_events(de)) != RA_OK) return st;

    char* ws = static_cast<char*>(workspace);
    float* rm = reinterpret_cast<float*>(ws + w.rm);
    float* rl = reinterpret_cast<float*>(ws + w.rl);
    Stager sg{prob, &s, static_cast<const char*>(k), static_cast<const char*>(v), blk,
              {ws + w.stage_k[0], ws + w.stage_k[1]}, {ws + w.stage_v[0], ws + w.stage_v[1]},
              de, cs, xs, sep, rope_on(prob)};
    hipError_t e;
    const void* qx = q;
    if (sg.rope) {  // the local queries, rotated once by their own positions
      void* qr = ws + w.qrot;
      ra::RopeParams r = make_rope(prob, s, true, prob->rank, prob->hq, prob->dtype == RA_BF16, q,
                                   prob->dtype == RA_BF16, qr, false, false);
      if ((e = ra::launch_rope(r, cs)) != hipSuccess) return hip_fail(e, "rope launch");
      qx = qr;
    }
    // the last step that launches the attention kernel also divides (no
    // separate finalize); a ring whose only launch is the empty fill of
    // step 0 keeps the finalize kernel
    int last = -1;
    for (int step = 0; step < n; ++step) {
      const ra::BlockGeom g = ra::block_geom(prob->causal, prob->layout, prob->rank,
                                             sg.block_of(step));
      if (g.kind != ra::kNoneVisible && prob->kv_len > 0) last = step;
    }
    if ((st = sg.start()) != RA_OK) return st;
    for (int step = 0; step < n; ++step) {
      const void *kb = nullptr, *vb = nullptr;
      if ((st = sg.advance(step, &kb, &vb)) != RA_OK) return st;
      const int j = sg.block_of(step);
      // the local block's partial starts the running state (m, l, out); each
      // later block's partial is merged into it by the attention kernel itself
      if ((st = enqueue_partial(prob, s, j, qx, kb, vb, rm, rl, out, cs, step > 0, step == last,
                                lse)) != RA_OK)
        return st;
      if ((st = sg.done(step)) != RA_OK) return st;
      if ((st = debug_sync(cs, sep ? xs : nullptr, "ring", step)) != RA_OK) return st;
    }
    if (last < 0) {
      e = ra::launch_finalize(s.rows, prob->head_dim, rm, rl, out, lse, cs);
      if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    return debug_sync(cs, nullptr, "finalize", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_ring_fwd(const ra_problem* prob, const void* q, const void* k, const void* v,
                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if ((st = check_fwd_grid(prob, s)) != RA_OK) return st;
    return ring_fwd_impl(prob, s, q, k, v, out, lse, workspace, workspace_bytes, compute_stream,
                         copy_stream);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_ring_fwd_noalloc(const ra_problem* prob, const void* q, const void* k,
                              const void* v, float* out, float* lse, void* compute_stream,
                              void* copy_stream) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if ((st = check_fwd_grid(prob, s)) != RA_OK) return st;
    if ((st = check_ring_fwd_tensors(prob, s, q, k, v, out, lse)) != RA_OK) return st;
    const size_t need = ws_layout(prob, s).total;
    if (need > kScratchBytes)
      return fail(RA_ERR_WORKSPACE,
                  "the allocation-free ring needs %zu bytes of workspace; its static workspace "
                  "holds %zu (use ra_ring_fwd with a caller workspace)",
                  need, kScratchBytes);
    if (s.rows == 0)
      return ring_fwd_impl(prob, s, q, k, v, out, lse, nullptr, 0, compute_stream, copy_stream);
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != RA_OK) return st;
    return ring_fwd_impl(prob, s, q, k, v, out, lse, ws, kScratchBytes, compute_stream,
                         copy_stream);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const float* out,
                            const void* dout, float* delta, void* hip_stream) {
  try {
    if (rows < 0) return fail(RA_ERR_INVALID_ARG, "rows %lld < 0", (long long)rows);
    if (dtype != RA_F32 && dtype != RA_BF16)
      return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_F32 or RA_BF16", dtype);
    if (head_dim <= 0) return fail(RA_ERR_INVALID_ARG, "head_dim %d <= 0", head_dim);
    if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
      return fail(RA_ERR_UNSUPPORTED, "head_dim %d unsupported (16, 32, 64, 128)", head_dim);
    if (rows > (int64_t(1) << 40)) return fail(RA_ERR_INVALID_ARG, "rows too large");
    const size_t ob = rows * head_dim * 4, db = rows * head_dim * (dtype == RA_BF16 ? 2 : 4);
    const size_t rb = rows * 4;
    ra_status st;
    if ((st = check_ptr(out, ob, "out")) || (st = check_ptr(dout, db, "dout")) ||
        (st = check_ptr(delta, rb, "delta")))
      return st;
    if (overlap(delta, rb, out, ob) || overlap(delta, rb, dout, db))
      return fail(RA_ERR_INVALID_ARG, "delta must not overlap out or dout");
    if (rows == 0) return RA_OK;
    hipError_t e = ra::launch_bwd_delta(rows, head_dim, dtype == RA_BF16, out, dout, delta,
                                        static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "delta launch");
    return debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "delta", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_block_attn_bwd(const ra_problem* prob, int32_t kv_block_j, const void* q,
                            const void* k, const void* v, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv,
                            void* hip_stream) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if (kv_block_j < 0 || kv_block_j >= prob->n_ring)
      return fail(RA_ERR_INVALID_ARG, "kv_block_j %d out of [0, n_ring=%d)", kv_block_j,
                  prob->n_ring);
    if ((st = check_bwd_grid(prob, s)) != RA_OK) return st;
    const size_t qb = s.q_elems * s.elem, kb = s.kv_elems * s.elem;
    const size_t rb = s.rows * 4, qfb = s.q_elems * 4, kfb = s.kv_elems * 4;
    if ((st = check_ptr(q, qb, "q")) || (st = check_ptr(k, kb, "k")) ||
        (st = check_ptr(v, kb, "v")) || (st = check_ptr(dout, qb, "dout")) ||
        (st = check_ptr(lse, rb, "lse")) || (st = check_ptr(delta, rb, "delta")) ||
        (st = check_ptr(dq, qfb, "dq")) || (st = check_ptr(dk, kfb, "dk")) ||
        (st = check_ptr(dv, kfb, "dv")))
      return st;
    const void* ins[6] = {q, k, v, dout, lse, delta};
    const size_t insz[6] = {qb, kb, kb, qb, rb, rb};
    const void* outs[3] = {dq, dk, dv};
    const size_t outsz[3] = {qfb, kfb, kfb};
    for (int o = 0; o < 3; ++o) {
      for (int i = 0; i < 6; ++i)
        if (overlap(outs[o], outsz[o], ins[i], insz[i]))
          return fail(RA_ERR_INVALID_ARG, "dq, dk and dv must not overlap any input");
      for (int o2 = o + 1; o2 < 3; ++o2)
        if (overlap(outs[o], outsz[o], outs[o2], outsz[o2]))
          return fail(RA_ERR_INVALID_ARG, "dq, dk and dv must not overlap each other");
    }
    if (s.rows == 0) return RA_OK;
    st = enqueue_bwd(prob, s, kv_block_j, q, k, v, dout, lse, delta, dq, dk, dv,
                     static_cast<hipStream_t>(hip_stream));
    return st != RA_OK ? st
                       : debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "block backward", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

size_t ra_ring_bwd_workspace_bytes(const ra_problem* prob) {
  try {
    Shape s;
    if (validate_problem(prob, &s) != RA_OK) return 0;
    return bwd_ws_layout(prob, s).total;
  } catch (...) {
    return 0;
  }
}

ra_status ra_ring_bwd(const ra_problem* prob, const void* q, const void* k, const void* v,
                      const float* out, const void* dout, const float* lse, float* dq,
                      float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if ((st = check_bwd_grid(prob, s)) != RA_OK) return st;
    const int n = prob->n_ring;
    const size_t qb = s.q_elems * s.elem, blk = s.kv_elems * s.elem, kvb = blk * n;
    const size_t qfb = s.q_elems * 4, rb = s.rows * 4, kfb = s.kv_elems * 4 * n;
    if ((st = check_ptr(q, qb, "q")) || (st = check_ptr(k, kvb, "k")) ||
        (st = check_ptr(v, kvb, "v")) || (st = check_ptr(out, qfb, "out")) ||
        (st = check_ptr(dout, qb, "dout")) || (st = check_ptr(lse, rb, "lse")) ||
        (st = check_ptr(dq, qfb, "dq")) || (st = check_ptr(dk, kfb, "dk")) ||
        (st = check_ptr(dv, kfb, "dv")))
      return st;
    if (blk % 16 != 0 && n > 1)
      return fail(RA_ERR_INVALID_ARG, "one KV block (%zu bytes) must be a multiple of 16 bytes",
                  blk);
    const BwdWsLayout w = bwd_ws_layout(prob, s);
    if (s.rows > 0) {
      if (workspace == nullptr || workspace_bytes < w.total)
        return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
      if (!aligned16(workspace))
        return fail(RA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    const void* ins[6] = {q, k, v, out, dout, lse};
    const size_t insz[6] = {qb, kvb, kvb, qfb, qb, rb};
    const void* outs[4] = {dq, dk, dv, s.rows > 0 ? workspace : nullptr};
    const size_t outsz[4] = {qfb, kfb, kfb, w.total};
    for (int o = 0; o < 4; ++o) {
      for (int i = 0; i < 6; ++i)
        if (overlap(outs[o], outsz[o], ins[i], insz[i]))
          return fail(RA_ERR_INVALID_ARG, "dq, dk, dv and workspace must not overlap any input");
      for (int o2 = o + 1; o2 < 4; ++o2)
        if (overlap(outs[o], outsz[o], outs[o2], outsz[o2]))
          return fail(RA_ERR_INVALID_ARG, "dq, dk, dv and workspace must not overlap each other");
    }
    if (s.rows == 0) return RA_OK;

    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    hipStream_t xs = static_cast<hipStream_t>(copy_stream);
    const bool sep = xs != nullptr && xs != cs && 2 * blk >= side_stream_min_bytes();
    DeviceEvents* de = nullptr;
    if ((st = get_events(&de)) != RA_OK) return st;
    std::lock_guard<std::mutex> lk(de->mu);
    if ((st = init_events(de)) != RA_OK) return st;

    char* ws = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(ws + w.delta);
    Stager sg{prob, &s, static_cast<const char*>(k), static_cast<const char*>(v), blk,
              {ws + w.stage_k[0], ws + w.stage_k[1]}, {ws + w.stage_v[0], ws + w.stage_v[1]},
              de, cs, xs, sep, rope_on(prob)};
    const size_t kelems = (size_t)s.kv_elems;  // floats per block of dk / dv
    const bool bf = prob->dtype == RA_BF16;
    hipError_t e;

    // D for every local row, dq from zero (the local queries rotated once
    // with rotary embedding), then the ring
    e = ra::launch_bwd_delta(s.rows, prob->head_dim, bf, out, dout, delta, cs);
    if (e != hipSuccess) return hip_fail(e, "delta launch");
    e = ra::launch_zero(dq, s.q_elems, cs);
    if (e != hipSuccess) return hip_fail(e, "zero launch");
    const void* qx = q;
    float* dktmp = reinterpret_cast<float*>(ws + w.dktmp);
    if (sg.rope) {
      void* qr = ws + w.qrot;
      ra::RopeParams r = make_rope(prob, s, true, prob->rank, prob->hq, bf, q, bf, qr, false, false);
      if ((e = ra::launch_rope(r, cs)) != hipSuccess) return hip_fail(e, "rope launch");
      qx = qr;
    }
    if ((st = sg.start()) != RA_OK) return st;
    for (int step = 0; step < n; ++step) {
      const void *kb = nullptr, *vb = nullptr;
      if ((st = sg.advance(step, &kb, &vb)) != RA_OK) return st;
      const int j = sg.block_of(step);
      if (!sg.rope) {
        if ((st = enqueue_bwd(prob, s, j, qx, kb, vb, dout, lse, delta, dq, dk + j * kelems,
                              dv + j * kelems, cs)) != RA_OK)
          return st;
      } else {
        // the dK addend is taken with respect to the rotated keys: form it
        // in a scratch block, turn it back and add it into dk[j]
        if ((e = ra::launch_zero(dktmp, s.kv_elems, cs)) != hipSuccess)
          return hip_fail(e, "zero launch");
        if ((st = enqueue_bwd(prob, s, j, qx, kb, vb, dout, lse, delta, dq, dktmp,
                              dv + j * kelems, cs)) != RA_OK)
          return st;
        ra::RopeParams r = make_rope(prob, s, false, j, prob->hkv, false, dktmp, false,
                                     dk + j * kelems, true, true);
        if ((e = ra::launch_rope(r, cs)) != hipSuccess) return hip_fail(e, "rope launch");
      }
      if ((st = sg.done(step)) != RA_OK) return st;
      if ((st = debug_sync(cs, sep ? xs : nullptr, "backward ring", step)) != RA_OK) return st;
    }
    if (sg.rope) {  // dq with respect to the unrotated queries
      ra::RopeParams r = make_rope(prob, s, true, prob->rank, prob->hq, false, dq, false, dq, true,
                                   false);
      if ((e = ra::launch_rope(r, cs)) != hipSuccess) return hip_fail(e, "rope launch");
    }
    return debug_sync(cs, nullptr, "backward ring end", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_rope_apply(const ra_problem* prob, int32_t target, int32_t block_j, int32_t heads,
                        int32_t in_dtype, const void* x, int32_t out_dtype, void* y,
                        int32_t inverse, int32_t accumulate, void* hip_stream) {
  try {
    Shape s;
    ra_status st = validate_problem(prob, &s);
    if (st != RA_OK) return st;
    if (!(prob->rope_theta > 0.f)) return fail(RA_ERR_INVALID_ARG, "rope_theta must be > 0");
    if (target != RA_ROPE_QUERIES && target != RA_ROPE_KEYS)
      return fail(RA_ERR_INVALID_ARG, "target %d unknown", target);
    if (block_j < 0 || block_j >= prob->n_ring)
      return fail(RA_ERR_INVALID_ARG, "block_j %d out of [0, n_ring=%d)", block_j, prob->n_ring);
    if (heads < 1) return fail(RA_ERR_INVALID_ARG, "heads %d < 1", heads);
    if ((in_dtype != RA_F32 && in_dtype != RA_BF16) || (out_dtype != RA_F32 && out_dtype != RA_BF16))
      return fail(RA_ERR_INVALID_ARG, "dtypes must be RA_F32 or RA_BF16");
    if (accumulate && out_dtype != RA_F32)
      return fail(RA_ERR_INVALID_ARG, "accumulate needs a float32 output");
    const bool queries = target == RA_ROPE_QUERIES;
    const int64_t len = queries ? prob->q_len : prob->kv_len;
    const int64_t elems = (int64_t)prob->batch * len * heads * prob->head_dim;
    if (elems > (int64_t(1) << 40)) return fail(RA_ERR_INVALID_ARG, "tensor too large");
    const size_t xb = elems * (in_dtype == RA_BF16 ? 2 : 4), yb = elems * (out_dtype == RA_BF16 ? 2 : 4);
    if ((st = check_ptr(x, xb, "x")) || (st = check_ptr(y, yb, "y"))) return st;
    if (x != y && overlap(x, xb, y, yb))
      return fail(RA_ERR_INVALID_ARG, "y partially overlaps x");
    if (x == y && (in_dtype != out_dtype || accumulate))
      return fail(RA_ERR_INVALID_ARG, "in place needs equal dtypes and no accumulate");
    if (elems == 0) return RA_OK;
    ra::RopeParams r = make_rope(prob, s, queries, queries ? prob->rank : block_j, heads,
                                 in_dtype == RA_BF16, x, out_dtype == RA_BF16, y, inverse != 0,
                                 accumulate != 0);
    hipError_t e = ra::launch_rope(r, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    return debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "rope", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

int32_t ra_tile_class_host(const ra_problem* prob, int32_t kv_block_j, int64_t a_lo, int64_t a_hi,
                           int64_t b_lo, int64_t b_hi) {
  Shape s;
  if (validate_problem(prob, &s) != RA_OK) return -1;
  if (kv_block_j < 0 || kv_block_j >= prob->n_ring) {
    fail(RA_ERR_INVALID_ARG, "kv_block_j out of range");
    return -1;
  }
  if (a_lo < 0 || a_hi < a_lo || a_hi >= prob->q_len || b_lo < 0 || b_hi < b_lo ||
      b_hi >= prob->kv_len) {
    fail(RA_ERR_INVALID_ARG, "tile bounds out of range");
    return -1;
  }
  ra::BlockGeom g = ra::block_geom(prob->causal, prob->layout, prob->rank, kv_block_j);
  if (s.packed) return ra::tile_class_packed(g, s.seg, a_lo, a_hi, b_lo, b_hi);
  return ra::tile_class(g, a_lo, a_hi, b_lo, b_hi, prob->kv_len);
}

static ra_status check_tiles(const ra_problem* prob, int32_t j, int32_t tq, int32_t tk,
                             Shape* s) {
  ra_status st = validate_problem(prob, s);
  if (st != RA_OK) return st;
  if (j < 0 || j >= prob->n_ring) return fail(RA_ERR_INVALID_ARG, "kv_block_j out of range");
  if (tq < 1 || tk < 1) return fail(RA_ERR_INVALID_ARG, "tile sizes must be >= 1");
  const int64_t nqt = (prob->q_len + tq - 1) / tq, nkt = (prob->kv_len + tk - 1) / tk;
  if (nqt * nkt > (int64_t(1) << 34)) return fail(RA_ERR_INVALID_ARG, "too many tiles");
  return RA_OK;
}

ra_status ra_tile_classes_host(const ra_problem* prob, int32_t kv_block_j, int32_t tq, int32_t tk,
                               int8_t* out_host) {
  try {
    Shape s;
    ra_status st = check_tiles(prob, kv_block_j, tq, tk, &s);
    if (st != RA_OK) return st;
    const int64_t nqt = (prob->q_len + tq - 1) / tq, nkt = (prob->kv_len + tk - 1) / tk;
    if (nqt * nkt > 0 && out_host == nullptr) return fail(RA_ERR_INVALID_ARG, "out is NULL");
    ra::BlockGeom g = ra::block_geom(prob->causal, prob->layout, prob->rank, kv_block_j);
    for (int64_t qt = 0; qt < nqt; ++qt) {
      const int64_t a_lo = qt * tq, a_hi = std::min<int64_t>(a_lo + tq, prob->q_len) - 1;
      for (int64_t kt = 0; kt < nkt; ++kt) {
        const int64_t b_lo = kt * tk, b_hi = std::min<int64_t>(b_lo + tk, prob->kv_len) - 1;
        out_host[qt * nkt + kt] =
            (int8_t)(s.packed ? ra::tile_class_packed(g, s.seg, a_lo, a_hi, b_lo, b_hi)
                              : ra::tile_class(g, a_lo, a_hi, b_lo, b_hi, prob->kv_len));
      }
    }
    return RA_OK;
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

ra_status ra_tile_classes_device(const ra_problem* prob, int32_t kv_block_j, int32_t tq,
                                 int32_t tk, int8_t* out_device, void* hip_stream) {
  try {
    Shape s;
    ra_status st = check_tiles(prob, kv_block_j, tq, tk, &s);
    if (st != RA_OK) return st;
    const int64_t nqt = (prob->q_len + tq - 1) / tq, nkt = (prob->kv_len + tk - 1) / tk;
    if (nqt * nkt == 0) return RA_OK;
    if (out_device == nullptr) return fail(RA_ERR_INVALID_ARG, "out is NULL");
    ra::BlockGeom g = ra::block_geom(prob->causal, prob->layout, prob->rank, kv_block_j);
    hipError_t e = ra::launch_tile_classes(g.kind, g.delta, prob->q_len, prob->kv_len, tq, tk,
                                           s.packed ? &s.seg : nullptr, out_device,
                                           static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "tile_classes launch");
    return debug_sync(static_cast<hipStream_t>(hip_stream), nullptr, "tile_classes", -1);
  } catch (...) {
    return fail(RA_ERR_HIP, "unexpected C++ exception");
  }
}

}  // extern "C"
