/*
 * ra.h -- C ABI of the MI355X (gfx950) Ring Attention per-device library.
 *
 * One device's share of Ring Attention: a fixed local query block attends to
 * N arriving key/value blocks; each block yields a partial (running max m,
 * normaliser l, unnormalised accumulator acc) and partials are merged by
 * online-softmax rescaling. On one GPU the ring is a loop of N steps whose
 * next block is staged by a double-buffered device-to-device copy on a side
 * stream.
 *
 * Pages defining the operations (cited by title and section):
 *   [UL] Ultralytics glossary "Ring Attention", section "How ring attention
 *        works": N blocks, each device keeps its query block, attends to the
 *        block it holds, forwards it and receives the next; running sums of
 *        exponentiated scores and of weighted values, divided at the end;
 *        max subtraction in production kernels; striped token assignment.
 *   [TS] troisinh.com "Ring Attention -- K/V truyen vong giua GPU, context
 *        trieu token", sections "Y tuong cot loi" (fixed Q, K/V rotating,
 *        associative merge) and "Tai sao no hoat dong" (the running max and
 *        normaliser update; output rescaled the same way).
 *   [JS] jisaku.com glossary "Ring Attention", sections on the processing
 *        flow and on overlapping communication with computation.
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major [batch, seq, heads, head_dim], head_dim
 *     contiguous. Query head h reads KV head h / (hq / hkv).
 *   - q, k, v are bfloat16 (RA_BF16) or float32 (RA_F32); m, l, acc, out,
 *     lse are float32. m is in natural-log units of scaled scores.
 *   - All pointers are device pointers the caller allocated; the library
 *     never allocates or frees device memory. Every data pointer must be
 *     16-byte aligned. Streams are hipStream_t passed as void* (NULL = the
 *     null stream of the current device); the current HIP device must be the
 *     device owning the pointers and streams.
 *   - Validation runs on the host before any HIP call. On failure an entry
 *     point returns a non-zero ra_status, sets ra_last_error(), and enqueues
 *     nothing. HIP API failures return RA_ERR_HIP. Work is asynchronous:
 *     device faults surface at the caller's next synchronisation. No C++
 *     exception crosses this ABI.
 *   - Empty problems (batch or q_len zero) return RA_OK and enqueue
 *     nothing.
 *
 * Environment (read at every call)
 *   RA_DEBUG_SYNC=1    after its launches (the rings: after every step) an
 *                      entry point waits for its streams and returns
 *                      RA_ERR_HIP naming the launch or step of the first
 *                      device error. Not for calls under graph capture.
 *   RA_DEBUG_POISON=1  the rings fill each staging buffer with NaN right
 *                      before the copy that refills it, so a read that
 *                      races the copy yields NaN rather than a stale block.
 *   RA_SIDE_STREAM_MIN_BYTES  see ra_ring_fwd.
 *   RA_WAVES=4 | 8     waves per workgroup of the bf16 attention kernel
 *                      (default: 8, or 4 when a launch of 8-wave workgroups
 *                      would have fewer workgroups than the GPU has CUs).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,  /* bad shape, pointer, alignment, enum, alias   */
  RA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim)         */
  RA_ERR_WORKSPACE = 3,    /* workspace missing or too small               */
  RA_ERR_HIP = 4           /* a HIP runtime call or launch failed          */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* Token layouts ([UL] striping remark; contiguous chunks per device; [AU]
 * names zigzag as a variant that rebalances causal work).
 * contiguous: block i holds global tokens [i*B, (i+1)*B).
 * striped:    token t belongs to block t mod N at local index t / N.
 * zigzag:     the sequence is cut into 2N chunks of B/2 tokens; block i holds
 *             chunk i (local 0..B/2-1) then chunk 2N-1-i. B must be even.
 *             Every device then does the same causal work.
 * The caller stores q, k, v already in the layout's token order. */
typedef enum {
  RA_LAYOUT_CONTIGUOUS = 0,
  RA_LAYOUT_STRIPED = 1,
  RA_LAYOUT_ZIGZAG = 2
} ra_layout;

/* Most packed sequences one problem may hold (ra_problem.n_seqs). */
#define RA_MAX_SEQS 256

/* Class of a (query tile, key tile) pair under the causal mask. */
typedef enum { RA_TILE_SKIP = 0, RA_TILE_PARTIAL = 1, RA_TILE_FULL = 2 } ra_tile_class;

typedef struct {
  int32_t dtype;     /* ra_dtype of q, k, v                                  */
  int32_t batch;     /* >= 0                                                 */
  int32_t hq;        /* query heads, >= 1                                    */
  int32_t hkv;       /* key/value heads, >= 1, hq % hkv == 0                 */
  int32_t head_dim;  /* 16, 32, 64 or 128 (others: RA_ERR_UNSUPPORTED)       */
  int64_t q_len;     /* local queries (this device's block), 0..2^30         */
  int64_t kv_len;    /* keys per KV block, 0..2^30                           */
  int32_t n_ring;    /* N >= 1                                               */
  int32_t rank;      /* r, 0 <= r < N: the device whose share is computed    */
  int32_t causal;    /* 0 or 1; causal requires q_len == kv_len              */
  int32_t layout;    /* ra_layout                                            */
  float scale;       /* score scale; <= 0 selects 1/sqrt(head_dim); NaN/inf
                        are invalid                                          */
  /* Packed variable-length sequences ([TS] "Trade-off thuc te": sequences
   * of different lengths). n_seqs = 0: one sequence per batch row (the
   * fields below are ignored). n_seqs >= 1: batch must be 1 and cu_seqlens
   * is a HOST array of n_seqs + 1 int64 offsets into the packed global
   * sequence (cu_seqlens[0] = 0, nondecreasing; read during the call only).
   * Every length L_s = cu_seqlens[s+1] - cu_seqlens[s] must be a multiple of
   * n_ring (of 2*n_ring for zigzag), and q_len == kv_len ==
   * cu_seqlens[n_seqs] / n_ring. Each sequence is split over the N blocks by
   * the layout on its own; a block holds the L_s / N tokens of sequence 0,
   * then those of sequence 1, and so on. A key is visible to a query only
   * inside the same sequence (and, if causal, at a position <= the
   * query's within it). At most RA_MAX_SEQS sequences. */
  int32_t n_seqs;
  const int64_t* cu_seqlens;
  /* Rotary position embedding applied on arrival ([TS] "RoPE va Position
   * Embedding": an arriving key block is rotated by m*theta for each token's
   * own position m, known from the block's position metadata). 0: none.
   * > 0: the base of theta_i = rope_theta^(-2i/head_dim); ra_ring_fwd and
   * ra_ring_bwd then rotate the local queries once and every K block while
   * staging it (head-dim pairs (2i, 2i+1) turn by pos * theta_i,
   * counter-clockwise; pos is the token's global position, within its
   * sequence when packed), and ra_ring_bwd returns gradients with respect
   * to the unrotated q and k. The block-level entry points ignore it (they
   * take already rotated inputs, see ra_rope_apply). Negative or non-finite
   * values are invalid. */
  float rope_theta;
} ra_problem;

/*
 * Partial attention of the local queries against one arriving KV block j
 * ([UL] "How ring attention works": the per-step computation against the
 * block the device currently holds; max subtraction as in production kernels).
 *
 *   q   [batch, q_len, hq, head_dim]   dtype, read
 *   k,v [batch, kv_len, hkv, head_dim] dtype, read: block j's tokens
 *   m,l [batch, q_len, hq]             float32, written
 *   acc [batch, q_len, hq, head_dim]   float32, written
 * For each query row: m = max visible scaled score, l = sum exp(s - m),
 * acc = sum exp(s - m) v. Rows with no visible key get (-inf, 0, 0). Global
 * positions come from (layout, n_ring, rank) for queries and (layout,
 * n_ring, j) for keys; causal masks keys whose position exceeds the query's;
 * packed sequences (n_seqs >= 1) also mask keys of other sequences.
 * Fully masked (query tile, key tile) pairs are never computed.
 * Outputs must not overlap the inputs.
 */
ra_status ra_block_attn_partial(const ra_problem* prob, int32_t kv_block_j,
                                const void* q, const void* k, const void* v,
                                float* m, float* l, float* acc, void* hip_stream);

/*
 * One ring step's running update ([UL] "How ring attention works": the
 * running sums grow with each arriving block; [TS] "Tai sao no hoat dong":
 * the running max and normaliser update, the output rescaled the same way):
 * block j's partial, as ra_block_attn_partial defines it, merged into the
 * running state (m, l, acc) in place with the merge of ra_merge_partials
 * (the running state as input 1). One kernel: the block's partial never
 * leaves the GPU's registers. m, l, acc are read and written; arguments,
 * shapes, validation and overlap rules as ra_block_attn_partial. A block
 * with no visible pair leaves the state unchanged (nothing is enqueued).
 * ra_ring_fwd takes the first block with ra_block_attn_partial's kernel and
 * every later one with this.
 */
ra_status ra_block_attn_accumulate(const ra_problem* prob, int32_t kv_block_j,
                                   const void* q, const void* k, const void* v,
                                   float* m, float* l, float* acc, void* hip_stream);

/*
 * Online-softmax merge of two partials ([TS] "Tai sao no hoat dong"):
 *   m = max(m1, m2); a_i = exp(m_i - m) (0 when m_i = -inf);
 *   l = a1 l1 + a2 l2; acc = a1 acc1 + a2 acc2.
 * Two empty partials merge to (-inf, 0, 0). rows = batch*q_len*hq;
 * m*, l* are [rows] and acc* [rows, head_dim], float32. The outputs may alias
 * input 1 or input 2 exactly (in-place running update), not partially.
 */
ra_status ra_merge_partials(int64_t rows, int32_t head_dim,
                            const float* m1, const float* l1, const float* acc1,
                            const float* m2, const float* l2, const float* acc2,
                            float* m_out, float* l_out, float* acc_out,
                            void* hip_stream);

/*
 * Final divide ([UL]: the accumulated numerator is divided by the
 * denominator at the end): acc <- acc / l in place, and, when lse is not
 * NULL, lse = m + ln l. Rows with l == 0 give 0 and lse = -inf.
 */
ra_status ra_finalize(int64_t rows, int32_t head_dim, const float* m, const float* l,
                      float* acc, float* lse, void* hip_stream);

/* Workspace bytes ra_ring_fwd needs for this problem (0 on invalid input):
 * two staging buffers for K and two for V and the running m and l (with
 * rope_theta > 0 also the rotated queries); the running acc is out. */
size_t ra_ring_workspace_bytes(const ra_problem* prob);

/*
 * One device's whole share of the ring ([UL] "How ring attention works";
 * [JS] processing flow and communication/compute overlap).
 *
 *   q     [batch, q_len, hq, head_dim]            dtype: local queries
 *   k, v  [n_ring, batch, kv_len, hkv, head_dim]  dtype: all N blocks,
 *         stored in the layout's token order (a stand-in for the blocks that
 *         would arrive from the previous device)
 *   out   [batch, q_len, hq, head_dim] float32: attention output; also used
 *         as the running accumulator
 *   lse   [batch, q_len, hq] float32 or NULL: m + ln l
 *   workspace: device buffer of at least ra_ring_workspace_bytes(prob)
 *
 * Step s uses block j = (rank - s) mod N. Step 0 reads the local block in
 * place; for s >= 1 block j is first copied into staging buffer s % 2 on
 * copy_stream while step s-1 computes on compute_stream (events order the
 * copy after the last read of that buffer, and the compute after the copy).
 * Step 0's partial starts the running state (m, l in the workspace, acc in
 * out); every later computed block is merged into it by the same kernel
 * (ra_block_attn_accumulate), and the last computed block's kernel also
 * divides, so the ring launches one kernel per computed block plus its
 * staging copies.
 * With rope_theta > 0 every step's K block, the local one included, is
 * staged and rotated on the way (V is copied as is).
 * Blocks whose every pair is masked are still staged but not computed.
 * copy_stream may be NULL or equal to compute_stream: copies then run in
 * order on compute_stream. They also run in order there when one step's
 * copy (its K and V block) is under 32 MiB: a second stream costs each step
 * two cross-stream waits on the critical path (about 10 us on MI355X),
 * more than copies that small take (environment RA_SIDE_STREAM_MIN_BYTES
 * overrides the size; 0 always uses copy_stream). The results are the same
 * bits either way. On return all work is enqueued; everything
 * enqueued on copy_stream is ordered before the last kernel on
 * compute_stream, so synchronising compute_stream is enough.
 * Calls on the same device are serialised internally while enqueuing;
 * concurrent calls must not share a workspace.
 */
ra_status ra_ring_fwd(const ra_problem* prob, const void* q, const void* k, const void* v,
                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream);

/* Bytes of the static workspace of ra_ring_fwd_noalloc (per GPU). */
#define RA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * ra_ring_fwd without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, results and stream
 * contract as ra_ring_fwd (bit-identical outputs: the same kernels run);
 * the workspace is instead a library-owned device array of
 * RA_NOALLOC_WORKSPACE_BYTES on each GPU, held from the moment a device
 * loads the library until the process ends.
 *
 * No call allocates or frees device memory. The first call on a device
 * resolves the array's address there and creates the ring's event pool;
 * later calls create nothing. Problems whose ra_ring_workspace_bytes
 * exceeds RA_NOALLOC_WORKSPACE_BYTES return RA_ERR_WORKSPACE with nothing
 * enqueued (64 MiB holds a bf16 share of about 2000 tokens with 32 KV
 * heads at head_dim 128, about 7900 with 8 KV heads).
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; nothing in it needs clearing, since every step overwrites what it
 * reads. Calls whose work overlaps on one GPU (different streams, or
 * several host threads) race on the array: serialise them.
 */
ra_status ra_ring_fwd_noalloc(const ra_problem* prob, const void* q, const void* k,
                              const void* v, float* out, float* lse,
                              void* compute_stream, void* copy_stream);

/*
 * Causal tile scheduler, host mirror. Class of the pair (query rows
 * [a_lo, a_hi], keys [b_lo, b_hi]) of block j (local indices, inclusive;
 * for packed sequences, indices into the packed local share).
 * Returns an ra_tile_class, or -1 on invalid input. The attention kernels
 * decide which tiles to visit and which to mask with the same rule.
 */
int32_t ra_tile_class_host(const ra_problem* prob, int32_t kv_block_j,
                           int64_t a_lo, int64_t a_hi, int64_t b_lo, int64_t b_hi);

/* Classes of the full grid of tq x tk tiles of block j, row-major
 * [ceil(q_len/tq), ceil(kv_len/tk)] int8, into host memory (host mirror) or
 * device memory (computed by a kernel with the device form of the rule). */
ra_status ra_tile_classes_host(const ra_problem* prob, int32_t kv_block_j, int32_t tq,
                               int32_t tk, int8_t* out_host);
ra_status ra_tile_classes_device(const ra_problem* prob, int32_t kv_block_j, int32_t tq,
                                 int32_t tk, int8_t* out_device, void* hip_stream);

/*
 * Backward pass ([TS] "Blockwise Backward": the backward does not keep the
 * attention matrix; it recomputes the attention statistics, each device
 * only on the K/V block visiting it). With the forward's out and lse and an
 * upstream gradient dout, for the local queries against block j:
 *   P  = exp(scale q k^T - lse) on visible pairs,  D = rowsum(dout * out),
 *   dS = P * (dout v^T - D),
 *   dq += scale dS k,   dk_j += scale dS^T q,   dv_j += P^T dout
 * (grouped query heads add into the KV head they read). dq stays with the
 * queries; dk_j and dv_j are this device's addends to block j's gradients,
 * which in a ring travel with block j and collect every device's addend.
 */

/* D = rowsum(dout * out): rows = batch*q_len*hq; out float32 [rows, d];
 * dout [rows, d] of dtype (RA_BF16 or RA_F32); delta float32 [rows]. */
ra_status ra_attn_bwd_delta(int64_t rows, int32_t head_dim, int32_t dtype, const float* out,
                            const void* dout, float* delta, void* hip_stream);

/*
 * One arriving block's share of the backward pass (addends ACCUMULATED into
 * dq, dk, dv; the caller zeroes them first when it wants the bare addends).
 *   q, dout [batch, q_len, hq, head_dim]   dtype
 *   k, v    [batch, kv_len, hkv, head_dim] dtype: block j
 *   lse, delta [batch, q_len, hq]          float32 (forward lse; D above)
 *   dq      [batch, q_len, hq, head_dim]   float32, +=
 *   dk, dv  [batch, kv_len, hkv, head_dim] float32, +=
 * Masking, layouts and packed sequences as in ra_block_attn_partial. Rows
 * whose lse is -inf contribute nothing. dq, dk, dv must not overlap each
 * other or any input.
 */
ra_status ra_block_attn_bwd(const ra_problem* prob, int32_t kv_block_j, const void* q,
                            const void* k, const void* v, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv,
                            void* hip_stream);

/* Workspace bytes ra_ring_bwd needs (0 on invalid input): two staging
 * buffers for K and two for V, and D (with rope_theta > 0 also the rotated
 * queries and one float32 block for the rotated dK addend). */
size_t ra_ring_bwd_workspace_bytes(const ra_problem* prob);

/*
 * One device's whole share of the backward ring, the mirror of ra_ring_fwd:
 *   q, dout [batch, q_len, hq, head_dim]               dtype
 *   k, v    [n_ring, batch, kv_len, hkv, head_dim]     dtype (as ra_ring_fwd)
 *   out     [batch, q_len, hq, head_dim] float32, lse [batch, q_len, hq]
 *           float32: the forward's results for this share
 *   dq      [batch, q_len, hq, head_dim] float32: WRITTEN (overwritten)
 *   dk, dv  [n_ring, batch, kv_len, hkv, head_dim] float32: this share's
 *           addend to block j is ADDED to dk[j], dv[j] (the accumulators that
 *           travel with the blocks; calling this for every rank of a ring on
 *           the same zeroed dk, dv leaves the full key/value gradients)
 * Step s uses block j = (rank - s) mod N with the forward's staging scheme
 * (local block in place, the others copied on copy_stream into two staging
 * buffers, ordered by events). Fully masked blocks are staged, not computed.
 */
ra_status ra_ring_bwd(const ra_problem* prob, const void* q, const void* k, const void* v,
                      const float* out, const void* dout, const float* lse, float* dq,
                      float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      void* compute_stream, void* copy_stream);

/* Which tokens ra_rope_apply rotates: the local queries (block = rank,
 * q_len tokens) or the keys of block j (kv_len tokens). */
typedef enum { RA_ROPE_QUERIES = 0, RA_ROPE_KEYS = 1 } ra_rope_target;

/*
 * Rotary embedding of one block-shaped tensor [batch, len, heads, head_dim]
 * ([TS] "RoPE va Position Embedding"), with the positions the problem's
 * layout and packing give its tokens, and base prob->rope_theta (which must
 * be > 0). inverse turns by the negative angles (the transpose: it maps a
 * gradient with respect to rotated inputs to one with respect to unrotated
 * inputs). x has in_dtype, y out_dtype (RA_BF16 or RA_F32); y may equal x
 * (same dtype) but must not partially overlap it. accumulate = 1 adds the
 * result into y (out_dtype RA_F32 only).
 */
ra_status ra_rope_apply(const ra_problem* prob, int32_t target, int32_t block_j, int32_t heads,
                        int32_t in_dtype, const void* x, int32_t out_dtype, void* y,
                        int32_t inverse, int32_t accumulate, void* hip_stream);

/* Thread-local message describing the last failure on this thread. */
const char* ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
