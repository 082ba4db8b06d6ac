// ra_rope.hip -- rotary position embedding applied on arrival.
//
// Page (cited by title and section): troisinh.com "Ring Attention -- K/V
// truyen vong giua GPU, context trieu token", section "RoPE va Position
// Embedding": a key block arriving from another device must be rotated by
// the angle m*theta of each token's own position m, known from position
// metadata carried with the block. The ring applies this while it stages
// the block (the copy already reads and writes every byte of it), and to the
// local queries once.
//
// One thread turns four head-dimension pairs of one (token, head): 8
// consecutive elements, one 16-byte (bf16) or two 16-byte (fp32) accesses.
// The angle pos * inv_freq reaches ~1e6 radians at a 1M-token position, far
// beyond float32's resolution there, so it is formed and reduced modulo 2*pi
// in float64 and only the reduced angle goes to float32 sine and cosine.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ra_device.h"
#include "ra_kernels.h"
#include "ra_sched.h"

namespace ra {

__global__ __launch_bounds__(kThreads) void rope_kernel(RopeParams p) {
  const int groups = p.head_dim / 8;  // 8-element groups per (token, head)
  const int64_t total = (int64_t)p.batch * p.len * p.heads * groups;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const double two_pi = 6.283185307179586;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int gi = (int)(i % groups);
    const int64_t th = i / groups;                 // (b, a, h) flattened
    const int a = (int)((th / p.heads) % p.len);
    int64_t pos;
    if (p.packed) {
      const int s = segment_of(p.seg, a);
      pos = token_position(p.layout, p.n_ring, p.block, p.seg.off[s + 1] - p.seg.off[s],
                           a - p.seg.off[s]);
    } else {
      pos = token_position(p.layout, p.n_ring, p.block, p.len, a);
    }
    float x[8];
    const int64_t e0 = th * p.head_dim + gi * 8;
    if (p.in_bf16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) + e0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.x) + e0);
      const f32x4 u = src[0], v = src[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = u[k];
        x[4 + k] = v[k];
      }
    }
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double ang = (double)pos * p.inv_freq[gi * 4 + k];
      float r = (float)(ang - two_pi * rint(ang / two_pi));
      if (p.inverse) r = -r;
      float sn, cs;
      sincosf(r, &sn, &cs);
      y[2 * k] = x[2 * k] * cs - x[2 * k + 1] * sn;
      y[2 * k + 1] = x[2 * k] * sn + x[2 * k + 1] * cs;
    }
    if (p.out_bf16) {
      f32x8 v8;
#pragma unroll
      for (int k = 0; k < 8; ++k) v8[k] = y[k];
      const bf16x8 b8 = __builtin_convertvector(v8, bf16x8);
      *reinterpret_cast<bf16x8*>(reinterpret_cast<uint16_t*>(p.y) + e0) = b8;
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.y) + e0);
      f32x4 u = {y[0], y[1], y[2], y[3]}, v = {y[4], y[5], y[6], y[7]};
      if (p.accumulate) {
        const f32x4 u0 = dst[0], v0 = dst[1];
        u += u0;
        v += v0;
      }
      dst[0] = u;
      dst[1] = v;
    }
  }
}

hipError_t launch_rope(const RopeParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.batch * p.len * p.heads * (p.head_dim / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
