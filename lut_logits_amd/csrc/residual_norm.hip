// residual_norm.hip -- the glue of the per-token decode loop around each MLP block.
//
// The pages give the compressed parts of the model, not the model around them.
// The decode loop takes Gemma-2's glue in its plainest form: the embedding row
// times sqrt(D) starts a residual stream; every MLP block reads the stream
// through an RMSNorm and its output is added back through another; a last
// RMSNorm feeds the head. The norms carry unit scales (Gemma-2 stores each
// scale as 1 + w, and w = 0 untrained):
//     rms(v) = v / sqrt(mean(v^2) + eps).
// One launch does a block's whole glue on the stream h:
//     h += rms(y)     (y: the block's output; skipped without one)
//     x  = rms(h)     (the next block's input, or the head's hidden vector)
// One workgroup: the vectors are a few thousand floats (the Gemma-2-2B stream
// is 2,304), so the launch, not the bytes, is the cost; it replaces the five
// or six elementwise and reduction launches the same glue takes in torch.
// Sums of squares are taken per thread in index order, then over the wave by
// lane shuffles, then over the waves in wave order: a fixed order, so the
// result is deterministic.
#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kNormThreads = 1024;
constexpr int kNormWaves = kNormThreads / 64;

// Sum of v over the workgroup (every thread gets it); red holds kNormWaves floats.
__device__ float block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();   // red may still be read from the previous sum
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kNormWaves; ++w) s += red[w];
  return s;
}

__global__ __launch_bounds__(kNormThreads) void residual_norm_kernel(const float* __restrict__ y, float* __restrict__ h,
                                                                     float* __restrict__ x, int D, float eps) {
  __shared__ float red[kNormWaves];
  const int tid = threadIdx.x;
  const float inv_d = 1.0f / (float)D;
  if (y) {   // (uniform: a kernel argument)
    float ss = 0.0f;
    for (int i = tid; i < D; i += kNormThreads) ss = fmaf(y[i], y[i], ss);
    const float ry = 1.0f / sqrtf(block_sum(ss, red) * inv_d + eps);
    for (int i = tid; i < D; i += kNormThreads) h[i] += y[i] * ry;
  }
  // each thread reads back only the elements it wrote itself: no barrier needed before the sum
  float ss = 0.0f;
  for (int i = tid; i < D; i += kNormThreads) ss = fmaf(h[i], h[i], ss);
  const float rh = 1.0f / sqrtf(block_sum(ss, red) * inv_d + eps);
  for (int i = tid; i < D; i += kNormThreads) x[i] = h[i] * rh;
}

}  // namespace

hipError_t launch_residual_norm(const float* y, float* h, float* x, int D, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(residual_norm_kernel, dim3(1), dim3(kNormThreads), 0, stream, y, h, x, D, eps);
  return hipGetLastError();
}

}  // namespace rq
