// stream_probe.hip -- measurement aids, not part of the method. The first
// reads a
// buffer once with 16-byte loads and nothing else, so that its rate is the
// HBM stream-read ceiling this GPU reaches. The lookup+sum pass is a code
// stream plus table lookups; its achieved bandwidth is reported against this
// ceiling as well as against the 8 TB/s specification.
//
// Workgroups of 1024 threads stride over the buffer as one grid: in every
// round the grid's loads cover one contiguous span, and each thread keeps U
// 16-byte loads in flight. The configurations differ in grid size (one to
// eight workgroups per CU) and U (1, 2, 4 or 8); the caller keeps the fastest.
// The second (below) measures random gathers from LDS, the roof of the lookups
// when a batch of vectors makes them, not the code stream, the bound.
#include <hip/hip_ext.h>

#include "rq_internal.h"

namespace rq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 1024;
struct StreamConfig {
  int wgs, unroll;
};
constexpr StreamConfig kStreamConfig[] = {{256, 4}, {512, 4}, {1024, 4}, {2048, 4},
                                          {256, 8}, {512, 8}, {256, 2}, {512, 2}, {256, 1}, {512, 1}};
constexpr int kStreamConfigs = sizeof(kStreamConfig) / sizeof(kStreamConfig[0]);

template <int kStreamUnroll>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // XOR of the workgroup's words (so the loads cannot be dropped, and the
  // sink's XOR over all workgroups is the XOR of every word of the buffer)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t s_acc[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < kStreamThreads / 64; ++k) w ^= s_acc[k];
    sink[blockIdx.x] = w;
  }
}

// ---- LDS random-gather probe: the on-chip roof of the batched lookups.
// One 1024-thread workgroup per CU fills 128 KB of LDS with word i = i *
// 2654435761, then every thread runs 8 independent linear congruential
// sequences (x = x * 1664525 + 1013904223, seeded with 8 * global thread id +
// chain) and reads, per step of each, the W-byte entry whose index is the top
// bits of x (a uniformly random entry of the 128 KB, as a code picks a random
// codeword). The looked-up words are XORed together, and each workgroup writes
// the XOR of its threads' results, so no read can be dropped and the host can
// recompute the sink exactly.
constexpr int kLdsProbeThreads = 1024;
constexpr int kLdsProbeBytes = 128 * 1024;
constexpr int kLdsProbeChains = 8;

template <int W>
__global__ __launch_bounds__(kLdsProbeThreads) void lds_gather_kernel(int reps, uint32_t* __restrict__ sink) {
  extern __shared__ __align__(16) uint32_t tab[];
  constexpr int kWords = kLdsProbeBytes / 4;
  constexpr int kEntries = kLdsProbeBytes / W;
  constexpr int kBits = __builtin_ctz(kEntries);
  const int tid = threadIdx.x;
  for (int i = tid; i < kWords; i += kLdsProbeThreads) tab[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  uint32_t x[kLdsProbeChains];
  const uint32_t gid = (uint32_t)(blockIdx.x * kLdsProbeThreads + tid);
#pragma unroll
  for (int c = 0; c < kLdsProbeChains; ++c) x[c] = gid * kLdsProbeChains + c;
  uint32_t acc = 0u;
  for (int r = 0; r < reps; ++r) {
    uint32_t v[kLdsProbeChains];
#pragma unroll
    for (int c = 0; c < kLdsProbeChains; ++c) {
      x[c] = x[c] * 1664525u + 1013904223u;
      const uint32_t idx = x[c] >> (32 - kBits);
      if constexpr (W == 2) {
        v[c] = reinterpret_cast<const uint16_t*>(tab)[idx];
      } else if constexpr (W == 4) {
        v[c] = tab[idx];
      } else if constexpr (W == 8) {
        const uint2 w = reinterpret_cast<const uint2*>(tab)[idx];
        v[c] = w.x ^ w.y;
      } else {
        const u32x4 w = reinterpret_cast<const u32x4*>(tab)[idx];
        v[c] = w[0] ^ w[1] ^ w[2] ^ w[3];
      }
    }
#pragma unroll
    for (int c = 0; c < kLdsProbeChains; ++c) acc ^= v[c];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t s_acc[kLdsProbeThreads / 64];
  if ((tid & 63) == 0) s_acc[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < kLdsProbeThreads / 64; ++k) w ^= s_acc[k];
    sink[blockIdx.x] = w;
  }
}

}  // namespace

size_t lds_gather_sink_words() { return (size_t)kCUs; }

hipError_t launch_lds_gather(int width, int reps, uint32_t* sink, hipStream_t stream) {
  auto kern = width == 2 ? lds_gather_kernel<2> : width == 4 ? lds_gather_kernel<4>
            : width == 8 ? lds_gather_kernel<8> : lds_gather_kernel<16>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsProbeBytes);
  if (e != hipSuccess) return e;
  hipEvent_t before, after;
  take_stage_events(&before, &after);
  if (before || after)
    hipExtLaunchKernelGGL(kern, dim3(kCUs), dim3(kLdsProbeThreads), kLdsProbeBytes, stream, before, after, 0, reps, sink);
  else
    hipLaunchKernelGGL(kern, dim3(kCUs), dim3(kLdsProbeThreads), kLdsProbeBytes, stream, reps, sink);
  return hipGetLastError();
}

int stream_read_configs() { return kStreamConfigs; }
size_t stream_read_sink_words(int config) { return (size_t)kStreamConfig[config].wgs; }

hipError_t launch_stream_read(const void* src, size_t bytes, int config, uint32_t* sink, hipStream_t stream) {
  const dim3 grid((unsigned)kStreamConfig[config].wgs);
  const int unroll = kStreamConfig[config].unroll;
  auto kern = unroll == 1   ? stream_read_kernel<1>
              : unroll == 2 ? stream_read_kernel<2>
              : unroll == 8 ? stream_read_kernel<8>
                            : stream_read_kernel<4>;
  const u32x4* s16 = static_cast<const u32x4*>(src);
  hipEvent_t before, after;
  take_stage_events(&before, &after);
  if (before || after)   // timed like the lookup+sum kernel: its own dispatch's start and end
    hipExtLaunchKernelGGL(kern, grid, dim3(kStreamThreads), 0, stream, before, after, 0, s16, bytes / 16, sink);
  else
    hipLaunchKernelGGL(kern, grid, dim3(kStreamThreads), 0, stream, s16, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace rq
