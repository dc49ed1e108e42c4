// dense_gemv.hip -- the comparison baseline: logits from a dense bf16 head.
//
// The pages' standard path keeps the head as a full bf16 matrix and computes
// logits with one matmul (Gemma-2-2B runtime-compression page, variant
// table, "Uncompressed" row). This kernel is that path on the same GPU, so the
// LUT head can be timed against it: E[rows][D] bf16 times up to 16 hidden
// vectors rounded to bf16, accumulated in fp32 on the matrix cores
// (v_mfma_f32_16x16x32_bf16), then the same softcap and argmax selection as
// the LUT head (best key per block, reduced by the selection kernel).
//
// A wave owns 16 rows at a time: each lane loads 16 bytes (8 bf16) of one row
// per k-step, so a wave-wide load is 16 rows x 64 contiguous bytes, and the
// hidden vectors (as bf16, padded to 16 columns) sit in LDS. Bound: HBM
// (2*D bytes per row); the matrix cores idle most of the time.
#include "rq_internal.h"

namespace rq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kDenseThreads = 256;
constexpr int kTilesPerWave = kDenseRowsPerBlock / 16 / (kDenseThreads / 64);
constexpr int kKUnroll = 8;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kDenseThreads) void dense_logits_kernel(const uint16_t* __restrict__ E, int64_t rows,
                                                                     int D, const float* __restrict__ h, int B,
                                                                     float softcap, float* __restrict__ logits,
                                                                     uint64_t* __restrict__ block_keys) {
  extern __shared__ __align__(16) uint16_t hs[];   // [16][Dp] bf16
  __shared__ unsigned long long bmax[16];
  const int Dp = D + 8;
  for (int i = threadIdx.x; i < 16 * D; i += kDenseThreads) {
    const int b = i / D;
    const int c = i - b * D;
    hs[b * Dp + c] = b < B ? f32_to_bf16(h[(size_t)b * D + c]) : (uint16_t)0;
  }
  if (threadIdx.x < 16) bmax[threadIdx.x] = 0ull;
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15;   // A: row within the tile; B and C: batch column
  const int kg = lane >> 4;    // which 8 of the 32 k-values this lane feeds
  const bf16x8 zero = {};
  for (int tile = 0; tile < kTilesPerWave; ++tile) {
    const int64_t row_base = (int64_t)blockIdx.x * kDenseRowsPerBlock + (int64_t)(wave * kTilesPerWave + tile) * 16;
    const int64_t row = row_base + i16;
    const bool rvalid = row < rows;
    const uint16_t* erow = E + (rvalid ? row : 0) * (int64_t)D;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < D; k0 += 32 * kKUnroll) {
      bf16x8 a[kKUnroll];
#pragma unroll
      for (int u = 0; u < kKUnroll; ++u) {
        const int col = k0 + u * 32 + 8 * kg;
        a[u] = (rvalid && col < D) ? load_bf16x8(erow + col) : zero;
      }
#pragma unroll
      for (int u = 0; u < kKUnroll; ++u) {
        const int col = k0 + u * 32 + 8 * kg;
        const bf16x8 bv = col < D ? *reinterpret_cast<const bf16x8*>(hs + i16 * Dp + col) : zero;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bv, acc, 0, 0, 0);
      }
    }
    // acc[t] = C[row_base + 4*kg + t][batch i16]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t r = row_base + 4 * kg + t;
      if (r < rows && i16 < B) {
        const float z = acc[t];
        const float v = softcap > 0.0f ? softcap * tanhf(z / softcap) : z;
        logits[(size_t)i16 * rows + r] = v;
        if (block_keys) atomicMax(&bmax[i16], (unsigned long long)select_key(v, (uint32_t)r));
      }
    }
  }
  if (!block_keys) return;
  __syncthreads();
  if (threadIdx.x < B) block_keys[(size_t)threadIdx.x * gridDim.x + blockIdx.x] = bmax[threadIdx.x];
}

}  // namespace

hipError_t launch_dense_logits(const uint16_t* E, int64_t rows, int D, const float* h, int B, float softcap,
                               float* logits, uint64_t* block_keys, hipStream_t stream) {
  const size_t lds = (size_t)16 * (D + 8) * sizeof(uint16_t);
  hipError_t e = hipFuncSetAttribute((const void*)dense_logits_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_logits_kernel, dim3((unsigned)dense_blocks(rows)), dim3(kDenseThreads), lds, stream, E,
                     rows, D, h, B, softcap, logits, block_keys);
  return hipGetLastError();
}

}  // namespace rq
