// dense_gemv.hip -- the comparison baseline: logits from a dense bf16 head.
//
// The pages' standard path keeps the head as a full bf16 matrix and computes
// logits with one matmul (Gemma-2-2B runtime-compression page, variant
// table, "Uncompressed" row). This kernel is that path on the same GPU, so the
// LUT head can be timed against it: E[rows][D] bf16 times up to 128 hidden
// vectors rounded to bf16, accumulated in fp32 on the matrix cores
// (v_mfma_f32_16x16x32_bf16), then the same softcap and argmax selection as
// the LUT head (best key per block of rows, reduced by the selection kernel).
//
// Layout: E is held tiled, [ceil(rows/16)][Dp/32][16][32] bf16 (Dp = D rounded
// up to 32, zeros past rows and D), written once by rq_pack_dense. A tile's
// 16 rows x 32 columns are one contiguous 1 KB block, which is exactly what one
// wave-wide 16-byte load of the MFMA's B operand covers: every load of the
// kernel reads 1 KB of contiguous memory (row-major, a wave load touched 16
// rows of 64 bytes each).
//
// Mapping: C[b][r] = sum_k h[b][k] * E[r][k], with A = 16 hidden vectors x 32
// k (from LDS) and B = 32 k x 16 rows of E (from HBM). Lane (i16, kg) loads
// 16 bytes (8 bf16) of row i16 of its tile per k-step and receives
// C[4kg .. 4kg+3][row i16]: a store of one batch entry covers 16 consecutive
// rows (64 contiguous bytes). The hidden vectors are rounded to bf16 once, by
// a small kernel, into the workspace.
//
// Work split: a workgroup owns 256 rows (4 waves x 4 tiles of 16) and all
// hidden vectors (NT tiles of 16). The hidden vectors are staged in LDS as
// bf16 in chunks of KC columns (all of Dp when it fits); each wave keeps the E
// loads of the next k-steps in flight while the matrix cores work on the
// current ones. Bound: HBM (2*D bytes per row) for every B up to 128; the
// matrix cores need 2*B*D flops per row (151 GFLOP at B=128 on the Gemma
// head, about 60 us at the bf16 peak). Two waves per SIMD are asked for (the
// accumulators of eight column tiles then stay in the 256 registers beside the
// load buffers) so that two workgroups share a CU.
#include "rq_internal.h"

namespace rq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDenseThreads = 256;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kTilesPerWave = kDenseRowsPerBlock / 16 / kDenseWaves;   // 4
static_assert(kTilesPerWave * 16 * kDenseWaves == kDenseRowsPerBlock, "rows per block");

// k-steps (of 32 columns) whose E loads are issued together, per column-tile count.
constexpr int unroll_for(int NT) { return NT <= 2 ? 4 : 2; }
// Columns of h staged per chunk: the whole row for 16 vectors, else a chunk of
// at most 64 KB of bf16 (so two workgroups share a CU).
inline int chunk_cols(int D, int NT) {
  const int kc = NT == 1 ? D : 2048 / NT;
  return std::min(D, kc);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// hb[n][c] = bf16(h[n][c]) (round to nearest even), zero for n >= B or c >= D: Bp x Dp.
__global__ void dense_h_kernel(const float* __restrict__ h, int B, int D, int Dp, int Bp, uint16_t* __restrict__ hb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Bp * Dp) return;
  const int n = (int)(i / Dp);
  const int c = (int)(i - (int64_t)n * Dp);
  hb[i] = (n < B && c < D) ? f32_to_bf16(h[(size_t)n * D + c]) : (uint16_t)0;
}

// Et = the tiled layout of E[rows][D]: one thread per 8 consecutive elements of
// a tile row (16 bytes), zero past rows and D.
__global__ void pack_dense_kernel(const uint16_t* __restrict__ E, int64_t rows, int D, int KS,
                                  uint16_t* __restrict__ Et, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int64_t e = i * 8;                // element index in Et
  const int64_t blk = e / 512;            // (tile, k-step) block of 16 x 32
  const int w = (int)(e - blk * 512);
  const int64_t tile = blk / KS;
  const int ks = (int)(blk - tile * KS);
  const int64_t r = tile * 16 + w / 32;
  const int c = ks * 32 + (w % 32);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < rows && c < D) v = *reinterpret_cast<const u32x4*>(E + r * D + c);   // D % 8 == 0: whole 16 bytes
  *reinterpret_cast<u32x4*>(Et + e) = v;
}

template <int NT>
__global__ __launch_bounds__(kDenseThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void dense_logits_kernel(const uint16_t* __restrict__ Et, int64_t rows, int D, const uint16_t* __restrict__ hb,
                         int B, int KC, float softcap, float* __restrict__ logits, uint64_t* __restrict__ block_keys) {
  // D here is the padded width Dp (a multiple of 32); Et is tiled (see the file comment)
  constexpr int T = kTilesPerWave;
  constexpr int U = unroll_for(NT);
  constexpr int Bp = 16 * NT;
  extern __shared__ __align__(16) uint16_t hs[];   // [Bp][KC + 40] bf16
  __shared__ unsigned long long bmax[Bp];
  // Row stride of 2*(KC+40) bytes: lanes of one k-group hit different banks. Columns
  // [kc, kc+32) of each row are zeros: k-steps past the chunk read them.
  const int ldh = KC + 40;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i16 = lane & 15;   // A: batch row within a tile; B and C: row of E within a tile
  const int kg = lane >> 4;    // which 8 of the 32 k-values this lane feeds; C rows 4kg .. 4kg+3
  if (tid < Bp) bmax[tid] = 0ull;

  const int KS = D / 32;                           // k-steps per tile
  const int64_t ntiles = (rows + 15) / 16;
  int64_t rbase[T];
  const uint16_t* etile[T];   // this lane's 16 bytes in k-step 0 of its tile (rows past the end: the last tile)
#pragma unroll
  for (int j = 0; j < T; ++j) {
    rbase[j] = (int64_t)blockIdx.x * kDenseRowsPerBlock + (int64_t)(wave * T + j) * 16;
    const int64_t tile = min(rbase[j] / 16, ntiles - 1);
    etile[j] = Et + tile * KS * 512 + i16 * 32 + kg * 8;
  }
  floatx4 acc[T][NT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < D; k0 += KC) {
    const int kc = min(KC, D - k0);
    // Groups of U k-steps, two register buffers used ping-pong: the E loads of
    // the next group are in flight while the matrix cores work on this one.
    // Loads are unconditional and feed the matrix cores as loaded (k-steps past
    // the chunk re-read its last one and meet the zero columns of h; tiles past
    // the end re-read the last tile and are never stored), so nothing makes the
    // compiler wait on a load before its group is computed.
    auto load = [&](bf16x8 (&a)[U][T], int s) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = (k0 + min(s + 32 * u, kc - 32)) / 32;      // past the chunk: its last k-step
#pragma unroll
        for (int j = 0; j < T; ++j)
          a[u][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(etile[j] + (int64_t)ks * 512));
      }
    };
    auto compute = [&](const bf16x8 (&a)[U][T], int s) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = min(s + 32 * u, kc) + 8 * kg;   // past the chunk: the zero columns
        bf16x8 hv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) hv[t] = *reinterpret_cast<const bf16x8*>(hs + (16 * t + i16) * ldh + col);
#pragma unroll
        for (int j = 0; j < T; ++j)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv[t], a[u][j], acc[j][t], 0, 0, 0);
      }
    };
    bf16x8 b0[U][T], b1[U][T];
    load(b0, 0);   // in flight during the staging of this chunk of h
    // stage hb[:, k0 .. k0+kc) (bf16, zero rows past B) with 16-byte copies, then 32 zero
    // columns; eight copies per thread are loaded before any is stored (one round trip, not eight)
    __syncthreads();
    const int n8 = (kc >> 3) + 4;
    const int total = Bp * n8;
    for (int i0 = 0; i0 < total; i0 += 8 * kDenseThreads) {
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kDenseThreads + tid;
        const int b = i / n8;
        const int c = (i - b * n8) * 8;
        v[q] = u32x4{0u, 0u, 0u, 0u};
        if (i < total && c < kc) v[q] = *reinterpret_cast<const u32x4*>(hb + (size_t)b * D + k0 + c);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kDenseThreads + tid;
        const int b = i / n8;
        const int c = (i - b * n8) * 8;
        if (i < total) *reinterpret_cast<u32x4*>(hs + b * ldh + c) = v[q];
      }
    }
    __syncthreads();
    for (int s0 = 0; s0 < kc; s0 += 64 * U) {
      load(b1, s0 + 32 * U);
      compute(b0, s0);
      load(b0, s0 + 64 * U);
      if (s0 + 32 * U < kc) compute(b1, s0 + 32 * U);   // (uniform)
    }
  }

  // acc[j][t][e] = C[batch 16t + 4kg + e][row rbase[j] + i16]: softcap, store, and the
  // best key of each batch entry over this wave's rows (max over tiles in registers,
  // then over the 16 lanes of a k-group), one LDS atomic per batch entry and wave.
  const int64_t r_of = i16;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 16 * t + 4 * kg + e;
      uint64_t kb = 0ull;
      if (b < B) {
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const int64_t r = rbase[j] + r_of;
          if (r >= rows) continue;
          const float z = acc[j][t][e];
          const float v = softcap > 0.0f ? softcap * tanhf(z / softcap) : z;
          logits[(size_t)b * rows + r] = v;
          kb = max_u64(kb, select_key(v, (uint32_t)r));
        }
      }
      if (block_keys) {   // (uniform: a kernel argument)
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {   // within the 16 lanes of this k-group
          const uint32_t lo = __shfl_xor((unsigned)(uint32_t)kb, m, 64);
          const uint32_t hi = __shfl_xor((unsigned)(uint32_t)(kb >> 32), m, 64);
          kb = max_u64(kb, ((uint64_t)hi << 32) | lo);
        }
        if (i16 == 0 && b < B) atomicMax(&bmax[b], (unsigned long long)kb);
      }
    }
  }
  if (!block_keys) return;
  __syncthreads();
  if (tid < B) block_keys[(size_t)tid * gridDim.x + blockIdx.x] = bmax[tid];
}

template <int NT>
hipError_t launch_nt(const uint16_t* Et, int64_t rows, int D, const float* h, int B, float softcap, float* logits,
                     uint64_t* block_keys, uint16_t* hb, hipStream_t stream) {
  const int Bp = 16 * NT;
  const int Dp = (D + 31) / 32 * 32;
  const int64_t n = (int64_t)Bp * Dp;
  hipLaunchKernelGGL(dense_h_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h, B, D, Dp, Bp, hb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  D = Dp;   // the kernel works on the padded width
  const int KC = chunk_cols(D, NT);
  const size_t lds = (size_t)16 * NT * (KC + 40) * sizeof(uint16_t);
  auto kern = dense_logits_kernel<NT>;
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)dense_blocks(rows)), dim3(kDenseThreads), lds, stream, Et, rows, D,
                     (const uint16_t*)hb, B, KC, softcap, logits, block_keys);
  return hipGetLastError();
}

}  // namespace

size_t dense_tiled_bytes(int64_t rows, int D) {
  return (size_t)((rows + 15) / 16) * (size_t)((D + 31) / 32) * 1024;
}

hipError_t launch_pack_dense(const uint16_t* E, int64_t rows, int D, uint16_t* Et, hipStream_t stream) {
  const int KS = (D + 31) / 32;
  const int64_t n8 = (int64_t)dense_tiled_bytes(rows, D) / 16;
  hipLaunchKernelGGL(pack_dense_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, E, rows, D, KS, Et,
                     n8);
  return hipGetLastError();
}

// Column tiles of 16 vectors the kernel runs for B vectors.
static int dense_nt(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : (B <= 64 ? 4 : 8)); }
size_t dense_hb_bytes(int D, int B) { return (size_t)16 * dense_nt(B) * D * sizeof(uint16_t); }

hipError_t launch_dense_logits(const uint16_t* Et, int64_t rows, int D, const float* h, int B, float softcap,
                               float* logits, uint64_t* block_keys, uint16_t* hb, hipStream_t stream) {
  if (B <= 16) return launch_nt<1>(Et, rows, D, h, B, softcap, logits, block_keys, hb, stream);
  if (B <= 32) return launch_nt<2>(Et, rows, D, h, B, softcap, logits, block_keys, hb, stream);
  if (B <= 64) return launch_nt<4>(Et, rows, D, h, B, softcap, logits, block_keys, hb, stream);
  return launch_nt<8>(Et, rows, D, h, B, softcap, logits, block_keys, hb, stream);
}

}  // namespace rq
