// decode_rows.hip -- on-demand reconstruction of selected rows, and the
// one-time repacking of codes into the serving layouts.
//
// Gemma-2-2B runtime-compression page, LUT-serving paragraph: the full
// embedding is never rebuilt; the rows of the input tokens are reconstructed
// on demand, a handful per prompt. Row r, element m*d + j, is the sum over
// the L levels of C[l][m][codes[r][l][m]][j].
//
// The level sum is taken in fp64 in level order and rounded once to fp32
// (then to bf16, nearest-even, if asked), so the result does not depend on how
// many levels are summed. The work is a few hundred kilobytes per prompt:
// latency-bound by design.
#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kDecodeThreads = 256;

template <typename CbT>
__device__ __forceinline__ double cb_value(const CbT* p);
template <>
__device__ __forceinline__ double cb_value<float>(const float* p) { return (double)*p; }
template <>
__device__ __forceinline__ double cb_value<uint16_t>(const uint16_t* p) { return (double)bf16_to_f32(*p); }

template <typename OutT>
__device__ __forceinline__ void out_store(OutT* p, float v);
template <>
__device__ __forceinline__ void out_store<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void out_store<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// One thread per output element (requested row i, subspace m, component j):
// it loads the row id, then the L codes of its subspace, then its L codebook
// entries, so a call is three dependent round trips whatever D is, and
// consecutive threads store consecutive elements.
template <typename CbT, typename OutT>
__global__ __launch_bounds__(kDecodeThreads) void decode_rows_kernel(CodeView cv, const CbT* __restrict__ cb,
                                                                     int64_t rows, int D, int M, int d, int K,
                                                                     int L, const int32_t* __restrict__ ids, int n,
                                                                     OutT* __restrict__ out,
                                                                     int32_t* __restrict__ bad) {
  const int64_t t = (int64_t)blockIdx.x * kDecodeThreads + threadIdx.x;
  if (t >= (int64_t)n * D) return;
  const int i = (int)(t / D);
  const int e = (int)(t - (int64_t)i * D);
  const int m = e / d;
  const int j = e - m * d;
  const int64_t id = ids[i];
  const bool ok = id >= 0 && id < rows;
  if (!ok) {
    if (e == 0 && bad) atomicAdd(bad, 1);
    out_store(out + t, 0.0f);
    return;
  }
  constexpr int kMaxL = RQ_MAX_L;
  uint32_t code[kMaxL];
  // A code >= K breaks the precondition; it is read as K-1 so that the
  // codebook load stays inside the caller's array.
#pragma unroll
  for (int l = 0; l < kMaxL; ++l)
    if (l < L) code[l] = min(code_at(cv, id, l * M + m), (uint32_t)(K - 1));
  double v[kMaxL];
#pragma unroll
  for (int l = 0; l < kMaxL; ++l)
    if (l < L) v[l] = cb_value(cb + ((size_t)(l * M + m) * K + code[l]) * d + j);
  double s = 0.0;
#pragma unroll
  for (int l = 0; l < kMaxL; ++l)
    if (l < L) s += v[l];
  out_store(out + t, (float)s);
}

// codes[r][p] (uint16, [rows][NP]) -> blocks[q][r] = codes[r][8q .. 8q+8) (16 bytes,
// zero past NP). A 64-row x 16-block tile goes through LDS so that the reads
// (256 contiguous bytes per row) and the writes (1 KB per block) stay coalesced.
constexpr int kPackRows = 64;
constexpr int kPackBlocks = 16;

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint16_t* __restrict__ src, int64_t rows, int NP,
                                                         uint4* __restrict__ dst) {
  __shared__ uint4 tile[kPackRows][kPackBlocks + 1];
  const int NQ = (NP + 7) >> 3;
  const int64_t r0 = (int64_t)blockIdx.x * kPackRows;
  const int q0 = blockIdx.y * kPackBlocks;
  for (int t = threadIdx.x; t < kPackRows * kPackBlocks; t += 256) {
    const int rr = t / kPackBlocks;
    const int qq = t - rr * kPackBlocks;
    const int64_t r = r0 + rr;
    const int q = q0 + qq;
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r < rows && q < NQ) {
      const uint16_t* row = src + r * NP + 8 * q;
      for (int i = 0; i < 8; ++i)
        if (8 * q + i < NP) c[i] = row[i];
    }
    tile[rr][qq] = make_uint4(c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16));
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kPackRows * kPackBlocks; t += 256) {
    const int qq = t / kPackRows;
    const int rr = t - qq * kPackRows;
    const int64_t r = r0 + rr;
    const int q = q0 + qq;
    if (r < rows && q < NQ) dst[(int64_t)q * rows + r] = tile[rr][qq];
  }
}

// codes[r][p] (uint16, [rows][NP]) -> RQ_CODES_PACKED10: thread (block q, row r)
// packs codes 12q .. 12q+11 of row r, three per 32-bit word (zero past NP);
// consecutive threads write consecutive rows' 16 bytes.
__global__ __launch_bounds__(256) void pack_codes10_kernel(const uint16_t* __restrict__ src, int64_t rows, int NP,
                                                           uint4* __restrict__ dst) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = blockIdx.y;
  if (r >= rows) return;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int t = 0; t < 12; ++t) {
    const int p = 12 * q + t;
    if (p < NP) w[t / 3] |= ((uint32_t)src[r * NP + p] & 0x3ffu) << (10 * (t % 3));
  }
  dst[(int64_t)q * rows + r] = make_uint4(w[0], w[1], w[2], w[3]);
}

// codes[r][p] (uint16, [rows][NP]) -> RQ_CODES_PACKED8: thread (block q, row r)
// packs codes 16q .. 16q+15 of row r, one byte each (zero past NP).
__global__ __launch_bounds__(256) void pack_codes8_kernel(const uint16_t* __restrict__ src, int64_t rows, int NP,
                                                          uint4* __restrict__ dst) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = blockIdx.y;
  if (r >= rows) return;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int t = 0; t < 16; ++t) {
    const int p = 16 * q + t;
    if (p < NP) w[t >> 2] |= ((uint32_t)src[r * NP + p] & 0xffu) << (8 * (t & 3));
  }
  dst[(int64_t)q * rows + r] = make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename CbT, typename OutT>
hipError_t decode_typed(const rq_matrix* W, const int32_t* ids, int n, void* out, int32_t* bad, hipStream_t stream) {
  const int64_t threads = (int64_t)n * W->D;
  const unsigned blocks = (unsigned)((threads + kDecodeThreads - 1) / kDecodeThreads);
  hipLaunchKernelGGL((decode_rows_kernel<CbT, OutT>), dim3(blocks), dim3(kDecodeThreads), 0, stream, code_view(W),
                     static_cast<const CbT*>(W->codebooks), W->rows, W->D, W->M, W->d, W->K, W->L, ids, n,
                     static_cast<OutT*>(out), bad);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_rows(const rq_matrix* W, const int32_t* ids, int n, int out_bf16, void* out,
                              int32_t* bad_ids, hipStream_t stream) {
  if (W->cb_dtype == RQ_BF16)
    return out_bf16 ? decode_typed<uint16_t, uint16_t>(W, ids, n, out, bad_ids, stream)
                    : decode_typed<uint16_t, float>(W, ids, n, out, bad_ids, stream);
  return out_bf16 ? decode_typed<float, uint16_t>(W, ids, n, out, bad_ids, stream)
                  : decode_typed<float, float>(W, ids, n, out, bad_ids, stream);
}

hipError_t launch_pack_codes(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream) {
  const int NQ = (NP + 7) >> 3;
  dim3 grid((unsigned)((rows + kPackRows - 1) / kPackRows), (unsigned)((NQ + kPackBlocks - 1) / kPackBlocks));
  hipLaunchKernelGGL(pack_codes_kernel, grid, dim3(256), 0, stream, src, rows, NP, reinterpret_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_codes10(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream) {
  const int NQ = (NP + 11) / 12;
  dim3 grid((unsigned)((rows + 255) / 256), (unsigned)NQ);
  hipLaunchKernelGGL(pack_codes10_kernel, grid, dim3(256), 0, stream, src, rows, NP, reinterpret_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_codes8(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream) {
  const int NQ = (NP + 15) / 16;
  dim3 grid((unsigned)((rows + 255) / 256), (unsigned)NQ);
  hipLaunchKernelGGL(pack_codes8_kernel, grid, dim3(256), 0, stream, src, rows, NP, reinterpret_cast<uint4*>(dst));
  return hipGetLastError();
}

CodeView code_view(const rq_matrix* W) {
  CodeView v;
  v.codes = W->codes;
  v.cbits = W->codes_layout == RQ_CODES_PACKED10 ? 10 : (W->codes_layout == RQ_CODES_PACKED8 ? 8 : 16);
  if (W->codes_layout != RQ_CODES_ROWS) {
    v.s_blk = 8 * W->rows;
    v.s_row = 8;
  } else {
    v.s_blk = 8;
    v.s_row = (int64_t)W->L * W->M;
  }
  return v;
}

}  // namespace rq
