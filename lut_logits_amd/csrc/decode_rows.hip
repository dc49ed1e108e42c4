// decode_rows.hip -- on-demand reconstruction of selected rows, and the
// one-time repacking of codes into the paired serving layout.
//
// Gemma-2-2B runtime-compression page, LUT-serving paragraph: the full
// embedding is never rebuilt; the rows of the input tokens are reconstructed
// on demand, a handful per prompt. Row r, element m*d + j, is the sum over
// the L levels of C[l][m][codes[r][l][m]][j].
//
// One workgroup per requested id. The level sum is taken in fp64 in level
// order and rounded once to fp32 (then to bf16, nearest-even, if asked), so
// the result does not depend on how many levels are summed. The work is a few
// hundred kilobytes per prompt: latency-bound by design.
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

template <typename CbT, typename OutT>
__global__ __launch_bounds__(kDecodeThreads) void decode_rows_kernel(CodeView cv, const CbT* __restrict__ cb,
                                                                     int64_t rows, int D, int M, int d, int K,
                                                                     int L, const int32_t* __restrict__ ids,
                                                                     OutT* __restrict__ out,
                                                                     int32_t* __restrict__ bad) {
  const int i = blockIdx.x;
  const int64_t id = ids[i];
  const bool ok = id >= 0 && id < rows;
  if (!ok && threadIdx.x == 0 && bad) atomicAdd(bad, 1);
  OutT* dst = out + (size_t)i * D;
  for (int e = threadIdx.x; e < D; e += kDecodeThreads) {
    double s = 0.0;
    if (ok) {
      const int m = e / d;
      const int j = e - m * d;
      for (int l = 0; l < L; ++l) {
        const int p = l * M + m;
        const uint32_t code = cv.codes[(int64_t)(p >> 1) * cv.s_blk + id * cv.s_row + (p & 1)];
        s += cb_value(cb + ((size_t)p * K + code) * d + j);
      }
    }
    out_store(dst + e, (float)s);
  }
}

// codes[r][p] (uint16, [rows][NP]) -> words[q][r] = codes[r][2q] | codes[r][2q+1] << 16.
// A 64-row x 64-word tile goes through LDS so both sides stay coalesced.
constexpr int kPackTile = 64;

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint16_t* __restrict__ src, int64_t rows, int NP,
                                                         uint32_t* __restrict__ dst) {
  __shared__ uint32_t tile[kPackTile][kPackTile + 1];
  const int NQ = (NP + 1) >> 1;
  const int64_t r0 = (int64_t)blockIdx.x * kPackTile;
  const int q0 = blockIdx.y * kPackTile;
  // read: each row's 128 consecutive codes (64 words), 4 rows per pass of 256 threads
  for (int t = threadIdx.x; t < kPackTile * kPackTile; t += 256) {
    const int rr = t / kPackTile;
    const int qq = t - rr * kPackTile;
    const int64_t r = r0 + rr;
    const int q = q0 + qq;
    uint32_t w = 0;
    if (r < rows && q < NQ) {
      const uint16_t* row = src + r * NP;
      const int p = 2 * q;
      w = row[p];
      if (p + 1 < NP) w |= (uint32_t)row[p + 1] << 16;
    }
    tile[rr][qq] = w;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kPackTile * kPackTile; t += 256) {
    const int qq = t / kPackTile;
    const int rr = t - qq * kPackTile;
    const int64_t r = r0 + rr;
    const int q = q0 + qq;
    if (r < rows && q < NQ) dst[(int64_t)q * rows + r] = tile[rr][qq];
  }
}

template <typename CbT, typename OutT>
hipError_t decode_typed(const rq_matrix* W, const int32_t* ids, int n, void* out, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL((decode_rows_kernel<CbT, OutT>), dim3((unsigned)n), dim3(kDecodeThreads), 0, stream,
                     code_view(W), static_cast<const CbT*>(W->codebooks), W->rows, W->D, W->M, W->d, W->K, W->L,
                     ids, static_cast<OutT*>(out), bad);
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
  const int NQ = (NP + 1) >> 1;
  dim3 grid((unsigned)((rows + kPackTile - 1) / kPackTile), (unsigned)((NQ + kPackTile - 1) / kPackTile));
  hipLaunchKernelGGL(pack_codes_kernel, grid, dim3(256), 0, stream, src, rows, NP, reinterpret_cast<uint32_t*>(dst));
  return hipGetLastError();
}

CodeView code_view(const rq_matrix* W) {
  CodeView v;
  v.codes = W->codes;
  if (W->codes_layout == RQ_CODES_PAIRED) {
    v.s_blk = 2 * W->rows;
    v.s_row = 2;
  } else {
    v.s_blk = 2;
    v.s_row = (int64_t)W->L * W->M;
  }
  return v;
}

}  // namespace rq
