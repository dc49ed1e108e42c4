// lut_build.hip -- the per-activation lookup table of an RQ-coded matrix.
//
//   LUT[l][m][k][b] = sum_{j<d} a[b][m*d + j] * C[l][m][k][j]
//
// (Gemma-2-2B runtime-compression page, LUT-serving paragraph: logits by
// lookup+sum; the table is the inner product of each subvector of the hidden
// state with every codeword of that subspace.)  a = x, or gelu_tanh(x) * x2
// for the down projection of a Gemma-2 MLP block (MLP RQ page, closing
// paragraphs).
//
// General kernel: one workgroup covers 256 codewords of one (level, subspace)
// pair p = l*M+m. It first stages a[b][m*d .. m*d+d) for all b in LDS
// (prologue applied once per workgroup), then each thread keeps its codeword
// in registers and writes B consecutive table entries. A single activation
// with d in {2, 6, 8} takes a vectorised path (build_lut_b1_kernel).
// Work: L*M*K*B*d FMAs; bytes: the codebooks once plus the table once -- a
// few microseconds at Gemma shapes, far from the matrix cores' territory, so
// plain VALU FMAs are used.
#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kBuildThreads = 256;
constexpr int kActStage = 4096;   // floats of the activation slice staged per workgroup
constexpr int kMaxRegD = 8;       // subspace widths up to this keep the codeword in registers

template <typename CbT>
__device__ __forceinline__ float cb_load(const CbT* p);
template <>
__device__ __forceinline__ float cb_load<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float cb_load<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename OutT>
__device__ __forceinline__ void lut_store(OutT* p, float v);
template <>
__device__ __forceinline__ void lut_store<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void lut_store<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float activation(const float* x, const float* x2, int gelu, size_t i) {
  const float v = x[i];
  return gelu ? gelu_tanh(v) * x2[i] : v;
}

// 16 bytes of table entries (8 bf16 or 4 fp32) from fp32 values, stored at once.
__device__ __forceinline__ void store16(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store16(uint16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename CbT, typename OutT>
__global__ __launch_bounds__(kBuildThreads) void build_lut_kernel(const CbT* __restrict__ cb,
                                                                  const float* __restrict__ x,
                                                                  const float* __restrict__ x2, int gelu, int B,
                                                                  int D, int M, int d, int K, int ktiles,
                                                                  OutT* __restrict__ lut) {
  __shared__ float act[kActStage];
  const int p = blockIdx.x / ktiles;                 // (level, subspace) pair
  const int m = p % M;
  const int k = (blockIdx.x - p * ktiles) * kBuildThreads + threadIdx.x;
  const bool staged = (int64_t)B * d <= kActStage;   // uniform over the workgroup
  const size_t col0 = (size_t)m * d;
  if (staged) {
    for (int i = threadIdx.x; i < B * d; i += kBuildThreads) {
      const int b = i / d;
      act[i] = activation(x, x2, gelu, (size_t)b * D + col0 + (i - b * d));
    }
    __syncthreads();
  }
  if (k >= K) return;
  const CbT* c = cb + ((size_t)p * K + k) * d;
  OutT* out = lut + ((size_t)p * K + k) * B;
  if (d <= kMaxRegD && staged) {
    float cw[kMaxRegD];
#pragma unroll
    for (int j = 0; j < kMaxRegD; ++j) cw[j] = (j < d) ? cb_load(c + j) : 0.0f;
    // B a multiple of VEC: a codeword's B entries are whole 16-byte units (the
    // table is 16-byte aligned), written one unit at a time
    constexpr int VEC = 16 / (int)sizeof(OutT);
    if (B % VEC == 0) {
      for (int b0 = 0; b0 < B; b0 += VEC) {
        float v[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float* a = act + (b0 + i) * d;
          float acc = 0.0f;
#pragma unroll
          for (int j = 0; j < kMaxRegD; ++j)
            if (j < d) acc = fmaf(a[j], cw[j], acc);
          v[i] = acc;
        }
        store16(out + b0, v);
      }
      return;
    }
    for (int b = 0; b < B; ++b) {
      const float* a = act + b * d;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxRegD; ++j)
        if (j < d) acc = fmaf(a[j], cw[j], acc);
      lut_store(out + b, acc);
    }
  } else {
    for (int b = 0; b < B; ++b) {
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) {
        const float a = staged ? act[b * d + j] : activation(x, x2, gelu, (size_t)b * D + col0 + j);
        acc = fmaf(a, cb_load(c + j), acc);
      }
      lut_store(out + b, acc);
    }
  }
}

// The same table for B a multiple of VEC (16 bytes of entries) with B / VEC
// dividing the workgroup: the B / VEC lanes of one codeword each own one
// 16-byte chunk of its B entries, so a wave's store covers whole consecutive
// codewords -- one contiguous 1 KB span -- instead of 16 bytes in each of 64
// lines (the per-codeword loop above, whose partial-line writes the memory
// system does not merge: 3.4x the table's bytes reached HBM at B=64). The
// workgroup's 256 codewords are first copied to LDS with 4-byte loads (one
// per lane per 1 KB, not d loads per lane per codeword), and each lane keeps
// its chunk's activation slices in registers; entries are computed in the
// same order as above, so the tables are bit-identical.
template <typename CbT, typename OutT>
__global__ __launch_bounds__(kBuildThreads) void build_lut_wide_kernel(const CbT* __restrict__ cb,
                                                                       const float* __restrict__ x,
                                                                       const float* __restrict__ x2, int gelu,
                                                                       int B, int D, int M, int d, int K, int ktiles,
                                                                       OutT* __restrict__ lut) {
  constexpr int VEC = 16 / (int)sizeof(OutT);
  __shared__ float act[kActStage];
  __shared__ uint32_t cws[kBuildThreads * kMaxRegD * sizeof(CbT) / 4];   // this tile's codewords
  const int p = blockIdx.x / ktiles;
  const int m = p % M;
  const int kt = blockIdx.x - p * ktiles;
  const size_t col0 = (size_t)m * d;
  for (int i = threadIdx.x; i < B * d; i += kBuildThreads) {
    const int b = i / d;
    act[i] = activation(x, x2, gelu, (size_t)b * D + col0 + (i - b * d));
  }
  // the tile's n codewords are n*d consecutive elements; the host guarantees
  // 4-byte alignment of their start and a whole number of words in every tile
  const int n = min(kBuildThreads, K - kt * kBuildThreads);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(cb + ((size_t)p * K + (size_t)kt * kBuildThreads) * d);
  const int words = n * d * (int)sizeof(CbT) / 4;
  for (int i = threadIdx.x; i < words; i += kBuildThreads) cws[i] = src[i];
  __syncthreads();
  const CbT* cwt = reinterpret_cast<const CbT*>(cws);
  const int cpc = B / VEC;                       // lanes per codeword
  const int bc = threadIdx.x % cpc;              // this lane's 16-byte chunk of the B entries
  const int per_iter = kBuildThreads / cpc;      // codewords per pass of the workgroup
  float a[VEC][kMaxRegD];
#pragma unroll
  for (int i = 0; i < VEC; ++i)
#pragma unroll
    for (int j = 0; j < kMaxRegD; ++j) a[i][j] = (j < d) ? act[(bc * VEC + i) * d + j] : 0.0f;
  for (int kk = threadIdx.x / cpc; kk < kBuildThreads; kk += per_iter) {
    const int k = kt * kBuildThreads + kk;
    if (k >= K) break;
    float cw[kMaxRegD];
#pragma unroll
    for (int j = 0; j < kMaxRegD; ++j) cw[j] = (j < d) ? cb_load(cwt + kk * d + j) : 0.0f;
    float v[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxRegD; ++j)
        if (j < d) acc = fmaf(a[i][j], cw[j], acc);
      v[i] = acc;
    }
    store16(lut + ((size_t)p * K + k) * B + bc * VEC, v);
  }
}

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// Fast path for one activation vector and a small compile-time subspace width:
// each thread reads CW consecutive codewords of one (level, subspace) pair with
// 16-byte loads (CW chosen so CW codewords fill whole 16-byte words) and writes
// their CW table entries. The activation slice is the same for every thread of
// the pair and comes from cache.
//
// gridDim.y == 2: a second matrix of the same shape (cb2, its table lut2) on
// the same activation, in the same launch (the MLP's gate and up).
template <typename CbT, typename OutT, int DS>
__global__ __launch_bounds__(kBuildThreads) void build_lut_b1_kernel(const CbT* __restrict__ cb1,
                                                                     const float* __restrict__ x,
                                                                     const float* __restrict__ x2, int gelu, int M,
                                                                     int K, int64_t total, OutT* __restrict__ lut1,
                                                                     const CbT* __restrict__ cb2,
                                                                     OutT* __restrict__ lut2) {
  const CbT* const cb = blockIdx.y ? cb2 : cb1;   // uniform
  OutT* const lut = blockIdx.y ? lut2 : lut1;
  constexpr int ES = (int)sizeof(CbT);
  constexpr int CW = 16 / gcd_int(16, DS * ES);
  constexpr int NV = CW * DS * ES / 16;
  const int64_t t = (int64_t)blockIdx.x * kBuildThreads + threadIdx.x;
  if (t >= total) return;
  const int per_pair = K / CW;
  const int p = (int)(t / per_pair);
  const int k0 = (int)(t - (int64_t)p * per_pair) * CW;
  const int m = p % M;
  const uint4* src = reinterpret_cast<const uint4*>(cb + ((size_t)p * K + k0) * DS);
  uint4 raw[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) raw[v] = src[v];
  float a[DS];
#pragma unroll
  for (int j = 0; j < DS; ++j) a[j] = activation(x, x2, gelu, (size_t)m * DS + j);
  const CbT* e = reinterpret_cast<const CbT*>(raw);
  OutT* out = lut + (size_t)p * K + k0;
#pragma unroll
  for (int w = 0; w < CW; ++w) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < DS; ++j) acc = fmaf(a[j], cb_load(e + w * DS + j), acc);
    lut_store(out + w, acc);
  }
}

// W2 (or null): a second matrix of W's shape whose table goes to lut2, in the same launch.
template <typename CbT, typename OutT, int DS>
bool try_b1(const rq_matrix* W, const float* x, const float* x2, int gelu, OutT* lut, hipStream_t stream,
            hipError_t* err, const rq_matrix* W2 = nullptr, OutT* lut2 = nullptr) {
  constexpr int ES = (int)sizeof(CbT);
  constexpr int CW = 16 / gcd_int(16, DS * ES);
  if (W->d != DS || W->K % CW != 0 || ((uintptr_t)W->codebooks & 15)) return false;
  if (W2 && ((uintptr_t)W2->codebooks & 15)) return false;
  const int64_t total = (int64_t)W->L * W->M * (W->K / CW);
  const CbT* cb = static_cast<const CbT*>(W->codebooks);
  hipLaunchKernelGGL((build_lut_b1_kernel<CbT, OutT, DS>),
                     dim3((unsigned)((total + kBuildThreads - 1) / kBuildThreads), W2 ? 2u : 1u), dim3(kBuildThreads),
                     0, stream, cb, x, x2, gelu, W->M, W->K, total, lut,
                     W2 ? static_cast<const CbT*>(W2->codebooks) : cb, W2 ? lut2 : lut);
  *err = hipGetLastError();
  return true;
}

template <typename CbT, typename OutT>
hipError_t launch_typed(const rq_matrix* W, const float* x, const float* x2, int gelu, int B, OutT* lut,
                        hipStream_t stream) {
  if (B == 1) {
    hipError_t e;
    if (try_b1<CbT, OutT, 6>(W, x, x2, gelu, lut, stream, &e)) return e;
    if (try_b1<CbT, OutT, 2>(W, x, x2, gelu, lut, stream, &e)) return e;
    if (try_b1<CbT, OutT, 8>(W, x, x2, gelu, lut, stream, &e)) return e;
  }
  const int NP = W->L * W->M;
  const int ktiles = (W->K + kBuildThreads - 1) / kBuildThreads;
  const int64_t blocks = (int64_t)NP * ktiles;
  constexpr int VEC = 16 / (int)sizeof(OutT);
  const int cpc = B / VEC;
  // whole 4-byte words per codeword tile: K*d*sizeof(CbT) and the last tile's
  // bytes multiples of 4 (a full tile of 256 codewords always is)
  const size_t es = sizeof(CbT);
  const bool words = ((uintptr_t)W->codebooks & 3) == 0 && ((size_t)W->K * W->d * es) % 4 == 0 &&
                     ((size_t)(W->K % kBuildThreads) * W->d * es) % 4 == 0;
  if (W->d <= kMaxRegD && (int64_t)B * W->d <= kActStage && B % VEC == 0 && cpc <= kBuildThreads &&
      kBuildThreads % cpc == 0 && ((uintptr_t)lut & 15) == 0 && words) {
    hipLaunchKernelGGL((build_lut_wide_kernel<CbT, OutT>), dim3((unsigned)blocks), dim3(kBuildThreads), 0, stream,
                       static_cast<const CbT*>(W->codebooks), x, x2, gelu, B, W->D, W->M, W->d, W->K, ktiles, lut);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((build_lut_kernel<CbT, OutT>), dim3((unsigned)blocks), dim3(kBuildThreads), 0, stream,
                     static_cast<const CbT*>(W->codebooks), x, x2, gelu, B, W->D, W->M, W->d, W->K, ktiles, lut);
  return hipGetLastError();
}

template <typename CbT>
bool try_b1_pair(const rq_matrix* W, const rq_matrix* W2, const float* x, float* lut, float* lut2, hipStream_t stream,
                 hipError_t* err) {
  return try_b1<CbT, float, 6>(W, x, nullptr, 0, lut, stream, err, W2, lut2) ||
         try_b1<CbT, float, 2>(W, x, nullptr, 0, lut, stream, err, W2, lut2) ||
         try_b1<CbT, float, 8>(W, x, nullptr, 0, lut, stream, err, W2, lut2);
}

}  // namespace

hipError_t launch_build_lut_pair(const rq_matrix* W, const rq_matrix* W2, const float* x, float* lut, float* lut2,
                                 hipStream_t stream) {
  const bool same = W->cb_dtype == W2->cb_dtype && W->L == W2->L && W->M == W2->M && W->K == W2->K &&
                    W->d == W2->d && W->D == W2->D;
  hipError_t e = hipSuccess;
  if (same && (W->cb_dtype == RQ_BF16 ? try_b1_pair<uint16_t>(W, W2, x, lut, lut2, stream, &e)
                                      : try_b1_pair<float>(W, W2, x, lut, lut2, stream, &e)))
    return e;
  e = launch_build_lut(W, x, nullptr, RQ_PRO_NONE, 1, 0, lut, stream);
  if (e == hipSuccess) e = launch_build_lut(W2, x, nullptr, RQ_PRO_NONE, 1, 0, lut2, stream);
  return e;
}

hipError_t launch_build_lut(const rq_matrix* W, const float* x, const float* x2, int prologue, int B,
                            int lut_bf16, void* lut, hipStream_t stream) {
  const int gelu = prologue == RQ_PRO_GELU_TANH_MUL;
  if (W->cb_dtype == RQ_BF16) {
    if (lut_bf16) return launch_typed<uint16_t, uint16_t>(W, x, x2, gelu, B, (uint16_t*)lut, stream);
    return launch_typed<uint16_t, float>(W, x, x2, gelu, B, (float*)lut, stream);
  }
  if (lut_bf16) return launch_typed<float, uint16_t>(W, x, x2, gelu, B, (uint16_t*)lut, stream);
  return launch_typed<float, float>(W, x, x2, gelu, B, (float*)lut, stream);
}

}  // namespace rq
