// lut_gather.hip -- lookup+sum over the code stream, the logits epilogue and
// the selection of argmax / top-k.
//
//   z[b][r] = sum_{l<L} sum_{m<M} LUT[l][m][codes[r][l][m]][b]
//
// (Gemma-2-2B runtime-compression page, LUT-serving paragraph: output logits
// by lookup+sum in place of a full matmul, then Gemma-2's own softcap.)
//
// Design for gfx950:
//  * The table of one activation is L*M*K entries (3 MiB in fp32 at Gemma
//    shapes), far larger than a CU's 160 KB of LDS. It is cut into chunks of
//    P (level, subspace) pairs; a workgroup stages one chunk in LDS with
//    coalesced 16-byte copies and then streams the codes of its row slab
//    against it. Pairs are split into G groups of chunks; every group writes
//    one partial sum per (row, batch), and the epilogue adds the G partials
//    in a fixed order, so results are bit-reproducible and no atomics touch
//    the sums.
//  * One lane owns one row (for 16-wide batch tiles, a quad of lanes owns one
//    row and each lane 4 batch entries, so a lookup is one contiguous 64-byte
//    LDS read per quad). Codes are read as 32-bit words holding two
//    consecutive pairs; in the paired layout the words of consecutive rows
//    are adjacent, so every wave-wide load is one contiguous run.
//  * Each lane issues the loads of all its row steps before touching LDS, so
//    up to NSTEP loads per lane are in flight to hide HBM latency.
//  * The workgroup -> (group, slab) mapping keeps all workgroups of one XCD on
//    the same group of chunks, so its L2 serves their table staging.
#include <math.h>

#include <algorithm>

#include "rq_internal.h"

namespace rq {
namespace {

struct GatherArgs {
  CodeView cv;
  const void* lut;      // [NP][K][B]
  int64_t rows;
  int NP, K, B;
  int P, chunks, cpg, G, steps, S, NBT;
  float* partial;       // [G][B][rows]
};

template <typename T, int N>
struct alignas(sizeof(T) * N) Vec {
  T v[N];
};

// Lookup of BQ consecutive batch entries of one table row, accumulated in fp32.
template <typename LutT, int BQ>
__device__ __forceinline__ void lookup_add(float* acc, const LutT* e);

template <>
__device__ __forceinline__ void lookup_add<float, 1>(float* acc, const float* e) { acc[0] += e[0]; }
template <>
__device__ __forceinline__ void lookup_add<float, 4>(float* acc, const float* e) {
  const float4 v = *reinterpret_cast<const float4*>(e);
  acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
}
template <>
__device__ __forceinline__ void lookup_add<uint16_t, 1>(float* acc, const uint16_t* e) { acc[0] += bf16_to_f32(e[0]); }
template <>
__device__ __forceinline__ void lookup_add<uint16_t, 4>(float* acc, const uint16_t* e) {
  const uint2 v = *reinterpret_cast<const uint2*>(e);
  acc[0] += bf16_to_f32(v.x & 0xffffu); acc[1] += bf16_to_f32(v.x >> 16);
  acc[2] += bf16_to_f32(v.y & 0xffffu); acc[3] += bf16_to_f32(v.y >> 16);
}

// Copy table rows [p0, p0+pc) x [0, K) x batch [b0, b0+BT) into LDS as [pc][K][BT]
// (entries beyond B are zero).
template <typename LutT, int BT>
__device__ __forceinline__ void stage_chunk(LutT* tab, const LutT* __restrict__ lut, int p0, int pc, int K, int B,
                                            int b0) {
  const int tid = threadIdx.x;
  const size_t n = (size_t)pc * K * BT;
  if (B == BT) {
    const LutT* src = lut + (size_t)p0 * K * B;
    const size_t nbytes = n * sizeof(LutT);
    if ((((size_t)K * B * sizeof(LutT)) & 15) == 0) {   // chunk starts 16-byte aligned
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(tab);
      const size_t n4 = nbytes / 16;
      size_t i = tid;
      for (; i + 3 * kGatherThreads < n4; i += 4 * kGatherThreads) {
        const uint4 a = s4[i], b = s4[i + kGatherThreads], c = s4[i + 2 * kGatherThreads],
                    d = s4[i + 3 * kGatherThreads];
        d4[i] = a; d4[i + kGatherThreads] = b; d4[i + 2 * kGatherThreads] = c; d4[i + 3 * kGatherThreads] = d;
      }
      for (; i < n4; i += kGatherThreads) d4[i] = s4[i];
      for (size_t e = n4 * 16 / sizeof(LutT) + tid; e < n; e += kGatherThreads) tab[e] = src[e];
    } else {
      for (size_t e = tid; e < n; e += kGatherThreads) tab[e] = src[e];
    }
  } else {
    for (size_t e = tid; e < n; e += kGatherThreads) {
      const int bb = (int)(e % BT);
      const size_t pk = e / BT;   // (pair - p0) * K + k
      const int b = b0 + bb;
      tab[e] = (b < B) ? lut[((size_t)p0 * K + pk) * B + b] : (LutT)0;
    }
  }
}

template <typename LutT, int BT, int NSTEP>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
  constexpr int QL = (BT >= 16) ? 4 : 1;   // lanes per row
  constexpr int BQ = BT / QL;              // batch entries per lane
  constexpr int RPS = kGatherThreads / QL; // rows per step
  extern __shared__ __align__(16) unsigned char smem[];
  LutT* tab = reinterpret_cast<LutT*>(smem);

  // XCD-aware numbering: consecutive workgroup ids land on different XCDs, so
  // give each XCD a contiguous range of logical ids (same chunk group).
  const int total = a.G * a.S * a.NBT;
  int li = blockIdx.x;
  if ((total & 7) == 0) li = (li & 7) * (total >> 3) + (li >> 3);
  const int bt = li % a.NBT;
  li /= a.NBT;
  const int s = li % a.S;
  const int g = li / a.S;

  const int tid = threadIdx.x;
  const int rq = tid % QL;
  const int rl = tid / QL;
  const int b0 = bt * BT;
  const int64_t row0 = (int64_t)s * a.steps * RPS + rl;

  float acc[NSTEP][BQ];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st)
#pragma unroll
    for (int i = 0; i < BQ; ++i) acc[st][i] = 0.0f;

  // Word offsets of this lane's rows (row r's word for block q is at q*s_blk + r*s_row).
  int64_t roff[NSTEP];
  bool live[NSTEP];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int64_t r = row0 + (int64_t)st * RPS;
    live[st] = (st < a.steps) && (r < a.rows);
    roff[st] = live[st] ? r * a.cv.s_row : 0;
  }

  const LutT* lut = static_cast<const LutT*>(a.lut);
  const int c_begin = g * a.cpg;
  const int c_end = min(a.chunks, c_begin + a.cpg);
  for (int c = c_begin; c < c_end; ++c) {
    const int p0 = c * a.P;
    const int pc = min(a.P, a.NP - p0);
    __syncthreads();
    stage_chunk<LutT, BT>(tab, lut, p0, pc, a.K, a.B, b0);
    __syncthreads();
    const int q0 = p0 >> 1;
    const int q1 = (p0 + pc + 1) >> 1;
    for (int q = q0; q < q1; ++q) {
      const uint16_t* blk = a.cv.codes + (int64_t)q * a.cv.s_blk;
      uint32_t w[NSTEP];
#pragma unroll
      for (int st = 0; st < NSTEP; ++st)
        w[st] = live[st] ? *reinterpret_cast<const uint32_t*>(blk + roff[st]) : 0u;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int pp = 2 * q + t - p0;        // pair index within the chunk (uniform)
        if (pp < 0 || pp >= pc) continue;
        const LutT* base = tab + (size_t)pp * a.K * BT + rq * BQ;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
          const uint32_t code = t ? (w[st] >> 16) : (w[st] & 0xffffu);
          lookup_add<LutT, BQ>(acc[st], base + (size_t)code * BT);
        }
      }
    }
  }

#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    if (!live[st]) continue;
    const int64_t r = row0 + (int64_t)st * RPS;
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int b = b0 + rq * BQ + i;
      if (b < a.B) a.partial[((size_t)g * a.B + b) * a.rows + r] = acc[st][i];
    }
  }
}

template <int BT>
constexpr int nstep_for() { return BT == 1 ? 8 : (BT == 4 ? 4 : 8); }

template <typename LutT, int BT>
hipError_t launch_gather_typed(const GatherArgs& a, const GatherPlan& plan, hipStream_t stream) {
  auto kern = gather_kernel<LutT, BT, nstep_for<BT>()>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.wgs()), dim3(kGatherThreads), plan.lds, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ epilogue

constexpr int kEpiThreads = 256;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = __shfl_xor((unsigned)(uint32_t)v, mask, 64);
  const uint32_t hi = __shfl_xor((unsigned)(uint32_t)(v >> 32), mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Sort s[0..n) descending (n a power of two) with all threads of the block.
__device__ void bitonic_sort_desc(uint64_t* s, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = s[i], y = s[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { s[i] = y; s[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
}

// z = sum of the G partials (fixed order), logits = softcap(z); per block of
// 1024 rows: the largest selection key and, with top-k, the block's k best keys.
__global__ __launch_bounds__(kEpiThreads) void epilogue_kernel(const float* __restrict__ partial, int G, int B,
                                                               int64_t rows, float softcap, float* __restrict__ out,
                                                               uint64_t* __restrict__ block_keys, int topk,
                                                               uint64_t* __restrict__ cand) {
  __shared__ uint64_t keys[kEpiRowsPerBlock];
  __shared__ uint64_t wmax[kEpiThreads / 64];
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int nblk = gridDim.x;
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < kEpiRowsPerBlock / kEpiThreads; ++i) {
    const int local = i * kEpiThreads + threadIdx.x;
    const int64_t r = (int64_t)blk * kEpiRowsPerBlock + local;
    uint64_t key = 0;
    if (r < rows) {
      float z = 0.0f;
      for (int g = 0; g < G; ++g) z += partial[((size_t)g * B + b) * rows + r];
      const float v = softcap > 0.0f ? softcap * tanhf(z / softcap) : z;
      if (out) out[(size_t)b * rows + r] = v;
      key = select_key(v, (uint32_t)r);
    }
    if (topk > 0) keys[local] = key;
    best = key > best ? key : best;
  }
  if (block_keys) {
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t m = wmax[0];
      for (int w = 1; w < kEpiThreads / 64; ++w) m = wmax[w] > m ? wmax[w] : m;
      block_keys[(size_t)b * nblk + blk] = m;
    }
  }
  if (topk > 0) {
    __syncthreads();
    bitonic_sort_desc(keys, kEpiRowsPerBlock);
    uint64_t* dst = cand + ((size_t)b * nblk + blk) * topk;
    for (int i = threadIdx.x; i < topk; i += kEpiThreads) dst[i] = keys[i];
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelCap = 4096;

// Per batch entry: argmax from the block maxima; top-k by merging the blocks'
// candidates through a 4096-key LDS buffer that always keeps the best k.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const uint64_t* __restrict__ block_keys, int nblk,
                                                             int32_t* __restrict__ argmax,
                                                             const uint64_t* __restrict__ cand, int topk,
                                                             int32_t* __restrict__ topk_ids,
                                                             float* __restrict__ topk_vals) {
  __shared__ uint64_t buf[kSelCap];
  __shared__ uint64_t wmax[kSelThreads / 64];
  const int b = blockIdx.x;
  if (argmax) {
    uint64_t best = 0;
    for (int i = threadIdx.x; i < nblk; i += kSelThreads) {
      const uint64_t k = block_keys[(size_t)b * nblk + i];
      best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t m = wmax[0];
      for (int w = 1; w < kSelThreads / 64; ++w) m = wmax[w] > m ? wmax[w] : m;
      argmax[b] = (int32_t)key_index(m);
    }
  }
  if (topk <= 0) return;
  const uint64_t* src = cand + (size_t)b * nblk * topk;
  const size_t total = (size_t)nblk * topk;
  const int room = kSelCap - topk;
  for (int i = threadIdx.x; i < topk; i += kSelThreads) buf[i] = 0;
  for (size_t start = 0; start < total; start += room) {
    for (int i = threadIdx.x; i < room; i += kSelThreads) {
      const size_t j = start + i;
      buf[topk + i] = j < total ? src[j] : 0;
    }
    __syncthreads();
    bitonic_sort_desc(buf, kSelCap);
  }
  for (int i = threadIdx.x; i < topk; i += kSelThreads) {
    topk_ids[(size_t)b * topk + i] = (int32_t)key_index(buf[i]);
    if (topk_vals) topk_vals[(size_t)b * topk + i] = key_value(buf[i]);
  }
}

// ------------------------------------------------------------------ planning

// Rough per-CU clock costs on gfx950 at 2.4 GHz, from measurements of this
// library's probes: HBM streams ~6.4 TB/s chip-wide, L2->LDS staging ~64 B/clk
// per CU, random 4-byte LDS lookups ~9 per clk per CU, quad-contiguous
// 64-byte lookups ~120 B/clk per CU.
double lookup_clk(int BT, int es) {
  if (BT == 1) return 1.0 / 9.0;
  if (BT == 4) return 4.0 * es / 60.0;
  return 16.0 * es / 120.0;
}

}  // namespace

GatherPlan plan_gather(const rq_matrix* W, int B, int lut_bf16) {
  const int NP = W->L * W->M;
  const int K = W->K;
  const int64_t rows = W->rows;
  const int es = lut_bf16 ? 2 : 4;
  const double hbm_bpc = 6.4e12 / 2.4e9;   // bytes per clock, whole chip
  GatherPlan best{};
  double best_cost = 1e300;
  const int bts[3] = {1, 4, 16};
  for (int bi = 0; bi < 3; ++bi) {
    const int BT = bts[bi];
    if ((B == 1) != (BT == 1)) continue;
    const size_t entry = (size_t)K * BT * es;
    if (entry > (size_t)kLdsBytes) continue;
    const int pmax = (int)std::min<int64_t>(NP, kLdsBytes / entry);
    const int QL = BT >= 16 ? 4 : 1;
    const int rps = kGatherThreads / QL;
    const int nstep = BT == 1 ? 8 : (BT == 4 ? 4 : 8);
    const int NBT = (B + BT - 1) / BT;
    for (int P = pmax; P >= 1 && P >= pmax / 2; --P) {
      if (P > 1 && P < NP && (P & 1)) continue;   // chunks start on a 2-pair word
      const int chunks = (NP + P - 1) / P;
      const size_t lds = (size_t)P * entry;
      const int per_cu = std::max(1, std::min(2, (int)(kLdsBytes / lds)));
      for (int steps = 1; steps <= nstep; ++steps) {
        const int64_t slab = (int64_t)steps * rps;
        const int64_t S = (rows + slab - 1) / slab;
        const int64_t slab_rows = std::min<int64_t>(rows, slab);
        int last_G = -1;
        for (int cpg = 1; cpg <= chunks; ++cpg) {
          const int G = (chunks + cpg - 1) / cpg;
          if (G == last_G) continue;
          last_G = G;
          const int64_t wgs = (int64_t)G * S * NBT;
          if (wgs > (int64_t)1 << 30) continue;
          const int64_t cap = (int64_t)kCUs * per_cu;
          const int64_t rounds = (wgs + cap - 1) / cap;
          const double t_stage = (double)cpg * lds / 64.0;
          const double t_look = (double)cpg * P * slab_rows * lookup_clk(BT, es);
          const double t_codes = (double)cpg * P * slab_rows * 2.0 / 32.0;
          // per_cu workgroups share one CU; a co-resident workgroup hides most of the staging
          const double t_round = std::max(t_look, t_codes) * per_cu;
          const double stage_exposed = per_cu == 1 ? t_stage : 0.3 * t_stage;
          const double hbm = ((double)rows * NP * 2.0 * NBT + (double)G * B * rows * 4.0 * 2.0) / hbm_bpc;
          const double cost = std::max(hbm, (double)rounds * t_round) + (double)rounds * stage_exposed;
          if (cost < best_cost * 0.999) {
            best_cost = cost;
            best.BT = BT; best.P = P; best.chunks = chunks; best.cpg = cpg; best.G = G;
            best.steps = steps; best.rps = rps; best.S = (int)S; best.NBT = NBT; best.lds = lds;
          }
        }
      }
    }
  }
  return best;
}

hipError_t launch_gather(const rq_matrix* W, const GatherPlan& plan, const void* lut, int lut_bf16, int B,
                         float* partial, uint64_t* /*zero_words*/, int /*n_zero_words*/, hipStream_t stream) {
  GatherArgs a;
  a.cv = code_view(W);
  a.lut = lut;
  a.rows = W->rows;
  a.NP = W->L * W->M;
  a.K = W->K;
  a.B = B;
  a.P = plan.P; a.chunks = plan.chunks; a.cpg = plan.cpg; a.G = plan.G;
  a.steps = plan.steps; a.S = plan.S; a.NBT = plan.NBT;
  a.partial = partial;
  if (lut_bf16) {
    if (plan.BT == 1) return launch_gather_typed<uint16_t, 1>(a, plan, stream);
    if (plan.BT == 4) return launch_gather_typed<uint16_t, 4>(a, plan, stream);
    return launch_gather_typed<uint16_t, 16>(a, plan, stream);
  }
  if (plan.BT == 1) return launch_gather_typed<float, 1>(a, plan, stream);
  if (plan.BT == 4) return launch_gather_typed<float, 4>(a, plan, stream);
  return launch_gather_typed<float, 16>(a, plan, stream);
}

hipError_t launch_epilogue(const float* partial, int G, int B, int64_t rows, float softcap, float* out,
                           uint64_t* block_keys, int topk, uint64_t* cand, hipStream_t stream) {
  dim3 grid((unsigned)epi_blocks(rows), (unsigned)B);
  hipLaunchKernelGGL(epilogue_kernel, grid, dim3(kEpiThreads), 0, stream, partial, G, B, rows, softcap, out,
                     block_keys, topk, cand);
  return hipGetLastError();
}

hipError_t launch_select(const uint64_t* block_keys, int nblk, int B, int32_t* argmax, const uint64_t* cand,
                         int topk, int32_t* topk_ids, float* topk_vals, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)B), dim3(kSelThreads), 0, stream, block_keys, nblk, argmax,
                     cand, topk, topk_ids, topk_vals);
  return hipGetLastError();
}

}  // namespace rq
