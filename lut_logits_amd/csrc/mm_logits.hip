// mm_logits.hip -- head logits for a batch of hidden vectors on the matrix
// cores, reading the same RQ codes but never building a per-vector table.
//
// What is computed is the runtime-compression page's lookup+sum (LUT-serving
// paragraph) in its other association: instead of LUT[l][m][k][b] =
// <h_b on subspace m, C[l][m][k]> followed by a sum of looked-up entries,
//     z[b][r] = sum_{l,m} < C[l][m][code[r][l][m]], h_b on subspace m >,
// which is the same number in exact arithmetic (distributivity). For B >= 16
// the table is B times larger than the codebook it comes from, and staging it
// through LDS dominates; the codebook costs 16 bytes per codeword whatever B
// is, and the B-fold work becomes a dense contraction for the matrix cores.
//
// Exactness. Codebooks are bf16 (exact MFMA operands). Each fp32 hidden value
// is split into three bf16 parts, x = p0 + p1 + p2 exactly (each part is the
// RNE of what the previous ones left; 3 x 8 significant bits cover fp32's 24).
// Every bf16 x bf16 product is exact in fp32 and the matrix cores accumulate in
// fp32, so the result carries fp32 accumulation error only, as the table path
// does.
//
// Mapping onto v_mfma_f32_16x16x32_bf16 (A: 16 rows x 32 k, B: 32 k x 16
// columns, C: 16 x 16 fp32):
//   - A rows are 16 vocab rows; the 32 k split into four slots of 8, one
//     subspace each (d <= 8 values, zero-padded).
//   - B columns are 16 hidden vectors; B's slot kg holds the same subspace's
//     slice of one part of h.
//   - Lane (i = lane % 16, kg = lane / 16) feeds A row i, slot kg, and receives
//     C rows 4*kg .. 4*kg+3 of column i.
// The serving code layouts give each row 16 bytes per block of pairs: 8 pairs
// of 16-bit codes (dword kg holds pairs 2kg and 2kg+1) or 12 pairs of 10-bit
// codes (dword kg holds pairs 3kg .. 3kg+2). So a lane loads exactly one dword
// per row tile and block (a wave reads 16 rows x 16 contiguous bytes, no byte
// twice) and the block is done as NSUB = 2 or 3 "sub-blocks": sub-block s uses
// pairs {PPB*q + NSUB*kg + s : kg < 4}, the s-th code field of each dword.
//
// Work split: workgroup (group g, slab s, batch tile bt) accumulates 16*NT
// hidden vectors over slab s's rows (8 waves x T tiles x 16 rows) for group
// g's code blocks. Half-blocks stream through a two-slot LDS ring: 4 pairs x K
// codewords (16 B each, padded) plus the three parts of h for those pairs; the
// next half's codebook sits in registers while the current one is in use.
// Partial sums go to [G][B][rows] and the finish kernel adds them in group
// order, applies the softcap and emits the selection keys.
#include "rq_internal.h"

namespace rq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMmThreads = 512;   // one workgroup per CU (LDS); 512: 2 waves per SIMD, 256 VGPRs each
constexpr int kMmWaves = kMmThreads / 64;
constexpr int kParts = 3;           // bf16 parts of each hidden value
constexpr int kMaxCwPerThread = 4 * kMmMaxK / kMmThreads;   // codewords of a half-block per thread
// One pair per ring slot (K above kMmMaxK, 16-bit blocked codes): a slot holds
// the K codewords of one (level, subspace) pair (64 KB at K = 4096) and the
// MFMA's four k-slots carry that pair's codeword against h's three bf16 parts
// and a zero: one MFMA per 16 rows x 16 vectors x pair, the three-part split
// folded into the contraction.
constexpr int kMmMaxKOnePair = 4 * kMmMaxK;

struct MmArgs {
  const uint16_t* cb;     // bf16 codebooks [NP][K][d]
  const uint16_t* codes;  // RQ_CODES_BLOCKED
  const u32x4* hp;        // [kParts][M][Bp] 8-bf16 vectors (zero past d and past B)
  float* partial;         // [G][B][rows] (G > 1)
  float* out;             // G == 1: logits [B][rows] after the softcap, or null
  float softcap;          // G == 1: <= 0 for none
  uint64_t* block_keys;   // G == 1: [B][S] best selection key per slab, or null
  int64_t rows;
  int K, M, NP, NQ, B, Bp, G, qpg, S;
};

// hp[part][m][n] = part `part` of h[n][m*d .. m*d+d), padded to 8 with zeros.
__global__ void split_h_kernel(const float* __restrict__ h, int B, int D, int M, int d, int Bp,
                               u32x4* __restrict__ hp) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M * Bp) return;
  const int m = t / Bp;
  const int n = t - m * Bp;
  uint32_t w[kParts][4];
#pragma unroll
  for (int pr = 0; pr < kParts; ++pr)
#pragma unroll
    for (int q = 0; q < 4; ++q) w[pr][q] = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x = (n < B && j < d) ? h[(size_t)n * D + (size_t)m * d + j] : 0.0f;
#pragma unroll
    for (int pr = 0; pr < kParts; ++pr) {
      const uint16_t b = f32_to_bf16(x);
      x -= bf16_to_f32(b);   // exact: the rounding error of an fp32 -> bf16 RNE fits fp32
      w[pr][j >> 1] |= (uint32_t)b << (16 * (j & 1));
    }
  }
#pragma unroll
  for (int pr = 0; pr < kParts; ++pr) {
    u32x4 v = {w[pr][0], w[pr][1], w[pr][2], w[pr][3]};
    hp[((size_t)pr * M + m) * Bp + n] = v;
  }
}

template <int DS, int NT, bool ONEPAIR = false>
struct Staged {
  // h vectors per thread: three parts x four slots, or (one pair) four slots
  static constexpr int kH = ((ONEPAIR ? 4 : kParts * 4) * 16 * NT + kMmThreads - 1) / kMmThreads;
  uint32_t cw[kMaxCwPerThread][DS / 2];
  u32x4 hv[kH];
};

// NSUB sub-blocks per code block: 2 for 16-bit codes (pairs 2kg, 2kg+1 in
// dword kg), 3 for RQ_CODES_PACKED10 (pairs 3kg .. 3kg+2, 10 bits each).
// ONEPAIR (16-bit codes only): a code block's 8 pairs are 8 sub-blocks of one
// pair each (see kMmMaxKOnePair).
template <int DS, int NT, int T, int NSUB, bool ONEPAIR = false>
__global__ __launch_bounds__(kMmThreads) void mm_logits_kernel(MmArgs a) {
  static_assert(!ONEPAIR || NSUB == 2, "one pair per slot: 16-bit codes");
  constexpr int PPB = 4 * NSUB;                 // pairs per code block
  constexpr int SB = ONEPAIR ? PPB : NSUB;      // sub-blocks (ring slots) per code block
  constexpr int SP = ONEPAIR ? 1 : 4;           // pairs per slot
  constexpr int CBITS = NSUB == 2 ? 16 : 10;    // bits per code
  constexpr uint32_t CMASK = (1u << CBITS) - 1u;
  extern __shared__ __align__(16) u32x4 ring[];   // [2][SP*K + h entries]
  const int K = a.K;
  const int cw_entries = SP * K;
  const int h_entries = (ONEPAIR ? 4 : kParts * 4) * 16 * NT;
  const int slot_entries = cw_entries + h_entries;

  // workgroup -> (batch tile, group, slab). Workgroups are dealt to the 8 XCDs
  // round robin (dispatch index mod 8); with g = index mod G and G dividing 8,
  // every workgroup of an XCD works on the same group(s) of code blocks, so
  // their codebooks stay in that XCD's L2.
  const int per_bt = a.G * a.S;
  const int bt = blockIdx.x / per_bt;
  const int li = blockIdx.x - bt * per_bt;
  const int g = li % a.G;
  const int s = li / a.G;
  const int q0 = g * a.qpg;
  const int q1 = min(a.NQ, q0 + a.qpg);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)s * (kMmWaves * T * 16) + (int64_t)wave * (T * 16);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)0xffffffffu,
                                                                        0x00020000);
  const uint32_t blk_bytes = (uint32_t)a.rows * 16u;
  // Code loads. Every vector-memory instruction costs the CU's load pipe about
  // the same whatever its width, so with T a multiple of 4 a lane loads whole
  // 16-byte rows: load v gives lane (i16, kg) row i16 of tile 4v + kg, and a
  // 4 x 4 transpose across the wave's four 16-lane rows (two 32-lane and two
  // 16-lane swaps) leaves dword kg of tile 4v + t's row i16 in codes[4v + t],
  // as a one-dword load per tile would. A quarter of the instructions.
  constexpr bool kWide = T % 4 == 0;
  constexpr int NV = kWide ? T / 4 : T;
  uint32_t voff[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t r = min(tile0 + 16 * (kWide ? 4 * v + kg : v) + i16, a.rows - 1);
    voff[v] = (uint32_t)r * 16u + (kWide ? 0u : (uint32_t)kg * 4u);
  }
  auto load_codes = [&](uint32_t (&dst)[T], int q) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (kWide) {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, voff[v], (uint32_t)q * blk_bytes, 0));
        dst[4 * v + 0] = w[0]; dst[4 * v + 1] = w[1]; dst[4 * v + 2] = w[2]; dst[4 * v + 3] = w[3];
      } else {
        dst[v] = __builtin_amdgcn_raw_buffer_load_b32(crs, voff[v], (uint32_t)q * blk_bytes, 0);
      }
    }
  };
  // After a wide load: row-of-lanes k holds tile 4v + k's row; give every row
  // of lanes its own dword of each tile instead.
  auto arrange_codes = [&](uint32_t (&c)[T]) {
    if constexpr (kWide) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const auto x02 = __builtin_amdgcn_permlane32_swap(c[4 * v + 0], c[4 * v + 2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(c[4 * v + 1], c[4 * v + 3], false, false);
        const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
        const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
        c[4 * v + 0] = y01[0]; c[4 * v + 1] = y01[1]; c[4 * v + 2] = y23[0]; c[4 * v + 3] = y23[1];
      }
    }
  };

  // ---- staging of one half-block into registers, then into a ring slot
  const int n_bt = 16 * NT;
  // Thread tid stages codeword entries (tid + u*kMmThreads) mod cw_entries and
  // h entries (tid + u*kMmThreads) mod h_entries: indices wrap instead of being
  // guarded, so some entries are written twice with the same value and no
  // branch (whose join would make the compiler wait for every load in flight)
  // is needed.
  // Pair held by slot position kk (0 .. SP-1) of sub-block hs of block q.
  auto slot_pair = [&](int q, int kk, int hs) { return ONEPAIR ? PPB * q + hs : PPB * q + NSUB * kk + hs; };
  auto stage_load = [&](Staged<DS, NT, ONEPAIR>& st, int q, int hs) {
#pragma unroll
    for (int u = 0; u < kMaxCwPerThread; ++u) {
      const int c = (tid + u * kMmThreads) % cw_entries;
      const int kk = c / K;
      const int k = c - kk * K;
      const int p = min(slot_pair(q, kk, hs), a.NP - 1);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.cb + ((size_t)p * K + k) * DS);
#pragma unroll
      for (int w = 0; w < DS / 2; ++w) st.cw[u][w] = src[w];
    }
#pragma unroll
    for (int u = 0; u < Staged<DS, NT, ONEPAIR>::kH; ++u) {
      const int e = (tid + u * kMmThreads) % h_entries;
      // ONEPAIR: entry (slot kg, vector n) is part kg of the pair's slice of h (kg < 3), the
      // fourth slot is zero; else entry (part, slot kk, vector n)
      const int pr = ONEPAIR ? min(e / n_bt, kParts - 1) : e / (4 * n_bt);
      const int rem = ONEPAIR ? e % n_bt : e - pr * 4 * n_bt;
      const int kk = ONEPAIR ? 0 : rem / n_bt;
      const int n = ONEPAIR ? rem : rem - kk * n_bt;
      const int p = min(slot_pair(q, kk, hs), a.NP - 1);
      const int m = p % a.M;
      st.hv[u] = a.hp[((size_t)pr * a.M + m) * a.Bp + (size_t)bt * n_bt + n];
    }
  };
  auto stage_store = [&](const Staged<DS, NT, ONEPAIR>& st, int slot, int q, int hs) {
    u32x4* base = ring + slot * slot_entries;
#pragma unroll
    for (int u = 0; u < kMaxCwPerThread; ++u) {
      const int c = (tid + u * kMmThreads) % cw_entries;
      const bool live = slot_pair(q, c / K, hs) < a.NP;
      u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < DS / 2; ++w) v[w] = live ? st.cw[u][w] : 0u;
      base[c] = v;
    }
#pragma unroll
    for (int u = 0; u < Staged<DS, NT, ONEPAIR>::kH; ++u) {
      const int e = (tid + u * kMmThreads) % h_entries;
      const int pr = e / (4 * n_bt);
      const int kk = ONEPAIR ? 0 : (e - pr * 4 * n_bt) / n_bt;
      const bool live = slot_pair(q, kk, hs) < a.NP && (!ONEPAIR || e < kParts * n_bt);
      const u32x4 z = {0u, 0u, 0u, 0u};
      base[cw_entries + e] = live ? st.hv[u] : z;
    }
  };

  floatx4 acc[T][NT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot, const uint32_t (&codes)[T], int hs) {
    const u32x4* base = ring + slot * slot_entries;
    if constexpr (ONEPAIR) {
      // B: slot kg of vector 16t + i16 is part kg of h (zero for kg = 3); A: every
      // k-slot holds the row's codeword of this pair, read by all four lanes of a
      // row (one address). The pair's code is in dword hs/2 of the row's block,
      // which the arranged codes give to the lanes of row-of-lanes hs/2.
      bf16x8 hb1[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) hb1[t] = __builtin_bit_cast(bf16x8, base[cw_entries + kg * n_bt + 16 * t + i16]);
      const int src_lane = i16 + 16 * (hs >> 1);
      const int shift = 16 * (hs & 1);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const uint32_t dw = (uint32_t)__shfl((int)codes[j], src_lane, 64);
        const bf16x8 av1 = __builtin_bit_cast(bf16x8, base[(dw >> shift) & 0xffffu]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av1, hb1[t], acc[j][t], 0, 0, 0);
      }
      return;
    }
    bf16x8 hb[kParts][NT];
#pragma unroll
    for (int pr = 0; pr < kParts; ++pr)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        hb[pr][t] = __builtin_bit_cast(bf16x8, base[cw_entries + (pr * 4 + kg) * n_bt + 16 * t + i16]);
    const u32x4* cwb = base + kg * K;
    // Software pipeline: the codewords of the next kI tiles are read from LDS
    // while the matrix cores work on the current kI tiles.
    constexpr int kI = 4;
    constexpr int kGroups = (T + kI - 1) / kI;
    bf16x8 av[2][kI];
#pragma unroll
    for (int u = 0; u < kI; ++u)
      av[0][u] = __builtin_bit_cast(bf16x8, cwb[(codes[min(u, T - 1)] >> (CBITS * hs)) & CMASK]);
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const int cur = gi & 1;
      if (gi + 1 < kGroups) {
#pragma unroll
        for (int u = 0; u < kI; ++u) {
          const int j = min((gi + 1) * kI + u, T - 1);
          av[cur ^ 1][u] = __builtin_bit_cast(bf16x8, cwb[(codes[j] >> (CBITS * hs)) & CMASK]);
        }
      }
#pragma unroll
      for (int pr = 0; pr < kParts; ++pr)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int u = 0; u < kI; ++u) {
            const int j = gi * kI + u;
            if (j < T) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cur][u], hb[pr][t], acc[j][t], 0, 0, 0);
          }
    }
  };

  if (q0 < q1) {
    uint32_t ca[T], cbk[T];
    Staged<DS, NT, ONEPAIR> st;
    load_codes(ca, q0);
    stage_load(st, q0, 0);
    int slot = 0;
    // One code block: its NSUB sub-blocks in turn, each staged in one ring slot
    // while the next one's codebook loads into registers; the first sub-block
    // also starts loading the next block's codes (into the other buffer).
    auto do_block = [&](int q, uint32_t (&cur)[T], uint32_t (&nxt)[T]) {
      arrange_codes(cur);
#pragma unroll
      for (int hs = 0; hs < SB; ++hs) {
        stage_store(st, slot, q, hs);
        __syncthreads();
        if (hs + 1 < SB) stage_load(st, q, hs + 1);
        else stage_load(st, min(q + 1, q1 - 1), 0);
        if (hs == 0) {
          __builtin_amdgcn_sched_barrier(0);   // keep the staging loads ahead of the code loads (vmcnt is in order)
          load_codes(nxt, min(q + 1, q1 - 1));
        }
        // Left alone, the scheduler sinks the code loads to the end of a long
        // compute and hoists the next sub-block's LDS stores (with their waits
        // on the loads just issued) into it, so both loads get a fraction of a
        // compute phase to land. With many tiles the compute is fenced on both
        // sides (B=16 head: 266 -> 253 us per call); a short one (few tiles)
        // gains from the overlap and is left to the scheduler.
        if constexpr (T >= 8) __builtin_amdgcn_sched_barrier(0);
        compute(slot, cur, hs);
        if constexpr (T >= 8) __builtin_amdgcn_sched_barrier(0);
        slot ^= 1;
      }
    };
    for (int q = q0; q < q1; q += 2) {
      do_block(q, ca, cbk);
      if (q + 1 < q1) do_block(q + 1, cbk, ca);
    }
  }

  // acc[j][t][e] = z[batch bt*16NT + 16t + i16][row tile0 + 16j + 4kg + e]
  if (a.G > 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int b = bt * n_bt + 16 * t + i16;
      if (b >= a.B) continue;
      float* dst = a.partial + ((size_t)g * a.B + b) * a.rows;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const int64_t r = tile0 + 16 * j + 4 * kg;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r + e < a.rows) dst[r + e] = acc[j][t][e];
      }
    }
    return;
  }
  // G == 1: the sums are final -- softcap, store, best selection key of this
  // slab for each hidden vector (the selection kernel reduces the S keys).
  __shared__ unsigned long long s_keys[16 * NT];
  if (tid < 16 * NT) s_keys[tid] = 0ull;
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int b = bt * n_bt + 16 * t + i16;
    unsigned long long kbest = 0ull;
    if (b < a.B) {
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const int64_t r = tile0 + 16 * j + 4 * kg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (r + e >= a.rows) continue;
          const float z = acc[j][t][e];
          const float v = a.softcap > 0.0f ? a.softcap * tanhf(z / a.softcap) : z;
          if (a.out) a.out[(size_t)b * a.rows + r + e] = v;
          const unsigned long long k = select_key(v, (uint32_t)(r + e));
          kbest = k > kbest ? k : kbest;
        }
      }
    }
    if (kbest) atomicMax(&s_keys[16 * t + i16], kbest);   // LDS atomics, this workgroup only
  }
  __syncthreads();
  if (a.block_keys && tid < 16 * NT) {
    const int b = bt * n_bt + tid;
    if (b < a.B) a.block_keys[(size_t)b * a.S + s] = s_keys[tid];
  }
}

// Row tiles per wave for NT column tiles: the accumulators (4*T*NT VGPRs), the
// code registers (2*T) and the staged half-block share a wave's 256 VGPRs.
// (Three sub-blocks per code block keep more values live: fewer tiles.) A
// multiple of 4 takes the wide code loads; 4 at NT = 4 uses 254 VGPRs.
// One pair per slot keeps a third of the h registers, so four column tiles take
// 8 row tiles (1,024 rows per staged slot and workgroup); codewords of 6 values
// take 6 and of 8 values 4 (their staging needs more registers; 8 spilled).
constexpr int tiles_for(int NT, int NSUB = 2, bool ONEPAIR = false, int DS = 2) {
  return ONEPAIR ? (NT == 1 ? 16 : (NT == 4 && DS >= 6 ? (DS == 8 ? 4 : 6) : 8))
                 : (NSUB == 2 ? (NT == 1 ? 16 : NT == 2 ? 8 : 4) : (NT == 1 ? 12 : NT == 2 ? 6 : 3));
}

template <int DS, int NT, int NSUB, bool ONEPAIR = false>
hipError_t launch_typed(const MmArgs& a, int wgs, size_t lds, hipStream_t stream) {
  auto kern = mm_logits_kernel<DS, NT, tiles_for(NT, NSUB, ONEPAIR, DS), NSUB, ONEPAIR>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kMmThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DS, int NSUB, bool ONEPAIR = false>
hipError_t launch_ds(const MmArgs& a, const MmPlan& p, hipStream_t stream) {
  const int wgs = p.G * p.S * p.NBT;
  if (p.NT == 1) return launch_typed<DS, 1, NSUB, ONEPAIR>(a, wgs, p.lds, stream);
  if (p.NT == 2) return launch_typed<DS, 2, NSUB, ONEPAIR>(a, wgs, p.lds, stream);
  return launch_typed<DS, 4, NSUB, ONEPAIR>(a, wgs, p.lds, stream);
}

template <int NSUB, bool ONEPAIR = false>
hipError_t launch_nsub(const MmArgs& a, const MmPlan& p, int d, hipStream_t stream) {
  switch (d) {
    case 2: return launch_ds<2, NSUB, ONEPAIR>(a, p, stream);
    case 4: return launch_ds<4, NSUB, ONEPAIR>(a, p, stream);
    case 6: return launch_ds<6, NSUB, ONEPAIR>(a, p, stream);
    default: return launch_ds<8, NSUB, ONEPAIR>(a, p, stream);
  }
}

}  // namespace

// One pair per ring slot for K beyond what four pairs per slot can stage.
static bool mm_one_pair(const rq_matrix* W) { return W->K > kMmMaxK; }

bool mm_supported(const rq_matrix* W) {
  if (W->cb_dtype != RQ_BF16 || W->d > 8 || (W->d % 2) != 0 || ((uintptr_t)W->codebooks % 4) != 0) return false;
  if (W->K <= kMmMaxK) return W->codes_layout == RQ_CODES_BLOCKED || W->codes_layout == RQ_CODES_PACKED10;
  return W->K <= kMmMaxKOnePair && W->codes_layout == RQ_CODES_BLOCKED;
}

MmPlan plan_mm(const rq_matrix* W, int B) {
  MmPlan p{};
  p.NT = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
  p.T = tiles_for(p.NT, W->codes_layout == RQ_CODES_PACKED10 ? 3 : 2, mm_one_pair(W), W->d);
  p.NBT = (B + 16 * p.NT - 1) / (16 * p.NT);
  p.Bp = p.NBT * 16 * p.NT;
  const int64_t slab = (int64_t)kMmWaves * p.T * 16;
  p.S = (int)((W->rows + slab - 1) / slab);
  p.NQ = (W->L * W->M + pairs_per_block(W) - 1) / pairs_per_block(W);
  // Group count: workgroups run in rounds of one per CU; a round costs the
  // blocks one workgroup handles (about 3.9 us per block for 8 waves of 16
  // 16x16 tiles, fitted to this kernel at the Gemma head), and G > 1 adds the
  // finish pass: G partial sums read and the logits written (~2.2 TB/s, plus a
  // launch). With G == 1 the kernel writes the logits itself.
  int G = 1;
  double best = 1e30;
  for (int g = 1; g <= std::min(p.NQ, 64); g *= 2) {   // powers of two: g = index mod G keeps XCDs on their groups
    const int qpg = (p.NQ + g - 1) / g;
    const int gg = (p.NQ + qpg - 1) / qpg;
    const int64_t wgs = (int64_t)gg * p.S * p.NBT;
    const double rounds = (double)((wgs + kCUs - 1) / kCUs);
    // one pair per slot: four times the slots per block, each a third of the MFMAs
    const double per_block = 3.9 * (double)(p.T * p.NT) / 16.0 * (double)pairs_per_block(W) / 8.0 *
                             (mm_one_pair(W) ? 4.0 / 3.0 : 1.0);
    const double cost = rounds * qpg * per_block + (gg > 1 ? 5.0 + (double)(gg + 1) * B * W->rows * 4.0 / 2.2e6 : 0.0);
    if (cost < best * 0.999) { best = cost; G = gg; }
  }
  p.qpg = (p.NQ + G - 1) / G;
  p.G = (p.NQ + p.qpg - 1) / p.qpg;
  p.lds = mm_one_pair(W) ? (size_t)2 * ((size_t)W->K + (size_t)4 * 16 * p.NT) * 16
                         : (size_t)2 * (4 * (size_t)W->K + (size_t)kParts * 4 * 16 * p.NT) * 16;
  return p;
}

size_t mm_hp_bytes(const rq_matrix* W, const MmPlan& p) { return (size_t)kParts * W->M * p.Bp * 16; }

hipError_t launch_mm_logits(const rq_matrix* W, const MmPlan& p, const float* h, int B, void* hp, float* partial,
                            float* out, float softcap, uint64_t* block_keys, hipStream_t stream) {
  const int n = W->M * p.Bp;
  hipLaunchKernelGGL(split_h_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, h, B, W->D, W->M, W->d,
                     p.Bp, static_cast<u32x4*>(hp));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MmArgs a;
  a.cb = static_cast<const uint16_t*>(W->codebooks);
  a.codes = W->codes;
  a.hp = static_cast<const u32x4*>(hp);
  a.partial = partial;
  a.out = out;
  a.softcap = softcap;
  a.block_keys = block_keys;
  a.rows = W->rows;
  a.K = W->K;
  a.M = W->M;
  a.NP = W->L * W->M;
  a.NQ = p.NQ;
  a.B = B;
  a.Bp = p.Bp;
  a.G = p.G;
  a.qpg = p.qpg;
  a.S = p.S;
  hipEvent_t before, after;
  take_stage_events(&before, &after);
  if (before && (e = hipEventRecord(before, stream)) != hipSuccess) return e;
  e = mm_one_pair(W)                            ? launch_nsub<2, true>(a, p, W->d, stream)
      : W->codes_layout == RQ_CODES_PACKED10 ? launch_nsub<3>(a, p, W->d, stream)
                                             : launch_nsub<2>(a, p, W->d, stream);
  if (e != hipSuccess) return e;
  if (after) e = hipEventRecord(after, stream);
  return e;
}

}  // namespace rq
