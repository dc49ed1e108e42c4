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
  uint32_t cb_bytes, hp_bytes;   // byte ranges of cb and hp (the one-pair kernels' buffer loads; < 2^32)
  const u32x4* cbp;       // mm_pad_kernel: the codebooks with each codeword padded to 16 bytes [NP][K], or null
  uint32_t cbp_bytes;
};

// hp[part][m][n] = part `part` of h[n][m*d .. m*d+d), padded to 8 with zeros.
// Threads past M*Bp, when cbp is set, copy the codebook with each codeword
// padded to 16 bytes: cbp[i] = codeword i (d bf16, then zeros), i < n_cw.
__global__ void split_h_kernel(const float* __restrict__ h, int B, int D, int M, int d, int Bp,
                               u32x4* __restrict__ hp, const uint16_t* __restrict__ cb, int64_t n_cw,
                               u32x4* __restrict__ cbp) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * Bp) {
    const int64_t i = t - (int64_t)M * Bp;
    if (!cbp || i >= n_cw) return;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(cb + i * d);   // d even: whole 4-byte words
    u32x4 v = {0u, 0u, 0u, 0u};
    for (int w = 0; w < d / 2; ++w) v[w] = src[w];
    cbp[i] = v;
    return;
  }
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

template <int DS, int NT>
struct Staged {
  static constexpr int kH = (kParts * 4 * 16 * NT + kMmThreads - 1) / kMmThreads;   // h vectors per thread
  uint32_t cw[kMaxCwPerThread][DS / 2];
  u32x4 hv[kH];
};

// Partial sums or finished logits of one workgroup: acc[j][t][e] is z for batch
// bt*16NT + 16t + i16 and row tile0 + 16j + 4kg + e (lane = 16kg + i16).
template <int NT, int T>
__device__ __forceinline__ void mm_epilogue(const MmArgs& a, const floatx4 (&acc)[T][NT], int bt, int g, int s,
                                            int64_t tile0, int tid) {
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int n_bt = 16 * NT;
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

// NSUB sub-blocks per code block: 2 for 16-bit codes (pairs 2kg, 2kg+1 in
// dword kg), 3 for RQ_CODES_PACKED10 (pairs 3kg .. 3kg+2, 10 bits each).
template <int DS, int NT, int T, int NSUB>
__global__ __launch_bounds__(kMmThreads) void mm_logits_kernel(MmArgs a) {
  constexpr int PPB = 4 * NSUB;                 // pairs per code block
  constexpr int CBITS = NSUB == 2 ? 16 : 10;    // bits per code
  constexpr uint32_t CMASK = (1u << CBITS) - 1u;
  extern __shared__ __align__(16) u32x4 ring[];   // [2][4*K + kParts*4*16*NT]
  const int K = a.K;
  const int cw_entries = 4 * K;
  const int h_entries = kParts * 4 * 16 * NT;
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
  auto stage_load = [&](Staged<DS, NT>& st, int q, int hs) {
#pragma unroll
    for (int u = 0; u < kMaxCwPerThread; ++u) {
      const int c = (tid + u * kMmThreads) % cw_entries;
      const int kk = c / K;
      const int k = c - kk * K;
      const int p = min(PPB * q + NSUB * kk + hs, a.NP - 1);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.cb + ((size_t)p * K + k) * DS);
#pragma unroll
      for (int w = 0; w < DS / 2; ++w) st.cw[u][w] = src[w];
    }
#pragma unroll
    for (int u = 0; u < Staged<DS, NT>::kH; ++u) {
      const int e = (tid + u * kMmThreads) % h_entries;
      const int pr = e / (4 * n_bt);
      const int rem = e - pr * 4 * n_bt;
      const int kk = rem / n_bt;
      const int n = rem - kk * n_bt;
      const int p = min(PPB * q + NSUB * kk + hs, a.NP - 1);
      const int m = p % a.M;
      st.hv[u] = a.hp[((size_t)pr * a.M + m) * a.Bp + (size_t)bt * n_bt + n];
    }
  };
  auto stage_store = [&](const Staged<DS, NT>& st, int slot, int q, int hs) {
    u32x4* base = ring + slot * slot_entries;
#pragma unroll
    for (int u = 0; u < kMaxCwPerThread; ++u) {
      const int c = (tid + u * kMmThreads) % cw_entries;
      const bool live = PPB * q + NSUB * (c / K) + hs < a.NP;
      u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < DS / 2; ++w) v[w] = live ? st.cw[u][w] : 0u;
      base[c] = v;
    }
#pragma unroll
    for (int u = 0; u < Staged<DS, NT>::kH; ++u) {
      const int e = (tid + u * kMmThreads) % h_entries;
      const int pr = e / (4 * n_bt);
      const int kk = (e - pr * 4 * n_bt) / n_bt;
      const bool live = PPB * q + NSUB * kk + hs < a.NP;
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
    Staged<DS, NT> st;
    load_codes(ca, q0);
    stage_load(st, q0, 0);
    int slot = 0;
    // One code block: its NSUB sub-blocks in turn, each staged in one ring slot
    // while the next one's codebook loads into registers; the first sub-block
    // also starts loading the next block's codes (into the other buffer).
    auto do_block = [&](int q, uint32_t (&cur)[T], uint32_t (&nxt)[T]) {
      arrange_codes(cur);
#pragma unroll
      for (int hs = 0; hs < NSUB; ++hs) {
        stage_store(st, slot, q, hs);
        __syncthreads();
        if (hs + 1 < NSUB) stage_load(st, q, hs + 1);
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

  mm_epilogue<NT, T>(a, acc, bt, g, s, tile0, tid);
}

// ---- K above kMmMaxK (16-bit blocked codes): one pair per ring slot.
//
// A slot holds the K codewords of one (level, subspace) pair exactly as they
// lie in the codebook (K*d bf16, 48 KB at K = 4096, d = 6) and the pair's slice
// of h's three bf16 parts. The MFMA's four k-slots carry the row's codeword
// against parts 0, 1, 2 and a zero: one 16x16x32 MFMA per 16 rows x 16
// vectors x pair, the three-part split folded into the contraction.
//
// Staging goes straight from global memory into LDS (global_load_lds, 16
// bytes per lane, lane-contiguous), so no registers hold the next slot and a
// wave takes 8 row tiles at four column tiles. Per pair: wait for this slot's
// copy, barrier, read the h fragments and the T codeword fragments, start the
// next pair's copy into the other slot, then the MFMAs. The wait is an explicit
// count, so the code loads issued after a copy stay in flight past it.
constexpr int kMmMaxKOnePair = 4 * kMmMaxK;
constexpr int kHSlot = 64;   // h entries per part in a slot (16-byte units; >= 16 NT)

// Codeword k of a slot's segment: DS bf16 values at byte 2 DS k, zero-extended to 8.
template <int DS>
__device__ __forceinline__ bf16x8 read_codeword(const unsigned char* seg, uint32_t k) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (DS == 8) {
    v = *reinterpret_cast<const u32x4*>(seg + k * 16u);
  } else if constexpr (DS == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(seg + k * 8u);
    v[0] = w.x;
    v[1] = w.y;
  } else if constexpr (DS == 2) {
    v[0] = *reinterpret_cast<const uint32_t*>(seg + k * 4u);
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(seg + k * 12u);
    v[0] = w[0];
    v[1] = w[1];
    v[2] = w[2];
  }
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with vmcnt(n) (n < 64: bits 3:0 and 15:14 of the immediate) and the other counters left alone.
#define RQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | (((n) >> 4) << 14))
// The same with lgkmcnt(0): this wave's LDS reads (and other LDS operations) are complete too.
#define RQ_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 0xF) | (((n) >> 4) << 14))

template <int DS, int NT, int T>
__global__ __launch_bounds__(kMmThreads) void mm_pair_kernel(MmArgs a) {
  constexpr int PPB = 8;   // pairs per 16-bit code block
  extern __shared__ __align__(16) unsigned char lds[];
  const int K = a.K;
  const int n_bt = 16 * NT;
  const int seg_words = K * DS / 8;   // 16-byte words of one pair's codewords (the host keeps K*DS % 8 == 0)
  // rounded up to whole copy rounds: every lane of every round lands inside the slot
  const int cw_words = (seg_words + kMmThreads - 1) / kMmThreads * kMmThreads;
  const int slot_bytes = (cw_words + 4 * kHSlot) * 16;

  const int per_bt = a.G * a.S;
  const int bt = blockIdx.x / per_bt;
  const int li = blockIdx.x - bt * per_bt;
  const int g = li % a.G;
  const int s = li / a.G;
  const int q0 = g * a.qpg;
  const int q1 = min(a.NQ, q0 + a.qpg);
  const int p_end = min(a.NP, PPB * q1);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)s * (kMmWaves * T * 16) + (int64_t)wave * (T * 16);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)0xffffffffu,
                                                                        0x00020000);
  const uint32_t blk_bytes = (uint32_t)a.rows * 16u;
  // code loads as in mm_logits_kernel: whole 16-byte rows for T a multiple of 4,
  // transposed across the wave's rows of lanes so that lane (i16, kg) holds
  // dword kg of every tile's row i16
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

  // The fourth h part of both slots is zero (written once, never copied over).
  if (tid < 2 * kHSlot) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(lds + (tid / kHSlot) * slot_bytes + (cw_words + 3 * kHSlot + tid % kHSlot) * 16) = z;
  }
  __syncthreads();
  // Copy pair p into slot r: its codewords (lane-contiguous 16-byte words;
  // lanes past the segment re-read its last word into the slot's slack) and,
  // by waves 0-2, parts 0-2 of h for this batch tile (lanes past the tile's
  // vectors re-read its last one into unused entries).
  auto copy_pair = [&](int r, int p) {
    unsigned char* sb = lds + r * slot_bytes;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.cb) + (size_t)p * seg_words;
    for (int w0 = 0; w0 < cw_words; w0 += kMmThreads)
      __builtin_amdgcn_global_load_lds((const void*)(src + min(w0 + tid, seg_words - 1)),
                                       (lds_ptr_t)(sb + (size_t)(w0 + wave * 64) * 16), 16, 0, 0);
    if (wave < kParts) {
      const u32x4* hsrc = a.hp + ((size_t)wave * a.M + p % a.M) * a.Bp + (size_t)bt * n_bt;
      __builtin_amdgcn_global_load_lds((const void*)(hsrc + min(lane, n_bt - 1)),
                                       (lds_ptr_t)(sb + (size_t)(cw_words + wave * kHSlot) * 16), 16, 0, 0);
    }
  };

  floatx4 acc[T][NT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (PPB * q0 < p_end) {
    uint32_t ca[T], cbk[T];
    load_codes(ca, q0);
    copy_pair(0, PPB * q0);
    // Block q: its 8 pairs, pair p in slot p & 1; the first pair also starts
    // the next block's code loads, after its copy of the next pair.
    auto do_block = [&](int q, uint32_t (&cur)[T], uint32_t (&nxt)[T]) {
      arrange_codes(cur);
#pragma unroll
      for (int hs = 0; hs < PPB; ++hs) {
        const int p = PPB * q + hs;
        if (p >= p_end) break;   // uniform
        // this pair's copy is done: only the code loads issued after it (by the
        // block's first pair) may still be in flight
        if (hs == 1) RQ_WAIT_VMCNT(NV);
        else RQ_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        const unsigned char* sb = lds + (hs & 1) * slot_bytes;
        bf16x8 hb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          hb[t] = *reinterpret_cast<const bf16x8*>(sb + (size_t)(cw_words + kg * kHSlot + 16 * t + i16) * 16);
        const int src_lane = i16 + 16 * (hs >> 1);
        bf16x8 av[T];
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const uint32_t dw = (uint32_t)__shfl((int)cur[j], src_lane, 64);
          av[j] = read_codeword<DS>(sb, (dw >> (16 * (hs & 1))) & 0xffffu);
        }
        __builtin_amdgcn_sched_barrier(0);   // this slot's reads before the copy into the other
        if (p + 1 < p_end) copy_pair((hs + 1) & 1, p + 1);
        __builtin_amdgcn_sched_barrier(0);   // the copy before the code loads (the waits count in order)
        if (hs == 0) load_codes(nxt, min(q + 1, q1 - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < T; ++j)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], hb[t], acc[j][t], 0, 0, 0);
      }
    };
    for (int q = q0; q < q1; q += 2) {
      do_block(q, ca, cbk);
      if (q + 1 < q1) do_block(q + 1, cbk, ca);
    }
  }
  mm_epilogue<NT, T>(a, acc, bt, g, s, tile0, tid);
}

// Row tiles per wave of the one-pair kernel: the accumulators (4*T*NT) beside
// the codeword fragments (4*T), the codes (2*T) and the h fragments (4*NT).
constexpr int pair_tiles_for(int NT) { return NT == 1 ? 16 : 8; }

// ---- The same with three slots (pairs whose codewords fit 48 KB): the copy of
// pair p + 2 starts while pair p is read, so each copy has two pairs' work to
// land. The slots sit at fixed offsets, every copy issues the same number of
// loads (kPair3Rounds rounds of codewords, past the segment clamped into the
// slot's slack, then one h part per wave), and codeword reads are masked to
// the slot: so the waits are counted exactly and the compiler can tell the
// slot being read from the two being filled.
constexpr int kPair3CwWords = 3072;                     // 48 KB of codewords per slot
constexpr int kPair3Rounds = kPair3CwWords / kMmThreads;   // copy rounds (6)
constexpr int kPair3SlotBytes = (kPair3CwWords + 4 * kHSlot) * 16;
constexpr int kPair3Ops = kPair3Rounds + 1;             // loads per copy, per thread

template <int DS, int NT, int T>
__global__ __launch_bounds__(kMmThreads) void mm_pair3_kernel(MmArgs a) {
  constexpr int PPB = 8;   // pairs per 16-bit code block
  constexpr uint32_t kCwMax = (uint32_t)(kPair3CwWords * 16 / (2 * DS)) - 1u;   // last codeword a slot holds
  extern __shared__ __align__(16) unsigned char lds[];
  const int K = a.K;
  const int n_bt = 16 * NT;
  const int seg_words = K * DS / 8;   // <= kPair3CwWords (host check)

  const int per_bt = a.G * a.S;
  const int bt = blockIdx.x / per_bt;
  const int li = blockIdx.x - bt * per_bt;
  const int g = li % a.G;
  const int s = li / a.G;
  const int q0 = g * a.qpg;
  const int q1 = min(a.NQ, q0 + a.qpg);
  const int p_begin = PPB * q0;
  const int p_end = min(a.NP, PPB * q1);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the copies' LDS bases and offsets are scalars
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)s * (kMmWaves * T * 16) + (int64_t)wave * (T * 16);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)0xffffffffu,
                                                                        0x00020000);
  const uint32_t blk_bytes = (uint32_t)a.rows * 16u;
  constexpr bool kWide = T % 4 == 0;
  constexpr int NV = kWide ? T / 4 : T;
  uint32_t voff[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t r = min(tile0 + 16 * (kWide ? 4 * v + kg : v) + i16, a.rows - 1);
    voff[v] = (uint32_t)r * 16u + (kWide ? 0u : (uint32_t)kg * 4u);
  }
  // Codes stay in the registers they are loaded into (u32x4 per wide load);
  // each block's arranged copy is a fresh value, so no loaded register is ever
  // moved (a move right after a load made the compiler wait for it, and for
  // the copy into LDS issued before it).
  static_assert(kWide, "the one-pair kernels take row tiles in multiples of 4");
  auto load_codes = [&](u32x4 (&dst)[NV], int q) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      dst[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, voff[v], (uint32_t)q * blk_bytes, 0));
  };
  auto arranged = [&](const u32x4 (&raw)[NV], uint32_t (&c)[T]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const auto x02 = __builtin_amdgcn_permlane32_swap(raw[v][0], raw[v][2], false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(raw[v][1], raw[v][3], false, false);
      const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
      const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
      c[4 * v + 0] = y01[0]; c[4 * v + 1] = y01[1]; c[4 * v + 2] = y23[0]; c[4 * v + 3] = y23[1];
    }
  };

  if (tid < 3 * kHSlot) {   // the fourth h part of every slot is zero
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(lds + (tid / kHSlot) * kPair3SlotBytes + (kPair3CwWords + 3 * kHSlot + tid % kHSlot) * 16) = z;
  }
  __syncthreads();
  // Copy pair p into slot R: kPair3Rounds rounds of lane-contiguous 16-byte
  // codeword words, then part (wave mod 3) of h (three waves copy each part, the
  // same bytes to the same place).
  // Buffer loads into LDS: the lane's byte offset is the same in every round
  // and copy (one register), the pair's and the round's offset a scalar. Words
  // past the pair's segment carry the next pair's codewords (or zeros past the
  // codebook: the buffer's range check) into the slot's slack, never read.
  const __amdgpu_buffer_rsrc_t cbrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.cb, (short)0, (int)a.cb_bytes,
                                                                         0x00020000);
  const __amdgpu_buffer_rsrc_t hprs = __builtin_amdgcn_make_buffer_rsrc((void*)a.hp, (short)0, (int)a.hp_bytes,
                                                                         0x00020000);
  const uint32_t cw_voff = (uint32_t)tid * 16u;
  const uint32_t h_voff = (uint32_t)min(lane, n_bt - 1) * 16u;
  auto copy_pair = [&](int R, int p) {
    unsigned char* sb = lds + R * kPair3SlotBytes;
    const uint32_t base = (uint32_t)p * (uint32_t)(seg_words * 16);
#pragma unroll
    for (int rd = 0; rd < kPair3Rounds; ++rd)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cbrs, (lds_ptr_t)(sb + (size_t)(rd * kMmThreads + wave * 64) * 16), 16,
                                               cw_voff, base + (uint32_t)(rd * kMmThreads * 16), 0, 0);
    const int part = wave % kParts;
    const uint32_t hbase = (uint32_t)((((size_t)part * a.M + p % a.M) * a.Bp + (size_t)bt * n_bt) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hprs, (lds_ptr_t)(sb + (size_t)(kPair3CwWords + part * kHSlot) * 16), 16,
                                             h_voff, hbase, 0, 0);
  };

  floatx4 acc[T][NT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Reads of pair p from its slot: the h fragments of the NT column tiles and
  // the codewords of row tiles [j0, j1) (the row's code broadcast from the lane
  // row that holds the dword of pair p).
  auto read_h = [&](bf16x8 (&hb)[NT], int p) {
    const unsigned char* sb = lds + ((p - p_begin) % 3) * kPair3SlotBytes;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      hb[t] = *reinterpret_cast<const bf16x8*>(sb + (size_t)(kPair3CwWords + kg * kHSlot + 16 * t + i16) * 16);
  };
  auto read_a = [&](bf16x8 (&av)[T], const uint32_t (&codes)[T], int p, int j0, int j1) {
    const unsigned char* sb = lds + ((p - p_begin) % 3) * kPair3SlotBytes;
    const int hs = p & (PPB - 1);
    const int src_lane = i16 + 16 * (hs >> 1);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const uint32_t dw = (uint32_t)__shfl((int)codes[j], src_lane, 64);
      av[j] = read_codeword<DS>(sb, min((dw >> (16 * (hs & 1))) & 0xffffu, kCwMax));
    }
  };
  auto mfma = [&](const bf16x8 (&av)[T], const bf16x8 (&hb)[NT], int j0, int j1) {
#pragma unroll
    for (int j = j0; j < j1; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], hb[t], acc[j][t], 0, 0, 0);
  };

  const int nsteps = p_end - p_begin;
  if (nsteps > 0) {
    // Software pipeline: the codewords and h of pair p + 1 are read from LDS
    // while the matrix cores work on pair p, so a wave's LDS reads and MFMAs
    // overlap instead of taking turns between barriers.
    //   prologue: copies of pairs 0, 1, 2 into slots 0, 1, 2; reads of pair 0.
    //   step for pair p (slot p mod 3):
    //     MFMAs of the first half of the row tiles (pair p);
    //     wait until pair p + 1's copy has landed and this wave's reads of
    //       pair p are done; barrier (every wave's are: slot p is free);
    //     copy of pair p + 3 into slot p mod 3 (issued even past the group's
    //       last pair, clamped, so that every step issues the same loads);
    //       at a code block's last pair, the loads of the codes two blocks on;
    //     reads of pair p + 1's h and of the first half's codewords;
    //     MFMAs of the second half (pair p), then reads of the second half's
    //       codewords (pair p + 1).
    // Each copy has two steps to land. The waits count vector-memory loads in
    // issue order: after pair p + 1's copy come pair p + 2's and, when p is a
    // block's first or second pair, one set of code loads.
    // Two code buffers alternate by block (codes_a: even blocks of the group,
    // codes_b: odd), so 16 steps make one unrolled round and no code register
    // is ever moved (a move would make the compiler wait for the loads in
    // flight). Rounds whose 16 steps all have a next pair run unguarded; the
    // last round checks each step.
    constexpr int TH = T / 2;
    u32x4 raw_a[NV], raw_b[NV];        // loaded codes of the group's even / odd blocks
    uint32_t codes_a[T], codes_b[T];   // their arranged copies
    bf16x8 av[T];
    bf16x8 hb0[NT], hb1[NT];
    load_codes(raw_a, q0);
    copy_pair(0, p_begin);
    copy_pair(1, min(p_begin + 1, a.NP - 1));
    copy_pair(2, min(p_begin + 2, a.NP - 1));
    RQ_WAIT_VMCNT(2 * kPair3Ops);
    __builtin_amdgcn_s_barrier();
    arranged(raw_a, codes_a);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(raw_b, min(q0 + 1, q1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    read_h(hb0, p_begin);
    read_a(av, codes_a, p_begin, 0, T);

    auto step = [&](auto kc, auto guarded, int i) {
      constexpr int k = decltype(kc)::value;   // position in the round of two code blocks
      constexpr bool checks = decltype(guarded)::value;
      constexpr bool odd = k & 1;
      constexpr bool block_end = (k & 7) == 7;
      constexpr bool read_b = k >= 7 && k < 15;   // pair p + 1 lies in an odd block
      bf16x8(&hc)[NT] = odd ? hb1 : hb0;
      bf16x8(&hn)[NT] = odd ? hb0 : hb1;
      uint32_t(&rd)[T] = read_b ? codes_b : codes_a;
      u32x4(&raw_rd)[NV] = read_b ? raw_b : raw_a;
      u32x4(&ld)[NV] = k == 7 ? raw_a : raw_b;   // (used at a block's last pair only)
      if (checks && i >= nsteps) return;
      const int p = p_begin + i;
      mfma(av, hc, 0, TH);
      __builtin_amdgcn_sched_barrier(0);
      const bool more = !checks || i + 1 < nsteps;
      if (more) {
        // with lgkmcnt(0): this wave's reads of slot p are complete
        if constexpr ((k & 7) <= 1) RQ_WAIT_VMCNT_LDS(kPair3Ops + NV);
        else RQ_WAIT_VMCNT_LDS(kPair3Ops);
        __builtin_amdgcn_s_barrier();
        copy_pair(i % 3, min(p + 3, a.NP - 1));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (block_end) {
          arranged(raw_rd, rd);
          __builtin_amdgcn_sched_barrier(0);
          load_codes(ld, min(((p + 1) >> 3) + 1, q1 - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        read_h(hn, p + 1);
        read_a(av, rd, p + 1, 0, TH);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma(av, hc, TH, T);
      __builtin_amdgcn_sched_barrier(0);
      if (more) read_a(av, rd, p + 1, TH, T);
    };
    auto round = [&](auto guarded, int i0) {
      step(std::integral_constant<int, 0>{}, guarded, i0 + 0);
      step(std::integral_constant<int, 1>{}, guarded, i0 + 1);
      step(std::integral_constant<int, 2>{}, guarded, i0 + 2);
      step(std::integral_constant<int, 3>{}, guarded, i0 + 3);
      step(std::integral_constant<int, 4>{}, guarded, i0 + 4);
      step(std::integral_constant<int, 5>{}, guarded, i0 + 5);
      step(std::integral_constant<int, 6>{}, guarded, i0 + 6);
      step(std::integral_constant<int, 7>{}, guarded, i0 + 7);
      step(std::integral_constant<int, 8>{}, guarded, i0 + 8);
      step(std::integral_constant<int, 9>{}, guarded, i0 + 9);
      step(std::integral_constant<int, 10>{}, guarded, i0 + 10);
      step(std::integral_constant<int, 11>{}, guarded, i0 + 11);
      step(std::integral_constant<int, 12>{}, guarded, i0 + 12);
      step(std::integral_constant<int, 13>{}, guarded, i0 + 13);
      step(std::integral_constant<int, 14>{}, guarded, i0 + 14);
      step(std::integral_constant<int, 15>{}, guarded, i0 + 15);
    };
    int i0 = 0;
    for (; i0 + 16 < nsteps; i0 += 16) round(std::false_type{}, i0);
    round(std::true_type{}, i0);
    RQ_WAIT_VMCNT(0);   // no copy into LDS may be in flight when the workgroup ends
  }
  mm_epilogue<NT, T>(a, acc, bt, g, s, tile0, tid);
}

// ---- All of 65..128 hidden vectors in one workgroup (eight column tiles),
// 16-bit blocked codes, a half-block's codewords within 48 KB (K <= 1024 at
// d = 6). With two batch tiles of 64 every slab of rows staged the codebook
// twice; here one staging serves all 128 vectors. The half-block goes straight
// into a two-slot LDS ring with buffer loads: the codewords as they lie in the
// codebook (d bf16 each; their LDS reads are few beside 24 MFMAs per read, so
// the 12-byte reads' bank conflicts do not matter) and the three h parts of
// the four pairs for the 128 vectors. Per step the copy of the next
// half-block is issued first and has the whole step (96 MFMAs per wave) to
// land; the h fragments are read from LDS one column tile and part at a time,
// the next one while the matrix cores work on the current one.
constexpr int kWideNT = 8;
constexpr int kWideTiles = 4;                                      // row tiles per wave (accumulators: 128 VGPRs)
constexpr int kWideCwWords = 3072;                                 // 48 KB of codewords per slot
constexpr int kWideHWords = kParts * 4 * 16 * kWideNT;             // 1536
constexpr int kWideSlotBytes = (kWideCwWords + kWideHWords) * 16;  // 72 KB
constexpr int kWideCwRounds = kWideCwWords / kMmThreads;           // 6
constexpr int kWideHRounds = kWideHWords / kMmThreads;             // 3
static_assert(kWideHWords % kMmThreads == 0 && 4 * 16 * kWideNT == kMmThreads, "h: one part per copy round");

template <int DS>
__global__ __launch_bounds__(kMmThreads) void mm_wide_kernel(MmArgs a) {
  constexpr int T = kWideTiles;
  constexpr int NT = kWideNT;
  constexpr int PPB = 8;
  constexpr int NV = T / 4;   // wide code loads per block
  extern __shared__ __align__(16) unsigned char lds[];
  const int K = a.K;
  const int seg_words = K * DS / 8;   // host: 4 * seg_words <= kWideCwWords
  const uint32_t seg_bytes = (uint32_t)seg_words * 16u;
  const uint32_t kmax = (uint32_t)K - 1u;

  const int g = blockIdx.x % a.G;     // one batch tile
  const int s = blockIdx.x / a.G;
  const int q0 = g * a.qpg;
  const int q1 = min(a.NQ, q0 + a.qpg);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)s * (kMmWaves * T * 16) + (int64_t)wave * (T * 16);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)0xffffffffu,
                                                                        0x00020000);
  const uint32_t blk_bytes = (uint32_t)a.rows * 16u;
  uint32_t voff[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t r = min(tile0 + 16 * (4 * v + kg) + i16, a.rows - 1);
    voff[v] = (uint32_t)r * 16u;
  }
  // Codes stay in the registers they are loaded into (u32x4 per wide load):
  // the arranged copy each block uses is a fresh value, so no loaded register
  // is ever moved (a move right after a load made the compiler wait for it).
  auto load_codes = [&](u32x4 (&dst)[NV], int q) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      dst[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, voff[v], (uint32_t)q * blk_bytes, 0));
  };
  auto arranged = [&](const u32x4 (&raw)[NV], uint32_t (&c)[T]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const auto x02 = __builtin_amdgcn_permlane32_swap(raw[v][0], raw[v][2], false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(raw[v][1], raw[v][3], false, false);
      const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
      const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
      c[4 * v + 0] = y01[0]; c[4 * v + 1] = y01[1]; c[4 * v + 2] = y23[0]; c[4 * v + 3] = y23[1];
    }
  };

  // Copy of half-block (q, hs) into slot R. Codewords: slot word w = rd * 512 +
  // tid is word (w mod seg_words) of pair 8q + 2 (w div seg_words) + hs, the
  // lane's offset past pair 8q + hs fixed per round. h: round rd copies part rd,
  // slot word rd * 512 + tid = (part * 4 + kk) * 128 + n for kk = tid / 128,
  // n = tid mod 128 (vectors past B are zero in the split h).
  const __amdgpu_buffer_rsrc_t cbrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.cb, (short)0, (int)a.cb_bytes,
                                                                         0x00020000);
  const __amdgpu_buffer_rsrc_t hprs = __builtin_amdgcn_make_buffer_rsrc((void*)a.hp, (short)0, (int)a.hp_bytes,
                                                                         0x00020000);
  uint32_t cw_voff[kWideCwRounds];
#pragma unroll
  for (int rd = 0; rd < kWideCwRounds; ++rd) {
    const int w = min(rd * kMmThreads + tid, 4 * seg_words - 1);   // past four segments: a copy of the last word
    const int kk = w / seg_words;
    cw_voff[rd] = (uint32_t)(2 * kk) * seg_bytes + (uint32_t)(w - kk * seg_words) * 16u;
  }
  const int h_kk = tid / (16 * NT);
  const int h_n = tid % (16 * NT);
  auto copy_half = [&](int R, int q, int hs) {
    unsigned char* sb = lds + R * kWideSlotBytes;
    const uint32_t base = (uint32_t)(PPB * q + hs) * seg_bytes;
#pragma unroll
    for (int rd = 0; rd < kWideCwRounds; ++rd)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cbrs, (lds_ptr_t)(sb + (size_t)(rd * kMmThreads + wave * 64) * 16), 16,
                                               cw_voff[rd], base, 0, 0);
    const int m = (PPB * q + 2 * h_kk + hs) % a.M;
    const uint32_t hv = (uint32_t)((size_t)m * a.Bp + h_n) * 16u;
#pragma unroll
    for (int rd = 0; rd < kWideHRounds; ++rd)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          hprs, (lds_ptr_t)(sb + (size_t)(kWideCwWords + rd * kMmThreads + wave * 64) * 16), 16, hv,
          (uint32_t)((size_t)rd * a.M * a.Bp * 16), 0, 0);
  };

  floatx4 acc[T][NT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One half-block from slot R: the row tiles' codewords, then for each column
  // tile and part one h fragment (the next one read while these four MFMAs
  // run). The codewords and the first fragment are read first (begin_reads),
  // before the step issues its copy and code loads, so their LDS latency runs
  // under those issues.
  bf16x8 av[T];
  bf16x8 hb[2];
  auto hl_of = [&](int R) {   // the lane's h fragment address in slot R; part and column tile are constant offsets
    return lds + R * kWideSlotBytes + (size_t)(kWideCwWords + kg * (16 * NT) + i16) * 16;
  };
  auto read_hb = [&](const unsigned char* hl, int t, int pr) {
    return *reinterpret_cast<const bf16x8*>(hl + (size_t)(pr * 4 * (16 * NT) + 16 * t) * 16);
  };
  auto begin_reads = [&](int R, const uint32_t (&codes)[T], int hs) {
    const unsigned char* seg = lds + R * kWideSlotBytes + (size_t)kg * seg_bytes;
#pragma unroll
    for (int j = 0; j < T; ++j) av[j] = read_codeword<DS>(seg, min((codes[j] >> (16 * hs)) & 0xffffu, kmax));
    hb[0] = read_hb(hl_of(R), 0, 0);
  };
  auto compute = [&](int R) {
    const unsigned char* hl = hl_of(R);
#pragma unroll
    for (int i = 0; i < NT * kParts; ++i) {
      const int t = i / kParts;
      if (i + 1 < NT * kParts) hb[(i + 1) & 1] = read_hb(hl, (i + 1) / kParts, (i + 1) % kParts);
#pragma unroll
      for (int j = 0; j < T; ++j) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], hb[i & 1], acc[j][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // one fragment read ahead, no more (registers)
    }
  };

  const int nsteps = 2 * (q1 - q0);   // half-blocks: step st is block q0 + st / 2, sub-block st mod 2
  if (nsteps > 0) {
    // Step st (slot st mod 2): wait until its copy has landed (issued at the
    // start of step st - 1; after it only the code loads of a block's first
    // half); barrier (every wave is done with slot st + 1's previous
    // contents); copy of step st + 1 into the other slot (clamped past the
    // group's end so every step issues the same loads); at a block's first
    // half, the codes of the next block; the half-block's MFMAs. Code buffers
    // alternate by block (codes_a: even blocks of the group), so a round of
    // four steps is unrolled and no loaded register is moved.
    u32x4 raw_a[NV], raw_b[NV];   // loaded codes of the group's even / odd blocks
    const int qlast = q1 - 1;
    load_codes(raw_a, q0);
    copy_half(0, q0, 0);
    auto step = [&](auto kc, auto guarded, int st, uint32_t (&cur)[T]) {
      constexpr int k = decltype(kc)::value;   // position in a round of two blocks
      constexpr bool checks = decltype(guarded)::value;
      constexpr int hs = k & 1;
      u32x4(&raw)[NV] = k < 2 ? raw_a : raw_b;
      u32x4(&nxt)[NV] = k < 2 ? raw_b : raw_a;
      if (checks && st >= nsteps) return;
      // (with lgkmcnt(0): this wave's reads of the slot the next copy overwrites are complete)
      if constexpr (hs == 1) RQ_WAIT_VMCNT_LDS(NV);   // this step's copy; the next block's codes may still fly
      else RQ_WAIT_VMCNT_LDS(0);                      // this step's copy and this block's codes
      __builtin_amdgcn_s_barrier();
      if constexpr (hs == 0) arranged(raw, cur);
      begin_reads(st & 1, cur, hs);
      __builtin_amdgcn_sched_barrier(0);
      const int st1 = st + 1;
      copy_half(st1 & 1, min(q0 + (st1 >> 1), qlast), st1 & 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (hs == 0) load_codes(nxt, min(q0 + (st >> 1) + 1, qlast));
      __builtin_amdgcn_sched_barrier(0);
      compute(st & 1);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto round = [&](auto guarded, int s0) {
      uint32_t cur_a[T], cur_b[T];   // arranged codes of this round's two blocks
      step(std::integral_constant<int, 0>{}, guarded, s0 + 0, cur_a);
      step(std::integral_constant<int, 1>{}, guarded, s0 + 1, cur_a);
      step(std::integral_constant<int, 2>{}, guarded, s0 + 2, cur_b);
      step(std::integral_constant<int, 3>{}, guarded, s0 + 3, cur_b);
    };
    int s0 = 0;
    for (; s0 + 4 <= nsteps; s0 += 4) round(std::false_type{}, s0);
    round(std::true_type{}, s0);
    RQ_WAIT_VMCNT(0);   // no copy into LDS may be in flight when the workgroup ends
  }
  mm_epilogue<NT, T>(a, acc, 0, g, s, tile0, tid);
}

// ---- Up to 16 vectors (one column tile), 16-bit blocked codes, K <= 1024:
// mm_logits_kernel's half-blocks, loaded straight into LDS from a copy of the
// codebooks with every codeword padded to 16 bytes (written by the split
// kernel into the workspace each call). The padding keeps the conflict-light
// 16-byte codeword reads of the register-staged kernel; the straight loads
// drop its register copies and LDS stores. Two slots of 64 KB + 3 KB: per step
// wait for this half-block's copy (issued at the start of the previous step),
// barrier, issue the next one into the other slot, then the MFMAs with the
// codewords of the next four row tiles read while the current four compute.
// Eight waves of sixteen row tiles (2,048 rows per workgroup); sixteen waves of
// eight measured 3% slower.
constexpr int kPadThreads = 512;
constexpr int kPadWaves = kPadThreads / 64;
constexpr int kPadTiles = 2048 / 16 / kPadWaves;                    // row tiles per wave (16)
constexpr int kPadCwWords = 4 * kMmMaxK;                            // 64 KB of codewords per slot
constexpr int kPadHWords = kParts * 4 * 16;                         // h parts of one column tile
constexpr int kPadSlotBytes = (kPadCwWords + kPadHWords) * 16;
constexpr int kPadCwRounds = kPadCwWords / kPadThreads;             // 8
static_assert(kPadHWords % 64 == 0 && kPadHWords <= kPadThreads, "one h load per lane");

__global__ __launch_bounds__(kPadThreads) void mm_pad_kernel(MmArgs a) {
  constexpr int T = kPadTiles;
  constexpr int PPB = 8;
  constexpr int NV = T / 4;
  extern __shared__ __align__(16) unsigned char lds[];
  const int K = a.K;
  const uint32_t kmax = (uint32_t)K - 1u;
  const uint32_t seg_bytes = (uint32_t)K * 16u;

  const int g = blockIdx.x % a.G;     // one batch tile
  const int s = blockIdx.x / a.G;
  const int q0 = g * a.qpg;
  const int q1 = min(a.NQ, q0 + a.qpg);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)s * (kPadWaves * T * 16) + (int64_t)wave * (T * 16);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)0xffffffffu,
                                                                        0x00020000);
  const uint32_t blk_bytes = (uint32_t)a.rows * 16u;
  uint32_t voff[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t r = min(tile0 + 16 * (4 * v + kg) + i16, a.rows - 1);
    voff[v] = (uint32_t)r * 16u;
  }
  // Codes stay in the registers they are loaded into (u32x4 per wide load):
  // the arranged copy each block uses is a fresh value, so no loaded register
  // is ever moved (a move right after a load made the compiler wait for it).
  auto load_codes = [&](u32x4 (&dst)[NV], int q) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      dst[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, voff[v], (uint32_t)q * blk_bytes, 0));
  };
  auto arranged = [&](const u32x4 (&raw)[NV], uint32_t (&c)[T]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const auto x02 = __builtin_amdgcn_permlane32_swap(raw[v][0], raw[v][2], false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(raw[v][1], raw[v][3], false, false);
      const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
      const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
      c[4 * v + 0] = y01[0]; c[4 * v + 1] = y01[1]; c[4 * v + 2] = y23[0]; c[4 * v + 3] = y23[1];
    }
  };

  // Copy of half-block (q, hs) into slot R. Codewords: slot word w = rd * 512 +
  // tid is codeword (w mod K) of pair 8q + 2 (w div K) + hs (a dead pair past
  // L*M reads zeros: the buffer's range check). h: slot word e = (part * 4 + kk)
  // * 16 + n; every wave loads one 64-word run (waves past the third repeat
  // the first runs: the same bytes to the same place).
  const __amdgpu_buffer_rsrc_t cbrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.cbp, (short)0, (int)a.cbp_bytes,
                                                                         0x00020000);
  const __amdgpu_buffer_rsrc_t hprs = __builtin_amdgcn_make_buffer_rsrc((void*)a.hp, (short)0, (int)a.hp_bytes,
                                                                         0x00020000);
  uint32_t cw_voff[kPadCwRounds];
#pragma unroll
  for (int rd = 0; rd < kPadCwRounds; ++rd) {
    const int w = min(rd * kPadThreads + tid, 4 * K - 1);   // past four segments (K < 1024): a copy of the last word
    const int kk = w / K;
    cw_voff[rd] = (uint32_t)(2 * kk) * seg_bytes + (uint32_t)(w - kk * K) * 16u;
  }
  const int h_run = wave % (kPadHWords / 64);
  const int h_e = h_run * 64 + lane;
  const int h_part = h_e / 64;
  const int h_kk = (h_e / 16) % 4;
  const int h_n = h_e % 16;
  auto copy_half = [&](int R, int q, int hs) {
    unsigned char* sb = lds + R * kPadSlotBytes;
    const uint32_t base = (uint32_t)(PPB * q + hs) * seg_bytes;
#pragma unroll
    for (int rd = 0; rd < kPadCwRounds; ++rd)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cbrs, (lds_ptr_t)(sb + (size_t)(rd * kPadThreads + wave * 64) * 16), 16,
                                               cw_voff[rd], base, 0, 0);
    const int m = (PPB * q + 2 * h_kk + hs) % a.M;
    const uint32_t hoff = (uint32_t)(((size_t)h_part * a.M + m) * a.Bp + h_n) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hprs, (lds_ptr_t)(sb + (size_t)(kPadCwWords + h_run * 64) * 16), 16,
                                             hoff, 0, 0, 0);
  };

  floatx4 acc[T];
#pragma unroll
  for (int j = 0; j < T; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Right after the barrier the step issues the next half-block's copy (so it
  // has the whole step to land), then reads the h fragments and the first four
  // row tiles' codewords (begin_reads), then the code loads; the codewords of
  // the next four row tiles are read while the current four compute. (Reads
  // first and the copy after them measured 4-5% slower per B=16 call.)
  constexpr int kI = 4;
  constexpr int kGroups = T / kI;
  bf16x8 hb[kParts];
  bf16x8 av[2][kI];
  auto cw = [&](int R, const uint32_t (&codes)[T], int hs, int j) {
    const unsigned char* cwb = lds + R * kPadSlotBytes + (size_t)kg * seg_bytes;
    return *reinterpret_cast<const bf16x8*>(cwb + min((codes[j] >> (16 * hs)) & 0xffffu, kmax) * 16u);
  };
  auto begin_reads = [&](int R, const uint32_t (&codes)[T], int hs) {
    const unsigned char* sb = lds + R * kPadSlotBytes;
#pragma unroll
    for (int pr = 0; pr < kParts; ++pr)
      hb[pr] = *reinterpret_cast<const bf16x8*>(sb + (size_t)(kPadCwWords + (pr * 4 + kg) * 16 + i16) * 16);
#pragma unroll
    for (int u = 0; u < kI; ++u) av[0][u] = cw(R, codes, hs, u);
  };
  auto compute = [&](int R, const uint32_t (&codes)[T], int hs) {
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const int cur = gi & 1;
      if (gi + 1 < kGroups) {
#pragma unroll
        for (int u = 0; u < kI; ++u) av[cur ^ 1][u] = cw(R, codes, hs, (gi + 1) * kI + u);
      }
#pragma unroll
      for (int pr = 0; pr < kParts; ++pr)
#pragma unroll
        for (int u = 0; u < kI; ++u)
          acc[gi * kI + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cur][u], hb[pr], acc[gi * kI + u], 0, 0, 0);
    }
  };

  const int nsteps = 2 * (q1 - q0);
  if (nsteps > 0) {
    // The same step structure as mm_wide_kernel: after this step's copy come
    // only the code loads of a block's first half (issued after the copy of
    // the step that began the block).
    u32x4 raw_a[NV], raw_b[NV];   // loaded codes of the group's even / odd blocks
    const int qlast = q1 - 1;
    load_codes(raw_a, q0);
    copy_half(0, q0, 0);
    auto step = [&](auto kc, auto guarded, int st, uint32_t (&cur)[T]) {
      constexpr int k = decltype(kc)::value;
      constexpr bool checks = decltype(guarded)::value;
      constexpr int hs = k & 1;
      u32x4(&raw)[NV] = k < 2 ? raw_a : raw_b;
      u32x4(&nxt)[NV] = k < 2 ? raw_b : raw_a;
      if (checks && st >= nsteps) return;
      if constexpr (hs == 1) RQ_WAIT_VMCNT_LDS(NV);
      else RQ_WAIT_VMCNT_LDS(0);
      __builtin_amdgcn_s_barrier();
      const int st1 = st + 1;
      copy_half(st1 & 1, min(q0 + (st1 >> 1), qlast), st1 & 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (hs == 0) arranged(raw, cur);
      begin_reads(st & 1, cur, hs);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (hs == 0) load_codes(nxt, min(q0 + (st >> 1) + 1, qlast));
      __builtin_amdgcn_sched_barrier(0);
      compute(st & 1, cur, hs);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto round = [&](auto guarded, int s0) {
      uint32_t cur_a[T], cur_b[T];   // arranged codes of this round's two blocks
      step(std::integral_constant<int, 0>{}, guarded, s0 + 0, cur_a);
      step(std::integral_constant<int, 1>{}, guarded, s0 + 1, cur_a);
      step(std::integral_constant<int, 2>{}, guarded, s0 + 2, cur_b);
      step(std::integral_constant<int, 3>{}, guarded, s0 + 3, cur_b);
    };
    int s0 = 0;
    for (; s0 + 4 <= nsteps; s0 += 4) round(std::false_type{}, s0);
    round(std::true_type{}, s0);
    RQ_WAIT_VMCNT(0);
  }
  mm_epilogue<1, T>(a, reinterpret_cast<const floatx4(&)[T][1]>(acc), 0, g, s, tile0, tid);
}

// Row tiles per wave for NT column tiles: the accumulators (4*T*NT VGPRs), the
// code registers (2*T) and the staged half-block share a wave's 256 VGPRs.
// (Three sub-blocks per code block keep more values live: fewer tiles.) A
// multiple of 4 takes the wide code loads; 4 at NT = 4 uses 254 VGPRs.
constexpr int tiles_for(int NT, int NSUB = 2) {
  return kMmThreads == 512 ? (NSUB == 2 ? (NT == 1 ? 16 : NT == 2 ? 8 : 4) : (NT == 1 ? 12 : NT == 2 ? 6 : 3))
                           : (NT == 1 ? 8 : NT == 2 ? 4 : 2);
}

template <int DS, int NT, int NSUB>
hipError_t launch_typed(const MmArgs& a, int wgs, size_t lds, hipStream_t stream) {
  auto kern = mm_logits_kernel<DS, NT, tiles_for(NT, NSUB), NSUB>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kMmThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DS, int NSUB>
hipError_t launch_ds(const MmArgs& a, const MmPlan& p, hipStream_t stream) {
  const int wgs = p.G * p.S * p.NBT;
  if (p.NT == 1) return launch_typed<DS, 1, NSUB>(a, wgs, p.lds, stream);
  if (p.NT == 2) return launch_typed<DS, 2, NSUB>(a, wgs, p.lds, stream);
  return launch_typed<DS, 4, NSUB>(a, wgs, p.lds, stream);
}

template <int NSUB>
hipError_t launch_nsub(const MmArgs& a, const MmPlan& p, int d, hipStream_t stream) {
  switch (d) {
    case 2: return launch_ds<2, NSUB>(a, p, stream);
    case 4: return launch_ds<4, NSUB>(a, p, stream);
    case 6: return launch_ds<6, NSUB>(a, p, stream);
    default: return launch_ds<8, NSUB>(a, p, stream);
  }
}

template <int DS, int NT>
hipError_t launch_pair_typed(const MmArgs& a, int wgs, size_t lds, hipStream_t stream) {
  auto kern = (int64_t)a.K * DS / 8 <= kPair3CwWords ? mm_pair3_kernel<DS, NT, pair_tiles_for(NT)>
                                                      : mm_pair_kernel<DS, NT, pair_tiles_for(NT)>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kMmThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DS>
hipError_t launch_pair_ds(const MmArgs& a, const MmPlan& p, hipStream_t stream) {
  const int wgs = p.G * p.S * p.NBT;
  if (p.NT == 1) return launch_pair_typed<DS, 1>(a, wgs, p.lds, stream);
  if (p.NT == 2) return launch_pair_typed<DS, 2>(a, wgs, p.lds, stream);
  return launch_pair_typed<DS, 4>(a, wgs, p.lds, stream);
}

hipError_t launch_pad(const MmArgs& a, const MmPlan& p, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)mm_pad_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mm_pad_kernel, dim3((unsigned)(p.G * p.S)), dim3(kPadThreads), p.lds, stream, a);
  return hipGetLastError();
}

template <int DS>
hipError_t launch_wide_ds(const MmArgs& a, const MmPlan& p, hipStream_t stream) {
  auto kern = mm_wide_kernel<DS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.G * p.S)), dim3(kMmThreads), p.lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_wide(const MmArgs& a, const MmPlan& p, int d, hipStream_t stream) {
  switch (d) {
    case 2: return launch_wide_ds<2>(a, p, stream);
    case 4: return launch_wide_ds<4>(a, p, stream);
    case 6: return launch_wide_ds<6>(a, p, stream);
    default: return launch_wide_ds<8>(a, p, stream);
  }
}

hipError_t launch_pair(const MmArgs& a, const MmPlan& p, int d, hipStream_t stream) {
  switch (d) {
    case 2: return launch_pair_ds<2>(a, p, stream);
    case 4: return launch_pair_ds<4>(a, p, stream);
    case 6: return launch_pair_ds<6>(a, p, stream);
    default: return launch_pair_ds<8>(a, p, stream);
  }
}

}  // namespace

// One pair per ring slot (mm_pair_kernel) for K beyond what four pairs per slot can stage.
static bool mm_one_pair(const rq_matrix* W) { return W->K > kMmMaxK; }

bool mm_supported(const rq_matrix* W) {
  if (W->cb_dtype != RQ_BF16 || W->d > 8 || (W->d % 2) != 0 || ((uintptr_t)W->codebooks % 4) != 0) return false;
  if (W->K <= kMmMaxK) return W->codes_layout == RQ_CODES_BLOCKED || W->codes_layout == RQ_CODES_PACKED10;
  // one pair per slot: 16-bit blocked codes, each pair's codewords a whole number of 16-byte words
  return W->K <= kMmMaxKOnePair && W->codes_layout == RQ_CODES_BLOCKED && ((int64_t)W->K * W->d) % 8 == 0 &&
         ((uintptr_t)W->codebooks % 16) == 0;
}

// Bytes of the bf16 codebooks [NP][K][d].
static size_t cb_bytes(const rq_matrix* W) { return (size_t)W->L * W->M * W->K * W->d * sizeof(uint16_t); }

bool mm_usable(const rq_matrix* W, int B) {
  if (B < RQ_MM_MIN_B || !mm_supported(W)) return false;
  if (!mm_one_pair(W)) return true;
  // the one-pair kernels address the codebooks and the split h with 32-bit buffer offsets
  return cb_bytes(W) < ((size_t)1 << 32) && mm_hp_bytes(W, plan_mm(W, B)) < ((size_t)1 << 32);
}

// Up to 16 vectors on 16-bit blocked codes, K <= 1024: mm_pad_kernel.
static bool mm_pad(const rq_matrix* W, int B) {
  return B <= 16 && !mm_one_pair(W) && W->codes_layout == RQ_CODES_BLOCKED &&
         (size_t)W->L * W->M * W->K * 16 < ((size_t)1 << 32);
}

// 65..128 vectors on 16-bit blocked codes whose half-block of codewords fits 48 KB: mm_wide_kernel.
static bool mm_wide(const rq_matrix* W, int B) {
  return B > 4 * 16 && B <= 16 * kWideNT && !mm_one_pair(W) && W->codes_layout == RQ_CODES_BLOCKED &&
         ((int64_t)W->K * W->d) % 8 == 0 && (int64_t)W->K * W->d / 2 <= kWideCwWords &&
         ((uintptr_t)W->codebooks % 16) == 0 && cb_bytes(W) < ((size_t)1 << 32) &&
         (size_t)kParts * W->M * 16 * kWideNT * 16 < ((size_t)1 << 32);
}

// Three slots when a pair's codewords fit one (mm_pair3_kernel), else two.
static bool pair3_fits(const rq_matrix* W) { return (int64_t)W->K * W->d / 8 <= kPair3CwWords; }

// Bytes of one ring slot of mm_pair_kernel.
static size_t pair_slot_bytes(const rq_matrix* W) {
  const size_t seg_words = (size_t)W->K * W->d / 8;
  const size_t cw_words = (seg_words + kMmThreads - 1) / kMmThreads * kMmThreads;
  return (cw_words + 4 * kHSlot) * 16;
}

MmPlan plan_mm(const rq_matrix* W, int B) {
  MmPlan p{};
  const bool wide = mm_wide(W, B);
  p.pad = mm_pad(W, B) ? 1 : 0;
  p.NT = wide ? kWideNT : (B <= 16 ? 1 : (B <= 32 ? 2 : 4));
  p.T = wide             ? kWideTiles
        : p.pad          ? kPadTiles
        : mm_one_pair(W) ? pair_tiles_for(p.NT)
                         : tiles_for(p.NT, W->codes_layout == RQ_CODES_PACKED10 ? 3 : 2);
  p.NBT = (B + 16 * p.NT - 1) / (16 * p.NT);
  p.Bp = p.NBT * 16 * p.NT;
  const int64_t slab = (int64_t)(p.pad ? kPadWaves : kMmWaves) * p.T * 16;   // rows per workgroup
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
  p.lds = wide              ? (size_t)2 * kWideSlotBytes
          : p.pad           ? (size_t)2 * kPadSlotBytes
          : !mm_one_pair(W) ? (size_t)2 * (4 * (size_t)W->K + (size_t)kParts * 4 * 16 * p.NT) * 16
          : pair3_fits(W)   ? (size_t)3 * kPair3SlotBytes
                            : 2 * pair_slot_bytes(W);
  return p;
}

static size_t split_bytes(const rq_matrix* W, const MmPlan& p) { return (size_t)kParts * W->M * p.Bp * 16; }

// The front of the workspace: the split h, then (mm_pad_kernel) the padded codebooks [NP][K] at 256 bytes.
size_t mm_hp_bytes(const rq_matrix* W, const MmPlan& p) {
  const size_t hp = split_bytes(W, p);
  return p.pad ? (hp + 255) / 256 * 256 + (size_t)W->L * W->M * W->K * 16 : hp;
}

hipError_t launch_mm_logits(const rq_matrix* W, const MmPlan& p, const float* h, int B, void* hp, float* partial,
                            float* out, float softcap, uint64_t* block_keys, hipStream_t stream) {
  const int64_t n = (int64_t)W->M * p.Bp;
  const int64_t n_cw = p.pad ? (int64_t)W->L * W->M * W->K : 0;
  u32x4* cbp = p.pad ? reinterpret_cast<u32x4*>(static_cast<char*>(hp) + (split_bytes(W, p) + 255) / 256 * 256) : nullptr;
  hipLaunchKernelGGL(split_h_kernel, dim3((unsigned)((n + n_cw + 255) / 256)), dim3(256), 0, stream, h, B, W->D, W->M,
                     W->d, p.Bp, static_cast<u32x4*>(hp), static_cast<const uint16_t*>(W->codebooks), n_cw, cbp);
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
  a.cb_bytes = (uint32_t)std::min<size_t>(cb_bytes(W), 0xffffffffu);
  a.hp_bytes = (uint32_t)std::min<size_t>(split_bytes(W, p), 0xffffffffu);
  a.cbp = cbp;
  a.cbp_bytes = (uint32_t)std::min<size_t>((size_t)n_cw * 16, 0xffffffffu);
  hipEvent_t before, after;
  take_stage_events(&before, &after);
  if (before && (e = hipEventRecord(before, stream)) != hipSuccess) return e;
  e = p.pad                                     ? launch_pad(a, p, stream)
      : p.NT == kWideNT                         ? launch_wide(a, p, W->d, stream)
      : mm_one_pair(W)                          ? launch_pair(a, p, W->d, stream)
      : W->codes_layout == RQ_CODES_PACKED10 ? launch_nsub<3>(a, p, W->d, stream)
                                             : launch_nsub<2>(a, p, W->d, stream);
  if (e != hipSuccess) return e;
  if (after) e = hipEventRecord(after, stream);
  return e;
}

}  // namespace rq
