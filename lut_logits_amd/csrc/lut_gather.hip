// lut_gather.hip -- lookup+sum over the code stream with the logits epilogue
// fused in, and the top-k selection.
//
//   z[b][r] = sum_{l<L} sum_{m<M} LUT[l][m][codes[r][l][m]][b]
//   out[b][r] = softcap * tanh(z / softcap)  (or z),   argmax[b] = first max
//
// (Gemma-2-2B runtime-compression page, LUT-serving paragraph: output logits
// by lookup+sum in place of a full matmul, handed to Gemma-2's softcap.)
//
// Design for gfx950:
//  * The table of one activation (L*M*K entries, 3 MiB in fp32 at Gemma
//    shapes) is far larger than a CU's 160 KB of LDS. It is cut into chunks of
//    P (level, subspace) pairs; a workgroup stages one chunk in LDS with
//    coalesced 16-byte copies and streams the codes of its row slab against
//    it. The pairs are split into G groups of consecutive chunks; a workgroup
//    owns one (group, slab, batch tile).
//  * One lane owns one row (for 16-wide batch tiles a quad of lanes owns one
//    row and each lane 4 batch entries, so one lookup is one contiguous 64-byte
//    LDS read per quad). Codes are read 16 bytes (8 consecutive pairs) per
//    row and load; in the blocked layout consecutive rows are adjacent, so a
//    wave-wide load is one contiguous 1 KB run. The next block is loaded while
//    the lookups of the current one run, across chunk switches too, so
//    2*NSTEP 16-byte loads per lane are in flight -- enough bytes in flight
//    (tens of MB chip-wide) to cover HBM latency at full bandwidth.
//  * Finishing: with G == 1 the gather kernel applies the softcap, stores the
//    logits and the best selection key of its slab. With G > 1 it stores
//    partial sums, and a finish kernel adds the G partials of each output in
//    group order (bit-reproducible, no atomics on the sums), applies the
//    softcap and stores the logits and per-block keys. A selection kernel
//    turns the keys into argmax ids. Cross-workgroup hand-offs go through
//    kernel boundaries only: on this multi-XCD part a device-scope fence
//    inside the kernel writes back and invalidates the XCD's L2, which cost
//    several times the whole pass when every workgroup issued one.
//  * The workgroup -> (group, slab) numbering keeps the workgroups of one XCD
//    on the same group of chunks, so that XCD's L2 serves their staging.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>

#include "rq_internal.h"

namespace rq {
namespace {

struct GatherArgs {
  CodeView cv;
  const void* lut;            // [NP][K][B] (fused table build: the fp32 codebooks [NP][K][d])
  const float* act;           // fused table build: the activation vector [D] (with act2: gelu_tanh(act) * act2)
  const float* act2;
  int D, M;                   // fused table build: row width and subspaces
  int64_t rows;
  int NP, K, B;
  int P, chunks, cpg, G, steps, S, NBT;
  int64_t slab_rows;          // rows of a slab (the last one may be shorter)
  float* partial;             // [G][B][rows] (G > 1)
  float* out;                 // [B][rows] or null (G == 1)
  float* out2;                // second matrix of a two-matrix launch: its out
  float softcap;              // <= 0: none
  uint64_t* block_keys;       // [B][S] best selection key per slab, or null (G == 1)
  int tiled;                  // lut is batch-tiled [NBT][NP][K][BT] (launch_tile_lut)
  int xcd_contiguous;         // give each XCD a contiguous range of workgroups (see gather_kernel)
  int mats;                   // host side: 1, or 2 for a two-matrix launch (gridDim.y)
  // gridDim.y == 2: a second matrix of the same shape and plan (cv2, lut2),
  // its partial sums to partial2 (the Gemma MLP's gate and up in one launch)
  CodeView cv2;
  const void* lut2;
  float* partial2;
  // Fused build with pro_partial set: the activation is gelu_tanh(g) * u with
  // g and u summed from partial sums [2][pro_G][pro_rows] (g's, then u's, B = 1)
  // in the finish kernel's order (pro_tpr parts), instead of read from act/act2.
  const float* pro_partial;
  int pro_G, pro_tpr;
  int64_t pro_rows;
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
    if ((((size_t)K * B * sizeof(LutT)) & 15) == 0) {   // chunk starts 16-byte aligned
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(tab);
      const size_t n4 = n * sizeof(LutT) / 16;
      // up to 8 loads per thread in flight before the first LDS write (one
      // round trip per chunk of up to 128 KB)
      size_t i = tid;
      for (; i + 7 * kGatherThreads < n4; i += 8 * kGatherThreads) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s4[i + u * kGatherThreads];
#pragma unroll
        for (int u = 0; u < 8; ++u) d4[i + u * kGatherThreads] = v[u];
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

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Value of one table entry as fp32 (BQ == 1).
template <typename LutT>
__device__ __forceinline__ float lut_value(const LutT* e);
template <>
__device__ __forceinline__ float lut_value<float>(const float* e) { return *e; }
template <>
__device__ __forceinline__ float lut_value<uint16_t>(const uint16_t* e) { return bf16_to_f32(*e); }

// Code t of a row's 16-byte block, by code width CB: 16-bit layouts hold 8
// codes (two per word), RQ_CODES_PACKED10 12 (three 10-bit fields per word),
// RQ_CODES_PACKED8 16 (four bytes per word).
template <int CB>
__device__ __forceinline__ uint32_t code_of(const uint4& w, int t) {
  if (CB == 10) {
    const int wi = t / 3;
    const uint32_t word = wi == 0 ? w.x : wi == 1 ? w.y : wi == 2 ? w.z : w.w;
    return (word >> (10 * (t - 3 * wi))) & 0x3ffu;
  }
  if (CB == 8) {
    const uint32_t word = (t >> 2) == 0 ? w.x : (t >> 2) == 1 ? w.y : (t >> 2) == 2 ? w.z : w.w;
    return (word >> (8 * (t & 3))) & 0xffu;
  }
  const uint32_t word = (t >> 1) == 0 ? w.x : (t >> 1) == 1 ? w.y : (t >> 1) == 2 ? w.z : w.w;
  return (t & 1) ? (word >> 16) : (word & 0xffffu);
}

// REG: the table slice of one chunk is contiguous and at most reg_stage()
// 16-byte words per thread (B == BT), so the next chunk is loaded into
// registers while the current one is in use and only written to LDS at the
// switch -- its HBM/L2 latency is hidden behind a whole chunk. Eight words
// (128 KB chunks) for the fused build and batch tiles; six (96 KB, the
// largest single-vector chunk the planner makes) for the single-vector
// table, whose lookup loop needs the registers.
constexpr int kRegStage = 8;
constexpr int reg_stage(int BT, int FD) { return (FD == 0 && BT == 1) ? 6 : kRegStage; }
// Pairs whose lookups are issued together in a block that lies wholly in range
// (fewer for lanes holding four rows).
constexpr int kLookGroup = 4;

// Cache policy bits of the code-stream loads: the default (non-temporal
// policies measured no faster).
constexpr int kCodeCachePolicy = 0;

// RS 16-byte words of a chunk held in registers. A native vector type keeps
// the copies first-class values (HIP's uint4 struct is copied through memory).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int RS>
struct ChunkRegs {
  u32x4 w[RS];
};
// Word i of a chunk whose last word is `last`: words past the end repeat the
// last one. With PAIRS (a codeword spread over two words, fused d = 8) an
// even index clamps to last - 1 and an odd one to last, so the two lanes that
// hold one codeword's halves keep holding one codeword (last is odd then).
template <bool PAIRS>
__device__ __forceinline__ int clamp_word(int i, int last) {
  return PAIRS ? min(i, last - 1 + (i & 1)) : min(i, last);
}
template <int RS, bool PAIRS = false>
__device__ __forceinline__ void chunk_to_regs(ChunkRegs<RS>& r, const u32x4* __restrict__ src, int tid, int last) {
#pragma unroll
  for (int i = 0; i < RS; ++i) r.w[i] = src[clamp_word<PAIRS>(tid + i * kGatherThreads, last)];
}
// Fused table build (B == 1, fp32 codebooks, subspace width FD in {1, 2, 4, 8}):
// the registers hold codebook words instead of table words; each word is 4/FD
// codewords of one pair (FD = 8: half a codeword), whose table entries
//     LUT[p][k] = sum_{j<FD} act[m*FD + j] * C[p][k][j]      (m = p mod M)
// are computed with the same fmaf chain as the table-build kernel and written
// to LDS. act sits in LDS after the chunk.
template <int FD>
__device__ __forceinline__ void fused_word(const u32x4 w, int i, float* tab, const float* act_s, int pl0, int K) {
  if constexpr (FD == 8) {
    // Words 2e and 2e+1 (codeword e) sit in adjacent lanes: the even lane runs
    // the chain over values 0..3, hands its sum to the odd lane, which runs it
    // on over values 4..7 -- one sequential chain, as in the table build.
    const int e = i >> 1;
    const int pl = pl0 + e / K;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t bits = w[j];
      acc = fmaf(act_s[pl * 8 + j], __uint_as_float(bits), acc);
    }
    acc = __shfl_xor(acc, 1, 64);
    if (i & 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t bits = w[j];
        acc = fmaf(act_s[pl * 8 + 4 + j], __uint_as_float(bits), acc);
      }
      tab[e] = acc;
    }
    return;
  }
  constexpr int EPW = 4 / (FD == 8 ? 4 : FD);
  const int e0 = i * EPW;                 // entry index within the chunk: (pair - p0) * K + k
  const int pl = pl0 + e0 / K;            // the pair's index within the group (its activation slice)
  float v[EPW];
#pragma unroll
  for (int t = 0; t < EPW; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < FD; ++j) {
      // element to a scalar first: hipcc folds __builtin_bit_cast of a vector
      // element to element 0
      const uint32_t bits = w[t * FD + j];
      acc = fmaf(act_s[pl * FD + j], __uint_as_float(bits), acc);
    }
    v[t] = acc;
  }
  if (EPW == 4) *reinterpret_cast<float4*>(tab + e0) = make_float4(v[0], v[1 % EPW], v[2 % EPW], v[3 % EPW]);
  else if (EPW == 2) *reinterpret_cast<float2*>(tab + e0) = make_float2(v[0], v[1 % EPW]);
  else tab[e0] = v[0];
}
template <int FD, int RS>
__device__ __forceinline__ void regs_to_lds_fused(const ChunkRegs<RS>& r, float* tab, const float* act_s, int tid,
                                                  int last, int pl0, int K) {
#pragma unroll
  for (int i = 0; i < RS; ++i)
    fused_word<FD>(r.w[i], clamp_word<FD == 8>(tid + i * kGatherThreads, last), tab, act_s, pl0, K);
}

template <int RS>
__device__ __forceinline__ void regs_to_lds(const ChunkRegs<RS>& r, u32x4* dst, int tid, int last) {
#pragma unroll
  for (int i = 0; i < RS; ++i) dst[min(tid + i * kGatherThreads, last)] = r.w[i];
}

// One 1024-thread workgroup per CU (its LDS chunk fills the CU), i.e. four
// waves per SIMD: the register budget is 128 VGPRs, stated explicitly so the
// compiler does not trade registers for an occupancy the LDS cannot reach.
// FD > 0: fused table build (see fused_word); requires LutT float, BT 1, REG.
// CB: code width of the layout (16, 10 for RQ_CODES_PACKED10, 8 for
// RQ_CODES_PACKED8): 8, 12 or 16 pairs per 16-byte block.
// RSET: row sets per workgroup. Each staged chunk serves RSET sets of
// steps x RPS rows one after the other (the code registers are reused, the
// sums of every set stay in registers), so a slab of RSET times the rows
// stages each chunk once: with several batch tiles the table restaging, not
// the code stream, bounds the pass.
// PIPE (one code block per chunk, K <= 1024; the fused build with FD = 2, or
// an fp32 table for one vector): see the pipelined loop below.
template <typename LutT, int BT, int NSTEP, bool REG, int FD = 0, int CB = 16, int RSET = 1, bool PIPE = false>
__global__ __launch_bounds__(kGatherThreads) __attribute__((amdgpu_waves_per_eu(1, 4)))
void gather_kernel(GatherArgs a) {
  constexpr int PPB = CB == 10 ? 12 : (CB == 8 ? 16 : 8);   // pairs per code block
  static_assert(FD == 0 || (BT == 1 && REG && sizeof(LutT) == 4 && (4 % FD == 0 || FD == 8)),
                "fused build: fp32, B=1, FD in {1, 2, 4, 8}");
  static_assert(!PIPE || ((FD == 2 || (FD == 0 && BT == 1 && sizeof(LutT) == 4)) && RSET == 1 && CB != 8),
                "pipelined kernel: fused build at d = 2 or an fp32 table for one vector; 16- or 10-bit codes");
  constexpr int QL = (BT >= 16) ? 4 : 1;   // lanes per row
  constexpr int BQ = BT / QL;              // batch entries per lane
  constexpr int RPS = kGatherThreads / QL; // rows per step
  extern __shared__ __align__(16) unsigned char smem[];
  LutT* tab = reinterpret_cast<LutT*>(smem);
  __shared__ unsigned long long s_keys[BT];

  // XCD-aware numbering (when the host asks for it): workgroups are dealt to
  // the 8 XCDs round robin in dispatch order, so give each XCD a contiguous
  // range of logical ids (the same chunk groups, whose tables then stay in
  // that XCD's L2). With N workgroups the first N % 8 XCDs get one more than
  // the others. With two matrices the logical ids run over both.
  const int total = a.G * a.S * a.NBT;
  const int all = total * (int)gridDim.y;
  const int idx = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  const int xcd = idx & 7;
  int li = a.xcd_contiguous ? xcd * (all >> 3) + min(xcd, all & 7) + (idx >> 3) : idx;
  const bool second = li >= total;   // uniform: the second matrix of a two-matrix launch
  if (second) li -= total;
  const CodeView cv = second ? a.cv2 : a.cv;
  float* const partial = second ? a.partial2 : a.partial;
  const int bt = li % a.NBT;
  li /= a.NBT;
  const int s = li % a.S;
  const int g = li / a.S;

  const int tid = threadIdx.x;
  const int rq = tid % QL;
  const int rl = tid / QL;
  const int b0 = bt * BT;
  const int64_t slab_lo = (int64_t)s * a.slab_rows;
  const int64_t slab_hi = min(slab_lo + a.slab_rows, a.rows);   // this slab's rows: [slab_lo, slab_hi)
  const int64_t row0 = slab_lo + rl;

  float acc[RSET][NSTEP][BQ];
#pragma unroll
  for (int rs = 0; rs < RSET; ++rs)
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int i = 0; i < BQ; ++i) acc[rs][st][i] = 0.0f;

  // Byte offsets of this lane's rows inside one block of codes. Rows past the
  // end read the last row (in bounds); their sums are never stored.
  // Steps beyond the slab repeat step 0's row, so every load is issued
  // unconditionally (a fixed number of loads per block keeps the wait counts
  // exact) without touching other slabs' codes.
  uint32_t roff[RSET][NSTEP];
#pragma unroll
  for (int rs = 0; rs < RSET; ++rs)
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int64_t r = min(row0 + (int64_t)(rs * a.steps + (st < a.steps ? st : 0)) * RPS, slab_hi - 1);
      roff[rs][st] = (uint32_t)(r * cv.s_row * 2);
    }
  // The code stream is read with buffer loads: a scalar resource, the row
  // offset in a VGPR and the block offset in an SGPR, so the hot loop holds no
  // 64-bit per-lane addresses. (The host keeps the code array below 4 GiB.)
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)cv.codes, (short)0, (int)0xffffffffu, 0x00020000);
  // A resource with no records: loads through it are out of range, return
  // zeros and touch no memory. The loads that run ahead past a group's last
  // block use it, so they keep the fixed count per block (and the exact wait
  // counts) without fetching that block again.
  const __amdgpu_buffer_rsrc_t none_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)cv.codes, (short)0, 0, 0x00020000);
  const uint32_t blk_bytes = (uint32_t)(cv.s_blk * 2);
  const int steps = a.steps;

  // batch-tiled table: this tile's [NP][K][BT] slice is contiguous
  const LutT* lut = static_cast<const LutT*>(second ? a.lut2 : a.lut) + (a.tiled ? (size_t)bt * a.NP * a.K * BT : 0);
  // This group's chunks [c_begin, c_end): cpg each, the last group the rest;
  // PIPE splits them evenly instead (cpg or cpg - 1 each), so that any number
  // of groups can be had. Its pairs are [pa, pb).
  const int c_begin = PIPE ? (int)((int64_t)g * a.chunks / a.G) : g * a.cpg;
  const int c_end = PIPE ? (int)((int64_t)(g + 1) * a.chunks / a.G) : min(a.chunks, c_begin + a.cpg);
  const int pa = c_begin * a.P;
  const int pb = min(a.NP, c_end * a.P);

  // 16 bytes = the codes of PPB consecutive pairs of one row. Two register
  // buffers alternate: while one block is looked up, the next one loads into
  // the other buffer (no register copy, so no wait on the load in flight).
  // live == false (uniform): a block past the group's end, whose codes are never looked up.
  auto load_block = [&](uint4 (&dst)[NSTEP], int q, int rs = 0, bool live = true) {
    const uint32_t boff = (uint32_t)q * blk_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = live ? code_rsrc : none_rsrc;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)roff[rs][st], (int)boff, kCodeCachePolicy);
      dst[st] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // Lookups of the pairs of block q that lie in [lo, hi), against the chunk staged at p0.
  auto lookup_block = [&](const uint4 (&w)[NSTEP], int q, int lo, int hi, int p0, int rs = 0) {
    // (not for bf16 tables at 4 rows per lane: that instance would spill)
    if (BQ == 1 && (sizeof(LutT) == 4 || NSTEP < 4) && PPB * q >= lo && PPB * q + PPB <= hi) {
      // The whole block is in range (uniform): the lookups of kLookGroup pairs
      // of every step are issued before any is added, so that many LDS reads
      // are in flight per wave. Each step still adds its pairs in order.
      constexpr int LG = NSTEP < 4 ? kLookGroup : kLookGroup / 2;   // 4 rows per lane: 2 pairs (registers)
      static_assert(PPB % LG == 0, "pairs per block");
#pragma unroll
      for (int t0 = 0; t0 < PPB; t0 += LG) {
        float v[LG][NSTEP];
#pragma unroll
        for (int t = 0; t < LG; ++t) {
          const LutT* base = tab + (size_t)(PPB * q + t0 + t - p0) * a.K * BT + rq * BQ;
#pragma unroll
          for (int st = 0; st < NSTEP; ++st) v[t][st] = lut_value(base + code_of<CB>(w[st], t0 + t) * BT);
        }
#pragma unroll
        for (int t = 0; t < LG; ++t)
#pragma unroll
          for (int st = 0; st < NSTEP; ++st) acc[rs][st][0] += v[t][st];
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < PPB; ++t) {
      const int p = PPB * q + t;               // uniform
      if (p < lo || p >= hi) continue;
      const LutT* base = tab + (size_t)(p - p0) * a.K * BT + rq * BQ;
      if (BQ == 1) {
        // issue every lookup of this pair before adding, so the LDS reads overlap
        float v[NSTEP];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) v[st] = lut_value(base + code_of<CB>(w[st], t) * BT);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) acc[rs][st][0] += v[st];
      } else {
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) lookup_add<LutT, BQ>(acc[rs][st], base + code_of<CB>(w[st], t) * BT);
      }
    }
  };
  uint4 wa[NSTEP], wb[NSTEP];
  constexpr int RS = reg_stage(BT, FD);
  ChunkRegs<RS> nxt;
  const u32x4* lut4 = reinterpret_cast<const u32x4*>(lut);
  // REG: 16-byte words per pair (of the table, or with FD of the codebook)
  const int words_per_pair = FD ? a.K * FD / 4 : a.K * BT * (int)sizeof(LutT) / 16;
  // REG: chunk c's words go to registers with a fixed count of unconditional
  // loads (clamped to the last word of the chunk).
  // PIPE: chunk i (of this group's nc) has its codebook words in cbA or cbB and
  // its code block in wA or wB (by the parity of i). Chunk i+2's words and
  // block are issued right after chunk i's build and lookups have used those
  // registers, so at any time the loads of the next two chunks are in flight,
  // and every wait is for loads issued before the ones still flying (waits
  // count loads in issue order): the codebook staging and the code stream
  // overlap. (One register buffer, as below, makes each chunk's lookups wait
  // for the next chunk's codebook, issued just before its codes.)
  // words of a chunk of PPB pairs at K <= 1024: 8 bytes of codebook per entry at d = 2, 4 of table
  constexpr int RSP = PIPE ? (FD ? PPB * FD / 4 : PPB / 4) : 1;
  ChunkRegs<RSP> cbA, cbB;
  uint4 wA[NSTEP], wB[NSTEP];
  const int nc = c_end - c_begin;
  // chunk i's first pair is a code block's first: P == PPB, or one chunk of P < PPB pairs
  auto blk_of = [&](int i) { return (c_begin + min(i, nc - 1)) * a.P / PPB; };
  auto pipe_words = [&](ChunkRegs<RSP>& cb, int i) {
    const int c = c_begin + min(i, nc - 1);   // past the group's end: its last chunk again
    const int n4 = min(a.P, a.NP - c * a.P) * words_per_pair;
    chunk_to_regs<RSP>(cb, lut4 + (size_t)c * a.P * words_per_pair, tid, n4 - 1);
  };
  if constexpr (PIPE) {
    // in this order, not interleaved: the loop's waits count on it
    pipe_words(cbA, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_block(wA, blk_of(0));
    __builtin_amdgcn_sched_barrier(0);
    pipe_words(cbB, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_block(wB, blk_of(1));
    __builtin_amdgcn_sched_barrier(0);
  } else if (REG) {
    const int n4 = min(a.P, a.NP - c_begin * a.P) * words_per_pair;
    chunk_to_regs<RS, FD == 8>(nxt, lut4 + (size_t)c_begin * a.P * words_per_pair, tid, n4 - 1);
  }
  // FD: the activation slices of this group's pairs [pa, pb) go to LDS after
  // the chunk, once (pair p uses elements (p % M)*FD .. +FD of the vector).
  // Their loads follow the first chunk's, so the two latencies overlap.
  float* act_s = reinterpret_cast<float*>(smem + (size_t)(PIPE ? 2 : 1) * a.P * a.K * sizeof(float));   // PIPE: two tables
  if (FD && a.pro_partial) {
    // g and u of each element: pro_tpr parts per element and matrix, part t
    // adding groups t, t+pro_tpr, ... in order, then the parts in order -- the
    // finish kernel's arithmetic, so the activation is bit-identical to
    // finishing g and u first.
    const int E = (pb - pa) * FD;
    const int TPR = a.pro_tpr;
    float* pro_s = act_s + (size_t)min(a.cpg * a.P, a.NP) * FD;   // [2][E][TPR]
    for (int task = tid; task < 2 * E * TPR; task += kGatherThreads) {
      const int mat = task / (E * TPR);
      const int rem = task - mat * E * TPR;
      const int i = rem / TPR;
      const int part = rem - i * TPR;
      const int p = pa + i / FD;
      const int src = (p % a.M) * FD + (i - (p - pa) * FD);
      const float* col = a.pro_partial + ((size_t)mat * a.pro_G) * a.pro_rows + src;
      float z = 0.0f;
      int gg = part;
      for (; gg + 3 * TPR < a.pro_G; gg += 4 * TPR) {
        const float v0 = col[(size_t)gg * a.pro_rows], v1 = col[(size_t)(gg + TPR) * a.pro_rows];
        const float v2 = col[(size_t)(gg + 2 * TPR) * a.pro_rows], v3 = col[(size_t)(gg + 3 * TPR) * a.pro_rows];
        z += v0; z += v1; z += v2; z += v3;
      }
      for (; gg < a.pro_G; gg += TPR) z += col[(size_t)gg * a.pro_rows];
      pro_s[(size_t)(mat * E + i) * TPR + part] = z;
    }
    __syncthreads();
    for (int i = tid; i < E; i += kGatherThreads) {
      float gv = pro_s[(size_t)i * TPR], uv = pro_s[(size_t)(E + i) * TPR];
      for (int t = 1; t < TPR; ++t) {
        gv += pro_s[(size_t)i * TPR + t];
        uv += pro_s[(size_t)(E + i) * TPR + t];
      }
      act_s[i] = gelu_tanh(gv) * uv;
    }
  } else if (FD) {
    for (int i = tid; i < (pb - pa) * FD; i += kGatherThreads) {
      const int p = pa + i / (FD ? FD : 1);
      const int src = (p % a.M) * FD + (i - (p - pa) * FD);
      act_s[i] = a.act2 ? gelu_tanh(a.act[src]) * a.act2[src] : a.act[src];
    }
  }
  // Stage chunk c (uniform): all lookups of the previous chunk are done before
  // LDS is overwritten, and the next chunk starts loading into registers.
  auto switch_chunk = [&](int c) {
    const int p0 = c * a.P;
    const int pc = min(a.P, a.NP - p0);
    __syncthreads();
    if (REG) {
      // words past the chunk were loaded clamped to its last word, so writing
      // them clamped stores that same value again
      if (FD)
        regs_to_lds_fused<FD ? FD : 1, RS>(nxt, reinterpret_cast<float*>(tab), act_s, tid, pc * words_per_pair - 1, p0 - pa,
                                       a.K);
      else
        regs_to_lds(nxt, reinterpret_cast<u32x4*>(tab), tid, pc * words_per_pair - 1);
      const int cn = min(c + 1, c_end - 1);
      const int n4n = min(a.P, a.NP - cn * a.P) * words_per_pair;
      chunk_to_regs<RS, FD == 8>(nxt, lut4 + (size_t)cn * a.P * words_per_pair, tid, n4n - 1);
    } else {
      stage_chunk<LutT, BT>(tab, lut, p0, pc, a.K, a.tiled ? BT : a.B, a.tiled ? 0 : b0);
    }
    __syncthreads();
  };
  // The loads are unconditional (past the group's end they go through the
  // no-record resource and fetch nothing), so the same count is always in flight.
  if constexpr (PIPE) {
    // Chunks in pairs, so each register buffer keeps its role, and two tables
    // in LDS, so one barrier per chunk suffices: chunk i's table is built into
    // table i % 2, which every wave stopped reading before the barrier of chunk
    // i - 1. A step past the group's end rebuilds its last chunk (the same
    // table) and looks nothing up.
    LutT* const tabs[2] = {tab, tab + (size_t)a.P * a.K};
    auto run = [&](ChunkRegs<RSP>& cb, uint4 (&w)[NSTEP], int i, int t) {
      const int ic = min(i, nc - 1);
      const int p0 = (c_begin + ic) * a.P;
      const int pc = min(a.P, a.NP - p0);
      if constexpr (FD != 0)
        regs_to_lds_fused<FD, RSP>(cb, reinterpret_cast<float*>(tabs[t]), act_s, tid, pc * words_per_pair - 1,
                                   p0 - pa, a.K);
      else
        regs_to_lds(cb, reinterpret_cast<u32x4*>(tabs[t]), tid, pc * words_per_pair - 1);
      __syncthreads();
      pipe_words(cb, i + 2);
      tab = tabs[t];   // the table lookup_block reads
      lookup_block(w, i < nc ? blk_of(i) : (c_end * a.P + PPB - 1) / PPB, pa, pb, p0);
      load_block(w, blk_of(i + 2), 0, i + 2 < nc);
    };
    __syncthreads();   // the activation slices are in LDS
    for (int i = 0; i < nc; i += 2) {
      run(cbA, wA, i, 0);
      run(cbB, wB, i + 1, 1);
    }
  } else if (RSET == 1 && BT == 1 && a.P % PPB == 0) {
    // Chunks hold whole code blocks: one flat loop over the group's blocks, so
    // the next block's codes are already in flight across a chunk switch.
    // (Batch tiles keep the per-chunk loop: both loops in one kernel spill.)
    const int bpc = a.P / PPB;
    const int qa = pa / PPB, qb = (pb + PPB - 1) / PPB;
    load_block(wa, qa);
    for (int q = qa; q < qb; q += 2) {
      if ((q - qa) % bpc == 0) switch_chunk(c_begin + (q - qa) / bpc);
      load_block(wb, min(q + 1, qb - 1), 0, q + 1 < qb);
      lookup_block(wa, q, pa, pb, (c_begin + (q - qa) / bpc) * a.P);
      if (q + 1 < qb && (q + 1 - qa) % bpc == 0) switch_chunk(c_begin + (q + 1 - qa) / bpc);
      load_block(wa, min(q + 2, qb - 1), 0, q + 2 < qb);
      lookup_block(wb, q + 1, pa, pb, (c_begin + (q + 1 - qa) / bpc) * a.P);
    }
  } else {
    for (int c = c_begin; c < c_end; ++c) {
      const int p0 = c * a.P;
      const int pc = min(a.P, a.NP - p0);
      const int lo = max(p0, pa), hi = min(p0 + pc, pb);
      const int q0 = lo / PPB, q1 = (hi + PPB - 1) / PPB;
      load_block(wa, q0);
      switch_chunk(c);
#pragma unroll
      for (int rs = 0; rs < RSET; ++rs) {
        if (rs > 0) load_block(wa, q0, rs);
        for (int q = q0; q < q1; q += 2) {
          load_block(wb, min(q + 1, q1 - 1), rs, q + 1 < q1);
          lookup_block(wa, q, lo, hi, p0, rs);
          load_block(wa, min(q + 2, q1 - 1), rs, q + 2 < q1);
          lookup_block(wb, q + 1, lo, hi, p0, rs);
        }
      }
    }
  }
  // ---- G > 1: store the partial sums; the finish kernel adds them in group order
  if (a.G > 1) {
#pragma unroll
    for (int rs = 0; rs < RSET; ++rs)
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int64_t r = row0 + (int64_t)(rs * steps + st) * RPS;
        if (st >= steps || r >= slab_hi) continue;
#pragma unroll
        for (int i = 0; i < BQ; ++i) {
          const int b = b0 + rq * BQ + i;
          if (b < a.B) partial[((size_t)g * a.B + b) * a.rows + r] = acc[rs][st][i];
        }
      }
    return;
  }

  // ---- G == 1: the sums are final: softcap, store, best selection key per slab
  unsigned long long kbest[BQ];
#pragma unroll
  for (int i = 0; i < BQ; ++i) kbest[i] = 0ull;
#pragma unroll
  for (int rs = 0; rs < RSET; ++rs)
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int64_t r = row0 + (int64_t)(rs * steps + st) * RPS;
    if (st >= steps || r >= slab_hi) continue;
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int b = b0 + rq * BQ + i;
      if (b >= a.B) continue;
      const float z = acc[rs][st][i];
      const float v = a.softcap > 0.0f ? a.softcap * tanhf(z / a.softcap) : z;
      float* const outp = second ? a.out2 : a.out;
      if (outp) outp[(size_t)b * a.rows + r] = v;
      kbest[i] = umax64(kbest[i], select_key(v, (uint32_t)r));
    }
  }
  if (!a.block_keys) return;
  if (tid < BT) s_keys[tid] = 0ull;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BQ; ++i)
    if (kbest[i]) atomicMax(&s_keys[rq * BQ + i], kbest[i]);   // LDS atomics, this workgroup only
  __syncthreads();
  if (tid < BT && b0 + tid < a.B) a.block_keys[(size_t)(b0 + tid) * a.S + s] = s_keys[tid];
}

template <typename LutT, int BT, int NSTEP, int FD = 0, int CB = 16, int RSET = 1, bool PIPE = false>
hipError_t launch_gather_typed(const GatherArgs& a, const GatherPlan& plan, hipStream_t stream) {
  if (plan.steps < 1 || plan.steps > NSTEP) return hipErrorInvalidValue;   // a lane holds NSTEP rows at most
  if (plan.rset != RSET) return hipErrorInvalidValue;                       // slabs are sized for this many row sets
  if (PIPE) {
    // one code block per chunk, and a chunk's codebook words fit the two register buffers
    constexpr int PPB = CB == 10 ? 12 : 8;
    if (!(plan.P == PPB || (plan.chunks == 1 && plan.P < PPB)) || a.K > 1024 ||
        ((size_t)a.K * (FD ? FD : BT) * sizeof(LutT)) % 16 != 0)
      return hipErrorInvalidValue;
  }
  const size_t chunk_bytes = (size_t)plan.P * a.K * BT * sizeof(LutT);
  const bool reg = (a.B == BT || a.tiled) && chunk_bytes % 16 == 0 &&
                   chunk_bytes <= (size_t)reg_stage(BT, FD) * 16 * kGatherThreads &&
                   ((size_t)a.K * BT * sizeof(LutT)) % 16 == 0;
  void (*kern)(GatherArgs);
  if constexpr (FD != 0 || PIPE)
    kern = gather_kernel<LutT, BT, NSTEP, true, FD, CB, 1, PIPE>;
  else
    kern = reg ? gather_kernel<LutT, BT, NSTEP, true, 0, CB, RSET> : gather_kernel<LutT, BT, NSTEP, false, 0, CB, RSET>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
  if (e != hipSuccess) return e;
  hipEvent_t before, after;
  take_stage_events(&before, &after);
  if (before || after) {
    // the events take the start and end of this kernel's own dispatch
    hipExtLaunchKernelGGL(kern, dim3((unsigned)plan.wgs(), (unsigned)a.mats), dim3(kGatherThreads), plan.lds, stream,
                          before, after, 0, a);
  } else {
    hipLaunchKernelGGL(kern, dim3((unsigned)plan.wgs(), (unsigned)a.mats), dim3(kGatherThreads), plan.lds, stream, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k

constexpr int kTopkThreads = 256;

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

// The k best selection keys of each 1024-row block of the logits, in any order
// (the merge sorts them). Selection keys are distinct (the row index is part
// of every key), so the block's k-th largest key T splits it exactly: the k
// keys >= T. T is found most significant byte first: a 256-bin histogram of
// the keys that agree with the bytes fixed so far, then the bin where the
// count from the top reaches the number still needed; it stops as soon as the
// keys that agree with the prefix are exactly the ones still needed (for
// random logits after two or three bytes). Rows past the end carry key 0,
// below every real key: a block with no more real keys than k gives all of
// them and zeros.
__global__ __launch_bounds__(kTopkThreads) void topk_block_kernel(const float* __restrict__ logits, int64_t rows,
                                                                  int topk, uint64_t* __restrict__ cand) {
  constexpr int KPT = kEpiRowsPerBlock / kTopkThreads;   // keys per thread
  static_assert(kTopkThreads >= 256, "one thread per histogram bin");
  __shared__ unsigned int hist[256];
  __shared__ unsigned int s_digit, s_above, s_out;
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t r0 = (int64_t)blk * kEpiRowsPerBlock;
  const int n_real = (int)min<int64_t>(kEpiRowsPerBlock, rows - r0);
  uint64_t* dst = cand + ((size_t)b * gridDim.x + blk) * topk;
  uint64_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int local = tid + j * kTopkThreads;
    key[j] = local < n_real ? select_key(logits[(size_t)b * rows + r0 + local], (uint32_t)(r0 + local)) : 0ull;
  }
  if (n_real <= topk) {   // uniform
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int local = tid + j * kTopkThreads;
      if (local < topk) dst[local] = key[j];
    }
    return;
  }
  if (tid == 0) s_out = 0u;
  uint64_t prefix = 0ull, pmask = 0ull;
  unsigned int need = (unsigned int)topk;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if ((key[j] & pmask) == prefix) atomicAdd(&hist[(unsigned int)(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255-4l .. 252-4l; an exclusive scan from the top
      unsigned int h[4], lsum = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * tid - i];
        lsum += h[i];
      }
      unsigned int incl = lsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned int t = (unsigned int)__shfl_up((int)incl, o, 64);
        if (tid >= o) incl += t;
      }
      unsigned int cum = incl - lsum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < need && need <= cum + h[i]) {
          s_digit = 255u - 4u * tid - i;
          s_above = cum;
        }
        cum += h[i];
      }
    }
    __syncthreads();
    const unsigned int d = s_digit;
    need -= s_above;
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)0xff << shift;
    const bool done = hist[d] == need;   // uniform: read from LDS
    __syncthreads();                      // before the next byte clears the histogram
    if (done) break;
  }
  // the keys whose fixed bytes are at or above the prefix: exactly k of them
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((key[j] & pmask) >= prefix) dst[atomicAdd(&s_out, 1u)] = key[j];
}

constexpr int kFinishThreads = 1024;

// z = sum of the G partial sums of each output in a fixed order, then the
// softcap; the best selection key of each block of rows.
// TPR "parts" per row: part t adds groups t, t+TPR, t+2*TPR, ... in order and
// the parts are then added in order 0..TPR-1 (fixed order, so bit-reproducible).
// A block covers kFinishThreads/TPR rows; each wave reads 64 consecutive rows of
// one group (coalesced). Many groups over few rows (MLP shapes) need TPR > 1 to
// keep enough loads in flight; TPR == 1 is a plain sum in group order.
template <int TPR>
__global__ __launch_bounds__(kFinishThreads) void finish_kernel(const float* __restrict__ partial, int G, int B,
                                                                int64_t rows, float softcap, float* __restrict__ out,
                                                                uint64_t* __restrict__ block_keys) {
  constexpr int RPB = kFinishThreads / TPR;
  __shared__ unsigned long long s_best;
  __shared__ float s_part[TPR > 1 ? TPR : 1][TPR > 1 ? RPB : 1];
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int part = threadIdx.x / RPB;
  const int local = threadIdx.x - part * RPB;
  const int64_t r = (int64_t)blk * RPB + local;
  if (threadIdx.x == 0) s_best = 0ull;
  float z = 0.0f;
  if (r < rows) {
    const float* src = partial + (size_t)b * rows + r;
    const size_t gstride = (size_t)B * rows;
    int g = part;
    for (; g + 3 * TPR < G; g += 4 * TPR) {   // four loads in flight, added in order
      const float v0 = src[(size_t)g * gstride], v1 = src[(size_t)(g + TPR) * gstride];
      const float v2 = src[(size_t)(g + 2 * TPR) * gstride], v3 = src[(size_t)(g + 3 * TPR) * gstride];
      z += v0; z += v1; z += v2; z += v3;
    }
    for (; g < G; g += TPR) z += src[(size_t)g * gstride];
  }
  if (TPR > 1) {
    s_part[part][local] = z;
    __syncthreads();
    if (part == 0) {
      z = s_part[0][local];
#pragma unroll
      for (int t = 1; t < TPR; ++t) z += s_part[t][local];
    }
  }
  unsigned long long key = 0ull;
  if (part == 0 && r < rows) {
    const float v = softcap > 0.0f ? softcap * tanhf(z / softcap) : z;
    if (out) out[(size_t)b * rows + r] = v;
    key = select_key(v, (uint32_t)r);
  }
  if (!block_keys) return;   // uniform: a kernel argument
  __syncthreads();
  const uint64_t w = wave_max_u64(key);
  if ((threadIdx.x & 63) == 0) atomicMax(&s_best, (unsigned long long)w);
  __syncthreads();
  if (threadIdx.x == 0) block_keys[(size_t)b * gridDim.x + blk] = s_best;
}

// finish_kernel<1> for many batch vectors (B >= 8: grid.y alone fills the
// chip): the same 1024-row blocks and keys, with 256 threads of 4 rows each,
// so every thread has the loads of four rows in flight. Each row adds its G
// partial sums in group order, as finish_kernel<1> does.
constexpr int kFinish4Threads = 256;
__global__ __launch_bounds__(kFinish4Threads) void finish4_kernel(const float* __restrict__ partial, int G, int B,
                                                                  int64_t rows, float softcap, float* __restrict__ out,
                                                                  uint64_t* __restrict__ block_keys) {
  __shared__ unsigned long long s_best;
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  if (threadIdx.x == 0) s_best = 0ull;
  const float* src = partial + (size_t)b * rows;
  const size_t gstride = (size_t)B * rows;
  int64_t r[4];
  float z[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = (int64_t)blk * kFinishThreads + threadIdx.x + k * kFinish4Threads;
    z[k] = 0.0f;
  }
  for (int g = 0; g < G; ++g) {
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = r[k] < rows ? src[(size_t)g * gstride + r[k]] : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] += v[k];
  }
  unsigned long long key = 0ull;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (r[k] >= rows) continue;
    const float v = softcap > 0.0f ? softcap * tanhf(z[k] / softcap) : z[k];
    if (out) out[(size_t)b * rows + r[k]] = v;
    key = umax64(key, select_key(v, (uint32_t)r[k]));
  }
  if (!block_keys) return;   // uniform: a kernel argument
  __syncthreads();
  const uint64_t w = wave_max_u64(key);
  if ((threadIdx.x & 63) == 0) atomicMax(&s_best, (unsigned long long)w);
  __syncthreads();
  if (threadIdx.x == 0) block_keys[(size_t)b * gridDim.x + blk] = s_best;
}

constexpr int kSelThreads = 1024;
constexpr int kSelCap = 1024;   // the largest k the entry points accept

// Argmax alone: one wave per batch entry takes the largest of the blocks' best
// keys (no LDS, no barrier).
__global__ __launch_bounds__(64) void argmax_kernel(const uint64_t* __restrict__ block_keys, int nkb,
                                                    int32_t* __restrict__ argmax) {
  const int b = blockIdx.x;
  const uint64_t* src = block_keys + (size_t)b * nkb;
  uint64_t best = 0;
  int i = threadIdx.x;
  for (; i + 192 < nkb; i += 256) {   // four loads in flight
    const uint64_t k0 = src[i], k1 = src[i + 64], k2 = src[i + 128], k3 = src[i + 192];
    best = k0 > best ? k0 : best;
    best = k1 > best ? k1 : best;
    best = k2 > best ? k2 : best;
    best = k3 > best ? k3 : best;
  }
  for (; i < nkb; i += 64) best = src[i] > best ? src[i] : best;
  best = wave_max_u64(best);
  if (threadIdx.x == 0) argmax[b] = (int32_t)key_index(best);
}

// Per batch entry: argmax from the blocks' best keys; top-k from the blocks'
// candidates: the k-th largest candidate T by the same most-significant-byte
// radix select as the per-block pass (the candidates stay in global memory,
// read once per byte), then the k candidates >= T sorted in LDS. The k-th
// largest is a real key (rows >= k), so the zero keys of short blocks never
// reach the selection.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const uint64_t* __restrict__ block_keys, int nkb,
                                                             int32_t* __restrict__ argmax, int ncb,
                                                             const uint64_t* __restrict__ cand, int topk,
                                                             int32_t* __restrict__ topk_ids,
                                                             float* __restrict__ topk_vals) {
  __shared__ uint64_t buf[kSelCap];
  __shared__ unsigned long long s_best;
  const int b = blockIdx.x;
  if (argmax) {
    if (threadIdx.x == 0) s_best = 0ull;
    __syncthreads();
    uint64_t best = 0;
    for (int i = threadIdx.x; i < nkb; i += kSelThreads) {
      const uint64_t k = block_keys[(size_t)b * nkb + i];
      best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0) atomicMax(&s_best, (unsigned long long)best);
    __syncthreads();
    if (threadIdx.x == 0) argmax[b] = (int32_t)key_index(s_best);
  }
  if (topk <= 0) return;
  const uint64_t* src = cand + (size_t)b * ncb * topk;
  const size_t total = (size_t)ncb * topk;
  __shared__ unsigned int hist[256];
  __shared__ unsigned int s_digit, s_above, s_out;
  const int tid = threadIdx.x;
  if (tid == 0) s_out = 0u;
  uint64_t prefix = 0ull, pmask = 0ull;
  unsigned int need = (unsigned int)topk;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (size_t i = tid; i < total; i += kSelThreads) {
      const uint64_t k = src[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(unsigned int)(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      unsigned int h[4], lsum = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * tid - i];
        lsum += h[i];
      }
      unsigned int incl = lsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned int t = (unsigned int)__shfl_up((int)incl, o, 64);
        if (tid >= o) incl += t;
      }
      unsigned int cum = incl - lsum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < need && need <= cum + h[i]) {
          s_digit = 255u - 4u * tid - i;
          s_above = cum;
        }
        cum += h[i];
      }
    }
    __syncthreads();
    const unsigned int d = s_digit;
    need -= s_above;
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)0xff << shift;
    const bool done = hist[d] == need;   // uniform: read from LDS
    __syncthreads();                      // before the next byte clears the histogram
    if (done) break;
  }
  // the k candidates at or above the threshold, then sorted (value desc, id asc)
  for (size_t i = tid; i < total; i += kSelThreads) {
    const uint64_t k = src[i];
    if ((k & pmask) >= prefix) {
      const unsigned int slot = atomicAdd(&s_out, 1u);
      if (slot < (unsigned int)topk) buf[slot] = k;   // exactly k for distinct nonzero keys
    }
  }
  int n2 = 1;
  while (n2 < topk) n2 <<= 1;
  for (int i = topk + tid; i < n2; i += kSelThreads) buf[i] = 0ull;
  __syncthreads();
  bitonic_sort_desc(buf, n2);
  for (int i = threadIdx.x; i < topk; i += kSelThreads) {
    topk_ids[(size_t)b * topk + i] = (int32_t)key_index(buf[i]);
    if (topk_vals) topk_vals[(size_t)b * topk + i] = key_value(buf[i]);
  }
}

// ------------------------------------------------------------------ planning

int nstep_for(int BT) { return 4; }


}  // namespace

namespace {

// Cost model of one lookup+sum pass, in microseconds, fitted to measurements
// of this kernel on MI355X: the code stream shares ~6.4 TB/s over the active
// CUs; each staged chunk costs a round trip (~2 us) plus its bytes at
// ~150 GB/s per CU (staging is not overlapped with the stream); random 4-byte
// LDS lookups run at ~9 per clock per CU (quad-contiguous 64-byte lookups at
// ~120 B/clock); G > 1 adds the partial-sum traffic and a finish launch.
// pipe: the pipelined fused build, whose staging shares the CU's bandwidth
// with the code stream instead of stalling it (one round trip at the start).
double plan_cost_us(int64_t rows, int NP, int K, int B, int es, int BT, int P, int steps, int G, int cpg,
                    int stage_es, int lane_steps, int mats, bool pipe = false) {
  const int QL = BT >= 16 ? 4 : 1;
  const int rps = kGatherThreads / QL;
  const int64_t S = (rows + (int64_t)steps * rps - 1) / ((int64_t)steps * rps);
  const int NBT = (B + BT - 1) / BT;
  const int64_t wgs = (int64_t)G * S * NBT * mats;
  const int64_t rounds = (wgs + kCUs - 1) / kCUs;
  const int64_t active = std::min<int64_t>(wgs, kCUs);
  const double slab_rows = (double)std::min<int64_t>(rows, (int64_t)steps * rps);
  const double pairs = (double)cpg * P;
  const double chunk_bytes = (double)P * K * BT * stage_es;
  const double t_stage = cpg * (2.0 + chunk_bytes / 150e3);
  // bytes per us; one CU of the pipelined kernel (codes and codebook streamed at once)
  // sustains about the chip's share per CU: fewer workgroups cannot draw the whole bandwidth
  const double per_cu_bw = pipe ? 6.4e6 / kCUs : std::min(150e3, 6.4e6 / (double)active);
  const double t_codes = slab_rows * pairs * 2.0 / per_cu_bw;
  const double lookups_per_us = BT == 1 ? 9.0 * 2400.0 : (120.0 * 2400.0) / (BT * es);
  // every lane looks up all lane_steps rows of its kernel, also those past
  // the slab or the last row
  const double t_look = (double)lane_steps * rps * pairs / lookups_per_us;
  // The pipelined kernel splits the chunks evenly over the G groups: a workgroup streams the
  // codes and codebook of NP / G pairs on average.
  const double pairs_avg = (double)NP / G;
  // (a tenth of the lookups is charged on top: the barrier per chunk exposes some of them,
  // and of two plans that stream alike the one with fewer idle lane steps wins)
  const double t_look_avg = t_look * pairs_avg / pairs;
  const double t_wg = pipe ? 2.0 + std::max((slab_rows * pairs_avg * 2.0 + pairs_avg * K * stage_es) / per_cu_bw,
                                            t_look_avg) + 0.1 * t_look_avg
                           : t_stage + std::max(t_codes, t_look);
  const double t_stream = (double)rows * NP * 2.0 * NBT * mats / 6.4e6;
  const double t_partial = G > 1 ? 5.0 + (double)G * B * rows * 8.0 * mats / 6.4e6 : 0.0;
  return std::max(t_stream, (double)rounds * t_wg) + t_partial;
}

// fused_d > 0: the table is built while staging from fp32 codebooks of
// subspace width fused_d (B == 1): a chunk's staged bytes are its codebook
// rows (4*fused_d per entry, at most 128 KB so they fit the staging
// registers), and the activation slices of the group's pairs share the LDS.
// Fused d = 2 (the Gemma MLP) has kernels for 2, 3 and 4 rows per lane, d = 8
// (its second attempt) for 2 and 3, so that a slab can cover a short matrix's
// rows with few idle lanes (more rows per lane spill at 128 VGPRs).
size_t fused_act_bytes(int P, int cpg, int NP, int fused_d) {
  return fused_d ? (size_t)std::min(cpg * P, NP) * fused_d * 4 : 0;
}

bool steps_allowed(int steps, int fused_d) {
  if (fused_d == 2) return steps >= 2 && steps <= 4;
  if (fused_d == 8) return steps == 2 || steps == 3;
  return steps >= 1 && steps <= 4;
}

GatherPlan search_plan(int64_t rows, int NP, int K, int B, int lut_bf16, int fused_d, int ppb, int mats) {
  const int es = lut_bf16 ? 2 : 4;
  const int stage_es = fused_d ? 4 * fused_d : es;
  GatherPlan best{};
  int BT = 1;
  if (B > 1) BT = ((size_t)K * 16 * es * 2 <= (size_t)kLdsBudget && B >= 16) ? 16 : 4;
  if ((size_t)K * BT * es > (size_t)kLdsBudget) BT = 1;
  if ((size_t)K * BT * es > (size_t)kLdsBudget) return best;
  const int QL = BT >= 16 ? 4 : 1;
  const int rps = kGatherThreads / QL;
  const int nstep = nstep_for(BT);
  const int NBT = (B + BT - 1) / BT;
  int pmax = (int)std::min<int64_t>(NP, kLdsBudget / ((size_t)K * BT * es));
  if (fused_d) {
    pmax = (int)std::min<int64_t>({(int64_t)NP, (int64_t)kLdsBudget / ((int64_t)K * 4),
                                   (int64_t)kRegStage * 16 * kGatherThreads / ((int64_t)K * stage_es)});
    if (pmax < 1) return best;
  }
  // One vector per lane: chunks of at most 24 pairs (whole blocks of both
  // serving layouts) measured faster than LDS-filling ones -- with the flat
  // block loop the code stream runs through chunk switches, and smaller
  // switches stall the workgroup for less time.
  if (BT == 1 && !fused_d) pmax = std::min(pmax, 24);
  // The pipelined kernel, whose chunks are one code block each (the words of
  // two chunks then fit its registers): fused build at d = 2 or an fp32 table
  // for one vector, 16- or 10-bit codes, K <= 1024, a matrix taller than one
  // slab and at least 64 blocks of pairs (so that a group holds several
  // chunks). Measured: the Gemma-2 MLP's gate and up 26.4 us against 30.3
  // (9,216 rows, 288 blocks, one launch); its down 29.1 against 27.2 (2,304
  // rows, one slab) and the second attempt's gate and up from their tables
  // 12.8 against 10.8 (48 blocks: one or two chunks per group) keep the
  // one-buffer kernel.
  // (A pair's table or codebook must be whole 16-byte words: K % 4 == 0 for
  // the table, K*d % 4 == 0 for the fused build.)
  const bool pipe = (fused_d == 2 || (fused_d == 0 && BT == 1 && !lut_bf16)) && (ppb == 8 || ppb == 12) &&
                    K <= 1024 && (K * (fused_d ? fused_d : 1)) % 4 == 0 && rows > 4 * (int64_t)kGatherThreads &&
                    (NP + ppb - 1) / ppb >= 64;
  if (pipe) pmax = std::min(NP, ppb);
  if (pmax < NP && pmax > 1 && !pipe) pmax &= ~1;
  double best_cost = 1e300;
  int tried = 0;
  for (int P = pmax; P >= 1 && P >= pmax / 2 && tried < 8; --P) {
    if (P < NP && P > 1 && (P & 1)) continue;
    // a chunk smaller than a code block loads every block once per chunk it
    // touches: only when nothing larger fits
    if (P < ppb && P < NP && pmax >= ppb) continue;
    if (pipe && P != pmax) continue;
    ++tried;
    const int chunks = (NP + P - 1) / P;
    for (int steps = nstep; steps >= 1; --steps) {
      if (!steps_allowed(steps, fused_d)) continue;
      const int64_t S = (rows + (int64_t)steps * rps - 1) / ((int64_t)steps * rps);
      if (S * NBT > (1 << 24)) continue;
      const int64_t gmax = std::max<int64_t>(1, std::min<int64_t>(chunks, 4 * kCUs / (S * NBT * mats) + 1));
      for (int64_t G0 = 1; G0 <= gmax; ++G0) {
        const int cpg = (int)((chunks + G0 - 1) / G0);
        const int G = pipe ? (int)G0 : (chunks + cpg - 1) / cpg;   // the pipelined kernel splits chunks evenly
        if (G != G0) continue;
        if ((size_t)(pipe ? 2 : 1) * P * K * 4 + fused_act_bytes(P, cpg, NP, fused_d) > (size_t)kLdsBudget && fused_d)
          continue;
        // prefer aligned chunks (staging outside the block loop) on near-ties
        const int lane_steps = (fused_d == 2 || fused_d == 8) ? steps : nstep;   // the kernel instances (dispatch_gather)
        const double cost = plan_cost_us(rows, NP, K, B, es, BT, P, steps, G, cpg, stage_es, lane_steps, mats, pipe) *
                            ((P % ppb == 0 || chunks == 1) ? 1.0 : 1.03);
        if (cost < best_cost * 0.999) {
          best_cost = cost;
          best.BT = BT; best.P = P; best.chunks = chunks; best.cpg = cpg; best.G = G;
          best.steps = steps; best.rps = rps; best.S = (int)S; best.NBT = NBT;
          best.pipe = pipe ? 1 : 0;
        }
      }
    }
  }
  // Several batch tiles (staged from the batch-tiled copy): eight groups of
  // pairs, whatever the model says. At the stress head (K=4096, L=4, B=64,
  // bf16 table) they measured 6.50 ms per call against 7.28 for the model's
  // single group (and 6.9 for four, 6.8 for sixteen); the model, which prices
  // rounds of workgroups, does not capture why.
  if (best.BT != 0 && best.NBT > 1 && best.G < 8 && best.chunks >= 8) {
    best.cpg = (best.chunks + 7) / 8;
    best.G = (best.chunks + best.cpg - 1) / best.cpg;
  }
  // Several bf16 batch tiles of 4: two row sets per workgroup, so every staged
  // chunk serves twice the rows (the kernel's time there falls as 1/rows per
  // slab: the table restaging bounds it).
  if (best.BT == 4 && best.NBT > 1 && lut_bf16 && !fused_d && best.S >= 2) {
    best.rset = 2;
    best.S = (int)((rows + 2 * (int64_t)best.steps * best.rps - 1) / (2 * (int64_t)best.steps * best.rps));
  }
  // fp32 tables for 16 vectors (slabs of only 4 x 256 rows): two row sets as
  // well, with enough groups of pairs to keep a workgroup per CU. At the
  // Gemma head with B=16: 1.30 ms per call for the model's single group, 1.17
  // for two groups, 0.96 for two groups of two row sets.
  if (best.BT == 16 && !lut_bf16 && !fused_d && best.S >= 2) {
    best.rset = 2;
    best.S = (int)((rows + 2 * (int64_t)best.steps * best.rps - 1) / (2 * (int64_t)best.steps * best.rps));
    const int64_t want = std::min<int64_t>(best.chunks, std::max<int64_t>(1, kCUs / ((int64_t)best.S * best.NBT)));
    if (best.G < want) {
      best.cpg = (int)((best.chunks + want - 1) / want);
      best.G = (best.chunks + best.cpg - 1) / best.cpg;
    }
  }
  // One vector on the pipelined kernel with fewer workgroups than CUs (the
  // Gemma head: 63 slabs of 4,096 rows x 4 groups = 252): shorter slabs, in
  // whole 8-row units (128-byte lines of codes), so that every CU has one
  // workgroup and each does less (64 slabs of 4,000 rows).
  if (best.pipe && !fused_d && BT == 1 && mats == 1 && best.NBT == 1 && best.G * (int64_t)best.S < kCUs) {
    const int64_t S2 = kCUs / best.G;
    const int64_t slab = ((rows + S2 - 1) / S2 + 7) / 8 * 8;
    if (slab >= 8 && slab < (int64_t)best.steps * best.rps && (rows + slab - 1) / slab * best.G <= kCUs) {
      best.slab = slab;
      best.S = (int)((rows + slab - 1) / slab);
    }
  }
  best.lds = (size_t)(best.pipe ? 2 : 1) * best.P * K * BT * es + fused_act_bytes(best.P, best.cpg, NP, fused_d);
  return best;
}

// Plans are a pure function of the shapes; a small memo keeps the search
// off the per-call path.
struct PlanKey {
  int64_t rows;
  int NP, K, B, bf16, fused_d, ppb, mats;
  bool operator==(const PlanKey& o) const {
    return rows == o.rows && NP == o.NP && K == o.K && B == o.B && bf16 == o.bf16 && fused_d == o.fused_d &&
           ppb == o.ppb && mats == o.mats;
  }
};
std::mutex g_plan_mu;
PlanKey g_plan_keys[32];
GatherPlan g_plans[32];
int g_plan_n = 0, g_plan_next = 0;

}  // namespace

// Tiling heuristic. The table staging traffic is S*NBT full tables whatever P
// and G are, so P is taken as large as LDS allows; then (steps, G) are chosen
// to fill every CU with one workgroup per round, preferring few groups
// (partial-sum traffic) and long slabs (loads in flight per lane).
GatherPlan plan_gather(const rq_matrix* W, int B, int lut_bf16, int fused, int mats) {
  const int fd = fused ? W->d : 0;
  const PlanKey key{W->rows, W->L * W->M, W->K, B, lut_bf16, fd, pairs_per_block(W), mats};
  GatherPlan plan{};
  bool hit = false;
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    for (int i = 0; i < g_plan_n; ++i)
      if (g_plan_keys[i] == key) { plan = g_plans[i]; hit = true; break; }
  }
  if (!hit) {
    plan = search_plan(key.rows, key.NP, key.K, B, lut_bf16, fd, key.ppb, mats);
    std::lock_guard<std::mutex> lock(g_plan_mu);
    g_plan_keys[g_plan_next] = key;
    g_plans[g_plan_next] = plan;
    g_plan_next = (g_plan_next + 1) % 32;
    if (g_plan_n < 32) ++g_plan_n;
  }
  return plan;
}

template <int CB>
hipError_t dispatch_gather(const GatherArgs& a, const GatherPlan& plan, int d, int lut_bf16, bool fused,
                           hipStream_t stream) {
  if (fused) {
    if (d == 1) return launch_gather_typed<float, 1, 4, 1, CB>(a, plan, stream);
    if (d == 2 && plan.pipe) {
      if constexpr (CB != 8) {
        switch (plan.steps) {
          case 2: return launch_gather_typed<float, 1, 2, 2, CB, 1, true>(a, plan, stream);
          case 3: return launch_gather_typed<float, 1, 3, 2, CB, 1, true>(a, plan, stream);
          default: return launch_gather_typed<float, 1, 4, 2, CB, 1, true>(a, plan, stream);
        }
      }
      return hipErrorInvalidValue;
    }
    if (d == 2) {
      switch (plan.steps) {
        case 2: return launch_gather_typed<float, 1, 2, 2, CB>(a, plan, stream);
        case 3: return launch_gather_typed<float, 1, 3, 2, CB>(a, plan, stream);
        default: return launch_gather_typed<float, 1, 4, 2, CB>(a, plan, stream);
      }
    }
    if (d == 8)   // 2 or 3 rows per lane (4 would spill)
      return plan.steps == 2 ? launch_gather_typed<float, 1, 2, 8, CB>(a, plan, stream)
                             : launch_gather_typed<float, 1, 3, 8, CB>(a, plan, stream);
    return launch_gather_typed<float, 1, 4, 4, CB>(a, plan, stream);
  }
  if (lut_bf16) {
    if (plan.BT == 1) return launch_gather_typed<uint16_t, 1, 4, 0, CB>(a, plan, stream);
    if (plan.BT == 4)
      return plan.rset == 2 ? launch_gather_typed<uint16_t, 4, 4, 0, CB, 2>(a, plan, stream)
                            : launch_gather_typed<uint16_t, 4, 4, 0, CB>(a, plan, stream);
    return launch_gather_typed<uint16_t, 16, 4, 0, CB>(a, plan, stream);
  }
  if (plan.BT == 1 && plan.pipe) {
    if constexpr (CB != 8) return launch_gather_typed<float, 1, 4, 0, CB, 1, true>(a, plan, stream);
    return hipErrorInvalidValue;
  }
  if (plan.BT == 1) return launch_gather_typed<float, 1, 4, 0, CB>(a, plan, stream);
  if (plan.BT == 4) return launch_gather_typed<float, 4, 4, 0, CB>(a, plan, stream);
  return plan.rset == 2 ? launch_gather_typed<float, 16, 4, 0, CB, 2>(a, plan, stream)
                        : launch_gather_typed<float, 16, 4, 0, CB>(a, plan, stream);
}

template <typename T>
__global__ void tile_lut_kernel(const T* __restrict__ src, int64_t NPK, int B, int BT, int NBT, T* __restrict__ dst) {
  // one thread per (row of the table, batch tile): BT consecutive entries
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= NPK * NBT) return;
  const int t = (int)(i % NBT);
  const int64_t pk = i / NBT;
  const T* s = src + pk * B + (int64_t)t * BT;
  T* d = dst + ((int64_t)t * NPK + pk) * BT;
  for (int j = 0; j < BT; ++j) d[j] = (t * BT + j < B) ? s[j] : (T)0;
}

// The same transposition through LDS, in 4-byte units (B and BT of 4-byte
// multiples): a workgroup reads R whole table rows contiguously, then writes
// each batch tile's R-row run contiguously (zero past B). Rows sit in LDS
// with one unit of padding, so the column reads do not collide in banks.
constexpr int kTileThreads = 256;
__global__ __launch_bounds__(kTileThreads) void tile_lut_lds_kernel(const uint32_t* __restrict__ src, int64_t NPK,
                                                                    int UB, int UT, int NBT, int R,
                                                                    uint32_t* __restrict__ dst) {
  extern __shared__ uint32_t rowbuf[];   // [R][UB + 1]
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int rows = (int)min<int64_t>(R, NPK - r0);
  for (int u = threadIdx.x; u < rows * UB; u += kTileThreads) {
    const int row = u / UB;
    rowbuf[row * (UB + 1) + (u - row * UB)] = src[(r0 + row) * UB + (u - row * UB)];
  }
  __syncthreads();
  const int per_tile = rows * UT;
  for (int v = threadIdx.x; v < NBT * per_tile; v += kTileThreads) {
    const int t = v / per_tile;
    const int rem = v - t * per_tile;
    const int row = rem / UT;
    const int c = rem - row * UT;
    const int col = t * UT + c;
    dst[((int64_t)t * NPK + r0 + row) * UT + c] = col < UB ? rowbuf[row * (UB + 1) + col] : 0u;
  }
}

// The same copy in 16-byte units, for whole 16-byte table rows (UB % 4 == 0)
// and 16-byte runs per tile (R * UT % 4 == 0): a tile's R rows are one
// contiguous run of R * UT units in the destination, so each lane gathers
// four consecutive units of a run from LDS and stores them at once. A quarter
// of the memory instructions of the 4-byte copy.
__global__ __launch_bounds__(kTileThreads) void tile_lut_lds16_kernel(const uint32_t* __restrict__ src, int64_t NPK,
                                                                      int UB, int UT, int NBT, int R,
                                                                      uint32_t* __restrict__ dst) {
  extern __shared__ uint32_t rowbuf[];   // [R][UB + 1]
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int rows = (int)min<int64_t>(R, NPK - r0);
  const int UB4 = UB / 4;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src + r0 * UB);
  for (int u = threadIdx.x; u < rows * UB4; u += kTileThreads) {
    const int row = u / UB4;
    const int c = (u - row * UB4) * 4;
    const u32x4 v = s4[u];
    uint32_t* b = rowbuf + row * (UB + 1) + c;
    b[0] = v[0]; b[1] = v[1]; b[2] = v[2]; b[3] = v[3];
  }
  __syncthreads();
  const int run = rows * UT;              // this block's units of one tile
  const int run4 = run / 4;               // whole 16-byte groups (rows * UT % 4 == 0 by the host's choice of R)
  for (int v = threadIdx.x; v < NBT * run4; v += kTileThreads) {
    const int t = v / run4;
    const int w0 = (v - t * run4) * 4;    // first unit of the group within the run
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (w0 + i) / UT;
      const int col = t * UT + (w0 + i - row * UT);
      w[i] = col < UB ? rowbuf[row * (UB + 1) + col] : 0u;
    }
    u32x4 o;
    o[0] = w[0]; o[1] = w[1]; o[2] = w[2]; o[3] = w[3];
    *reinterpret_cast<u32x4*>(dst + ((int64_t)t * NPK + r0) * UT + w0) = o;
  }
}

hipError_t launch_tile_lut(const void* lut, int lut_bf16, int NP, int K, int B, int BT, void* dst, hipStream_t stream) {
  const int NBT = (B + BT - 1) / BT;
  const int64_t NPK = (int64_t)NP * K;
  const int es = lut_bf16 ? 2 : 4;
  if ((B * es) % 4 == 0 && (BT * es) % 4 == 0) {
    const int UB = B * es / 4, UT = BT * es / 4;
    const int R = std::max(1, std::min(64, 16384 / (UB + 1)));   // at most 64 KB of LDS
    const size_t lds = (size_t)R * (UB + 1) * 4;
    const unsigned blocks = (unsigned)((NPK + R - 1) / R);
    // 16-byte units: whole 16-byte table rows, every block's run per tile (the
    // last block's too) a whole number of 16-byte units, 16-byte aligned ends
    const int64_t last_rows = NPK - (int64_t)(blocks - 1) * R;
    if (UB % 4 == 0 && ((int64_t)R * UT) % 4 == 0 && (last_rows * UT) % 4 == 0 && (NPK * UT) % 4 == 0 &&
        ((uintptr_t)lut & 15) == 0 && ((uintptr_t)dst & 15) == 0) {
      hipLaunchKernelGGL(tile_lut_lds16_kernel, dim3(blocks), dim3(kTileThreads), lds, stream,
                         static_cast<const uint32_t*>(lut), NPK, UB, UT, NBT, R, static_cast<uint32_t*>(dst));
      return hipGetLastError();
    }
    hipLaunchKernelGGL(tile_lut_lds_kernel, dim3(blocks), dim3(kTileThreads), lds, stream,
                       static_cast<const uint32_t*>(lut), NPK, UB, UT, NBT, R, static_cast<uint32_t*>(dst));
    return hipGetLastError();
  }
  const int64_t n = NPK * NBT;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (lut_bf16)
    hipLaunchKernelGGL(tile_lut_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(lut), NPK,
                       B, BT, NBT, static_cast<uint16_t*>(dst));
  else
    hipLaunchKernelGGL(tile_lut_kernel<float>, dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(lut), NPK, B,
                       BT, NBT, static_cast<float*>(dst));
  return hipGetLastError();
}

bool fused_build_supported(const rq_matrix* W, int B) {
  return B == 1 && W->cb_dtype == RQ_F32 && (W->d == 1 || W->d == 2 || W->d == 4 || W->d == 8) &&
         ((uintptr_t)W->codebooks % 16) == 0 && ((size_t)W->K * W->d) % 4 == 0;
}

namespace {

GatherArgs gather_args(const rq_matrix* W, const GatherPlan& plan, const void* lut, int B, const GatherOut& o,
                       const float* fused_act, const float* fused_x2) {
  GatherArgs a{};
  a.cv = code_view(W);
  a.lut = fused_act ? W->codebooks : lut;
  a.act = fused_act;
  a.act2 = fused_x2;
  a.D = W->D;
  a.M = W->M;
  a.rows = W->rows;
  a.NP = W->L * W->M;
  a.K = W->K;
  a.B = B;
  a.P = plan.P; a.chunks = plan.chunks; a.cpg = plan.cpg; a.G = plan.G;
  a.steps = plan.steps; a.S = plan.S; a.NBT = plan.NBT;
  a.slab_rows = plan.slab_rows();
  a.partial = o.partial;
  a.out = o.out;
  a.softcap = o.softcap;
  a.block_keys = plan.G == 1 ? o.block_keys : nullptr;
  a.tiled = o.lut_tiled;
  a.mats = 1;
  // Contiguous per-XCD ranges let the few slabs of one group share its staged
  // chunks in one L2 (gate/up of the Gemma MLP: 3 slabs, 24.5 -> 18.5 us).
  // With many slabs per group (the head: 63) the workgroups of an XCD would
  // all switch to the same chunks at once, which measured slower (69 -> 74 us),
  // so dispatch order is kept there.
  a.xcd_contiguous = plan.S >= 2 && plan.S <= 8;
  return a;
}

hipError_t dispatch(const rq_matrix* W, const GatherArgs& a, const GatherPlan& plan, int lut_bf16, bool fused,
                    hipStream_t stream) {
  if (W->codes_layout == RQ_CODES_PACKED10) return dispatch_gather<10>(a, plan, W->d, lut_bf16, fused, stream);
  if (W->codes_layout == RQ_CODES_PACKED8) return dispatch_gather<8>(a, plan, W->d, lut_bf16, fused, stream);
  return dispatch_gather<16>(a, plan, W->d, lut_bf16, fused, stream);
}

}  // namespace

hipError_t launch_gather(const rq_matrix* W, const GatherPlan& plan, const void* lut, int lut_bf16, int B,
                         const GatherOut& o, hipStream_t stream, const float* fused_act, const float* fused_x2) {
  const GatherArgs a = gather_args(W, plan, lut, B, o, fused_act, fused_x2);
  hipError_t e = dispatch(W, a, plan, lut_bf16, fused_act != nullptr, stream);
  if (e != hipSuccess || plan.G == 1) return e;
  return launch_finish(o.partial, plan.G, B, W->rows, o.softcap, o.out, o.block_keys, stream);
}

hipError_t launch_gather_pair(const rq_matrix* W1, const rq_matrix* W2, const GatherPlan& plan, const float* x,
                              const float* lut1, const float* lut2, float* part1, float* part2, hipStream_t stream) {
  GatherOut o{};
  o.partial = part1;
  o.out = plan.G == 1 ? part1 : nullptr;   // one group: the sums themselves
  GatherArgs a = gather_args(W1, plan, lut1, 1, o, x, nullptr);
  a.cv2 = code_view(W2);
  a.lut2 = x ? W2->codebooks : static_cast<const void*>(lut2);
  a.partial2 = part2;
  a.out2 = plan.G == 1 ? part2 : nullptr;
  a.mats = 2;
  return dispatch(W1, a, plan, 0, x != nullptr, stream);
}

size_t gather_pro_lds(const rq_matrix* W, const GatherPlan& plan, int pro_G) {
  const size_t E = (size_t)std::min(plan.cpg * plan.P, W->L * W->M) * W->d;
  return plan.lds + 2 * E * finish_parts(pro_G) * sizeof(float);
}

hipError_t launch_gather_pro(const rq_matrix* W, const GatherPlan& plan, const float* pro_partial, int pro_G,
                             int64_t pro_rows, const GatherOut& o, hipStream_t stream) {
  GatherPlan p = plan;
  p.lds = gather_pro_lds(W, plan, pro_G);
  if (p.lds > (size_t)kLdsBudget) return hipErrorInvalidValue;
  GatherArgs a = gather_args(W, p, nullptr, 1, o, pro_partial, nullptr);
  a.pro_partial = pro_partial;
  a.pro_G = pro_G;
  a.pro_tpr = finish_parts(pro_G);
  a.pro_rows = pro_rows;
  hipError_t e = dispatch(W, a, p, 0, true, stream);
  if (e != hipSuccess || p.G == 1) return e;
  return launch_finish(o.partial, p.G, 1, W->rows, o.softcap, o.out, o.block_keys, stream);
}

int finish_parts(int G) { return G <= 8 ? 1 : (G <= 64 ? 4 : 16); }
int finish_rows_per_block(int G) { return kFinishThreads / finish_parts(G); }

hipError_t launch_finish(const float* partial, int G, int B, int64_t rows, float softcap, float* out,
                         uint64_t* block_keys, hipStream_t stream) {
  const int tpr = finish_parts(G);
  const int rpb = kFinishThreads / tpr;
  dim3 grid((unsigned)((rows + rpb - 1) / rpb), (unsigned)B);
  if (tpr == 1 && B >= 8)
    hipLaunchKernelGGL(finish4_kernel, grid, dim3(kFinish4Threads), 0, stream, partial, G, B, rows, softcap, out,
                       block_keys);
  else if (tpr == 1)
    hipLaunchKernelGGL(finish_kernel<1>, grid, dim3(kFinishThreads), 0, stream, partial, G, B, rows, softcap, out,
                       block_keys);
  else if (tpr == 4)
    hipLaunchKernelGGL(finish_kernel<4>, grid, dim3(kFinishThreads), 0, stream, partial, G, B, rows, softcap, out,
                       block_keys);
  else
    hipLaunchKernelGGL(finish_kernel<16>, grid, dim3(kFinishThreads), 0, stream, partial, G, B, rows, softcap, out,
                       block_keys);
  return hipGetLastError();
}

int key_blocks(const GatherPlan& plan, int64_t rows) {
  return plan.G == 1 ? plan.S : finish_key_blocks(plan.G, rows);
}

int finish_key_blocks(int G, int64_t rows) {
  const int rpb = finish_rows_per_block(G);
  return (int)((rows + rpb - 1) / rpb);
}

hipError_t launch_select(const uint64_t* block_keys, int nkb, int B, int32_t* argmax, const float* logits,
                         int64_t rows, int topk, uint64_t* cand, int32_t* topk_ids, float* topk_vals,
                         hipStream_t stream) {
  const int ncb = epi_blocks(rows);
  if (topk > 0) {
    hipLaunchKernelGGL(topk_block_kernel, dim3((unsigned)ncb, (unsigned)B), dim3(kTopkThreads), 0, stream, logits,
                       rows, topk, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (topk <= 0) {
    if (!argmax) return hipSuccess;
    hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)B), dim3(64), 0, stream, block_keys, nkb, argmax);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)B), dim3(kSelThreads), 0, stream, block_keys, nkb, argmax, ncb,
                     cand, topk, topk_ids, topk_vals);
  return hipGetLastError();
}

}  // namespace rq
