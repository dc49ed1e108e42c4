// rq_internal.h -- declarations shared by the HIP sources of librq_lut.so.
//
// Device helpers (bf16 conversion, selection keys) and the host-side launch
// functions each kernel file provides to the C-ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "rq_lut.h"
#include "rq_lut_measure.h"

namespace rq {

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bit pattern, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Selection key with a total order: a larger value gives a larger key, and
// among equal values the lower index gives the larger key. -0 counts as +0.
__device__ __forceinline__ uint64_t select_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) { return 0xffffffffu - (uint32_t)key; }
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

__device__ __forceinline__ float gelu_tanh(float t) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * t * (1.0f + tanhf(k * (t + 0.044715f * t * t * t)));
}

// Code of pair p for row r. 16-bit layouts (cbits 16): codes[(p >> 3) * s_blk
// + r * s_row + (p & 7)]; RQ_CODES_ROWS: s_blk = 8, s_row = NP;
// RQ_CODES_BLOCKED: s_blk = 8 * rows, s_row = 8. RQ_CODES_PACKED10 (cbits 10):
// blocks of 12 pairs, s_blk = 8 * rows and s_row = 8 in 16-bit units; pair
// 12q + 3w + i sits at bits [10i, 10i+10) of the row's 32-bit word w of block
// q. RQ_CODES_PACKED8 (cbits 8): blocks of 16 pairs, same strides; pair
// 16q + i is byte i of the row's 16 bytes of block q.
struct CodeView {
  const uint16_t* codes;
  int64_t s_blk;
  int64_t s_row;
  int cbits;
};

__device__ __forceinline__ uint32_t code_at(const CodeView& cv, int64_t r, int p) {
  if (cv.cbits == 8) {
    const int q = p >> 4;
    return reinterpret_cast<const uint8_t*>(cv.codes + q * cv.s_blk + r * cv.s_row)[p & 15];
  }
  if (cv.cbits == 10) {
    const int q = p / 12;
    const int t = p - 12 * q;
    const int w = t / 3;
    const uint32_t word = *reinterpret_cast<const uint32_t*>(cv.codes + q * cv.s_blk + r * cv.s_row + 2 * w);
    return (word >> (10 * (t - 3 * w))) & 0x3ffu;
  }
  return cv.codes[(int64_t)(p >> 3) * cv.s_blk + r * cv.s_row + (p & 7)];
}

// Pairs per 16-byte code block of a serving layout.
inline int pairs_per_block(const rq_matrix* W) {
  return W->codes_layout == RQ_CODES_PACKED10 ? 12 : (W->codes_layout == RQ_CODES_PACKED8 ? 16 : 8);
}

// ---------------------------------------------------------------- host side

constexpr int kCUs = 256;                 // MI355X compute units
constexpr int kLdsBytes = 160 * 1024;     // LDS per workgroup on gfx950
constexpr int kLdsBudget = kLdsBytes - 1024;   // for the staged table (the rest: small static arrays)
constexpr int kGatherThreads = 1024;

CodeView code_view(const rq_matrix* W);

// Tiling of one lookup+sum pass (chosen from the shapes alone).
struct GatherPlan {
  int BT;        // batch values per table entry staged on chip (1, 4 or 16)
  int P;         // (level, subspace) pairs per staged chunk
  int chunks;    // ceil(NP / P)
  int cpg;       // chunks per group
  int G;         // groups: partial sums per output, reduced in a fixed order
  int steps;     // row steps per row set
  int rps;       // rows per step
  int S;         // row slabs of slab_rows() rows
  int rset = 1;  // row sets per workgroup (2: bf16 tables in several batch tiles of 4, fp32 tables of 16 vectors)
  int NBT;       // batch tiles
  size_t lds;    // dynamic LDS bytes per workgroup
  int pipe = 0;  // fused build, d = 2: one code block per chunk, two chunks in flight (the pipelined kernel)
  int64_t slab = 0;  // rows per slab when shorter than rset * steps * rps (0: that many)
  int64_t slab_rows() const { return slab ? slab : (int64_t)rset * steps * rps; }
  int64_t wgs() const { return (int64_t)G * S * NBT; }
};
// fused != 0: the table is built while staging (fused_build_supported).
// mats = 2: one launch covers two matrices of W's shape (launch_gather_pair).
GatherPlan plan_gather(const rq_matrix* W, int B, int lut_bf16, int fused = 0, int mats = 1);
// Whether the lookup+sum can build the table itself while staging: one
// activation vector, fp32 codebooks with d in {1, 2, 4, 8}, 16-byte aligned.
bool fused_build_supported(const rq_matrix* W, int B);

// Launchers: return hipSuccess or the launch error. All enqueue on `stream`.
hipError_t launch_build_lut(const rq_matrix* W, const float* x, const float* x2, int prologue, int B,
                            int lut_bf16, void* lut, hipStream_t stream);
// Fp32 tables of two matrices of one shape on the same vector (B = 1), in one launch where the
// single-vector kernel takes them (else two launches): the MLP's gate and up.
hipError_t launch_build_lut_pair(const rq_matrix* W, const rq_matrix* W2, const float* x, float* lut, float* lut2,
                                 hipStream_t stream);
// Outputs and workspace of one lookup+sum pass.
struct GatherOut {
  float* partial;        // [G][B][rows] partial sums (G > 1)
  float* out;            // [B][rows] results after the softcap, or null
  float softcap;         // <= 0: none
  uint64_t* block_keys;  // [B][key_blocks()] best selection key per block of rows, or null
  int lut_tiled;         // the table is in the batch-tiled layout of launch_tile_lut
};
// Table [NP][K][B] -> batch-tiled [ceil(B/BT)][NP][K][BT] (zero past B), so that
// a batch tile's chunk of pairs is contiguous and stages with 16-byte copies.
hipError_t launch_tile_lut(const void* lut, int lut_bf16, int NP, int K, int B, int BT, void* dst, hipStream_t stream);
// The lookup+sum pass: the gather kernel, and for G > 1 the finish kernel that
// adds the partial sums in group order.
// One-shot events around the next lookup+sum launch of this thread (rq_set_stage_events).
void take_stage_events(hipEvent_t* before, hipEvent_t* after);

// fused_act != null: build the table while staging from W's codebooks and the
// activation vector fused_act [D], or gelu_tanh(fused_act) * fused_x2 when
// fused_x2 != null (plan from plan_gather(W, 1, 0, 1)); lut is ignored.
hipError_t launch_gather(const rq_matrix* W, const GatherPlan& plan, const void* lut, int lut_bf16, int B,
                         const GatherOut& o, hipStream_t stream, const float* fused_act = nullptr,
                         const float* fused_x2 = nullptr);
// Whether a plan's chunks span at least one 16-byte code block (or the matrix
// is one chunk). A fused build whose register stage holds fewer pairs than a
// block (d = 8 at K = 1024: 4 pairs) loads every block once per chunk it
// touches, and measured slower than building the table first.
inline bool plan_covers_blocks(const rq_matrix* W, const GatherPlan& p) {
  return p.chunks == 1 || p.P >= pairs_per_block(W);
}
// Two matrices of the same shape (W1, W2) and one activation vector, in one
// launch: with x != null the fused table build (plan from plan_gather(W1, 1, 0,
// 1, 2)), else the fp32 tables lut1 / lut2 (plan from plan_gather(W1, 1, 0, 0,
// 2)). Each writes its partial sums [G][1][rows] (G > 1), or with G == 1 its
// sums, to part1 / part2. No finish pass.
hipError_t launch_gather_pair(const rq_matrix* W1, const rq_matrix* W2, const GatherPlan& plan, const float* x,
                              const float* lut1, const float* lut2, float* part1, float* part2, hipStream_t stream);
// Fused table build whose activation is gelu_tanh(g) * u, g and u summed from
// the partial sums [2][pro_G][pro_rows] of launch_gather_pair in the finish
// pass's order (bit-identical to finishing them first); then as launch_gather.
// Returns hipErrorInvalidValue when the extra LDS does not fit.
hipError_t launch_gather_pro(const rq_matrix* W, const GatherPlan& plan, const float* pro_partial, int pro_G,
                             int64_t pro_rows, const GatherOut& o, hipStream_t stream);
size_t gather_pro_lds(const rq_matrix* W, const GatherPlan& plan, int pro_G);
int key_blocks(const GatherPlan& plan, int64_t rows);
// argmax from the per-block keys (argmax may be null) and, with topk > 0, the
// top-k of the logits (cand: [B][epi_blocks(rows)][topk] scratch).
hipError_t launch_select(const uint64_t* block_keys, int nkb, int B, int32_t* argmax, const float* logits,
                         int64_t rows, int topk, uint64_t* cand, int32_t* topk_ids, float* topk_vals,
                         hipStream_t stream);
// The finish pass alone: adds G partial sums [G][B][rows] in a fixed order,
// applies the softcap, writes out [B][rows] and one selection key per block of
// rows (block_keys [B][finish_key_blocks(G, rows)], or null).
int finish_key_blocks(int G, int64_t rows);
int finish_parts(int G);   // threads per row of the finish pass (its summation order)
hipError_t launch_finish(const float* partial, int G, int B, int64_t rows, float softcap, float* out,
                         uint64_t* block_keys, hipStream_t stream);

// Batched head on the matrix cores (bf16 codebooks staged in LDS, hidden
// vectors split into three bf16 parts): partial sums [G][B][rows].
constexpr int kMmMaxK = 1024;
struct MmPlan {
  int NT;      // 16-column MFMA tiles per batch tile
  int T;       // 16-row tiles per wave
  int NBT;     // batch tiles
  int Bp;      // padded batch (NBT * 16 * NT)
  int S;       // row slabs
  int NQ;      // code blocks of 8 (level, subspace) pairs
  int G;       // groups of code blocks (partial sums per output)
  int qpg;     // code blocks per group
  size_t lds;  // dynamic LDS bytes per workgroup
  int pad;     // 1: the codebooks are copied, codewords padded to 16 bytes, into the workspace after the split h
};
bool mm_supported(const rq_matrix* W);
// The matrix-core method runs this matrix at batch B (B >= RQ_MM_MIN_B and mm_supported, plus the size
// limits of its kernels).
bool mm_usable(const rq_matrix* W, int B);
MmPlan plan_mm(const rq_matrix* W, int B);
size_t mm_hp_bytes(const rq_matrix* W, const MmPlan& p);
// G > 1: partial sums [G][B][rows] (then launch_finish). G == 1: the logits
// after the softcap go to out (if not null) and the best selection key of each
// slab to block_keys [B][S] (if not null).
hipError_t launch_mm_logits(const rq_matrix* W, const MmPlan& p, const float* h, int B, void* hp, float* partial,
                            float* out, float softcap, uint64_t* block_keys, hipStream_t stream);

// Measurement aid: one read of [src, src + bytes) with 16-byte loads; one
// 32-bit XOR per workgroup to sink (stream_read_sink_words(config) words).
int stream_read_configs();
size_t stream_read_sink_words(int config);
hipError_t launch_stream_read(const void* src, size_t bytes, int config, uint32_t* sink, hipStream_t stream);
// Measurement aid: random gathers of width-byte entries from 128 KB of LDS
// (lds_gather_sink_words() words of sink).
size_t lds_gather_sink_words();
hipError_t launch_lds_gather(int width, int reps, uint32_t* sink, hipStream_t stream);

hipError_t launch_decode_rows(const rq_matrix* W, const int32_t* ids, int n, int out_bf16, void* out,
                              int32_t* bad_ids, hipStream_t stream);
hipError_t launch_pack_codes(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream);
hipError_t launch_pack_codes10(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream);
hipError_t launch_pack_codes8(const uint16_t* src, int64_t rows, int NP, uint16_t* dst, hipStream_t stream);
// The decode loop's glue around an MLP block: h += rms(y) (y may be null), x = rms(h).
hipError_t launch_residual_norm(const float* y, float* h, float* x, int D, float eps, hipStream_t stream);
// Dense comparator: hb is a bf16 copy of h padded to whole 16-vector tiles
// (dense_hb_bytes), written first by the same call.
size_t dense_hb_bytes(int D, int B);
// Et is E[rows][D] tiled as [ceil(rows/16)][ceil(D/32)][16][32] bf16 (dense_tiled_bytes, written by launch_pack_dense).
size_t dense_tiled_bytes(int64_t rows, int D);
hipError_t launch_pack_dense(const uint16_t* E, int64_t rows, int D, uint16_t* Et, hipStream_t stream);
hipError_t launch_dense_logits(const uint16_t* Et, int64_t rows, int D, const float* h, int B, float softcap,
                               float* logits, uint64_t* block_keys, uint16_t* hb, hipStream_t stream);

constexpr int kEpiRowsPerBlock = 1024;   // rows per epilogue workgroup
inline int epi_blocks(int64_t rows) { return (int)((rows + kEpiRowsPerBlock - 1) / kEpiRowsPerBlock); }
constexpr int kDenseRowsPerBlock = 256;
inline int dense_blocks(int64_t rows) { return (int)((rows + kDenseRowsPerBlock - 1) / kDenseRowsPerBlock); }

}  // namespace rq
