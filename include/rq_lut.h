/*
 * rq_lut.h -- C ABI of librq_lut.so: serving residual product-quantized (RQ)
 * matrices on an MI355X (gfx950) without ever rebuilding the dense matrix.
 *
 * The operations are the ones the Gemma-2-2B runtime-compression page
 * describes in its "LUT serving" paragraph, for the tied embedding / LM head
 * coded with M=384 subspaces, K=1024 codewords and L=2 residual levels:
 *   - output logits by lookup+sum in place of a full matmul, handed to
 *     Gemma-2's own softcap            -> rq_build_lut + rq_lut_logits
 *   - input rows reconstructed on demand, a handful per prompt
 *                                      -> rq_decode_rows
 * and the non-materialising path for RQ-coded MLP weights that the Gemma-2-2B
 * MLP RQ page names as its natural follow-up   -> rq_lut_matvec (one matrix)
 *                                                 and rq_lut_mlp (a whole block).
 *
 * The coded matrix. W[rows][D] with D = M*d is split into M contiguous
 * subspaces of width d; row r's subvector in subspace m is the sum over L
 * residual levels of one codeword per level from that level's own codebook:
 *     W[r][m*d + j] = sum_{l<L} C[l][m][ codes[r][l][m] ][j].
 * (Residual PQ: runtime-compression page, opening and LUT-serving
 * paragraphs; one codebook per level and subspace is what makes the page's
 * 412 MB artifact add up.)
 *
 * Conventions for every entry point:
 *   - Memory. All array pointers are DEVICE pointers owned by the caller. The
 *     library allocates nothing, keeps no state between calls (apart from the
 *     thread-local text behind rq_last_error) and never synchronises: work is
 *     enqueued on `stream` and completes asynchronously. (The measurement
 *     aids of rq_lut_measure.h are outside these serving calls.)
 *   - Errors. Arguments are checked on the host before anything is launched;
 *     a failed check returns a negative rq_status and enqueues nothing. A
 *     failed launch returns RQ_ERR_HIP. rq_last_error() describes the last
 *     failure on the calling thread.
 *   - Empty work. B == 0, n == 0 or rows == 0 return RQ_OK and enqueue
 *     nothing.
 *   - Codes must be < K. A larger code breaks that precondition: the lookup
 *     kernels then read some other entry of their on-chip table or codebook
 *     copy (the result is undefined) and rq_decode_rows reads it as K-1; no
 *     call reads or writes memory outside the arrays it is given.
 *   - Alignment. codes and lut must be 16-byte aligned, other arrays 4-byte
 *     aligned, workspaces 256-byte aligned (torch allocations satisfy this).
 *   - Workspaces hold per-call scratch only (no state carries over between
 *     calls, no initial contents are required). Calls that overlap in time
 *     must not share a workspace. A workspace may be NULL when its query
 *     returns 0.
 *   - Concurrency. Calls on different streams may run concurrently as long as
 *     they do not share output or workspace buffers.
 */
#ifndef RQ_LUT_H
#define RQ_LUT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rq_status {
  RQ_OK = 0,
  RQ_ERR_NULL = -1,       /* a required pointer is NULL                        */
  RQ_ERR_SHAPE = -2,      /* inconsistent or unsupported sizes                 */
  RQ_ERR_DTYPE = -3,      /* unknown dtype / prologue value                    */
  RQ_ERR_ALIGN = -4,      /* a pointer misses its required alignment           */
  RQ_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than the query returned */
  RQ_ERR_HIP = -6         /* a HIP launch failed                               */
} rq_status;

typedef enum rq_dtype { RQ_F32 = 0, RQ_BF16 = 1 } rq_dtype;

typedef enum rq_prologue {
  RQ_PRO_NONE = 0,          /* the activation is x                                    */
  RQ_PRO_GELU_TANH_MUL = 1  /* the activation is gelu_tanh(x) * x2 (Gemma-2 MLP down) */
} rq_prologue;

/*
 * Code layouts. The pages fix only that codes are 16-bit integers; the order
 * in memory is this library's choice. With NP = L*M (level, subspace) pairs
 * numbered p = l*M + m:
 *   RQ_CODES_ROWS     codes[r][l][m]: uint16 [rows][NP], the interchange layout
 *   RQ_CODES_BLOCKED  codes[p/8][r][p%8]: uint16 [ceil(NP/8)][rows][8]; each
 *                     row's codes for 8 consecutive pairs are 16 contiguous
 *                     bytes, and consecutive rows are adjacent. Unused slots
 *                     of the last block (NP not a multiple of 8) are 0.
 *   RQ_CODES_PACKED10 the 10-bit code stream (K <= 1024): [ceil(NP/12)][rows]
 *                     of 16 bytes; in block q, 32-bit word w of a row holds
 *                     the codes of pairs 12q + 3w + i at bits [10i, 10i+10),
 *                     i < 3 (bits 30-31 and unused slots are 0). 1024 bytes
 *                     per Gemma-head row instead of 1536, the 10-bit packing
 *                     behind the runtime-compression page's 265 MB artifact,
 *                     laid out so every load stays 16-byte aligned and every
 *                     code is one bit-field extract.
 *   RQ_CODES_PACKED8  the 8-bit code stream (K <= 256): [ceil(NP/16)][rows]
 *                     of 16 bytes; in block q, byte i of a row holds the code
 *                     of pair 16q + i (unused slots are 0). The uint8 codes of
 *                     the MLP RQ page's K=256 down projections.
 * Every entry point reads all four. BLOCKED and PACKED10 are serving layouts:
 * a wave loads 64 rows x 16 bytes as one contiguous 1 KB run, whatever chunk of
 * pairs it works on. rq_pack_codes, rq_pack_codes10 and rq_pack_codes8 convert
 * ROWS to them once, at load. With RQ_CODES_ROWS, rq_lut_logits and rq_lut_matvec need
 * NP % 8 == 0.
 */
typedef enum rq_codes_layout {
  RQ_CODES_ROWS = 0,
  RQ_CODES_BLOCKED = 1,
  RQ_CODES_PACKED10 = 2,
  RQ_CODES_PACKED8 = 3
} rq_codes_layout;

/*
 * Non-owning description of one RQ-coded matrix W[rows][D].
 *   rows          vocabulary size V for a head, out_features for an MLP matrix,
 *                 0 <= rows < 2^29
 *   D, M, d       D == M*d, all >= 1
 *   K             codewords per codebook, 1 <= K <= 65536 (but see RQ_MAX_K_F32)
 *   L             residual levels, 1 <= L <= RQ_MAX_L
 *   cb_dtype      RQ_F32 or RQ_BF16, the storage type of the codebooks
 *   codes_layout  RQ_CODES_ROWS, RQ_CODES_BLOCKED, RQ_CODES_PACKED10 (K <= 1024)
 *                 or RQ_CODES_PACKED8 (K <= 256)
 *   codebooks     device [L][M][K][d] of cb_dtype
 *   codes         device uint16 in codes_layout, 16-byte aligned
 */
typedef struct rq_matrix {
  int64_t rows;
  int32_t D, M, d, K, L;
  int32_t cb_dtype;
  int32_t codes_layout;
  const void* codebooks;
  const uint16_t* codes;
} rq_matrix;

/* Bytes of the RQ_CODES_BLOCKED layout: ceil(L*M/8) * rows * 16. */
size_t rq_blocked_codes_bytes(int64_t rows, int32_t L, int32_t M);

/*
 * Convert codes from RQ_CODES_ROWS (src, uint16 [rows][L*M]) to
 * RQ_CODES_BLOCKED (dst, rq_blocked_codes_bytes bytes). src and dst must not
 * overlap. A pure permutation: the codes are copied bit for bit.
 */
rq_status rq_pack_codes(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst,
                        hipStream_t stream);

/* Bytes of the RQ_CODES_PACKED10 layout: ceil(L*M/12) * rows * 16. */
size_t rq_packed10_codes_bytes(int64_t rows, int32_t L, int32_t M);

/*
 * Convert codes from RQ_CODES_ROWS (src, uint16 [rows][L*M]) to
 * RQ_CODES_PACKED10 (dst, rq_packed10_codes_bytes bytes). Codes must be below
 * 1024 (a precondition: the bits above the tenth are dropped). src and dst
 * must not overlap.
 */
rq_status rq_pack_codes10(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst,
                          hipStream_t stream);

/* Bytes of the RQ_CODES_PACKED8 layout: ceil(L*M/16) * rows * 16. */
size_t rq_packed8_codes_bytes(int64_t rows, int32_t L, int32_t M);

/*
 * Convert codes from RQ_CODES_ROWS (src, uint16 [rows][L*M]) to
 * RQ_CODES_PACKED8 (dst, rq_packed8_codes_bytes bytes). Codes must be below
 * 256 (a precondition: the bits above the eighth are dropped). src and dst
 * must not overlap.
 */
rq_status rq_pack_codes8(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst,
                         hipStream_t stream);

/* Largest K whose per-subspace table (K entries) fits the kernels' on-chip
 * staging: 32768 for fp32 tables, 65536 for bf16 tables. */
#define RQ_MAX_K_F32 32768
#define RQ_MAX_K_BF16 65536
#define RQ_MAX_L 16

/*
 * Bytes of the lookup table rq_build_lut writes for B activation vectors:
 * L*M*K*B elements of lut_dtype. Returns 0 for invalid arguments.
 */
size_t rq_lut_bytes(const rq_matrix* W, int32_t B, int32_t lut_dtype);

/*
 * Build the lookup table of each activation vector (runtime-compression page,
 * LUT-serving paragraph: logits by lookup+sum):
 *     LUT[l][m][k][b] = sum_{j<d} a[b][m*d + j] * C[l][m][k][j]
 * with a = x (prologue RQ_PRO_NONE) or a = gelu_tanh(x) * x2 elementwise
 * (RQ_PRO_GELU_TANH_MUL; gelu_tanh(t) = 0.5 t (1 + tanh(sqrt(2/pi) (t +
 * 0.044715 t^3)))), computed in fp32 and stored as lut_dtype (bf16: round to
 * nearest even).
 *   x, x2   device fp32 [B][D] (x2 only read with the GELU prologue)
 *   lut     device, rq_lut_bytes(W, B, lut_dtype) bytes, layout [L][M][K][B]
 *           (the batch index innermost)
 * W->codes is not read and may be NULL.
 */
rq_status rq_build_lut(const rq_matrix* W, const float* x, const float* x2, int32_t prologue,
                       int32_t B, int32_t lut_dtype, void* lut, hipStream_t stream);

/*
 * Workspace bytes rq_lut_logits needs for this matrix, batch, top-k size and
 * table dtype (0 for invalid arguments).
 */
size_t rq_lut_logits_workspace(const rq_matrix* W, int32_t B, int32_t topk, int32_t lut_dtype);

/*
 * Head logits by lookup+sum, then Gemma-2's final-logit softcap and the
 * selection of the next token (runtime-compression page, LUT-serving
 * paragraph):
 *     z[b][r]      = sum_{l<L} sum_{m<M} LUT[l][m][codes[r][l][m]][b]   (fp32)
 *     logits[b][r] = softcap * tanh(z[b][r] / softcap)   (softcap <= 0: z)
 *     argmax[b]    = lowest r with the largest logits[b][r]
 *     top-k        = the topk largest logits of each b, ordered by value
 *                    descending then index ascending
 *   lut        the table rq_build_lut wrote for the same W and B
 *   logits     device fp32 [B][rows], or NULL to skip storing logits
 *   argmax     device int32 [B], or NULL
 *   topk       0 (no top-k) or 1..min(rows, 1024); topk_ids int32 [B][topk]
 *              and topk_vals fp32 [B][topk] (topk_vals may be NULL)
 *   ws         device workspace of at least rq_lut_logits_workspace() bytes
 * Each logit is summed in a fixed order, so repeated calls give
 * bit-identical results; argmax and top-k are taken on the fp32 logits the
 * call produces. Rows with equal logits are selected by lowest index.
 */
rq_status rq_lut_logits(const rq_matrix* W, const void* lut, int32_t lut_dtype, int32_t B,
                        float softcap, float* logits, int32_t* argmax, int32_t topk,
                        int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * rq_lut_logits for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results as rq_lut_logits, without the
 * workspace: the call uses a scratch array of RQ_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on (allocated with the code object, kept
 * until the process ends) and calls no allocator.
 *   - A call that needs more scratch than that (rq_lut_logits_workspace is
 *     the measure; the B=1 Gemma head with top-50 needs about 4.2 MB) returns
 *     RQ_ERR_WORKSPACE and enqueues nothing.
 *   - The scratch is per GPU (the calling thread's current device, which must
 *     own `stream`) and shared by every call on it: calls that overlap in time
 *     on one GPU race, whatever their streams. Nothing in it must start at zero.
 */
#define RQ_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
rq_status rq_lut_logits_static(const rq_matrix* W, const void* lut, int32_t lut_dtype, int32_t B,
                               float softcap, float* logits, int32_t* argmax, int32_t topk,
                               int32_t* topk_ids, float* topk_vals, hipStream_t stream);

/*
 * One-call head: the same logits, argmax and top-k as rq_build_lut followed by
 * rq_lut_logits with an fp32 table, computed from the hidden vectors directly
 * (runtime-compression page, LUT-serving paragraph; the sum is regrouped by
 * distributivity, which is exact in exact arithmetic):
 *     z[b][r] = sum_{l<L} sum_{m<M} < C[l][m][codes[r][l][m]], h[b][m*d .. m*d+d) >
 * The library picks the method from the shapes:
 *   - the table path (rq_build_lut into the workspace, then the lookup+sum);
 *   - for B >= RQ_MM_MIN_B with bf16 codebooks, even d <= 8, K <= 1024 and
 *     RQ_CODES_BLOCKED codes: the codebooks are staged on chip and the
 *     contraction with h runs on the matrix cores, h split exactly into three
 *     bf16 parts (fp32-level accuracy, like the fp32 table).
 *   h       device fp32 [B][D]
 *   other arguments as for rq_lut_logits; ws of at least rq_logits_workspace()
 *   bytes.
 * Results are deterministic for a given (W, B) but, being summed in a
 * different order, are not bit-identical to the two-call form.
 */
#define RQ_MM_MIN_B 8
#define RQ_METHOD_TABLE 0
#define RQ_METHOD_MATRIX_CORES 1
/* The method rq_logits uses for this matrix and batch (RQ_METHOD_*), or a
 * negative rq_status for invalid arguments. */
int32_t rq_logits_method(const rq_matrix* W, int32_t B);
size_t rq_logits_workspace(const rq_matrix* W, int32_t B, int32_t topk);
rq_status rq_logits(const rq_matrix* W, const float* h, int32_t B, float softcap, float* logits,
                    int32_t* argmax, int32_t topk, int32_t* topk_ids, float* topk_vals, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * On-demand reconstruction of selected rows (runtime-compression page,
 * LUT-serving paragraph: input token rows rebuilt on demand):
 *     out[i][m*d + j] = sum_{l<L} C[l][m][codes[ids[i]][l][m]][j]
 * summed in fp64 in level order, rounded once to fp32, then (out_dtype
 * RQ_BF16) rounded to bf16 to nearest even.
 *   ids      device int32 [n]; an id outside [0, rows) yields a zero row and,
 *            when bad_ids is not NULL, one atomic increment of *bad_ids
 *   out      device [n][D] of out_dtype
 *   bad_ids  device int32 counter or NULL (not reset by the call)
 */
rq_status rq_decode_rows(const rq_matrix* W, const int32_t* ids, int32_t n, int32_t out_dtype,
                         void* out, int32_t* bad_ids, hipStream_t stream);

/*
 * Workspace bytes rq_lut_matvec needs (the fp32 table and partial
 * sums).
 */
size_t rq_lut_matvec_workspace(const rq_matrix* W, int32_t B);

/*
 * Matrix-vector product with an RQ-coded weight, by lookup+sum, never
 * materialising W (the non-materialising MLP path of the Gemma-2-2B MLP RQ
 * page, final paragraphs):
 *     y[b][r] = sum_{l,m} LUT_a[l][m][codes[r][l][m]][b] = <W[r], a[b]>
 * with a = x or a = gelu_tanh(x) * x2 as in rq_build_lut, fp32 table and fp32
 * sums. A Gemma-2 MLP block is three calls: g = gate(x), u = up(x),
 * y = down(gelu_tanh(g) * u) via RQ_PRO_GELU_TANH_MUL.
 *   x, x2  device fp32 [B][D];  y  device fp32 [B][rows]
 *   ws     device workspace of at least rq_lut_matvec_workspace() bytes
 */
rq_status rq_lut_matvec(const rq_matrix* W, const float* x, const float* x2, int32_t prologue,
                        int32_t B, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * A whole Gemma-2 MLP block with RQ-coded weights (MLP RQ page, final
 * paragraphs: the three projections as LUT matvecs):
 *     y = down( gelu_tanh(gate(x)) * up(x) )
 * with the arithmetic of the three rq_lut_matvec calls. With one activation
 * vector and fused table builds (fp32 codebooks, d in {1, 2, 4, 8}) it takes
 * three launches instead of six: gate and up in one lookup+sum launch, down
 * with its activation summed straight from their partial sums in the finish
 * pass's order, then down's finish. Gate and up may then be split into a
 * different (fixed) number of partial sums than a single call would use, so
 * the result agrees with the three calls to fp32 rounding (exactly when no sum
 * rounds) and is deterministic. Otherwise it runs the three matvecs.
 *   gate, up  same rows, D, M, d, K, L, codebook dtype and code layout
 *   down      down->D == gate->rows
 *   x         device fp32 [B][gate->D];  y  device fp32 [B][down->rows]
 *   ws        device workspace of at least rq_lut_mlp_workspace() bytes,
 *             256-byte aligned
 * Shape mismatches return RQ_ERR_SHAPE; other checks as rq_lut_matvec.
 */
size_t rq_lut_mlp_workspace(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, int32_t B);
rq_status rq_lut_mlp(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, const float* x,
                     int32_t B, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Comparison baseline: the standard dense path with the head stored as a
 * dense bf16 matrix E[rows][D], as deployed before LUT serving
 * (runtime-compression page, variant table "Uncompressed" row):
 *     logits[b][r] = softcap(sum_i E[r][i] * bf16(h[b][i])) in fp32, plus argmax
 * (a GEMV at B=1, a GEMM on the matrix cores for larger batches).
 *
 * The matrix is held tiled: Et = [ceil(rows/16)][ceil(D/32)][16][32] bf16,
 * zero past rows and D, so each 16-row x 32-column tile is one contiguous
 * 1 KB block (one wave-wide load of the matrix-core operand).
 * rq_dense_tiled_bytes gives its size (0 when rows <= 0 or D is out of range);
 * rq_pack_dense writes it, stream-ordered, from row-major E:
 *   E       device bf16 bit patterns [rows][D], 16-byte aligned, D % 8 == 0,
 *           8 <= D <= 4096; rows < 2^31
 *   Et      device, 16-byte aligned, rq_dense_tiled_bytes(rows, D) bytes,
 *           not overlapping E
 * rq_dense_logits:
 *   Et      the tiled matrix of rows x D written by rq_pack_dense
 *   h       device fp32 [B][D], 0 <= B <= 128
 *   logits  device fp32 [B][rows] (required); argmax device int32 [B] or NULL
 *   ws      device workspace of at least rq_dense_logits_workspace() bytes
 *           (the bf16 copy of h and the per-block selection keys)
 * Shapes out of range return RQ_ERR_SHAPE, NULL buffers RQ_ERR_NULL,
 * misaligned ones RQ_ERR_ALIGN, a short workspace RQ_ERR_WORKSPACE.
 */
size_t rq_dense_tiled_bytes(int64_t rows, int32_t D);
rq_status rq_pack_dense(const uint16_t* E, int64_t rows, int32_t D, uint16_t* Et, hipStream_t stream);
size_t rq_dense_logits_workspace(int64_t rows, int32_t B);
rq_status rq_dense_logits(const uint16_t* Et, int64_t rows, int32_t D, const float* h, int32_t B,
                          float softcap, float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                          hipStream_t stream);


/*
 * Glue of a per-token decode loop around each MLP block (not part of the
 * pages' method: Gemma-2's residual stream, read in its plainest form), in one
 * launch on the residual stream h, with the unit-scale RMSNorm
 *     rms(v) = v / sqrt(mean(v^2) + eps):
 *     if y != NULL:  h += rms(y)   (a block's output, normalised, added back)
 *     x = rms(h)                   (the next block's input, or the head's vector)
 *   y   device fp32 [D] or NULL; h device fp32 [D], updated in place;
 *   x   device fp32 [D], written; x must not overlap h or y;
 *   1 <= D <= 1048576, eps > 0. All 4-byte aligned. One workgroup, stream-ordered.
 * Bad sizes return RQ_ERR_SHAPE, NULL h or x RQ_ERR_NULL, misaligned buffers
 * RQ_ERR_ALIGN.
 */
rq_status rq_residual_norm(const float* y, float* h, float* x, int32_t D, float eps, hipStream_t stream);

/* Static text for a status code. Takes any int (an rq_status value converts
 * to it); a value that is no rq_status gives "unknown status". */
const char* rq_status_string(int32_t s);
/* Description of the last failure on the calling thread ("" if none). */
const char* rq_last_error(void);
/* Library version, "major.minor.patch". */
const char* rq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_LUT_H */
