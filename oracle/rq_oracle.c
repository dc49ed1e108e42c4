/*
 * rq_oracle.c -- CPU oracle for residual product-quantized (RQ) LUT serving.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow reference that the
 * GPU path is checked against. Only the test suite, the package smoke check
 * and the bench's CPU-baseline leg may load it; the library in
 * lut_logits_amd/ never calls it and shares no code with it.
 *
 * Everything is computed in fp64 from the values exactly as stored (fp32 or
 * bf16 codebooks, fp32 activations), with no blocking, fusion or reordering
 * beyond the definitions below.
 *
 * Definitions (all from the Gemma-2-2B runtime-compression page, "LUT
 * serving" paragraph, which reuses the residual-PQ embedding of the Phase 1
 * page with M=384, K=1024, L=2):
 *   - A matrix W[rows][D] is split into M contiguous subspaces of width d
 *     (D = M*d).  Row r's subvector in subspace m is the sum over L residual
 *     levels of one codeword per level, taken from that level's own codebook
 *     for that subspace:
 *        W[r][m*d + j] = sum_{l<L} C[l][m][ code[r][l][m] ][j].
 *   - Logits of the tied head: z[b][r] = <W[r], h[b]>, followed by Gemma-2's
 *     final-logit softcap  c * tanh(z / c)  (disabled when c <= 0).
 *   - The LUT form: LUT[b][l][m][k] = <h_b restricted to subspace m,
 *     C[l][m][k]>, and z[b][r] = sum_{l,m} LUT[b][l][m][code[r][l][m]].  By
 *     distributivity this equals the decode+matmul form; the page's own
 *     correctness table gates exactly this equivalence (in fp32).
 *   - Input rows are reconstructed on demand by decoding only the requested
 *     token ids.
 *   - MLP weights coded the same way (Gemma-2-2B MLP RQ page) are applied as
 *     plain matrix-vector products; gelu_tanh(t) = 0.5 t (1 + tanh(sqrt(2/pi)
 *     (t + 0.044715 t^3))) joins gate and up projections.
 *
 * Storage layouts (readings taken where the pages are silent):
 *   codes      uint16 [rows][L][M]      (pages: "codes as int16")
 *   codebooks  fp32 or bf16 [L][M][K][d] (pages: small fp32 codebooks; one
 *              per level and subspace, which the page's 412 MB total fixes)
 *   h, x       fp32 [B][D]
 * Argmax takes the lowest index among equal maxima. Top-k orders by value
 * descending, then index ascending.
 *
 * Error returns: 0 ok, -1 null pointer, -2 bad shape, -7 a code >= K.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_NULL -1
#define OR_ERR_SHAPE -2
#define OR_ERR_CODE -7

/* ---- stored values, widened exactly to fp64 ---------------------------- */

static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double codebook_value(const void* cb, int cb_is_bf16, size_t i) {
  if (cb_is_bf16) return bf16_to_double(((const uint16_t*)cb)[i]);
  return (double)((const float*)cb)[i];
}

/* position of C[l][m][k][j] in the [L][M][K][d] codebook array */
static size_t cb_pos(int l, int m, int k, int j, int M, int K, int d) {
  return (((size_t)l * M + m) * (size_t)K + k) * (size_t)d + j;
}

/* position of code[r][l][m] in the [rows][L][M] code array */
static size_t code_pos(int64_t r, int l, int m, int L, int M) {
  return ((size_t)r * L + l) * (size_t)M + m;
}

static int check_shape(int64_t rows, int D, int M, int d, int K, int L) {
  if (rows < 0 || M < 1 || d < 1 || K < 1 || K > 65536 || L < 1) return OR_ERR_SHAPE;
  if ((int64_t)M * d != D) return OR_ERR_SHAPE;
  return OR_OK;
}

/* All codes must index an existing codeword. */
int oracle_check_codes(int64_t rows, int M, int K, int L, const uint16_t* codes) {
  if (!codes && rows > 0) return OR_ERR_NULL;
  size_t n = (size_t)rows * L * M;
  for (size_t i = 0; i < n; ++i)
    if (codes[i] >= K) return OR_ERR_CODE;
  return OR_OK;
}

/* ---- row decode: W[r][m*d+j] = sum_l C[l][m][code[r][l][m]][j] --------- */

void oracle_decode_row(const uint16_t* codes, const void* cb, int cb_is_bf16, int64_t r,
                       int M, int d, int K, int L, double* w) {
  for (int m = 0; m < M; ++m) {
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int l = 0; l < L; ++l) {
        int k = codes[code_pos(r, l, m, L, M)];
        s += codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d));
      }
      w[(size_t)m * d + j] = s;
    }
  }
}

/* ---- softcap and activation ------------------------------------------- */

double oracle_softcap(double z, double c) {
  if (c <= 0.0) return z;
  return c * tanh(z / c);
}

double oracle_gelu_tanh(double t) {
  const double k = sqrt(2.0 / M_PI);
  return 0.5 * t * (1.0 + tanh(k * (t + 0.044715 * t * t * t)));
}

/* a[i] = gelu_tanh(g[i]) * u[i] */
void oracle_gelu_mul(const double* g, const double* u, int64_t n, double* a) {
  for (int64_t i = 0; i < n; ++i) a[i] = oracle_gelu_tanh(g[i]) * u[i];
}

/* ---- matrix-vector products by direct decode ------------------------- */

/*
 * y[b][r] = sum_{i<D} W[r][i] * x[b][i] for every row r, with W decoded row by
 * row in fp64. x is fp64 [B][D]; y is fp64 [B][rows].
 */
int oracle_matvec(int64_t rows, int D, int M, int d, int K, int L,
                  const void* cb, int cb_is_bf16, const uint16_t* codes,
                  const double* x, int B, double* y, int nthreads) {
  if (check_shape(rows, D, M, d, K, L) != OR_OK || B < 0) return OR_ERR_SHAPE;
  if (rows == 0 || B == 0) return OR_OK;
  if (!cb || !codes || !x || !y) return OR_ERR_NULL;
  int rc = oracle_check_codes(rows, M, K, L, codes);
  if (rc != OR_OK) return rc;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      oracle_decode_row(codes, cb, cb_is_bf16, r, M, d, K, L, w);
      for (int b = 0; b < B; ++b) {
        const double* xb = x + (size_t)b * D;
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += w[i] * xb[i];
        y[(size_t)b * rows + r] = acc;
      }
    }
    free(w);
  }
  return OR_OK;
}

/*
 * Head logits by direct decode + matmul, then the softcap.
 * h is fp32 [B][D] (widened exactly); z and logits are fp64 [B][V].
 * z may be NULL.
 */
int oracle_logits(int64_t V, int D, int M, int d, int K, int L,
                  const void* cb, int cb_is_bf16, const uint16_t* codes,
                  const float* h, int B, double softcap,
                  double* z, double* logits, int nthreads) {
  if (check_shape(V, D, M, d, K, L) != OR_OK || B < 0) return OR_ERR_SHAPE;
  if (V == 0 || B == 0) return OR_OK;
  if (!h || !logits) return OR_ERR_NULL;
  double* x = (double*)malloc(sizeof(double) * (size_t)B * D);
  double* zz = z ? z : (double*)malloc(sizeof(double) * (size_t)B * V);
  for (size_t i = 0; i < (size_t)B * D; ++i) x[i] = (double)h[i];
  int rc = oracle_matvec(V, D, M, d, K, L, cb, cb_is_bf16, codes, x, B, zz, nthreads);
  if (rc == OR_OK)
    for (size_t i = 0; i < (size_t)B * V; ++i) logits[i] = oracle_softcap(zz[i], softcap);
  if (!z) free(zz);
  free(x);
  return rc;
}

/* ---- the LUT form ---------------------------------------------------- */

/*
 * LUT[b][l][m][k] = sum_{j<d} x[b][m*d+j] * C[l][m][k][j]   (fp64, [B][L][M][K])
 */
int oracle_build_lut(int D, int M, int d, int K, int L, const void* cb, int cb_is_bf16,
                     const double* x, int B, double* lut) {
  if (check_shape(0, D, M, d, K, L) != OR_OK || B < 0) return OR_ERR_SHAPE;
  if (B == 0) return OR_OK;
  if (!cb || !x || !lut) return OR_ERR_NULL;
  for (int b = 0; b < B; ++b)
    for (int l = 0; l < L; ++l)
      for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
          double s = 0.0;
          for (int j = 0; j < d; ++j)
            s += x[(size_t)b * D + (size_t)m * d + j] * codebook_value(cb, cb_is_bf16, cb_pos(l, m, k, j, M, K, d));
          lut[(((size_t)b * L + l) * M + m) * (size_t)K + k] = s;
        }
  return OR_OK;
}

/*
 * z[b][r] = sum_{l<L} sum_{m<M} LUT[b][l][m][code[r][l][m]]   (fp64)
 */
int oracle_lut_sum(int64_t rows, int M, int K, int L, const uint16_t* codes,
                   const double* lut, int B, double* z, int nthreads) {
  if (rows < 0 || M < 1 || K < 1 || L < 1 || B < 0) return OR_ERR_SHAPE;
  if (rows == 0 || B == 0) return OR_OK;
  if (!codes || !lut || !z) return OR_ERR_NULL;
  int rc = oracle_check_codes(rows, M, K, L, codes);
  if (rc != OR_OK) return rc;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < B; ++b) {
      double acc = 0.0;
      for (int l = 0; l < L; ++l)
        for (int m = 0; m < M; ++m) {
          int k = codes[code_pos(r, l, m, L, M)];
          acc += lut[(((size_t)b * L + l) * M + m) * (size_t)K + k];
        }
      z[(size_t)b * rows + r] = acc;
    }
  }
  return OR_OK;
}

/* ---- selection --------------------------------------------------------- */

/* out[b] = lowest index v with logits[b][v] maximal (NaN-free input). */
void oracle_argmax(const double* logits, int B, int64_t V, int32_t* out) {
  for (int b = 0; b < B; ++b) {
    const double* row = logits + (size_t)b * V;
    int64_t best = 0;
    for (int64_t v = 1; v < V; ++v)
      if (row[v] > row[best]) best = v;
    out[b] = (int32_t)best;
  }
}

typedef struct { double val; int64_t id; } scored;

static int by_value_then_id(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->val > b->val) return -1;
  if (a->val < b->val) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id);
}

/* The k best entries of each row, ordered by value descending then id ascending. */
int oracle_topk(const double* logits, int B, int64_t V, int k, int32_t* ids, double* vals) {
  if (k < 0 || k > V) return OR_ERR_SHAPE;
  scored* s = (scored*)malloc(sizeof(scored) * (size_t)(V > 0 ? V : 1));
  for (int b = 0; b < B; ++b) {
    for (int64_t v = 0; v < V; ++v) { s[v].val = logits[(size_t)b * V + v]; s[v].id = v; }
    qsort(s, (size_t)V, sizeof(scored), by_value_then_id);
    for (int i = 0; i < k; ++i) {
      ids[(size_t)b * k + i] = (int32_t)s[i].id;
      if (vals) vals[(size_t)b * k + i] = s[i].val;
    }
  }
  free(s);
  return OR_OK;
}

/* ---- on-demand row decode with output rounding ------------------------ */

/* fp32 bit pattern -> bf16 bit pattern, round to nearest, ties to even. */
static uint16_t fp32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/*
 * out[i][:] = decoded row ids[i], rounded once to fp32 (out_is_bf16 == 0) or
 * to fp32 then bf16 (out_is_bf16 == 1). Ids outside [0, V) give a zero row and
 * are counted in *bad.
 */
int oracle_decode_rows(int64_t V, int D, int M, int d, int K, int L,
                       const void* cb, int cb_is_bf16, const uint16_t* codes,
                       const int32_t* ids, int n, int out_is_bf16, void* out, int64_t* bad) {
  if (check_shape(V, D, M, d, K, L) != OR_OK || n < 0) return OR_ERR_SHAPE;
  if (n == 0) return OR_OK;
  if (!ids || !out) return OR_ERR_NULL;
  double* w = (double*)malloc(sizeof(double) * (size_t)D);
  int64_t nbad = 0;
  for (int i = 0; i < n; ++i) {
    int64_t r = ids[i];
    int ok = (r >= 0 && r < V);
    if (ok) {
      for (int l = 0; l < L; ++l)
        for (int m = 0; m < M; ++m)
          if (codes[code_pos(r, l, m, L, M)] >= K) { free(w); return OR_ERR_CODE; }
      oracle_decode_row(codes, cb, cb_is_bf16, r, M, d, K, L, w);
    } else {
      ++nbad;
      for (int c = 0; c < D; ++c) w[c] = 0.0;
    }
    for (int c = 0; c < D; ++c) {
      float f = (float)w[c];
      if (out_is_bf16) ((uint16_t*)out)[(size_t)i * D + c] = fp32_to_bf16_rne(f);
      else ((float*)out)[(size_t)i * D + c] = f;
    }
  }
  free(w);
  if (bad) *bad = nbad;
  return OR_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
