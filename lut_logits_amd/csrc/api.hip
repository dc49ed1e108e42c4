// api.hip -- the C ABI of librq_lut.so (declared in include/rq_lut.h).
//
// Host-side argument checks (run before anything is launched), workspace
// sizing and the launch sequence of each entry point. No allocation, no
// synchronisation: everything is enqueued on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "rq_internal.h"

// The scratch of rq_lut_logits_static: one copy per GPU the library runs on,
// held until the process ends. Host code uses the device address that
// hipGetSymbolAddress gives for the current device (static_scratch below),
// never this name, which on the host is only a stand-in for the symbol.
__device__ __align__(256) unsigned char scratch[RQ_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_stage_before = nullptr, g_stage_after = nullptr;

rq_status fail(rq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

rq_status launched(hipError_t e, const char* what) {
  if (e == hipSuccess) return RQ_OK;
  return fail(RQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A roctx range named for the entry point, open for the call (argument checks
// and launches; the kernels themselves run later, on the caller's stream).
// With no profiler attached a push or pop costs a few nanoseconds.
struct CallRange {
  explicit CallRange(const char* name) { roctxRangePushA(name); }
  ~CallRange() { roctxRangePop(); }
  CallRange(const CallRange&) = delete;
  CallRange& operator=(const CallRange&) = delete;
};

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

bool valid_dtype(int32_t t) { return t == RQ_F32 || t == RQ_BF16; }

// Shape, dtype, layout and pointer checks of a matrix descriptor.
rq_status check_matrix(const rq_matrix* W, bool need_codes) {
  if (!W) return fail(RQ_ERR_NULL, "matrix descriptor is NULL");
  if (W->rows < 0 || W->rows >= ((int64_t)1 << 29)) return fail(RQ_ERR_SHAPE, "rows=%lld out of range", (long long)W->rows);
  if (W->M < 1 || W->d < 1 || (int64_t)W->M * W->d != W->D)
    return fail(RQ_ERR_SHAPE, "need D == M*d with M, d >= 1 (D=%d M=%d d=%d)", W->D, W->M, W->d);
  if (W->K < 1 || W->K > 65536) return fail(RQ_ERR_SHAPE, "K=%d outside [1, 65536]", W->K);
  if (W->L < 1 || W->L > RQ_MAX_L) return fail(RQ_ERR_SHAPE, "L=%d outside [1, %d]", W->L, RQ_MAX_L);
  if ((int64_t)W->L * W->M > (1 << 24)) return fail(RQ_ERR_SHAPE, "L*M=%lld too large", (long long)W->L * W->M);
  if (!valid_dtype(W->cb_dtype)) return fail(RQ_ERR_DTYPE, "unknown codebook dtype %d", W->cb_dtype);
  if (W->codes_layout != RQ_CODES_ROWS && W->codes_layout != RQ_CODES_BLOCKED &&
      W->codes_layout != RQ_CODES_PACKED10 && W->codes_layout != RQ_CODES_PACKED8)
    return fail(RQ_ERR_DTYPE, "unknown codes layout %d", W->codes_layout);
  if (W->codes_layout == RQ_CODES_PACKED10 && W->K > 1024)
    return fail(RQ_ERR_SHAPE, "10-bit packed codes need K <= 1024 (K=%d)", W->K);
  if (W->codes_layout == RQ_CODES_PACKED8 && W->K > 256)
    return fail(RQ_ERR_SHAPE, "8-bit packed codes need K <= 256 (K=%d)", W->K);
  if (!W->codebooks) return fail(RQ_ERR_NULL, "codebooks is NULL");
  if (!aligned(W->codebooks, W->cb_dtype == RQ_F32 ? 4 : 2)) return fail(RQ_ERR_ALIGN, "codebooks misaligned");
  if (need_codes) {
    if (!W->codes) return fail(RQ_ERR_NULL, "codes is NULL");
    if (!aligned(W->codes, 16)) return fail(RQ_ERR_ALIGN, "codes must be 16-byte aligned");
  }
  return RQ_OK;
}

size_t lut_elems(const rq_matrix* W, int32_t B) { return (size_t)W->L * W->M * W->K * (size_t)B; }

// Largest K the lookup kernels can stage for one (level, subspace) pair.
rq_status check_table_fits(const rq_matrix* W, int lut_bf16) {
  const int kmax = lut_bf16 ? RQ_MAX_K_BF16 : RQ_MAX_K_F32;
  if (W->K > kmax) return fail(RQ_ERR_SHAPE, "K=%d exceeds %d for %s tables", W->K, kmax, lut_bf16 ? "bf16" : "fp32");
  return RQ_OK;
}

// Workspace of rq_lut_logits, in this order (each part 256-byte aligned):
//   partial sums [G][B][rows] fp32 (G > 1 only), a logits scratch [B][rows]
//   fp32 (top-k without a logits output), the per-block selection keys
//   [B][key_blocks] uint64, the top-k candidates [B][nblk][topk] uint64 and,
//   with more than one batch tile, the batch-tiled copy of the table.
struct LogitsWs {
  size_t partial, scratch, keys, cand, tiled, total;
};

// Bytes of the batch-tiled copy of the table (launch_tile_lut) that a plan
// with more than one batch tile stages from; 0 otherwise.
size_t tiled_bytes(const rq_matrix* W, const rq::GatherPlan& plan, bool lut_bf16) {
  if (plan.NBT <= 1) return 0;
  return round_up((size_t)plan.NBT * W->L * W->M * W->K * plan.BT * (lut_bf16 ? 2 : 4), 256);
}

LogitsWs logits_ws(const rq_matrix* W, const rq::GatherPlan& plan, int32_t B, int32_t topk, bool logits_out,
                   bool lut_bf16) {
  LogitsWs w;
  w.partial = 0;
  w.scratch = w.partial + (plan.G > 1 ? round_up((size_t)plan.G * B * W->rows * sizeof(float), 256) : 0);
  w.keys = w.scratch + (topk > 0 && !logits_out ? round_up((size_t)B * W->rows * sizeof(float), 256) : 0);
  w.cand = w.keys + round_up((size_t)B * rq::key_blocks(plan, W->rows) * sizeof(uint64_t), 256);
  w.tiled = w.cand + (topk > 0 ? round_up((size_t)B * rq::epi_blocks(W->rows) * topk * sizeof(uint64_t), 256) : 0);
  w.total = w.tiled + tiled_bytes(W, plan, lut_bf16);
  return w;
}

rq_status check_lut_call(const rq_matrix* W, int32_t B, int32_t lut_dtype) {
  rq_status s = check_matrix(W, true);
  if (s != RQ_OK) return s;
  if (B < 0 || B > 65535) return fail(RQ_ERR_SHAPE, "B=%d outside [0, 65535]", B);
  if (!valid_dtype(lut_dtype)) return fail(RQ_ERR_DTYPE, "unknown table dtype %d", lut_dtype);
  s = check_table_fits(W, lut_dtype == RQ_BF16);
  if (s != RQ_OK) return s;
  if (W->codes_layout == RQ_CODES_ROWS && ((W->L * W->M) & 7))
    return fail(RQ_ERR_ALIGN, "row-major codes need L*M %% 8 == 0 (L*M=%d); pack them with rq_pack_codes", W->L * W->M);
  const int64_t ppb = rq::pairs_per_block(W);
  const int64_t code_bytes = W->codes_layout == RQ_CODES_ROWS ? W->rows * (int64_t)W->L * W->M * 2
                                                              : W->rows * (((int64_t)W->L * W->M + ppb - 1) / ppb) * 16;
  if (code_bytes >= ((int64_t)1 << 32))
    return fail(RQ_ERR_SHAPE, "code array of %lld bytes exceeds the 4 GiB a lookup pass addresses", (long long)code_bytes);
  return RQ_OK;
}

}  // namespace

namespace rq {
void take_stage_events(hipEvent_t* before, hipEvent_t* after) {
  *before = g_stage_before;
  *after = g_stage_after;
  g_stage_before = g_stage_after = nullptr;
}
}  // namespace rq

extern "C" {

const char* rq_version(void) { return "0.1.0"; }

rq_status rq_set_stage_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr)) return fail(RQ_ERR_NULL, "rq_set_stage_events: both events or neither");
  g_stage_before = before;
  g_stage_after = after;
  return RQ_OK;
}

const char* rq_last_error(void) { return g_last_error; }

const char* rq_status_string(int32_t s) {
  switch (s) {
    case RQ_OK: return "ok";
    case RQ_ERR_NULL: return "null pointer";
    case RQ_ERR_SHAPE: return "bad shape";
    case RQ_ERR_DTYPE: return "bad dtype";
    case RQ_ERR_ALIGN: return "misaligned pointer";
    case RQ_ERR_WORKSPACE: return "workspace too small";
    case RQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

size_t rq_blocked_codes_bytes(int64_t rows, int32_t L, int32_t M) {
  if (rows < 0 || L < 1 || M < 1) return 0;
  return (size_t)(((int64_t)L * M + 7) / 8) * (size_t)rows * 16;
}

rq_status rq_pack_codes(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst, hipStream_t stream) {
  CallRange range(__func__);
  if (rows < 0 || rows >= ((int64_t)1 << 29) || L < 1 || L > RQ_MAX_L || M < 1 || (int64_t)L * M > (1 << 24))
    return fail(RQ_ERR_SHAPE, "bad pack shape rows=%lld L=%d M=%d", (long long)rows, L, M);
  if (rows == 0) return RQ_OK;
  if (!src || !dst) return fail(RQ_ERR_NULL, "pack: NULL buffer");
  if (!aligned(src, 2) || !aligned(dst, 16)) return fail(RQ_ERR_ALIGN, "pack: misaligned buffer");
  return launched(rq::launch_pack_codes(src, rows, L * M, dst, stream), "rq_pack_codes");
}

size_t rq_packed10_codes_bytes(int64_t rows, int32_t L, int32_t M) {
  if (rows < 0 || L < 1 || M < 1) return 0;
  return (size_t)(((int64_t)L * M + 11) / 12) * (size_t)rows * 16;
}

rq_status rq_pack_codes10(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst,
                          hipStream_t stream) {
  CallRange range(__func__);
  if (rows < 0 || rows >= ((int64_t)1 << 29) || L < 1 || L > RQ_MAX_L || M < 1 || (int64_t)L * M > (1 << 24))
    return fail(RQ_ERR_SHAPE, "bad pack shape rows=%lld L=%d M=%d", (long long)rows, L, M);
  if (rows == 0) return RQ_OK;
  if (!src || !dst) return fail(RQ_ERR_NULL, "pack10: NULL buffer");
  if (!aligned(src, 2) || !aligned(dst, 16)) return fail(RQ_ERR_ALIGN, "pack10: misaligned buffer");
  return launched(rq::launch_pack_codes10(src, rows, L * M, dst, stream), "rq_pack_codes10");
}

size_t rq_packed8_codes_bytes(int64_t rows, int32_t L, int32_t M) {
  if (rows < 0 || L < 1 || M < 1) return 0;
  return (size_t)(((int64_t)L * M + 15) / 16) * (size_t)rows * 16;
}

rq_status rq_pack_codes8(const uint16_t* src, int64_t rows, int32_t L, int32_t M, uint16_t* dst,
                         hipStream_t stream) {
  CallRange range(__func__);
  if (rows < 0 || rows >= ((int64_t)1 << 29) || L < 1 || L > RQ_MAX_L || M < 1 || (int64_t)L * M > (1 << 24))
    return fail(RQ_ERR_SHAPE, "bad pack shape rows=%lld L=%d M=%d", (long long)rows, L, M);
  if (rows == 0) return RQ_OK;
  if (!src || !dst) return fail(RQ_ERR_NULL, "pack8: NULL buffer");
  if (!aligned(src, 2) || !aligned(dst, 16)) return fail(RQ_ERR_ALIGN, "pack8: misaligned buffer");
  return launched(rq::launch_pack_codes8(src, rows, L * M, dst, stream), "rq_pack_codes8");
}

size_t rq_lut_bytes(const rq_matrix* W, int32_t B, int32_t lut_dtype) {
  if (!W || B < 0 || !valid_dtype(lut_dtype) || W->L < 1 || W->M < 1 || W->K < 1) return 0;
  return lut_elems(W, B) * (lut_dtype == RQ_BF16 ? 2 : 4);
}

rq_status rq_build_lut(const rq_matrix* W, const float* x, const float* x2, int32_t prologue, int32_t B,
                       int32_t lut_dtype, void* lut, hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_matrix(W, false);
  if (s != RQ_OK) return s;
  if (B < 0 || B > 65535) return fail(RQ_ERR_SHAPE, "B=%d outside [0, 65535]", B);
  if (!valid_dtype(lut_dtype)) return fail(RQ_ERR_DTYPE, "unknown table dtype %d", lut_dtype);
  if (prologue != RQ_PRO_NONE && prologue != RQ_PRO_GELU_TANH_MUL) return fail(RQ_ERR_DTYPE, "unknown prologue %d", prologue);
  if (B == 0) return RQ_OK;
  if (!x || !lut || (prologue == RQ_PRO_GELU_TANH_MUL && !x2)) return fail(RQ_ERR_NULL, "build_lut: NULL buffer");
  if (!aligned(x, 4) || (x2 && !aligned(x2, 4)) || !aligned(lut, 16)) return fail(RQ_ERR_ALIGN, "build_lut: misaligned buffer");
  return launched(rq::launch_build_lut(W, x, x2, prologue, B, lut_dtype == RQ_BF16, lut, stream), "rq_build_lut");
}

size_t rq_lut_logits_workspace(const rq_matrix* W, int32_t B, int32_t topk, int32_t lut_dtype) {
  if (check_lut_call(W, B, lut_dtype) != RQ_OK || topk < 0) return 0;
  if (B == 0 || W->rows == 0) return 0;
  const rq::GatherPlan plan = rq::plan_gather(W, B, lut_dtype == RQ_BF16);
  if (plan.BT == 0) return 0;
  return logits_ws(W, plan, B, topk, false, lut_dtype == RQ_BF16).total;   // enough with or without a logits output
}

rq_status rq_lut_logits(const rq_matrix* W, const void* lut, int32_t lut_dtype, int32_t B, float softcap,
                        float* logits, int32_t* argmax, int32_t topk, int32_t* topk_ids, float* topk_vals, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_lut_call(W, B, lut_dtype);
  if (s != RQ_OK) return s;
  if (topk < 0 || topk > 1024 || (W->rows > 0 && topk > W->rows))
    return fail(RQ_ERR_SHAPE, "topk=%d outside [0, min(rows, 1024)]", topk);
  if (B == 0 || W->rows == 0) return RQ_OK;
  if (!lut) return fail(RQ_ERR_NULL, "lut is NULL");
  if (topk > 0 && !topk_ids) return fail(RQ_ERR_NULL, "topk_ids is NULL");
  if (!aligned(lut, 16)) return fail(RQ_ERR_ALIGN, "lut must be 16-byte aligned");
  if ((logits && !aligned(logits, 4)) || (argmax && !aligned(argmax, 4)) || (topk_ids && !aligned(topk_ids, 4)) ||
      (topk_vals && !aligned(topk_vals, 4)))
    return fail(RQ_ERR_ALIGN, "output misaligned");
  const rq::GatherPlan plan = rq::plan_gather(W, B, lut_dtype == RQ_BF16);
  if (plan.BT == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", W->K);
  const LogitsWs w = logits_ws(W, plan, B, topk, logits != nullptr, lut_dtype == RQ_BF16);
  if (ws_bytes < w.total || (!ws && w.total > 0)) return fail(RQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  if (!aligned(ws, 256)) return fail(RQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  const bool select = argmax || topk > 0;
  rq::GatherOut o;
  o.partial = reinterpret_cast<float*>(base + w.partial);
  o.out = logits ? logits : (topk > 0 ? reinterpret_cast<float*>(base + w.scratch) : nullptr);
  o.softcap = softcap;
  o.block_keys = select ? reinterpret_cast<uint64_t*>(base + w.keys) : nullptr;
  o.lut_tiled = 0;
  if (plan.NBT > 1) {   // several batch tiles: stage from a batch-tiled copy with 16-byte copies
    hipError_t et = rq::launch_tile_lut(lut, lut_dtype == RQ_BF16, W->L * W->M, W->K, B, plan.BT, base + w.tiled, stream);
    if (et != hipSuccess) return launched(et, "rq_lut_logits: table tiling");
    lut = base + w.tiled;
    o.lut_tiled = 1;
  }
  hipError_t e = rq::launch_gather(W, plan, lut, lut_dtype == RQ_BF16, B, o, stream);
  if (e != hipSuccess) return launched(e, "rq_lut_logits: lookup+sum");
  if (!select) return RQ_OK;
  e = rq::launch_select(o.block_keys, rq::key_blocks(plan, W->rows), B, argmax, o.out, W->rows, topk,
                        reinterpret_cast<uint64_t*>(base + w.cand), topk_ids, topk_vals, stream);
  return launched(e, "rq_lut_logits: selection");
}

// Workspace of rq_logits. Matrix-core method: the split hidden vectors, then
// the partial sums [G][B][rows]; table method: the fp32 table [L][M][K][B], then
// the partial sums of the lookup+sum. Both continue with the logits scratch
// (top-k without a logits output), the selection keys and the top-k
// candidates; the table method with several batch tiles ends with the
// batch-tiled copy of the table.
struct HeadWs {
  bool mm;
  rq::MmPlan mp;
  rq::GatherPlan gp;
  size_t front, partial, scratch, keys, cand, tiled, total;
  int nkb;
};

static HeadWs head_ws(const rq_matrix* W, int32_t B, int32_t topk, bool logits_out) {
  HeadWs w{};
  w.mm = rq::mm_usable(W, B);
  size_t partial_bytes;
  w.front = 0;
  if (w.mm) {
    w.mp = rq::plan_mm(W, B);
    w.partial = round_up(rq::mm_hp_bytes(W, w.mp), 256);
    partial_bytes = w.mp.G > 1 ? (size_t)w.mp.G * B * W->rows * sizeof(float) : 0;
    w.nkb = w.mp.G > 1 ? rq::finish_key_blocks(w.mp.G, W->rows) : w.mp.S;
  } else {
    w.gp = rq::plan_gather(W, B, 0);
    w.partial = round_up(lut_elems(W, B) * sizeof(float), 256);
    partial_bytes = w.gp.G > 1 ? (size_t)w.gp.G * B * W->rows * sizeof(float) : 0;
    w.nkb = rq::key_blocks(w.gp, W->rows);
  }
  w.scratch = w.partial + round_up(partial_bytes, 256);
  w.keys = w.scratch + (topk > 0 && !logits_out ? round_up((size_t)B * W->rows * sizeof(float), 256) : 0);
  w.cand = w.keys + round_up((size_t)B * w.nkb * sizeof(uint64_t), 256);
  w.tiled = w.cand + (topk > 0 ? round_up((size_t)B * rq::epi_blocks(W->rows) * topk * sizeof(uint64_t), 256) : 0);
  w.total = w.tiled + (w.mm ? 0 : tiled_bytes(W, w.gp, false));
  return w;
}

int32_t rq_logits_method(const rq_matrix* W, int32_t B) {
  const rq_status s = check_lut_call(W, B, RQ_F32);
  if (s != RQ_OK) return s;
  return rq::mm_usable(W, B) ? RQ_METHOD_MATRIX_CORES : RQ_METHOD_TABLE;
}

size_t rq_logits_workspace(const rq_matrix* W, int32_t B, int32_t topk) {
  if (check_lut_call(W, B, RQ_F32) != RQ_OK || topk < 0) return 0;
  if (B == 0 || W->rows == 0) return 0;
  const HeadWs w = head_ws(W, B, topk, false);
  if (!w.mm && w.gp.BT == 0) return 0;
  return w.total;
}

rq_status rq_logits(const rq_matrix* W, const float* h, int32_t B, float softcap, float* logits, int32_t* argmax,
                    int32_t topk, int32_t* topk_ids, float* topk_vals, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_lut_call(W, B, RQ_F32);
  if (s != RQ_OK) return s;
  if (topk < 0 || topk > 1024 || (W->rows > 0 && topk > W->rows))
    return fail(RQ_ERR_SHAPE, "topk=%d outside [0, min(rows, 1024)]", topk);
  if (B == 0 || W->rows == 0) return RQ_OK;
  if (!h) return fail(RQ_ERR_NULL, "h is NULL");
  if (topk > 0 && !topk_ids) return fail(RQ_ERR_NULL, "topk_ids is NULL");
  if (!aligned(h, 4) || (logits && !aligned(logits, 4)) || (argmax && !aligned(argmax, 4)) ||
      (topk_ids && !aligned(topk_ids, 4)) || (topk_vals && !aligned(topk_vals, 4)))
    return fail(RQ_ERR_ALIGN, "argument misaligned");
  const HeadWs w = head_ws(W, B, topk, logits != nullptr);
  if (!w.mm && w.gp.BT == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", W->K);
  if (ws_bytes < w.total || (!ws && w.total > 0)) return fail(RQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  if (!aligned(ws, 256)) return fail(RQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  const bool select = argmax || topk > 0;
  float* partial = reinterpret_cast<float*>(base + w.partial);
  float* out = logits ? logits : (topk > 0 ? reinterpret_cast<float*>(base + w.scratch) : nullptr);
  uint64_t* keys = select ? reinterpret_cast<uint64_t*>(base + w.keys) : nullptr;
  hipError_t e;
  if (w.mm) {
    e = rq::launch_mm_logits(W, w.mp, h, B, base + w.front, partial, out, softcap, keys, stream);
    if (e != hipSuccess) return launched(e, "rq_logits: matrix-core pass");
    if (w.mp.G > 1) {
      e = rq::launch_finish(partial, w.mp.G, B, W->rows, softcap, out, keys, stream);
      if (e != hipSuccess) return launched(e, "rq_logits: finish");
    }
  } else {
    void* lut = base + w.front;
    e = rq::launch_build_lut(W, h, nullptr, RQ_PRO_NONE, B, 0, lut, stream);
    if (e != hipSuccess) return launched(e, "rq_logits: table build");
    rq::GatherOut o;
    o.partial = partial;
    o.out = out;
    o.softcap = softcap;
    o.block_keys = keys;
    o.lut_tiled = 0;
    if (w.gp.NBT > 1) {
      e = rq::launch_tile_lut(lut, 0, W->L * W->M, W->K, B, w.gp.BT, base + w.tiled, stream);
      if (e != hipSuccess) return launched(e, "rq_logits: table tiling");
      lut = base + w.tiled;
      o.lut_tiled = 1;
    }
    e = rq::launch_gather(W, w.gp, lut, 0, B, o, stream);
    if (e != hipSuccess) return launched(e, "rq_logits: lookup+sum");
  }
  if (!select) return RQ_OK;
  e = rq::launch_select(keys, w.nkb, B, argmax, out, W->rows, topk, reinterpret_cast<uint64_t*>(base + w.cand),
                        topk_ids, topk_vals, stream);
  return launched(e, "rq_logits: selection");
}

rq_status rq_decode_rows(const rq_matrix* W, const int32_t* ids, int32_t n, int32_t out_dtype, void* out,
                         int32_t* bad_ids, hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_matrix(W, true);
  if (s != RQ_OK) return s;
  if (n < 0) return fail(RQ_ERR_SHAPE, "n=%d < 0", n);
  if (!valid_dtype(out_dtype)) return fail(RQ_ERR_DTYPE, "unknown output dtype %d", out_dtype);
  if (n == 0) return RQ_OK;
  if (!ids || !out) return fail(RQ_ERR_NULL, "decode_rows: NULL buffer");
  if (!aligned(ids, 4) || !aligned(out, 4) || (bad_ids && !aligned(bad_ids, 4)))
    return fail(RQ_ERR_ALIGN, "decode_rows: misaligned buffer");
  return launched(rq::launch_decode_rows(W, ids, n, out_dtype == RQ_BF16, out, bad_ids, stream), "rq_decode_rows");
}

// Workspace of rq_lut_matvec. Fused table build (one activation vector, fp32
// codebooks, d in {1, 2, 4, 8}): the partial sums [G][rows]. Otherwise: the fp32
// table [L][M][K][B], the partial sums [G][B][rows] (G > 1) and, with more
// than one batch tile, the batch-tiled copy of the table.
struct MatvecWs {
  bool fused;
  rq::GatherPlan plan;
  size_t front, partial, tiled, total;
};

static MatvecWs matvec_ws(const rq_matrix* W, int32_t B) {
  MatvecWs m{};
  m.fused = rq::fused_build_supported(W, B);
  if (m.fused) {
    m.plan = rq::plan_gather(W, B, 0, 1);
    if (m.plan.BT == 0 || !rq::plan_covers_blocks(W, m.plan)) m.fused = false;
  }
  if (!m.fused) m.plan = rq::plan_gather(W, B, 0);
  m.front = 0;
  m.partial = m.fused ? 0 : round_up(lut_elems(W, B) * sizeof(float), 256);
  m.tiled = m.partial + (m.plan.G > 1 ? round_up((size_t)m.plan.G * B * W->rows * sizeof(float), 256) : 0);
  m.total = m.tiled + (m.fused ? 0 : tiled_bytes(W, m.plan, false));
  return m;
}

size_t rq_lut_matvec_workspace(const rq_matrix* W, int32_t B) {
  if (check_lut_call(W, B, RQ_F32) != RQ_OK || B == 0 || W->rows == 0) return 0;
  const MatvecWs m = matvec_ws(W, B);
  if (m.plan.BT == 0) return 0;
  return m.total;
}

rq_status rq_lut_matvec(const rq_matrix* W, const float* x, const float* x2, int32_t prologue, int32_t B, float* y,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_lut_call(W, B, RQ_F32);
  if (s != RQ_OK) return s;
  if (prologue != RQ_PRO_NONE && prologue != RQ_PRO_GELU_TANH_MUL) return fail(RQ_ERR_DTYPE, "unknown prologue %d", prologue);
  if (B == 0 || W->rows == 0) return RQ_OK;
  if (!x || !y || (prologue == RQ_PRO_GELU_TANH_MUL && !x2)) return fail(RQ_ERR_NULL, "lut_matvec: NULL buffer");
  if (!aligned(x, 4) || (x2 && !aligned(x2, 4)) || !aligned(y, 4)) return fail(RQ_ERR_ALIGN, "lut_matvec: misaligned buffer");
  const MatvecWs m = matvec_ws(W, B);
  if (m.plan.BT == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", W->K);
  if (ws_bytes < m.total || (!ws && m.total > 0)) return fail(RQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, m.total);
  if (!aligned(ws, 256)) return fail(RQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  rq::GatherOut o;
  o.partial = reinterpret_cast<float*>(base + m.partial);
  o.out = y;
  o.softcap = 0.0f;
  o.block_keys = nullptr;
  o.lut_tiled = 0;
  hipError_t e;
  if (m.fused)
    return launched(rq::launch_gather(W, m.plan, nullptr, 0, B, o, stream, x,
                                      prologue == RQ_PRO_GELU_TANH_MUL ? x2 : nullptr),
                    "rq_lut_matvec: fused lookup+sum");
  float* lut = reinterpret_cast<float*>(base + m.front);
  e = rq::launch_build_lut(W, x, x2, prologue, B, 0, lut, stream);
  if (e != hipSuccess) return launched(e, "rq_lut_matvec: table build");
  if (m.plan.NBT > 1) {
    e = rq::launch_tile_lut(lut, 0, W->L * W->M, W->K, B, m.plan.BT, base + m.tiled, stream);
    if (e != hipSuccess) return launched(e, "rq_lut_matvec: table tiling");
    lut = reinterpret_cast<float*>(base + m.tiled);
    o.lut_tiled = 1;
  }
  return launched(rq::launch_gather(W, m.plan, lut, 0, B, o, stream), "rq_lut_matvec: lookup+sum");
}

// Workspace of rq_lut_mlp. Fused route: the partial sums of gate and up
// [2][Gg][rows] (their sums when Gg == 1), then down's partial sums
// [Gd][down rows] (Gd > 1), then -- when gate and up do not build their
// tables while staging (pair_tables) -- their two fp32 tables. Otherwise: g
// and u [2][B][rows], then one rq_lut_matvec workspace large enough for the
// three calls.
struct MlpWs {
  bool fused, pair_tables;
  rq::GatherPlan pgu, pd;
  size_t down_part, tables, mv, total;
};

static rq_status check_mlp(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, int32_t B) {
  rq_status s = check_lut_call(gate, B, RQ_F32);
  if (s == RQ_OK) s = check_lut_call(up, B, RQ_F32);
  if (s == RQ_OK) s = check_lut_call(down, B, RQ_F32);
  if (s != RQ_OK) return s;
  if (gate->rows != up->rows || gate->D != up->D || gate->M != up->M || gate->d != up->d || gate->K != up->K ||
      gate->L != up->L || gate->cb_dtype != up->cb_dtype || gate->codes_layout != up->codes_layout)
    return fail(RQ_ERR_SHAPE, "lut_mlp: gate and up differ in shape, codebook dtype or code layout");
  if ((int64_t)down->D != gate->rows)
    return fail(RQ_ERR_SHAPE, "lut_mlp: down->D=%d != gate->rows=%lld", down->D, (long long)gate->rows);
  return RQ_OK;
}

static MlpWs mlp_ws(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, int32_t B) {
  MlpWs w{};
  w.fused = rq::fused_build_supported(gate, B) && rq::fused_build_supported(up, B) &&
            rq::fused_build_supported(down, B);
  if (w.fused) {
    const int pair_mats = 2;
    w.pgu = rq::plan_gather(gate, B, 0, 1, pair_mats);
    if (w.pgu.BT != 0 && !rq::plan_covers_blocks(gate, w.pgu)) {   // gate and up from tables built first
      w.pair_tables = true;
      w.pgu = rq::plan_gather(gate, B, 0, 0, pair_mats);
    }
    w.pd = rq::plan_gather(down, B, 0, 1);
    w.fused = w.pgu.BT != 0 && w.pd.BT != 0 && rq::plan_covers_blocks(down, w.pd) &&
              rq::gather_pro_lds(down, w.pd, w.pgu.G) <= (size_t)rq::kLdsBudget;
  }
  if (w.fused) {
    w.down_part = round_up((size_t)2 * w.pgu.G * gate->rows * sizeof(float), 256);
    w.tables = w.down_part + (w.pd.G > 1 ? round_up((size_t)w.pd.G * down->rows * sizeof(float), 256) : 0);
    w.total = w.tables + (w.pair_tables ? 2 * round_up(lut_elems(gate, B) * sizeof(float), 256) : 0);
    return w;
  }
  w.mv = round_up((size_t)2 * B * gate->rows * sizeof(float), 256);
  const MatvecWs mg = matvec_ws(gate, B), mu = matvec_ws(up, B), md = matvec_ws(down, B);
  if (mg.plan.BT == 0 || mu.plan.BT == 0 || md.plan.BT == 0) return w;   // total 0: no tiling fits
  w.total = w.mv + std::max(mg.total, std::max(mu.total, md.total));
  return w;
}

size_t rq_lut_mlp_workspace(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, int32_t B) {
  if (check_mlp(gate, up, down, B) != RQ_OK || B == 0 || down->rows == 0) return 0;
  return mlp_ws(gate, up, down, B).total;
}

rq_status rq_lut_mlp(const rq_matrix* gate, const rq_matrix* up, const rq_matrix* down, const float* x, int32_t B,
                     float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_mlp(gate, up, down, B);
  if (s != RQ_OK) return s;
  if (B == 0 || down->rows == 0) return RQ_OK;
  if (!x || !y) return fail(RQ_ERR_NULL, "lut_mlp: NULL buffer");
  if (!aligned(x, 4) || !aligned(y, 4)) return fail(RQ_ERR_ALIGN, "lut_mlp: misaligned buffer");
  const MlpWs w = mlp_ws(gate, up, down, B);
  if (w.total == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", gate->K);
  if (ws_bytes < w.total || (!ws && w.total > 0)) return fail(RQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  if (!aligned(ws, 256)) return fail(RQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  if (w.fused) {
    float* pg = reinterpret_cast<float*>(base);
    float* pu = pg + (size_t)w.pgu.G * gate->rows;
    hipError_t e;
    if (w.pair_tables) {
      float* tg = reinterpret_cast<float*>(base + w.tables);
      float* tu = reinterpret_cast<float*>(base + w.tables + round_up(lut_elems(gate, B) * sizeof(float), 256));
      e = B == 1 ? rq::launch_build_lut_pair(gate, up, x, tg, tu, stream)
                 : rq::launch_build_lut(gate, x, nullptr, RQ_PRO_NONE, B, 0, tg, stream);
      if (e == hipSuccess && B != 1) e = rq::launch_build_lut(up, x, nullptr, RQ_PRO_NONE, B, 0, tu, stream);
      if (e != hipSuccess) return launched(e, "rq_lut_mlp: gate and up tables");
      e = rq::launch_gather_pair(gate, up, w.pgu, nullptr, tg, tu, pg, pu, stream);
    } else {
      e = rq::launch_gather_pair(gate, up, w.pgu, x, nullptr, nullptr, pg, pu, stream);
    }
    if (e != hipSuccess) return launched(e, "rq_lut_mlp: gate and up lookup+sum");
    rq::GatherOut o{};
    o.partial = reinterpret_cast<float*>(base + w.down_part);
    o.out = y;
    return launched(rq::launch_gather_pro(down, w.pd, pg, w.pgu.G, gate->rows, o, stream),
                    "rq_lut_mlp: down lookup+sum");
  }
  float* g = reinterpret_cast<float*>(base);
  float* u = g + (size_t)B * gate->rows;
  void* mws = base + w.mv;
  const size_t mbytes = ws_bytes - w.mv;
  s = rq_lut_matvec(gate, x, nullptr, RQ_PRO_NONE, B, g, mws, mbytes, stream);
  if (s == RQ_OK) s = rq_lut_matvec(up, x, nullptr, RQ_PRO_NONE, B, u, mws, mbytes, stream);
  if (s == RQ_OK) s = rq_lut_matvec(down, g, u, RQ_PRO_GELU_TANH_MUL, B, y, mws, mbytes, stream);
  return s;
}

// Workspace of rq_dense_logits: the bf16 copy of h (padded to 16-vector tiles),
// then the per-block selection keys [B][dense_blocks].
size_t rq_dense_logits_workspace(int64_t rows, int32_t B) {
  if (rows <= 0 || B < 1 || B > 128) return 0;
  return round_up(rq::dense_hb_bytes(4096, B), 256) + round_up((size_t)B * rq::dense_blocks(rows) * sizeof(uint64_t), 256);
}

rq_status rq_residual_norm(const float* y, float* h, float* x, int32_t D, float eps, hipStream_t stream) {
  CallRange range(__func__);
  if (D < 1 || D > (1 << 20) || !(eps > 0.0f)) return fail(RQ_ERR_SHAPE, "residual_norm needs 1 <= D <= 2^20 and eps > 0");
  if (!h || !x) return fail(RQ_ERR_NULL, "residual_norm: NULL buffer");
  if (!aligned(h, 4) || !aligned(x, 4) || (y && !aligned(y, 4))) return fail(RQ_ERR_ALIGN, "residual_norm: misaligned buffer");
  const uintptr_t xb = (uintptr_t)x, xe = xb + (size_t)D * 4;
  auto overlaps = [&](const void* p) { return p && (uintptr_t)p < xe && xb < (uintptr_t)p + (size_t)D * 4; };
  if (overlaps(h) || overlaps(y)) return fail(RQ_ERR_SHAPE, "residual_norm: x overlaps h or y");
  return launched(rq::launch_residual_norm(y, h, x, D, eps, stream), "rq_residual_norm");
}

size_t rq_dense_tiled_bytes(int64_t rows, int32_t D) {
  if (rows <= 0 || rows >= ((int64_t)1 << 31) || D < 8 || D % 8 != 0 || D > 4096) return 0;
  return rq::dense_tiled_bytes(rows, D);
}

rq_status rq_pack_dense(const uint16_t* E, int64_t rows, int32_t D, uint16_t* Et, hipStream_t stream) {
  CallRange range(__func__);
  if (rows < 0 || rows >= ((int64_t)1 << 31)) return fail(RQ_ERR_SHAPE, "rows out of range");
  if (D < 8 || D % 8 != 0 || D > 4096) return fail(RQ_ERR_SHAPE, "dense head needs D %% 8 == 0 and 8 <= D <= 4096");
  if (rows == 0) return RQ_OK;
  if (!E || !Et) return fail(RQ_ERR_NULL, "pack_dense: NULL buffer");
  if (!aligned(E, 16) || !aligned(Et, 16)) return fail(RQ_ERR_ALIGN, "pack_dense: buffers must be 16-byte aligned");
  return launched(rq::launch_pack_dense(E, rows, D, Et, stream), "rq_pack_dense");
}

rq_status rq_dense_logits(const uint16_t* E, int64_t rows, int32_t D, const float* h, int32_t B, float softcap,
                          float* logits, int32_t* argmax, void* ws, size_t ws_bytes, hipStream_t stream) {
  CallRange range(__func__);
  if (rows < 0 || rows >= ((int64_t)1 << 31)) return fail(RQ_ERR_SHAPE, "rows out of range");
  if (D < 8 || D % 8 != 0 || D > 4096) return fail(RQ_ERR_SHAPE, "dense head needs D %% 8 == 0 and 8 <= D <= 4096");
  if (B < 0 || B > 128) return fail(RQ_ERR_SHAPE, "dense head supports 0 <= B <= 128");
  if (rows == 0 || B == 0) return RQ_OK;
  if (!E || !h || !logits) return fail(RQ_ERR_NULL, "dense_logits: NULL buffer");
  if (!aligned(E, 16) || !aligned(h, 4) || !aligned(logits, 4) || (argmax && !aligned(argmax, 4)))
    return fail(RQ_ERR_ALIGN, "dense_logits: misaligned buffer");
  const size_t need = rq_dense_logits_workspace(rows, B);
  if (!ws || ws_bytes < need) return fail(RQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(RQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  uint16_t* hb = static_cast<uint16_t*>(ws);
  uint64_t* keys = argmax ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + round_up(rq::dense_hb_bytes(4096, B), 256))
                          : nullptr;
  hipError_t e = rq::launch_dense_logits(E, rows, D, h, B, softcap, logits, keys, hb, stream);
  if (e != hipSuccess || !argmax) return launched(e, "rq_dense_logits");
  return launched(rq::launch_select(keys, rq::dense_blocks(rows), B, argmax, logits, rows, 0, nullptr, nullptr,
                                    nullptr, stream),
                  "rq_dense_logits: argmax");
}

rq_status rq_lut_logits_plan(const rq_matrix* W, int32_t B, int32_t lut_dtype, int32_t plan[10]) {
  rq_status s = check_lut_call(W, B, lut_dtype);
  if (s != RQ_OK) return s;
  if (!plan) return fail(RQ_ERR_NULL, "plan is NULL");
  if (B < 1 || W->rows == 0) return fail(RQ_ERR_SHAPE, "a plan needs B >= 1 and rows >= 1");
  const rq::GatherPlan p = rq::plan_gather(W, B, lut_dtype == RQ_BF16);
  if (p.BT == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", W->K);
  const int32_t v[10] = {p.BT, p.P, p.chunks, p.cpg, p.G, p.steps, p.rps, p.S, p.rset, p.NBT};
  for (int i = 0; i < 10; ++i) plan[i] = v[i];
  return RQ_OK;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, resolved once per device
// with that device current (the calling thread's current device).
rq_status static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RQ_ERR_HIP, "rq_lut_logits_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RQ_ERR_HIP, "rq_lut_logits_static: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RQ_ERR_HIP, "rq_lut_logits_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return RQ_OK;
}

}  // namespace

extern "C" {

rq_status rq_lut_logits_static(const rq_matrix* W, const void* lut, int32_t lut_dtype, int32_t B, float softcap,
                               float* logits, int32_t* argmax, int32_t topk, int32_t* topk_ids, float* topk_vals,
                               hipStream_t stream) {
  CallRange range(__func__);
  rq_status s = check_lut_call(W, B, lut_dtype);
  if (s != RQ_OK) return s;
  if (topk < 0 || topk > 1024 || (W->rows > 0 && topk > W->rows))
    return fail(RQ_ERR_SHAPE, "topk=%d outside [0, min(rows, 1024)]", topk);
  if (B == 0 || W->rows == 0) return RQ_OK;
  const rq::GatherPlan plan = rq::plan_gather(W, B, lut_dtype == RQ_BF16);
  if (plan.BT == 0) return fail(RQ_ERR_SHAPE, "no table tiling fits on chip for K=%d", W->K);
  const size_t need = logits_ws(W, plan, B, topk, logits != nullptr, lut_dtype == RQ_BF16).total;
  if (need > (size_t)RQ_STATIC_SCRATCH_BYTES)
    return fail(RQ_ERR_WORKSPACE, "rq_lut_logits_static: this call needs %zu bytes of scratch, more than the %zu the "
                "library holds (use rq_lut_logits with a workspace)", need, (size_t)RQ_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = static_scratch(&ws);
  if (s != RQ_OK) return s;
  return rq_lut_logits(W, lut, lut_dtype, B, softcap, logits, argmax, topk, topk_ids, topk_vals, ws,
                       (size_t)RQ_STATIC_SCRATCH_BYTES, stream);
}

size_t rq_lds_gather_sink_words(void) { return rq::lds_gather_sink_words(); }

rq_status rq_lds_gather(int32_t width, int32_t reps, uint32_t* sink, hipStream_t stream) {
  CallRange range(__func__);
  if (width != 2 && width != 4 && width != 8 && width != 16) return fail(RQ_ERR_SHAPE, "lds_gather: width %d", width);
  if (reps < 0) return fail(RQ_ERR_SHAPE, "lds_gather: reps %d < 0", reps);
  if (!sink) return fail(RQ_ERR_NULL, "lds_gather: sink is NULL");
  if (!aligned(sink, 4)) return fail(RQ_ERR_ALIGN, "lds_gather: sink misaligned");
  return launched(rq::launch_lds_gather(width, reps, sink, stream), "rq_lds_gather");
}

int32_t rq_stream_read_configs(void) { return rq::stream_read_configs(); }

size_t rq_stream_read_sink_words(int32_t config) {
  if (config < 0 || config >= rq::stream_read_configs()) return 0;
  return rq::stream_read_sink_words(config);
}

rq_status rq_stream_read(const void* src, size_t bytes, int32_t config, uint32_t* sink, hipStream_t stream) {
  CallRange range(__func__);
  if (config < 0 || config >= rq::stream_read_configs())
    return fail(RQ_ERR_SHAPE, "stream_read: config %d outside [0, %d)", config, rq::stream_read_configs());
  if (bytes == 0) return RQ_OK;
  if (!src || !sink) return fail(RQ_ERR_NULL, "stream_read: NULL buffer");
  if (!aligned(src, 16) || bytes % 16 != 0 || !aligned(sink, 4))
    return fail(RQ_ERR_ALIGN, "stream_read: src must be 16-byte aligned and bytes a multiple of 16");
  return launched(rq::launch_stream_read(src, bytes, config, sink, stream), "rq_stream_read");
}

}  // extern "C"
