"""The C-ABI library on the host: it loads, exports every declared symbol, and rejects bad
arguments before launching anything (no GPU needed: every call here fails its host checks)."""
import ctypes
import os
import re

import pytest

from lut_logits_amd import binding as B

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 14
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_version_and_status_strings():
    lib = B.lib()
    assert lib.rq_version().decode().count(".") == 2
    for s in range(-6, 1):
        assert lib.rq_status_string(s)
    assert lib.rq_status_string(-99) == b"unknown status"


def gemma_desc(**kw):
    f = dict(rows=256000, D=2304, M=384, d=6, K=1024, L=2, cb_dtype=B.RQ_BF16, codes_layout=B.RQ_CODES_BLOCKED,
             codebooks=0x10000, codes=0x20000)
    f.update(kw)
    return B.rq_matrix(**f)


def call_logits(W, Bn=1, topk=0, lut=0x30000, ws=0x40000, ws_bytes=1 << 40, lut_dtype=B.RQ_F32, topk_ids=0x50000):
    lib = B.lib()
    return lib.rq_lut_logits(ctypes.byref(W) if W is not None else None, lut, lut_dtype, Bn, 30.0, 0x60000, 0x70000,
                             topk, topk_ids, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=2305), B.RQ_ERR_SHAPE),
    (dict(K=0), B.RQ_ERR_SHAPE),
    (dict(K=65537), B.RQ_ERR_SHAPE),
    (dict(K=40000), B.RQ_ERR_SHAPE),          # fp32 table of one pair does not fit on chip
    (dict(L=0), B.RQ_ERR_SHAPE),
    (dict(L=17), B.RQ_ERR_SHAPE),
    (dict(rows=-1), B.RQ_ERR_SHAPE),
    (dict(rows=1 << 29), B.RQ_ERR_SHAPE),
    (dict(cb_dtype=7), B.RQ_ERR_DTYPE),
    (dict(codes_layout=5), B.RQ_ERR_DTYPE),
    (dict(codes_layout=B.RQ_CODES_PACKED10, K=1025), B.RQ_ERR_SHAPE),   # 10-bit codes need K <= 1024
    (dict(codebooks=0), B.RQ_ERR_NULL),
    (dict(codes=0), B.RQ_ERR_NULL),
    (dict(codes=0x20002), B.RQ_ERR_ALIGN),
    (dict(codes_layout=B.RQ_CODES_ROWS, L=1, M=383, D=2298), B.RQ_ERR_ALIGN),   # L*M % 8 != 0 needs the blocked layout
])
def test_lut_logits_rejects(kw, status):
    assert call_logits(gemma_desc(**kw)) == status
    assert B.lib().rq_last_error()


def test_lut_logits_argument_checks():
    W = gemma_desc()
    assert call_logits(None) == B.RQ_ERR_NULL
    assert call_logits(W, Bn=-1) == B.RQ_ERR_SHAPE
    assert call_logits(W, topk=1025) == B.RQ_ERR_SHAPE
    assert call_logits(W, topk=5, topk_ids=0) == B.RQ_ERR_NULL
    assert call_logits(W, lut=0) == B.RQ_ERR_NULL
    assert call_logits(W, lut=0x30004) == B.RQ_ERR_ALIGN
    assert call_logits(W, ws=0) == B.RQ_ERR_WORKSPACE
    assert call_logits(W, ws_bytes=100) == B.RQ_ERR_WORKSPACE
    assert call_logits(W, ws=0x40010) == B.RQ_ERR_ALIGN
    assert call_logits(W, lut_dtype=9) == B.RQ_ERR_DTYPE
    # empty work is a no-op even with no buffers
    assert call_logits(W, Bn=0, lut=0, ws=0, ws_bytes=0) == B.RQ_OK
    assert call_logits(gemma_desc(rows=0), lut=0, ws=0, ws_bytes=0) == B.RQ_OK


def test_workspace_queries():
    lib = B.lib()
    W = gemma_desc()
    ws1 = lib.rq_lut_logits_workspace(ctypes.byref(W), 1, 0, B.RQ_F32)
    assert ws1 > 0 and ws1 % 256 == 0
    assert lib.rq_lut_logits_workspace(ctypes.byref(W), 16, 50, B.RQ_F32) > ws1
    assert lib.rq_lut_logits_workspace(ctypes.byref(gemma_desc(D=1)), 1, 0, B.RQ_F32) == 0
    assert lib.rq_lut_bytes(ctypes.byref(W), 1, B.RQ_F32) == 2 * 384 * 1024 * 4
    assert lib.rq_lut_bytes(ctypes.byref(W), 3, B.RQ_BF16) == 2 * 384 * 1024 * 3 * 2
    assert lib.rq_blocked_codes_bytes(256000, 2, 384) == 393_216_000
    assert lib.rq_blocked_codes_bytes(10, 1, 5) == 1 * 10 * 16
    assert lib.rq_blocked_codes_bytes(10, 3, 3) == 2 * 10 * 16
    assert lib.rq_packed10_codes_bytes(256000, 2, 384) == 64 * 256000 * 16   # 1024 bytes per Gemma-head row
    assert lib.rq_packed10_codes_bytes(10, 1, 13) == 2 * 10 * 16
    Wm = gemma_desc(rows=9216, D=2304, M=1152, d=2, cb_dtype=B.RQ_F32)
    # one vector with fp32 codebooks builds its table while staging: no table in the workspace
    assert 0 < lib.rq_lut_matvec_workspace(ctypes.byref(Wm), 1) < 2 * 1152 * 1024 * 4
    assert lib.rq_lut_matvec_workspace(ctypes.byref(Wm), 2) >= 2 * 1152 * 1024 * 4 * 2
    assert lib.rq_dense_logits_workspace(256000, 1) > 0
    assert lib.rq_dense_logits_workspace(256000, 129) == 0
    # tiled dense matrix: 16-row x 32-column tiles of 1 KB, rows and D padded up
    assert lib.rq_dense_tiled_bytes(256000, 2304) == 256000 * 2304 * 2
    assert lib.rq_dense_tiled_bytes(17, 40) == 2 * 2 * 1024
    assert lib.rq_dense_tiled_bytes(0, 2304) == 0
    assert lib.rq_dense_tiled_bytes(16, 2300) == 0
    assert lib.rq_dense_tiled_bytes(16, 4104) == 0


def test_other_entry_points_reject():
    lib = B.lib()
    W = gemma_desc()
    assert lib.rq_build_lut(ctypes.byref(W), None, None, 0, 1, 0, 0x30000, None) == B.RQ_ERR_NULL
    assert lib.rq_build_lut(ctypes.byref(W), 0x1000, None, 1, 1, 0, 0x30000, None) == B.RQ_ERR_NULL   # GELU needs x2
    assert lib.rq_build_lut(ctypes.byref(W), 0x1000, None, 3, 1, 0, 0x30000, None) == B.RQ_ERR_DTYPE
    assert lib.rq_build_lut(ctypes.byref(W), 0x1000, None, 0, 1, 0, 0x30008, None) == B.RQ_ERR_ALIGN
    assert lib.rq_build_lut(ctypes.byref(W), None, None, 0, 0, 0, None, None) == B.RQ_OK
    assert lib.rq_decode_rows(ctypes.byref(W), None, 4, 0, 0x1000, None, None) == B.RQ_ERR_NULL
    assert lib.rq_decode_rows(ctypes.byref(W), 0x1000, -1, 0, 0x1000, None, None) == B.RQ_ERR_SHAPE
    assert lib.rq_decode_rows(ctypes.byref(W), 0x1000, 4, 2, 0x1000, None, None) == B.RQ_ERR_DTYPE
    assert lib.rq_decode_rows(ctypes.byref(W), None, 0, 0, None, None, None) == B.RQ_OK
    assert lib.rq_lut_matvec(ctypes.byref(W), 0x1000, None, 0, 1, 0x2000, None, 0, None) == B.RQ_ERR_WORKSPACE
    assert lib.rq_lut_matvec(ctypes.byref(W), 0x1000, None, 1, 1, 0x2000, None, 0, None) == B.RQ_ERR_NULL
    # a matrix whose workspace query returns 0 takes a NULL workspace: the checks pass (without a GPU the
    # launch itself then fails)
    Ws = gemma_desc(rows=160, D=8, M=4, d=2, K=64, cb_dtype=B.RQ_F32)   # 8 pairs: one chunk, one group
    assert lib.rq_lut_matvec_workspace(ctypes.byref(Ws), 1) == 0
    assert lib.rq_lut_matvec(ctypes.byref(Ws), 0x1000, None, 0, 1, 0x2000, None, 0, None) not in (
        B.RQ_OK, B.RQ_ERR_WORKSPACE, B.RQ_ERR_NULL, B.RQ_ERR_ALIGN)
    assert lib.rq_pack_codes(None, 10, 2, 3, 0x1000, None) == B.RQ_ERR_NULL
    assert lib.rq_pack_codes(0x1000, 10, 0, 3, 0x1000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_pack_codes(0x1000, 10, 2, 3, 0x1008, None) == B.RQ_ERR_ALIGN
    assert lib.rq_pack_codes10(None, 10, 2, 3, 0x1000, None) == B.RQ_ERR_NULL
    assert lib.rq_pack_codes10(0x1000, 10, 0, 3, 0x1000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_pack_codes10(0x1000, 10, 2, 3, 0x1008, None) == B.RQ_ERR_ALIGN
    assert lib.rq_pack_codes10(None, 0, 2, 3, None, None) == B.RQ_OK
    assert lib.rq_residual_norm(None, None, 0x2000, 16, 1e-6, None) == B.RQ_ERR_NULL
    assert lib.rq_residual_norm(None, 0x1000, None, 16, 1e-6, None) == B.RQ_ERR_NULL
    assert lib.rq_residual_norm(None, 0x1000, 0x2000, 0, 1e-6, None) == B.RQ_ERR_SHAPE
    assert lib.rq_residual_norm(None, 0x1000, 0x2000, (1 << 20) + 1, 1e-6, None) == B.RQ_ERR_SHAPE
    assert lib.rq_residual_norm(None, 0x1000, 0x2000, 16, 0.0, None) == B.RQ_ERR_SHAPE
    assert lib.rq_residual_norm(None, 0x1002, 0x2000, 16, 1e-6, None) == B.RQ_ERR_ALIGN
    assert lib.rq_residual_norm(0x3001, 0x1000, 0x2000, 16, 1e-6, None) == B.RQ_ERR_ALIGN
    assert lib.rq_residual_norm(None, 0x1000, 0x1020, 16, 1e-6, None) == B.RQ_ERR_SHAPE   # x overlaps h
    assert lib.rq_residual_norm(0x2030, 0x1000, 0x2000, 16, 1e-6, None) == B.RQ_ERR_SHAPE   # x overlaps y
    assert lib.rq_pack_dense(None, 100, 2304, 0x1000, None) == B.RQ_ERR_NULL
    assert lib.rq_pack_dense(0x1000, 100, 2300, 0x2000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_pack_dense(0x1000, -1, 2304, 0x2000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_pack_dense(0x1008, 100, 2304, 0x2000, None) == B.RQ_ERR_ALIGN
    assert lib.rq_pack_dense(None, 0, 2304, None, None) == B.RQ_OK
    assert lib.rq_dense_logits(0x1000, 100, 2300, 0x2000, 1, 30.0, 0x3000, None, None, 0, None) == B.RQ_ERR_SHAPE
    assert lib.rq_dense_logits(0x1000, 100, 2304, 0x2000, 129, 30.0, 0x3000, None, None, 0, None) == B.RQ_ERR_SHAPE
    assert lib.rq_dense_logits(0x1000, 100, 2304, 0x2000, 1, 30.0, 0x3000, 0x4000, None, 0, None) == B.RQ_ERR_WORKSPACE


def test_logits_method_and_checks():
    """rq_logits routes B >= RQ_MM_MIN_B with bf16 codebooks and even d <= 8 to the matrix cores when the codes
    are blocked (K <= 4096; above 1024 one pair per staged slot) or 10-bit (K <= 1024), everything else to the
    table path; its host checks run before any launch."""
    lib = B.lib()
    W = gemma_desc()
    m = lambda w, b: lib.rq_logits_method(ctypes.byref(w), b)
    assert m(W, 1) == B.RQ_METHOD_TABLE
    assert m(W, 7) == B.RQ_METHOD_TABLE
    assert m(W, 8) == B.RQ_METHOD_MATRIX_CORES
    assert m(W, 128) == B.RQ_METHOD_MATRIX_CORES
    assert m(gemma_desc(cb_dtype=B.RQ_F32), 16) == B.RQ_METHOD_TABLE           # fp32 codebooks
    assert m(gemma_desc(K=4096, L=4), 64) == B.RQ_METHOD_MATRIX_CORES          # one pair per staged slot
    assert m(gemma_desc(K=4097, L=4), 64) == B.RQ_METHOD_TABLE                 # K above the staged maximum
    assert m(gemma_desc(K=2048, codes_layout=B.RQ_CODES_ROWS), 64) == B.RQ_METHOD_TABLE
    assert m(gemma_desc(K=1025), 64) == B.RQ_METHOD_TABLE                      # a pair's codewords not whole 16 B
    assert m(gemma_desc(codes_layout=B.RQ_CODES_ROWS), 16) == B.RQ_METHOD_TABLE
    assert m(gemma_desc(M=256, d=9), 16) == B.RQ_METHOD_TABLE                  # d > 8
    assert m(gemma_desc(M=768, d=3), 16) == B.RQ_METHOD_TABLE                  # odd d
    assert m(gemma_desc(M=1152, d=2), 16) == B.RQ_METHOD_MATRIX_CORES
    assert m(gemma_desc(codes_layout=B.RQ_CODES_PACKED10), 16) == B.RQ_METHOD_MATRIX_CORES
    assert m(gemma_desc(D=2305), 16) == B.RQ_ERR_SHAPE
    ws16 = lib.rq_logits_workspace(ctypes.byref(W), 16, 0)
    assert ws16 > 0 and ws16 % 256 == 0
    assert lib.rq_logits_workspace(ctypes.byref(W), 16, 50) > ws16
    assert lib.rq_logits_workspace(ctypes.byref(W), 1, 0) >= 2 * 384 * 1024 * 4   # holds the fp32 table
    call = lambda **kw: lib.rq_logits(ctypes.byref(kw.pop("W", W)), kw.pop("h", 0x1000), kw.pop("Bn", 16), 30.0,
                                      0x60000, 0x70000, kw.pop("topk", 0), kw.pop("ids", 0x50000), None,
                                      kw.pop("ws", 0x40000), kw.pop("ws_bytes", 1 << 40), None)
    assert call(h=0) == B.RQ_ERR_NULL
    assert call(h=0x1002) == B.RQ_ERR_ALIGN
    assert call(ws=0) == B.RQ_ERR_WORKSPACE
    assert call(ws_bytes=ws16 - 1) == B.RQ_ERR_WORKSPACE
    assert call(ws=0x40040) == B.RQ_ERR_ALIGN
    assert call(topk=3, ids=0) == B.RQ_ERR_NULL
    assert call(Bn=-2) == B.RQ_ERR_SHAPE
    assert call(Bn=0, h=0, ws=0, ws_bytes=0) == B.RQ_OK


def test_mlp_workspace_and_rejects():
    """rq_lut_mlp: the fused route's workspace holds partial sums only (no tables); mismatched shapes and
    missing buffers are rejected on the host before any launch."""
    lib = B.lib()
    gate = gemma_desc(rows=9216, D=2304, M=1152, d=2, cb_dtype=B.RQ_F32)
    up = gemma_desc(rows=9216, D=2304, M=1152, d=2, cb_dtype=B.RQ_F32, codebooks=0x30000, codes=0x40000)
    down = gemma_desc(rows=2304, D=9216, M=4608, d=2, cb_dtype=B.RQ_F32, codebooks=0x50000, codes=0x60000)
    g, u, d = (ctypes.byref(m) for m in (gate, up, down))
    ws1 = lib.rq_lut_mlp_workspace(g, u, d, 1)
    assert 0 < ws1 < 2 * 1152 * 1024 * 4 and ws1 % 256 == 0          # no table in the fused route
    assert lib.rq_lut_mlp_workspace(g, u, d, 2) >= 2 * 2 * 9216 * 4      # g and u, then matvec workspaces
    assert lib.rq_lut_mlp_workspace(g, u, d, 0) == 0
    bad_up = gemma_desc(rows=9215, D=2304, M=1152, d=2, cb_dtype=B.RQ_F32)
    assert lib.rq_lut_mlp(g, ctypes.byref(bad_up), d, 0x1000, 1, 0x2000, 0x100000, 1 << 30, None) == B.RQ_ERR_SHAPE
    bad_down = gemma_desc(rows=2304, D=9214, M=4607, d=2, cb_dtype=B.RQ_F32)
    assert lib.rq_lut_mlp(g, u, ctypes.byref(bad_down), 0x1000, 1, 0x2000, 0x100000, 1 << 30, None) == B.RQ_ERR_SHAPE
    assert lib.rq_lut_mlp(g, u, d, None, 1, 0x2000, 0x100000, 1 << 30, None) == B.RQ_ERR_NULL
    assert lib.rq_lut_mlp(g, u, d, 0x1000, 1, 0x2000, 0x100000, 16, None) == B.RQ_ERR_WORKSPACE
    assert lib.rq_lut_mlp(g, u, d, 0x1000, 1, 0x2000, 0x100008, 1 << 30, None) == B.RQ_ERR_ALIGN
    assert lib.rq_lut_mlp(g, u, d, None, 0, None, None, 0, None) == B.RQ_OK


def test_packed8_layout_checks():
    """The 8-bit layout: byte counts, pack argument checks, and K <= 256 enforced on every entry point."""
    lib = B.lib()
    assert lib.rq_packed8_codes_bytes(256000, 2, 384) == 48 * 256000 * 16   # 768 bytes per Gemma-head row
    assert lib.rq_packed8_codes_bytes(10, 1, 17) == 2 * 10 * 16
    assert lib.rq_pack_codes8(None, 10, 2, 3, 0x1000, None) == B.RQ_ERR_NULL
    assert lib.rq_pack_codes8(0x1000, 10, 0, 3, 0x1000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_pack_codes8(0x1000, 10, 2, 3, 0x1008, None) == B.RQ_ERR_ALIGN
    assert lib.rq_pack_codes8(None, 0, 2, 3, None, None) == B.RQ_OK
    W = gemma_desc(codes_layout=B.RQ_CODES_PACKED8)                        # K = 1024: too large
    assert lib.rq_lut_logits_workspace(ctypes.byref(W), 1, 0, B.RQ_F32) == 0
    assert call_logits(W) == B.RQ_ERR_SHAPE
    W = gemma_desc(codes_layout=B.RQ_CODES_PACKED8, K=256)
    assert lib.rq_lut_logits_workspace(ctypes.byref(W), 1, 0, B.RQ_F32) > 0
    assert lib.rq_logits_method(ctypes.byref(W), 16) == B.RQ_METHOD_TABLE  # no matrix-core staging of 8-bit codes


def test_stream_read_checks():
    """The stream-read probe (a measurement aid): configurations, sink sizes and host-side rejections
    (no launch)."""
    lib = B.lib()
    n = lib.rq_stream_read_configs()
    assert n >= 1
    assert all(lib.rq_stream_read_sink_words(c) in (256, 512, 1024, 2048) for c in range(n))
    assert lib.rq_stream_read_sink_words(-1) == 0 and lib.rq_stream_read_sink_words(n) == 0
    assert lib.rq_stream_read(0x1000, 4096, n, 0x2000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_stream_read(0x1000, 4096, -1, 0x2000, None) == B.RQ_ERR_SHAPE
    assert lib.rq_stream_read(None, 4096, 0, 0x2000, None) == B.RQ_ERR_NULL
    assert lib.rq_stream_read(0x1000, 4096, 0, None, None) == B.RQ_ERR_NULL
    assert lib.rq_stream_read(0x1008, 4096, 0, 0x2000, None) == B.RQ_ERR_ALIGN
    assert lib.rq_stream_read(0x1000, 4100, 0, 0x2000, None) == B.RQ_ERR_ALIGN
    assert lib.rq_stream_read(None, 0, 0, None, None) == B.RQ_OK


def test_roctx_ranges_linked():
    """Each C-ABI call opens a roctx range (shown by rocprofv3 --marker-trace): the library imports the roctx
    push/pop pair and every compute entry point calls them."""
    import subprocess
    syms = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "roctxRangePushA" in syms and "roctxRangePop" in syms
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "lut_logits_amd", "csrc",
                            "api.hip")).read()
    for name in ("rq_build_lut", "rq_lut_logits", "rq_logits", "rq_decode_rows", "rq_lut_matvec", "rq_lut_mlp",
                 "rq_dense_logits", "rq_lut_logits_static", "rq_pack_codes"):
        head = src.split(f"\nrq_status {name}(", 1)[1].split("{", 1)[1]
        assert head.lstrip().startswith("CallRange range(__func__);"), name


def _plan(W, Bn=1, lut_dtype=B.RQ_F32):
    buf = (ctypes.c_int32 * 10)()
    assert B.lib().rq_lut_logits_plan(ctypes.byref(W), Bn, lut_dtype, buf) == B.RQ_OK
    return dict(zip(B.PLAN_FIELDS, list(buf)))


@pytest.mark.parametrize("layout", [B.RQ_CODES_BLOCKED, B.RQ_CODES_PACKED10])
def test_head_plan_fills_every_cu(layout):
    """The single-vector plan at the Gemma head (host-side planner, no GPU): 4 groups of pairs and slabs
    shorter than 4 x 1,024 rows, so that exactly one workgroup per CU (256) covers the 256,000 rows."""
    p = _plan(gemma_desc(codes_layout=layout))
    assert p["BT"] == 1 and p["G"] == 4 and p["steps"] == 4 and p["rps"] == 1024, p
    assert p["S"] == 64 and p["G"] * p["S"] == 256, p


def test_tall_matrix_plan_keeps_full_slabs():
    """A matrix tall enough that its slabs give a workgroup per CU or more keeps slabs of steps x rows per step."""
    p = _plan(gemma_desc(rows=2_000_000))
    assert p["S"] == -(-2_000_000 // (p["steps"] * p["rps"])), p
