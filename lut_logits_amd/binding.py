"""ctypes binding of librq_lut.so (include/rq_lut.h), one Python function per C entry point.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's
kernels. The library is loaded on first use and a missing build raises.
"""
import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librq_lut.so")

RQ_OK, RQ_ERR_NULL, RQ_ERR_SHAPE, RQ_ERR_DTYPE, RQ_ERR_ALIGN, RQ_ERR_WORKSPACE, RQ_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
RQ_F32, RQ_BF16 = 0, 1
RQ_PRO_NONE, RQ_PRO_GELU_TANH_MUL = 0, 1
RQ_CODES_ROWS, RQ_CODES_BLOCKED, RQ_CODES_PACKED10, RQ_CODES_PACKED8 = 0, 1, 2, 3
_LAYOUTS = {"rows": RQ_CODES_ROWS, "blocked": RQ_CODES_BLOCKED, "packed10": RQ_CODES_PACKED10,
            "packed8": RQ_CODES_PACKED8}
RQ_METHOD_TABLE, RQ_METHOD_MATRIX_CORES = 0, 1

# Every symbol include/rq_lut.h declares.
EXPORTS = ("rq_blocked_codes_bytes", "rq_pack_codes", "rq_packed10_codes_bytes", "rq_pack_codes10",
           "rq_packed8_codes_bytes", "rq_pack_codes8", "rq_lut_bytes", "rq_build_lut", "rq_lut_logits_workspace",
           "rq_lut_logits", "rq_logits_method", "rq_logits_workspace", "rq_logits", "rq_decode_rows", "rq_lut_matvec_workspace", "rq_lut_matvec",
           "rq_lut_mlp_workspace", "rq_lut_mlp", "rq_dense_logits_workspace", "rq_dense_logits", "rq_stream_read_configs",
           "rq_stream_read_sink_words", "rq_stream_read", "rq_set_stage_events", "rq_status_string", "rq_last_error", "rq_version")


class RQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"rq status {status}: {msg}")
        self.status = status


class rq_matrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("D", ctypes.c_int32), ("M", ctypes.c_int32), ("d", ctypes.c_int32),
                ("K", ctypes.c_int32), ("L", ctypes.c_int32), ("cb_dtype", ctypes.c_int32),
                ("codes_layout", ctypes.c_int32), ("codebooks", ctypes.c_void_p), ("codes", ctypes.c_void_p)]


_lib = None
_i32, _i64, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_MP = ctypes.POINTER(rq_matrix)


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "rq_blocked_codes_bytes": (_sz, [_i64, _i32, _i32]),
            "rq_pack_codes": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
            "rq_packed10_codes_bytes": (_sz, [_i64, _i32, _i32]),
            "rq_pack_codes10": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
            "rq_packed8_codes_bytes": (_sz, [_i64, _i32, _i32]),
            "rq_pack_codes8": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
            "rq_lut_bytes": (_sz, [_MP, _i32, _i32]),
            "rq_build_lut": (_i32, [_MP, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
            "rq_lut_logits_workspace": (_sz, [_MP, _i32, _i32, _i32]),
            "rq_lut_logits": (_i32, [_MP, _vp, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
            "rq_logits_method": (_i32, [_MP, _i32]),
            "rq_logits_workspace": (_sz, [_MP, _i32, _i32]),
            "rq_logits": (_i32, [_MP, _vp, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
            "rq_decode_rows": (_i32, [_MP, _vp, _i32, _i32, _vp, _vp, _vp]),
            "rq_lut_matvec_workspace": (_sz, [_MP, _i32]),
            "rq_lut_matvec": (_i32, [_MP, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
            "rq_lut_mlp_workspace": (_sz, [_MP, _MP, _MP, _i32]),
            "rq_lut_mlp": (_i32, [_MP, _MP, _MP, _vp, _i32, _vp, _vp, _sz, _vp]),
            "rq_dense_logits_workspace": (_sz, [_i64, _i32]),
            "rq_dense_logits": (_i32, [_vp, _i64, _i32, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
            "rq_stream_read_configs": (_i32, []),
            "rq_stream_read_sink_words": (_sz, [_i32]),
            "rq_stream_read": (_i32, [_vp, _sz, _i32, _vp, _vp]),
            "rq_set_stage_events": (_i32, [_vp, _vp]),
            "rq_status_string": (ctypes.c_char_p, [_i32]),
            "rq_last_error": (ctypes.c_char_p, []),
            "rq_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def check(status):
    if status != RQ_OK:
        raise RQError(status, lib().rq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(name):
    return {"f32": RQ_F32, "bf16": RQ_BF16}[name]


class DeviceMatrix:
    """An RQ-coded matrix resident on the GPU: codes (uint16, in rq layout) and codebooks.

    Holds the torch tensors that own the memory and the rq_matrix descriptor
    that points into them."""

    def __init__(self, rows, D, M, K, L, cb_dtype, codebooks, codes, layout):
        self.rows, self.D, self.M, self.d, self.K, self.L = rows, D, M, D // M, K, L
        self.cb_dtype, self.layout = cb_dtype, layout
        self.codebooks, self.codes = codebooks, codes
        self.desc = rq_matrix(rows, D, M, D // M, K, L, _dtype_code(cb_dtype),
                              _LAYOUTS[layout],
                              codebooks.data_ptr(), codes.data_ptr() if codes is not None else 0)

    @property
    def ref(self):
        return ctypes.byref(self.desc)

    def resident_bytes(self):
        return self.codebooks.numel() * self.codebooks.element_size() + self.codes.numel() * self.codes.element_size()


def to_device(mat, layout="blocked", device="cuda"):
    """Upload a host RQMatrix (lut_logits_amd.synth) and, for the paired layout, repack its codes on the GPU."""
    cb_np = mat.codebooks.view(np.int16) if mat.cb_is_bf16 else mat.codebooks
    cb = torch.from_numpy(np.ascontiguousarray(cb_np)).to(device)
    rows_codes = torch.from_numpy(np.ascontiguousarray(mat.codes).view(np.int16)).to(device)
    if layout == "rows":
        return DeviceMatrix(mat.rows, mat.D, mat.M, mat.K, mat.L, mat.cb_dtype, cb, rows_codes, "rows")
    packer = {"packed10": pack_codes10, "packed8": pack_codes8}.get(layout, pack_codes)
    packed = packer(rows_codes, mat.rows, mat.L, mat.M)
    del rows_codes
    return DeviceMatrix(mat.rows, mat.D, mat.M, mat.K, mat.L, mat.cb_dtype, cb, packed, layout)


def blocked_codes_bytes(rows, L, M):
    return lib().rq_blocked_codes_bytes(rows, L, M)


def pack_codes(rows_codes, rows, L, M):
    """rq_pack_codes: [rows][L*M] uint16 -> the paired layout (returned as an int16 tensor)."""
    nbytes = blocked_codes_bytes(rows, L, M)
    dst = torch.empty(nbytes // 2, dtype=torch.int16, device=rows_codes.device)
    check(lib().rq_pack_codes(_ptr(rows_codes), rows, L, M, _ptr(dst), _stream()))
    return dst


def packed8_codes_bytes(rows, L, M):
    return lib().rq_packed8_codes_bytes(rows, L, M)


def pack_codes8(rows_codes, rows, L, M):
    """rq_pack_codes8: [rows][L*M] uint16 (codes < 256) -> the 8-bit layout (an int16 tensor)."""
    dst = torch.empty(packed8_codes_bytes(rows, L, M) // 2, dtype=torch.int16, device=rows_codes.device)
    check(lib().rq_pack_codes8(_ptr(rows_codes), rows, L, M, _ptr(dst), _stream()))
    return dst


def packed10_codes_bytes(rows, L, M):
    return lib().rq_packed10_codes_bytes(rows, L, M)


def pack_codes10(rows_codes, rows, L, M):
    """rq_pack_codes10: [rows][L*M] uint16 (codes < 1024) -> the 10-bit layout (an int16 tensor)."""
    dst = torch.empty(packed10_codes_bytes(rows, L, M) // 2, dtype=torch.int16, device=rows_codes.device)
    check(lib().rq_pack_codes10(_ptr(rows_codes), rows, L, M, _ptr(dst), _stream()))
    return dst


def lut_bytes(W, B, lut_dtype="f32"):
    return lib().rq_lut_bytes(W.ref, B, _dtype_code(lut_dtype))


def build_lut(W, x, lut_dtype="f32", x2=None, prologue=RQ_PRO_NONE, out=None):
    """rq_build_lut: the [L][M][K][B] table of the rows of x (fp32 [B][D])."""
    B = x.shape[0]
    if out is None:
        n = lut_bytes(W, B, lut_dtype) // (2 if lut_dtype == "bf16" else 4)
        out = torch.empty(n, dtype=torch.int16 if lut_dtype == "bf16" else torch.float32, device=x.device)
    check(lib().rq_build_lut(W.ref, _ptr(x), _ptr(x2), prologue, B, _dtype_code(lut_dtype), _ptr(out), _stream()))
    return out


def lut_logits_workspace(W, B, topk=0, lut_dtype="f32"):
    return lib().rq_lut_logits_workspace(W.ref, B, topk, _dtype_code(lut_dtype))


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned device workspace (the library needs no particular initial contents)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def lut_logits(W, lut, B, softcap=30.0, lut_dtype="f32", logits=True, argmax=True, topk=0, ws=None, out=None,
               argmax_out=None):
    """rq_lut_logits: returns (logits [B][rows] | None, argmax [B] | None, topk_ids | None, topk_vals | None)."""
    dev = lut.device
    lg = (out if out is not None else torch.empty((B, W.rows), dtype=torch.float32, device=dev)) if logits else None
    am = (argmax_out if argmax_out is not None else torch.empty(B, dtype=torch.int32, device=dev)) if argmax else None
    ti = torch.empty((B, topk), dtype=torch.int32, device=dev) if topk else None
    tv = torch.empty((B, topk), dtype=torch.float32, device=dev) if topk else None
    if ws is None:
        ws = workspace(lut_logits_workspace(W, B, topk, lut_dtype), dev)
    check(lib().rq_lut_logits(W.ref, _ptr(lut), _dtype_code(lut_dtype), B, softcap, _ptr(lg), _ptr(am), topk,
                              _ptr(ti), _ptr(tv), _ptr(ws), ws.numel(), _stream()))
    return lg, am, ti, tv


def logits_method(W, B):
    """rq_logits_method: RQ_METHOD_TABLE or RQ_METHOD_MATRIX_CORES."""
    m = lib().rq_logits_method(W.ref, B)
    if m < 0:
        raise RQError(m, lib().rq_last_error().decode())
    return m


def logits_workspace(W, B, topk=0):
    return lib().rq_logits_workspace(W.ref, B, topk)


def logits(W, h, softcap=30.0, logits=True, argmax=True, topk=0, ws=None, out=None, argmax_out=None):
    """rq_logits (one call from the hidden vectors h [B][D] fp32): returns
    (logits [B][rows] | None, argmax [B] | None, topk_ids | None, topk_vals | None)."""
    B = h.shape[0]
    dev = h.device
    lg = (out if out is not None else torch.empty((B, W.rows), dtype=torch.float32, device=dev)) if logits else None
    am = (argmax_out if argmax_out is not None else torch.empty(B, dtype=torch.int32, device=dev)) if argmax else None
    ti = torch.empty((B, topk), dtype=torch.int32, device=dev) if topk else None
    tv = torch.empty((B, topk), dtype=torch.float32, device=dev) if topk else None
    if ws is None:
        ws = workspace(logits_workspace(W, B, topk), dev)
    check(lib().rq_logits(W.ref, _ptr(h), B, softcap, _ptr(lg), _ptr(am), topk, _ptr(ti), _ptr(tv), _ptr(ws),
                          ws.numel(), _stream()))
    return lg, am, ti, tv


def decode_rows(W, ids, out_dtype="f32", bad_ids=None, out=None):
    """rq_decode_rows: rows [n][D] (fp32, or bf16 bit patterns as int16)."""
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, W.D), dtype=torch.int16 if out_dtype == "bf16" else torch.float32, device=ids.device)
    check(lib().rq_decode_rows(W.ref, _ptr(ids), n, _dtype_code(out_dtype), _ptr(out), _ptr(bad_ids), _stream()))
    return out


def lut_matvec_workspace(W, B):
    return lib().rq_lut_matvec_workspace(W.ref, B)


def lut_matvec(W, x, x2=None, prologue=RQ_PRO_NONE, ws=None, out=None):
    """rq_lut_matvec: y [B][rows] = W a, a = x or gelu_tanh(x) * x2."""
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, W.rows), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(lut_matvec_workspace(W, B), x.device)
    check(lib().rq_lut_matvec(W.ref, _ptr(x), _ptr(x2), prologue, B, _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def lut_mlp_workspace(gate, up, down, B):
    return lib().rq_lut_mlp_workspace(gate.ref, up.ref, down.ref, B)


def lut_mlp(gate, up, down, x, ws=None, out=None):
    """rq_lut_mlp: y [B][down.rows] = down(gelu_tanh(gate(x)) * up(x))."""
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, down.rows), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(lut_mlp_workspace(gate, up, down, B), x.device)
    check(lib().rq_lut_mlp(gate.ref, up.ref, down.ref, _ptr(x), B, _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def stream_read_configs():
    """rq_stream_read_configs: number of grid configurations of the stream-read probe."""
    return lib().rq_stream_read_configs()


def stream_read(buf, config, sink=None):
    """rq_stream_read: one read of the whole of `buf` (a device tensor, 16-byte aligned, nbytes % 16 == 0)
    with 16-byte loads; returns the uint32 sink (one XOR per workgroup) as an int32 tensor."""
    if sink is None:
        sink = torch.empty(lib().rq_stream_read_sink_words(config), dtype=torch.int32, device=buf.device)
    check(lib().rq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), config, _ptr(sink), _stream()))
    return sink


def dense_logits_workspace(rows, B):
    return lib().rq_dense_logits_workspace(rows, B)


def dense_logits(E, h, softcap=30.0, argmax=True, ws=None, out=None):
    """rq_dense_logits: the dense bf16 comparison head; E is [rows][D] bf16 bits (int16 tensor)."""
    rows, D = E.shape
    B = h.shape[0]
    lg = out if out is not None else torch.empty((B, rows), dtype=torch.float32, device=h.device)
    am = torch.empty(B, dtype=torch.int32, device=h.device) if argmax else None
    if ws is None and argmax:
        ws = workspace(dense_logits_workspace(rows, B), h.device)
    check(lib().rq_dense_logits(_ptr(E), rows, D, _ptr(h), B, softcap, _ptr(lg), _ptr(am), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream()))
    return lg, am


def set_stage_events(before, after):
    """rq_set_stage_events: bracket the next lookup+sum kernel launched from this thread with two
    torch.cuda.Event objects (timing enabled), or clear the hook with (None, None)."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:   # torch creates the HIP event lazily, on first record
            ev.record()
        return ctypes.c_void_p(ev.cuda_event)
    check(lib().rq_set_stage_events(handle(before), handle(after)))
