"""ctypes binding of librq_lut.so (include/rq_lut.h), one Python function per C entry point.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's
kernels. The library is loaded on first use and a missing build raises.
RQ_LUT_LIB names another build of the same sources to load instead (the
host-only sanitizer build of the CPU test run uses it).
"""
import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RQ_LUT_LIB") or os.path.join(HERE, "librq_lut.so")

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
           "rq_lut_logits", "rq_lut_logits_static", "rq_logits_method", "rq_logits_workspace", "rq_logits", "rq_decode_rows", "rq_lut_matvec_workspace", "rq_lut_matvec",
           "rq_lut_mlp_workspace", "rq_lut_mlp", "rq_residual_norm", "rq_dense_tiled_bytes", "rq_pack_dense", "rq_dense_logits_workspace", "rq_dense_logits", "rq_stream_read_configs",
           "rq_stream_read_sink_words", "rq_stream_read", "rq_lds_gather_sink_words", "rq_lds_gather",
           "rq_set_stage_events", "rq_lut_logits_plan", "rq_status_string",
           "rq_last_error", "rq_version")


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
            "rq_lut_logits_static": (_i32, [_MP, _vp, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp]),
            "rq_logits_method": (_i32, [_MP, _i32]),
            "rq_logits_workspace": (_sz, [_MP, _i32, _i32]),
            "rq_logits": (_i32, [_MP, _vp, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
            "rq_decode_rows": (_i32, [_MP, _vp, _i32, _i32, _vp, _vp, _vp]),
            "rq_lut_matvec_workspace": (_sz, [_MP, _i32]),
            "rq_lut_matvec": (_i32, [_MP, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
            "rq_lut_mlp_workspace": (_sz, [_MP, _MP, _MP, _i32]),
            "rq_lut_mlp": (_i32, [_MP, _MP, _MP, _vp, _i32, _vp, _vp, _sz, _vp]),
            "rq_residual_norm": (_i32, [_vp, _vp, _vp, _i32, _f32, _vp]),
            "rq_dense_tiled_bytes": (_sz, [_i64, _i32]),
            "rq_pack_dense": (_i32, [_vp, _i64, _i32, _vp, _vp]),
            "rq_dense_logits_workspace": (_sz, [_i64, _i32]),
            "rq_dense_logits": (_i32, [_vp, _i64, _i32, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
            "rq_stream_read_configs": (_i32, []),
            "rq_stream_read_sink_words": (_sz, [_i32]),
            "rq_stream_read": (_i32, [_vp, _sz, _i32, _vp, _vp]),
            "rq_lds_gather_sink_words": (_sz, []),
            "rq_lds_gather": (_i32, [_i32, _i32, _vp, _vp]),
            "rq_set_stage_events": (_i32, [_vp, _vp]),
            "rq_lut_logits_plan": (_i32, [_MP, _i32, _i32, ctypes.POINTER(_i32)]),
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


def _arg(t, name, dtype, shape=None, numel=None, min_numel=None):
    """Validate a tensor argument before its pointer reaches the library: dtype, shape (or element
    count), contiguity and device. The library sees only pointers and sizes, so a tensor of the
    wrong type or size here would otherwise be read or written out of its bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _gpu(**tensors):
    """Every tensor argument of a call must live on the GPU (checked after the per-argument checks)."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name}: must be a GPU tensor (device {t.device})")


_LUT_TORCH = {"f32": torch.float32, "bf16": torch.int16}


def _lut_dtype_of(lut, lut_dtype):
    """The table's dtype name from its tensor (float32: fp32 entries, int16: bf16 bit patterns);
    an explicit lut_dtype must agree with it."""
    if not isinstance(lut, torch.Tensor):
        raise TypeError("lut: expected a torch.Tensor")
    have = {torch.float32: "f32", torch.int16: "bf16"}.get(lut.dtype)
    if have is None:
        raise ValueError(f"lut: dtype {lut.dtype}; tables are float32 (fp32) or int16 (bf16 bits)")
    if lut_dtype is not None and lut_dtype != have:
        raise ValueError(f"lut_dtype={lut_dtype!r} but the table tensor holds {have} entries ({lut.dtype})")
    return have


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
    B = x.shape[0] if x.dim() == 2 else -1
    _arg(x, "x", torch.float32, shape=(B, W.D))
    if x2 is not None:
        _arg(x2, "x2", torch.float32, shape=(B, W.D))
    n = lut_bytes(W, B, lut_dtype) // (2 if lut_dtype == "bf16" else 4)
    if out is None:
        out = torch.empty(n, dtype=_LUT_TORCH[lut_dtype], device=x.device)
    _arg(out, "out", _LUT_TORCH[lut_dtype], numel=n)
    _gpu(x=x, x2=x2, out=out)
    check(lib().rq_build_lut(W.ref, _ptr(x), _ptr(x2), prologue, B, _dtype_code(lut_dtype), _ptr(out), _stream()))
    return out


def lut_logits_workspace(W, B, topk=0, lut_dtype="f32"):
    return lib().rq_lut_logits_workspace(W.ref, B, topk, _dtype_code(lut_dtype))


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned device workspace (the library needs no particular initial contents)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _outputs(W, B, topk, dev, logits, argmax, out, argmax_out):
    """Logits, argmax and top-k output tensors of a head call (the caller's, checked, or new ones)."""
    lg = am = None
    if logits:
        lg = out if out is not None else torch.empty((B, W.rows), dtype=torch.float32, device=dev)
        _arg(lg, "out", torch.float32, numel=B * W.rows)
    if argmax:
        am = argmax_out if argmax_out is not None else torch.empty(B, dtype=torch.int32, device=dev)
        _arg(am, "argmax_out", torch.int32, numel=B)
    ti = torch.empty((B, topk), dtype=torch.int32, device=dev) if topk else None
    tv = torch.empty((B, topk), dtype=torch.float32, device=dev) if topk else None
    return lg, am, ti, tv


def _ws(ws, need, dev):
    if ws is None:
        return workspace(need, dev)
    return _arg(ws, "ws", torch.uint8, min_numel=need)


def lut_logits(W, lut, B, softcap=30.0, lut_dtype=None, logits=True, argmax=True, topk=0, ws=None, out=None,
               argmax_out=None):
    """rq_lut_logits: returns (logits [B][rows] | None, argmax [B] | None, topk_ids | None, topk_vals | None).
    The table's dtype is taken from the tensor (float32 or int16 bf16 bits); lut_dtype, if given, must agree."""
    lut_dtype = _lut_dtype_of(lut, lut_dtype)
    _arg(lut, "lut", lut.dtype, numel=lut_bytes(W, B, lut_dtype) // lut.element_size())
    dev = lut.device
    lg, am, ti, tv = _outputs(W, B, topk, dev, logits, argmax, out, argmax_out)
    ws = _ws(ws, lut_logits_workspace(W, B, topk, lut_dtype), dev)
    _gpu(lut=lut, out=lg, argmax_out=am, ws=ws)
    check(lib().rq_lut_logits(W.ref, _ptr(lut), _dtype_code(lut_dtype), B, softcap, _ptr(lg), _ptr(am), topk,
                              _ptr(ti), _ptr(tv), _ptr(ws), ws.numel(), _stream()))
    return lg, am, ti, tv


def lut_logits_static(W, lut, B, softcap=30.0, lut_dtype=None, logits=True, argmax=True, topk=0, out=None,
                      argmax_out=None):
    """rq_lut_logits_static: rq_lut_logits on the library's own per-GPU scratch (no workspace, no allocation
    inside the call; the outputs are allocated here unless given)."""
    lut_dtype = _lut_dtype_of(lut, lut_dtype)
    _arg(lut, "lut", lut.dtype, numel=lut_bytes(W, B, lut_dtype) // lut.element_size())
    lg, am, ti, tv = _outputs(W, B, topk, lut.device, logits, argmax, out, argmax_out)
    _gpu(lut=lut, out=lg, argmax_out=am)
    check(lib().rq_lut_logits_static(W.ref, _ptr(lut), _dtype_code(lut_dtype), B, softcap, _ptr(lg), _ptr(am), topk,
                                     _ptr(ti), _ptr(tv), _stream()))
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
    B = h.shape[0] if h.dim() == 2 else -1
    _arg(h, "h", torch.float32, shape=(B, W.D))
    dev = h.device
    lg, am, ti, tv = _outputs(W, B, topk, dev, logits, argmax, out, argmax_out)
    ws = _ws(ws, logits_workspace(W, B, topk), dev)
    _gpu(h=h, out=lg, argmax_out=am, ws=ws)
    check(lib().rq_logits(W.ref, _ptr(h), B, softcap, _ptr(lg), _ptr(am), topk, _ptr(ti), _ptr(tv), _ptr(ws),
                          ws.numel(), _stream()))
    return lg, am, ti, tv


def decode_rows(W, ids, out_dtype="f32", bad_ids=None, out=None):
    """rq_decode_rows: rows [n][D] (fp32, or bf16 bit patterns as int16)."""
    n = ids.shape[0] if ids.dim() == 1 else -1
    _arg(ids, "ids", torch.int32, shape=(n,))
    if bad_ids is not None:
        _arg(bad_ids, "bad_ids", torch.int32, min_numel=1)
    odt = torch.int16 if out_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty((n, W.D), dtype=odt, device=ids.device)
    _arg(out, "out", odt, numel=n * W.D)
    _gpu(ids=ids, bad_ids=bad_ids, out=out)
    check(lib().rq_decode_rows(W.ref, _ptr(ids), n, _dtype_code(out_dtype), _ptr(out), _ptr(bad_ids), _stream()))
    return out


def lut_matvec_workspace(W, B):
    return lib().rq_lut_matvec_workspace(W.ref, B)


def lut_matvec(W, x, x2=None, prologue=RQ_PRO_NONE, ws=None, out=None):
    """rq_lut_matvec: y [B][rows] = W a, a = x or gelu_tanh(x) * x2."""
    B = x.shape[0] if x.dim() == 2 else -1
    _arg(x, "x", torch.float32, shape=(B, W.D))
    if x2 is not None:
        _arg(x2, "x2", torch.float32, shape=(B, W.D))
    y = out if out is not None else torch.empty((B, W.rows), dtype=torch.float32, device=x.device)
    _arg(y, "out", torch.float32, numel=B * W.rows)
    ws = _ws(ws, lut_matvec_workspace(W, B), x.device)
    _gpu(x=x, x2=x2, out=y, ws=ws)
    check(lib().rq_lut_matvec(W.ref, _ptr(x), _ptr(x2), prologue, B, _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def lut_mlp_workspace(gate, up, down, B):
    return lib().rq_lut_mlp_workspace(gate.ref, up.ref, down.ref, B)


def lut_mlp(gate, up, down, x, ws=None, out=None):
    """rq_lut_mlp: y [B][down.rows] = down(gelu_tanh(gate(x)) * up(x))."""
    B = x.shape[0] if x.dim() == 2 else -1
    _arg(x, "x", torch.float32, shape=(B, gate.D))
    y = out if out is not None else torch.empty((B, down.rows), dtype=torch.float32, device=x.device)
    _arg(y, "out", torch.float32, numel=B * down.rows)
    ws = _ws(ws, lut_mlp_workspace(gate, up, down, B), x.device)
    _gpu(x=x, out=y, ws=ws)
    check(lib().rq_lut_mlp(gate.ref, up.ref, down.ref, _ptr(x), B, _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def stream_read_configs():
    """rq_stream_read_configs: number of grid configurations of the stream-read probe."""
    return lib().rq_stream_read_configs()


def stream_read(buf, config, sink=None):
    """rq_stream_read: one read of the whole of `buf` (a device tensor, 16-byte aligned, nbytes % 16 == 0)
    with 16-byte loads; returns the uint32 sink (one XOR per workgroup) as an int32 tensor."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf: must be a contiguous GPU tensor")
    words = lib().rq_stream_read_sink_words(config)
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    _arg(sink, "sink", torch.int32, min_numel=words)
    _gpu(sink=sink)
    check(lib().rq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), config, _ptr(sink), _stream()))
    return sink


def lds_gather(width, reps, sink=None):
    """rq_lds_gather: the LDS random-gather probe; returns its sink (one word per workgroup) as int32."""
    words = lib().rq_lds_gather_sink_words()
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device="cuda")
    _arg(sink, "sink", torch.int32, min_numel=words)
    _gpu(sink=sink)
    check(lib().rq_lds_gather(width, reps, _ptr(sink), _stream()))
    return sink


def residual_norm(h, x, y=None, eps=1e-6):
    """rq_residual_norm: h += rms(y) (when y is given), then x = rms(h); fp32 vectors of one length
    ([D] or [1][D]) on the GPU, x not overlapping h or y. Returns x."""
    D = h.numel()
    _arg(h, "h", torch.float32, numel=D)
    _arg(x, "x", torch.float32, numel=D)
    if y is not None:
        _arg(y, "y", torch.float32, numel=D)
    _gpu(h=h, x=x, y=y)
    check(lib().rq_residual_norm(_ptr(y), _ptr(h), _ptr(x), D, eps, _stream()))
    return x


class DenseHead:
    """A dense bf16 matrix E[rows][D] in the tiled layout rq_dense_logits reads
    ([ceil(rows/16)][ceil(D/32)][16][32] bf16, zero padded), made by pack_dense."""

    def __init__(self, tiles, rows, D):
        self.tiles, self.rows, self.D = tiles, rows, D

    @property
    def nbytes(self):
        return self.tiles.numel() * self.tiles.element_size()


def dense_tiled_bytes(rows, D):
    return lib().rq_dense_tiled_bytes(rows, D)


def pack_dense(E):
    """rq_pack_dense: the tiled copy of E ([rows][D] bf16 bits, int16 tensor on the GPU)."""
    if E.dim() != 2:
        raise ValueError("E: expected [rows][D] bf16 bits")
    rows, D = E.shape
    _arg(E, "E", torch.int16, shape=(rows, D))
    nb = dense_tiled_bytes(rows, D)
    if nb == 0:
        raise RQError(RQ_ERR_SHAPE, f"dense matrix {rows} x {D} out of range")
    Et = torch.empty(nb // 2, dtype=torch.int16, device=E.device)
    _gpu(E=E, Et=Et)
    check(lib().rq_pack_dense(_ptr(E), rows, D, _ptr(Et), _stream()))
    return DenseHead(Et, rows, D)


def dense_logits_workspace(rows, B):
    return lib().rq_dense_logits_workspace(rows, B)


def dense_logits(head, h, softcap=30.0, argmax=True, ws=None, out=None):
    """rq_dense_logits: the dense bf16 comparison head (a DenseHead from pack_dense)."""
    if not isinstance(head, DenseHead):
        raise TypeError("dense_logits takes the DenseHead that pack_dense returns")
    rows, D = head.rows, head.D
    _arg(head.tiles, "head.tiles", torch.int16, numel=dense_tiled_bytes(rows, D) // 2)
    B = h.shape[0] if h.dim() == 2 else -1
    _arg(h, "h", torch.float32, shape=(B, D))
    lg = out if out is not None else torch.empty((B, rows), dtype=torch.float32, device=h.device)
    _arg(lg, "out", torch.float32, numel=B * rows)
    am = torch.empty(B, dtype=torch.int32, device=h.device) if argmax else None
    ws = _ws(ws, dense_logits_workspace(rows, B), h.device)
    _gpu(Et=head.tiles, h=h, out=lg, ws=ws)
    check(lib().rq_dense_logits(_ptr(head.tiles), rows, D, _ptr(h), B, softcap, _ptr(lg), _ptr(am), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream()))
    return lg, am


PLAN_FIELDS = ("BT", "P", "chunks", "cpg", "G", "steps", "rps", "S", "rset", "NBT")


def lut_logits_plan(W, B, lut_dtype="f32"):
    """rq_lut_logits_plan: the tiling rq_lut_logits uses, as a dict of PLAN_FIELDS."""
    buf = (_i32 * 10)()
    check(lib().rq_lut_logits_plan(W.ref, B, _dtype_code(lut_dtype), buf))
    return dict(zip(PLAN_FIELDS, list(buf)))


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
