"""affine_q4_gemv_amd -- affine-Q4 row-batched GEMV for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libq4mv.so`` (declared in ``include/q4mv.h``).
The functions here have the same names as the C entry points and only marshal arguments:
they check dtypes, shapes and devices of torch tensors, allocate outputs with torch when the
caller passes none, and hand raw device pointers and the current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no other path. If
the library cannot be loaded, importing works but every call raises.

Tensor conventions (all on one GPU, contiguous):
  codes  uint8   [n_mat, out_dim, in_dim]      one 4-bit code per byte
  w      int32   [n_mat, out_dim, in_dim // 8] packed codes (bit pattern of u32 words)
  scales bfloat16 [n_mat, out_dim, in_dim // 64] (bias the same)
  x      float32 [n_rows, in_dim]              n_rows = n_mat * nb
  xe, xo float16 [n_rows, in_dim // 2]
  xsum   float32 [n_rows, in_dim // 32]
  y      float32 [n_mat, nb, out_dim]
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4mv.so")

Q4MV_OK = 0
PATH_AUTO, PATH_VALU, PATH_VALU_2ROW, PATH_MFMA = 0, 1, 2, 3
MAX_NB = 16

_lib = None


class Q4mvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


def lib():
    """The loaded ``libq4mv.so`` with argument types set (builds it first if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.q4mv_pack_codes.argtypes = [p, p, i64, p]
        L.q4mv_prepare_x.argtypes = [p, i32, i32, p, p, p, p]
        gemv = [p, p, p, p, p, p, p, i32, i32, i32, i32]
        L.q4mv.argtypes = gemv + [p]
        L.q4mv_2row.argtypes = gemv + [p]
        L.q4mv_path.argtypes = gemv + [i32, p]
        L.q4mv_fused.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, p]
        L.q4mv_silu.argtypes = gemv + [f32, p]
        L.q4mv_path_silu.argtypes = gemv + [f32, i32, p]
        L.q4mv_swiglu_prep.argtypes = [p, i32, i32, p, p, p, p]
        L.q4mv_quantize.argtypes = [p, p, p, p, i64, i32, p]
        L.q4mv_pack_lowbit.argtypes = [i32, p, p, i64, i32, p]
        L.q4mv_lowbit.argtypes = [i32] + [p] * 7 + [i32] * 5 + [p]
        L.q4mv_experts.argtypes = [p, p, p, i32, p, i32, p, p, p, p] + [i32] * 5 + [p]
        L.q4mv_experts_fused.argtypes = [p, p, p, i32, p, i32, p, p] + [i32] * 6 + [p]
        L.q4mv_combine.argtypes = [p, p, p, i32, i32, i32, p]
        L.q4mv_auto_path.argtypes = [i32, i32, i32, i32]
        L.q4mv_status_str.argtypes = [i32]
        L.q4mv_status_str.restype = ctypes.c_char_p
        L.q4mv_version.argtypes = []
        for fn in ("q4mv_pack_codes", "q4mv_prepare_x", "q4mv", "q4mv_2row", "q4mv_path",
                   "q4mv_fused",
                   "q4mv_silu", "q4mv_path_silu", "q4mv_swiglu_prep", "q4mv_quantize",
                   "q4mv_auto_path",
                   "q4mv_version"):
            getattr(L, fn).restype = i32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().q4mv_status_str(int(status)).decode()


def _torch():
    import torch
    return torch


def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return _torch().cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _check(fn, status):
    if status != Q4MV_OK:
        raise Q4mvError(fn, status)


def q4mv_pack_codes(codes, w=None, stream=None):
    """Pack u8 codes [..., in_dim] eight per u32 word, low nibble first -> int32 [..., in_dim/8]."""
    torch = _torch()
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous():
        raise ValueError("codes: contiguous uint8 GPU tensor expected")
    if codes.shape[-1] % 8:
        raise ValueError("codes: last dimension must be a multiple of 8")
    shape = (*codes.shape[:-1], codes.shape[-1] // 8)
    if w is None:
        w = torch.empty(shape, dtype=torch.int32, device=codes.device)
    _need(w, torch.int32, shape, "w")
    _check("q4mv_pack_codes", lib().q4mv_pack_codes(codes.data_ptr(), w.data_ptr(),
                                                     codes.numel(), _stream(codes, stream)))
    return w


def q4mv_prepare_x(x, xe=None, xo=None, xsum=None, stream=None):
    """x f32 [n_rows, in_dim] -> (xe, xo f16 [n_rows, in_dim/2], xsum f32 [n_rows, in_dim/32])."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x: expected [n_rows, in_dim]")
    n, k = x.shape
    _need(x, torch.float32, (n, k), "x")
    dev = x.device
    xe = torch.empty((n, k // 2), dtype=torch.float16, device=dev) if xe is None else xe
    xo = torch.empty((n, k // 2), dtype=torch.float16, device=dev) if xo is None else xo
    xsum = torch.empty((n, k // 32), dtype=torch.float32, device=dev) if xsum is None else xsum
    _need(xe, torch.float16, (n, k // 2), "xe")
    _need(xo, torch.float16, (n, k // 2), "xo")
    _need(xsum, torch.float32, (n, k // 32), "xsum")
    _check("q4mv_prepare_x", lib().q4mv_prepare_x(x.data_ptr(), n, k, xe.data_ptr(),
                                                   xo.data_ptr(), xsum.data_ptr(),
                                                   _stream(x, stream)))
    return xe, xo, xsum


def _gemv(fn_name, w, scales, biases, xe, xo, xsum, nb, y, stream, path=None, div=None):
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w: expected [n_mat, out_dim, in_dim/8]")
    n_mat, out_dim, w8 = w.shape
    in_dim = w8 * 8
    _need(w, torch.int32, (n_mat, out_dim, w8), "w")
    _need(scales, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "scales")
    _need(biases, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "biases")
    _need(xe, torch.float16, (n_mat * nb, in_dim // 2), "xe")
    _need(xo, torch.float16, (n_mat * nb, in_dim // 2), "xo")
    _need(xsum, torch.float32, (n_mat * nb, in_dim // 32), "xsum")
    if y is None:
        y = torch.empty((n_mat, nb, out_dim), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, (n_mat, nb, out_dim), "y")
    args = [w.data_ptr(), scales.data_ptr(), biases.data_ptr(), xe.data_ptr(), xo.data_ptr(),
            xsum.data_ptr(), y.data_ptr(), n_mat, out_dim, in_dim, nb]
    if div is not None:
        args.append(float(div))
    if path is not None:
        args.append(int(path))
    args.append(_stream(w, stream))
    _check(fn_name, getattr(lib(), fn_name)(*args))
    return y


def q4mv(w, scales, biases, xe, xo, xsum, nb, y=None, stream=None):
    """y[m, r, o] for all n_mat matrices and nb activation rows (automatic kernel choice)."""
    return _gemv("q4mv", w, scales, biases, xe, xo, xsum, nb, y, stream)


def q4mv_2row(w, scales, biases, xe, xo, xsum, nb, y=None, stream=None):
    """Two output rows per lane group; bitwise equal to :func:`q4mv`. out_dim must be even."""
    return _gemv("q4mv_2row", w, scales, biases, xe, xo, xsum, nb, y, stream)


def q4mv_path(w, scales, biases, xe, xo, xsum, nb, path, y=None, stream=None):
    """:func:`q4mv` with an explicit kernel (PATH_VALU, PATH_VALU_2ROW, PATH_MFMA)."""
    return _gemv("q4mv_path", w, scales, biases, xe, xo, xsum, nb, y, stream, path=path)


def q4mv_fused(w, scales, biases, x, nb, path=PATH_AUTO, y=None, stream=None):
    """:func:`q4mv_prepare_x` + :func:`q4mv_path` in one launch from f32 activations
    x [n_mat*nb, in_dim]; bitwise the two-call result on the same path."""
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w: expected [n_mat, out_dim, in_dim/8]")
    n_mat, out_dim, w8 = w.shape
    in_dim = w8 * 8
    _need(w, torch.int32, (n_mat, out_dim, w8), "w")
    _need(scales, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "scales")
    _need(biases, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "biases")
    _need(x, torch.float32, (n_mat * nb, in_dim), "x")
    if y is None:
        y = torch.empty((n_mat, nb, out_dim), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, (n_mat, nb, out_dim), "y")
    _check("q4mv_fused", lib().q4mv_fused(w.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                           x.data_ptr(), y.data_ptr(), n_mat, out_dim, in_dim,
                                           nb, int(path), _stream(w, stream)))
    return y


def q4mv_silu(w, scales, biases, xe, xo, xsum, nb, div, y=None, stream=None):
    """silu(q4mv(...) / div), fused into the GEMV's store."""
    return _gemv("q4mv_silu", w, scales, biases, xe, xo, xsum, nb, y, stream, div=div)


def q4mv_path_silu(w, scales, biases, xe, xo, xsum, nb, div, path, y=None, stream=None):
    """:func:`q4mv_silu` with an explicit kernel path."""
    return _gemv("q4mv_path_silu", w, scales, biases, xe, xo, xsum, nb, y, stream, path=path,
                 div=div)


def q4mv_quantize(wf, stream=None):
    """Dense f32 weights [..., in_dim] -> (w int32 [..., in_dim/8], scales, biases bfloat16
    [..., in_dim/64]): affine-Q4 with per-64 min/max (see include/q4mv.h)."""
    torch = _torch()
    if wf.dtype != torch.float32 or not wf.is_cuda or not wf.is_contiguous():
        raise ValueError("wf: contiguous float32 GPU tensor expected")
    in_dim = wf.shape[-1]
    lead = tuple(wf.shape[:-1])
    n_rows = wf.numel() // in_dim if in_dim else 0
    w = torch.empty(lead + (in_dim // 8,), dtype=torch.int32, device=wf.device)
    s = torch.empty(lead + (in_dim // 64,), dtype=torch.bfloat16, device=wf.device)
    b = torch.empty_like(s)
    _check("q4mv_quantize", lib().q4mv_quantize(wf.data_ptr(), w.data_ptr(), s.data_ptr(),
                                                 b.data_ptr(), n_rows, in_dim,
                                                 _stream(wf, stream)))
    return w, s, b


def q4mv_swiglu_prep(gu, xe=None, xo=None, xsum=None, stream=None):
    """gu f32 [n_rows, 2*inter] (gate | up) -> prep of h = silu(gate)*up:
    (xe, xo f16 [n_rows, inter/2], xsum f32 [n_rows, inter/32])."""
    torch = _torch()
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu: expected [n_rows, 2*inter]")
    n, k2 = gu.shape
    k = k2 // 2
    _need(gu, torch.float32, (n, k2), "gu")
    dev = gu.device
    xe = torch.empty((n, k // 2), dtype=torch.float16, device=dev) if xe is None else xe
    xo = torch.empty((n, k // 2), dtype=torch.float16, device=dev) if xo is None else xo
    xsum = torch.empty((n, k // 32), dtype=torch.float32, device=dev) if xsum is None else xsum
    _need(xe, torch.float16, (n, k // 2), "xe")
    _need(xo, torch.float16, (n, k // 2), "xo")
    _need(xsum, torch.float32, (n, k // 32), "xsum")
    _check("q4mv_swiglu_prep", lib().q4mv_swiglu_prep(gu.data_ptr(), n, k, xe.data_ptr(),
                                                       xo.data_ptr(), xsum.data_ptr(),
                                                       _stream(gu, stream)))
    return xe, xo, xsum


def q4mv_pack_lowbit(bits, codes, stream=None):
    """4-bit codes uint8 [..., in_dim] -> the Q2 / Q3 packed words int32 [..., in_dim/32*bits]
    (the low-bit code is the 4-bit code's top bits)."""
    torch = _torch()
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous():
        raise ValueError("codes: contiguous uint8 GPU tensor expected")
    in_dim = codes.shape[-1]
    n_rows = codes.numel() // in_dim if in_dim else 0
    w = torch.empty((*codes.shape[:-1], in_dim // 32 * int(bits)), dtype=torch.int32,
                    device=codes.device)
    _check("q4mv_pack_lowbit", lib().q4mv_pack_lowbit(int(bits), codes.data_ptr(), w.data_ptr(),
                                                       n_rows, in_dim, _stream(codes, stream)))
    return w


def q4mv_lowbit(bits, w, scales, biases, xe, xo, xsum, nb, path=PATH_AUTO, y=None,
                stream=None):
    """Q2 / Q3 GEMV: w int32 [n_mat, out_dim, in_dim/32*bits] -> y f32 [n_mat, nb, out_dim]."""
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w: expected [n_mat, out_dim, in_dim/32*bits]")
    n_mat, out_dim, wpr = w.shape
    if bits not in (2, 3) or wpr % bits:
        raise ValueError("bits must be 2 or 3 and w's last dimension a multiple of it")
    in_dim = wpr // bits * 32
    _need(w, torch.int32, (n_mat, out_dim, wpr), "w")
    _need(scales, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "scales")
    _need(biases, torch.bfloat16, (n_mat, out_dim, in_dim // 64), "biases")
    _need(xe, torch.float16, (n_mat * nb, in_dim // 2), "xe")
    _need(xo, torch.float16, (n_mat * nb, in_dim // 2), "xo")
    _need(xsum, torch.float32, (n_mat * nb, in_dim // 32), "xsum")
    if y is None:
        y = torch.empty((n_mat, nb, out_dim), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, (n_mat, nb, out_dim), "y")
    _check("q4mv_lowbit", lib().q4mv_lowbit(
        int(bits), w.data_ptr(), scales.data_ptr(), biases.data_ptr(), xe.data_ptr(),
        xo.data_ptr(), xsum.data_ptr(), y.data_ptr(), n_mat, out_dim, in_dim, nb, int(path),
        _stream(w, stream)))
    return y


def q4mv_experts(w, scales, biases, sel, xe, xo, xsum, nb, x_shared, path=PATH_AUTO, y=None,
                 stream=None):
    """Slot u = bank matrix sel[u] (int32 GPU tensor) over its activation rows: rows 0..nb-1
    for every slot when x_shared, else rows u*nb .. u*nb+nb-1 -> y f32 [n_sel, nb, out_dim]."""
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w: expected [n_bank, out_dim, in_dim/8]")
    n_bank, out_dim, w8 = w.shape
    in_dim = w8 * 8
    _need(w, torch.int32, (n_bank, out_dim, w8), "w")
    _need(scales, torch.bfloat16, (n_bank, out_dim, in_dim // 64), "scales")
    _need(biases, torch.bfloat16, (n_bank, out_dim, in_dim // 64), "biases")
    if sel.dim() != 1:
        raise ValueError("sel: expected [n_sel]")
    n_sel = sel.shape[0]
    _need(sel, torch.int32, (n_sel,), "sel")
    rows = nb if x_shared else n_sel * nb
    _need(xe, torch.float16, (rows, in_dim // 2), "xe")
    _need(xo, torch.float16, (rows, in_dim // 2), "xo")
    _need(xsum, torch.float32, (rows, in_dim // 32), "xsum")
    if y is None:
        y = torch.empty((n_sel, nb, out_dim), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, (n_sel, nb, out_dim), "y")
    _check("q4mv_experts", lib().q4mv_experts(
        w.data_ptr(), scales.data_ptr(), biases.data_ptr(), n_bank, sel.data_ptr(), n_sel,
        xe.data_ptr(), xo.data_ptr(), xsum.data_ptr(), y.data_ptr(), out_dim, in_dim, nb,
        int(bool(x_shared)), int(path), _stream(w, stream)))
    return y


def q4mv_experts_fused(w, scales, biases, sel, x, nb, x_shared, swiglu=False, path=PATH_AUTO,
                       y=None, stream=None):
    """:func:`q4mv_experts` with the activation prep inside the launch, from f32 rows x:
    [rows, in_dim], or with swiglu [rows, 2*in_dim] gate|up rows whose activations are
    silu(gate)*up (rows = nb when x_shared, else n_sel*nb). Bitwise the two-call result."""
    torch = _torch()
    if w.dim() != 3:
        raise ValueError("w: expected [n_bank, out_dim, in_dim/8]")
    n_bank, out_dim, w8 = w.shape
    in_dim = w8 * 8
    _need(w, torch.int32, (n_bank, out_dim, w8), "w")
    _need(scales, torch.bfloat16, (n_bank, out_dim, in_dim // 64), "scales")
    _need(biases, torch.bfloat16, (n_bank, out_dim, in_dim // 64), "biases")
    if sel.dim() != 1:
        raise ValueError("sel: expected [n_sel]")
    n_sel = sel.shape[0]
    _need(sel, torch.int32, (n_sel,), "sel")
    rows = nb if x_shared else n_sel * nb
    _need(x, torch.float32, (rows, 2 * in_dim if swiglu else in_dim), "x")
    if y is None:
        y = torch.empty((n_sel, nb, out_dim), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, (n_sel, nb, out_dim), "y")
    _check("q4mv_experts_fused", lib().q4mv_experts_fused(
        w.data_ptr(), scales.data_ptr(), biases.data_ptr(), n_bank, sel.data_ptr(), n_sel,
        x.data_ptr(), y.data_ptr(), out_dim, in_dim, nb, int(bool(x_shared)),
        int(bool(swiglu)), int(path), _stream(w, stream)))
    return y


def q4mv_combine(y, wmap, out=None, stream=None):
    """y f32 [n_u, nb, out_dim], wmap f32 [nb, n_u] -> out f32 [nb, out_dim]."""
    torch = _torch()
    if y.dim() != 3:
        raise ValueError("y: expected [n_u, nb, out_dim]")
    n_u, nb, out_dim = y.shape
    _need(y, torch.float32, (n_u, nb, out_dim), "y")
    _need(wmap, torch.float32, (nb, n_u), "wmap")
    if out is None:
        out = torch.empty((nb, out_dim), dtype=torch.float32, device=y.device)
    _need(out, torch.float32, (nb, out_dim), "out")
    _check("q4mv_combine", lib().q4mv_combine(y.data_ptr(), wmap.data_ptr(), out.data_ptr(),
                                               n_u, nb, out_dim, _stream(y, stream)))
    return out


def q4mv_auto_path(in_dim: int, nb: int, two_row: bool = False, out_dim: int = 2) -> int:
    return lib().q4mv_auto_path(int(in_dim), int(nb), int(bool(two_row)), int(out_dim))


def q4mv_version() -> int:
    return lib().q4mv_version()
