"""CPU oracle for the affine-Q4 row-batched GEMV -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code with the device library ``affine_q4_gemv_amd`` and
never imports it.

* :func:`gemv` / :func:`gemv_rows` -- the plain definition, in double precision, from
  ``q4ref.c`` (C, pthreads). Codes are taken unpacked (u8 per code).
* :func:`prepare_x` -- what the activation prep produces: the f16 even/odd streams and the
  per-32-chunk sums of the same f16-rounded values. Follows the Constant BATCH_MSL page,
  quantized_rows consumers and the ``fn_norm_prep_b`` / ``fn_moe_act_b`` kernels: element
  ``2k`` goes to ``xe[k]``, element ``2k+1`` to ``xo[k]``, and each 32-element chunk
  contributes one sum. The sum is taken over the f16-rounded values, as ``fn_moe_act_b``
  does (``fn_norm_prep_b`` sums the f32 values instead; the f16 reading keeps the bias term
  and the code term on the same x).
* :func:`silu`, :func:`gemv_silu`, :func:`swiglu` -- the fused epilogues of the same page:
  ``fn_qmv_silu_b`` stores silu(y / div), and ``fn_moe_act_b`` forms silu(gate) * up from the
  stacked gate/up output before the down projection's prep.
* :func:`gemv_lowbit`, :func:`pack_lowbit` -- the Q2 / Q3 variants (dense double
  reconstruction at the range midpoints; the packed layout the device reads).
* :func:`experts`, :func:`combine` -- the selected-expert dispatch (a bank, expert ids,
  shared or per-expert activation rows) and the routing-weighted sum of the expert outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4ref.c")
_LIB = os.path.join(_HERE, "libq4ref.so")
_lib = None

GROUP = 64


def build(force: bool = True) -> str:
    """Compile ``q4ref.c`` into ``oracle/libq4ref.so`` with the host C compiler."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.q4ref_gemv.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p, ctypes.c_int]
        lib.q4ref_gemv.restype = ctypes.c_int
        lib.q4ref_gemv_rows.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p, i64, p, p,
                                        ctypes.c_int]
        lib.q4ref_gemv_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _check(codes, scales, biases, x):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if codes.ndim != 3 or x.ndim != 3:
        raise ValueError("codes [n_mat][out][in] and x [n_mat][nb][in] expected")
    n_mat, out_dim, in_dim = codes.shape
    if in_dim % GROUP or scales.shape != (n_mat, out_dim, in_dim // GROUP) \
            or biases.shape != scales.shape or x.shape[0] != n_mat or x.shape[2] != in_dim:
        raise ValueError("inconsistent shapes")
    if codes.size and codes.max() > 15:
        raise ValueError("codes must be 0..15")
    return codes, scales, biases, x


def gemv(codes, scales, biases, x, nthreads: int | None = None, with_bound: bool = True):
    """y[m][r][o] (f64 [n_mat][nb][out]) and the per-element bound sum_i |Sqx|+|Bx|."""
    codes, scales, biases, x = _check(codes, scales, biases, x)
    n_mat, out_dim, in_dim = codes.shape
    nb = x.shape[1]
    y = np.empty((n_mat, nb, out_dim), dtype=np.float64)
    bound = np.empty_like(y) if with_bound else None
    rc = _load().q4ref_gemv(codes.ctypes.data, scales.ctypes.data, biases.ctypes.data,
                            x.ctypes.data, n_mat, out_dim, in_dim, nb, y.ctypes.data,
                            bound.ctypes.data if with_bound else None,
                            nthreads or default_threads())
    if rc:
        raise ValueError(f"q4ref_gemv returned {rc}")
    return y, bound


def gemv_rows(codes, scales, biases, x, mats, rows, nthreads: int | None = None):
    """Selected outputs: for each (mats[t], rows[t]) all nb values -> y, bound [n_sel][nb]."""
    codes, scales, biases, x = _check(codes, scales, biases, x)
    n_mat, out_dim, in_dim = codes.shape
    nb = x.shape[1]
    mats = np.ascontiguousarray(mats, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if mats.shape != rows.shape or mats.ndim != 1:
        raise ValueError("mats and rows must be 1-D of equal length")
    y = np.empty((mats.size, nb), dtype=np.float64)
    bound = np.empty_like(y)
    rc = _load().q4ref_gemv_rows(codes.ctypes.data, scales.ctypes.data, biases.ctypes.data,
                                 x.ctypes.data, n_mat, out_dim, in_dim, nb, mats.ctypes.data,
                                 rows.ctypes.data, mats.size, y.ctypes.data,
                                 bound.ctypes.data, nthreads or default_threads())
    if rc:
        raise ValueError(f"q4ref_gemv_rows returned {rc}")
    return y, bound


def prepare_x(x):
    """Activation prep: x f32 [n][in] -> (xe, xo) f16 [n][in/2] and xsum f64 [n][in/32].

    f32 -> f16 is IEEE round-to-nearest-even (numpy's conversion); xsum[n][c] is the exact
    sum (in double) of the 32 f16-rounded values of chunk c."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % 32:
        raise ValueError("x must be [n_rows][in_dim] with in_dim % 32 == 0")
    with np.errstate(over="ignore"):  # |x| > 65504 -> inf, as IEEE conversion does
        xh = x.astype(np.float16)
    xe = np.ascontiguousarray(xh[:, 0::2])
    xo = np.ascontiguousarray(xh[:, 1::2])
    xsum = xh.astype(np.float64).reshape(x.shape[0], x.shape[1] // 32, 32).sum(axis=2)
    return xe, xo, xsum


def xsum_error_bound(x):
    """Bound on |f32 sum - exact sum| for each 32-chunk of f16 values summed in f32 in any
    order: 31 * 2^-24 * sum |x_i| (standard recursive-summation bound, 31 additions)."""
    with np.errstate(over="ignore"):
        xh = np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)
    a = np.abs(xh).reshape(xh.shape[0], xh.shape[1] // 32, 32).sum(axis=2)
    return 31.0 * 2.0 ** -24 * a


def silu(t):
    """silu(t) = t / (1 + e^-t) in double (the output of fn_qmv_silu_b and the gate of
    fn_moe_act_b on the Constant BATCH_MSL page). Written as t * e^t / (1 + e^t) for t < 0 so
    that e^-t never overflows."""
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(t)
    pos = t >= 0
    out[pos] = t[pos] / (1.0 + np.exp(-t[pos]))
    e = np.exp(t[~pos])
    out[~pos] = t[~pos] * e / (1.0 + e)
    return out


# max |d silu / dt| (attained near t = 2.4): an error e in t moves silu(t) by at most 1.1 e
SILU_LIPSCHITZ = 1.1


def gemv_silu(codes, scales, biases, x, div, nthreads: int | None = None):
    """silu(y / div) for the GEMV y (fn_qmv_silu_b), and the propagated per-element bound:
    an error within bound in y moves the output by at most SILU_LIPSCHITZ * bound / |div|."""
    y, bound = gemv(codes, scales, biases, x, nthreads=nthreads)
    return silu(y / div), SILU_LIPSCHITZ * bound / abs(div)


def swiglu(gu):
    """h = silu(gate) * up for rows of gu = [gate | up] (f64 [n][2*inter] -> [n][inter]), the
    activation of fn_moe_act_b on the Constant BATCH_MSL page."""
    gu = np.asarray(gu, dtype=np.float64)
    if gu.ndim != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [n_rows][2*inter]")
    k = gu.shape[1] // 2
    return silu(gu[:, :k]) * gu[:, k:]


def experts(codes, scales, biases, sel, x, x_shared, nthreads: int | None = None):
    """Selected-expert GEMV (launch_qmatvec_bf16w_sel on the memra-engine qwen4exp_gpu.rs page:
    a bank of matrices, a list of expert ids and an activation stride that may be zero; the
    unique-expert loop of fn_moe_gate_up_b / fn_moe_down_b on the Constant BATCH_MSL page).
    Slot u applies bank matrix sel[u] to activation rows x [nb][in] when x_shared, else to
    x[u] of x [n_sel][nb][in]. Returns y and the per-element bound, f64 [n_sel][nb][out]; a
    slot whose id is outside the bank is NaN (bound 0)."""
    codes = np.asarray(codes)
    sel = np.asarray(sel, dtype=np.int64)
    x = np.asarray(x, dtype=np.float32)
    if sel.ndim != 1 or sel.size == 0:
        raise ValueError("sel must be a non-empty 1-D id list")
    ok = (sel >= 0) & (sel < codes.shape[0])
    e = np.where(ok, sel, 0)
    if x_shared:
        if x.ndim != 2:
            raise ValueError("shared activations: x [nb][in] expected")
        xs = np.broadcast_to(x[None], (sel.size,) + x.shape)
    else:
        if x.ndim != 3 or x.shape[0] != sel.size:
            raise ValueError("per-slot activations: x [n_sel][nb][in] expected")
        xs = x
    y, bound = gemv(codes[e], np.asarray(scales)[e], np.asarray(biases)[e], xs,
                    nthreads=nthreads)
    y[~ok] = np.nan
    bound[~ok] = 0.0
    return y, bound


def combine(y, wmap):
    """Routing-weighted expert sum (the expert sum of fn_moe_combine_b on the Constant
    BATCH_MSL page): out[r][o] = sum_u wmap[r][u] * y[u][r][o] in f64, for y [n_u][nb][out]
    and wmap [nb][n_u]. Also returns sum_u |wmap[r][u] * y[u][r][o]|, the scale of the
    rounding error of any order of f32 multiply-adds."""
    y = np.asarray(y, dtype=np.float64)
    wmap = np.asarray(wmap, dtype=np.float64)
    if y.ndim != 3 or wmap.shape != (y.shape[1], y.shape[0]):
        raise ValueError("y [n_u][nb][out] and wmap [nb][n_u] expected")
    terms = wmap.T[:, :, None] * y
    return terms.sum(axis=0), np.abs(terms).sum(axis=0)


# Low-bit reconstruction w = (K q + M) s + b of fn_q2_rows_h / fn_q3_rows_h on the Constant
# BATCH_MSL page: q is the 4-bit code's top `bits` bits (q4 >> 2, q4 >> 1), placed at the middle
# of the range of 4-bit codes it stands for.
LOWBIT_KM = {2: (4.0, 1.5), 3: (2.0, 0.5)}


def _bf16_to_f64(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gemv_lowbit(bits, codes, scales, biases, x, rows=None):
    """Q2 / Q3 GEMV from 4-bit codes u8 [n_mat][out][in] (the low-bit code is q4 >> (4-bits)),
    in double: y[m][r][o] = sum_i ((K q + M) S + B) x with (K, M) from LOWBIT_KM, and the
    per-element bound sum_i |(K q + M) S x| + |B x|. rows: optional 1-D list of output rows
    (then y and bound are [n_mat][nb][len(rows)])."""
    k, mid = LOWBIT_KM[bits]
    codes = np.asarray(codes)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        codes, scales, biases = codes[:, rows], np.asarray(scales)[:, rows], \
            np.asarray(biases)[:, rows]
    q = (codes.astype(np.uint8) & 15) >> (4 - bits)
    s = np.repeat(_bf16_to_f64(scales), GROUP, axis=2)
    b = np.repeat(_bf16_to_f64(biases), GROUP, axis=2)
    sq = (k * q.astype(np.float64) + mid) * s
    xd = np.asarray(x, dtype=np.float32).astype(np.float64)
    y = np.matmul(xd, np.transpose(sq + b, (0, 2, 1)))
    bound = np.matmul(np.abs(xd), np.transpose(np.abs(sq) + np.abs(b), (0, 2, 1)))
    return y, bound


def pack_lowbit(bits, codes):
    """The packed low-bit words of 4-bit codes u8 [n_rows][in] -> u32 [n_rows][in/32*bits].
    Per 32-code chunk c, column t = 16i + 8u + p (i, u < 2, p < 8) holds q = q4 >> (4-bits):
    Q2: q at bit 4p + 2u of word 2c+i;
    Q3: q >> 1 at that bit of word 3c+i, and q & 1 at bit 4p + 2i + u of word 3c+2 (a chunk
    is its two upper-bit words, then its lowest-bit word).
    Column t's field sits in nibble p of the word that (shifted by 2u) lines up with the
    8 columns 16i + 8u + 0..7: one shift and one mask give a chunk's codes per nibble, and
    per f16 lane pair (p, p + 4) in place."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    C = k // 32
    q = ((codes & 15) >> (4 - bits)).astype(np.uint32).reshape(n, C, 32)
    up = np.zeros((n, C, 2), dtype=np.uint32)
    low = np.zeros((n, C), dtype=np.uint32)
    for t in range(32):
        i, u, p = t // 16, (t // 8) % 2, t % 8
        pos = 4 * p + 2 * u
        if bits == 2:
            up[:, :, i] |= q[:, :, t] << pos
        else:
            up[:, :, i] |= (q[:, :, t] >> 1) << pos
            low |= (q[:, :, t] & 1) << (4 * p + 2 * i + u)
    if bits == 2:
        return up.reshape(n, 2 * C)
    return np.concatenate([up, low[:, :, None]], axis=2).reshape(n, 3 * C)


def _bf16_rne_bits(x):
    """f32 -> bf16 bit pattern, round to nearest even (f32_to_bf16_rne on the memra-engine
    qwen4exp_gpu.rs page); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def quantize(wf):
    """Affine-Q4 quantiser for dense f32 rows [n][in] (in % 64 == 0), following the steps of
    the affine 5-bit host codec host_quant_q5_row (memra-engine qwen4exp_gpu.rs page) with
    16 levels and 64-wide groups, in f32: mn, mx = min, max of the group; d = (mx - mn) / 15;
    id = 1 / d (0 when d == 0 or 1/d is not finite); q = clamp(rint((w - mn) * id), 0, 15).
    Returns codes u8 [n][in], scales and biases as bf16 bits [n][in/64] (bf16(d), bf16(mn)),
    and the f32 d and mn."""
    wf = np.ascontiguousarray(wf, dtype=np.float32)
    if wf.ndim != 2 or wf.shape[1] % GROUP:
        raise ValueError("wf must be [n_rows][in_dim] with in_dim % 64 == 0")
    n, k = wf.shape
    g = wf.reshape(n, k // GROUP, GROUP)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    d = ((mx - mn) / np.float32(15.0)).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    inv[~np.isfinite(inv)] = 0.0
    t = np.rint((g - mn[:, :, None]) * inv[:, :, None]).astype(np.float32)
    q = np.clip(t, 0, 15).astype(np.uint8).reshape(n, k)
    return q, _bf16_rne_bits(d), _bf16_rne_bits(mn), d, mn
