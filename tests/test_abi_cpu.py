"""The C ABI without a GPU: the library loads, exports every declared entry point, and
rejects invalid arguments on the host with the documented status, launching nothing."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4mv.h")

OK, ENULL, ESHAPE, EODD, EALIGN, ELAUNCH, EPATH, EVALUE = 0, -1, -2, -3, -4, -5, -6, -7
A = 0x10000  # a 16-byte aligned fake address: validation fails before anything reads it


@pytest.fixture(scope="module")
def L():
    import affine_q4_gemv_amd as q
    return q.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q4mv\w*)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    fns = declared_functions()
    for name in ("q4mv_prepare_x", "q4mv", "q4mv_2row", "q4mv_pack_codes", "q4mv_path",
                 "q4mv_silu", "q4mv_path_silu", "q4mv_swiglu_prep", "q4mv_auto_path",
                 "q4mv_quantize", "q4mv_experts", "q4mv_combine", "q4mv_pack_lowbit",
                 "q4mv_lowbit", "q4mv_fused", "q4mv_experts_fused",
                 "q4mv_status_str", "q4mv_version"):
        assert name in fns


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    import affine_q4_gemv_amd as q
    for st in (OK, ENULL, ESHAPE, EODD, EALIGN, ELAUNCH, EPATH, EVALUE):
        assert q.status_str(st) and q.status_str(st) != "unknown status"
    assert q.status_str(12345) == "unknown status"
    assert L.q4mv_version() >= 300


def gemv_args(**kw):
    a = dict(w=A, s=A, b=A, xe=A, xo=A, xsum=A, y=A, n_mat=1, out=8, ind=128, nb=1)
    a.update(kw)
    return [a["w"], a["s"], a["b"], a["xe"], a["xo"], a["xsum"], a["y"], a["n_mat"], a["out"],
            a["ind"], a["nb"]]


@pytest.mark.parametrize("fn", ["q4mv", "q4mv_2row"])
def test_gemv_validation(L, fn):
    f = getattr(L, fn)
    for k in ("w", "s", "b", "xe", "xo", "xsum", "y"):
        assert f(*gemv_args(**{k: None}), None) == ENULL
    for kw in (dict(n_mat=0), dict(n_mat=65536), dict(out=0), dict(ind=0), dict(ind=96),
               dict(ind=32), dict(nb=0), dict(nb=17), dict(ind=-64)):
        assert f(*gemv_args(**kw), None) == ESHAPE, kw
    for kw in (dict(w=A + 4), dict(xe=A + 8), dict(xo=A + 2), dict(s=A + 1), dict(b=A + 1),
               dict(xsum=A + 2), dict(y=A + 1)):
        assert f(*gemv_args(**kw), None) == EALIGN, kw


def test_two_row_needs_even_rows(L):
    assert L.q4mv_2row(*gemv_args(out=7), None) == EODD
    assert L.q4mv_path(*gemv_args(out=7), 2, None) == EODD


def test_path_validation(L):
    assert L.q4mv_path(*gemv_args(), 4, None) == EPATH
    assert L.q4mv_path(*gemv_args(), -1, None) == EPATH
    assert L.q4mv_path(*gemv_args(nb=0), 1, None) == ESHAPE


def test_prep_validation(L):
    f = L.q4mv_prepare_x
    assert f(None, 1, 128, A, A, A, None) == ENULL
    assert f(A, 1, 128, A, None, A, None) == ENULL
    assert f(A, 0, 128, A, A, A, None) == ESHAPE
    assert f(A, 1, 96, A, A, A, None) == ESHAPE
    assert f(A + 4, 1, 128, A, A, A, None) == EALIGN
    assert f(A, 1, 128, A + 8, A, A, None) == EALIGN
    assert f(A, 1, 128, A, A, A + 2, None) == EALIGN


def test_pack_validation(L):
    f = L.q4mv_pack_codes
    assert f(None, A, 64, None) == ENULL
    assert f(A, A, 12, None) == ESHAPE
    assert f(A, A, 0, None) == ESHAPE
    assert f(A + 4, A, 64, None) == EALIGN
    assert f(A, A + 2, 64, None) == EALIGN


def test_auto_path(L):
    """The automatic choice depends on nb and out_dim only (never on n_mat)."""
    assert L.q4mv_auto_path(2560, 1, 0, 10) == 1      # one activation row: one-row kernel
    assert L.q4mv_auto_path(2560, 2, 0, 9) == 1       # short launches: one-row kernel
    assert L.q4mv_auto_path(2560, 2, 0, 10) == 1
    assert L.q4mv_auto_path(2560, 2, 0, 9728) == 1    # 304 tiles: one-row kernel at nb 2
    assert L.q4mv_auto_path(2560, 3, 0, 9728) == 3    # and the MFMA kernel at nb 3
    assert L.q4mv_auto_path(2560, 3, 0, 8192) == 3    # 256 tiles
    assert L.q4mv_auto_path(2560, 3, 0, 8160) == 1    # 255 tiles
    assert L.q4mv_auto_path(2560, 4, 0, 32) == 3      # from nb 4 on every shape
    assert L.q4mv_auto_path(640, 1, 1, 2560) == 2     # q4mv_2row: two-row kernel
    assert L.q4mv_auto_path(2560, 3, 1, 2560) == 2
    assert L.q4mv_auto_path(2560, 2, 0, 32768) == 3   # 1024 tiles: the MFMA kernel from 2 rows
    assert L.q4mv_auto_path(2560, 2, 1, 32768) == 3   # q4mv_2row follows q4mv onto it
    assert L.q4mv_auto_path(2560, 2, 0, 32737) == 3
    assert L.q4mv_auto_path(2560, 2, 0, 32736) == 1   # 1023 tiles
    assert L.q4mv_auto_path(2560, 4, 0, 2560) == 3
    assert L.q4mv_auto_path(640, 4, 1, 2560) == 3
    assert L.q4mv_auto_path(2560, 16, 1, 2560) == 3
    assert L.q4mv_auto_path(8192, 16, 0, 8) == 3      # K-sliced where the row does not fit
    assert L.q4mv_auto_path(1 << 20, 16, 0, 8) == 3
    assert L.q4mv_auto_path(640, 1, 1, 7) == EODD
    assert L.q4mv_auto_path(96, 1, 0, 8) == ESHAPE
    assert L.q4mv_auto_path(2560, 17, 0, 8) == ESHAPE
    assert L.q4mv_auto_path(2560, 1, 0, 0) == ESHAPE


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import affine_q4_gemv_amd as q
    with pytest.raises(ValueError):
        q.q4mv_prepare_x(torch.zeros(1, 128))


def test_silu_validation(L):
    for fn, extra in (("q4mv_silu", []), ("q4mv_path_silu", [0])):
        f = getattr(L, fn)
        for div in (0.0, float("inf"), float("-inf"), float("nan")):
            assert f(*gemv_args(), div, *extra, None) == EVALUE, (fn, div)
        # the GEMV's own checks come first
        assert f(*gemv_args(w=None), 2.0, *extra, None) == ENULL
        assert f(*gemv_args(ind=96), 2.0, *extra, None) == ESHAPE
        assert f(*gemv_args(w=A + 4), 2.0, *extra, None) == EALIGN
    assert L.q4mv_path_silu(*gemv_args(), 2.0, 7, None) == EPATH
    assert L.q4mv_path_silu(*gemv_args(out=7), 2.0, 2, None) == EODD


def test_swiglu_prep_validation(L):
    f = L.q4mv_swiglu_prep
    assert f(None, 1, 640, A, A, A, None) == ENULL
    assert f(A, 1, 640, A, None, A, None) == ENULL
    assert f(A, 0, 640, A, A, A, None) == ESHAPE
    assert f(A, 1, 32, A, A, A, None) == ESHAPE
    assert f(A, 1, 96, A, A, A, None) == ESHAPE
    assert f(A + 4, 1, 640, A, A, A, None) == EALIGN
    assert f(A, 1, 640, A + 8, A, A, None) == EALIGN
    assert f(A, 1, 640, A, A, A + 2, None) == EALIGN


def test_quantize_validation(L):
    f = L.q4mv_quantize
    assert f(None, A, A, A, 1, 64, None) == ENULL
    assert f(A, A, None, A, 1, 64, None) == ENULL
    assert f(A, A, A, A, 0, 64, None) == ESHAPE
    assert f(A, A, A, A, 1, 96, None) == ESHAPE
    assert f(A + 4, A, A, A, 1, 64, None) == EALIGN
    assert f(A, A + 2, A, A, 1, 64, None) == EALIGN
    assert f(A, A, A + 1, A, 1, 64, None) == EALIGN


def experts_args(**kw):
    a = dict(w=A, s=A, b=A, n_bank=4, sel=A, n_sel=2, xe=A, xo=A, xsum=A, y=A, out=8, ind=128,
             nb=1, shared=0, path=0)
    a.update(kw)
    return [a[k] for k in ("w", "s", "b", "n_bank", "sel", "n_sel", "xe", "xo", "xsum", "y",
                           "out", "ind", "nb", "shared", "path")] + [None]


def test_experts_validation(L):
    f = L.q4mv_experts
    for k in ("w", "s", "b", "sel", "xe", "xo", "xsum", "y"):
        assert f(*experts_args(**{k: None})) == ENULL, k
    for kw in (dict(n_bank=0), dict(n_sel=0), dict(n_sel=65536), dict(out=0), dict(ind=96),
               dict(ind=32), dict(nb=0), dict(nb=17)):
        assert f(*experts_args(**kw)) == ESHAPE, kw
    for kw in (dict(w=A + 4), dict(sel=A + 2), dict(xe=A + 8), dict(xo=A + 2), dict(s=A + 1),
               dict(b=A + 1), dict(xsum=A + 2), dict(y=A + 1)):
        assert f(*experts_args(**kw)) == EALIGN, kw
    assert f(*experts_args(path=4)) == EPATH
    assert f(*experts_args(path=-1)) == EPATH
    assert f(*experts_args(path=2, out=7)) == EODD


def test_combine_validation(L):
    f = L.q4mv_combine
    assert f(None, A, A, 2, 1, 8, None) == ENULL
    assert f(A, None, A, 2, 1, 8, None) == ENULL
    assert f(A, A, None, 2, 1, 8, None) == ENULL
    for n_u, nb, out in ((0, 1, 8), (2, 0, 8), (2, 1, 0), (2, 65536, 65536)):
        assert f(A, A, A, n_u, nb, out, None) == ESHAPE
    assert f(A + 2, A, A, 2, 1, 8, None) == EALIGN
    assert f(A, A + 1, A, 2, 1, 8, None) == EALIGN
    assert f(A, A, A + 3, 2, 1, 8, None) == EALIGN


def test_lowbit_validation(L):
    f = L.q4mv_lowbit
    for bits in (2, 3):
        for k in ("w", "s", "b", "xe", "xo", "xsum", "y"):
            assert f(bits, *gemv_args(**{k: None}), 0, None) == ENULL, k
        for kw in (dict(n_mat=0), dict(n_mat=65536), dict(out=0), dict(ind=96), dict(ind=32),
                   dict(nb=0), dict(nb=17)):
            assert f(bits, *gemv_args(**kw), 0, None) == ESHAPE, kw
        for kw in (dict(w=A + 4), dict(xe=A + 8), dict(xo=A + 2), dict(s=A + 1), dict(xsum=A + 2),
                   dict(y=A + 1)):
            assert f(bits, *gemv_args(**kw), 0, None) == EALIGN, kw
        # the matrix-core kernel needs in_dim/64 % 4 == 0 and 8-byte aligned scales/biases
        assert f(bits, *gemv_args(), 3, None) == ESHAPE
        assert f(bits, *gemv_args(ind=256, s=A + 2), 3, None) == ESHAPE
        assert f(bits, *gemv_args(ind=256, b=A + 4), 3, None) == ESHAPE
        assert f(bits, *gemv_args(), 4, None) == EPATH
        assert f(bits, *gemv_args(), -1, None) == EPATH
        assert f(bits, *gemv_args(out=7), 2, None) == EODD
    for bits in (1, 4, 0):
        assert f(bits, *gemv_args(), 0, None) == EVALUE
    g = L.q4mv_pack_lowbit
    assert g(2, None, A, 1, 64, None) == ENULL
    assert g(3, A, None, 1, 64, None) == ENULL
    assert g(4, A, A, 1, 64, None) == EVALUE
    assert g(2, A, A, 0, 64, None) == ESHAPE
    assert g(2, A, A, 1, 96, None) == ESHAPE
    assert g(3, A, A, 1 << 26, 2048, None) == ESHAPE
    assert g(2, A + 8, A, 1, 64, None) == EALIGN
    assert g(3, A, A + 2, 1, 64, None) == EALIGN


def test_fused_validation(L):
    """q4mv_fused: f32 x instead of the prep buffers; the other checks as q4mv_path."""
    def args(**kw):
        a = dict(w=A, s=A, b=A, x=A, y=A, n_mat=1, out=8, ind=128, nb=1, path=0)
        a.update(kw)
        return [a["w"], a["s"], a["b"], a["x"], a["y"], a["n_mat"], a["out"], a["ind"],
                a["nb"], a["path"], None]
    for k in ("w", "s", "b", "x", "y"):
        assert L.q4mv_fused(*args(**{k: None})) == ENULL
    for kw in (dict(n_mat=0), dict(out=0), dict(ind=96), dict(nb=0), dict(nb=17)):
        assert L.q4mv_fused(*args(**kw)) == ESHAPE, kw
    for kw in (dict(w=A + 4), dict(x=A + 8), dict(s=A + 1), dict(y=A + 2)):
        assert L.q4mv_fused(*args(**kw)) == EALIGN, kw
    assert L.q4mv_fused(*args(path=4)) == EPATH
    assert L.q4mv_fused(*args(out=7, path=2)) == EODD


def test_experts_fused_validation(L):
    """q4mv_experts_fused: f32 x (16-byte aligned), swiglu 0 or 1; the rest as q4mv_experts."""
    def args(**kw):
        a = dict(w=A, s=A, b=A, n_bank=4, sel=A, n_sel=2, x=A, y=A, out=8, ind=128, nb=1,
                 shared=1, swiglu=0, path=0)
        a.update(kw)
        return [a["w"], a["s"], a["b"], a["n_bank"], a["sel"], a["n_sel"], a["x"], a["y"],
                a["out"], a["ind"], a["nb"], a["shared"], a["swiglu"], a["path"], None]
    for k in ("w", "s", "b", "sel", "x", "y"):
        assert L.q4mv_experts_fused(*args(**{k: None})) == ENULL
    for kw in (dict(n_bank=0), dict(n_sel=0), dict(n_sel=65536), dict(out=0), dict(ind=96),
               dict(nb=17)):
        assert L.q4mv_experts_fused(*args(**kw)) == ESHAPE, kw
    for kw in (dict(x=A + 8), dict(sel=A + 2), dict(w=A + 4)):
        assert L.q4mv_experts_fused(*args(**kw)) == EALIGN, kw
    assert L.q4mv_experts_fused(*args(swiglu=2)) == EVALUE
    assert L.q4mv_experts_fused(*args(path=5)) == EPATH
    assert L.q4mv_experts_fused(*args(out=7, path=2)) == EODD


PROBE_HEADER = os.path.join(ROOT, "include", "q4mv_probe.h")


@pytest.fixture(scope="module")
def P():
    import ctypes
    path = os.path.join(ROOT, "affine_q4_gemv_amd", "libq4mv_probe.so")
    if not os.path.exists(path):
        from affine_q4_gemv_amd import build
        build.build()
    L = ctypes.CDLL(path)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.q4mv_probe_read.argtypes = [p, i64, p, i32, p]
    L.q4mv_probe_sink_words.argtypes = [i32]
    L.q4mv_probe_sink_words.restype = i64
    L.q4mv_probe_empty.argtypes = [i32, p]
    return L


def test_probe_exports_and_validation(P):
    """The measurement library exports what its header declares and rejects bad arguments
    before launching."""
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q4mv_probe\w*)\s*\(", text, re.M)
    assert sorted(names) == ["q4mv_probe_empty", "q4mv_probe_read", "q4mv_probe_sink_words"]
    for n in names:
        assert hasattr(P, n)
    assert P.q4mv_probe_read(None, 64, A, 2, None) == ENULL
    assert P.q4mv_probe_read(A, 64, None, 2, None) == ENULL
    for nbytes, bpc in ((0, 2), (40, 2), (64, 0), (64, 17)):
        assert P.q4mv_probe_read(A, nbytes, A, bpc, None) == ESHAPE
    assert P.q4mv_probe_read(A + 8, 64, A, 2, None) == EALIGN
    assert P.q4mv_probe_read(A, 64, A + 2, 2, None) == EALIGN
    assert P.q4mv_probe_sink_words(0) == ESHAPE and P.q4mv_probe_sink_words(17) == ESHAPE
    assert P.q4mv_probe_sink_words(2) % 512 == 0
    assert P.q4mv_probe_empty(0, None) == ESHAPE
    assert P.q4mv_probe_empty((1 << 20) + 1, None) == ESHAPE
