"""Rows whose staged activations do not fit in LDS: the product runs as K slices (one launch
per slice, each later slice adding to y, the epilogue with the last), on every kernel path,
through the C ABI. Checked against the oracle at the 9728-wide down projection that pairs
with the 9728 x 2560 up projection (NB 8 and 16), an 8192-wide row at NB 16, ragged and very
long rows; and bitwise between the fused and the two-call forms, which slice alike."""
import numpy as np
import pytest
import torch

import affine_q4_gemv_amd as q4
import workloads
from q4_gpu import ELEM, REL_L2, bf16_tensor, dev, flush, parity, seeds_for, upload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = [q4.PATH_AUTO, "2row", q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA]

# (n_mat, out_dim, in_dim, nb): nb * in_dim beyond what one LDS staging holds on every path
# (the VALU kernels stage up to 8 rows, about 75000 values; the MFMA kernel fewer), slice
# boundaries on 512-, 256- and 64-column multiples, ragged out_dim (a shifted last MFMA tile
# whose overlap must not be added twice), several matrices
SHAPES = [(1, 2560, 9728, 8), (1, 2560, 9728, 16), (1, 512, 8192, 16), (2, 45, 4160, 16),
          (1, 9, 80000, 1), (1, 70, 80000, 3), (1, 33, 20736, 5), (3, 40, 12288, 12)]


def run(d, path, y=None):
    if path == "2row":
        out = q4.q4mv_2row(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], y=y)
    elif path == q4.PATH_AUTO:
        out = q4.q4mv(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], y=y)
    else:
        out = q4.q4mv_path(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], path,
                           y=y)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_kslice_parity(oracle_lib, shape):
    n_mat, out_dim, in_dim, nb = shape
    for k in range(seeds_for(n_mat * nb * out_dim)):
        case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 11 + 1000 * k)
        y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
        d = upload(case)
        ys = {}
        for path in PATHS:
            if out_dim % 2 and path in ("2row", q4.PATH_VALU_2ROW):
                continue
            flush(f"[kslice] {shape} seed {k} path={path}")
            # y starts as garbage: the first slice must overwrite it, not add to it
            y0 = torch.full((n_mat, nb, out_dim), 1e30, dtype=torch.float32, device=dev())
            ys[path] = run(d, path, y=y0)
            parity(ys[path].cpu().numpy(), y_ref, bound, f"{shape} seed {k} path={path}",
                   key=f"{shape} path={path}")
    # the two VALU kernels slice alike and stay bitwise equal; q4mv_2row follows q4mv
    if out_dim % 2 == 0:
        assert torch.equal(ys[q4.PATH_VALU], ys[q4.PATH_VALU_2ROW])
        assert torch.equal(ys[q4.PATH_AUTO], ys["2row"])
    auto = q4.q4mv_auto_path(in_dim, nb, False, out_dim)
    assert torch.equal(ys[q4.PATH_AUTO], ys[auto])


@pytest.mark.parametrize("shape", SHAPES[:4], ids=["x".join(map(str, s)) for s in SHAPES[:4]])
def test_kslice_fused_equals_two_calls(shape):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 12)
    d = upload(case)
    for path in (q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_MFMA):
        flush(f"[kslice fused] {shape} path={path}")
        want = q4.q4mv_path(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], nb, path)
        got = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], nb, path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{shape} path={path}"


def test_kslice_silu(oracle_lib):
    """The silu(y / div) epilogue applies once, to the sum of every slice."""
    shape = (1, 300, 9728, 8)
    case = workloads.make_shape(*shape, seed=77)
    div = 1.5
    y_ref, bound = oracle_lib.gemv_silu(case["codes"], case["scales"], case["biases"],
                                        case["x"], div)
    budget = ELEM * bound + 1e-6 * np.abs(y_ref)
    d = upload(case)
    for path in (q4.PATH_VALU, q4.PATH_MFMA):
        flush(f"[kslice silu] {shape} path={path}")
        y = q4.q4mv_path_silu(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], 8, div, path)
        y = y.cpu().numpy().astype(np.float64)
        err = np.abs(y - y_ref)
        assert np.linalg.norm(err) / np.linalg.norm(y_ref) <= REL_L2
        assert np.all(err <= budget), f"path {path}: {np.max(err / budget):.3f}x the budget"


def test_kslice_experts_swiglu():
    """Routed experts with a down projection whose intermediate rows do not fit: the SwiGLU
    of [gate | up] rows read at the slice's columns of both halves, bitwise what
    q4mv_swiglu_prep + q4mv_experts give."""
    n_bank, out_dim, inter, nb = 3, 96, 9728, 8
    case = workloads.make_shape(n_bank, out_dim, inter, 1, seed=78)
    d = upload(case)
    sel = torch.tensor([2, 0, 2], dtype=torch.int32, device=dev())
    rng = np.random.default_rng(79)
    gu = torch.from_numpy((2 * rng.standard_normal((3 * nb, 2 * inter))).astype(np.float32)).to(dev())
    he, ho, hsum = q4.q4mv_swiglu_prep(gu)
    for path in (q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_MFMA):
        flush(f"[kslice experts] path={path}")
        want = q4.q4mv_experts(d["w"], d["s"], d["b"], sel, he, ho, hsum, nb, False, path)
        got = q4.q4mv_experts_fused(d["w"], d["s"], d["b"], sel, gu, nb, False, True, path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"path={path}"
        # slot 0 is what q4mv gives for its matrix (bank matrix 2) and rows
        one = q4.q4mv_path(d["w"][2:3].contiguous(), d["s"][2:3].contiguous(),
                           d["b"][2:3].contiguous(), he[:nb].contiguous(), ho[:nb].contiguous(),
                           hsum[:nb].contiguous(), nb, path)
        torch.cuda.synchronize()
        assert torch.equal(want[0], one[0]), f"path={path}"


@pytest.mark.parametrize("bits", [2, 3])
def test_kslice_lowbit(oracle_lib, bits):
    shape = (1, 96, 16384, 8)
    case = workloads.make_shape(*shape, seed=80 + bits)
    y_ref, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"], case["biases"],
                                          case["x"])
    w = q4.q4mv_pack_lowbit(bits, torch.from_numpy(case["codes"]).to(dev()))
    x = torch.from_numpy(case["x"].reshape(8, shape[2])).to(dev())
    xe, xo, xsum = q4.q4mv_prepare_x(x)
    s, b = bf16_tensor(case["scales"]), bf16_tensor(case["biases"])
    for path in (0, 1, 2, 3):
        flush(f"[kslice lowbit] bits={bits} path={path}")
        y = q4.q4mv_lowbit(bits, w, s, b, xe, xo, xsum, 8, path=path)
        torch.cuda.synchronize()
        parity(y.cpu().numpy(), y_ref, bound, f"Q{bits} path={path}")
