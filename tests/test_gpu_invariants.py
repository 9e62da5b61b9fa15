"""GPU invariants and closed forms of the affine-Q4 GEMV, through the C ABI.

* two-row == one-row, bitwise (the two-row helper on the Constant BATCH_MSL page is stated
  to give bit-identical results);
* row r of an nb-batch == the nb = 1 call on that row, bitwise, on the VALU kernels (the
  per-row reduction order does not depend on nb), and n_mat batching == separate launches;
* y(2x) == 2 y(x) bitwise (all scalings are by powers of two);
* nothing is written past y; closed forms hold (exact where the arithmetic is exact).
"""
import numpy as np
import pytest
import torch

import workloads
from q4_gpu import bf16_tensor, flush, parity, run, upload
import affine_q4_gemv_amd as q4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ONE = 0x3F80


@pytest.mark.parametrize("shape", [(8, 2560, 640, 4), (1, 258, 2560, 1), (2, 96, 512, 3),
                                   (1, 64, 2560, 12), (1, 40, 4096, 2)])
def test_two_row_bitwise(shape):
    n_mat, out_dim, in_dim, nb = shape
    d = upload(workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=3))
    flush(f"[2row] {shape}")
    a = run(d, q4.PATH_VALU)
    b = run(d, q4.PATH_VALU_2ROW)
    c = run(d, "2row")
    e = run(d, q4.PATH_AUTO)
    assert torch.equal(a, b)
    assert torch.equal(c, e)


@pytest.mark.parametrize("shape", [(2, 100, 2560, 5), (1, 64, 640, 12), (3, 7, 192, 4)])
def test_batch_rows_bitwise(shape):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=4)
    d = upload(case)
    for path in (q4.PATH_VALU, q4.PATH_VALU_2ROW):
        if path == q4.PATH_VALU_2ROW and out_dim % 2:
            continue
        flush(f"[batch-rows] {shape} path={path}")
        yb = run(d, path)
        for r in range(nb):
            c1 = dict(case)
            c1["x"] = np.ascontiguousarray(case["x"][:, r:r + 1, :])
            y1 = run(upload(c1), path)
            assert torch.equal(yb[:, r, :], y1[:, 0, :]), (path, r)


# (n_mat, out_dim, in_dim, nb): batches whose total tile count crosses the MFMA kernel's
# launch-shape thresholds (256 and 1024 32-row tiles) while one matrix stays below them, so
# a shape choice taken from the batch instead of the matrix would change the bits
BATCHES = [(3, 130, 640, 4), (8, 2560, 2560, 4), (4, 8192, 2560, 4), (5, 6400, 1024, 12)]


@pytest.mark.parametrize("path", [q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
@pytest.mark.parametrize("n_mat,out_dim,in_dim,nb", BATCHES,
                         ids=[f"{m}x{o}x{i}-nb{b}" for m, o, i, b in BATCHES])
def test_matrix_batch_bitwise(path, n_mat, out_dim, in_dim, nb):
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=5 + out_dim)
    d = upload(case)
    flush(f"[batch bitwise] {n_mat}x{out_dim}x{in_dim} nb={nb} path={path}")
    yb = run(d, path)
    for m in range(n_mat):
        c1 = dict(case, codes=case["codes"][m:m + 1], scales=case["scales"][m:m + 1],
                  biases=case["biases"][m:m + 1], x=case["x"][m:m + 1])
        assert torch.equal(yb[m:m + 1], run(upload(c1), path)), m


@pytest.mark.parametrize("path", [q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_power_of_two_scaling(path):
    case = workloads.make_shape(2, 66, 2560, 3, seed=6)
    # keep every f16 operand a normal: for f16 subnormals rounding does not commute with
    # doubling, so y(2x) = 2 y(x) would not hold bit for bit. The MFMA kernel stages odd
    # positions as x/16, which is normal for |x| >= 2^-10.
    x = case["x"]
    tiny = np.abs(x) < 2.0 ** -9
    x[tiny] = np.copysign(np.float32(2.0 ** -9), x[tiny])
    y1 = run(upload(case), path)
    c2 = dict(case, x=case["x"] * np.float32(2.0))
    y2 = run(upload(c2), path)
    assert torch.equal(y2, 2.0 * y1)


@pytest.mark.parametrize("path", [q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_no_write_past_output(path):
    case = workloads.make_shape(2, 34, 640, 5, seed=7)
    d = upload(case)
    n = 2 * 5 * 34
    buf = torch.full((n + 4096,), float("nan"), device="cuda")
    y = run(d, path, y=buf[:n].view(2, 5, 34))
    assert torch.isfinite(y).all()
    assert torch.isnan(buf[n:]).all()


def _closed_case(n_mat, out_dim, in_dim, nb, codes, s_bits, b_bits, x):
    return dict(codes=np.ascontiguousarray(codes, np.uint8),
                scales=np.ascontiguousarray(np.broadcast_to(s_bits, (n_mat, out_dim, in_dim // 64)),
                                            np.uint16),
                biases=np.ascontiguousarray(np.broadcast_to(b_bits, (n_mat, out_dim, in_dim // 64)),
                                            np.uint16),
                x=np.ascontiguousarray(x, np.float32))


@pytest.mark.parametrize("path", [q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_row_sums_exact(path):
    """S = 1, B = 0, x = 1: y is the integer sum of each row's codes, exactly."""
    n_mat, out_dim, in_dim, nb = 2, 70, 2560, 4
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 16, (n_mat, out_dim, in_dim), dtype=np.uint8)
    case = _closed_case(n_mat, out_dim, in_dim, nb, codes, ONE, 0,
                        np.ones((n_mat, nb, in_dim)))
    y = run(upload(case), path).cpu().numpy()
    want = codes.astype(np.int64).sum(axis=2)
    assert np.array_equal(y, np.broadcast_to(want[:, None, :], y.shape).astype(np.float32))


@pytest.mark.parametrize("path", [q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_one_hot_layout(path):
    """A single code 1 at (m, o, i), S = 1, B = 0: y[m][r][o] = x[m][r][i] and every other
    output is 0. Two exact activation probes, (k mod 512) + 1 + 512 r and
    1 + k // 64 + 41 r (both integers <= 2048, so exact in f16), identify the column k
    together; this pins packing, nibble order, row, group and output indexing end to end."""
    n_mat, out_dim, in_dim, nb = 2, 6, 2560, 3
    k = np.arange(in_dim)
    probes = [np.stack([(k % 512) + 1 + 512 * r for r in range(nb)]),
              np.stack([1 + k // 64 + 41 * r for r in range(nb)])]
    rng = np.random.default_rng(9)
    for (m, o, i) in [(0, 0, 0), (1, 5, 2559), (0, 3, 7), (1, 2, 1000)] + \
            [tuple(rng.integers([n_mat, out_dim, in_dim])) for _ in range(4)]:
        codes = np.zeros((n_mat, out_dim, in_dim), np.uint8)
        codes[m, o, i] = 1
        for px in probes:
            x = np.broadcast_to(px.astype(np.float32), (n_mat, nb, in_dim))
            y = run(upload(_closed_case(n_mat, out_dim, in_dim, nb, codes, ONE, 0, x)),
                    path).cpu().numpy()
            want = np.zeros_like(y)
            want[m, :, o] = x[m, :, i]
            assert np.array_equal(y, want), (m, o, i)


@pytest.mark.parametrize("path", [q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_zero_at_mid_code(oracle_lib, path):
    """codes == 8 with B = -8 S: the weight is zero; the GPU result stays within the bound."""
    case = workloads.make_shape(1, 64, 2560, 2, seed=10)
    case["codes"][:] = 8
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    assert np.all(y_ref == 0)
    y = run(upload(case), path).cpu().numpy()
    assert np.all(np.abs(y) <= 2e-3 * bound)
