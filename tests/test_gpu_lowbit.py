"""GPU parity of the Q2 / Q3 low-bit variants (fn_q2_rows_h, fn_q3_rows_h on the Constant
BATCH_MSL page) through the C ABI: the packed layout bit for bit against the oracle's packer,
and q4mv_lowbit against the oracle's midpoint-reconstruction GEMV on every path (the VALU
kernels, and the MFMA kernel where in_dim/64 is a multiple of 4), at the workload shapes,
ragged shapes, and the full LM head on sampled rows."""
import numpy as np
import pytest
import torch

import affine_q4_gemv_amd as q4
import workloads
from q4_gpu import bf16_tensor, dev, flush, parity, seeds_for

pytestmark = pytest.mark.gpu


def upload_lowbit(case, bits):
    codes = torch.from_numpy(case["codes"]).to(dev())
    w = q4.q4mv_pack_lowbit(bits, codes)
    del codes
    n_mat, nb, in_dim = case["x"].shape
    x = torch.from_numpy(case["x"].reshape(n_mat * nb, in_dim)).to(dev())
    xe, xo, xsum = q4.q4mv_prepare_x(x)
    return dict(w=w, s=bf16_tensor(case["scales"]), b=bf16_tensor(case["biases"]), xe=xe,
                xo=xo, xsum=xsum, nb=nb)


def mfma_ok(in_dim, nb, out_dim):
    """Whether q4mv_lowbit accepts path 3 for the shape (groups per row a multiple of 4; long
    rows run as K slices)."""
    return (in_dim // 64) % 4 == 0


def run(d, bits, path):
    y = q4.q4mv_lowbit(bits, d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"],
                       path=path)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("rows,in_dim", [(3, 640), (2, 2560), (5, 64), (1, 4160)])
def test_pack_lowbit_bitexact(oracle_lib, bits, rows, in_dim):
    rng = np.random.default_rng(rows * in_dim + bits)
    codes = rng.integers(0, 256, (rows, in_dim), dtype=np.uint8)  # high bits must be ignored
    flush(f"[pack lowbit] bits={bits} {rows}x{in_dim}")
    w = q4.q4mv_pack_lowbit(bits, torch.from_numpy(codes).to(dev())).cpu().numpy()
    assert np.array_equal(w.view(np.uint32), oracle_lib.pack_lowbit(bits, codes))


CASES = [("tiny", 1), ("tiny", 4), ("tiny", 16), ("dense", 1), ("dense", 2), ("moe_down", 4),
         ("moe_down", 2), ("up", 1), ("up", 8)]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("name,nb", CASES, ids=[f"{n}-nb{b}" for n, b in CASES])
def test_lowbit_parity(oracle_lib, bits, name, nb):
    case = workloads.make_case(name, nb=nb)
    y_ref, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"], case["biases"],
                                          case["x"])
    d = upload_lowbit(case, bits)
    paths = [1, 2] if case["out_dim"] % 2 == 0 else [1]
    ys = {}
    for path in paths + [0]:
        flush(f"[lowbit] bits={bits} {name} nb={nb} path={path}")
        ys[path] = run(d, bits, path)
        parity(ys[path].cpu().numpy(), y_ref, bound, f"Q{bits} {name} nb={nb} path={path}")
    for path in paths[1:]:
        assert torch.equal(ys[path], ys[1]), f"path {path} differs bitwise from path 1"
    auto_mfma = nb > 3 and mfma_ok(case["in_dim"], nb, case["out_dim"])
    if mfma_ok(case["in_dim"], nb, case["out_dim"]):
        flush(f"[lowbit] bits={bits} {name} nb={nb} path=3")
        ys[3] = run(d, bits, 3)
        parity(ys[3].cpu().numpy(), y_ref, bound, f"Q{bits} {name} nb={nb} MFMA")
    # the automatic choice is bitwise the path it takes (MFMA from nb = 4 where it fits)
    assert torch.equal(ys[0], ys[3] if auto_mfma else ys[1]), "automatic path"



RAGGED = [(1, 1, 64, 1), (1, 77, 192, 3), (2, 33, 4160, 2), (1, 130, 640, 16),
          (3, 64, 2560, 5), (2, 45, 1024, 7), (1, 1000, 256, 16), (1, 3, 512, 4),
          (1, 40003, 512, 12)]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n_mat,out_dim,in_dim,nb", RAGGED,
                         ids=[f"{m}x{o}x{i}-nb{b}" for m, o, i, b in RAGGED])
def test_lowbit_ragged(oracle_lib, bits, n_mat, out_dim, in_dim, nb):
    paths = [1, 2] if out_dim % 2 == 0 else [1]
    if mfma_ok(in_dim, nb, out_dim):
        paths.append(3)
    for k in range(seeds_for(n_mat * nb * out_dim)):
        case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=90 + out_dim + 1000 * k)
        y_ref, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"],
                                              case["biases"], case["x"])
        d = upload_lowbit(case, bits)
        for path in paths:
            flush(f"[lowbit ragged] bits={bits} {n_mat}x{out_dim}x{in_dim} nb={nb} seed {k} "
                  f"path={path}")
            parity(run(d, bits, path).cpu().numpy(), y_ref, bound, f"Q{bits} seed {k} path {path}",
                   key=f"Q{bits} path {path}")


@pytest.mark.parametrize("bits", [2, 3])
def test_lowbit_lm_head_sampled(oracle_lib, bits):
    """The full LM head (151936 x 2560) at NB=1 in the automatic launch, checked on 768
    sampled rows: the first and last 128 and 512 random ones."""
    case = workloads.make_case("lm_head", nb=1)
    out_dim = case["out_dim"]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(out_dim - 128, out_dim),
                                     rng.integers(0, out_dim, 512)]))
    flush(f"[lowbit lm_head] bits={bits}")
    d = upload_lowbit(case, bits)
    y = run(d, bits, 0).cpu().numpy()
    y_ref, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"], case["biases"],
                                          case["x"], rows=rows)
    parity(y[:, :, rows], y_ref, bound, f"Q{bits} lm_head sampled")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("nb", [4, 16])
def test_lowbit_lm_head_mfma(oracle_lib, bits, nb):
    """The full LM head on the MFMA kernel (16x16x32, K-split 2), 768 sampled rows."""
    case = workloads.make_case("lm_head", nb=nb)
    out_dim = case["out_dim"]
    rng = np.random.default_rng(6 + nb)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(out_dim - 128, out_dim),
                                     rng.integers(0, out_dim, 512)]))
    flush(f"[lowbit lm_head mfma] bits={bits} nb={nb}")
    d = upload_lowbit(case, bits)
    y = run(d, bits, 3).cpu().numpy()
    y_ref, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"], case["biases"],
                                          case["x"], rows=rows)
    parity(y[:, :, rows], y_ref, bound, f"Q{bits} lm_head nb={nb} MFMA")
