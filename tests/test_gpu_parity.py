"""GPU parity: every kernel path of libq4mv against the CPU oracle, through the C ABI.

Bar (per case): relative L2 error <= 1e-3 over all outputs AND, for every output,
|y_gpu - y_oracle| <= 2e-3 * sum_i(|S q x| + |B x|). Byte work (packing, f16 conversion) is
bit-exact. Full-size cases run the full oracle except the LM head, where sampled rows (first,
last and random ones) are computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from q4_gpu import flush, parity, run, seeds_for, upload
import affine_q4_gemv_amd as q4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = [q4.PATH_AUTO, "2row", q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA]


def paths_for(out_dim):
    return [p for p in PATHS if out_dim % 2 == 0 or p not in ("2row", q4.PATH_VALU_2ROW)]


def test_pack_codes_bit_exact():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(3, 17, 192), dtype=np.uint8)  # high nibbles ignored
    w = q4.q4mv_pack_codes(torch.from_numpy(codes).cuda()).cpu().numpy().view(np.uint32)
    c = (codes & 15).astype(np.uint32).reshape(3, 17, 24, 8)
    want = np.zeros((3, 17, 24), np.uint32)
    for i in range(8):
        want |= c[..., i] << np.uint32(4 * i)
    assert np.array_equal(w, want)


def test_prepare_x(oracle_lib):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 320)).astype(np.float32)
    x[1, :64] = np.ldexp(rng.random(64), rng.integers(-30, -12, 64)).astype(np.float32)
    x[2, :4] = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, -(1 + 2.0 ** -11)]
    xe, xo, xsum = q4.q4mv_prepare_x(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    re_, ro_, rsum = oracle_lib.prepare_x(x)
    assert np.array_equal(xe.cpu().numpy().view(np.uint16), re_.view(np.uint16))
    assert np.array_equal(xo.cpu().numpy().view(np.uint16), ro_.view(np.uint16))
    err = np.abs(xsum.cpu().numpy().astype(np.float64) - rsum)
    assert np.all(err <= oracle_lib.xsum_error_bound(x))
    # overflow to inf is IEEE's, like the oracle's
    big = np.full((1, 64), 70000.0, np.float32)
    be, _, _ = q4.q4mv_prepare_x(torch.from_numpy(big).cuda())
    assert torch.isinf(be.float()).all()


CONFIGS = [("tiny", 1), ("tiny", 4), ("tiny", 8), ("tiny", 16), ("dense", 1), ("dense", 4),
           ("dense", 8), ("moe_down", 4), ("moe_down", 1), ("moe_down", 8), ("up", 8),
           ("up", 1), ("up", 4)]


@pytest.mark.parametrize("name,nb", CONFIGS, ids=[f"{n}-nb{b}" for n, b in CONFIGS])
def test_config_parity(oracle_lib, name, nb):
    case = workloads.make_case(name, nb=nb)
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    d = upload(case)
    for path in paths_for(case["out_dim"]):
        flush(f"[parity] {name} nb={nb} path={path}")
        y = run(d, path).cpu().numpy()
        parity(y, y_ref, bound, f"{name} nb={nb} path={path}")


@pytest.mark.parametrize("nb", [1, 4, 8, 16])
def test_lm_head_sampled(oracle_lib, nb):
    """The LM head at full size in the launch configuration the benchmark times."""
    case = workloads.make_case("lm_head", nb=nb)
    d = upload(case)
    out = case["out_dim"]
    rng = np.random.default_rng(nb)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(out - 128, out),
                                     rng.integers(0, out, 3840)]))
    mats = np.zeros_like(rows)
    y_ref, bound = oracle_lib.gemv_rows(case["codes"], case["scales"], case["biases"],
                                        case["x"], mats, rows)
    paths = [q4.PATH_AUTO, "2row"] + ([q4.PATH_VALU] if nb == 1 else [q4.PATH_MFMA])
    for path in paths:
        flush(f"[parity] lm_head nb={nb} path={path}")
        y = run(d, path)[0].cpu().numpy()          # [nb][out]
        parity(y[:, rows].T, y_ref, bound, f"lm_head nb={nb} path={path}")


RAGGED = [(1, 1, 64, 1), (2, 3, 128, 2), (3, 5, 192, 3), (1, 257, 320, 1), (2, 130, 576, 5),
          (1, 1000, 4096, 2), (1, 77, 8192, 1), (1, 64, 16384, 4), (2, 33, 640, 16),
          (1, 2, 1024, 16), (1, 31, 4096, 16), (3, 18, 448, 7), (1, 4098, 2560, 9),
          (1, 10, 7168, 3),
          # short launches with one quad per wave (rows of 3, 5, 6, 10, 12 quads; the last
          # quad partly filled at 704 and 1216 columns)
          (2, 100, 768, 4), (1, 77, 1280, 8), (1, 45, 1536, 7), (1, 300, 3072, 8),
          (3, 70, 704, 6), (1, 33, 1216, 5), (1, 2600, 2560, 4), (4, 64, 640, 16)]


@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
def test_ragged_shapes(oracle_lib, shape):
    n_mat, out_dim, in_dim, nb = shape
    for k in range(seeds_for(n_mat * nb * out_dim)):
        case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 1000 * k)
        y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
        d = upload(case)
        for path in paths_for(out_dim):
            flush(f"[ragged] {shape} seed {k} path={path}")
            parity(run(d, path).cpu().numpy(), y_ref, bound, f"{shape} seed {k} path={path}",
                   key=f"{shape} path={path}")


# many tiles (the MFMA kernel's 16x16x32 range: at least 1024 tiles, K-split <= 2, nb
# outside 5..8) with ragged row counts, short and long rows, and the 32x32x16 range at nb 6
LARGE = [(1, 40007, 512, 3), (1, 33001, 256, 12), (2, 17000, 1024, 16), (1, 36001, 640, 6),
         (1, 32800, 2560, 1)]


@pytest.mark.parametrize("shape", LARGE, ids=["x".join(map(str, s)) for s in LARGE])
def test_mfma_many_tiles(oracle_lib, shape):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 1)
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    d = upload(case)
    for path in (q4.PATH_MFMA, q4.PATH_AUTO):
        flush(f"[many tiles] {shape} path={path}")
        parity(run(d, path).cpu().numpy(), y_ref, bound, f"{shape} path={path}")


# Long one-row launches at nb = 1 (every wave runs several row steps): the kernel reads a
# step's scales and biases as two contiguous blocks. Ragged row counts make the last step's
# block end inside a 16-byte segment (read element by element up to the array's end).
BLOCK_SCALES = [(1, 40003, 2560, 1), (1, 65537, 512, 1), (1, 16385, 2048, 1)]


@pytest.mark.parametrize("shape", BLOCK_SCALES, ids=["x".join(map(str, s)) for s in BLOCK_SCALES])
def test_block_loaded_scales(oracle_lib, shape):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 2)
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    d = upload(case)
    flush(f"[block scales] {shape}")
    y1 = run(d, q4.PATH_VALU)
    parity(y1.cpu().numpy(), y_ref, bound, f"{shape} one-row")
    # the same values through the per-chunk scale loads: the two-row kernel (bitwise the
    # one-row result) and scale/bias arrays that are only 8-byte aligned
    if out_dim % 2 == 0:
        assert torch.equal(run(d, q4.PATH_VALU_2ROW), y1)
    for name in ("s", "b"):
        t = d[name]
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
        d[name] = buf[4:4 + t.numel()].view(t.shape)
        d[name].copy_(t)
        assert d[name].data_ptr() % 16 == 8
    flush(f"[block scales] {shape} 8-byte aligned scales")
    assert torch.equal(run(d, q4.PATH_VALU), y1)


# Small activations: the MFMA kernel stages activations as 16 x and x (exact in f16), so its
# error stays that of the f16 activation format itself, like the VALU kernels'. Few and many
# tiles (32x32x16 and 16x16x32 matrix-core shapes).
SMALL_X = [(1, 2560, 2560, 4), (1, 512, 2560, 16), (1, 40000, 512, 4)]


@pytest.mark.parametrize("x_scale", [1e-3, 1e-4])
@pytest.mark.parametrize("shape", SMALL_X, ids=["x".join(map(str, s)) for s in SMALL_X])
def test_small_activations(oracle_lib, shape, x_scale):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 3, x_scale=x_scale)
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    d = upload(case)
    for path in (q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_MFMA):
        flush(f"[small x] {shape} x_scale={x_scale} path={path}")
        parity(run(d, path).cpu().numpy(), y_ref, bound, f"{shape} x{x_scale} path={path}")


# Activations of 4096 or more: 16 x would overflow f16, so the MFMA kernel stages those rows'
# block with x and x/16 instead (output scale 2^24); rows just below stay on the x16 staging.
@pytest.mark.parametrize("peak", [4094.0, 4096.0, 6.0e4])
def test_large_activations(oracle_lib, peak):
    n_mat, out_dim, in_dim, nb = 2, 300, 1024, 4
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=int(peak) % 97)
    case["x"][1, 2, 77] = peak          # an even column of matrix 1
    case["x"][0, 0, 513] = -peak / 2    # an odd column of matrix 0
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    d = upload(case)
    for path in (q4.PATH_VALU, q4.PATH_MFMA):
        flush(f"[large x] peak={peak} path={path}")
        y = run(d, path)
        parity(y.cpu().numpy(), y_ref, bound, f"peak {peak} path={path}")
        fused = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], nb, path)
        torch.cuda.synchronize()
        assert torch.equal(fused, y), f"peak {peak} path={path}: fused differs"
