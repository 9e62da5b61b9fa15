"""q4mv_fused (activation prep done inside the GEMV's staging) against q4mv_prepare_x +
q4mv_path: bitwise equal on every kernel path, and within the tolerance of the oracle."""
import numpy as np
import pytest
import torch

import workloads
from q4_gpu import flush, parity, upload
import affine_q4_gemv_amd as q4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = [q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA]


def check_paths(d, what, out_dim):
    for path in PATHS:
        if path == q4.PATH_VALU_2ROW and out_dim % 2:
            continue
        if path == q4.PATH_MFMA and d["nb"] > 3 and \
                q4.q4mv_auto_path(d["w"].shape[2] * 8, d["nb"], False, out_dim) != q4.PATH_MFMA:
            continue  # the MFMA kernel's LDS does not fit this shape
        flush(f"[fused] {what} path={path}")
        want = q4.q4mv_path(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], path)
        got = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], d["nb"], path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{what} path={path}"
    return got


CASES = [("tiny", 1), ("tiny", 4), ("tiny", 16), ("dense", 1), ("dense", 8), ("moe_down", 4),
         ("up", 1), ("up", 8)]


@pytest.mark.parametrize("name,nb", CASES, ids=[f"{n}-nb{b}" for n, b in CASES])
def test_fused_equals_two_calls(oracle_lib, name, nb):
    case = workloads.make_case(name, nb=nb)
    d = upload(case)
    y = check_paths(d, f"{name} nb={nb}", case["out_dim"])
    y_ref, bound = oracle_lib.gemv(case["codes"], case["scales"], case["biases"], case["x"])
    parity(y.cpu().numpy(), y_ref, bound, f"fused {name} nb={nb}")


# ragged shapes: generic and specialised row lengths, odd out_dim, several matrices, nb past
# 8 (two VALU launches over activation-row ranges), a long launch at nb = 1 (block-loaded
# scales), values that round to f16 subnormals and ties
RAGGED = [(1, 1, 64, 1), (3, 5, 192, 3), (2, 130, 576, 5), (1, 77, 8192, 1), (2, 33, 640, 16),
          (1, 4098, 2560, 9), (1, 40003, 2560, 1), (2, 1100, 1024, 12)]


@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
def test_fused_ragged(shape):
    n_mat, out_dim, in_dim, nb = shape
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=sum(shape) + 5)
    x = case["x"]
    rng = np.random.default_rng(sum(shape))
    x.reshape(-1)[:60] = np.ldexp(rng.random(60), rng.integers(-30, -12, 60)).astype(np.float32)
    x.reshape(-1)[60:64] = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, -(1 + 2.0 ** -11)]
    d = upload(case)
    check_paths(d, str(shape), out_dim)


@pytest.mark.parametrize("nb", [1, 16])
def test_fused_lm_head(nb):
    """The full LM head in the launch configuration the benchmark times."""
    case = workloads.make_case("lm_head", nb=nb)
    d = upload(case)
    flush(f"[fused] lm_head nb={nb}")
    want = q4.q4mv(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], nb)
    got = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], nb)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
