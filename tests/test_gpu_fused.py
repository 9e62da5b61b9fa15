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
        flush(f"[fused] {what} path={path}")
        want = q4.q4mv_path(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], path)
        got = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], d["nb"], path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{what} path={path}"
    return got


# dense and up at NB 16: more activation words per thread than the short-launch kernels
# load ahead of the weight loads (the rest are staged in rounds after them)
CASES = [("tiny", 1), ("tiny", 4), ("tiny", 16), ("dense", 1), ("dense", 8), ("dense", 16),
         ("moe_down", 4), ("up", 1), ("up", 8), ("up", 16)]


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
def test_fused_lm_head(oracle_lib, nb):
    """The full LM head in the launch configuration the benchmark times: bitwise the
    two-call result, and within the tolerance of the oracle on sampled rows (the first and
    last 128 and random ones, computed one by one)."""
    case = workloads.make_case("lm_head", nb=nb)
    d = upload(case)
    flush(f"[fused] lm_head nb={nb}")
    want = q4.q4mv(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], nb)
    got = q4.q4mv_fused(d["w"], d["s"], d["b"], d["x"], nb)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    out = case["out_dim"]
    rng = np.random.default_rng(100 + nb)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(out - 128, out),
                                     rng.integers(0, out, 1792)]))
    y_ref, bound = oracle_lib.gemv_rows(case["codes"], case["scales"], case["biases"],
                                        case["x"], np.zeros_like(rows), rows)
    parity(got[0].cpu().numpy()[:, rows].T, y_ref, bound, f"fused lm_head nb={nb}")


# ---- routed experts with the prep (and the SwiGLU of the expert MLP) inside the launch

def same_bits(a, b):
    """Equal bit patterns (NaN rows of out-of-bank ids compare equal too)."""
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def expert_bank(n_bank, out_dim, in_dim, seed):
    case = workloads.make_shape(n_bank, out_dim, in_dim, 1, seed=seed)
    d = upload(case)
    return d["w"], d["s"], d["b"]


# (n_bank, out_dim, in_dim, nb, sel): the MoE gate/up and down shapes, odd rows, the MFMA
# range, repeated and unordered ids and one outside the bank (NaN rows); the down shape at
# NB 8 stages more [gate | up] words per thread than its kernel loads ahead
EXPERTS = [(6, 1280, 2560, 4, [5, 1, 1, 0, 3]), (6, 2560, 640, 4, [2, 4, 0, 9]),
           (6, 2560, 640, 8, [1, 5, 3]), (3, 77, 256, 1, [2, 0, 2, 1]),
           (4, 96, 512, 16, [3, 3, 0])]
EXP_PATHS = [q4.PATH_AUTO, q4.PATH_VALU, q4.PATH_MFMA, q4.PATH_VALU_2ROW]


@pytest.mark.parametrize("case", EXPERTS, ids=[f"{c[0]}x{c[1]}x{c[2]}-nb{c[3]}" for c in EXPERTS])
def test_experts_fused_equals_two_calls(case):
    n_bank, out_dim, in_dim, nb, sel = case
    w, s, b = expert_bank(n_bank, out_dim, in_dim, seed=60 + nb)
    sel_d = torch.tensor(sel, dtype=torch.int32, device="cuda")
    n_sel = len(sel)
    rng = np.random.default_rng(nb)
    for shared in (True, False):
        rows = nb if shared else n_sel * nb
        x = torch.from_numpy(rng.standard_normal((rows, in_dim)).astype(np.float32)).cuda()
        xe, xo, xsum = q4.q4mv_prepare_x(x)
        # gate|up rows of the same slots for the SwiGLU form
        gu = torch.from_numpy(
            (2 * rng.standard_normal((rows, 2 * in_dim))).astype(np.float32)).cuda()
        he, ho, hsum = q4.q4mv_swiglu_prep(gu)
        for path in EXP_PATHS:
            if path == q4.PATH_VALU_2ROW and out_dim % 2:
                continue
            flush(f"[experts fused] {case} shared={shared} path={path}")
            want = q4.q4mv_experts(w, s, b, sel_d, xe, xo, xsum, nb, shared, path)
            got = q4.q4mv_experts_fused(w, s, b, sel_d, x, nb, shared, False, path)
            want_g = q4.q4mv_experts(w, s, b, sel_d, he, ho, hsum, nb, shared, path)
            got_g = q4.q4mv_experts_fused(w, s, b, sel_d, gu, nb, shared, True, path)
            torch.cuda.synchronize()
            assert same_bits(got, want), f"{case} shared={shared} path={path}"
            assert same_bits(got_g, want_g), f"{case} swiglu shared={shared} path={path}"


def test_moe_layer_fused_equals_five_launches():
    """The decode MoE layer (4 tokens, top-8 of 32 experts, hidden 2560, intermediate 640)
    in three launches -- gate|up over the routed experts from the f32 token rows, the down
    projection with the SwiGLU in its staging, the combine -- bitwise equal to the five-launch
    chain (prep, gate|up, SwiGLU prep, down, combine) that the oracle chain checks."""
    n_exp, hidden, inter, nb, top_k = 32, 2560, 640, 4, 8
    sel, wmap = workloads.make_routing(nb, n_exp, top_k, seed=71)
    n_u = sel.size
    gu_bank = workloads.make_shape(n_exp, 2 * inter, hidden, nb, seed=72)
    dn_bank = workloads.make_weights(n_exp, hidden, inter, seed=73)
    d1 = upload(gu_bank)
    w1, s1, b1 = d1["w"], d1["s"], d1["b"]
    w2 = q4.q4mv_pack_codes(torch.from_numpy(dn_bank[0]).cuda())
    from q4_gpu import bf16_tensor
    s2, b2 = bf16_tensor(dn_bank[1]), bf16_tensor(dn_bank[2])
    sel_d, wmap_d = torch.from_numpy(sel).cuda(), torch.from_numpy(wmap).cuda()
    x = torch.from_numpy(np.ascontiguousarray(gu_bank["x"][0])).cuda()
    flush(f"[moe layer fused] {n_u} routed experts of {n_exp}")
    xe, xo, xsum = q4.q4mv_prepare_x(x)
    gu = q4.q4mv_experts(w1, s1, b1, sel_d, xe, xo, xsum, nb, True)
    xe2, xo2, xsum2 = q4.q4mv_swiglu_prep(gu.view(n_u * nb, 2 * inter))
    y = q4.q4mv_experts(w2, s2, b2, sel_d, xe2, xo2, xsum2, nb, False)
    out = q4.q4mv_combine(y, wmap_d)
    gu_f = q4.q4mv_experts_fused(w1, s1, b1, sel_d, x, nb, True)
    y_f = q4.q4mv_experts_fused(w2, s2, b2, sel_d, gu_f.view(n_u * nb, 2 * inter), nb, False,
                                swiglu=True)
    out_f = q4.q4mv_combine(y_f, wmap_d)
    torch.cuda.synchronize()
    assert torch.equal(gu_f, gu) and torch.equal(y_f, y) and torch.equal(out_f, out)


def test_fused_graph_replays():
    """q4mv_fused and the fused expert chain captured in a HIP graph: every replay (with
    eager work and synchronisations between them, and new inputs copied in) equals the eager
    result bit for bit."""
    case = workloads.make_shape(2, 1000, 2560, 4, seed=91)
    d = upload(case)
    n_mat, nb = 2, 4
    y = torch.empty((n_mat, nb, 1000), dtype=torch.float32, device="cuda")
    sel = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    gu = torch.empty((n_mat * nb, 2 * 2560), dtype=torch.float32, device="cuda")
    ye = torch.empty((2, nb, 1000), dtype=torch.float32, device="cuda")
    x_in = d["x"].clone()
    gu_in = torch.randn(n_mat * nb, 2 * 2560, device="cuda")

    def body():
        q4.q4mv_fused(d["w"], d["s"], d["b"], x_in, nb, y=y)
        q4.q4mv_experts_fused(d["w"], d["s"], d["b"], sel, gu, nb, False, swiglu=True, y=ye)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gu.copy_(gu_in)
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    rng = np.random.default_rng(5)
    for rep in range(3):
        x_in.copy_(torch.from_numpy(rng.standard_normal(tuple(x_in.shape)).astype(np.float32)))
        gu.copy_(torch.from_numpy(rng.standard_normal(tuple(gu.shape)).astype(np.float32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_y, got_ye = y.clone(), ye.clone()
        flush(f"[fused graph] replay {rep}")
        want_y = q4.q4mv_fused(d["w"], d["s"], d["b"], x_in, nb)
        want_ye = q4.q4mv_experts_fused(d["w"], d["s"], d["b"], sel, gu, nb, False, swiglu=True)
        torch.cuda.synchronize()
        assert torch.equal(got_y, want_y) and torch.equal(got_ye, want_ye), f"replay {rep}"


# Pair sums of f16 values that fall on f32 rounding ties (2048 + 2^-13 rounds down to even,
# 2048 + 3 * 2^-13 up; the same at 4096, which also takes the MFMA kernel's fallback
# staging) and signed zeros (-0 + -0 = -0): the fused staging's sums against the prep's.
@pytest.mark.parametrize("big", [False, True], ids=["x16-staging", "fallback-staging"])
def test_fused_pair_sum_ties(oracle_lib, big):
    n_mat, out_dim, in_dim, nb = 1, 96, 512, 4
    case = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=123)
    x = case["x"].reshape(-1)
    a = 4096.0 if big else 2048.0
    ulp = a * 2.0 ** -23
    pairs = [(a, ulp / 2), (a, 1.5 * ulp), (-a, -ulp / 2), (-a, -1.5 * ulp), (-0.0, -0.0),
             (0.0, -0.0), (-0.0, 0.0), (ulp / 2, a)]
    for k, (p, q) in enumerate(pairs):
        for rep in range(4):  # several rows and chunks
            at = 2 * k + 130 * rep * 4
            x[at], x[at + 1] = p, q
    x[256:288] = -0.0  # a whole chunk of negative zeros
    d = upload(case)
    check_paths(d, f"pair-sum ties big={big}", out_dim)
    # an all-negative-zero chunk sums to -0 in the prep
    xs = d["xsum"].cpu().numpy()
    assert np.signbit(xs[0, 256 // 32]) and xs[0, 256 // 32] == 0.0
