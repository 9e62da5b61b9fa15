"""GPU parity of the fused epilogues of the Constant BATCH_MSL page, through the C ABI:
fn_qmv_silu_b's silu(y / div) store (q4mv_silu), fn_moe_act_b's SwiGLU activation fused with
the down projection's prep (q4mv_swiglu_prep), and the expert MLP chain they serve
(stacked gate/up GEMV -> SwiGLU prep -> down GEMV), each against the oracle."""
import numpy as np
import pytest
import torch

import affine_q4_gemv_amd as q4
import workloads
from q4_gpu import ELEM, REL_L2, bf16_tensor, dev, flush, upload

pytestmark = pytest.mark.gpu

# the epilogue itself is one f32 division and one single-precision exp (a few ulp): relative
EPI_REL = 1e-6


def check(y_gpu, y_ref, budget, rel_tol, what):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    err = np.abs(y_gpu - y_ref)
    rel = np.linalg.norm(err) / max(np.linalg.norm(y_ref), 1e-300)
    ratio = np.max(err / (budget + 1e-30))
    assert rel <= rel_tol, f"{what}: relative L2 error {rel:.3e} > {rel_tol}"
    assert ratio <= 1.0, f"{what}: per-element error {ratio:.3f}x the budget"
    return rel


SILU = [("tiny", 1, 1.0), ("tiny", 4, -3.0), ("tiny", 16, 2.5), ("dense", 1, 4.0),
        ("moe_down", 4, 0.5), ("up", 8, 1.7)]


@pytest.mark.parametrize("name,nb,div", SILU, ids=[f"{n}-nb{b}-div{d}" for n, b, d in SILU])
def test_silu_parity(oracle_lib, name, nb, div):
    case = workloads.make_case(name, nb=nb)
    y_ref, bound = oracle_lib.gemv_silu(case["codes"], case["scales"], case["biases"], case["x"],
                                        div)
    budget = ELEM * bound + EPI_REL * np.abs(y_ref)
    d = upload(case)
    args = (d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], div)
    paths = [q4.PATH_VALU, q4.PATH_MFMA] + ([q4.PATH_VALU_2ROW] if case["out_dim"] % 2 == 0 else [])
    for path in paths:
        flush(f"[silu] {name} nb={nb} div={div} path={path}")
        y = q4.q4mv_path_silu(*args, path).cpu().numpy()
        check(y, y_ref, budget, REL_L2, f"{name} nb={nb} path={path}")
    y = q4.q4mv_silu(*args).cpu().numpy()
    check(y, y_ref, budget, REL_L2, f"{name} nb={nb} auto")


def f16_interleave(xe, xo):
    e = xe.cpu().numpy().astype(np.float64)
    o = xo.cpu().numpy().astype(np.float64)
    h = np.empty((e.shape[0], 2 * e.shape[1]))
    h[:, 0::2] = e
    h[:, 1::2] = o
    return h


@pytest.mark.parametrize("n_rows,inter", [(5, 640), (32, 1024), (1, 64)])
def test_swiglu_prep(oracle_lib, n_rows, inter):
    rng = np.random.default_rng(n_rows * 7 + inter)
    gu = np.concatenate([rng.normal(0, 2, (n_rows, inter)), rng.normal(0, 1, (n_rows, inter))],
                        axis=1).astype(np.float32)
    gu[0, :8] = [-80, -20, -1, 0, 1e-8, 3, 20, 80]  # saturated and tiny gates
    flush(f"[swiglu] rows={n_rows} inter={inter}")
    xe, xo, xsum = q4.q4mv_swiglu_prep(torch.from_numpy(gu).to(dev()))
    torch.cuda.synchronize()
    h_dev = f16_interleave(xe, xo)
    h_ref = oracle_lib.swiglu(gu.astype(np.float64))
    # each value is one f16 rounding (half an ulp, <= 2^-11 relative, or 2^-25 among
    # subnormals) of an f32 result within a few ulp of the exact value
    assert np.all(np.abs(h_dev - h_ref) <= 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24)
    # the chunk sums are f32 sums of the device's own f16 values
    s_dev = xsum.cpu().numpy().astype(np.float64)
    s_own = h_dev.reshape(n_rows, inter // 32, 32).sum(axis=2)
    a_own = np.abs(h_dev).reshape(n_rows, inter // 32, 32).sum(axis=2)
    assert np.all(np.abs(s_dev - s_own) <= 31 * 2.0 ** -24 * a_own)


def test_moe_mlp_chain(oracle_lib):
    """8 experts, hidden 2560, intermediate 640, 4 token rows per expert: the stacked
    gate|up GEMV (fn_moe_gate_up_b's [u*NB+b][2*inter] output is q4mv's y layout), the fused
    SwiGLU prep, then the down GEMV (the MoE down projection workload)."""
    n_mat, hidden, inter, nb = 8, 2560, 640, 4
    up = workloads.make_shape(n_mat, 2 * inter, hidden, nb, seed=21)
    dn = workloads.make_shape(n_mat, hidden, inter, nb, seed=22, x_scale=0.5)
    d1 = upload(up)
    flush("[moe chain] gate/up GEMV")
    gu = q4.q4mv(d1["w"], d1["s"], d1["b"], d1["xe"], d1["xo"], d1["xsum"], nb)
    xe2, xo2, xsum2 = q4.q4mv_swiglu_prep(gu.view(n_mat * nb, 2 * inter))
    w2 = q4.q4mv_pack_codes(torch.from_numpy(dn["codes"]).to(dev()))
    s2, b2 = bf16_tensor(dn["scales"]), bf16_tensor(dn["biases"])
    flush("[moe chain] down GEMV")
    y = q4.q4mv(w2, s2, b2, xe2, xo2, xsum2, nb).cpu().numpy()

    g_ref, g_bound = oracle_lib.gemv(up["codes"], up["scales"], up["biases"], up["x"])
    g_ref = g_ref.reshape(n_mat * nb, 2 * inter)
    g_bound = g_bound.reshape(n_mat * nb, 2 * inter)
    h_ref = oracle_lib.swiglu(g_ref)
    # the down projection's input as the device holds it: f16-rounded h
    x_dn = h_ref.astype(np.float32).astype(np.float16).astype(np.float32)
    y_ref, bound = oracle_lib.gemv(dn["codes"], dn["scales"], dn["biases"],
                                   x_dn.reshape(n_mat, nb, inter))
    # error budget: the down GEMV's own, plus what its input may differ by. The gate/up GEMV
    # is within ELEM * bound of the oracle; silu moves that by at most 1.1x (times |up|), up
    # is multiplied by |silu(gate)|; then f32 arithmetic and the f16 rounding on both sides.
    g, u = g_ref[:, :inter], g_ref[:, inter:]
    eg, eu = ELEM * g_bound[:, :inter], ELEM * g_bound[:, inter:]
    e = (oracle_lib.SILU_LIPSCHITZ * eg * (np.abs(u) + eu) + np.abs(oracle_lib.silu(g)) * eu
         + 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24)
    # sum_i |W[o][i]| e_i <= sum_i (|S| q + |B|) e_i: the oracle GEMV with |S|, |B| and x = e
    absS, absB = dn["scales"] & 0x7FFF, dn["biases"] & 0x7FFF
    prop, _ = oracle_lib.gemv(dn["codes"], absS, absB,
                              e.astype(np.float32).reshape(n_mat, nb, inter))
    budget = ELEM * bound + prop
    # relative L2: gate/up 1e-3, through silu (<= 1.1x) and the f16 rounding (<= 4.9e-4),
    # plus the down GEMV's 1e-3
    rel = check(y, y_ref, budget, 3e-3, "moe chain")
    flush(f"[moe chain] relative L2 {rel:.2e}")
