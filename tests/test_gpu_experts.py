"""GPU parity of the selected-expert dispatch through the C ABI: q4mv_experts (a bank of
matrices, a device array of expert ids, shared or per-slot activation rows; the selected-expert
launch of the memra-engine qwen4exp_gpu.rs page and the unique-expert loop of the Constant
BATCH_MSL page) and q4mv_combine (the routing-weighted expert sum), up to a whole MoE layer:
gate/up over the routed experts, SwiGLU prep, down projection, combine."""
import numpy as np
import pytest
import torch

import affine_q4_gemv_amd as q4
import workloads
from q4_gpu import ELEM, REL_L2, bf16_tensor, dev, flush, parity, upload

pytestmark = pytest.mark.gpu

U = 2.0 ** -24  # f32 unit roundoff


def paths_for(out_dim):
    """Every kernel (the MFMA kernel's LDS fits all shapes here), two-row for even out_dim."""
    return [q4.PATH_VALU, q4.PATH_MFMA] + ([q4.PATH_VALU_2ROW] if out_dim % 2 == 0 else [])


def put_bank(case):
    d = upload(case)
    return d["w"], d["s"], d["b"]


def prep_rows(x):
    """x f32 [rows][in] (numpy) -> device prep through the library."""
    return q4.q4mv_prepare_x(torch.from_numpy(np.ascontiguousarray(x)).to(dev()))


# (n_bank, out_dim, in_dim, nb, sel): the MoE gate/up and down shapes, an odd row count, the
# MFMA range, repeats and any order in sel
EXPERT_CASES = [
    (6, 1280, 2560, 4, [5, 1, 1, 0, 3]),
    (6, 2560, 640, 4, [2, 4, 0]),
    (3, 77, 256, 1, [2, 0, 2, 1]),
    (4, 96, 512, 16, [3, 3, 0]),
    (2, 40, 64, 2, [1]),
]


@pytest.mark.parametrize("n_bank,out_dim,in_dim,nb,sel", EXPERT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-nb{c[3]}" for c in EXPERT_CASES])
@pytest.mark.parametrize("shared", [False, True], ids=["per-slot", "shared"])
def test_experts_equal_q4mv_and_oracle(oracle_lib, n_bank, out_dim, in_dim, nb, sel, shared):
    case = workloads.make_shape(n_bank, out_dim, in_dim, nb, seed=40 + n_bank + nb)
    w, s, b = put_bank(case)
    sel_np = np.array(sel, dtype=np.int32)
    n_sel = sel_np.size
    sel_d = torch.from_numpy(sel_np).to(dev())
    xrows = workloads.make_x(1 if shared else n_sel, nb, in_dim, seed=50 + nb)
    xe, xo, xsum = prep_rows(xrows.reshape(-1, in_dim))
    # the same slots as plain q4mv over a stacked copy of the selected matrices
    idx = sel_d.long()
    ws, ss, bs = w[idx].contiguous(), s[idx].contiguous(), b[idx].contiguous()
    if shared:
        xe_s, xo_s, xsum_s = (t.repeat(n_sel, 1).contiguous() for t in (xe, xo, xsum))
    else:
        xe_s, xo_s, xsum_s = xe, xo, xsum
    y_ref, bound = oracle_lib.experts(case["codes"], case["scales"], case["biases"], sel_np,
                                      xrows[0] if shared else xrows, shared)
    for path in paths_for(out_dim) + [q4.PATH_AUTO]:
        flush(f"[experts] bank={n_bank} {out_dim}x{in_dim} nb={nb} sel={sel} "
              f"shared={shared} path={path}")
        y = q4.q4mv_experts(w, s, b, sel_d, xe, xo, xsum, nb, shared, path=path)
        y_q = q4.q4mv_path(ws, ss, bs, xe_s, xo_s, xsum_s, nb, path) if path else \
            q4.q4mv(ws, ss, bs, xe_s, xo_s, xsum_s, nb)
        torch.cuda.synchronize()
        assert torch.equal(y, y_q), f"path {path}: q4mv_experts differs from q4mv"
        parity(y.cpu().numpy(), y_ref, bound, f"experts path {path}")


@pytest.mark.parametrize("path", [q4.PATH_VALU, q4.PATH_VALU_2ROW, q4.PATH_MFMA])
def test_experts_bad_ids_give_nan(oracle_lib, path):
    n_bank, out_dim, in_dim, nb = 3, 64, 256, 4
    case = workloads.make_shape(n_bank, out_dim, in_dim, nb, seed=61)
    w, s, b = put_bank(case)
    sel_np = np.array([1, 7, -3, 0], dtype=np.int32)
    xrows = workloads.make_x(1, nb, in_dim, seed=62)
    xe, xo, xsum = prep_rows(xrows.reshape(nb, in_dim))
    flush(f"[experts] bad ids path={path}")
    y = q4.q4mv_experts(w, s, b, torch.from_numpy(sel_np).to(dev()), xe, xo, xsum, nb, True,
                        path=path).cpu().numpy()
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    y_ref, bound = oracle_lib.experts(case["codes"], case["scales"], case["biases"], sel_np,
                                      xrows[0], True)
    parity(y[[0, 3]], y_ref[[0, 3]], bound[[0, 3]], "valid slots next to bad ids")


@pytest.mark.parametrize("n_u,nb,out_dim", [(21, 4, 2560), (1, 1, 7), (8, 16, 333)])
def test_combine(oracle_lib, n_u, nb, out_dim):
    rng = np.random.default_rng(n_u * 100 + nb)
    y = rng.normal(size=(n_u, nb, out_dim)).astype(np.float32)
    wmap = (rng.uniform(-1, 1, size=(nb, n_u)) * (rng.uniform(size=(nb, n_u)) < 0.5)) \
        .astype(np.float32)
    yd, wd = torch.from_numpy(y).to(dev()), torch.from_numpy(wmap).to(dev())
    flush(f"[combine] n_u={n_u} nb={nb} out={out_dim}")
    out = q4.q4mv_combine(yd, wd)
    again = q4.q4mv_combine(yd, wd)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "combine is not deterministic"
    ref, mag = oracle_lib.combine(y, wmap)
    # n_u rounded multiply-adds in f32: each rounding is at most U times a partial sum,
    # and every partial sum is at most mag
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= (n_u + 1) * U * mag), np.max(err / ((n_u + 1) * U * mag + 1e-300))


def test_moe_layer(oracle_lib):
    """A decode MoE layer over 4 tokens: 32 experts, hidden 2560, intermediate 640, top-8
    routing. Gate/up of every routed expert over all 4 token rows (shared activations), the
    fused SwiGLU prep, the down projection of each expert's own rows, and the combine."""
    n_exp, hidden, inter, nb, top_k = 32, 2560, 640, 4, 8
    sel, wmap = workloads.make_routing(nb, n_exp, top_k, seed=71)
    n_u = sel.size
    gu_bank = workloads.make_shape(n_exp, 2 * inter, hidden, nb, seed=72)
    dn_bank = workloads.make_weights(n_exp, hidden, inter, seed=73)
    x = gu_bank["x"][0]  # [nb][hidden], the token rows
    flush(f"[moe layer] {n_u} routed experts of {n_exp}")
    w1, s1, b1 = put_bank(gu_bank)
    w2 = q4.q4mv_pack_codes(torch.from_numpy(dn_bank[0]).to(dev()))
    s2, b2 = bf16_tensor(dn_bank[1]), bf16_tensor(dn_bank[2])
    sel_d, wmap_d = torch.from_numpy(sel).to(dev()), torch.from_numpy(wmap).to(dev())
    xe, xo, xsum = prep_rows(x)
    gu = q4.q4mv_experts(w1, s1, b1, sel_d, xe, xo, xsum, nb, True)
    xe2, xo2, xsum2 = q4.q4mv_swiglu_prep(gu.view(n_u * nb, 2 * inter))
    y = q4.q4mv_experts(w2, s2, b2, sel_d, xe2, xo2, xsum2, nb, False)
    out = q4.q4mv_combine(y, wmap_d).cpu().numpy()

    g_ref, g_bound = oracle_lib.experts(gu_bank["codes"], gu_bank["scales"],
                                        gu_bank["biases"], sel, x, True)
    g_ref = g_ref.reshape(n_u * nb, 2 * inter)
    g_bound = g_bound.reshape(n_u * nb, 2 * inter)
    h_ref = oracle_lib.swiglu(g_ref)
    x_dn = h_ref.astype(np.float32).astype(np.float16).astype(np.float32)
    y_ref, bound = oracle_lib.experts(*dn_bank, sel, x_dn.reshape(n_u, nb, inter), False)
    # error of the down projection's input: the gate/up GEMV's (within ELEM * bound), moved
    # at most 1.1x by silu and multiplied by |up| (and |silu(gate)| for up's own error), then
    # f32 arithmetic and the f16 rounding on both sides
    g, u = g_ref[:, :inter], g_ref[:, inter:]
    eg, eu = ELEM * g_bound[:, :inter], ELEM * g_bound[:, inter:]
    e = (oracle_lib.SILU_LIPSCHITZ * eg * (np.abs(u) + eu) + np.abs(oracle_lib.silu(g)) * eu
         + 2.0 ** -10 * np.abs(h_ref) + 2.0 ** -24)
    # through the down matrix: sum_i |W[o][i]| e_i <= the oracle GEMV with |S|, |B| and x = e
    absS, absB = dn_bank[1] & 0x7FFF, dn_bank[2] & 0x7FFF
    prop, _ = oracle_lib.experts(dn_bank[0], absS, absB, sel,
                                 e.astype(np.float32).reshape(n_u, nb, inter), False)
    y_budget = ELEM * bound + prop
    out_ref, mag = oracle_lib.combine(y_ref, wmap)
    budget = np.einsum("ru,uro->ro", np.abs(wmap.astype(np.float64)), y_budget) \
        + (n_u + 1) * U * mag
    err = np.abs(out.astype(np.float64) - out_ref)
    assert np.all(np.isfinite(out))
    rel = np.linalg.norm(err) / np.linalg.norm(out_ref)
    assert np.all(err <= budget), f"per-element error {np.max(err / budget):.3f}x the budget"
    # relative L2: as the expert MLP chain (gate/up 1e-3, silu and f16, down 1e-3); the
    # combine is a convex mix per token and adds only f32 rounding
    assert rel <= 3e-3, f"relative L2 {rel:.2e}"
    flush(f"[moe layer] relative L2 {rel:.2e}")
