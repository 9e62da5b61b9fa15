"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: a dense double matvec built with a
different bf16 decoder (torch's), exact rational arithmetic, closed forms whose value is known
before anything is computed, one-hot layout probes and invariants. Each pin is written so that
a plausible mistake in the oracle (a dropped or sign-flipped term, a wrong scale/bias/x/code
index, a wrong bf16 decode) fails at least one of them; ``test_mutants_are_caught`` plants
such mistakes in copies of the oracle source and checks exactly that.
"""
import ctypes
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import quant_ties
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ONE_BF16 = 0x3F80  # bf16 bits of 1.0


def bf16_torch(bits):
    """Independent bf16 decode: reinterpret through torch's bfloat16 dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).double().numpy()


def pow2_bf16(e):
    """bf16 bits of 2**e (exact)."""
    return np.uint16(((int(e) + 127) & 0xFF) << 7)


def dense_reference(codes, scales, biases, x):
    """Dequantise to a dense double W and multiply with numpy: y [m][nb][out]."""
    s = bf16_torch(scales)
    b = bf16_torch(biases)
    w = s.repeat(64, axis=2) * codes.astype(np.float64) + b.repeat(64, axis=2)
    xd = x.astype(np.float64)
    y = np.matmul(xd, np.transpose(w, (0, 2, 1)))
    bound = np.matmul(np.abs(xd), np.transpose(np.abs(s.repeat(64, axis=2) * codes)
                                               + np.abs(b.repeat(64, axis=2)), (0, 2, 1)))
    return y, bound


# --------------------------------------------------------------------------------------
# the pin battery, parameterised by the gemv under test (so mutants can be run through it)

def _case(n_mat, out_dim, in_dim, nb, seed):
    c = workloads.make_shape(n_mat, out_dim, in_dim, nb, seed=seed)
    return c["codes"], c["scales"], c["biases"], c["x"]


def pin_bruteforce(gemv):
    for (m, o, i, nb, seed) in [(1, 1, 64, 1, 1), (2, 3, 128, 2, 2), (1, 8, 192, 3, 3),
                                (2, 5, 320, 2, 4)]:
        q, s, b, x = _case(m, o, i, nb, seed)
        y, bound = gemv(q, s, b, x)
        yr, br = dense_reference(q, s, b, x)
        if not np.all(np.abs(y - yr) <= 1e-12 * br + 1e-300):
            return False
        if not np.allclose(bound, br, rtol=1e-12, atol=0):
            return False
    return True


def pin_zero_at_midcode(gemv):
    """codes == 8 and B = -8 S  =>  W == 0, so y == 0 exactly for any x and any S."""
    q, s, b, x = _case(2, 7, 256, 3, 5)
    q[:] = 8
    y, _ = gemv(q, s, b, x)
    return bool(np.all(y == 0.0))


def pin_row_sum(gemv):
    """S = 1, B = 0, x = 1  =>  y = sum of the row's codes (an integer)."""
    q, s, b, x = _case(2, 9, 320, 2, 6)
    s[:] = ONE_BF16
    b[:] = 0
    x[:] = 1.0
    y, _ = gemv(q, s, b, x)
    want = q.astype(np.int64).sum(axis=2)  # [m][out]
    return bool(np.all(y == want[:, None, :]))


def pin_one_hot(gemv):
    """A single code 1 at (m, o, i), S = 1, B = 0, distinct exact x: y[m][r][o] = x[m][r][i]."""
    rng = np.random.default_rng(7)
    n_mat, out_dim, in_dim, nb = 3, 5, 192, 3
    x = (np.arange(n_mat * nb * in_dim, dtype=np.float32) + 1).reshape(n_mat, nb, in_dim)
    for _ in range(6):
        m, o, i = rng.integers(n_mat), rng.integers(out_dim), rng.integers(in_dim)
        q = np.zeros((n_mat, out_dim, in_dim), np.uint8)
        q[m, o, i] = 1
        s = np.full((n_mat, out_dim, in_dim // 64), ONE_BF16, np.uint16)
        b = np.zeros_like(s)
        y, _ = gemv(q, s, b, x)
        want = np.zeros((n_mat, nb, out_dim))
        want[m, :, o] = x[m, :, i]
        if not np.array_equal(y, want):
            return False
    return True


def pin_scale_position(gemv):
    """q = 1, B = 0, S[m][o][g] = 2^(g + 3o + 7m), x = 1 on group g0 only: y = 64 S[m][o][g0]."""
    n_mat, out_dim, in_dim, nb = 2, 4, 384, 2
    g = in_dim // 64
    e = (np.arange(g)[None, None, :] + 3 * np.arange(out_dim)[None, :, None]
         + 7 * np.arange(n_mat)[:, None, None])
    s = np.vectorize(pow2_bf16)(e - 20).astype(np.uint16)
    q = np.ones((n_mat, out_dim, in_dim), np.uint8)
    b = np.zeros_like(s)
    for g0 in range(g):
        x = np.zeros((n_mat, nb, in_dim), np.float32)
        x[:, :, 64 * g0:64 * g0 + 64] = 1.0
        y, _ = gemv(q, s, b, x)
        want = 64.0 * np.exp2(e[:, :, g0] - 20.0)
        if not np.array_equal(y, np.broadcast_to(want[:, None, :], y.shape)):
            return False
    return True


def pin_bias_position(gemv):
    """q = 0, B[m][o][g] = 2^(g + 3o + 7m), x = 1 on group g0 only: y = 64 B[m][o][g0]."""
    n_mat, out_dim, in_dim, nb = 2, 4, 384, 2
    g = in_dim // 64
    e = (np.arange(g)[None, None, :] + 3 * np.arange(out_dim)[None, :, None]
         + 7 * np.arange(n_mat)[:, None, None])
    b = np.vectorize(pow2_bf16)(e - 20).astype(np.uint16)
    q = np.zeros((n_mat, out_dim, in_dim), np.uint8)
    s = np.full_like(b, ONE_BF16)
    for g0 in range(g):
        x = np.zeros((n_mat, nb, in_dim), np.float32)
        x[:, :, 64 * g0:64 * g0 + 64] = 1.0
        y, _ = gemv(q, s, b, x)
        want = 64.0 * np.exp2(e[:, :, g0] - 20.0)
        if not np.array_equal(y, np.broadcast_to(want[:, None, :], y.shape)):
            return False
    return True


def pin_activation_rows(gemv):
    """Row r of the output depends on activation row r only; matrices are independent."""
    q, s, b, x = _case(3, 6, 256, 4, 8)
    y, _ = gemv(q, s, b, x)
    perm = np.array([2, 0, 3, 1])
    yp, _ = gemv(q, s, b, np.ascontiguousarray(x[:, perm, :]))
    if not np.array_equal(yp, y[:, perm, :]):
        return False
    for m in range(3):
        ym, _ = gemv(q[m:m + 1], s[m:m + 1], b[m:m + 1], x[m:m + 1])
        if not np.array_equal(ym[0], y[m]):
            return False
    return True


def pin_bound(gemv):
    """bound >= |y| everywhere and bound equals |W| . |x| from the dense reference."""
    q, s, b, x = _case(2, 11, 256, 2, 9)
    y, bound = gemv(q, s, b, x)
    _, br = dense_reference(q, s, b, x)
    return bool(np.all(bound >= np.abs(y)) and np.allclose(bound, br, rtol=1e-12, atol=0))


PINS = [pin_bruteforce, pin_zero_at_midcode, pin_row_sum, pin_one_hot, pin_scale_position,
        pin_bias_position, pin_activation_rows, pin_bound]


def oracle_gemv(q, s, b, x):
    import oracle
    return oracle.gemv(q, s, b, x, nthreads=2)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(oracle_lib, pin):
    assert pin(oracle_gemv)


def test_exact_rational(oracle_lib):
    """The double oracle agrees with an exact rational evaluation of the definition."""
    q, s, b, x = _case(1, 3, 128, 2, 11)
    y, bound = oracle_lib.gemv(q, s, b, x)
    sf = bf16_torch(s)
    bf = bf16_torch(b)
    for r in range(2):
        for o in range(3):
            tot = Fraction(0)
            for i in range(128):
                w = Fraction(sf[0, o, i // 64]) * int(q[0, o, i]) + Fraction(bf[0, o, i // 64])
                tot += w * Fraction(float(x[0, r, i]))
            assert abs(Fraction(y[0, r, o]) - tot) <= Fraction(1e-14) * Fraction(bound[0, r, o])


def test_rows_matches_full(oracle_lib):
    q, s, b, x = _case(2, 13, 192, 3, 12)
    y, bound = oracle_lib.gemv(q, s, b, x)
    mats = np.array([0, 1, 1, 0, 1])
    rows = np.array([0, 12, 5, 7, 0])
    ys, bs = oracle_lib.gemv_rows(q, s, b, x, mats, rows)
    assert np.array_equal(ys, y[mats, :, rows])
    assert np.array_equal(bs, bound[mats, :, rows])


def test_rejects_bad_shapes(oracle_lib):
    q, s, b, x = _case(1, 2, 64, 1, 0)
    with pytest.raises(ValueError):
        oracle_lib.gemv(q[:, :, :32], s, b, x)
    with pytest.raises(ValueError):
        oracle_lib.gemv(q, s, b, x[:, :, :32])
    bad = q.copy()
    bad[0, 0, 0] = 16
    with pytest.raises(ValueError):
        oracle_lib.gemv(bad, s, b, x)
    with pytest.raises(ValueError):
        oracle_lib.gemv_rows(q, s, b, x, [0], [2])


def test_tiny_workload_rel_to_dense(oracle_lib):
    c = workloads.make_case("tiny")
    y, bound = oracle_lib.gemv(c["codes"], c["scales"], c["biases"], c["x"])
    yr, _ = dense_reference(c["codes"], c["scales"], c["biases"], c["x"])
    assert np.all(np.abs(y - yr) <= 1e-12 * bound)


# --------------------------------------------------------------------------------------
# activation prep oracle

def test_prep_layout_and_sums(oracle_lib):
    x = (np.arange(2 * 128, dtype=np.float32).reshape(2, 128) - 50.0) * 0.25  # exact in f16
    xe, xo, xsum = oracle_lib.prepare_x(x)
    assert np.array_equal(xe.astype(np.float32), x[:, 0::2])
    assert np.array_equal(xo.astype(np.float32), x[:, 1::2])
    # chunk c of row n holds elements 32c..32c+31: closed-form arithmetic series sum
    for n in range(2):
        for c in range(4):
            k = np.arange(32 * c, 32 * c + 32) + 128 * n
            assert xsum[n, c] == float(((k - 50.0) * 0.25).sum())


def test_prep_f16_rounding_matches_torch(oracle_lib):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[0, :64] = np.ldexp(rng.random(64), rng.integers(-30, -12, 64)).astype(np.float32)
    # ties: 1 + 2^-11 -> 1 (even), 1 + 3*2^-11 -> 1 + 2^-9, 2^-25 -> 0, 65520 -> inf
    x[1, :4] = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 65520.0]
    xe, xo, _ = oracle_lib.prepare_x(x)
    th = torch.from_numpy(x).half().numpy()
    assert np.array_equal(xe.view(np.uint16), np.ascontiguousarray(th[:, 0::2]).view(np.uint16))
    assert np.array_equal(xo.view(np.uint16), np.ascontiguousarray(th[:, 1::2]).view(np.uint16))
    # x[1,0] -> xe[1,0], x[1,1] -> xo[1,0], x[1,2] -> xe[1,1], x[1,3] -> xo[1,1]
    assert xe[1, 0].view(np.uint16) == 0x3C00
    assert xo[1, 0].view(np.uint16) == 0x3C02
    assert xe[1, 1].view(np.uint16) == 0x0000
    assert np.isinf(xo[1, 1])


def test_prep_constant_sum(oracle_lib):
    x = np.full((1, 96), 0.1, np.float32)
    _, _, xsum = oracle_lib.prepare_x(x)
    assert np.all(xsum == 32.0 * float(np.float16(0.1)))


# --------------------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle source must fail at least one pin

MUTANTS = {
    "dropped_bias_term": ("acc += s * qx + b * xs;", "acc += s * qx;"),
    "bias_sign": ("acc += s * qx + b * xs;", "acc += s * qx - b * xs;"),
    "scale_group_shift": ("const double s = bf16_value(srow[g]);",
                          "const double s = bf16_value(srow[(g + 1) % groups]);"),
    "bias_reads_scales": ("const double b = bf16_value(brow[g]);",
                          "const double b = bf16_value(srow[g]);"),
    "x_transposed": ("const double xv = (double)xr[g * GROUP + j];",
                     "const double xv = (double)xr[j * groups + g];"),
    "code_ignores_matrix": ("const uint8_t *qrow = q + (m * out_dim + o) * in_dim;",
                            "const uint8_t *qrow = q + o * in_dim;"),
    "x_ignores_row": ("const float *xr = x + (m * nb + r) * in_dim;",
                      "const float *xr = x + (m * nb) * in_dim;"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "bound_signed_bias": ("bnd += fabs(s) * qax + fabs(b) * ax;", "bnd += fabs(s) * qax + b * ax;"),
    "code_scale_swapped": ("qx += qv * xv;", "qx += (15.0 - qv) * xv;"),
}


def _load_variant(path):
    lib = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q4ref_gemv.argtypes = [p, p, p, p, i64, i64, i64, i64, p, p, ctypes.c_int]
    lib.q4ref_gemv.restype = ctypes.c_int

    def gemv(q, s, b, x):
        q = np.ascontiguousarray(q, np.uint8)
        s = np.ascontiguousarray(s, np.uint16)
        b = np.ascontiguousarray(b, np.uint16)
        x = np.ascontiguousarray(x, np.float32)
        n_mat, out_dim, in_dim = q.shape
        nb = x.shape[1]
        y = np.empty((n_mat, nb, out_dim))
        bound = np.empty_like(y)
        assert lib.q4ref_gemv(q.ctypes.data, s.ctypes.data, b.ctypes.data, x.ctypes.data,
                              n_mat, out_dim, in_dim, nb, y.ctypes.data, bound.ctypes.data,
                              1) == 0
        return y, bound
    return gemv


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_mutants_are_caught(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "q4ref.c")).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        mpath = tmp_path / f"{name}.c"
        mpath.write_text(src.replace(old, new))
        so = tmp_path / f"lib{name}.so"
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-pthread", str(mpath), "-o",
                        str(so), "-lm"], check=True)
        gemv = _load_variant(str(so))
        failed = [p.__name__ for p in PINS if not p(gemv)]
        assert failed, f"mutant {name} passed every pin"


# --- fused epilogues (Constant BATCH_MSL page, fn_qmv_silu_b and fn_moe_act_b) -------------

def test_silu_identities(oracle_lib):
    oracle = oracle_lib
    # silu(t) - silu(-t) = t exactly, and silu(t) = (t/2)(1 + tanh(t/2)): the second form uses
    # tanh instead of exp, so it checks the exp-based oracle against independent arithmetic
    t = np.concatenate([np.linspace(-60, 60, 2401), [0.0, 1e-300, -1e-300, 700.0, -700.0]])
    s = oracle.silu(t)
    np.testing.assert_allclose(s - oracle.silu(-t), t, rtol=1e-15, atol=1e-300)
    # (the tanh form cancels for t << 0, so there it is compared in absolute terms)
    th = 0.5 * t * (1.0 + np.tanh(0.5 * t))
    near = t > -5
    np.testing.assert_allclose(s[near], th[near], rtol=1e-13, atol=1e-300)
    assert np.all(np.abs(s - th) <= 1e-14 * np.abs(t) + 1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert np.all(np.isfinite(s))


def test_silu_lipschitz_constant(oracle_lib):
    oracle = oracle_lib
    # the bound used for the epilogue: max |silu'| over a fine grid stays below 1.1
    t = np.linspace(-20, 20, 400001)
    d = np.gradient(oracle.silu(t), t)
    assert d.max() < oracle.SILU_LIPSCHITZ and d.max() > 1.09


def test_gemv_silu_sign_symmetry(oracle_lib):
    oracle = oracle_lib
    # the GEMV is linear in x: y(-x) = -y(x), so silu(y(-x) / -div) = silu(y(x) / div), and
    # the odd identity gives silu(y/div) - silu(-y/div) = y / div
    c = workloads.make_shape(2, 40, 256, 3, seed=11)
    a, _ = oracle.gemv_silu(c["codes"], c["scales"], c["biases"], c["x"], 3.0)
    b, _ = oracle.gemv_silu(c["codes"], c["scales"], c["biases"], -c["x"], -3.0)
    np.testing.assert_array_equal(a, b)
    m, _ = oracle.gemv_silu(c["codes"], c["scales"], c["biases"], -c["x"], 3.0)
    y, _ = oracle.gemv(c["codes"], c["scales"], c["biases"], c["x"])
    np.testing.assert_allclose(a - m, y / 3.0, rtol=1e-12, atol=1e-12)


def test_swiglu_closed_forms(oracle_lib):
    oracle = oracle_lib
    rng = np.random.default_rng(5)
    g = rng.normal(size=(3, 64)) * 4
    u = rng.normal(size=(3, 64))
    h = oracle.swiglu(np.concatenate([g, u], axis=1))
    # odd identity in the gate, linearity in up, and the saturated gate
    h_neg = oracle.swiglu(np.concatenate([-g, u], axis=1))
    np.testing.assert_allclose(h - h_neg, g * u, rtol=1e-13, atol=1e-13)
    h2 = oracle.swiglu(np.concatenate([g, 2 * u], axis=1))
    np.testing.assert_array_equal(h2, 2 * h)
    big = oracle.swiglu(np.concatenate([np.full((1, 64), 50.0), u[:1]], axis=1))
    np.testing.assert_allclose(big, 50.0 * u[:1], rtol=1e-15)
    assert np.all(oracle.swiglu(np.concatenate([np.zeros((1, 64)), u[:1]], axis=1)) == 0)


# --- affine-Q4 quantiser (steps of host_quant_q5_row, memra-engine qwen4exp_gpu.rs page) ----
# The pins take the quantiser under test, so planted mistakes can be run through them.

def qpin_reconstruction_bound(quantize):
    # every weight is within d/2 of d*q + mn (the rounding step), up to f32 slack, and the
    # group's minimum gets code 0 and its maximum code 15
    rng = np.random.default_rng(3)
    wf = (rng.normal(0, 0.02, (6, 512)) + rng.normal(0, 0.1, (6, 1))).astype(np.float32)
    q, s_bits, b_bits, d, mn = quantize(wf)
    g = wf.reshape(6, 8, 64).astype(np.float64)
    rec = d[:, :, None].astype(np.float64) * q.reshape(6, 8, 64) + mn[:, :, None]
    slack = 4 * 2.0 ** -24 * (np.abs(g).max(axis=2) + 15 * d)[:, :, None]
    ok = np.all(np.abs(rec - g) <= d[:, :, None] / 2 + slack)
    qq = q.reshape(6, 8, 64)
    ok &= np.all(qq[np.arange(6)[:, None], np.arange(8)[None, :], g.argmin(axis=2)] == 0)
    ok &= np.all(qq[np.arange(6)[:, None], np.arange(8)[None, :], g.argmax(axis=2)] == 15)
    # the stored bf16 values decode to within half a bf16 ulp (2^-8 relative) of d and mn
    sd = bf16_torch(s_bits)
    bd = bf16_torch(b_bits)
    ok &= np.all(np.abs(sd - d) <= 2.0 ** -8 * np.abs(d))
    ok &= np.all(np.abs(bd - mn) <= 2.0 ** -8 * np.abs(mn))
    return bool(ok)


def qpin_closed_forms(quantize):
    # a group on an exact grid mn + k*2^-6 (k = 0..15) gets codes k, d = 2^-6 and bias mn; a
    # constant group gets d = 0, codes 0 and bias = the constant
    k = np.arange(64) % 16
    wf = np.stack([-0.25 + k * 2.0 ** -6, np.full(64, 0.75)]).astype(np.float32)
    q, s_bits, b_bits, d, mn = quantize(wf)
    return bool(np.array_equal(q[0], k) and d[0, 0] == np.float32(2.0 ** -6)
                and mn[0, 0] == np.float32(-0.25) and s_bits[0, 0] == 0x3C80
                and b_bits[0, 0] == 0xBE80 and np.all(q[1] == 0) and d[1, 0] == 0
                and s_bits[1, 0] == 0 and b_bits[1, 0] == 0x3F40)


def qpin_code_ties(quantize):
    # (w - mn) / d lands exactly on k + 1/2: round half to even (round_ties_even)
    rows, codes, _, _ = quant_ties.tie_rows()
    q = quantize(rows)[0]
    return all(np.array_equal(q[r, 64 * g:64 * g + 64], c) for (r, g), c in codes.items())


def qpin_bf16_ties(quantize):
    # d and mn whose f32 low half is exactly 0x8000: stored rounded to nearest even
    rows, _, s_want, b_want = quant_ties.tie_rows()
    _, s_bits, b_bits, _, _ = quantize(rows)
    return (all(int(s_bits[r, g]) == w for (r, g), w in s_want.items())
            and all(int(b_bits[r, g]) == w for (r, g), w in b_want.items()))


QPINS = [qpin_reconstruction_bound, qpin_closed_forms, qpin_code_ties, qpin_bf16_ties]


@pytest.mark.parametrize("pin", QPINS, ids=[p.__name__ for p in QPINS])
def test_quantize_pin(oracle_lib, pin):
    assert pin(oracle_lib.quantize)


# planted mistakes in the quantiser (text edits of the oracle's own source, run on the CPU):
# each must fail at least one pin
QMUTANTS = {
    "code_round_half_up": ("t = np.rint((g - mn[:, :, None]) * inv[:, :, None])",
                           "t = np.floor((g - mn[:, :, None]) * inv[:, :, None] + np.float32(0.5))"),
    "code_truncate": ("t = np.rint((g - mn[:, :, None]) * inv[:, :, None])",
                      "t = np.trunc((g - mn[:, :, None]) * inv[:, :, None])"),
    "bf16_round_half_up": ("return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)",
                           "return ((u + 0x8000) >> 16).astype(np.uint16)"),
    "bf16_truncate": ("return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)",
                      "return (u >> 16).astype(np.uint16)"),
    "sixteen_steps": ("d = ((mx - mn) / np.float32(15.0)).astype(np.float32)",
                      "d = ((mx - mn) / np.float32(16.0)).astype(np.float32)"),
    "bias_is_max": ("return q, _bf16_rne_bits(d), _bf16_rne_bits(mn), d, mn",
                    "return q, _bf16_rne_bits(d), _bf16_rne_bits(mx), d, mn"),
    "codes_clipped_at_14": ("q = np.clip(t, 0, 15)", "q = np.clip(t, 0, 14)"),
}


def test_quantize_mutants_are_caught():
    path = os.path.join(ROOT, "oracle", "__init__.py")
    src = open(path).read()
    for name, (old, new) in QMUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        ns = {"__name__": f"oracle_mutant_{name}", "__file__": path}
        exec(compile(src.replace(old, new), f"<{name}>", "exec"), ns)
        failed = []
        for pin in QPINS:
            try:
                if not pin(ns["quantize"]):
                    failed.append(pin.__name__)
            except Exception:
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every quantiser pin"


def test_quantize_then_gemv(oracle_lib):
    # the quantised matrix times x stays within sum_i |x_i| * (d/2 + bf16 rounding of the
    # scale (times up to 15) and the bias) of the
    # dense product, computed by the GEMV oracle on the stored codes, scales and biases
    rng = np.random.default_rng(8)
    wf = rng.normal(0, 0.02, (96, 256)).astype(np.float32)
    x = rng.normal(0, 1, (1, 2, 256)).astype(np.float32)
    q, s_bits, b_bits, d, mn = oracle_lib.quantize(wf)
    y, _ = oracle_lib.gemv(q.reshape(1, 96, 256), s_bits.reshape(1, 96, 4),
                           b_bits.reshape(1, 96, 4), x)
    dense = (x[0].astype(np.float64) @ wf.T.astype(np.float64))
    dmax = np.repeat(d, 64, axis=1).astype(np.float64)
    mabs = np.repeat(np.abs(mn), 64, axis=1).astype(np.float64)
    per_w = dmax / 2 + 2.0 ** -8 * (15 * dmax + mabs) + 1e-7
    lim = np.abs(x[0]).astype(np.float64) @ per_w.T
    assert np.all(np.abs(y[0] - dense) <= lim)


def _probe_bank(n_bank, out_dim, in_dim):
    """All codes 0, so y = sum_g bias * sum_x; bank matrix e, row o has bias (e+1) + 8*o in
    every group (small integers, exact in bf16): the output names the matrix and the row."""
    codes = np.zeros((n_bank, out_dim, in_dim), dtype=np.uint8)
    vals = (np.arange(n_bank)[:, None] + 1 + 8 * np.arange(out_dim)[None, :]).astype(np.float32)
    biases = np.repeat(workloads.f32_to_bf16_bits(vals)[:, :, None], in_dim // 64, axis=2)
    rng = np.random.default_rng(3)
    scales = workloads.f32_to_bf16_bits(rng.normal(0, 1, biases.shape).astype(np.float32))
    return codes, scales, biases, vals


def test_experts_pick_matrix_and_rows(oracle_lib):
    n_bank, out_dim, in_dim, nb = 5, 4, 128, 3
    codes, scales, biases, vals = _probe_bank(n_bank, out_dim, in_dim)
    sel = np.array([3, 0, 3, 4], dtype=np.int32)  # repeats and any order
    # per-slot rows: slot u row r is the constant (u*nb + r + 1) / 64 (exact)
    c = (np.arange(sel.size * nb) + 1).reshape(sel.size, nb) / 64.0
    x = np.repeat(c[:, :, None], in_dim, axis=2).astype(np.float32)
    y, bound = oracle_lib.experts(codes, scales, biases, sel, x, x_shared=False)
    want = in_dim * c[:, :, None] * vals[sel][:, None, :]
    assert np.array_equal(y, want)
    assert np.array_equal(bound, np.abs(want))
    # shared rows: every slot reads rows 0..nb-1 (row r = (r + 1) / 64)
    y, _ = oracle_lib.experts(codes, scales, biases, sel, x[0], x_shared=True)
    assert np.array_equal(y, in_dim * c[0][None, :, None] * vals[sel][:, None, :])


def test_experts_bad_ids_are_nan(oracle_lib):
    codes, scales, biases, vals = _probe_bank(3, 2, 64)
    x = np.ones((2, 64), dtype=np.float32)
    y, bound = oracle_lib.experts(codes, scales, biases, [2, -1, 3, 1], x, x_shared=True)
    assert np.all(np.isnan(y[[1, 2]])) and np.all(bound[[1, 2]] == 0)
    assert np.array_equal(y[0], np.broadcast_to(64 * vals[2], (2, 2)))
    assert np.array_equal(y[3], np.broadcast_to(64 * vals[1], (2, 2)))


def test_experts_equal_stacked_gemv(oracle_lib):
    """Slot u over bank matrix sel[u] equals the dense double matvec of that matrix (a
    reference with its own bf16 decoder)."""
    case = workloads.make_shape(6, 48, 192, 2, seed=31)
    sel = np.array([5, 1, 1, 0], dtype=np.int32)
    x = workloads.make_x(sel.size, 2, 192, seed=32)
    y, _ = oracle_lib.experts(case["codes"], case["scales"], case["biases"], sel, x, False)
    ref, _ = dense_reference(case["codes"][sel], case["scales"][sel], case["biases"][sel], x)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_combine_closed_forms(oracle_lib):
    rng = np.random.default_rng(5)
    n_u, nb, out_dim = 4, 3, 5
    y = rng.normal(size=(n_u, nb, out_dim))
    # one-hot weights select a slot per token
    pick = np.array([2, 0, 3])
    onehot = np.zeros((nb, n_u))
    onehot[np.arange(nb), pick] = 1.0
    out, _ = oracle_lib.combine(y, onehot)
    assert np.array_equal(out, y[pick, np.arange(nb)])
    # all-ones weights sum the slots; zero weights give zero
    out, mag = oracle_lib.combine(y, np.ones((nb, n_u)))
    assert np.allclose(out, y.sum(axis=0), rtol=1e-15, atol=1e-15)
    assert np.allclose(mag, np.abs(y).sum(axis=0), rtol=1e-15)
    out, mag = oracle_lib.combine(y, np.zeros((nb, n_u)))
    assert not out.any() and not mag.any()
    # hand-worked: token 0 = 2*y[0] - y[1], token 1 = y[1]/2 (integers, exact)
    y = np.arange(2 * 2 * 3, dtype=np.float64).reshape(2, 2, 3)
    out, mag = oracle_lib.combine(y, [[2.0, -1.0], [0.0, 0.5]])
    assert np.array_equal(out, [[-6.0, -5.0, -4.0], [4.5, 5.0, 5.5]])
    assert np.array_equal(mag, [[6.0, 9.0, 12.0], [4.5, 5.0, 5.5]])


# ---- low-bit variants (Q2 / Q3)

# (column within a 64-code row, word index, bit) written out by hand from the placement rule:
# column t = 16i + 8u + p of chunk c sits in nibble p of word 2c + i shifted by 2u (bit
# 4p + 2u), so columns t and t + 4 lie 16 bits apart (the two f16 halves of one lane); the
# lowest bits of Q3 sit at bit 4p + 2i + u of the chunk's low-bit word.
Q2_PROBES = [(0, 0, 0), (1, 0, 4), (3, 0, 12), (4, 0, 16), (7, 0, 28), (8, 0, 2), (11, 0, 14),
             (12, 0, 18), (15, 0, 30), (16, 1, 0), (20, 1, 16), (24, 1, 2), (31, 1, 30),
             (32, 2, 0), (45, 2, 22), (63, 3, 30)]
# Q3: chunk c is words 3c, 3c + 1 (the upper two bits, at the Q2 positions of words 2c,
# 2c + 1) and its lowest-bit word 3c + 2 (words 2 and 5 here)
Q3_LOW_PROBES = [(0, 2, 0), (4, 2, 16), (8, 2, 1), (13, 2, 21), (16, 2, 2), (20, 2, 18),
                 (25, 2, 7), (31, 2, 31), (32, 5, 0), (63, 5, 31)]


# the lowest-bit positions of the Q2 probe columns, from the same rule (4p + 2i + u)
Q3_LOW_BIT = {0: 0, 1: 4, 3: 12, 4: 16, 7: 28, 8: 1, 11: 13, 12: 17, 15: 29, 16: 2, 20: 18,
              24: 3, 31: 31, 32: 0, 45: 21, 63: 31}


def test_lowbit_pack_probes(oracle_lib):
    for col, word, bit in Q2_PROBES:
        codes = np.zeros((1, 64), dtype=np.uint8)
        codes[0, col] = 15
        want = np.zeros(4, dtype=np.uint32)
        want[word] = np.uint32(3) << bit
        assert np.array_equal(oracle_lib.pack_lowbit(2, codes)[0], want), col
        # Q3: the upper two bits at the Q2 position, the lowest bit in the low-bit word
        codes[0, col] = 0b1110  # q3 = 7 -> upper 3, lowest 1
        w3 = oracle_lib.pack_lowbit(3, codes)[0]
        c, i = word // 2, word % 2
        want = np.zeros(6, dtype=np.uint32)
        want[3 * c + i] = np.uint32(3) << bit
        want[3 * c + 2] = np.uint32(1) << Q3_LOW_BIT[col]
        assert np.array_equal(w3, want), col
    for col, word, bit in Q3_LOW_PROBES:
        codes = np.zeros((1, 64), dtype=np.uint8)
        codes[0, col] = 0b0010  # q3 = 1: only the lowest bit
        w3 = oracle_lib.pack_lowbit(3, codes)[0]
        want = np.zeros(6, dtype=np.uint32)
        want[word] = np.uint32(1) << bit
        assert np.array_equal(w3, want), col
    # only the top bits of the 4-bit code count, and every bit is used once
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (5, 128), dtype=np.uint8)
    for bits in (2, 3):
        full = oracle_lib.pack_lowbit(bits, codes | 0xF0)
        assert np.array_equal(full, oracle_lib.pack_lowbit(bits, codes))
        ones = oracle_lib.pack_lowbit(bits, np.full((1, 128), 15, dtype=np.uint8))
        assert np.all(ones == 0xFFFFFFFF)


def test_lowbit_midpoints(oracle_lib):
    """Each low-bit code stands for a range of 4-bit codes and is reconstructed at the mean
    of that range: with S = 1, B = 0 and a one-hot x the output is that mean."""
    for bits in (2, 3):
        for q4 in range(16):
            same = [v for v in range(16) if v >> (4 - bits) == q4 >> (4 - bits)]
            codes = np.full((1, 1, 64), q4, dtype=np.uint8)
            x = np.zeros((1, 1, 64), dtype=np.float32)
            x[0, 0, 5] = 1.0
            y, _ = oracle_lib.gemv_lowbit(bits, codes, np.full((1, 1, 1), ONE_BF16, np.uint16),
                                          np.zeros((1, 1, 1), np.uint16), x)
            assert y[0, 0, 0] == sum(same) / len(same), (bits, q4)


def test_lowbit_decomposition(oracle_lib):
    """y_lowbit = K * (GEMV of the low-bit codes, no bias) + M * (bias-only GEMV with S as the
    bias) + (bias-only GEMV with B), each term from the C oracle, which shares no code with
    gemv_lowbit; and the bound against a brute-force sum on a small case."""
    case = workloads.make_shape(2, 24, 192, 3, seed=77)
    zeros = np.zeros_like(case["codes"])
    for bits in (2, 3):
        K, M = oracle_lib.LOWBIT_KM[bits]
        y, bound = oracle_lib.gemv_lowbit(bits, case["codes"], case["scales"], case["biases"],
                                          case["x"])
        q = case["codes"] >> (4 - bits)
        t1, _ = oracle_lib.gemv(q, case["scales"], np.zeros_like(case["biases"]), case["x"])
        t2, _ = oracle_lib.gemv(zeros, case["scales"], case["scales"], case["x"])
        t3, _ = oracle_lib.gemv(zeros, case["scales"], case["biases"], case["x"])
        assert np.allclose(y, K * t1 + M * t2 + t3, rtol=1e-12, atol=1e-12)
        s = bf16_torch(case["scales"])
        b = bf16_torch(case["biases"])
        m, r, o = 1, 2, 17
        brute = sum(abs((K * int(q[m, o, i]) + M) * s[m, o, i // 64] * float(case["x"][m, r, i]))
                    + abs(b[m, o, i // 64] * float(case["x"][m, r, i])) for i in range(192))
        assert bound[m, r, o] == pytest.approx(brute, rel=1e-12)
    # selected rows agree with the full result
    y, bound = oracle_lib.gemv_lowbit(3, case["codes"], case["scales"], case["biases"], case["x"])
    ys, bs = oracle_lib.gemv_lowbit(3, case["codes"], case["scales"], case["biases"], case["x"],
                                    rows=[23, 0, 5])
    assert np.array_equal(ys, y[:, :, [23, 0, 5]]) and np.array_equal(bs, bound[:, :, [23, 0, 5]])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    """The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
    only) runs exactly-sized buffers through both entry points with no report."""
    exe = tmp_path / "q4ref_sanitized"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
                    os.path.join(ROOT, "oracle", "q4ref.c"),
                    os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-o", str(exe), "-lm"],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
