"""GPU parity of the affine-Q4 quantiser (q4mv_quantize) against the oracle, bit for bit
(codes, scale and bias bits), and the quantise -> GEMV pipeline against the dense product."""
import numpy as np
import pytest
import torch

import affine_q4_gemv_amd as q4
import quant_ties
import workloads
from q4_gpu import ELEM, dev, flush

pytestmark = pytest.mark.gpu


def unpack(w):
    """int32 [..., in/8] packed words -> u8 codes [..., in] (code i of a word at bits 4i)."""
    u = w.cpu().numpy().view(np.uint32)
    return ((u[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 15).astype(np.uint8) \
        .reshape(*u.shape[:-1], u.shape[-1] * 8)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def weights(n, k, seed):
    rng = np.random.default_rng(seed)
    wf = (rng.normal(0, 0.02, (n, k)) + rng.normal(0, 0.05, (n, 1))).astype(np.float32)
    if n >= 4 and k >= 128:
        wf[0, :64] = 0.75                                   # constant group: d = 0
        wf[1, :64] = -0.25 + (np.arange(64) % 16) * 2.0 ** -6  # exact grid
        wf[2, :64] = rng.normal(0, 1e4, 64)                  # large magnitudes
        wf[3, :64] = rng.normal(0, 1e-30, 64)                # tiny: 1/d overflows -> id = 0
    if n >= 8 and k >= 128:
        # codes, scales and biases on exact rounding ties (round half to even)
        wf[4:8, :128] = quant_ties.tie_rows()[0]
    return wf


@pytest.mark.parametrize("n,k", [(8, 128), (37, 640), (300, 2560), (9728, 2560)])
def test_quantize_bit_exact(oracle_lib, n, k):
    wf = weights(n, k, seed=n + k)
    flush(f"[quantize] {n}x{k}")
    w, s, b = q4.q4mv_quantize(torch.from_numpy(wf).to(dev()))
    torch.cuda.synchronize()
    q_ref, s_ref, b_ref, _, _ = oracle_lib.quantize(wf)
    np.testing.assert_array_equal(unpack(w), q_ref)
    np.testing.assert_array_equal(bits(s), s_ref)
    np.testing.assert_array_equal(bits(b), b_ref)
    # the tie groups against the values the rounding rule itself gives
    _, codes, s_want, b_want = quant_ties.tie_rows()
    got_q, got_s, got_b = unpack(w), bits(s), bits(b)
    for (r, g), c in codes.items():
        np.testing.assert_array_equal(got_q[4 + r, 64 * g:64 * g + 64], c)
    for (r, g), want in s_want.items():
        assert int(got_s[4 + r, g]) == want
    for (r, g), want in b_want.items():
        assert int(got_b[4 + r, g]) == want


def test_quantize_then_gemv(oracle_lib):
    # dense f32 weights -> q4mv_quantize -> q4mv (3 activation rows, three matrices): within
    # the GEMV tolerance of the oracle on the stored codes, and within the quantisation bound
    # of the dense product
    n_mat, out_dim, in_dim, nb = 3, 1000, 2560, 3
    wf = weights(n_mat * out_dim, in_dim, seed=5).reshape(n_mat, out_dim, in_dim)
    x = np.random.default_rng(6).normal(0, 1, (n_mat, nb, in_dim)).astype(np.float32)
    w, s, b = q4.q4mv_quantize(torch.from_numpy(wf).to(dev()))
    xe, xo, xsum = q4.q4mv_prepare_x(torch.from_numpy(x.reshape(-1, in_dim)).to(dev()))
    flush("[quantize -> gemv]")
    y = q4.q4mv(w, s, b, xe, xo, xsum, nb).cpu().numpy().astype(np.float64)
    q_ref, s_ref, b_ref, d, mn = oracle_lib.quantize(wf.reshape(-1, in_dim))
    y_ref, bound = oracle_lib.gemv(q_ref.reshape(n_mat, out_dim, in_dim),
                                   s_ref.reshape(n_mat, out_dim, -1),
                                   b_ref.reshape(n_mat, out_dim, -1), x)
    assert np.all(np.abs(y - y_ref) <= ELEM * bound)
    dense = np.einsum("mri,moi->mro", x.astype(np.float64), wf.astype(np.float64))
    per_w = (np.repeat(d, 64, axis=1) / 2 + 2.0 ** -8 * (15 * np.repeat(d, 64, axis=1)
             + np.repeat(np.abs(mn), 64, axis=1))).reshape(n_mat, out_dim, in_dim)
    lim = np.einsum("mri,moi->mro", np.abs(x).astype(np.float64), per_w.astype(np.float64))
    assert np.all(np.abs(y - dense) <= lim + ELEM * bound)
