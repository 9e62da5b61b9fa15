"""Helpers for the GPU tests: move generated inputs to the device through the library's own
entry points, run a kernel path, and check parity against the oracle."""
import numpy as np
import torch

import affine_q4_gemv_amd as q4

REL_L2 = 1e-3       # relative L2 error over all outputs
ELEM = 2e-3         # per element: |err| <= ELEM * sum_i(|S q x| + |B x|)
# The relative L2 error is an aggregate: over a handful of outputs it is the relative error of
# single values, which cancellation in y (W has mean about 0) can make large while the error
# itself stays within the per-element bound. Results of fewer than REL_L2_MIN_N outputs
# therefore go to a pool per test and key (by default the description); at the end of the
# test the pool of each key must hold at least REL_L2_MIN_N outputs (tests of small shapes
# run several seeds) and meet the relative L2 bar as a whole (tests/conftest.py).
REL_L2_MIN_N = 64
SMALL = {}          # key -> list of (error, reference) arrays of the current test


def seeds_for(n_outputs):
    """Seeds a test of a shape with n_outputs outputs runs so that its small results pool at
    least REL_L2_MIN_N outputs."""
    return max(1, -(-REL_L2_MIN_N // max(1, n_outputs)))


def dev():
    return torch.device("cuda:0")


def bf16_tensor(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(dev()).view(torch.bfloat16)


def upload(case):
    """codes -> packed words on the device (q4mv_pack_codes), scales/biases, x -> prep."""
    codes = torch.from_numpy(case["codes"]).to(dev())
    w = q4.q4mv_pack_codes(codes)
    del codes
    s = bf16_tensor(case["scales"])
    b = bf16_tensor(case["biases"])
    n_mat, nb, in_dim = case["x"].shape
    x = torch.from_numpy(case["x"].reshape(n_mat * nb, in_dim)).to(dev())
    xe, xo, xsum = q4.q4mv_prepare_x(x)
    return dict(w=w, s=s, b=b, x=x, xe=xe, xo=xo, xsum=xsum, nb=nb)


def run(d, path=q4.PATH_AUTO, y=None):
    if path == "2row":
        out = q4.q4mv_2row(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], y=y)
    elif path == q4.PATH_AUTO:
        out = q4.q4mv(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], y=y)
    else:
        out = q4.q4mv_path(d["w"], d["s"], d["b"], d["xe"], d["xo"], d["xsum"], d["nb"], path,
                           y=y)
    torch.cuda.synchronize()
    return out


def parity(y_gpu, y_ref, bound, what="", key=None):
    """Both halves of the tolerance (the relative L2 half pooled for small results, see
    SMALL); returns (rel_l2, worst per-element ratio)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    ratio = np.max(err / (ELEM * bound + 1e-300)) if err.size else 0.0
    assert ratio <= 1.0, f"{what}: per-element error {ratio:.3f}x the bound"
    if y_gpu.size >= REL_L2_MIN_N:
        assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    else:
        SMALL.setdefault(what if key is None else key, []).append(
            (err.ravel(), np.asarray(y_ref, dtype=np.float64).ravel()))
    return rel, ratio


def check_small_pool():
    """The relative L2 bar over each key's pooled small results (called after each test)."""
    pool = dict(SMALL)
    SMALL.clear()
    for key, parts in pool.items():
        err = np.concatenate([e for e, _ in parts])
        ref = np.concatenate([r for _, r in parts])
        assert err.size >= REL_L2_MIN_N, \
            f"{key}: only {err.size} outputs pooled for the relative L2 check (run more seeds)"
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        assert rel <= REL_L2, f"{key}: pooled relative L2 error {rel:.3e} > {REL_L2}"


def flush(msg):
    print(msg, flush=True)
