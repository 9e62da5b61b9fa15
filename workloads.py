"""Seeded synthetic inputs for the affine-Q4 row-batched GEMV.

This module is shared by the oracle side and the device side of every test and of the
benchmark. It holds none of the GEMV's arithmetic: it only draws codes, scales, biases and
activations with the shapes and value distributions of the decode-engine projections on the
pages, and stores them in their storage types:

* codes: ``u8 [n_mat][out_dim][in_dim]``, one code 0..15 per byte (unpacked; packing into
  u32 words is a device-side step of the library);
* scales, biases: bf16 bit patterns ``u16 [n_mat][out_dim][in_dim/64]``;
* activations: ``f32 [n_mat][nb][in_dim]``.

Value recipe (one reading, stated once):

* codes i.i.d. uniform on {0, ..., 15}, both ends included;
* scale = bf16(N(0, 0.02)) where 0.02 is the standard deviation; the f32 draw is rounded to
  bf16 to nearest-even, the rounding rule of ``f32_to_bf16_rne`` on the memra-engine
  ``qwen4exp_gpu.rs`` page;
* bias = -8 * scale, formed from the bf16-rounded scale (exact in bf16: x8 moves the exponent);
* x i.i.d. N(0, 1) in f32, times ``x_scale`` (0.5 for the expert down projection, whose
  inputs are post-SwiGLU magnitudes).

Random streams: ``numpy.random.SeedSequence(seed).spawn(3)`` gives three independent PCG64
streams, used for codes, scales and activations in that order.
"""
from __future__ import annotations

import numpy as np

GROUP = 64  # codes per scale/bias group

# Named workloads: the projection shapes of the decode engines on the pages.
WORKLOADS = {
    # small case the oracle finishes in well under a second
    "tiny": dict(n_mat=1, out_dim=256, in_dim=512, nb=1, x_scale=1.0),
    # dense decode projection, hidden 2560 -> 2560
    "dense": dict(n_mat=1, out_dim=2560, in_dim=2560, nb=1, x_scale=1.0),
    # MoE expert down projection: 8 experts, each its own 2560x640 matrix and 4 token rows
    "moe_down": dict(n_mat=8, out_dim=2560, in_dim=640, nb=4, x_scale=0.5),
    # MLP up projection 2560 -> 9728 with 8 activation rows
    "up": dict(n_mat=1, out_dim=9728, in_dim=2560, nb=8, x_scale=1.0),
    # LM head 2560 -> 151936 (NB 1 and 16)
    "lm_head": dict(n_mat=1, out_dim=151936, in_dim=2560, nb=1, x_scale=1.0),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Adds 0x7fff plus the lowest kept bit to the f32 pattern and keeps the high half, the
    rule of ``f32_to_bf16_rne`` on the memra-engine ``qwen4exp_gpu.rs`` page. Inputs must be
    finite (the generator's normal draws always are)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return ((u >> 16) & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> f32 values (the 16 bits are the high half of an f32)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]


def make_weights(n_mat: int, out_dim: int, in_dim: int, seed: int = 0):
    """Codes (u8, unpacked), scale and bias bf16 patterns for ``n_mat`` matrices."""
    if in_dim % GROUP:
        raise ValueError("in_dim must be a multiple of 64")
    rc, rs, _ = _streams(seed)
    codes = rc.integers(0, 16, size=(n_mat, out_dim, in_dim), dtype=np.uint8)
    s32 = (rs.standard_normal(size=(n_mat, out_dim, in_dim // GROUP), dtype=np.float32)
           * np.float32(0.02))
    scales = f32_to_bf16_bits(s32)
    b32 = bf16_bits_to_f32(scales) * np.float32(-8.0)  # exact: power-of-two factor
    biases = f32_to_bf16_bits(b32)
    return codes, scales, biases


def make_x(n_mat: int, nb: int, in_dim: int, seed: int = 0, x_scale: float = 1.0):
    """Activations f32 [n_mat][nb][in_dim] ~ x_scale * N(0, 1)."""
    _, _, rx = _streams(seed)
    x = rx.standard_normal(size=(n_mat, nb, in_dim), dtype=np.float32)
    if x_scale != 1.0:
        x = x * np.float32(x_scale)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_case(name: str, nb: int | None = None, seed: int = 0):
    """All inputs of a named workload: dict with codes, scales, biases, x and the shape."""
    w = dict(WORKLOADS[name])
    if nb is not None:
        w["nb"] = nb
    codes, scales, biases = make_weights(w["n_mat"], w["out_dim"], w["in_dim"], seed)
    x = make_x(w["n_mat"], w["nb"], w["in_dim"], seed, w["x_scale"])
    return dict(name=name, seed=seed, codes=codes, scales=scales, biases=biases, x=x, **w)


def make_shape(n_mat: int, out_dim: int, in_dim: int, nb: int, seed: int = 0,
               x_scale: float = 1.0):
    """Inputs of an arbitrary shape with the same value recipe (ragged and edge tests)."""
    codes, scales, biases = make_weights(n_mat, out_dim, in_dim, seed)
    x = make_x(n_mat, nb, in_dim, seed, x_scale)
    return dict(name=f"{n_mat}x{out_dim}x{in_dim}", seed=seed, codes=codes, scales=scales,
                biases=biases, x=x, n_mat=n_mat, out_dim=out_dim, in_dim=in_dim, nb=nb,
                x_scale=x_scale)


def make_routing(nb: int, n_experts: int, top_k: int, seed: int = 0):
    """Synthetic top-k routing of nb tokens over n_experts: each token picks top_k distinct
    experts uniformly at random, with weights drawn uniform on [0.05, 1) and divided by their
    sum in f32. Returns the union of the picked experts (``sel``, sorted ascending, i32) and
    ``wmap`` f32 [nb][len(sel)], token r's weight for slot u (0 where r did not pick it)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    picks = [rng.choice(n_experts, size=top_k, replace=False) for _ in range(nb)]
    sel = np.unique(np.concatenate(picks)).astype(np.int32)
    wmap = np.zeros((nb, sel.size), dtype=np.float32)
    for r, p in enumerate(picks):
        w = rng.uniform(0.05, 1.0, size=top_k).astype(np.float32)
        wmap[r, np.searchsorted(sel, p)] = w / w.sum(dtype=np.float32)
    return sel, wmap


def weight_bytes(n_mat: int, out_dim: int, in_dim: int) -> int:
    """Bytes of packed codes (0.5 B per weight) plus bf16 scale and bias per 64-group."""
    return n_mat * out_dim * (in_dim // 2 + 4 * (in_dim // GROUP))
