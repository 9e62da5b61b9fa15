"""Quantiser inputs whose intermediate values fall exactly on rounding ties, with the result
each tie must take. The affine host codec (host_quant_q5_row on the memra-engine
qwen4exp_gpu.rs page) rounds codes with round-half-to-even, and its f32_to_bf16_rne stores
scale and bias rounded to nearest, ties to even. Each expected value here is written down from
that rule, not computed by the oracle."""
import numpy as np

STEP = np.float32(2.0 ** -6)


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def code_tie_group(mn):
    """mn, mn + 15 * 2^-6 and mn + (k + 1/2) * 2^-6 for k = 0..14: d = 2^-6 exactly, 1/d = 64,
    and (w - mn) * 64 = k + 1/2 exactly in f32 (mn a multiple of 2^-6 of small magnitude).
    Returns the 64 values and the codes round-half-to-even gives: k + 1/2 -> the even one of
    k, k + 1; mn -> 0; mn + 15 * 2^-6 -> 15."""
    ks = np.concatenate([np.arange(15), np.arange(15), np.arange(15), np.arange(15), [0, 1]])
    vals = [np.float32(mn), np.float32(mn) + 15 * STEP] + \
        [np.float32(mn) + (np.float32(k) + np.float32(0.5)) * STEP for k in ks]
    codes = [0, 15] + [int(k + (k & 1)) for k in ks]
    return np.array(vals, np.float32), np.array(codes, np.uint8)


# d = (max - min) / 15 whose f32 pattern has a low half of exactly 0x8000: a bf16 tie.
# (upper half even: nearest-even keeps it; odd: rounds up)
D_TIES = [(0x3C808000, 0x3C80), (0x3C818000, 0x3C82)]
# group minima on bf16 ties, both signs (the sign bit does not enter the tie)
MN_TIES = [(0x3F808000, 0x3F80), (0x3F818000, 0x3F82), (0xBF808000, 0xBF80),
           (0xBF818000, 0xBF82)]


def d_tie_group(d_bits):
    """Min 0 and max 15 d (exact in f32: d has 9 significant bits), so d comes out exactly."""
    d = f32(d_bits)
    g = np.zeros(64, np.float32)
    g[-1] = np.float32(15) * d
    assert np.float32(g[-1]) / np.float32(15) == d
    return g


def mn_tie_group(mn_bits):
    mn = f32(mn_bits)
    g = np.full(64, mn, np.float32)
    g[32:] = mn + np.float32(1.0)
    return g


def tie_rows():
    """Four rows of 128 (two groups each) holding every tie group above, with the expected
    codes of the code-tie groups, and the expected scale and bias bits per group (None where
    the group is not a tie for that value)."""
    rows = np.zeros((4, 128), np.float32)
    codes = {}
    s_bits = {}
    b_bits = {}
    for gi, mn in enumerate((0.0, -0.234375)):
        v, c = code_tie_group(mn)
        rows[0, 64 * gi:64 * gi + 64] = v
        codes[(0, gi)] = c
    for gi, (db, want) in enumerate(D_TIES):
        rows[1, 64 * gi:64 * gi + 64] = d_tie_group(db)
        s_bits[(1, gi)] = want
    for t, (mb, want) in enumerate(MN_TIES):
        r, gi = 2 + t // 2, t % 2
        rows[r, 64 * gi:64 * gi + 64] = mn_tie_group(mb)
        b_bits[(r, gi)] = want
    return rows, codes, s_bits, b_bits
