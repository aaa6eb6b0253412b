"""CPU emulation of the decode kernels' fixed-point query (host-side check of
the scheme the HIP query prep implements; no GPU).

The split kernels score a token as exact integer dot products of its 4-bit
codes with the query held in fixed point: per lane slice of channels (32 at
head dim 128, 48 at 96, 16 at 64) one power-of-two scale, the query as 24-bit
integers (six signed base-16 digits) and the rotated query q' = R_K q as
20-bit integers (five digits). These tests emulate that representation in
NumPy and check (1) that the digit planes reconstruct every integer of the
range exactly, (2) the scale choice, and (3) that attention with the emulated
query stays within the parity tolerance (max-abs 2e-3, rel-L2 1e-3) when one
query channel is 100x or 1000x larger than the rest, where one 16-bit scale
per row does not.
"""
import numpy as np
import pytest

import workloads as W

QUERY_LIMBS, ROT_LIMBS = 6, 5


def qmax(nl):
    return 7 * (16 ** nl - 1) // 15


def digits(v, nl):
    """Signed base-16 digits (each -8..7) of integers v, least significant
    first, as the kernel stores them: nibble d of v + 8 (16^nl - 1)/15, minus 8."""
    u = np.asarray(v, dtype=np.int64) + 8 * (16 ** nl - 1) // 15
    return [((u >> (4 * d)) & 15) - 8 for d in range(nl)]


def slice_shift(amax, nl):
    """Largest s with amax * 2^s <= qmax(nl) (0 for amax = 0)."""
    if amax == 0:
        return 0
    e = np.frexp(amax)[1]
    s = int(np.floor(np.log2(qmax(nl)))) - e
    return s + 1 if np.ldexp(amax, s + 1) <= qmax(nl) else s


def to_fixed(x, nl, slice_len):
    """x [.., D] -> (integers, per-channel shift) with one shift per slice."""
    x = np.asarray(x, dtype=np.float64)
    shifts = np.zeros(x.shape, dtype=np.int64)
    for idx in np.ndindex(x.shape[:-1]):
        for s0 in range(0, x.shape[-1], slice_len):
            sl = x[idx][s0:s0 + slice_len]
            shifts[idx][s0:s0 + slice_len] = slice_shift(float(np.abs(sl).max()), nl)
    v = np.rint(np.ldexp(x, shifts)).astype(np.int64)
    return v, shifts


@pytest.mark.parametrize("nl", [4, 5, 6])
def test_digit_planes_reconstruct_exactly(nl):
    rng = np.random.default_rng(nl)
    m = qmax(nl)
    v = np.concatenate([rng.integers(-m, m + 1, 20000), [-m, m, 0, -1, 1, 7, 8, -8, -9]])
    ds = digits(v, nl)
    for d in ds:
        assert d.min() >= -8 and d.max() <= 7
    back = sum(d * 16 ** i for i, d in enumerate(ds))
    np.testing.assert_array_equal(back, v)
    # the 4-bit two's-complement nibble of digit d is nibble_d(u) ^ 8
    u = v + 8 * (16 ** nl - 1) // 15
    for i, d in enumerate(ds):
        np.testing.assert_array_equal(((u >> (4 * i)) & 15) ^ 8, d & 15)


@pytest.mark.parametrize("nl", [5, 6])
def test_slice_shift_is_largest_in_range(nl):
    rng = np.random.default_rng(7)
    for amax in np.concatenate([np.exp(rng.uniform(-20, 10, 500)), [1.0, 0.5, 2.0 ** -30]]):
        s = slice_shift(amax, nl)
        assert np.ldexp(amax, s) <= qmax(nl) < np.ldexp(amax, s + 1)


def test_bf16_channels_exact_down_to_2e_minus_15_of_slice_max():
    """A bf16 value whose magnitude is at least 2^-15 of its slice's largest
    has a spacing of at least the fixed-point unit, so it is stored exactly."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        big = float(W.bf16_round(rng.uniform(1, 1000)))
        x = W.bf16_round(big * np.exp2(-rng.uniform(0, 15, 31)) * rng.choice([-1, 1], 31))
        row = np.concatenate([[big], x])
        v, sh = to_fixed(row, QUERY_LIMBS, 32)
        np.testing.assert_array_equal(np.ldexp(v.astype(np.float64), -sh), row)


def _attention(q, qr, ref, res, vv, tau):
    s = (np.einsum("hd,hnd->hn", q, ref) + np.einsum("hd,hnd->hn", qr, res)) * tau
    s -= s.max(-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(-1, keepdims=True)
    return np.einsum("hn,hnd->hd", p, vv)


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("mult", [100.0, 1000.0])
def test_outlier_channel_within_tolerance(D, mult):
    """Scores = q.ref + q'.res with K/V drawn like the workloads (lognormal
    channel scales, 2% x10 outlier channels, residual sigma up to 0.4): the
    emulated fixed-point query keeps attention within the parity tolerance."""
    rng = np.random.default_rng([D, int(mult)])
    H, N = 8, 1024
    slice_len = {64: 16, 96: 48, 128: 32}[D]
    sc = np.exp(0.5 * rng.standard_normal((H, D)))
    for h in range(H):
        sc[h, rng.permutation(D)[:round(0.02 * D)]] *= 10
    ref = sc[:, None, :] * rng.standard_normal((H, N, D))
    res = 0.4 * rng.standard_normal((H, N, D))
    vv = sc[:, None, :] * rng.standard_normal((H, N, D))
    rot = np.linalg.qr(rng.standard_normal((H, D, D)))[0]
    q = rng.standard_normal((H, D)) / np.sqrt(D)
    q[np.arange(H), rng.integers(0, D, H)] *= mult
    q = W.bf16_round(q)
    qr = np.einsum("hij,hj->hi", rot, q)
    tau = 1 / np.sqrt(D)
    want = _attention(q, qr, ref, res, vv, tau)

    def emulate(nlq, nlr, sl):
        vq, sq = to_fixed(q, nlq, sl)
        vr, sr = to_fixed(qr, nlr, sl)
        return _attention(np.ldexp(vq.astype(np.float64), -sq), np.ldexp(vr.astype(np.float64), -sr),
                          ref, res, vv, tau)

    got = emulate(QUERY_LIMBS, ROT_LIMBS, slice_len)
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err <= 2e-3 / 4 and rel <= 1e-3 / 4, (err, rel)
    if mult == 1000.0:
        # one 16-bit scale per row: outside the tolerance
        old = emulate(4, 4, D)
        assert np.abs(old - want).max() > 2e-3
