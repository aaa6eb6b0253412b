"""Pins of the fp64 oracle against closed forms, invariants and library routines.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed rotation, a wrong rounding mode) fails it.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W


# --------------------------------------------------------------- rounding
def _f16_nearest_even(x: float) -> float:
    """RNE to binary16 by exact rational comparison of the two neighbours."""
    h = np.float16(x)                      # a candidate; check it against its neighbours
    cands = {float(h), float(np.nextafter(h, np.float16(np.inf))), float(np.nextafter(h, np.float16(-np.inf)))}
    cands = {c for c in cands if np.isfinite(c)}
    fx = Fraction(x)
    best = sorted(cands, key=lambda c: (abs(Fraction(c) - fx),
                                         int(np.array([c], np.float16).view(np.uint16)[0]) & 1))
    return best[0]


def test_meta_round_is_rne_from_double():
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(400) * 10.0 ** rng.integers(-6, 4, 400))
    # exact ties between fp16 neighbours (odd multiples of half a spacing) and
    # values a hair off a tie, which a double->float->half path can misround
    for e in (-3, 0, 2):
        sp = 2.0 ** (e - 10)
        for k in (1, 3, 5, 1023):
            t = 2.0 ** e + (k + 0.5) * sp
            xs += [t, np.nextafter(t, 0), np.nextafter(t, 10)]
    xs += [2.0 ** -24 * 1.5, 2.0 ** -25, 65504.0, 6.1e-5]
    got = O.meta_round(np.array(xs), "f16")
    for x, g in zip(xs, got):
        assert g == _f16_nearest_even(float(x)), x


# ------------------------------------------------------------- least squares
def test_alpha_is_least_squares_minimiser():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 64))
    ref = rng.standard_normal((50, 64)) * 3
    a = O.ls_alpha(x, ref)
    # normal equation: the residual is orthogonal to the reference
    resid = x - a[:, None] * ref
    dots = np.abs(np.sum(resid * ref, -1)) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(ref, axis=-1))
    assert dots.max() < 1e-12
    # and any other scale is worse
    err = lambda s: np.sum((x - s[:, None] * ref) ** 2, -1)
    for eps in (1e-3, -1e-3, 0.1):
        assert np.all(err(a + eps) > err(a))
    # against a least-squares library solve, column by column
    for i in range(5):
        sol = np.linalg.lstsq(ref[i][:, None], x[i], rcond=None)[0][0]
        assert abs(sol - a[i]) < 1e-13 * max(1, abs(sol))


def test_alpha_special_cases():
    ref = np.array([1.0, -2.0, 0.5, 4.0])
    assert O.ls_alpha(0.75 * ref, ref) == 0.75
    assert O.ls_alpha(ref, ref) == 1.0
    assert O.ls_alpha(ref, np.zeros(4)) == 0.0


def test_alpha_recovers_generator_scale():
    w = W.get(1).replace(batch=2, context=64, heads=4)
    st = W.structure(w)
    kv = W.kv_numpy(w, batch=2, context=64, st=st)          # [L][2][B][N+1][H][D]
    ref = kv[-1]
    for l in range(w.loops - 1):
        a = O.ls_alpha(kv[l], ref)                           # [2][B][N+1][H]
        true = st["alpha"][l][:, None, None, :]
        bound = 6 * st["sigma"][l] / np.linalg.norm(ref, axis=-1) + 2.0 ** -7
        assert np.all(np.abs(a - true) <= bound)


# ------------------------------------------------------------------ rotation
def test_generator_rotations_orthogonal():
    for key in (0, 1, 3):
        st = W.structure(W.get(key).replace(heads=2))
        R = st["rot64"]
        I = np.eye(R.shape[-1])
        for h in range(R.shape[0]):
            for kv in range(2):
                assert np.abs(R[h, kv].T @ R[h, kv] - I).max() <= 1e-12
                assert np.abs(R[h, kv] @ R[h, kv].T - I).max() <= 1e-12
        R32 = st["rot32"].astype(np.float64)
        assert np.abs(np.einsum("hkji,hkjl->hkil", R32, R32) - I).max() < 1e-6


# ----------------------------------------------------------------- quantizer
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("meta", ["f16", "f32"])
def test_quantizer_levels_and_error(bits, meta):
    rng = np.random.default_rng(bits)
    y = rng.standard_normal((300, 128)) * np.exp(rng.standard_normal((300, 1)))
    G = 32
    q = O.quantize(y, bits, G, meta)
    qmax = (1 << bits) - 1
    cg = q.codes.reshape(300, 4, G)
    yg = y.reshape(300, 4, G)
    # min maps to code 0 and max to the top code in every group
    imin, imax = yg.argmin(-1), yg.argmax(-1)
    assert np.all(np.take_along_axis(cg, imin[..., None], -1) == 0)
    assert np.all(np.take_along_axis(cg, imax[..., None], -1) == qmax)
    # every level is used across the tensor
    assert set(np.unique(q.codes)) == set(range(qmax + 1))
    # per-element error: half a step, plus the rounding of step and zero
    deq = O.dequantize(q.codes, q.scale, q.zero, G)
    dt = np.float16 if meta == "f16" else np.float32
    ulp = lambda v: np.spacing(np.abs(v).astype(dt)).astype(np.float64)
    bound = (q.scale / 2 + (1 << bits) * ulp(q.scale) + ulp(q.zero))
    err = np.abs(y - deq).reshape(300, 4, G)
    assert np.all(err <= bound[..., None] * (1 + 1e-12))
    # codes are the nearest level to (y - z)/s
    inner = (q.u >= 0) & (q.u <= qmax)
    assert np.all(np.abs(q.u[inner] - q.codes[inner]) <= 0.5)


def test_quantizer_round_half_even_and_degenerate():
    # group [0, 1, 2, 3] * 1/3 scale: u values exactly 0..3
    y = np.array([[0.0, 0.5, 1.5, 3.0]])
    q = O.quantize(y, 2, 4, "f32")                       # step 1.0, zero 0
    assert q.scale[0, 0] == 1.0 and list(q.codes[0]) == [0, 0, 2, 3]   # 0.5 -> 0, 1.5 -> 2 (ties to even)
    q = O.quantize(np.full((1, 8), 2.5), 4, 8, "f16")
    assert q.scale[0, 0] == 0 and q.zero[0, 0] == 2.5 and not q.codes.any()
    assert np.all(O.dequantize(q.codes, q.scale, q.zero, 8) == 2.5)


def test_quantizer_group_independence():
    # groups must not mix: changing one group leaves the others' codes alone
    rng = np.random.default_rng(3)
    y = rng.standard_normal((1, 128))
    q1 = O.quantize(y, 2, 32, "f16")
    y2 = y.copy()
    y2[0, 40:64] *= 100
    q2 = O.quantize(y2, 2, 32, "f16")
    np.testing.assert_array_equal(q1.codes[0, :32], q2.codes[0, :32])
    np.testing.assert_array_equal(q1.codes[0, 64:], q2.codes[0, 64:])
    assert not np.array_equal(q1.codes[0, 32:64], q2.codes[0, 32:64])


# ------------------------------------------------------------------- encode
def _small(key, **kw):
    w = W.get(key).replace(**kw)
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)                                 # [L][2][B][N+1][H][D]
    L, _, B, N1, H, D = kv.shape
    kvt = kv.reshape(L, 2, B * N1, H, D)
    return w, st, kvt


@pytest.mark.parametrize("key,kw", [(0, {}), (1, dict(batch=1, context=40, heads=3)),
                                    (3, dict(batch=1, context=20, heads=2))])
def test_reconstruction_bound(key, kw):
    w, st, kv = _small(key, **kw)
    enc = O.encode(kv, st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    xh = O.reconstruct(enc, st["rot32"])
    G = w.group_size
    D = w.head_dim
    eref = np.abs(xh[-1] - kv[-1])
    sref = np.repeat(enc.ref.scale, G, axis=-1)
    assert np.all(eref <= sref / 2 * (1 + 1e-3) + 1e-2 * sref)
    R = st["rot32"].astype(np.float64)
    for l in range(w.loops - 1):
        q = enc.res[l]
        a = enc.alpha[l]
        d = kv[l] - a[..., None] * kv[-1]
        r = np.einsum("hkij,kthj->kthi", R, d)
        deq = O.dequantize(q.codes, q.scale, q.zero, G)
        e_r = np.abs(deq - r).max(-1)
        bound = np.abs(a) * eref.max(-1) + np.sqrt(D) * e_r * (1 + 1e-6) + 1e-6 * np.abs(d).max(-1) * D
        err = np.abs(xh[l] - kv[l]).max(-1)
        assert np.all(err <= bound + 1e-12)
        # residual range is far below the raw range (the point of the method)
        assert np.median(np.repeat(q.scale, G, -1)) < 0.5 * np.median(sref)


def test_reconstruction_detects_transposed_rotation():
    w, st, kv = _small(1, batch=1, context=16, heads=2)
    enc = O.encode(kv, st["rot32"], (4, 4, 4), w.group_size, w.meta_dtype)
    a = enc.alpha[0][..., None]
    d = kv[0] - a * kv[-1]                       # what the rotated residual encodes

    def part(rot):                               # residual part of the reconstruction
        xh = O.reconstruct(enc, rot)
        return xh[0] - a * xh[-1]
    rms = lambda e: np.sqrt(np.mean(e ** 2))
    good = rms(part(st["rot32"]) - d)
    bad = rms(part(np.swapaxes(st["rot32"], -1, -2)) - d)
    assert bad > 4 * good


def test_identical_loops_give_zero_point_residual():
    w, st, kv = _small(1, batch=1, context=24, heads=2)
    kv = kv.copy()
    kv[0] = kv[-1]
    enc = O.encode(kv, st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    assert np.all(enc.alpha64[0] == 1.0) and np.all(enc.alpha[0] == 1.0)
    q = enc.res[0]
    assert not q.codes.any() and not q.scale.any() and not q.zero.any()
    xh = O.reconstruct(enc, st["rot32"])
    np.testing.assert_array_equal(xh[0], xh[-1])


def test_residual_rounding_exact_in_float64():
    # d = x - alpha*ref is exact for bf16 x/ref and fp16 alpha: equals an fma
    w, st, kv = _small(1, batch=1, context=30, heads=2)
    enc = O.encode(kv, st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    a = enc.alpha[0][..., None]
    d = kv[0] - a * kv[-1]
    exact = [Fraction(float(x)) - Fraction(float(al)) * Fraction(float(r))
             for x, al, r in zip(kv[0].ravel()[:500], np.broadcast_to(a, kv[0].shape).ravel()[:500], kv[-1].ravel()[:500])]
    assert all(Fraction(float(v)) == e for v, e in zip(d.ravel()[:500], exact))


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_exhaustive(bits):
    allb = np.arange(256, dtype=np.uint8)[:, None]
    c = O.unpack_codes(allb, bits)
    assert c.shape == (256, 8 // bits) and c.max() == (1 << bits) - 1
    np.testing.assert_array_equal(O.pack_codes(c, bits), allb)


def test_pack_spec_vectors():
    assert list(O.pack_codes(np.array([1, 2, 3, 4, 15, 0, 7, 8]), 4)) == [0x21, 0x43, 0x0F, 0x87]
    assert list(O.pack_codes(np.array([1, 2, 3, 0, 3, 3, 3, 3]), 2)) == [0x39, 0xFF]


# ---------------------------------------------------------- pool and paging
def test_pool_roundtrip_and_gather():
    w = W.get(3).replace(batch=2, context=37, heads=3)
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)                                 # [L][2][B][N+1][H][D]
    L, _, B, N1, H, D = kv.shape
    table, nblk = W.block_table(w, shuffled=True)
    lay = O.PoolLayout(H, D, w.group_size, L, w.res_bits, w.meta_dtype, nblk)
    assert all(lay.rec_bytes(l) % 16 == 0 for l in range(L))
    pool = np.zeros(lay.pool_bytes, np.uint8)
    pos = np.tile(np.arange(N1), (B, 1))
    slots = W.slot_mapping(table, pos).reshape(-1)
    kvt = kv.reshape(L, 2, B * N1, H, D)
    enc = O.encode(kvt, st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    O.write_tokens(pool, lay, enc, slots)
    for b in range(B):
        for h in range(H):
            for l in range(L):
                for k in range(2):
                    c, s, z, a = O.gather_sequence(pool, lay, table[b], N1, h, l, k)
                    q = enc.ref if l == L - 1 else enc.res[l]
                    sl = slice(b * N1, (b + 1) * N1)
                    np.testing.assert_array_equal(c, q.codes[k, sl, h])
                    np.testing.assert_array_equal(s, q.scale[k, sl, h])
                    np.testing.assert_array_equal(z, q.zero[k, sl, h])
                    if l < L - 1:
                        np.testing.assert_array_equal(a, enc.alpha[l][k, sl, h])
            xh = O.reconstruct(enc, st["rot32"])
            for l in range(L):
                Kh, Vh = O.reconstruct_sequence(pool, lay, table[b], N1, h, l, st["rot32"][h])
                np.testing.assert_allclose(Kh, xh[l, 0, b * N1:(b + 1) * N1, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(Vh, xh[l, 1, b * N1:(b + 1) * N1, h], rtol=0, atol=1e-12)


# ----------------------------------------------------------------- attention
def test_attention_against_library_softmax():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    for n in (1, 2, 7, 300):
        q = rng.standard_normal(64)
        K = rng.standard_normal((n, 64)) * 3
        V = rng.standard_normal((n, 64))
        tau = 0.125
        o = O.attention(q, K, V, tau)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], scale=tau)[0, 0, 0].numpy()
        np.testing.assert_allclose(o, t, rtol=1e-12, atol=1e-12)


def test_attention_invariants():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((50, 16))
    V = rng.standard_normal((50, 16))
    q = rng.standard_normal(16)
    np.testing.assert_allclose(O.attention(np.zeros(16), K, V, 0.25), V.mean(0), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(O.attention(q, K[:1], V[:1], 0.25), V[0])
    perm = rng.permutation(50)
    np.testing.assert_allclose(O.attention(q, K[perm], V[perm], 0.25), O.attention(q, K, V, 0.25), atol=1e-14)
    assert not O.attention(q, K[:0], V[:0], 0.25).any()
    # tail token is just one more key
    np.testing.assert_allclose(O.attention(q, K[:-1], V[:-1], 0.25, K[-1], V[-1]),
                               O.attention(q, K, V, 0.25), atol=1e-14)
    # two keys: p1 = sigmoid(score difference)
    o = O.attention(q, K[:2], V[:2], 0.25)
    p1 = 1 / (1 + np.exp(-0.25 * (K[1] - K[0]) @ q))
    np.testing.assert_allclose(o, (1 - p1) * V[0] + p1 * V[1], atol=1e-14)


def test_decode_attention_matches_dense_on_reconstruction():
    # attention over the pool equals attention over the reconstruction of the
    # same encoded tokens (pool indexing, paging and per-loop reconstruction)
    w = W.get(1).replace(batch=2, context=33, heads=2)
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)
    L, _, B, N1, H, D = kv.shape
    N = N1 - 1
    table, nblk = W.block_table(w, shuffled=True)
    lay = O.PoolLayout(H, D, w.group_size, L, w.res_bits, w.meta_dtype, nblk)
    pool = np.zeros(lay.pool_bytes, np.uint8)
    slots = W.slot_mapping(table, np.tile(np.arange(N), (B, 1))).reshape(-1)
    enc = O.encode(kv[:, :, :, :N].reshape(L, 2, B * N, H, D), st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    O.write_tokens(pool, lay, enc, slots)
    xh = O.reconstruct(enc, st["rot32"]).reshape(L, 2, B, N, H, D)
    qs = W.queries_numpy(w)
    tau = 1 / np.sqrt(D)
    for l in range(L):
        out = O.decode_attention(pool, lay, l, qs[l], st["rot32"], table, [N] * B, tau,
                                 kv[l, 0, :, N], kv[l, 1, :, N])
        for b in range(B):
            for h in range(H):
                ref = O.attention(qs[l, b, h], xh[l, 0, b, :, h], xh[l, 1, b, :, h], tau,
                                  kv[l, 0, b, N, h], kv[l, 1, b, N, h])
                np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_bf16_baseline_attention():
    w = W.get(1).replace(batch=2, context=21, heads=2)
    kv = W.kv_numpy(w)
    L, _, B, N1, H, D = kv.shape
    N = N1 - 1
    table, nblk = W.block_table(w)
    kc = np.zeros((nblk, H, 16, D))
    vc = np.zeros((nblk, H, 16, D))
    slots = W.slot_mapping(table, np.tile(np.arange(N), (B, 1))).reshape(-1)
    O.bf16_pool_write(kc, vc, kv[1, :, :, :N].reshape(2, B * N, H, D), slots)
    q = W.queries_numpy(w)[1]
    out = O.bf16_decode_attention(kc, vc, q, table, [N] * B, 0.1)
    for b in range(B):
        for h in range(H):
            ref = O.attention(q[b, h], kv[1, 0, b, :N, h], kv[1, 1, b, :N, h], 0.1)
            np.testing.assert_allclose(out[b, h], ref, atol=1e-13)


# ------------------------------------------------ direct per-loop baseline
def test_direct_layout_hand_derived():
    """Direct mode record bytes derived by hand: D=4, G=4, loops (INT2, INT4),
    fp16 metadata, one block, one head. Loop 0 record: 16 tokens x 1 B codes +
    16 x (scale, zero) x 2 B = 80 B (no alpha); loop 1: 16 x 2 B + 64 = 96 B.
    Token at slot 5 of loop 0, K = [0, 1, 2, 3]: scale 1, zero 0, codes
    0,1,2,3 -> one byte 0b11_10_01_00 = 0xE4 at record byte 5; scale 1.0 is
    f16 0x3C00 and zero 0x0000 at record bytes 16 + 5*4 .. +3 (little
    endian: 00 3C 00 00)."""
    lay = O.PoolLayout(1, 4, 4, 2, (), "f16", 1, direct_bits=(2, 4))
    assert (lay.rec_bytes(0), lay.rec_bytes(1), lay.slab_bytes) == (80, 96, 352)
    assert lay.record_offset(0, 0, 0, 1) == 80 and lay.record_offset(0, 0, 1, 0) == 160
    kv = np.zeros((2, 2, 1, 1, 4))
    kv[0, 0, 0, 0] = [0.0, 1.0, 2.0, 3.0]
    kv[0, 1, 0, 0] = [5.0, 5.0, 5.0, 5.0]          # constant group: scale 0, zero 5 (0x4500)
    kv[1, 0, 0, 0] = [0.0, 15.0, 3.0, 7.0]         # INT4: scale 1, codes 0, 15, 3, 7
    enc = O.encode_direct(kv, (2, 4), 4, "f16")
    pool = np.zeros(lay.pool_bytes, np.uint8)
    O.write_tokens(pool, lay, enc, np.array([5]))
    assert pool[5] == 0xE4
    assert list(pool[16 + 20: 16 + 24]) == [0x00, 0x3C, 0x00, 0x00]
    assert pool[80 + 5] == 0x00                               # V: all codes 0
    assert list(pool[80 + 16 + 20: 80 + 16 + 24]) == [0x00, 0x00, 0x00, 0x45]
    assert list(pool[160 + 10: 160 + 12]) == [0xF0, 0x73]     # codes (0,15),(3,7) low nibble first
    assert list(pool[160 + 32 + 20: 160 + 32 + 24]) == [0x00, 0x3C, 0x00, 0x00]
    # nothing else written
    touched = {5, 36, 37, 38, 39, 85, 116, 117, 118, 119, 170, 171, 212, 213, 214, 215}
    assert all(pool[i] == 0 for i in range(lay.pool_bytes) if i not in touched)


def test_direct_reconstruction_and_attention_by_hand():
    """Values on the quantization grid (INT2 steps 1 and 2, fp16-exact)
    reconstruct exactly in direct mode, and decode attention over them is the
    softmax of the hand-computed scores."""
    D, L = 4, 2
    lay = O.PoolLayout(1, D, 4, L, (), "f16", 2, direct_bits=(2, 2))
    K = np.array([[0.0, 1.0, 2.0, 3.0], [3.0, 2.0, 1.0, 0.0], [1.0, 1.0, 4.0, 4.0]])
    V = np.array([[2.0, 0.0, 0.0, 6.0], [0.0, 2.0, 4.0, 6.0], [6.0, 6.0, 0.0, 0.0]])
    # loop 0 holds K/V, the final loop something else: loop 0 must read only its own record
    kv = np.random.default_rng(3).normal(size=(L, 2, 3, 1, D))
    kv[0, 0, :, 0] = K
    kv[0, 1, :, 0] = V
    enc = O.encode_direct(kv, (2, 2), 4, "f16")
    pool = np.zeros(lay.pool_bytes, np.uint8)
    table = np.array([[1, 0]])
    O.write_tokens(pool, lay, enc, table[0, 0] * 16 + np.arange(3))
    Kh, Vh = O.reconstruct_sequence(pool, lay, table[0], 3, 0, 0, None)
    np.testing.assert_array_equal(Kh, K)
    np.testing.assert_array_equal(Vh, V)
    q = np.array([[[0.5, -1.0, 0.25, 1.0]]])
    tau = 0.5
    s = tau * np.array([0.0 - 1.0 + 0.5 + 3.0, 1.5 - 2.0 + 0.25 + 0.0, 0.5 - 1.0 + 1.0 + 4.0])
    p = np.exp(s - s.max())
    want = (p[:, None] * V).sum(0) / p.sum()
    got = O.decode_attention(pool, lay, 0, q, None, table, [3], tau)[0, 0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


# ---------------------------------------------------------- rotation fitting
def test_procrustes_matches_brute_force_in_2d():
    """The Procrustes step against a search over every 2-D orthogonal matrix
    (rotations and reflections by angle): both maximize trace(R^T M)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        M = rng.normal(size=(2, 2))
        R = O.procrustes(M)
        th = np.linspace(0, 2 * np.pi, 2000001)
        c, s_ = np.cos(th), np.sin(th)
        # trace(Q^T M) for Q = [[c, -s], [s, c]] and for the reflection [[c, s], [s, -c]]
        rot = c * M[0, 0] + s_ * M[1, 0] - s_ * M[0, 1] + c * M[1, 1]
        ref = c * M[0, 0] + s_ * M[1, 0] + s_ * M[0, 1] - c * M[1, 1]
        best = float(max(rot.max(), ref.max()))
        assert abs(float(np.trace(R.T @ M)) - best) < 1e-8
        np.testing.assert_allclose(R @ R.T, np.eye(2), atol=1e-12)


def test_fit_rotation_orthogonal_and_never_worse():
    """The fitted R is orthogonal to 1e-12 and its error is the minimum of
    the trajectory, no larger than the starting rotation's; on residuals with
    outlier channels the fit lowers the error."""
    w = W.get(1)
    st = W.structure(w)
    rng = np.random.default_rng(5)
    D = w.head_dim
    scale = np.ones(D)
    scale[rng.permutation(D)[:3]] = 10.0
    samples = rng.normal(size=(1024, D)) * scale * 0.1
    R0 = st["rot32"][0, 0]
    R, hist = O.fit_rotation(samples, R0, 2, D, "f16", 8)
    np.testing.assert_allclose(R @ R.T, np.eye(D), atol=1e-12)
    err = O.rotation_quant_error(samples, R, 2, D, "f16")
    assert err == min(hist) and err <= hist[0]
    assert err < hist[0]


# ----------------------------------------------------------- chunked prefill
def test_chunk_attention_against_library_masked_softmax():
    """Chunked attention over the packed cache equals torch's scaled-dot-
    product attention (fp64, CPU) with an explicit mask: every cached token
    visible, chunk tokens causally (query i sees chunk tokens 0..i)."""
    import torch
    w = W.get(1).replace(batch=2, heads=2, context=37)
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)                                 # [L][2][B][N+1][H][D]
    L, _, B, N1, H, D = kv.shape
    N = N1 - 1
    table, nblk = W.block_table(w, shuffled=True)
    lay = O.PoolLayout(H, D, w.group_size, L, w.res_bits, w.meta_dtype, nblk)
    pool = np.zeros(lay.pool_bytes, np.uint8)
    pos = np.tile(np.arange(N), (B, 1))
    slots = W.slot_mapping(table, pos).reshape(-1)
    enc = O.encode(kv[:, :, :, :N].reshape(L, 2, B * N, H, D), st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    O.write_tokens(pool, lay, enc, slots)
    rng = np.random.default_rng(5)
    C = 5
    q = rng.normal(size=(B, C, H, D)) / np.sqrt(D)
    ck = rng.normal(size=(B, C, H, D))
    cv = rng.normal(size=(B, C, H, D))
    seq = [N, 11]
    tau = 1 / np.sqrt(D)
    for l in (0, L - 1):
        got = O.chunk_attention(pool, lay, l, q, st["rot32"], table, seq, tau, ck, cv)
        for b in range(B):
            for h in range(H):
                K, V = O.reconstruct_sequence(pool, lay, table[b], seq[b], h, l, st["rot32"][h])
                Kall = torch.from_numpy(np.concatenate([K, ck[b, :, h]]))
                Vall = torch.from_numpy(np.concatenate([V, cv[b, :, h]]))
                n = seq[b]
                mask = torch.zeros((C, n + C), dtype=torch.bool)
                mask[:, :n] = True
                mask[:, n:] = torch.tril(torch.ones((C, C), dtype=torch.bool))
                want = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[b, :, h])[None], Kall[None], Vall[None], attn_mask=mask[None], scale=tau)[0]
                np.testing.assert_allclose(got[b, :, h], want.numpy(), rtol=0, atol=1e-12)


def test_chunk_attention_special_cases():
    """C = 1 is decode attention with the chunk token as the current token;
    with nothing cached, the first query returns the first chunk value
    exactly and the last query sees every chunk token."""
    w = W.get(0)
    st = W.structure(w)
    kv = W.kv_numpy(w, st=st)
    L, _, B, N1, H, D = kv.shape
    N = N1 - 1
    table, nblk = W.block_table(w)
    lay = O.PoolLayout(H, D, w.group_size, L, w.res_bits, w.meta_dtype, nblk)
    pool = np.zeros(lay.pool_bytes, np.uint8)
    enc = O.encode(kv[:, :, 0, :N], st["rot32"], w.res_bits, w.group_size, w.meta_dtype)
    O.write_tokens(pool, lay, enc, np.arange(N))
    q = W.queries_numpy(w)                                      # [L][B][H][D]
    tau = 1 / np.sqrt(D)
    for l in range(L):
        want = O.decode_attention(pool, lay, l, q[l], st["rot32"], table, [N], tau, kv[l, 0, :, N], kv[l, 1, :, N])
        got = O.chunk_attention(pool, lay, l, q[l][:, None], st["rot32"], table, [N], tau,
                                kv[l, 0, :, N][:, None], kv[l, 1, :, N][:, None])
        np.testing.assert_array_equal(got[:, 0], want)
    rng = np.random.default_rng(2)
    C = 4
    qc, ck, cv = (rng.normal(size=(1, C, H, D)) for _ in range(3))
    got = O.chunk_attention(pool, lay, 0, qc, st["rot32"], table, [0], tau, ck, cv)
    np.testing.assert_array_equal(got[0, 0, 0], cv[0, 0, 0])
    s = tau * ck[0, :, 0] @ qc[0, C - 1, 0]
    p = np.exp(s - s.max())
    np.testing.assert_allclose(got[0, C - 1, 0], p @ cv[0, :, 0] / p.sum(), rtol=0, atol=1e-14)
