"""Pins of the oracle against hand-derived worked examples (tests/golden/)."""
import numpy as np

import oracle as O


def _f16(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def _example(g, which):
    x_ref = np.array(g["x_ref"], dtype=np.float64)
    x0 = np.array(g["x_0"], dtype=np.float64)
    # [L][2][T][H][D] with K = V, one token, one head
    kv = np.stack([x0, x_ref])[:, None, None, None, :].repeat(2, axis=1)
    R = np.array(g[which + "_rot"], dtype=np.float64).reshape(4, 4)
    rot32 = np.stack([R, R])[None].astype(np.float32)          # [H=1][2][4][4]
    return kv, rot32


def test_worked_example_encode(golden):
    g = golden("worked_example_d4.txt")
    for which in ("A", "B"):
        kv, rot32 = _example(g, which)
        enc = O.encode(kv, rot32, res_bits=(2,), G=4, meta="f16")
        for k in range(2):
            assert list(enc.ref.codes[k, 0, 0]) == g["ref_codes"]
            assert enc.ref.scale[k, 0, 0, 0] == _f16(g["ref_scale_f16"])
            assert enc.ref.zero[k, 0, 0, 0] == _f16(g["ref_zero_f16"])
            assert enc.alpha[0][k, 0, 0] == _f16(g["alpha_f16"])
            assert list(enc.res[0].codes[k, 0, 0]) == g[which + "_res_codes"]
            assert enc.res[0].scale[k, 0, 0, 0] == _f16(g[which + "_res_scale_f16"])
            assert enc.res[0].zero[k, 0, 0, 0] == _f16(g[which + "_res_zero_f16"])
        assert list(O.pack_codes(enc.ref.codes[0, 0, 0], 4)) == g["ref_packed"]
        p = O.pack_codes(enc.res[0].codes[0, 0, 0], 2)
        assert list(p) == [g[which + "_res_packed"]]


def test_worked_example_reconstruct(golden):
    g = golden("worked_example_d4.txt")
    for which in ("A", "B"):
        kv, rot32 = _example(g, which)
        enc = O.encode(kv, rot32, res_bits=(2,), G=4, meta="f16")
        xh = O.reconstruct(enc, rot32)
        np.testing.assert_array_equal(xh[1, 0, 0, 0], g["x_ref_hat"])
        np.testing.assert_allclose(xh[0, 0, 0, 0], g[which + "_x0_hat"], rtol=0, atol=1e-15)


def test_worked_layout_bytes(golden):
    """Every byte of a slab holding one hand-derived token (D = 16, K = V,
    R = I; worked_layout_d16.txt): token-major K codes, V codes in their
    column-lane order, metadata and alpha."""
    lg = golden("worked_layout_d16.txt")
    x_ref = np.arange(16, dtype=np.float64)
    k = np.array([3, 2, 1, 0, 0, 1, 2, 3, 3, 2, 1, 0, 0, 1, 2, 3], dtype=np.float64)
    x0 = x_ref + (k - 1.5)
    kv = np.stack([x0, x_ref])[:, None, None, None, :].repeat(2, axis=1)     # [L][2][T][H][D]
    rot32 = np.stack([np.eye(16), np.eye(16)])[None].astype(np.float32)
    enc = O.encode(kv, rot32, res_bits=(2,), G=16, meta="f16")
    lay = O.PoolLayout(H=1, D=16, G=16, L=2, res_bits=(2,), meta="f16", num_blocks=1)
    assert lay.slab_bytes == lg["slab_bytes"][0]
    assert [lay.rec_bytes(0), lay.rec_bytes(1)] == lg["rec_bytes"]
    pool = np.zeros(lay.pool_bytes, dtype=np.uint8)
    O.write_tokens(pool, lay, enc, np.array([5]))
    want = np.zeros(lay.pool_bytes, dtype=np.uint8)
    for off, val in lg["nz"]:
        want[off] = val
    np.testing.assert_array_equal(pool, want)
    # and reading it back returns the encoded values
    for kvi in range(2):
        c, s_, z, a = O.read_pages(pool, lay, [0], 0, 0, kvi)
        assert list(c[0, 5]) == list(k) and a[0, 5] == 1.0
        assert s_[0, 5, 0] == 1.0 and z[0, 5, 0] == -1.5
        c, s_, z, a = O.read_pages(pool, lay, [0], 0, 1, kvi)
        assert list(c[0, 5]) == list(range(16)) and a is None


def test_v_code_order_hand_derived(golden):
    """Single V code positions derived by hand from the storage order,
    including a partial last word (D = 96, INT2)."""
    for D, bits, t, c, byte, bit in golden("v_code_order.txt")["pos"]:
        p = O.v_code_bits(16, D, bits)[t, c]
        assert (p // 8, p % 8) == (byte, bit), (D, bits, t, c)


def test_v_code_order_is_a_packing():
    """Every code of a page gets its own aligned field, the fields tile the
    code block exactly, and writing tokens in any slot order over stale bytes
    then reading the page returns every code (every supported width, and the
    tiny D used by hand examples)."""
    rng = np.random.default_rng(0)
    for D in (4, 16, 64, 96, 128):
        for bits in (2, 4):
            p = O.v_code_bits(16, D, bits)
            assert np.unique(p).size == p.size and (p % bits == 0).all()
            assert p.min() == 0 and p.max() == 16 * D * bits - bits
            lay = O.PoolLayout(H=1, D=D, G=D, L=1, res_bits=(), meta="f16", num_blocks=2, direct_bits=(bits,))
            codes = rng.integers(0, 1 << bits, size=(2, 16, 1, D)).astype(np.uint8)
            q = O.Quantized(codes=codes, scale=np.ones((2, 16, 1, 1)), zero=np.zeros((2, 16, 1, 1)),
                            u=codes.astype(np.float64), bits=bits)
            enc = O.DirectEncoded(q=[q], G=D, meta="f16")
            pool = np.full(lay.pool_bytes, 0xA5, dtype=np.uint8)          # stale bytes get overwritten
            slots = 16 + rng.permutation(16)                                # token i -> page 1, offset slots[i]-16
            O.write_tokens(pool, lay, enc, slots)
            for kvi in range(2):
                c, *_ = O.read_pages(pool, lay, [1], 0, 0, kvi)
                np.testing.assert_array_equal(c[0, slots - 16], codes[kvi, :, 0])


def test_worked_attention_closed_form():
    # scores 0, ln 2, ln 5 -> softmax 1/8, 2/8, 5/8 (tau = 1/sqrt(4) = 0.5, q = [2,0,0,0])
    q = np.array([2.0, 0, 0, 0])
    K = np.array([[0, 1, 2, 3], [np.log(2), -1, 0, 0], [np.log(5), 4, 4, 4]], dtype=np.float64)
    V = np.array([[8.0, 0, 0, 1], [0, 8, 0, 1], [0, 0, 8, 1]])
    o = O.attention(q, K[:2], V[:2], 0.5, tail_k=K[2], tail_v=V[2])
    np.testing.assert_allclose(o, [1.0, 2.0, 5.0, 1.0], rtol=0, atol=1e-13)


def test_worked_example_rounded_alpha(golden):
    g = golden("worked_example_d4.txt")
    x_ref = np.array(g["C_x_ref"], dtype=np.float64)
    x0 = np.array(g["C_x_0"], dtype=np.float64)
    kv = np.stack([x0, x_ref])[:, None, None, None, :].repeat(2, axis=1)
    rot32 = np.stack([np.eye(4), np.eye(4)])[None].astype(np.float32)
    enc = O.encode(kv, rot32, res_bits=(2,), G=4, meta="f16")
    assert enc.alpha[0][0, 0, 0] == _f16(g["C_alpha_f16"])
    assert list(enc.res[0].codes[0, 0, 0]) == g["C_res_codes"]
    assert enc.res[0].scale[0, 0, 0, 0] == _f16(g["C_res_scale_f16"])
    assert enc.res[0].zero[0, 0, 0, 0] == _f16(g["C_res_zero_f16"])


def test_worked_layout_offsets(golden):
    lg = golden("worked_layout_d16.txt")
    lay = O.PoolLayout(H=2, D=16, G=16, L=2, res_bits=(2,), meta="f16", num_blocks=3)
    assert lay.pool_bytes == lg["pool_bytes"][0]
    for blk, head, loop, kv, off in lg["offset"]:
        assert lay.record_offset(blk, head, loop, kv) == off


# ------------------------------------------------ rotation-fitting objective
def test_rotation_objective_hand_derived(golden):
    """Objective of a non-symmetric rotation on two rows, derived by hand
    (tests/golden/rotation_objective_d4.txt): pins that the rows are rotated
    as R d (not R^T d) before quantization."""
    g = golden("rotation_objective_d4.txt")
    S = np.array(g["S_rot"], dtype=np.float64).reshape(4, 4)
    rows = np.array(g["obj_rows"], dtype=np.float64).reshape(2, 4)
    assert O.rotation_quant_error(rows, S, 2, 4, "f16") == g["obj_value"][0]
    # the per-row quantization behind it
    q = O.quantize(rows @ S.T, 2, 4, "f16")
    np.testing.assert_array_equal(q.codes[0], g["obj_row1_codes"])
    np.testing.assert_array_equal(q.codes[1], g["obj_row2_codes"])
    f16 = lambda v: np.array([v], np.uint16).view(np.float16).astype(np.float64)[0]
    assert q.scale[0, 0] == f16(g["obj_row1_scale_f16"][0]) and q.zero[0, 0] == f16(g["obj_row1_zero_f16"][0])
    assert q.scale[1, 0] == f16(g["obj_row2_scale_f16"][0]) and q.zero[1, 0] == f16(g["obj_row2_zero_f16"][0])
    # the transposed rotation gives another value (the fixture discriminates)
    assert O.rotation_quant_error(rows, S.T, 2, 4, "f16") != g["obj_value"][0]


def test_one_procrustes_step_hand_derived(golden):
    """One alternation step from R0 = S on rows S^T e_j: every rotated row is a
    unit vector, quantized to (4095/4096) e_j, so M = (4095/4096) S and the
    polar factor is S again; history [2^-24, 2^-24]."""
    g = golden("rotation_objective_d4.txt")
    S = np.array(g["S_rot"], dtype=np.float64).reshape(4, 4)
    rows = np.array(g["step_rows"], dtype=np.float64).reshape(4, 4)
    np.testing.assert_array_equal(rows, (S.T @ np.eye(4)).T)      # d_j = S^T e_j
    Y = rows @ S.T
    q = O.quantize(Y, 2, 4, "f16")
    Yh = O.dequantize(q.codes, q.scale, q.zero, 4)
    np.testing.assert_array_equal(Yh, g["step_yhat_scale"][0] * np.eye(4))
    M = Yh.T @ rows
    np.testing.assert_array_equal(M, g["step_M_scale"][0] * S)
    np.testing.assert_allclose(O.procrustes(M), S, rtol=0, atol=1e-15)
    R, hist = O.fit_rotation(rows, S, 2, 4, "f16", 1)
    np.testing.assert_array_equal(hist, g["step_history"])
    np.testing.assert_array_equal(R, S)
    # a full-rank M = R_true * (symmetric positive definite) has polar factor R_true
    P = np.diag([2.25, 9.0, 0.5625, 36.0])
    np.testing.assert_allclose(O.procrustes(S @ P), S, rtol=0, atol=1e-15)
