"""rq_fit_rotation (host code of the library) against the oracle's fit: the
same alternation of quantization and orthogonal Procrustes steps from the
same start gives the same error trajectory and the same rotation."""
import numpy as np
import pytest

import oracle as O
import workloads as W

import looped_transformer_decode_rq_amd as R


def _outlier_residuals(D, n, seed):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.normal(0, 0.5, D))
    scale[rng.permutation(D)[: max(1, round(0.02 * D))]] *= 10.0
    return (rng.normal(size=(n, D)) * scale * 0.1).astype(np.float32)


@pytest.mark.parametrize("D,G,bits,meta", [(64, 64, 2, "f16"), (128, 128, 2, "f16"), (64, 16, 4, "f32"),
                                           (96, 96, 4, "f16")])
def test_fit_matches_oracle(D, G, bits, meta):
    x = _outlier_residuals(D, 512, D + bits)
    rng = np.random.default_rng(7)
    q, r = np.linalg.qr(rng.normal(size=(D, D)))
    R0 = (q * np.sign(np.diag(r))).astype(np.float32)
    Rl, obj_l = R.fit_rotation(x, R0, bits, G, meta, iters=3)
    Ro, obj_o = O.fit_rotation(x.astype(np.float64), R0, bits, G, meta, 3)
    np.testing.assert_allclose(obj_l, obj_o, rtol=1e-9, atol=0)
    np.testing.assert_allclose(Rl, Ro.astype(np.float32), rtol=0, atol=2e-6)
    np.testing.assert_allclose(Rl.astype(np.float64) @ Rl.T.astype(np.float64), np.eye(D), atol=1e-5)
    assert obj_l.min() <= obj_l[0]


def test_rotation_and_fit_on_outlier_residuals():
    """On residuals with a few x10 channels: a random orthogonal rotation
    lowers the INT2 quantization error several times against no rotation
    (the outliers' range is spread over all channels); the fit lowers the
    error on its own rows, and on held-out rows it stays within a few percent
    of the random start (on such i.i.d. rows a random rotation is already
    about as good as an orthogonal one gets for this quantizer)."""
    D = 128
    x = _outlier_residuals(D, 12288, 1)
    train, held = x[:8192], x[8192:].astype(np.float64)
    st = W.structure(W.get(1))
    R0 = st["rot32"][0, 0]
    e_id = O.rotation_quant_error(held, np.eye(D), 2, D, "f16")
    e0 = O.rotation_quant_error(held, R0, 2, D, "f16")
    assert e_id > 2.0 * e0
    Rf, obj = R.fit_rotation(train, R0, 2, D, "f16", iters=6)
    assert obj.min() < obj[0]
    e1 = O.rotation_quant_error(held, Rf, 2, D, "f16")
    assert e1 < 1.05 * e0


def test_fit_validation():
    import ctypes
    L = R.lib()
    x = np.zeros((4, 64), np.float32)
    r = np.eye(64, dtype=np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.rq_fit_rotation(None, 4, 64, 2, 64, 1, p(r), 1, p(r), None) == -1
    assert L.rq_fit_rotation(p(x), 0, 64, 2, 64, 1, p(r), 1, p(r), None) == -2
    assert L.rq_fit_rotation(p(x), 4, 64, 3, 64, 1, p(r), 1, p(r), None) == -3
    assert L.rq_fit_rotation(p(x), 4, 64, 2, 48, 1, p(r), 1, p(r), None) == -2
    assert L.rq_fit_rotation(p(x), 4, 256, 2, 64, 1, p(r), 1, p(r), None) == -2


@pytest.mark.parametrize("n,zero_channels", [(512, 4), (40, 0), (40, 3)])
def test_fit_rank_deficient_stays_orthogonal(n, zero_channels):
    """Calibration rows with channels that are zero in every row, or fewer
    rows than channels: M has rank < D, the polar factor is not unique there,
    and the fit must still return an orthogonal rotation whose action on the
    rows (hence every objective value) equals the oracle's."""
    D = 64
    x = _outlier_residuals(D, n, 11)
    x[:, np.random.default_rng(3).permutation(D)[:zero_channels]] = 0.0
    rng = np.random.default_rng(5)
    q, r = np.linalg.qr(rng.normal(size=(D, D)))
    R0 = (q * np.sign(np.diag(r))).astype(np.float32)
    Rl, obj_l = R.fit_rotation(x, R0, 2, D, "f16", iters=3)
    Ro, obj_o = O.fit_rotation(x.astype(np.float64), R0, 2, D, "f16", 3)
    Rl64 = Rl.astype(np.float64)
    np.testing.assert_allclose(Rl64 @ Rl64.T, np.eye(D), rtol=0, atol=1e-6)
    np.testing.assert_allclose(obj_l, obj_o, rtol=1e-9, atol=0)
    X = x.astype(np.float64)
    np.testing.assert_allclose(X @ Rl64.T, X @ Ro.astype(np.float32).astype(np.float64).T, rtol=0, atol=2e-6)


def test_fit_device_validation():
    """Argument checks of the device fit that return before any GPU work."""
    import ctypes
    L = R.lib()
    r = np.eye(64, dtype=np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert R.fit_workspace_bytes(64) > 64 * 64 * 8 * 64
    assert R.fit_workspace_bytes(80) == 0
    fake = ctypes.c_void_p(256)          # never dereferenced: every call below fails validation first
    ws = ctypes.c_void_p(4096)
    big = R.fit_workspace_bytes(64)
    assert L.rq_fit_rotation_device(None, 4, 64, 2, 64, 1, p(r), 1, p(r), None, ws, big, None) == -1
    assert L.rq_fit_rotation_device(fake, 0, 64, 2, 64, 1, p(r), 1, p(r), None, ws, big, None) == -2
    assert L.rq_fit_rotation_device(fake, 4, 64, 3, 64, 1, p(r), 1, p(r), None, ws, big, None) == -3
    assert L.rq_fit_rotation_device(fake, 4, 80, 2, 16, 1, p(r), 1, p(r), None, ws, big, None) == -3
    assert L.rq_fit_rotation_device(fake, 4, 64, 2, 48, 1, p(r), 1, p(r), None, ws, big, None) == -2
    assert L.rq_fit_rotation_device(fake, 4, 64, 2, 64, 1, p(r), 1, p(r), None, ws, big - 8, None) == -4
