"""GPU path of the rotation fit (rq_fit_rotation_device): every pass of the
alternation runs as a float64 kernel over device-resident calibration rows;
the trajectory of the objective and the fitted rotation must equal the
oracle's fit (reading R18 of the oracle; the pages give the rotation's role,
per layer, head and K|V, rit.work summary, section on how each pass's KV
cache is restored) and the host library's, and two runs must agree bit for
bit (fixed summation order)."""
import numpy as np
import pytest

import oracle as O

from gpu_util import dev, torch

pytestmark = pytest.mark.gpu


def _rows(D, n, seed, zero_channels=0):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.normal(0, 0.5, D))
    scale[rng.permutation(D)[: max(1, round(0.02 * D))]] *= 10.0
    x = (rng.normal(size=(n, D)) * scale * 0.1).astype(np.float32)
    x[:, rng.permutation(D)[:zero_channels]] = 0.0
    return x


@pytest.mark.parametrize("D,G,bits,meta,n,zc", [(64, 64, 2, "f16", 700, 0), (128, 128, 2, "f16", 2048, 0),
                                                 (128, 32, 4, "f32", 1000, 0), (96, 96, 4, "f16", 513, 0),
                                                 (64, 16, 2, "f16", 40, 3)])
def test_device_fit_matches_oracle(D, G, bits, meta, n, zc):
    import looped_transformer_decode_rq_amd as R
    T = torch()
    x = _rows(D, n, D + bits + n, zc)
    rng = np.random.default_rng(9)
    q, r = np.linalg.qr(rng.normal(size=(D, D)))
    R0 = (q * np.sign(np.diag(r))).astype(np.float32)
    xd = T.from_numpy(x).to(dev())
    ws = T.empty(R.fit_workspace_bytes(D), dtype=T.uint8, device=dev())
    Rd, obj_d = R.fit_rotation_device(xd, R0, bits, G, ws, meta, iters=3)
    Rd2, obj_d2 = R.fit_rotation_device(xd, R0, bits, G, ws, meta, iters=3)
    np.testing.assert_array_equal(obj_d, obj_d2)
    np.testing.assert_array_equal(Rd, Rd2)
    Ro, obj_o = O.fit_rotation(x.astype(np.float64), R0, bits, G, meta, 3)
    np.testing.assert_allclose(obj_d, obj_o, rtol=1e-9, atol=0)
    X = x.astype(np.float64)
    Rd64 = Rd.astype(np.float64)
    np.testing.assert_allclose(Rd64 @ Rd64.T, np.eye(D), rtol=0, atol=1e-5)
    # the rotation's action on the rows (unique even where M is rank deficient)
    np.testing.assert_allclose(X @ Rd64.T, X @ Ro.astype(np.float32).astype(np.float64).T, rtol=0, atol=2e-6)
    Rh, obj_h = R.fit_rotation(x, R0, bits, G, meta, iters=3)
    np.testing.assert_allclose(obj_d, obj_h, rtol=1e-12, atol=0)
