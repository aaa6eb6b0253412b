"""The contiguous-read bandwidth reference (rq_read_probe): its checksum is the
XOR of every 32-bit word of the buffer, so each byte is read exactly once."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (8 << 20) + 16 * 37, 64 << 20])
def test_read_probe_checksum(nbytes):
    import torch
    import looped_transformer_decode_rq_amd as R
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=max(nbytes // 4, 1), dtype=np.uint64).astype(np.uint32)[: nbytes // 4]
    buf = torch.from_numpy(host.view(np.int32).copy()).cuda() if nbytes else torch.empty(0, dtype=torch.int32,
                                                                                          device="cuda")
    for words in (1, 7, 8192):                  # shared words, an odd count, one word per wave
        sink = torch.zeros(words, dtype=torch.int32, device="cuda")
        R.read_probe(buf, sink)
        torch.cuda.synchronize()
        want = int(np.bitwise_xor.reduce(host)) if nbytes else 0
        assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == want, words
