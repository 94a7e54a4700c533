"""The read-only streaming reference (a measurement aid, not a step of the
method): every wavefront's word must be the XOR of the 32-bit words it covers,
so the launch provably reads every byte once, including a ragged last
wavefront and the decode layer's full size."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

WAVE_BYTES = 4608


@pytest.mark.parametrize("nbytes", [12, 4608, 4620, 18432 * 3 + 600, 79251456])
def test_stream_read_xor(nbytes):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq
    print(f"stream_read: {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    buf = rng.integers(0, 256, nbytes, dtype=np.uint8)
    sink = owq.stream_read(torch.from_numpy(buf).to("cuda:0"))
    torch.cuda.synchronize()
    words = -(-nbytes // WAVE_BYTES)
    pad = np.zeros(words * WAVE_BYTES, dtype=np.uint8)
    pad[:nbytes] = buf
    want = np.bitwise_xor.reduce(pad.view(np.uint32).reshape(words, WAVE_BYTES // 4), axis=1)
    got = sink.cpu().numpy().view(np.uint32)
    assert got.shape == (words,)
    assert np.array_equal(got, want)
