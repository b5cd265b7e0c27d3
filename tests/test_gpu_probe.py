"""GPU: the measurement probes read every byte of their source exactly once.

Each thread folds what it read by XOR into its sink word, so the XOR of all
sink words equals the XOR of every 32-bit word of the source exactly when
each 16-byte word was read once (a word read twice or never would cancel or
be missing).  Sizes cover whole 256 KB chunks, a ragged tail and a source
smaller than one chunk."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import mxfp4_moe_expert_02_amd as M
    return M


@pytest.mark.parametrize("nbytes", [16, 4096, (256 << 10) - 16, 5 * (256 << 10) + 48,
                                    (64 << 20) + (37 << 4)])
@pytest.mark.parametrize("which", ["stream", "cached"])
def test_probe_reads_every_word_once(M, nbytes, which):
    import torch
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.zeros(M.moe_probe_sink_words(), dtype=torch.int32, device="cuda")
    fn = M.moe_probe_stream_read if which == "stream" else M.moe_probe_read_cached
    fn(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
