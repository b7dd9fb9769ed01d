"""The streaming-read probe that the bench uses as its same-size ceiling: it
must read every 16-byte element of the buffer exactly once, in every launch
width, including sizes whose last round is partial (those rounds issue
clamped loads past the end and drop them)."""
import numpy as np
import pytest
import torch

import speculative_verify_amd as svq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svq.load()
    yield
    torch.cuda.synchronize()


# One full round is 32 KiB a workgroup (256 threads x 8 loads x 16 B).
@pytest.mark.parametrize("nbytes", [16, 32768, 32768 + 16, 7_094_272, 8_667_136, 20 * (1 << 20) + 48])
@pytest.mark.parametrize("wgs_per_cu", [0, 1, 2, 4])
def test_stream_read_reads_every_element_once(nbytes, wgs_per_cu):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    # Guard words after the buffer: a read past the end would fold them in.
    guard = rng.integers(0, 1 << 32, size=64, dtype=np.uint32)
    buf = torch.from_numpy(np.concatenate([host, guard]).view(np.int32)).cuda()
    sink = torch.zeros(8 * 1024, dtype=torch.int32, device="cuda")
    print(f"stream_read nbytes={nbytes} wgs_per_cu={wgs_per_cu}", flush=True)
    svq.svq_stream_read(buf, nbytes, sink, wgs_per_cu)
    torch.cuda.synchronize()
    # Each workgroup stores the XOR of the dwords it read; unused entries
    # stay zero.  The XOR over all of them is the buffer's XOR exactly when
    # no element is skipped or read twice (for random data).
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
