"""The streaming-read hook (kvd_debug_stream_read), which the benchmark uses
as the practical read ceiling of a decode launch: it must read every byte
exactly once -- the XOR of its per-work-item sinks equals the XOR of all
32-bit words of the buffer -- for sizes that leave the last stride partly
filled and for several grids."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 20) + 48, 3 * (1 << 22) + 16 * 77])
@pytest.mark.parametrize("grid", [1, 7, 512])
def test_stream_read_covers_every_word_once(nbytes, grid):
    import torch
    import decode_attention_paged_04_amd as kvd
    rng = np.random.default_rng(nbytes + grid)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    data = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    kvd.kvd_debug_stream_read(data, sink, grid)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
