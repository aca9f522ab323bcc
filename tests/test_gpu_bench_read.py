"""The streaming-read measurement kernel reads every word of its buffer: the
XOR of its per-workgroup folds equals the XOR of all 32-bit words."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16 * 7, 1 << 24, (1 << 24) + 48])
def test_read_kernel_covers_every_word(nbytes):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_uniform_paged_amd import api
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(api.TG_BENCH_READ_BLOCKS, dtype=torch.int32, device="cuda")
    api.tg_bench_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
