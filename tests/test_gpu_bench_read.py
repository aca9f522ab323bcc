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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    api.tg_bench_read(src, sink, events=ev)  # with the kernel's start and end recorded
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_kernel_reads_each_listed_chunk():
    """The paged-stream read kernel: stream w's fold is the XOR of every word
    of the chunks on its list (ids modulo the chunk count; empty lists, lists
    past one 64-id window, repeated and negative ids)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_uniform_paged_amd import api
    rng = np.random.default_rng(7)
    n_chunks = 300
    host = rng.integers(0, 2**32, size=n_chunks * 2048, dtype=np.uint32)
    words = host.reshape(n_chunks, 2048)
    lengths = [0, 1, 2, 3, 7, 16, 63, 64, 65, 130, 5, 0, 200]
    chunks = [rng.integers(-2 * n_chunks, 3 * n_chunks, size=k) for k in lengths]
    chunks[4][1] = chunks[4][0]  # a repeated chunk cancels
    off = np.zeros(len(lengths) + 1, np.int32)
    off[1:] = np.cumsum(lengths)
    flat = np.concatenate(chunks).astype(np.int32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(len(lengths), dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    api.tg_bench_streams(src, torch.from_numpy(flat).cuda(), torch.from_numpy(off).cuda(), sink, events=ev)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    got = sink.cpu().numpy().view(np.uint32)
    for w, ids in enumerate(chunks):
        want = np.uint32(0)
        for c in ids:
            want ^= np.bitwise_xor.reduce(words[int(c) % n_chunks])
        assert got[w] == want, (w, lengths[w])
