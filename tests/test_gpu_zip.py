"""GPU parity of the lossless bf16 exponent codec (tg_zip_encode /
tg_zip_decode): the compressed buffer equals the oracle's byte for byte
(header, codebook, streams, escapes in position order) and decoding gives
the input back bit for bit."""
import numpy as np
import pytest

from oracle import splitzip as Z

pytestmark = pytest.mark.gpu


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _inputs():
    g = np.random.default_rng(21)
    normal = (g.standard_normal(1 << 20).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return {
        "eight": np.array([0x3F80, 0xBF80, 0x4000, 0x3F81, 0x0001, 0x8000, 0x7F80, 0x3E00], np.uint16),
        "all-patterns": g.integers(0, 2 ** 16, size=65536, dtype=np.uint16),
        "normal-1M": normal,
        "cauchy-ragged": (g.standard_cauchy(8192 * 3 + 8).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16),
        "one-exponent": np.full(4096, 0x4049, np.uint16),
        # seventeen exponents, 512 values each: the tie at rank 16 goes to the
        # smaller exponent and the largest one is escaped
        "seventeen-tied": _tied(g),
        # escapes only in the last 1000 values of a long buffer
        "late-escapes": np.concatenate([normal[:1 << 19], ((np.arange(1000) % 50 + 200) << 7).astype(np.uint16),
                                        normal[:24]]),
    }


def _tied(g):
    e = np.repeat(np.arange(100, 117), 512)
    x = (g.integers(0, 2, e.size) << 15) | (e << 7) | g.integers(0, 128, e.size)
    return x[g.permutation(e.size)].astype(np.uint16)


@pytest.mark.parametrize("name", list(_inputs()))
def test_codec_matches_oracle_and_round_trips(name):
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    x = _inputs()[name]
    n = x.size
    print(f"case {name}: n={n}", flush=True)
    src = torch.from_numpy(x.view(np.int16)).cuda()
    dst = torch.zeros(api.tg_zip_bound(n), dtype=torch.uint8, device="cuda")
    ws = torch.empty(api.tg_zip_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    api.tg_zip_encode(src, dst, ws)
    torch.cuda.synchronize()
    ref = Z.encode(x)
    size = api.zip_compressed_bytes(dst)
    assert size == len(ref)
    got = dst[:size].cpu().numpy().tobytes()
    assert got == ref
    out = torch.empty_like(src)
    api.tg_zip_decode(dst, n, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), x)
