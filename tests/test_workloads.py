"""The seeded generator: determinism, prefix-stable streams, and the
deduplicated row store reproducing every logical sequence."""
import numpy as np

from workloads import make_workload, bf16_round, bf16_bits_to_f32


def test_bf16_round_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9], np.float32)
    got = bf16_bits_to_f32(bf16_round(x))
    assert list(got) == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 1.0]


def test_streams_deterministic_and_prefix_stable():
    w = make_workload("llama8b", B=2)
    k1, v1 = w.stream_rows(("seq", 1, 3), 100)
    k2, v2 = w.stream_rows(("seq", 1, 3), 37)
    assert np.array_equal(k1[:37], k2) and np.array_equal(v1[:37], v2)
    assert not np.array_equal(k1[:37], v1[:37])
    w2 = make_workload("llama8b", B=2)
    assert np.array_equal(w.q(), w2.q())


def test_source_buffer_reproduces_logical_rows_with_sharing():
    w = make_workload("radix", B=6, share=dict(prefix=40, branch=20, n_branches=2, suffix=(5, 30)))
    L = np.array([[60 + 3 * h + r for h in range(w.Hkv)] for r in range(w.B)])
    rows, index, off = w.source_buffer(L)
    for r in range(w.B):
        for h in range(w.Hkv):
            K, V = w.logical_kv(r, h, int(L[r, h]))
            sel = index[off[r * w.Hkv + h]:off[r * w.Hkv + h + 1]]
            assert np.array_equal(rows[sel, 0], K) and np.array_equal(rows[sel, 1], V)
    # the shared prefix of head 0 is stored once for all requests
    assert rows.shape[0] < int(L.sum())


def test_outlier_channel_scaled():
    w = make_workload("ragged", B=2)
    K, V = w.stream_rows(("seq", 0, 2), 4000)
    kf, vf = bf16_bits_to_f32(K), bf16_bits_to_f32(V)
    c = w.outlier_channels[2][0]
    assert 6 < kf[:, c].std() < 10 and 0.9 < np.delete(kf, c, axis=1).std() < 1.1
    assert 0.9 < vf[:, c].std() < 1.1
