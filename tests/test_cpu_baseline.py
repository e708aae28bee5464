"""The all-core CPU baseline routes each core's contiguous token chunk as a
microbatch of its own.  That is the same per-token work as routing the whole
batch: top-k, gate weights and row statistics depend on the token alone, and
the chunks' histograms add up to the batch's."""
import numpy as np

import oracle


def test_chunked_routing_matches_whole_batch():
    rng = np.random.default_rng(11)
    T, E, k = 3000, 64, 4
    L = (rng.standard_normal((T, E)) + rng.normal(0, 0.5, E)).astype(np.float32)
    whole = oracle.route(L, k, capacity_factor=1.25, renorm=True)
    bounds = [(0, 700), (700, 1500), (1500, 2999), (2999, 3000)]
    counts = np.zeros(E, np.int64)
    for a, b in bounds:
        part = oracle.route(L[a:b], k, capacity_factor=1.25, renorm=True)
        assert np.array_equal(part["topk_idx"], whole["topk_idx"][a:b])
        assert np.array_equal(part["topk_w"], whole["topk_w"][a:b])
        assert np.array_equal(part["row_max"], whole["row_max"][a:b])
        assert np.array_equal(part["row_sum"], whole["row_sum"][a:b])
        counts += part["counts"][0]
    assert np.array_equal(counts, whole["counts"][0])
