"""The global output-channel precision search in the library (host C++) against the oracle
(talk notes, グローバル混合精度探索; the pages' Algorithm 1).  CPU only."""
import numpy as np
import pytest

import oracle as O
from tests import pins
from weight_activation_quantized_amd import mixllm as L
from weight_activation_quantized_amd import workloads as WL


def _layer(n, k, seed):
    sh = WL.Shape(0, "edge", 1, n, k, 0)
    w, _ = WL.make_layer_weights(sh)
    rng = np.random.default_rng(seed)
    return w, rng


@pytest.mark.parametrize("n,k,d", [(37, 256, 5), (64, 512, 3), (5, 1024, 1)])
def test_salience_matches_oracle(n, k, d):
    w, rng = _layer(n, k, n + k + d)
    g = rng.normal(0, 1, size=(d, n, k)).astype(np.float32)
    g[:, 0] *= 1e3  # a large-gradient channel: the second-order term matters
    got = L.mixllm_channel_salience(w, g)
    want = O.channel_salience(w, g)
    # both fp64; only the summation order of the dot products differs
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_salience_hand_example():
    """The hand-derived values of the oracle pin, through the library."""
    w = pins._salience_channels()
    g = np.zeros((2, 3, 128), np.float32)
    g[:, 0, 2] = [64.0, -128.0]
    g[:, 2, 2] = [128.0, 128.0]
    g[:, 1, :] = 9.0
    assert list(L.mixllm_channel_salience(w, g)) == [2.25, 0.0, 0.0]


def test_assignment_matches_oracle():
    rng = np.random.default_rng(5)
    sizes = [7, 1, 30, 12]
    scores = [rng.random(s) * 10.0 ** rng.integers(-3, 3) for s in sizes]
    total = sum(sizes)
    for t in [0, 1, 5, 17, total - 1, total]:
        got = L.mixllm_assign_channels(scores, t)
        want = O.assign_channels(scores, t)
        assert len(got) == len(want)
        for a, b in zip(got, want):
            assert np.array_equal(a, b), t


def test_assignment_ties():
    got = L.mixllm_assign_channels([np.array([1.0, 2.0]), np.array([2.0, 0.5])], 1)
    assert [list(x) for x in got] == [[1], []]
    got = L.mixllm_assign_channels([np.array([3.0, 3.0, 3.0])], 2)
    assert [list(x) for x in got] == [[0, 1]]


def test_assignment_errors():
    lib = L.library_handle()
    s = np.array([1.0, 2.0, np.nan])
    n = np.array([3], np.int32)
    idx = np.zeros(3, np.int32)
    n8 = np.zeros(1, np.int32)
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 1, 1, idx.ctypes.data, n8.ctypes.data) == -2
    s = np.array([1.0, 2.0, 3.0])
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 1, 4, idx.ctypes.data, n8.ctypes.data) == -2
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 1, -1, idx.ctypes.data, n8.ctypes.data) == -2
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 0, 1, idx.ctypes.data, n8.ctypes.data) == -2
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 1, 1, None, n8.ctypes.data) == -1
    assert lib.mixllm_assign_channels(s.ctypes.data, n.ctypes.data, 1, 0, None, n8.ctypes.data) == 0
    w = np.zeros((2, 128), np.float16)
    g = np.zeros((1, 2, 128), np.float32)
    out = np.zeros(2)
    assert lib.mixllm_channel_salience(w.ctypes.data, g.ctypes.data, 2, 128, 64, 1, out.ctypes.data) == -3
    assert lib.mixllm_channel_salience(w.ctypes.data, g.ctypes.data, 2, 100, 128, 1, out.ctypes.data) == -2
    assert lib.mixllm_channel_salience(w.ctypes.data, g.ctypes.data, 2, 128, 128, 0, out.ctypes.data) == -2
    assert lib.mixllm_channel_salience(None, g.ctypes.data, 2, 128, 128, 1, out.ctypes.data) == -1


def test_search_then_pack():
    """Salience of three layers from synthetic gradients, the global top 10%, and each
    layer packed with its share: the blobs record the chosen counts."""
    layers = [(_layer(96, 256, 1)[0]), (_layer(40, 128, 2)[0]), (_layer(64, 384, 3)[0])]
    rng = np.random.default_rng(9)
    scores = []
    for i, w in enumerate(layers):
        g = rng.normal(0, 1.0 + 4 * i, size=(2,) + w.shape).astype(np.float32)
        scores.append(L.mixllm_channel_salience(w, g))
    total = sum(w.shape[0] for w in layers)
    t = int(np.ceil(0.1 * total))
    idx8 = L.mixllm_assign_channels(scores, t)
    assert sum(len(x) for x in idx8) == t
    flat = np.concatenate(scores)
    cut = np.sort(flat)[::-1][t - 1]
    for w, s, x in zip(layers, scores, idx8):
        assert np.all(s[x] >= cut)
        blob = L.mixllm_pack_weights(w, x)
        assert L.mixllm_blob_get_info(blob)["n8"] == len(x)
