"""Pins of the projection oracle (oracle/projection.py) against what does not rest on it:
a brute-force triple loop, closed forms of structured weights (each output block a
known multiple of the input), and linearity. All exact in fp64 on small integers."""
import numpy as np
import pytest

from oracle.projection import qkv_project, qkv_project_rows


def test_matches_brute_force_loops():
    rng = np.random.default_rng(0)
    t, hidden, h_q, h_kv, d = 3, 5, 2, 1, 2
    x = rng.integers(-3, 4, (t, hidden)).astype(float)
    w = rng.integers(-3, 4, ((h_q + 2 * h_kv) * d, hidden)).astype(float)
    q, k, v = qkv_project(x, w, h_q, h_kv, d)
    for i in range(t):
        feats = []
        for n in range(w.shape[0]):
            acc = 0.0
            for j in range(hidden):
                acc += x[i, j] * w[n, j]
            feats.append(acc)
        assert list(q[i].ravel()) == feats[: h_q * d]
        assert list(k[i].ravel()) == feats[h_q * d: (h_q + h_kv) * d]
        assert list(v[i].ravel()) == feats[(h_q + h_kv) * d:]


def test_block_order_and_head_layout():
    """W = [1 I; 2 I; 3 I] for MHA (h_q d = h_kv d = hidden): Q = x, K = 2x, V = 3x, heads
    in order of the features."""
    t, h, d = 4, 3, 2
    hidden = h * d
    x = np.arange(t * hidden, dtype=float).reshape(t, hidden) - 7
    eye = np.eye(hidden)
    q, k, v = qkv_project(x, np.concatenate([eye, 2 * eye, 3 * eye]), h, h, d)
    assert np.array_equal(q, x.reshape(t, h, d))
    assert np.array_equal(k, 2 * x.reshape(t, h, d))
    assert np.array_equal(v, 3 * x.reshape(t, h, d))


def test_gqa_selects_feature_blocks():
    """h_q = 4, h_kv = 1, d = 2: K and V are the two 2-feature blocks after the 8 Q features."""
    hidden = 8
    x = np.arange(2 * hidden, dtype=float).reshape(2, hidden)
    w = np.zeros((12, hidden))
    w[:8] = np.eye(hidden)
    w[8, 0] = w[9, 1] = 5.0          # K = 5 * x[:, :2]
    w[10, 7] = w[11, 6] = -1.0        # V = -(x7, x6)
    q, k, v = qkv_project(x, w, 4, 1, 2)
    assert np.array_equal(q.reshape(2, 8), x)
    assert np.array_equal(k[:, 0], 5 * x[:, :2])
    assert np.array_equal(v[:, 0], -x[:, [7, 6]])


def test_linear_in_the_tokens():
    rng = np.random.default_rng(3)
    x1 = rng.integers(-4, 5, (6, 16)).astype(float)
    x2 = rng.integers(-4, 5, (6, 16)).astype(float)
    w = rng.integers(-2, 3, (16, 16)).astype(float)
    a = qkv_project(x1 + 2 * x2, w, 2, 1, 4)
    b1, b2 = qkv_project(x1, w, 2, 1, 4), qkv_project(x2, w, 2, 1, 4)
    for y, y1, y2 in zip(a, b1, b2):
        assert np.array_equal(y, y1 + 2 * y2)


def test_rows_subset_and_shape_check():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 8))
    w = rng.standard_normal((16, 8))
    full = qkv_project(x, w, 2, 1, 4)
    sub = qkv_project_rows(x, w, [7, 2], 2, 1, 4)
    for f, s in zip(full, sub):
        assert np.array_equal(f[[7, 2]], s)
    with pytest.raises(ValueError):
        qkv_project(x, w[:12], 2, 1, 4)
