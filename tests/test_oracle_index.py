"""Pins for the oracle's DSA indexer scores and causal top-k."""
import numpy as np

from tests.util import bf16_to_f64, block_table, randn_bf16, rand_u, scatter_rows

THETA = 10000.0


def index_pool(orc, keys_bf16, seed=0, extra=2):
    """One sequence whose ratio-4 index pool holds the given entries [n][d] (bf16 bits)."""
    n, d = keys_bf16.shape
    mb = (4 * n + 255) // 256 + 1
    bt = block_table(seed, 1, mb, extra_pages=extra)
    pool = orc.HostPool(4, 2, d, 0, THETA, orc.BF16, mb + extra)
    scatter_rows(pool.rows, bt, 0, 4, keys_bf16.view(np.uint8).reshape(n, 2 * d))
    return pool, bt


def bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_closed_form_scores_and_ties(orc):
    # one-hot keys: sigma(i) = w0*relu(a_i) + w1*relu(-b_i) for key a_i e0 + b_i e1,
    # queries q0 = e0, q1 = -e1
    d = 32
    a = np.array([3, -1, 2, 0, 5, 2, -4, 1], np.float32)
    b = np.array([-1, 2, 0, -3, 1, 0, -1, 0], np.float32)
    keys = np.zeros((8, d), np.float32)
    keys[:, 0], keys[:, 1] = a, b
    pool, bt = index_pool(orc, bf16(keys))
    q = np.zeros((1, 2, d), np.float32)
    q[0, 0, 0], q[0, 1, 1] = 1.0, -1.0
    w = np.array([[0.5, 0.25]], np.float32)
    topk, kth, sc, f = orc.index_topk(pool, bt, [0], [32], bf16(q), w, 4, want_scores=True, max_cand=8)
    want = 0.5 * np.maximum(a, 0) + 0.25 * np.maximum(-b, 0)
    assert f == 0 and np.array_equal(sc[0], want)
    # sorted: 2.5(4) 1.75(0) 1.0(2) 1.0(5) 0.75(3) ... -> ties at 1.0 keep the lower index 2 then 5
    assert topk[0].tolist() == [0, 2, 4, 5] and kth[0] == 1.0
    topk3, kth3, _, _ = orc.index_topk(pool, bt, [0], [32], bf16(q), w, 3)
    assert topk3[0].tolist() == [0, 2, 4] and kth3[0] == 1.0


def test_topk_is_prefix_of_full_sort(orc):
    n, d, nq, H = 300, 32, 6, 4
    keys = randn_bf16(3, 1, (n, d))
    pool, bt = index_pool(orc, keys)
    q = randn_bf16(3, 2, (nq, H, d))
    w = rand_u(3, 3, (nq, H)).astype(np.float32)
    pos = np.array([1200, 1199, 1000, 37, 4, 3], np.int64)
    topk, kth, sc, f = orc.index_topk(pool, bt, np.zeros(nq, np.int32), pos, q, w, 64, want_scores=True,
                                      max_cand=n)
    assert f == 0
    kf, qf = bf16_to_f64(keys), bf16_to_f64(q)
    for j in range(nq):
        nc = int(pos[j]) // 4
        # brute-force scores from the definition
        s = (w[j][:, None] * np.maximum(qf[j] @ kf[:nc].T, 0)).sum(0)
        assert np.allclose(sc[j, :nc], s, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(sc[j, nc:]))
        order = np.lexsort((np.arange(nc), -sc[j, :nc]))
        want = np.sort(order[:64])
        got = topk[j][topk[j] >= 0]
        assert np.array_equal(got, want)
        assert np.all(topk[j][len(want):] == -1)
        assert np.all(np.diff(got) > 0)
        if nc:
            assert kth[j] == sc[j, order[min(64, nc) - 1]]
        else:
            assert np.isneginf(kth[j])


def test_causal_cut(orc):
    # the entry holding position p (or later) must never be picked, whatever its score
    n, d = 64, 32
    keys = np.zeros((n, d), np.float32)
    keys[:, 0] = np.arange(n, dtype=np.float32)   # score grows with the index
    pool, bt = index_pool(orc, bf16(keys))
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    for p in [4, 7, 8, 100, 103, 104, 255]:
        topk, _, _, _ = orc.index_topk(pool, bt, [0], [p], bf16(q), np.ones((1, 1), np.float32), 2)
        last = p // 4 - 1      # last entry whose 4 own tokens end before p
        want = [i for i in (last - 1, last) if i >= 0]
        assert topk[0][topk[0] >= 0].tolist() == want, p


def test_unmapped_page_counts_fault(orc):
    keys = randn_bf16(4, 1, (128, 32))
    pool, bt = index_pool(orc, keys)
    bt[0, 1] = -1
    _, _, _, f = orc.index_topk(pool, bt, [0], [512], randn_bf16(4, 2, (1, 2, 32)), np.ones((1, 2), np.float32), 8)
    assert f == 64
