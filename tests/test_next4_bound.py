"""Why the index top-k has no certified fp4 pre-filter stage.

A two-stage indexer that scores every visible entry on its fp4 (MXFP4) row,
keeps only the entries whose score could still reach the top k, and re-scores
those in bf16 is exact only if the first stage carries a certified bound on
its error.  With w the head weights, q the index heads and delta_d a bound on
element d's fp4 error, ReLU being 1-Lipschitz gives

    |sigma_fp4 - sigma_bf16| <= eps = sum_d (sum_h |w_h| |q_hd|) delta_d,

and the candidates are the entries with sigma_fp4 + eps >= tau, tau the k-th
largest sigma_fp4 - eps; every true top-k entry passes.  On the index keys of
the c4a decode workload (N(0,1) keys and queries, 16 heads of 128 dims, weights
U(0,1)), eps is about ten times the spread of the scores, so no entry is ever
pruned: the stage would read the fp4 and the bf16 row of every entry.  This
test checks both facts on a seeded sample of the workload (one query, 4096
entries, k scaled to 64 as 512 of 32768), with the rows quantised by the
oracle's MXFP4 codec.
"""
import numpy as np

from synth import workloads as W
from tests.util import fp4_rows

# E2M1 magnitudes and the largest distance from a code's value to an input that
# rounds to it, in units of the block scale (the top code takes inputs up to 8:
# the scale rule keeps a block's maximum below 8 X)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
REACH = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 2.0])


def test_certified_fp4_prefilter_prunes_nothing_on_the_workload(orc):
    w = W.c4a_decode()
    n, d, k = 4096, w.idx_dim, 64
    qd = W.queries(w)
    q = qd["q_idx"][0].float().numpy().astype(np.float64)      # [H][d], bf16 values
    wh = qd["w_idx"][0].numpy().astype(np.float64)              # [H]
    keys = W.index_keys(w, 0, 0, n).float().numpy().astype(np.float64)
    rows = fp4_rows(orc, keys)
    deq = orc.decode_rows(rows, d, orc.FP4)
    X = np.repeat(np.ldexp(1.0, rows[:, d // 2:d // 2 + d // 32].astype(np.int64) - 127), 32, axis=1)
    mag = np.abs(deq) / X
    code = np.abs(mag[..., None] - E2M1).argmin(-1)
    delta = REACH[code] * X
    sig = (np.maximum(keys @ q.T, 0.0) * wh).sum(1)
    sig4 = (np.maximum(deq @ q.T, 0.0) * wh).sum(1)
    Q = (np.abs(wh)[:, None] * np.abs(q)).sum(0)
    eps = delta @ Q
    # the bound is a certificate: it holds for every entry
    assert np.all(np.abs(sig4 - sig) <= eps)
    tau = np.sort(sig4 - eps)[-k]
    kept = int(np.count_nonzero(sig4 + eps >= tau))
    # ... and it keeps every entry: the bound dwarfs the scores' spread
    assert np.median(eps) > 5 * np.std(sig)
    assert kept == n


def test_certified_page_bound_prunes_nothing_on_the_workload():
    """The other exact first stage a two-stage indexer could use: skip a 64-entry page
    when an upper bound of its scores is below the k-th score.  Per head, q.k over a
    page is bounded by sum_d max(q_d kmax_d, q_d kmin_d) with the page's per-dim
    extremes, and w_h ReLU(.) is monotone, so the bound holds for every entry.  Even
    against the exact k-th score (the most a first stage could know) it prunes no
    page of the decode workload's index keys: the bound is about 25 times the k-th
    score."""
    w = W.c4a_decode()
    n, k = 4096, 64
    qd = W.queries(w)
    q = qd["q_idx"][0].float().numpy().astype(np.float64)
    wh = qd["w_idx"][0].numpy().astype(np.float64)
    keys = W.index_keys(w, 0, 0, n).float().numpy().astype(np.float64)
    sig = (np.maximum(keys @ q.T, 0.0) * wh).sum(1)
    tau = np.sort(sig)[-k]
    pages = keys.reshape(n // 64, 64, -1)
    kmax, kmin = pages.max(1), pages.min(1)
    bound = (np.maximum(np.clip(q, 0, None) @ kmax.T + np.clip(q, None, 0) @ kmin.T, 0.0) * wh[:, None]).sum(0)
    assert np.all(bound >= sig.reshape(n // 64, 64).max(1) - 1e-9)  # a certificate
    assert int(np.count_nonzero(bound < tau)) == 0
    assert bound.min() > 10 * tau
