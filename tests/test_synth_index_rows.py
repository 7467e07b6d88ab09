"""The random index rows the gradient tests feed both sides: valid rows of
the form the selection produces (distinct positions of 0..p in increasing
order, min(K, p+1) of them, then -1; nothing for rows past the history)."""
import numpy as np

import synth


def test_index_rows_valid():
    qo = np.array([0, 90, 5], np.int32)
    kl = np.array([40, 100, 5], np.int32)
    K = 12
    idx = synth.index_rows(qo, kl, 30, K, seed=3)
    assert idx.shape == (3, 30, K) and idx.dtype == np.int32
    for b in range(3):
        for i in range(30):
            p = int(qo[b]) + i
            row = idx[b, i]
            if p >= kl[b]:
                assert (row == -1).all()
                continue
            n = min(K, p + 1)
            assert (row[n:] == -1).all()
            sel = row[:n]
            assert (sel >= 0).all() and (sel <= p).all()
            assert (np.diff(sel) > 0).all()
            if p + 1 <= K:
                assert (sel == np.arange(p + 1)).all()
    # seeded: the same seed gives the same rows, another seed other rows
    assert np.array_equal(idx, synth.index_rows(qo, kl, 30, K, seed=3))
    assert not np.array_equal(idx, synth.index_rows(qo, kl, 30, K, seed=4))
