"""Pins for the oracle's dispatch step: a stable counting sort of the T*k
(token, slot) pairs by expert.  The page ("Welcome Beam: a 501B open model you
can own, customize, and scale", section "Mixture of Experts") only implies the
step: each token runs on its 8 chosen experts, so the rows bound for one expert
must be brought together.  Pinned by numpy's bincount / cumsum and a stable
argsort."""
import numpy as np
import pytest


def _ids(T, k, E, seed, hot=None):
    rng = np.random.default_rng(seed)
    out = np.empty((T, k), np.int32)
    for t in range(T):
        if hot is not None and rng.random() < 0.7:
            pool = rng.permutation(hot)[:k] if len(hot) >= k else None
            if pool is not None:
                out[t] = pool
                continue
        out[t] = rng.permutation(E)[:k]
    return out


@pytest.mark.parametrize("T,k,E,hot", [(64, 4, 16, None), (128, 8, 256, None),
                                       (1000, 8, 256, list(range(40, 56))),
                                       (3, 1, 5, None), (0, 8, 256, None)])
def test_permute_against_numpy(oracle_mod, T, k, E, hot):
    ids = _ids(T, k, E, seed=T + k + E, hot=hot)
    off, sp, pr = oracle_mod.permute(ids, E)
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable").astype(np.int32))
    # pair_rows is the inverse permutation
    np.testing.assert_array_equal(sp[pr], np.arange(T * k, dtype=np.int32))
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)


def test_permute_rejects_out_of_range(oracle_mod):
    ids = np.array([[0, 3], [1, 4]], np.int32)
    with pytest.raises(ValueError):
        oracle_mod.permute(ids, 4)
