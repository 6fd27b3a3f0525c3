"""The test helpers' own logic, on the CPU: the near-tie rule of the routing
comparison and the sampling of tile-edge rows."""
import numpy as np

from _parity import GAP, edge_rows, stratified_tokens, valid_near_tie


def _scores_with_group_tie():
    # E=8, G=4 groups of 2, TG=2, k=2.  Groups 0 and 1 tie at the boundary
    # (group score 1.0 each, the 2nd best); group 2 is clearly best.  Keeping
    # group 0 selects experts {4, 0}; keeping group 1 selects {4, 2}, whose
    # score sum is lower by far more than k * GAP, yet both are valid.
    s = np.array([0.9, 0.1, 0.55, 0.45, 0.95, 0.2, 0.05, 0.04], np.float32)
    gs = np.array([s[0] + s[1], s[2] + s[3], s[4] + s[5], s[6] + s[7]], np.float32)
    return s, gs


def test_group_boundary_tie_accepts_either_resolution():
    s, gs = _scores_with_group_tie()
    assert abs(float(gs[0]) - float(gs[1])) <= GAP
    assert valid_near_tie(np.array([4, 0]), s, gs, 8, 4, 2, 2)
    assert valid_near_tie(np.array([2, 4]), s, gs, 8, 4, 2, 2)
    # an expert of an unkept group, or a non-top expert of a kept group, is not
    assert not valid_near_tie(np.array([4, 6]), s, gs, 8, 4, 2, 2)
    assert not valid_near_tie(np.array([4, 1]), s, gs, 8, 4, 2, 2)


def test_expert_boundary_tie():
    # one group, k=2: experts 1 and 2 tie for the second place
    s = np.array([0.9, 0.5, 0.5 + GAP / 4, 0.1], np.float32)
    gs = np.array([s[0] + s[2]], np.float32)
    assert valid_near_tie(np.array([0, 1]), s, gs, 4, 1, 1, 2)
    assert valid_near_tie(np.array([0, 2]), s, gs, 4, 1, 1, 2)
    assert not valid_near_tie(np.array([0, 3]), s, gs, 4, 1, 1, 2)


def test_edge_rows_and_stratified_sample():
    off = np.array([0, 3, 3, 300, 1400])   # experts of 3, 0, 297 and 1100 rows
    q = edge_rows(off)
    for want in (0, 2, 3, 299, 3 + 191, 3 + 192, 3 + 255, 3 + 256, 300, 1399, 300 + 511, 300 + 512):
        assert want in q, want
    assert q.max() < 1400 and len(set(q.tolist())) == q.size
    rng = np.random.default_rng(0)
    sp = rng.permutation(1400)
    t = stratified_tokens(off, sp, 4, 350, 64, rng, always=[349])
    assert t.size == 64 and 349 in t and len(set(t.tolist())) == 64 and t.max() < 350
