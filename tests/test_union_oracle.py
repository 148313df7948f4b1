"""Pins for the union-of-selections oracle (CPU only): a hand-worked example,
and set identities the union must satisfy (idempotence, order of the lists,
each list's valid entries contained, invalid entries ignored, the cap keeps
the smallest indices and the count stays exact)."""
import numpy as np

import oracle


def test_hand_example():
    a = np.array([[5, 1, -1, 9]], dtype=np.int32)
    b = np.array([[9, 3, 12, 1]], dtype=np.int32)      # 12 >= T is ignored
    idx, cnt = oracle.oracle_union([a, b], T=10, cap=6)
    assert idx.tolist() == [[1, 3, 5, 9, -1, -1]]
    assert cnt.tolist() == [4]
    idx, cnt = oracle.oracle_union([a, b], T=10, cap=2)
    assert idx.tolist() == [[1, 3]] and cnt.tolist() == [4]


def test_set_identities():
    rng = np.random.default_rng(3)
    lists = [rng.integers(-3, 60, size=(4, 2, w)).astype(np.int32) for w in (7, 13, 5)]
    u, c = oracle.oracle_union(lists, T=50, cap=64)
    # idempotent and independent of list order
    u2, c2 = oracle.oracle_union(lists[::-1] + [lists[0]], T=50, cap=64)
    assert (u == u2).all() and (c == c2).all()
    for pos in np.ndindex(4, 2):
        got = [v for v in u[pos].tolist() if v >= 0]
        assert got == sorted(set(got)) and len(got) == c[pos]
        for li in lists:                                # every valid entry of every list
            for v in li[pos].tolist():
                if 0 <= v < 50:
                    assert v in got
        assert all(0 <= v < 50 for v in got)
        assert c[pos] <= sum(li.shape[-1] for li in lists)
