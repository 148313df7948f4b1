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


def _tiny_layer(kvals, qvals=(1.0, -1.0), q_pos0=4):
    """One indexer layer with H = D = 1, m = 1, T = 6: the score of key s for
    query row i is max(q_i * k_s, 0) (weight 1), so every score is read off by
    eye.  Row i sits at position q_pos0 + i and sees keys 0 .. q_pos0 + i."""
    S_q, T = len(qvals), len(kvals)
    return dict(dtype="f32", B=1, S_q=S_q, T=T, H=1, D=1, m=1, q_pos0=q_pos0, topk=2,
                q=np.array(qvals, np.float32).reshape(1, S_q, 1, 1),
                k=np.array(kvals, np.float32).reshape(1, T, 1),
                w=np.ones((1, S_q, 1), np.float32), kv_len=None, causal=True)


def test_multilayer_hand_example():
    """Two layers, threshold tau = 0.5 (keep I > 0), cap 2 per layer, union.

    Layer 0 keys [3, -1, 5, 2, 0, 4], layer 1 keys [-1, 6, -2, 0, 0, -3].
      row 0 (q = +1, keys 0..4): layer 0 scores [3,0,5,2,0] -> survivors
        {0,2,3} -> best 2: {2,0}; layer 1 scores [0,6,0,0,0] -> {1}.
        Union {0,1,2}, size 3.
      row 1 (q = -1, keys 0..5): layer 0 scores [0,1,0,0,0,0] -> {1};
        layer 1 scores [1,0,2,0,0,3] -> survivors {0,2,5} -> best 2: {5,2}.
        Union {1,2,5}, size 3.
    A union cap of 2 keeps the two smallest indices; the counts stay 3."""
    layers = [_tiny_layer([3, -1, 5, 2, 0, 4]), _tiny_layer([-1, 6, -2, 0, 0, -3])]
    idx, cnt = oracle.oracle_multilayer(layers, 0.5, cap=2, union_cap=4)
    assert idx.tolist() == [[[0, 1, 2, -1], [1, 2, 5, -1]]]
    assert cnt.tolist() == [[3, 3]]
    idx, cnt = oracle.oracle_multilayer(layers, 0.5, cap=2, union_cap=2)
    assert idx.tolist() == [[[0, 1], [1, 2]]] and cnt.tolist() == [[3, 3]]
    # a bias of +1 moves the threshold to I > -1: every visible key survives,
    # and the cap picks by score, ties to the lower index
    idx, cnt = oracle.oracle_multilayer(layers, 0.5, cap=2, union_cap=6, logit_bias=1.0)
    # row 0: layer 0 best 2 of [3,0,5,2,0] = {2,0}; layer 1 [0,6,0,0,0] = {1, 0}
    # row 1: layer 0 [0,1,0,0,0,0] = {1, 0}; layer 1 [1,0,2,0,0,3] = {5, 2}
    assert idx.tolist() == [[[0, 1, 2, -1, -1, -1], [0, 1, 2, 5, -1, -1]]]
    assert cnt.tolist() == [[3, 4]]


def test_multilayer_pin_rejects_plausible_mistakes():
    """The hand example tells the threshold reading apart from a plain per-layer
    top-k (which would keep non-survivors) and from an uncapped threshold
    selection (which would keep every survivor)."""
    layers = [_tiny_layer([3, -1, 5, 2, 0, 4]), _tiny_layer([-1, 6, -2, 0, 0, -3])]
    want, _ = oracle.oracle_multilayer(layers, 0.5, cap=2, union_cap=6)
    plain = oracle.oracle_union([oracle.oracle_topk(p, topk=2)[0] for p in layers], 6, 6)[0]
    uncapped = oracle.oracle_union([oracle.oracle_threshold(p, 0.5, 0.0, cap=6)[0] for p in layers], 6, 6)[0]
    assert not np.array_equal(want, plain)
    assert not np.array_equal(want, uncapped)
