"""Pins for the projection oracle (query, head weights, compressed keys), CPU only.

Each pin is fixed by linear algebra, not by the oracle's own code: an
explicit sum over k on tiny inputs; identity weights return the input; with
r = H*D and W_q = I, q[t, j, d] is latent element j*D + d (head-major
layout); a one-hot W_w row picks one hidden component; W_k = [I 0 0 0] picks
the first token of each group of m, [0 0 0 I] the last, [I I I I] sums the
group.  ``test_pins_catch_planted_mistakes`` runs the same pins against
plausible wrong versions (transposed weights, strided groups, dim-major
heads, a dropped last term) and requires each to fail at least one pin.
"""
import numpy as np
import pytest

import csa_inputs
import oracle
from oracle import csa_projection_oracle as cpo


def _bits(x):
    return csa_inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _pins():
    """Run every pin with the module's current functions; return failed names
    (a pin that raises counts as failed)."""
    failed = []
    rng = np.random.default_rng(7)

    def check(name, fn):
        try:
            ok = bool(fn())
        except (ValueError, IndexError):
            ok = False
        if not ok:
            failed.append(name)

    # explicit sum over k, tiny shapes (K != N so a transposed use cannot pass)
    x = rng.integers(-3, 4, size=(2, 3, 5)).astype(np.float32)
    w = rng.integers(-3, 4, size=(4, 5)).astype(np.float32)
    want = np.zeros((2, 3, 4))
    for a in range(2):
        for t in range(3):
            for n in range(4):
                want[a, t, n] = sum(float(x[a, t, kk]) * float(w[n, kk]) for kk in range(5))

    def explicit():
        y = oracle.project(_bits(x), _bits(w))
        return y.shape == want.shape and np.array_equal(y, want)
    check("explicit_sum", explicit)
    # identity weights, and a non-symmetric square weight
    xi = rng.integers(-5, 6, size=(7, 6)).astype(np.float32)
    check("identity", lambda: np.array_equal(oracle.project(_bits(xi), _bits(np.eye(6))), xi))
    ws = np.triu(np.ones((6, 6), np.float32))          # y_n = sum_{k >= n} x_k
    want_t = np.stack([xi[:, n:].sum(1) for n in range(6)], 1)
    check("upper_triangular", lambda: np.array_equal(oracle.project(_bits(xi), _bits(ws)), want_t))
    # query layout: r = H*D, W_q = I
    H, D = 3, 4
    c = rng.integers(-8, 9, size=(2, 5, H * D)).astype(np.float32)

    def layout():
        q = oracle.oracle_query(_bits(c), _bits(np.eye(H * D)), H, D)
        return all(q[b, t, j, d] == c[b, t, j * D + d] for b in range(2) for t in range(5)
                   for j in range(H) for d in range(D))
    check("query_layout", layout)
    # head weights: one-hot rows
    hx = rng.integers(-8, 9, size=(2, 5, 7)).astype(np.float32)
    pick = [6, 0, 3]
    ww = np.zeros((3, 7), np.float32)
    ww[np.arange(3), pick] = 1.0
    check("head_weights", lambda: np.array_equal(oracle.oracle_head_weights(_bits(hx), _bits(ww)), hx[:, :, pick]))
    # key compression, m = 4, d_z = 3, D = 3
    m, dz = 4, 3
    z = rng.integers(-8, 9, size=(2, 12, dz)).astype(np.float32)
    I0 = np.zeros((dz, m * dz), np.float32)
    I0[:, :dz] = np.eye(dz)
    I3 = np.zeros((dz, m * dz), np.float32)
    I3[:, 3 * dz:] = np.eye(dz)
    Isum = np.tile(np.eye(dz, dtype=np.float32), (1, m))
    check("compress_first", lambda: np.array_equal(oracle.oracle_compress_keys(_bits(z), _bits(I0), m), z[:, 0::m]))
    check("compress_last", lambda: np.array_equal(oracle.oracle_compress_keys(_bits(z), _bits(I3), m), z[:, 3::m]))
    check("compress_sum", lambda: np.array_equal(oracle.oracle_compress_keys(_bits(z), _bits(Isum), m),
                                                 z.reshape(2, 3, m, dz).sum(2)))
    return failed


def test_oracle_pins():
    assert _pins() == []


def _transposed(x_bits, w_bits):
    x, w = oracle.decode_bf16(x_bits), oracle.decode_bf16(w_bits)
    if w.shape[0] != x.shape[-1]:
        raise ValueError("shape")
    return x @ w


def _dropped_term(x_bits, w_bits):
    x, w = oracle.decode_bf16(x_bits), oracle.decode_bf16(w_bits)
    return x[..., :-1] @ w[:, :-1].T


def _strided_compress(z_bits, wk_bits, m):
    B, S, dz = z_bits.shape
    T = S // m
    groups = np.concatenate([z_bits[:, i * T:(i + 1) * T] for i in range(m)], axis=-1)
    return cpo.project(groups, wk_bits)


def _dim_major_query(c_bits, wq_bits, H, D):
    B, S, _ = c_bits.shape
    return cpo.project(c_bits, wq_bits).reshape(B, S, D, H).transpose(0, 1, 3, 2)


@pytest.mark.parametrize("name", ["transposed", "dropped_term", "strided_compress", "dim_major_query"])
def test_pins_catch_planted_mistakes(name, monkeypatch):
    if name == "transposed":
        monkeypatch.setattr(cpo, "project", _transposed)
        monkeypatch.setattr(oracle, "project", _transposed)
    elif name == "dropped_term":
        monkeypatch.setattr(cpo, "project", _dropped_term)
        monkeypatch.setattr(oracle, "project", _dropped_term)
    elif name == "strided_compress":
        monkeypatch.setattr(oracle, "oracle_compress_keys", _strided_compress)
    else:
        monkeypatch.setattr(oracle, "oracle_query", _dim_major_query)
    assert _pins(), f"planted mistake {name} passed every pin"
