"""Pins for the sparse-attention oracle (CSA stage 4), CPU only.

Each pin is fixed by the mathematics of softmax attention, not by the
oracle's own code: a single selected key returns its value row; equal
logits average the selected value rows; two keys with a known logit gap give
a closed-form mixture; a dominant logit returns its value row; invalid
entries are ignored and an empty selection gives zeros; the order of the
entries does not matter.  ``test_pins_catch_planted_mistakes`` runs the same
pins against plausible wrong versions of the attention row (no scale,
softmax over the wrong axis, keys in place of values, a missing
normalisation) and requires each to fail at least one pin.
"""
import math

import numpy as np
import pytest

import csa_inputs
import oracle
from oracle import csa_attention_oracle as cao


def _bits(x):
    return csa_inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _prob(q, k, v):
    q = np.asarray(q, dtype=np.float32)
    return dict(q=_bits(q), k=_bits(k), v=_bits(v))


def _pins(row_fn):
    """Run every pin with `row_fn` as the attention row; return failed names."""
    failed = []
    rng = np.random.default_rng(5)
    H, Dk, Dv, T = 3, 8, 5, 12
    k = rng.integers(-3, 4, size=(1, T, Dk)).astype(np.float32)
    v = rng.integers(-3, 4, size=(1, T, Dv)).astype(np.float32)
    q = rng.integers(-2, 3, size=(1, 1, H, Dk)).astype(np.float32)
    p = _prob(q, k, v)
    scale = 0.25

    def run(prob, idx, sc=scale):
        orig = cao.attention_row
        cao.attention_row = row_fn
        try:
            return oracle.oracle_attention(prob, np.asarray(idx, dtype=np.int32)[None, None, :], sc)[0, 0]
        finally:
            cao.attention_row = orig

    # single selected key: every head returns that value row
    o = run(p, [7])
    if not np.allclose(o, np.repeat(v[0, 7][None], H, 0), atol=1e-12):
        failed.append("single")
    # zero query: equal logits, so the mean of the selected value rows
    pz = _prob(np.zeros_like(q), k, v)
    sel = [1, 4, 9, 10]
    o = run(pz, sel)
    if not np.allclose(o, np.repeat(v[0, sel].mean(0)[None], H, 0), atol=1e-12):
        failed.append("mean")
    # an index listed twice counts twice
    o = run(pz, [2, 2, 5])
    if not np.allclose(o, np.repeat(((2 * v[0, 2] + v[0, 5]) / 3)[None], H, 0), atol=1e-12):
        failed.append("duplicate")
    # two keys, logit gap c = scale * (q.k1 - q.k2): closed-form mixture
    q2 = np.zeros((1, 1, 1, Dk), np.float32)
    q2[0, 0, 0, 0] = 1.0
    k2 = np.zeros((1, 2, Dk), np.float32)
    k2[0, 0, 0] = 3.0                                   # q.k = 3 and 0
    v2 = np.array([[[1, 0, 0, 0, 2], [0, 1, 0, 0, -2]]], np.float32)
    o = run(_prob(q2, k2, v2), [0, 1], sc=0.5)
    c = 0.5 * 3.0
    want = (v2[0, 0] + math.exp(-c) * v2[0, 1]) / (1.0 + math.exp(-c))
    if not np.allclose(o[0], want, atol=1e-12):
        failed.append("gap")
    # a dominant logit returns its value row
    k3 = np.zeros((1, 3, Dk), np.float32)
    k3[0, 1, 0] = 64.0
    v3 = rng.integers(-3, 4, size=(1, 3, Dv)).astype(np.float32)
    o = run(_prob(q2, k3, v3), [0, 1, 2], sc=16.0)
    if not np.allclose(o[0], v3[0, 1], atol=1e-12):
        failed.append("dominant")
    # invalid entries are skipped; an empty selection is all zeros
    o_ref = run(p, [3, 6])
    o = run(p, [3, -1, 6, T, T + 5])
    if not np.allclose(o, o_ref, atol=1e-12):
        failed.append("invalid")
    if not np.array_equal(run(p, [-1, T]), np.zeros((H, Dv))):
        failed.append("empty")
    # entry order does not matter
    if not np.allclose(run(p, [0, 5, 11, 2]), run(p, [11, 2, 0, 5]), atol=1e-12):
        failed.append("order")
    return failed


def test_oracle_pins():
    assert _pins(cao.attention_row) == []


def _plain(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    z = scale * (q @ k.T)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v


def _wrong_axis(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    z = scale * (q @ k.T)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    return (e / e.sum(axis=0, keepdims=True)) @ v


def _keys_as_values(q, k, v, scale):
    return _plain(q, k, k[:, : v.shape[1]], scale)


def _unnormalised(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    z = scale * (q @ k.T)
    return np.exp(z - z.max(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("name,fn", [("no_scale", lambda q, k, v, s: _plain(q, k, v, 1.0)),
                                     ("wrong_axis", _wrong_axis),
                                     ("keys_as_values", _keys_as_values),
                                     ("unnormalised", _unnormalised)])
def test_pins_catch_planted_mistakes(name, fn):
    assert _pins(fn), f"planted mistake {name} passed every pin"


def test_oracle_matches_direct_sum_on_random_rows():
    """The vectorised oracle against an explicit per-head, per-entry loop."""
    p = csa_inputs.make_attention(2, 3, 50, H=4, Dk=16, Dv=8, n_sel=12, seed=3, pad=2)
    o = oracle.oracle_attention(p, p["idx"], p["scale"])
    q = oracle.decode_bf16(p["q"])
    k = oracle.decode_bf16(p["k"])
    v = oracle.decode_bf16(p["v"])
    for b in range(2):
        for t in range(3):
            ent = [int(e) for e in p["idx"][b, t] if 0 <= e < 50]
            for h in range(4):
                z = [p["scale"] * float(np.dot(q[b, t, h], k[b, e])) for e in ent]
                m = max(z)
                w = [math.exp(x - m) for x in z]
                acc = sum(wi * v[b, e] for wi, e in zip(w, ent)) / sum(w)
                assert np.allclose(o[b, t, h], acc, atol=1e-12)
