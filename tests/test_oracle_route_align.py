"""Pins of the oracle's routing and alignment: hand-derived worked examples,
brute force by other algorithms, closed-form special cases and invariants."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


# ---------------------------------------------------------------- routing ----

@pytest.mark.parametrize("case", GOLDEN["route"])
def test_route_worked_examples(case):
    if "logits_ln_of" in case:
        lg = np.log(np.array([case["logits_ln_of"]], dtype=np.float64))
    else:
        lg = np.array([case["logits"]], dtype=np.float64)
    ids, w = O.route(lg, case["topk"])
    assert ids[0].tolist() == case["ids"]
    expect = np.array([n / d for n, d in case["weights"]])
    np.testing.assert_allclose(w[0], expect, rtol=1e-15, atol=0)


def _route_by_rank(lg, k):
    """Brute force: the rank of expert i counts experts that beat it (larger
    logit, or equal logit and lower index); rank < k selects, rank is the slot."""
    T, E = lg.shape
    ids = np.full((T, k), -1)
    for t in range(T):
        for i in range(E):
            r = sum(1 for j in range(E) if lg[t, j] > lg[t, i] or (lg[t, j] == lg[t, i] and j < i))
            if r < k:
                ids[t, r] = i
    return ids


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (33, 8), (64, 64)])
def test_route_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.integers(-3, 4, size=(40, E)).astype(np.float64)    # many ties
    ids, w = O.route(lg, k)
    np.testing.assert_array_equal(ids, _route_by_rank(lg, k))
    lg2 = rng.standard_normal((40, E)).astype(np.float32).astype(np.float64)
    ids2, _ = O.route(lg2, k)
    np.testing.assert_array_equal(ids2, _route_by_rank(lg2, k))


def test_route_weights_invariants():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((200, 128)).astype(np.float32).astype(np.float64)
    ids, w = O.route(lg, 8)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in ids.tolist())


def test_route_equals_softmax_topk_renormalise():
    """Softmax over all experts (library routine), keep the top k, renormalise."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((50, 32)) * 3
    ids, w = O.route(lg, 6)
    p = softmax(lg, axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    _, w_full = O.route(lg, 6, renormalize=False)
    np.testing.assert_allclose(w_full, sel, rtol=1e-13)


def test_route_k_equals_E_is_full_softmax_and_E1_is_one():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((10, 12))
    ids, w = O.route(lg, 12)
    full = softmax(lg, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13)
    ids1, w1 = O.route(rng.standard_normal((5, 1)), 1)
    assert np.all(ids1 == 0) and np.all(w1 == 1.0)


# -------------------------------------------------------------- alignment ----

@pytest.mark.parametrize("case", GOLDEN["align"])
def test_align_worked_examples(case):
    a = O.align(np.array(case["ids"]), case["E"], case["block_m"])
    assert a["sorted_token_ids"].tolist() == case["sorted_token_ids"]
    assert a["expert_ids"].tolist() == case["expert_ids"]
    assert a["num_tokens_post_padded"] == case["num_tokens_post_padded"]
    assert a["inv"].tolist() == case["inv"]


def _align_brute(ids, E, B):
    """Build the padded layout by concatenating per-expert lists."""
    T, k = ids.shape
    R = T * k
    flat = ids.reshape(-1).tolist()
    out, blocks = [], []
    for e in range(E):
        rows = [f for f in range(R) if flat[f] == e]
        if not rows:
            continue
        pad = (-len(rows)) % B
        out += rows + [R] * pad
        blocks += [e] * ((len(rows) + pad) // B)
    padded = len(out)
    cap = R + E * (B - 1)
    out += [R] * (cap - padded)
    nb = -(-cap // B)
    blocks += [-1] * (nb - len(blocks))
    inv = [-1] * R
    for p, f in enumerate(out[:padded]):
        if f < R:
            inv[f] = p
    return out, blocks, padded, inv


@pytest.mark.parametrize("T,k,E,B", [(1, 1, 1, 1), (7, 2, 5, 4), (64, 8, 16, 16), (33, 3, 40, 8), (100, 4, 7, 64)])
def test_align_brute_force(T, k, E, B):
    rng = np.random.default_rng(T * 1000 + E)
    ids = rng.integers(-1, E + 1, size=(T, k))       # includes invalid ids and duplicates
    a = O.align(ids, E, B)
    s, b, p, inv = _align_brute(ids, E, B)
    assert a["sorted_token_ids"].tolist() == s
    assert a["expert_ids"].tolist() == b
    assert a["num_tokens_post_padded"] == p
    assert a["inv"].tolist() == inv
    assert a["capacity"] == O.align_capacity(T, k, E, B) == len(s)


def test_align_invariants_and_roundtrip():
    rng = np.random.default_rng(4)
    T, k, E, B = 300, 8, 64, 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    a = O.align(ids, E, B)
    st, inv, R = a["sorted_token_ids"], a["inv"], T * k
    valid = st[st < R]
    assert sorted(valid.tolist()) == list(range(R))               # a permutation
    assert np.all(st[inv] == np.arange(R))                         # scatter then gather = identity
    np.testing.assert_array_equal(inv[st[st < R]], np.nonzero(st < R)[0])
    eb = a["expert_ids"]
    used = eb[eb >= 0]
    assert np.all(np.diff(used) > 0) or len(used) <= 1 or np.all(np.diff(used) >= 0)
    assert a["num_tokens_post_padded"] % B == 0
    # inside each block rows belong to that block's expert and ascend
    flat = ids.reshape(-1)
    for b, e in enumerate(eb):
        rows = st[b * B:(b + 1) * B]
        rows = rows[rows < R]
        if e < 0:
            assert len(rows) == 0
        else:
            assert np.all(flat[rows] == e) and np.all(np.diff(rows) > 0)
    # the data round trip: permute a payload into sorted order and back
    payload = rng.standard_normal(R)
    perm = np.zeros(len(st))
    perm[st < R] = payload[st[st < R]]
    np.testing.assert_array_equal(perm[inv], payload)
