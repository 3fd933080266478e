"""Pins of the oracle's top-k softmax gate against brute force, closed forms
and invariants (CPU only).

The gate is the fused softmax + top-k op of the "Upstream Reference:
Deep-Spark xllm + vllm" page, section "Call Chain: MoE topk_softmax on
BI-V100".  Equal logits go to the lower expert index.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


def _beats(v, a, b):
    """a ranks above b: larger logit, or equal logit and lower index."""
    return v[a] > v[b] or (v[a] == v[b] and a < b)


def brute_force_topk(v, K):
    """Enumerate all K-subsets; exactly one has every member ranking above
    every non-member.  Order the members by how many other members each one
    beats (a count, not a sort)."""
    E = len(v)
    found = []
    for S in itertools.combinations(range(E), K):
        rest = [j for j in range(E) if j not in S]
        if all(_beats(v, a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    S = found[0]
    ranked = [None] * K
    for a in S:
        wins = sum(_beats(v, a, b) for b in S if b != a)
        ranked[K - 1 - wins] = a
    return ranked


def test_exhaustive_small_alphabet_all_tie_shapes():
    # every row of 6 experts with values in {0, 1, 2}: 729 rows, every tie shape
    rows = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=6)), dtype=np.float32)
    for K in range(1, 7):
        _, ids, _ = oracle.topk_softmax(rows, K, False, "f32")
        for t in range(rows.shape[0]):
            assert list(ids[t]) == brute_force_topk(rows[t].astype(np.float64), K), (rows[t], K)


def test_random_rows_vs_brute_force():
    rng = np.random.default_rng(7)
    for E in (1, 2, 3, 5, 8):
        for K in range(1, E + 1):
            v = rng.standard_normal((40, E)).astype(np.float32)
            v[::3, 0] = v[::3, -1]  # force some ties
            _, ids, _ = oracle.topk_softmax(v, K, False, "f32")
            for t in range(v.shape[0]):
                assert list(ids[t]) == brute_force_topk(v[t].astype(np.float64), K)


def test_bf16_rows_vs_brute_force():
    # bf16 logits (2*N(0,1)) tie often; brute force on 8-expert rows
    bits = synth.gate_logits_bf16(300, 8, seed=3)
    for K in (1, 2, 4, 8):
        _, ids, _ = oracle.topk_softmax(bits, K, False, "bf16")
        v = oracle.decode_bf16(bits)
        for t in range(bits.shape[0]):
            assert list(ids[t]) == brute_force_topk(v[t], K)


def test_k1_is_first_argmax():
    bits = synth.gate_logits_bf16(2000, 160, seed=1, tie_fraction=0.5)
    _, ids, _ = oracle.topk_softmax(bits, 1, False, "bf16")
    assert np.array_equal(ids[:, 0], np.argmax(oracle.decode_bf16(bits), axis=1))


def test_signed_zero_is_a_tie():
    # -0.0 and +0.0 are the same logit: the lower index wins
    v = np.array([[-1.0, -0.0, 0.0, -2.0], [-1.0, 0.0, -0.0, -2.0]], dtype=np.float32)
    _, ids, _ = oracle.topk_softmax(v, 2, False, "f32")
    assert ids.tolist() == [[1, 2], [1, 2]]


def test_softmax_closed_forms():
    # two experts: p0 = 1 / (1 + exp(v1 - v0))
    v = np.array([[0.5, -1.25]], dtype=np.float32)
    w, ids, _ = oracle.topk_softmax(v, 2, False, "f32")
    assert ids.tolist() == [[0, 1]]
    assert w[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-1.75)), rel=1e-15)
    # logits log(1), log(2), log(3): probabilities 1/6, 2/6, 3/6
    v64 = np.log(np.array([[1.0, 2.0, 3.0]], dtype=np.float64))
    w, ids, _ = oracle.topk_softmax(v64, 3, False, "f32")
    assert ids.tolist() == [[2, 1, 0]]
    np.testing.assert_allclose(w[0], [0.5, 1 / 3, 1 / 6], rtol=1e-14)
    # all-equal row: uniform weights, ids 0..K-1
    w, ids, _ = oracle.topk_softmax(np.zeros((1, 10), np.float32), 4, False, "f32")
    assert ids.tolist() == [[0, 1, 2, 3]]
    np.testing.assert_allclose(w, 0.1, rtol=1e-15)
    w, ids, _ = oracle.topk_softmax(np.zeros((1, 10), np.float32), 4, True, "f32")
    np.testing.assert_allclose(w, 0.25, rtol=1e-15)


def test_invariants_on_gate_workload():
    c = synth.gate_case(160, T=2048, K=8, seed=5)
    v = oracle.decode_bf16(c.logits)
    # with K = E and no renormalisation the weights are the whole softmax: sum 1
    w_all, ids_all, _ = oracle.topk_softmax(c.logits, 160, False, "bf16")
    np.testing.assert_allclose(w_all.sum(axis=1), 1.0, rtol=0, atol=160 * 2.0 ** -52)
    assert np.all(np.sort(ids_all, axis=1) == np.arange(160))
    w, ids, tei = oracle.topk_softmax(c.logits, 8, False, "bf16")
    assert np.all(np.diff(w, axis=1) <= 0)  # best first
    # chosen logits are non-increasing, and equal logits appear in index order
    cv = np.take_along_axis(v, ids.astype(np.int64), axis=1)
    assert np.all(np.diff(cv, axis=1) <= 0)
    eq = np.diff(cv, axis=1) == 0
    assert np.all(np.diff(ids, axis=1)[eq] > 0)
    # every unchosen logit is <= the K-th chosen one (and if equal, has a larger index)
    for t in range(0, 2048, 17):
        rest = np.setdiff1d(np.arange(160), ids[t])
        assert np.all((v[t, rest] < cv[t, -1]) | ((v[t, rest] == cv[t, -1]) & (rest > ids[t, -1])))
    wr, idsr, _ = oracle.topk_softmax(c.logits, 8, True, "bf16")
    assert np.array_equal(idsr, ids)
    np.testing.assert_allclose(wr.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(wr, w / w.sum(axis=1, keepdims=True), rtol=1e-14)
    # token_expert_indices is a permutation of 0..T*K-1, k-major
    assert np.array_equal(np.sort(tei.reshape(-1)), np.arange(2048 * 8))
    assert tei[5, 3] == 3 * 2048 + 5


def test_shift_invariance():
    rng = np.random.default_rng(11)
    v = (rng.integers(-64, 64, size=(200, 24)) / 8.0).astype(np.float32)  # exact in f32, many ties
    w0, i0, _ = oracle.topk_softmax(v, 6, False, "f32")
    w1, i1, _ = oracle.topk_softmax(v + np.float32(3.0), 6, False, "f32")
    assert np.array_equal(i0, i1)
    np.testing.assert_allclose(w0, w1, rtol=1e-13)


def test_injected_ties_present():
    c = synth.gate_case(128, T=65536, K=8, seed=0)
    v = c.logits
    n_tie_rows = sum(len(np.unique(v[t])) < v.shape[1] for t in range(0, 65536, 64))
    assert n_tie_rows > 0


# ---------------------------------------------------------------------------
# sigmoid-scoring gate


def test_sigmoid_ids_equal_softmax_ids():
    # the sigmoid and the softmax are both increasing in the logit, so the
    # chosen experts (already pinned by brute force) must be identical
    rng = np.random.default_rng(21)
    for E, K in ((8, 2), (40, 6), (128, 8), (160, 8)):
        x = (rng.integers(-3, 4, size=(300, E)) * 0.5).astype(np.float32)  # many ties
        _, ids_s, tei_s = oracle.topk_sigmoid(x, K, False)
        _, ids_m, tei_m = oracle.topk_softmax(x, K, False)
        assert np.array_equal(ids_s, ids_m) and np.array_equal(tei_s, tei_m)


def test_sigmoid_closed_forms():
    x = np.array([[0.0, np.log(3.0), -np.log(3.0), -5.0]], dtype=np.float64)
    w, ids, _ = oracle.topk_sigmoid(x, 2, False, "f32")
    assert ids.tolist() == [[1, 0]]
    assert w[0, 0] == pytest.approx(0.75, abs=1e-15) and w[0, 1] == 0.5
    w, _, _ = oracle.topk_sigmoid(x, 2, True, "f32")
    assert w[0].tolist() == pytest.approx([0.6, 0.4], abs=1e-15)


def test_sigmoid_symmetry_and_independence():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((50, 16)) * 3
    w_pos, ids, _ = oracle.topk_sigmoid(x, 16, False, "f32")
    # with K = E every expert is chosen: s(x) + s(-x) = 1 for each of them
    w_neg, ids_n, _ = oracle.topk_sigmoid(-x, 16, False, "f32")
    sp = np.zeros_like(x)
    sn = np.zeros_like(x)
    np.put_along_axis(sp, ids.astype(np.int64), w_pos, axis=1)
    np.put_along_axis(sn, ids_n.astype(np.int64), w_neg, axis=1)
    assert np.allclose(sp + sn, 1.0, atol=1e-15)
    # unlike the softmax, a chosen weight does not depend on the other logits
    w1, ids1, _ = oracle.topk_sigmoid(x, 4, False, "f32")
    y = x.copy()
    for t in range(x.shape[0]):
        others = np.setdiff1d(np.arange(16), ids1[t])
        y[t, others] -= 1.0  # lower the losers: same winners
    w2, ids2, _ = oracle.topk_sigmoid(y, 4, False, "f32")
    assert np.array_equal(ids1, ids2) and np.array_equal(w1, w2)


def test_sigmoid_renormalised_sums_to_one():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((200, 64)).astype(np.float32) * 2
    w, _, _ = oracle.topk_sigmoid(x, 8, True)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
