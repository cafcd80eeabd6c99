"""Pins of the oracle's draft-logits path (q formed in the library).

q_j is the draft's logits row put through the same processing as p_j
([WR] §2.3, [MN] §二: p and q are both the distributions after the decoding
rules).  These CPU tests pin that composition to what the pages and the
mathematics fix:

* the pages' worked examples, fed as draft logits ln q (tests/golden);
* brute-force kept sets and closed-form temperature of q;
* exact enumeration: the emitted-token law is p also when the draft's kept
  set differs from the target's ([WR] §7.3);
* the zero-q and non-finite rules at ids outside the draft's kept set and on
  rows without a q.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def ln(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


@pytest.mark.parametrize("ex", GOLDEN["single_position"], ids=lambda e: e["id"])
def test_worked_examples_through_draft_logits(ex):
    p = np.array(ex["p"])
    q = np.array(ex["q"])
    drafts = [ex["draft"]] if "draft" in ex else list(range(len(p)))
    expected_a = [ex["accept_prob"]] if "accept_prob" in ex else ex["accept_prob_per_draft"]
    for d, a_exp in zip(drafts, expected_a):
        z_rows = np.stack([ln(p), ln(p)])
        alpha, z_pq, z_qp, a = oracle.stats_request_draft_logits(z_rows, ln(q)[None], [d], 1.0)
        assert a[0] == pytest.approx(a_exp, abs=1e-12)
        assert alpha[0] == pytest.approx(ex["alpha"], abs=1e-12)
        assert z_pq[0] == pytest.approx(ex["Z"], abs=1e-12)
        assert z_qp[0] == pytest.approx(ex["Z"], abs=1e-12)
        if a_exp < 1.0:
            # just above the acceptance probability: rejected, replaced from the residual
            res = oracle.verify_request_draft_logits(z_rows, ln(q)[None], [d], [a_exp + 1e-3], [0.5, 0.5], 1.0)
            assert res.n_accepted == 0
            assert res.tokens.tolist() == [int(np.argmax(ex["residual"])), -1]
            res = oracle.verify_request_draft_logits(z_rows, ln(q)[None], [d], [a_exp - 1e-3], [0.5, 0.0], 1.0)
            assert res.n_accepted == 1 and res.tokens[0] == d


def test_q_kept_set_brute_force():
    """Draft top-k keeps the k largest draft logits (ties kept) and
    renormalises softmax(z / T) over them; top-p the smallest most probable
    prefix of mass >= top_p."""
    rng = np.random.default_rng(7)
    V, T = 9, 0.7
    dz = rng.normal(0, 2, (3, V))
    for k in (1, 3, 5):
        rows, _ = oracle.draft_q_rows(dz, T, top_k=k)
        for z, q in zip(dz, rows):
            keep = np.zeros(V, bool)
            keep[np.argsort(-z)[:k]] = True
            e = np.where(keep, np.exp((z - z.max()) / np.float32(T)), 0.0)
            np.testing.assert_allclose(q, e / e.sum(), rtol=1e-13, atol=0)
    rows, _ = oracle.draft_q_rows(dz, T, top_p=0.6)
    for z, q in zip(dz, rows):
        e = np.exp((z - z.max()) / np.float32(T))
        full = e / e.sum()
        order = np.argsort(-full)
        n = int(np.nonzero(np.cumsum(full[order]) >= np.float32(0.6))[0][0]) + 1
        keep = np.zeros(V, bool)
        keep[order[:n]] = True
        np.testing.assert_allclose(q, np.where(keep, full, 0) / full[keep].sum(), rtol=1e-13, atol=0)


def test_draft_temperature_closed_form():
    """q = softmax(z / T): for two tokens q_0 = 1 / (1 + exp((z1 - z0) / T))."""
    for T in (0.25, 1.0, 3.0):
        rows, _ = oracle.draft_q_rows(np.array([[1.0, 2.5]]), T)
        Tf = float(np.float32(T))
        assert rows[0][0] == pytest.approx(1.0 / (1.0 + np.exp(1.5 / Tf)), rel=1e-14)


def _grid(K):
    return (np.arange(K) + 0.5) / K


def _law(z_rows, dz_rows, q_rows, K, top_k=0):
    gamma = len(dz_rows)
    V = len(z_rows[0])
    law = {}
    for ids in itertools.product(range(V), repeat=gamma):
        wq = np.prod([q_rows[j][ids[j]] for j in range(gamma)])
        if wq == 0:
            continue
        for ua in itertools.product(_grid(K), repeat=gamma):
            for v in _grid(K):
                r = oracle.verify_request_draft_logits(z_rows, dz_rows, ids, ua, [v] * (gamma + 1), 1.0, top_k)
                key = tuple(r.tokens[: r.n_accepted + 1].tolist())
                law[key] = law.get(key, 0.0) + wq / K ** (gamma + 1)
    return law


def test_enumerated_law_is_p():
    """gamma = 1 from logits on both sides: first slot ~ p_0, acceptance
    = sum min(p_0, q_0), second slot ~ p_1 ([WR] §5.1 proof, [BS] §五)."""
    p0 = np.array([0.5, 0.3, 0.2])
    q0 = np.array([0.25, 0.5, 0.25])
    p1 = np.array([0.1, 0.6, 0.3])
    law = _law(np.stack([ln(p0), ln(p1)]), ln(q0)[None], [q0], K=20)
    first, second, acc = np.zeros(3), np.zeros(3), 0.0
    for key, pr in law.items():
        first[key[0]] += pr
        if len(key) == 2:
            acc += pr
            second[key[1]] += pr
    np.testing.assert_allclose(first, p0, atol=1e-12)
    assert acc == pytest.approx(np.minimum(p0, q0).sum(), abs=1e-12)
    np.testing.assert_allclose(second / acc, p1, atol=1e-12)


def test_enumerated_law_with_different_kept_sets():
    """top-k = 2 on both sides with different top-2 sets ([WR] §7.3): the
    draft never proposes the target's second token, which then comes only
    from the residual, and the emitted law is still the processed p."""
    zt = ln([0.4, 0.4, 0.15, 0.05])   # target keeps {0, 1}: p = (1/2, 1/2, 0, 0)
    zd = ln([0.6, 0.1, 0.2, 0.1])     # draft keeps {0, 2}: q = (3/4, 0, 1/4, 0)
    p = np.array([0.5, 0.5, 0.0, 0.0])
    q = np.array([0.75, 0.0, 0.25, 0.0])
    rows, _ = oracle.draft_q_rows(zd[None], 1.0, top_k=2)
    np.testing.assert_allclose(rows[0], q, atol=1e-15)
    # acceptance 2/3 at id 0, 0 at id 2; the residual is the single point 1
    law = _law(np.stack([zt, zt]), zd[None], [q], K=30, top_k=2)
    first = np.zeros(4)
    for key, pr in law.items():
        first[key[0]] += pr
    np.testing.assert_allclose(first, p, atol=1e-12)
    # a draft id outside the draft's kept set has q(d) = 0: accepted iff p(d) > 0
    r = oracle.verify_request_draft_logits(np.stack([zt, zt]), zd[None], [1], [0.99], [0.5, 0.5], 1.0, 2)
    assert r.flags & oracle.FLAG_Q_ZERO and r.n_accepted == 1
    r = oracle.verify_request_draft_logits(np.stack([zt, zt]), zd[None], [3], [0.01], [0.5, 0.5], 1.0, 2)
    assert r.flags & oracle.FLAG_Q_ZERO and r.n_accepted == 0


def test_z_identity_from_logits():
    """Both sides normalised: Z = Z' = 1 - alpha ([RL] §2, [BS] §五)."""
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, (4, 50))
    dz = z[:3] + rng.normal(0, 1, (3, 50))
    for top_k, top_p in ((0, 1.0), (7, 1.0), (0, 0.8), (10, 0.9)):
        alpha, zpq, zqp, _ = oracle.stats_request_draft_logits(z, dz, [0, 1, 2], 0.9, top_k, top_p)
        np.testing.assert_allclose(zpq, 1 - alpha, atol=1e-13)
        np.testing.assert_allclose(zqp, 1 - alpha, atol=1e-13)


def test_draft_row_without_q():
    """A NaN / +Inf / all -Inf draft row gives a NaN q row: a valid id there
    makes the request non-finite; the statistics of that position are NaN."""
    z = np.log(np.array([[0.5, 0.3, 0.2]] * 3))
    for bad in (np.nan, np.inf):
        dz = np.log(np.array([[0.2, 0.3, 0.5], [0.2, 0.3, 0.5]]))
        dz[1, 2] = bad
        r = oracle.verify_request_draft_logits(z, dz, [0, 1], [0.1, 0.1], [0.5, 0.5, 0.5], 1.0)
        assert r.flags == oracle.FLAG_NONFINITE and r.n_accepted == 0
        st = oracle.stats_request_draft_logits(z, dz, [0, 1], 1.0)
        assert np.isfinite(st[:, 0]).all() and np.isnan(st[:, 1]).all()
    dz = np.log(np.array([[0.2, 0.3, 0.5], [0.2, 0.3, 0.5]]))
    dz[0] = -np.inf
    r = oracle.verify_request_draft_logits(z, dz, [0, 1], [0.1, 0.1], [0.5, 0.5, 0.5], 1.0)
    assert r.flags == oracle.FLAG_NONFINITE


def test_same_as_dense_oracle_on_processed_q():
    """The batched draft-logits functions equal the q-input ones fed the
    processed draft rows (composition, on random rows with truncation)."""
    rng = np.random.default_rng(11)
    B, G, V = 5, 3, 40
    z = rng.normal(0, 2, (B, G + 1, V))
    dz = z[:, :G] + rng.normal(0, 0.7, (B, G, V))
    ids = rng.integers(0, V, (B, G))
    ua = rng.random((B, G))
    ur = rng.random((B, G + 1))
    for top_k, top_p in ((0, 1.0), (6, 1.0), (0, 0.85)):
        q = np.stack([np.stack(oracle.draft_q_rows(dz[b], 0.8, top_k, top_p)[0]) for b in range(B)])
        a = oracle.verify_sample_draft_logits(z, dz, ids, ua, ur, 0.8, top_k, top_p)
        b = oracle.verify_sample(z, q, ids, ua, ur, 0.8, top_k, top_p)
        for key in ("tokens", "n_accepted", "flags"):
            np.testing.assert_array_equal(a[key], b[key])
        sa = oracle.accept_stats_draft_logits(z, dz, ids, 0.8, top_k, top_p)
        sb = oracle.accept_stats(z, q, ids, 0.8, top_k, top_p)
        for x, y in zip(sa, sb):
            np.testing.assert_array_equal(x, y)
