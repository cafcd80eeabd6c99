"""Pins of the oracle's ragged-batch and end-of-sequence rules.

* Ragged batches ([WR] §11.2, [MN] §九 point 3: gamma is adapted per
  request): a packed batch must give, request by request, what the
  single-request verify gives on that request's own gamma_b rows.  The test
  builds the packed arrays by concatenation from padded ones, a construction
  independent of the oracle's offset arithmetic.
* End of sequence ([WR] §14.3: nothing is committed after an EOS): the
  output with an EOS id is the output without it, cut after its first EOS;
  and by exact enumeration the emitted law is still the target's, with
  nothing ever following an EOS.
"""

import itertools

import numpy as np
import pytest

import oracle

EOS = 1


def _rows(rng, n, V):
    p = rng.dirichlet(np.ones(V), size=n)
    return np.log(p)


def _cut(tokens, eos):
    t = [int(x) for x in tokens if x >= 0]
    if eos in t:
        t = t[: t.index(eos) + 1]
    return t


def test_eos_output_is_the_cut_output():
    rng = np.random.default_rng(5)
    V, G = 4, 3
    n_cut = n_tail = 0
    for _ in range(400):
        z = _rows(rng, G + 1, V)
        q = rng.dirichlet(np.ones(V), size=G)
        ids = rng.integers(0, V, G)
        ua, ur = rng.random(G), rng.random(G + 1)
        plain = oracle.verify_request(z, q, ids, ua, ur, 1.0)
        cut = oracle.verify_request(z, q, ids, ua, ur, 1.0, eos=EOS)
        exp = _cut(plain.tokens, EOS)
        got = [int(x) for x in cut.tokens if x >= 0]
        assert got == exp
        assert (cut.tokens[len(got):] == -1).all()
        # the last emitted token is at slot n_accepted
        assert cut.n_accepted == len(got) - 1
        assert bool(cut.flags & oracle.FLAG_EOS) == (EOS in got)
        assert (cut.flags & ~oracle.FLAG_EOS) == (plain.flags & ~oracle.FLAG_EOS) or EOS in got
        if EOS in got and len(got) < plain.n_accepted + 1:
            n_cut += 1
        if got and got[-1] == EOS and len(got) == plain.n_accepted + 1:
            n_tail += 1
    assert n_cut > 20 and n_tail > 20  # both ways of emitting an EOS occur


def test_eos_accepted_draft_stops_verification():
    """p = q: every draft passes (u < 1); the accepted EOS ends the output,
    no token is drawn and later positions are never evaluated."""
    p = np.array([[0.25, 0.25, 0.25, 0.25]] * 4)
    q = p[:3].copy()
    q[2] = 0.0  # position 2 would raise Q_ZERO if it were evaluated
    r = oracle.verify_from_processed(list(p), list(q), [2, EOS, 3], [0.9, 0.9, 0.9], [0.5] * 4, eos=EOS)
    assert r.tokens.tolist() == [2, EOS, -1, -1]
    assert r.n_accepted == 1 and r.flags == oracle.FLAG_EOS
    # an EOS that is rejected is replaced as usual and nothing is cut
    p2 = np.array([[0.5, 0.0, 0.5]] * 3)
    q2 = np.array([[0.0, 1.0, 0.0]] * 2)
    r = oracle.verify_from_processed(list(p2), list(q2), [EOS, 0], [0.3, 0.3], [0.2, 0.2, 0.2], eos=EOS)
    assert r.n_accepted == 0 and r.tokens.tolist() == [0, -1, -1] and r.flags == 0


def test_eos_as_the_drawn_token():
    """A bonus token equal to EOS is emitted and flagged; nothing to cut."""
    p = [np.array([1.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0])]
    r = oracle.verify_from_processed(p, [np.array([1.0, 0.0, 0.0])], [0], [0.5], [0.5, 0.5], eos=EOS)
    assert r.tokens.tolist() == [0, EOS] and r.n_accepted == 1 and r.flags == oracle.FLAG_EOS


def _grid(K):
    return (np.arange(K) + 0.5) / K


def test_eos_enumerated_law():
    """gamma = 2, V = 3, EOS = 1: slot 0 ~ p_0; nothing follows an EOS; a
    slot that exists after a non-EOS token is distributed as that position's
    p ([WR] §5.1 proof applied slot by slot); and the chance that slot 1
    exists after token x is what it is without the EOS rule."""
    # every acceptance ratio and CDF step is a multiple of 1/K, so the
    # midpoint grids integrate the uniforms exactly
    p = [np.array([0.5, 0.3, 0.2]), np.array([0.2, 0.3, 0.5]), np.array([0.6, 0.1, 0.3])]
    q = [np.array([0.25, 0.5, 0.25]), np.array([0.25, 0.25, 0.5])]
    K = 10
    law, law_plain = {}, {}
    for ids in itertools.product(range(3), repeat=2):
        wq = q[0][ids[0]] * q[1][ids[1]]
        for ua in itertools.product(_grid(K), repeat=2):
            for v in _grid(K):
                w = wq / K ** 3
                r = oracle.verify_from_processed(p, q, list(ids), list(ua), [v] * 3, eos=EOS)
                key = tuple(int(x) for x in r.tokens if x >= 0)
                law[key] = law.get(key, 0.0) + w
                r0 = oracle.verify_from_processed(p, q, list(ids), list(ua), [v] * 3)
                key0 = tuple(int(x) for x in r0.tokens if x >= 0)
                law_plain[key0] = law_plain.get(key0, 0.0) + w
    assert sum(law.values()) == pytest.approx(1.0, abs=1e-12)
    for key in law:
        assert EOS not in key[:-1]
    slot0 = np.zeros(3)
    for key, pr in law.items():
        slot0[key[0]] += pr
    np.testing.assert_allclose(slot0, p[0], atol=1e-12)
    for s in (1, 2):
        # law of slot s given the tokens before it (none of them EOS)
        for prefix in itertools.product([0, 2], repeat=s):
            cond = np.zeros(3)
            for key, pr in law.items():
                if len(key) > s and key[:s] == prefix:
                    cond[key[s]] += pr
            if cond.sum() > 0:
                np.testing.assert_allclose(cond / cond.sum(), p[s], atol=1e-12)
            exists = sum(pr for key, pr in law_plain.items() if len(key) > s and key[:s] == prefix)
            assert cond.sum() == pytest.approx(exists, abs=1e-12)


def test_greedy_eos():
    rng = np.random.default_rng(9)
    for _ in range(300):
        z = rng.integers(0, 4, (4, 5)).astype(np.float64)
        g = np.argmax(z, axis=1)
        ids = np.where(rng.random(3) < 0.7, g[:3], rng.integers(0, 5, 3))
        plain = oracle.greedy_request(z, ids)
        cut = oracle.greedy_request(z, ids, eos=EOS)
        got = [int(x) for x in cut.tokens if x >= 0]
        assert got == _cut(plain.tokens, EOS)
        assert cut.n_accepted == len(got) - 1
        assert bool(cut.flags & oracle.FLAG_EOS) == (EOS in got)
    # [WR] §7.1-style chain: drafts match the argmax up to an EOS
    z = np.full((4, 5), 0.0)
    z[0, 3] = z[1, EOS] = z[2, 2] = z[3, 4] = 1.0
    r = oracle.greedy_request(z, [3, EOS, 2], eos=EOS)
    assert r.tokens.tolist() == [3, EOS, -1, -1] and r.n_accepted == 1 and r.flags == oracle.FLAG_EOS


def _packed(rng, B, G, V, gam):
    """Padded per-request arrays and their packed concatenation."""
    z = rng.normal(0, 1.5, (B, G + 1, V))
    q = rng.dirichlet(np.ones(V), size=(B, G))
    ids = rng.integers(0, V, (B, G))
    ua, ur = rng.random((B, G)), rng.random((B, G + 1))
    pk = dict(
        z=np.concatenate([z[b, : gam[b] + 1] for b in range(B)]),
        q=np.concatenate([q[b, : gam[b]] for b in range(B)]).reshape(-1, V),
        ids=np.concatenate([ids[b, : gam[b]] for b in range(B)]).astype(np.int64),
        ua=np.concatenate([ua[b, : gam[b]] for b in range(B)]),
        ur=np.concatenate([ur[b, : gam[b] + 1] for b in range(B)]),
        cu=np.concatenate([[0], np.cumsum(gam)]).astype(np.int64),
    )
    return (z, q, ids, ua, ur), pk


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (3, 1.0), (0, 0.8)])
def test_ragged_batch_is_per_request(top_k, top_p):
    rng = np.random.default_rng(21)
    B, G, V = 9, 4, 12
    gam = np.array([0, 4, 1, 3, 0, 2, 4, 4, 1])
    (z, q, ids, ua, ur), pk = _packed(rng, B, G, V, gam)
    for eos in (-1, 5):
        out = oracle.verify_sample_ragged(pk["z"], pk["q"], pk["ids"], pk["cu"], pk["ua"], pk["ur"], G, 0.9,
                                          top_k, top_p, eos)
        gr = oracle.verify_greedy_ragged(pk["z"], pk["ids"], pk["cu"], G, eos)
        for b in range(B):
            g = gam[b]
            r = oracle.verify_request(z[b, : g + 1], q[b, :g], ids[b, :g], ua[b, :g], ur[b, : g + 1], 0.9, top_k,
                                      top_p, eos)
            assert out["tokens"][b].tolist() == r.tokens.tolist() + [-1] * (G - g)
            assert out["n_accepted"][b] == r.n_accepted and out["flags"][b] == r.flags
            rg = oracle.greedy_request(z[b, : g + 1], ids[b, :g], eos)
            assert gr["tokens"][b].tolist() == rg.tokens.tolist() + [-1] * (G - g)
            assert gr["n_accepted"][b] == rg.n_accepted and gr["flags"][b] == rg.flags
    # gamma_b = 0 is plain sampling from that request's single row
    assert out["n_accepted"][0] == 0 and out["tokens"][0][1:].tolist() == [-1] * G


def test_ragged_bad_spans():
    """Out-of-order, out-of-range and too-long spans emit nothing and are
    flagged; the other requests are unaffected."""
    rng = np.random.default_rng(4)
    B, G, V = 5, 3, 7
    gam = np.array([2, 3, 1, 0, 2])
    _, pk = _packed(rng, B, G, V, gam)
    ref = oracle.verify_sample_ragged(pk["z"], pk["q"], pk["ids"], pk["cu"], pk["ua"], pk["ur"], G, 1.0)
    for bad_cu, bad in (
        ([0, 2, 1, 6, 6, 8], {1}),           # request 1 ends before it starts
        ([0, 2, 5, 6, 6, 9], {4}),           # request 4 runs past N = 8
        ([0, 2, 5, 6, 6, 8], set()),         # the valid offsets
        ([-1, 2, 5, 6, 6, 8], {0}),          # negative start
    ):
        out = oracle.verify_sample_ragged(pk["z"], pk["q"], pk["ids"], np.array(bad_cu), pk["ua"], pk["ur"], G, 1.0)
        for b in range(B):
            if b in bad:
                assert out["flags"][b] == oracle.FLAG_BAD_SPAN and out["n_accepted"][b] == 0
                assert (out["tokens"][b] == -1).all()
            elif bad_cu[b] == pk["cu"][b] and bad_cu[b + 1] == pk["cu"][b + 1]:
                assert out["tokens"][b].tolist() == ref["tokens"][b].tolist()
    # a span longer than gamma_max
    out = oracle.verify_sample_ragged(pk["z"], pk["q"], pk["ids"], pk["cu"], pk["ua"], pk["ur"], 2, 1.0)
    assert out["flags"][1] == oracle.FLAG_BAD_SPAN and out["tokens"].shape == (B, 3)
    assert out["flags"][0] != oracle.FLAG_BAD_SPAN


def test_ragged_draft_logits_is_per_request():
    """Ragged batch with q from the draft's logits: request by request, the
    single-request draft-logits verify on that request's own rows."""
    rng = np.random.default_rng(8)
    B, G, V = 6, 3, 10
    gam = np.array([3, 0, 2, 1, 3, 2])
    (z, q, ids, ua, ur), pk = _packed(rng, B, G, V, gam)
    dz = rng.normal(0, 1.5, (B, G, V))
    dz_pk = np.concatenate([dz[b, : gam[b]] for b in range(B)]).reshape(-1, V)
    for top_k, top_p in ((0, 1.0), (4, 1.0), (0, 0.7)):
        out = oracle.verify_sample_ragged_draft_logits(pk["z"], dz_pk, pk["ids"], pk["cu"], pk["ua"], pk["ur"], G,
                                                       0.9, top_k, top_p)
        for b in range(B):
            g = gam[b]
            r = oracle.verify_request_draft_logits(z[b, : g + 1], dz[b, :g], ids[b, :g], ua[b, :g],
                                                   ur[b, : g + 1], 0.9, top_k, top_p)
            assert out["tokens"][b].tolist() == r.tokens.tolist() + [-1] * (G - g)
            assert out["n_accepted"][b] == r.n_accepted and out["flags"][b] == r.flags
