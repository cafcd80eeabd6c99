"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU (no GPU marker).  The pins are chosen so that
a plausible slip anywhere in the oracle (a dropped term, a swapped p/q, a
wrong index, a non-strict comparison, a missing bonus token, resampling from
p instead of the residual) fails at least one of them:

* worked examples printed on the pages (tests/golden/worked_examples.json);
* the identity Z = sum (p-q)_+ = sum (q-p)_+ = 1 - alpha = P(reject);
* exact enumeration of the output law on tiny rational inputs (draft ids
  weighted by q, uniforms on a grid whose points never touch a boundary);
* closed forms for temperature, E[N] and the truncated geometric law;
* brute-force definitions of the top-k / top-p kept sets and of argmax.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def ln(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ex", GOLDEN["single_position"], ids=lambda e: e["id"])
def test_single_position_examples(ex):
    p = np.array(ex["p"])
    q = np.array(ex["q"])
    # Through the logits path: logits = ln p with T = 1 must give p back.
    proc = oracle.process_row(ln(p), 1.0)
    np.testing.assert_allclose(proc.p, p, rtol=0, atol=1e-15)
    drafts = [ex["draft"]] if "draft" in ex else list(range(len(p)))
    expected_a = [ex["accept_prob"]] if "accept_prob" in ex else ex["accept_prob_per_draft"]
    for d, a_exp in zip(drafts, expected_a):
        z_rows = np.stack([ln(p), ln(p)])  # position 0 verifies, position 1 is the bonus row
        alpha, z_pq, z_qp, a = oracle.stats_request(z_rows, q[None], [d], 1.0)
        assert a[0] == pytest.approx(a_exp, abs=1e-12)
        assert alpha[0] == pytest.approx(ex["alpha"], abs=1e-12)
        assert z_pq[0] == pytest.approx(ex["Z"], abs=1e-12)
        assert z_qp[0] == pytest.approx(ex["Z"], abs=1e-12)
    w = oracle.residual_weights(p, q)
    if "residual_unnormalised" in ex:
        np.testing.assert_allclose(w, ex["residual_unnormalised"], atol=1e-15)
    np.testing.assert_allclose(w / w.sum(), ex["residual"], atol=1e-12)
    # A rejected draft is replaced from the residual: with a one-point
    # residual every uniform gives that token.
    d = drafts[-1]
    a_d = min(1.0, p[d] / q[d])
    if a_d < 1.0:
        for ur in (0.0, 0.3, 0.999):
            res = oracle.verify_from_processed([p, p], [q], [d], [a_d + 1e-3], [ur, 0.5])
            assert res.n_accepted == 0
            assert res.tokens.tolist() == [int(np.argmax(ex["residual"])), -1]
        res = oracle.verify_from_processed([p, p], [q], [d], [a_d - 1e-3], [0.5, 0.0])
        assert res.n_accepted == 1 and res.tokens[0] == d


def test_monte_carlo_single_step():
    """The single-position Monte-Carlo of [WR] §8: output law p, acceptance alpha."""
    mc = GOLDEN["monte_carlo"]
    p = np.array(mc["p"])
    q = np.array(mc["q"])
    n = mc["trials"]
    rng = np.random.default_rng(2024)
    cdf_q = np.cumsum(q)
    d = np.minimum(np.searchsorted(cdf_q, rng.random(n), side="right"), 2)
    ua = rng.random(n)
    ur = rng.random(n)
    counts = np.zeros(3)
    acc = 0
    for i in range(n):
        r = oracle.verify_from_processed([p, p], [q], [d[i]], [ua[i]], [ur[i], 0.5])
        counts[r.tokens[0]] += 1
        acc += r.n_accepted
    sigma = np.sqrt(np.array(mc["expected_output_law"]) * 0.5 / n) * 2
    assert np.all(np.abs(counts / n - mc["expected_output_law"]) < 4 * sigma + 1e-9)
    assert abs(acc / n - mc["expected_accept_rate"]) < 4 * math.sqrt(0.75 * 0.25 / n)


@pytest.mark.parametrize("ex", GOLDEN["greedy"], ids=lambda e: e["id"])
def test_greedy_examples(ex):
    if "p" in ex:
        z = np.stack([ln(ex["p"]), ln(ex["p"])])
        r = oracle.greedy_request(z, [ex["draft"]])
        assert r.n_accepted == ex["n_accepted"]
        assert r.tokens[: r.n_accepted + 1].tolist() == ex["emitted"]
        return
    V = len(ex["vocab"])
    top1 = ex["target_top1_first4"] + [3]
    z = np.full((5, V), -1.0)
    for j, t in enumerate(top1):
        z[j, t] = 2.0
    r = oracle.greedy_request(z, ex["drafts"])
    assert r.n_accepted == ex["n_accepted"]
    assert r.tokens[: r.n_accepted + 1].tolist() == ex["emitted"]
    # Had the target's fourth top-1 been the draft's "dog", all four pass and
    # the bonus position adds a fifth token.
    z2 = z.copy()
    z2[3] = -1.0
    z2[3, 3] = 2.0
    r2 = oracle.greedy_request(z2, ex["drafts"])
    assert r2.n_accepted == 4 and (r2.tokens >= 0).sum() == ex["all_accepted_emits"]


# --------------------------------------------------------------------------
# Identities and closed forms
# --------------------------------------------------------------------------

def test_z_identity_and_reject_probability():
    """Z = sum(p-q)+ = sum(q-p)+ = 1 - sum min(p,q) = P(reject) ([RL] §2, [BS] §五)."""
    rng = np.random.default_rng(5)
    for V in (2, 3, 7, 50):
        for _ in range(20):
            p = rng.dirichlet(np.ones(V) * 0.7)
            q = rng.dirichlet(np.ones(V) * 0.7)
            z = np.stack([ln(p), ln(p)])
            alpha, zpq, zqp, _ = oracle.stats_request(z, q[None], [0], 1.0)
            proc = oracle.process_row(ln(p), 1.0).p
            reject = sum(q[y] * (1.0 - min(1.0, proc[y] / q[y])) for y in range(V) if q[y] > 0)
            assert zpq[0] == pytest.approx(zqp[0], abs=1e-12)
            assert zpq[0] == pytest.approx(1.0 - alpha[0], abs=1e-12)
            assert zpq[0] == pytest.approx(reject, abs=1e-12)
            # alpha = 1 - TV(p, q)  ([WR] §4.2, [MN] §三)
            assert alpha[0] == pytest.approx(1 - 0.5 * np.abs(proc - q).sum(), abs=1e-12)


def test_temperature_closed_form():
    """Two tokens: p(0) = 1 / (1 + exp((z1 - z0) / T)) ([WR] §7.2)."""
    for z0, z1, T in [(0.0, 1.0, 1.0), (2.0, -1.5, 0.7), (3.25, 3.0, 0.25), (-4.0, 5.0, 2.0)]:
        p = oracle.process_row([z0, z1], T).p
        Tf = float(np.float32(T))
        assert p[0] == pytest.approx(1.0 / (1.0 + math.exp((z1 - z0) / Tf)), rel=1e-14)
        assert p.sum() == pytest.approx(1.0, abs=1e-15)


def expected_tokens_closed_form(a, gamma):
    return (1 - a ** (gamma + 1)) / (1 - a)


def test_expected_tokens_table():
    """The closed form E = (1 - a^{g+1}) / (1 - a) reproduces the printed values."""
    et = GOLDEN["expected_tokens_per_round"]
    ex = et["WR-10-example"]
    assert sum(ex["a"] ** i for i in range(ex["gamma"] + 1)) == pytest.approx(ex["E"], abs=1e-12)
    assert expected_tokens_closed_form(ex["a"], ex["gamma"]) == pytest.approx(ex["E"], abs=1e-12)
    for e in et["MN-4-examples"]:
        assert round(expected_tokens_closed_form(e["a"], e["gamma"]), 2) == pytest.approx(e["E"])
    tab = et["MN-4-table"]
    for g, row in tab["rows"].items():
        for a, v in zip(tab["alpha"], row):
            assert round(expected_tokens_closed_form(a, int(g)), 2) == pytest.approx(v, abs=1e-9)


# --------------------------------------------------------------------------
# Exact enumeration of the output law on tiny rational inputs
# --------------------------------------------------------------------------

def _grid(K):
    return (np.arange(K) + 0.5) / K


def _enumerate_law(p_rows, q_rows, K):
    """Exact law of (n_accepted, emitted tokens) by enumeration.

    Draft ids are enumerated with weight prod_j q_j(d_j); each used uniform
    runs over a K-point midpoint grid.  Only u_accept[0..gamma-1] and one
    resample uniform are ever consumed, so all resample slots share one
    value.  With every probability a multiple of 1/K, no grid point sits on a
    decision boundary and the grid frequencies are exact.
    """
    gamma = len(q_rows)
    V = len(p_rows[0])
    law = {}
    for ids in itertools.product(range(V), repeat=gamma):
        wq = np.prod([q_rows[j][ids[j]] for j in range(gamma)])
        if wq == 0:
            continue
        for ua in itertools.product(_grid(K), repeat=gamma):
            for v in _grid(K):
                r = oracle.verify_from_processed(p_rows, q_rows, ids, ua, [v] * (gamma + 1))
                key = tuple(r.tokens[: r.n_accepted + 1].tolist())
                law[key] = law.get(key, 0.0) + wq / K ** (gamma + 1)
    return law


def test_enumerated_output_law_gamma1():
    """Marginal of the emitted token is p; the second slot (after acceptance)
    follows the bonus row ([WR] §5.1 proof, [BS] §五, [RL] §2 path table)."""
    p0 = np.array([0.5, 0.3, 0.2])
    q0 = np.array([0.25, 0.5, 0.25])
    p1 = np.array([0.1, 0.6, 0.3])
    law = _enumerate_law([p0, p1], [q0], K=20)
    first = np.zeros(3)
    second = np.zeros(3)
    acc = 0.0
    for key, pr in law.items():
        first[key[0]] += pr
        if len(key) == 2:
            acc += pr
            second[key[1]] += pr
    np.testing.assert_allclose(first, p0, atol=1e-12)
    assert acc == pytest.approx(np.minimum(p0, q0).sum(), abs=1e-12)
    np.testing.assert_allclose(second / acc, p1, atol=1e-12)


def test_enumerated_output_law_gamma2():
    """Two drafts: slot laws p_0, p_1, p_2 and E[N] = 1 + a_0 + a_0 a_1 ([WR] §6, §10)."""
    p = [np.array([0.4, 0.4, 0.2]), np.array([0.2, 0.2, 0.6]), np.array([0.7, 0.1, 0.2])]
    q = [np.array([0.2, 0.6, 0.2]), np.array([0.6, 0.2, 0.2])]
    law = _enumerate_law(p, q, K=30)
    slot = np.zeros((3, 3))
    reach = np.zeros(3)
    EN = 0.0
    for key, pr in law.items():
        EN += pr * len(key)
        for j, t in enumerate(key):
            slot[j, t] += pr
            reach[j] += pr
    for j in range(3):
        np.testing.assert_allclose(slot[j] / reach[j], p[j], atol=1e-12)
    a0 = np.minimum(p[0], q[0]).sum()
    a1 = np.minimum(p[1], q[1]).sum()
    assert EN == pytest.approx(1 + a0 + a0 * a1, abs=1e-12)


def test_support_mismatch_residual():
    """Target keeps {A,B,C}, draft only {A,B}: C comes only from the residual,
    with total probability p(C) ([WR] §7.3)."""
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.6, 0.4, 0.0])
    law = _enumerate_law([p, p], [q], K=12)  # acceptances 5/6 and 3/4
    pc = sum(pr for key, pr in law.items() if key[0] == 2)
    assert pc == pytest.approx(0.2, abs=1e-12)
    first = np.zeros(3)
    for key, pr in law.items():
        first[key[0]] += pr
    np.testing.assert_allclose(first, p, atol=1e-12)


def test_wrong_rule_fails_enumeration(monkeypatch):
    """Negative control ([WR] §8 closing remark, §13.3): resampling from the full
    p after a rejection breaks the law; the enumeration must notice."""
    p0 = np.array([0.5, 0.3, 0.2])
    q0 = np.array([0.25, 0.5, 0.25])
    monkeypatch.setattr(oracle.verify, "residual_weights", lambda p, q: np.asarray(p, dtype=np.float64))
    law = _enumerate_law([p0, p0], [q0], K=20)
    first = np.zeros(3)
    for key, pr in law.items():
        first[key[0]] += pr
    assert np.abs(first - p0).max() > 0.05


def test_inverse_cdf_grid_and_strictness():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    K = 40
    counts = np.zeros(5)
    for u in _grid(K):
        counts[oracle.inverse_cdf(w, u)[0]] += 1
    np.testing.assert_allclose(counts / K, w / w.sum(), atol=0)
    # t exactly on a running sum goes to the next token (strict >).
    assert oracle.inverse_cdf(w, 0.25)[0] == 3
    assert oracle.inverse_cdf(w, 0.0)[0] == 1
    assert oracle.inverse_cdf(w, 0.75)[0] == 4
    # unnormalised weights: only ratios matter
    assert oracle.inverse_cdf(w * 7.0, 0.3)[0] == oracle.inverse_cdf(w, 0.3)[0]
    tok, boundary = oracle.inverse_cdf(w, 0.25 + 1e-9)
    assert tok == 3 and boundary


# --------------------------------------------------------------------------
# Truncation, greedy and edge cases against brute-force definitions
# --------------------------------------------------------------------------

def test_top_k_matches_count_definition():
    """Kept set of top-k = tokens with fewer than k strictly larger logits."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        V = int(rng.integers(2, 12))
        z = rng.integers(-3, 4, size=V).astype(np.float64)  # many ties
        k = int(rng.integers(1, V + 2))
        r = oracle.process_row(z, 1.0, top_k=k)
        brute = np.array([(z > z[x]).sum() < k for x in range(V)]) if k < V else np.ones(V, bool)
        assert (r.kept == brute).all()
        e = np.where(brute, np.exp(z - z.max()), 0.0)
        np.testing.assert_allclose(r.p, e / e.sum(), rtol=1e-14, atol=0)


def test_top_p_matches_mass_definition():
    """Kept set of top-p = tokens whose strictly-more-probable mass is < top_p."""
    rng = np.random.default_rng(12)
    for _ in range(300):
        V = int(rng.integers(2, 10))
        z = rng.integers(-3, 4, size=V).astype(np.float64) * 0.5
        T = float(rng.choice([0.5, 1.0, 2.0]))
        top_p = float(np.float32(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95])))
        r = oracle.process_row(z, T, top_p=top_p)
        full = np.exp(z / T - (z / T).max())
        full /= full.sum()
        above = np.array([full[z > z[x]].sum() for x in range(V)])
        brute = above < top_p
        if np.any(np.abs(above - top_p) < 1e-9):
            continue  # exact tie with the threshold: either side is rounding
        assert (r.kept == brute).all(), (z, T, top_p)
        e = np.where(brute, full, 0.0)
        np.testing.assert_allclose(r.p, e / e.sum(), rtol=1e-12, atol=0)


def test_top_k_then_top_p():
    """top-p acts on the renormalised top-k distribution (processing order)."""
    z = np.array([3.0, 2.0, 2.0, 1.0, 0.0, -1.0])
    # top-4 keeps {0,1,2,3}; there p(0) = 1/(1 + 2/e + 1/e^2) = 0.534...
    r = oracle.process_row(z, 1.0, top_k=4, top_p=0.6)
    assert r.kept.tolist() == [True, True, True, False, False, False]
    # 0.52 lies between p(0) over the full row (0.5157) and over the top-4
    # set (0.534): top-k first keeps {0}; top-p alone would also keep the tie.
    assert oracle.process_row(z, 1.0, top_k=4, top_p=0.52).kept.tolist() == [True] + [False] * 5
    assert oracle.process_row(z, 1.0, top_p=0.52).kept.tolist() == [True, True, True, False, False, False]


def test_greedy_argmax_first_occurrence():
    rng = np.random.default_rng(13)
    for _ in range(300):
        V = int(rng.integers(1, 9))
        G = int(rng.integers(0, 4))
        z = rng.integers(-2, 3, size=(G + 1, V)).astype(np.float64)
        ids = rng.integers(0, V, size=G)
        g = []
        for j in range(G + 1):
            best = 0
            for x in range(V):
                if z[j, x] > z[j, best]:
                    best = x
            g.append(best)
        n = G
        for j in range(G):
            if ids[j] != g[j]:
                n = j
                break
        r = oracle.greedy_request(z, ids)
        assert r.n_accepted == n
        assert r.tokens[:n].tolist() == list(ids[:n]) and r.tokens[n] == g[n]
        assert (r.tokens[n + 1:] == -1).all()


def test_greedy_is_one_hot_limit_of_sampling():
    """One-hot p and q: the sampling rule accepts iff draft = argmax ([BS] §六)."""
    rng = np.random.default_rng(14)
    for _ in range(200):
        V, G = 6, 3
        z = rng.normal(size=(G + 1, V))
        ids = rng.integers(0, V, size=G)
        g = z.argmax(axis=1)
        p_rows = [np.eye(V)[g[j]] for j in range(G + 1)]
        q_rows = [np.eye(V)[ids[j]] for j in range(G)]
        s = oracle.verify_from_processed(p_rows, q_rows, ids, rng.random(G), rng.random(G + 1))
        gr = oracle.greedy_request(z, ids)
        assert s.n_accepted == gr.n_accepted
        assert s.tokens.tolist() == gr.tokens.tolist()


def test_special_cases():
    rng = np.random.default_rng(15)
    p = rng.dirichlet(np.ones(8))
    # p = q: nothing is ever rejected ([RL] §2: Z = 0 means p = q)
    for _ in range(50):
        ids = rng.integers(0, 8, size=3)
        r = oracle.verify_from_processed([p] * 4, [p] * 3, ids, rng.random(3), rng.random(4))
        assert r.n_accepted == 3 and r.flags == 0
    # disjoint supports: always rejected at position 0, replacement ~ p
    p2 = np.array([0.5, 0.5, 0.0, 0.0])
    q2 = np.array([0.0, 0.0, 0.5, 0.5])
    for u in _grid(10):
        r = oracle.verify_from_processed([p2, p2], [q2], [2], [0.0], [u, u])
        assert r.n_accepted == 0 and r.tokens[0] == (0 if u < 0.5 else 1)


def test_gamma_zero_is_plain_sampling():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    for u in _grid(20):
        r = oracle.verify_request(ln(p)[None], np.zeros((0, 4)), [], [], [u], 1.0)
        assert r.n_accepted == 0
        assert r.tokens.tolist() == [oracle.inverse_cdf(oracle.process_row(ln(p), 1.0).p, u)[0]]


def test_flags():
    p = np.array([0.5, 0.5, 0.0])
    q = np.array([0.5, 0.0, 0.5])
    # q(d) = 0 with p(d) > 0: accepted, flagged
    r = oracle.verify_from_processed([p, p], [q], [1], [0.99], [0.1, 0.1])
    assert r.n_accepted == 1 and r.flags == oracle.FLAG_Q_ZERO
    # bad id: rejected at its position, flagged
    r = oracle.verify_from_processed([p, p], [q], [7], [0.0], [0.1, 0.1])
    assert r.n_accepted == 0 and r.flags == oracle.FLAG_BAD_ID and r.tokens[0] == 1  # (p-q)+ = [0, .5, 0]
    # unnormalised q = 2p: a rejection leaves no residual -> sample from p
    p3 = np.array([0.25, 0.75])
    r = oracle.verify_from_processed([p3, p3], [2 * p3], [1], [0.9], [0.2, 0.5])
    assert r.n_accepted == 0 and r.flags == oracle.FLAG_Z_DEGENERATE and r.tokens[0] == 0
    # non-finite logits / q(d)
    z = np.array([[0.0, np.nan, 1.0], [0.0, 0.0, 0.0]])
    r = oracle.verify_request(z, [q], [0], [0.5], [0.5, 0.5], 1.0)
    assert r.flags == oracle.FLAG_NONFINITE and r.n_accepted == 0 and (r.tokens == -1).all()
    z = np.array([[0.0, np.inf, 1.0], [0.0, 0.0, 0.0]])
    assert oracle.verify_request(z, [q], [0], [0.5], [0.5, 0.5], 1.0).flags == oracle.FLAG_NONFINITE
    z = np.array([[0.0, -np.inf, 1.0], [-np.inf] * 3])
    assert oracle.verify_request(z, [q], [0], [0.5], [0.5, 0.5], 1.0).flags == oracle.FLAG_NONFINITE
    z = np.array([[0.0, -np.inf, 1.0], [0.0, 0.0, 0.0]])
    r = oracle.verify_request(z, [q], [0], [0.0], [0.5, 0.5], 1.0)
    assert r.flags == 0 and r.n_accepted == 1
    qn = np.array([np.nan, 0.5, 0.5])
    r = oracle.verify_request(np.zeros((2, 3)), [qn], [0], [0.5], [0.5, 0.5], 1.0)
    assert r.flags == oracle.FLAG_NONFINITE


def test_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == np.inf and v[3] == -np.inf
    assert v[4] == 2.0 ** -133 and v[5] == 0.0 and math.copysign(1, v[5]) < 0
    assert v[6] == 3.140625
