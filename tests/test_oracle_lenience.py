"""Pins of the oracle's lenient acceptance ([MN] §八: the draft is scaled to
beta * q before it is compared with the target, 0 < beta <= 1).

The pages state the acceptance min(1, p / (beta q)) and one guarantee: no
token is emitted with more than 1/beta times its target probability.  They
give no residual for this variant; the oracle keeps the lossless step with
beta * q in place of q, so the replacement comes from (p - beta q)_+ (a
reading, not pinned by the pages).  What the pages and the mathematics fix,
pinned here by exact enumeration over uniform grids fine enough to hit every
breakpoint:

* beta = 1 is the lossless rule;
* the acceptance rate is sum_x q min(1, p / (beta q)) = sum_x min(q, p / beta);
* every token is emitted with probability <= p / beta (the pages' bound),
  with equality where beta q >= p;
* the emitted law of the reading, min(q, p/beta) + P(reject) (p - beta q)_+ / W.
"""

import itertools

import numpy as np
import pytest

import oracle


def _grid(K):
    return (np.arange(K) + 0.5) / K


def _law(p0, q0, p1, beta, K):
    """Exact law of the first emitted token and the acceptance rate, gamma = 1."""
    law = np.zeros(len(p0))
    acc = 0.0
    for d in range(len(p0)):
        if q0[d] == 0.0:
            continue
        for ua, ur in itertools.product(_grid(K), repeat=2):
            r = oracle.verify_from_processed([p0, p1], [q0], [d], [ua], [ur, ur], beta=beta)
            w = q0[d] / K ** 2
            law[r.tokens[0]] += w
            acc += w * (r.n_accepted == 1)
    return law, acc


# (p0, q0, beta, K): every ratio p / (beta q) below 1 and every residual CDF
# step is a multiple of 1/K
CASES = [
    (np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.1, 0.8]), 0.5, 14),
    (np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.1, 0.8]), 0.8, 32),
    (np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.1, 0.8]), 0.25, 4),
    (np.array([0.6, 0.2, 0.2]), np.array([0.2, 0.4, 0.4]), 0.75, 12),
]


@pytest.mark.parametrize("p0,q0,beta,K", CASES)
def test_lenient_law(p0, q0, beta, K):
    p1 = np.array([0.2, 0.5, 0.3])
    law, acc = _law(p0, q0, p1, beta, K)
    assert acc == pytest.approx(np.minimum(q0, p0 / beta).sum(), abs=1e-12)
    # the pages' guarantee: never more than 1/beta times the target probability
    assert (law <= p0 / beta + 1e-12).all()
    tight = beta * q0 >= p0
    np.testing.assert_allclose(law[tight], (p0 / beta)[tight], atol=1e-12)
    # the reading's law in closed form
    res = np.maximum(p0 - beta * q0, 0.0)
    expect = np.minimum(q0, p0 / beta) + (1.0 - acc) * res / res.sum()
    np.testing.assert_allclose(law, expect, atol=1e-12)
    assert law.sum() == pytest.approx(1.0, abs=1e-12)


def test_lenience_loosens_acceptance_and_beta_one_is_lossless():
    p0, q0, p1 = np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.1, 0.8]), np.array([0.2, 0.5, 0.3])
    law1, acc1 = _law(p0, q0, p1, 1.0, 12)
    np.testing.assert_allclose(law1, p0, atol=1e-12)  # lossless: the target's law
    _, acc5 = _law(p0, q0, p1, 0.5, 14)
    assert acc5 > acc1  # a looser test accepts more
    rng = np.random.default_rng(3)
    for _ in range(200):
        z = np.log(rng.dirichlet(np.ones(6), size=3))
        q = rng.dirichlet(np.ones(6), size=2)
        ids = rng.integers(0, 6, 2)
        ua, ur = rng.random(2), rng.random(3)
        a = oracle.verify_request(z, q, ids, ua, ur, 1.0)
        b = oracle.verify_request(z, q, ids, ua, ur, 1.0, beta=1.0)
        assert a.tokens.tolist() == b.tokens.tolist() and a.flags == b.flags


def test_lenient_worked_decisions():
    """One position, p(d) = 0.2, q(d) = 0.8: lossless accepts iff u < 0.25;
    beta = 0.5 iff u < 0.5; beta = 0.25 always."""
    p = [np.array([0.5, 0.3, 0.2]), np.array([0.2, 0.5, 0.3])]
    q = [np.array([0.1, 0.1, 0.8])]
    for beta, u, acc in ((1.0, 0.24, 1), (1.0, 0.26, 0), (0.5, 0.49, 1), (0.5, 0.51, 0), (0.25, 0.999, 1)):
        r = oracle.verify_from_processed(p, q, [2], [u], [0.5, 0.5], beta=beta)
        assert r.n_accepted == acc, (beta, u)
    # a rejection under beta = 0.5 draws from (p - 0.5 q)_+ = (0.45, 0.25, 0)
    r = oracle.verify_from_processed(p, q, [2], [0.9], [0.6, 0.5], beta=0.5)
    assert r.tokens.tolist() == [0, -1]       # 0.6 * 0.7 = 0.42 < 0.45
    r = oracle.verify_from_processed(p, q, [2], [0.9], [0.7, 0.5], beta=0.5)
    assert r.tokens.tolist() == [1, -1]       # 0.49 > 0.45
