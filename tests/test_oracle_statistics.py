"""Statistical pins of the oracle on the toy workload (CPU).

* each emitted slot follows its target row p_j (chi-square, 1e6 rounds;
  [WR] §5.1 and §14.1, [RL] §2, [BS] §五);
* resampling from p instead of the residual fails the same test (negative
  control, [WR] §13.3);
* tokens per round: E[N] = 1 + sum_i prod_{k<=i} alpha_k ([WR] §10), and at
  constant alpha the truncated geometric law of [MN] §四 with mean
  (1 - alpha^{g+1}) / (1 - alpha) ([RL] §3);
* the toy's closed form: with q = 0.6 p + 0.4 / 5, Z = 0.4 sum (p - 0.2)_+.
"""

import numpy as np
import pytest
from scipy import stats

import oracle
from workloads import generate


def _run_rounds(w, n):
    z = w.logits[0].double().numpy()
    q = w.q[0].double().numpy()
    G = w.cfg.gamma
    p_rows = [oracle.process_row(z[j], w.cfg.temperature).p for j in range(G + 1)]
    ids = w.ids[:n].numpy()
    ua = w.u_accept[:n].numpy()
    ur = w.u_resample[:n].numpy()
    toks = np.empty((n, G + 1), np.int32)
    nacc = np.empty(n, np.int32)
    for b in range(n):
        r = oracle.verify_from_processed(p_rows, q, ids[b], ua[b], ur[b])
        toks[b] = r.tokens
        nacc[b] = r.n_accepted
    return p_rows, q, toks, nacc


def _slot_pvalues(p_rows, toks, nacc):
    V = p_rows[0].size
    out = []
    for j in range(len(p_rows)):
        reached = nacc >= j
        counts = np.bincount(toks[reached, j], minlength=V)
        exp = p_rows[j] * reached.sum()
        out.append(stats.chisquare(counts, exp).pvalue)
    return out


@pytest.fixture(scope="module")
def toy_million():
    w = generate("toy", B=1_000_000)
    return _run_rounds(w, 1_000_000)


@pytest.mark.slow
def test_chi_square_each_slot_follows_p(toy_million):
    p_rows, q, toks, nacc = toy_million
    pv = _slot_pvalues(p_rows, toks, nacc)
    assert min(pv) > 1e-4, pv
    # empirical total variation shrinks like 1/sqrt(n) ([WR] §14.1)
    V = p_rows[0].size
    emp = np.bincount(toks[:, 0], minlength=V) / len(toks)
    tv = 0.5 * np.abs(emp - p_rows[0]).sum()
    assert tv < 3 * np.sqrt(V / len(toks))


@pytest.mark.slow
def test_expected_tokens_product_form(toy_million):
    p_rows, q, toks, nacc = toy_million
    G = len(q)
    alpha = [np.minimum(p_rows[j], q[j]).sum() for j in range(G)]
    EN = 1 + sum(np.prod(alpha[: i + 1]) for i in range(G))
    N = nacc + 1
    assert abs(N.mean() - EN) < 4 * N.std() / np.sqrt(len(N))


def test_negative_control_resample_from_p(monkeypatch):
    w = generate("toy", B=200_000)
    monkeypatch.setattr(oracle.verify, "residual_weights", lambda p, q: np.asarray(p, dtype=np.float64))
    p_rows, q, toks, nacc = _run_rounds(w, 200_000)
    pv = _slot_pvalues(p_rows, toks, nacc)
    assert pv[0] < 1e-12


def test_constant_alpha_truncated_geometric():
    w = generate("toy", name="toy_const", B=200_000)
    p_rows, q, toks, nacc = _run_rounds(w, 200_000)
    G = len(q)
    a = np.minimum(p_rows[0], q[0]).sum()
    law = np.array([a ** (k - 1) * (1 - a) for k in range(1, G + 1)] + [a ** G])
    assert law.sum() == pytest.approx(1.0, abs=1e-12)
    N = nacc + 1
    counts = np.bincount(N, minlength=G + 2)[1:]
    assert stats.chisquare(counts, law * len(N)).pvalue > 1e-4
    mean = (1 - a ** (G + 1)) / (1 - a)
    assert abs(N.mean() - mean) < 4 * N.std() / np.sqrt(len(N))


def test_toy_residual_closed_form():
    w = generate("toy", B=1)
    z = w.logits[0].double().numpy()
    alpha, zpq, zqp, _ = oracle.stats_request(z, w.q[0].numpy(), w.ids[0].numpy(), 1.0)
    for j in range(w.cfg.gamma):
        p = oracle.process_row(z[j], 1.0).p
        assert zpq[j] == pytest.approx(0.4 * np.maximum(p - 0.2, 0).sum(), abs=3e-7)
        assert zqp[j] == pytest.approx(zpq[j], abs=3e-7)
