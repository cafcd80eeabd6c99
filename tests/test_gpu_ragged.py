"""GPU parity of the ragged-batch calls (a draft length per request, packed
inputs) and of the end-of-sequence rule, against the oracle's ragged
functions: exact tokens / lengths / flags outside the boundary band."""

import numpy as np
import pytest
import torch

import oracle
import speculative_sampling_verification_sample_amd as sv
from parity import widen
from workloads import generate, pack_ragged, ragged_gammas

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _np(t):
    return t.detach().cpu().numpy()


def oracle_ragged(r, eos=-1, requests=None, greedy=False, cu_override=None, draft_logits=False):
    c = r.cfg
    B = r.cu.shape[0] - 1
    req = np.arange(B) if requests is None else np.asarray(requests)
    cu = _np(r.cu if cu_override is None else cu_override).astype(np.int64)
    N = r.ids.shape[0]
    V = r.logits.shape[1]
    if r.logits.numel() <= 50_000_000:
        # small batch: the whole packed arrays, widened once
        lg = widen(r.logits)
        ids = _np(r.ids).astype(np.int64)
        if greedy:
            return oracle.verify_greedy_ragged(lg, ids, cu, r.gamma_max, eos, requests=req)
        if draft_logits:
            dz = widen(r.draft_logits).reshape(-1, V)
            return oracle.verify_sample_ragged_draft_logits(lg, dz, ids, cu, _np(r.u_accept), _np(r.u_resample),
                                                            r.gamma_max, c.temperature, c.top_k, c.top_p, eos,
                                                            requests=req)
        q = _np(r.q).reshape(-1, V)
        return oracle.verify_sample_ragged(lg, q, ids, cu, _np(r.u_accept), _np(r.u_resample), r.gamma_max,
                                           c.temperature, c.top_k, c.top_p, eos, requests=req)
    # large batch: each sampled request's rows as a batch of its own
    out = []
    for b in req:
        lo, hi = int(cu[b]), int(cu[b + 1])
        sp = oracle.ragged_span(cu, b, N, r.gamma_max)
        if sp is None:
            # a one-request batch with the same invalid span
            o1 = (oracle.verify_greedy_ragged(np.zeros((1, V)), np.zeros(0, np.int64), np.array([lo, hi]),
                                              r.gamma_max, eos) if greedy else
                  oracle.verify_sample_ragged(np.zeros((1, V)), np.zeros((0, V)), np.zeros(0, np.int64),
                                              np.array([lo, hi]), np.zeros(0), np.zeros(1), r.gamma_max,
                                              c.temperature, c.top_k, c.top_p, eos))
            out.append(o1)
            continue
        ri = torch.arange(lo + b, hi + b + 1, device=r.logits.device)
        di = torch.arange(lo, hi, device=r.logits.device)
        lg = widen(r.logits.index_select(0, ri))
        ids = _np(r.ids.index_select(0, di)).astype(np.int64)
        cu1 = np.array([0, hi - lo])
        if greedy:
            o1 = oracle.verify_greedy_ragged(lg, ids, cu1, r.gamma_max, eos)
        elif draft_logits:
            dz = widen(r.draft_logits.index_select(0, di)).reshape(-1, V)
            ua = _np(r.u_accept.index_select(0, di))
            ur = _np(r.u_resample.index_select(0, ri))
            o1 = oracle.verify_sample_ragged_draft_logits(lg, dz, ids, cu1, ua, ur, r.gamma_max, c.temperature,
                                                           c.top_k, c.top_p, eos)
        else:
            q = _np(r.q.index_select(0, di)).reshape(-1, V)
            ua = _np(r.u_accept.index_select(0, di))
            ur = _np(r.u_resample.index_select(0, ri))
            o1 = oracle.verify_sample_ragged(lg, q, ids, cu1, ua, ur, r.gamma_max, c.temperature, c.top_k,
                                              c.top_p, eos)
        out.append(o1)
    keys = ("tokens", "n_accepted", "flags", "accept_boundary", "cdf_boundary", "top_p_boundary")
    return {k: np.concatenate([o[k] for o in out]) for k in keys}


def gpu_ragged(r, eos=-1, greedy=False, cu=None, draft_logits=False):
    c = r.cfg
    cu = r.cu if cu is None else cu
    if draft_logits:
        tok, nacc, fl = sv.verify_sample_ragged_draft_logits(r.logits, r.draft_logits, r.ids, cu, r.u_accept,
                                                             r.u_resample, r.gamma_max, c.temperature, c.top_k,
                                                             c.top_p, eos_id=eos)
    elif greedy:
        tok, nacc, fl = sv.verify_greedy_ragged(r.logits, r.ids, cu, r.gamma_max, eos_id=eos)
    else:
        tok, nacc, fl = sv.verify_sample_ragged(r.logits, r.q, r.ids, cu, r.u_accept, r.u_resample, r.gamma_max,
                                                c.temperature, c.top_k, c.top_p, eos_id=eos)
    torch.cuda.synchronize()
    return _np(tok), _np(nacc), _np(fl).astype(np.uint32)


def compare_ragged(r, eos=-1, requests=None, label="", greedy=False, cu=None, draft_logits=False):
    tok, nacc, fl = gpu_ragged(r, eos, greedy, cu, draft_logits)
    B = r.cu.shape[0] - 1
    req = np.arange(B) if requests is None else np.asarray(requests)
    o = oracle_ragged(r, eos, req, greedy, cu, draft_logits)
    g_tok, g_nacc, g_fl = tok[req], nacc[req], fl[req]
    mism = (g_tok != o["tokens"]).any(axis=1) | (g_nacc != o["n_accepted"]) | (g_fl != o["flags"])
    boundary = o["accept_boundary"] | o["cdf_boundary"] | o["top_p_boundary"]
    hard = mism & ~boundary
    print(f"[{label}] requests={len(req)} mismatches={int(mism.sum())} boundary_rows={int(boundary.sum())} "
          f"mean_accepted={g_nacc.mean():.3f} eos_rows={int(((g_fl & 16) != 0).sum())} "
          f"flags={np.unique(g_fl).tolist()}", flush=True)
    if hard.any():
        i = int(np.nonzero(hard)[0][0])
        raise AssertionError(
            f"[{label}] request {int(req[i])}: gpu tokens {g_tok[i].tolist()} n={g_nacc[i]} flags={g_fl[i]} vs "
            f"oracle {o['tokens'][i].tolist()} n={o['n_accepted'][i]} flags={o['flags'][i]}")
    return o, (tok, nacc, fl)


def _ragged(name, seed=0, gammas=None, **kw):
    w = generate(name, DEV, **kw)
    G = w.ids.shape[1]
    g = ragged_gammas(w.cfg.B, G, seed) if gammas is None else np.asarray(gammas)
    return w, pack_ragged(w, g)


@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=9)),
    ("c3", dict(B=7)),
    ("c5", dict(B=5)),
    ("c2", dict(B=6, gamma=3, V=10007)),
    ("c3", dict(B=6, gamma=2, V=40003)),
    ("c5", dict(B=4, gamma=3, V=70001)),
])
def test_sample_small_and_ragged_vocab(name, kw):
    _, r = _ragged(name, seed=1, **kw)
    compare_ragged(r, label=f"ragged {name} {kw} gammas={r.gammas.tolist()}")


def test_toy_with_eos():
    """V = 5: end-of-sequence cuts (accepted drafts) and emitted EOS
    replacements and bonus tokens are all frequent."""
    _, r = _ragged("toy", seed=2, B=20000)
    o, (tok, nacc, fl) = compare_ragged(r, eos=2, label="ragged toy eos=2")
    cut = (o["flags"] & oracle.FLAG_EOS) != 0
    assert cut.sum() > 1000
    compare_ragged(r, label="ragged toy")


def test_all_full_equals_uniform_call():
    """gamma_b = gamma for every request: the ragged call gives the uniform
    call's outputs exactly."""
    for name, kw in (("c3", dict(B=6, V=20000)), ("c2", dict(B=5, V=9000)), ("c5", dict(B=4, V=30000))):
        w = generate(name, DEV, **kw)
        r = pack_ragged(w, [w.ids.shape[1]] * kw["B"])
        c = w.cfg
        a = sv.verify_sample(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p)
        b = sv.verify_sample_ragged(r.logits, r.q, r.ids, r.cu, r.u_accept, r.u_resample, r.gamma_max,
                                    c.temperature, c.top_k, c.top_p)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), name


def test_all_gamma_zero():
    """n_draft = 0: plain sampling from each request's single row."""
    for name in ("c2", "c3", "c5"):
        _, r = _ragged(name, gammas=[0] * 5, B=5, V=12000)
        assert r.ids.shape[0] == 0
        o, (tok, nacc, fl) = compare_ragged(r, label=f"ragged all-zero {name}")
        assert (nacc == 0).all() and (tok[:, 1:] == -1).all()


def _plant_eos(w, E, plant):
    """Make request b's draft j equal E with p(E) ~ 1 at that position, so it
    is accepted: boost E in target row j and set the draft id."""
    lg = w.logits.clone()
    ids = w.ids.clone()
    for b, j in plant:
        lg[b, j, E] = 60.0
        ids[b, j] = E
    w.logits, w.ids = lg.contiguous(), ids.contiguous()


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_eos_cut(name):
    w = generate(name, DEV, B=8, V=20000)
    E = 1234
    _plant_eos(w, E, [(0, 0), (1, 2), (2, 3), (3, 1), (5, 2), (6, 0)])
    gam = [3, 4, 1, 2, 0, 4, 2, 3]  # request 2's EOS lies beyond its span
    r = pack_ragged(w, gam)
    o, (tok, nacc, fl) = compare_ragged(r, eos=E, label=f"ragged eos {name}")
    for b in (0, 6):  # an EOS first draft with p(E) ~ 1 is always accepted
        assert fl[b] & oracle.FLAG_EOS and nacc[b] == 0 and tok[b, 0] == E
    compare_ragged(r, label=f"ragged no-eos {name}")


def test_greedy_ragged_with_eos():
    w = generate("c4", DEV, B=12, V=30011)
    G = w.ids.shape[1]
    g = ragged_gammas(12, G, 5)
    r = pack_ragged(w, g)
    compare_ragged(r, label="ragged greedy", greedy=True)
    # an EOS that is the target's argmax at a draft position of a few requests
    w2 = generate("c4", DEV, B=12, V=30011)
    E = 777
    _plant_eos(w2, E, [(0, 1), (2, 0), (4, 3), (7, 5)])
    r2 = pack_ragged(w2, [8, 3, 2, 0, 6, 1, 4, 7, 8, 2, 5, 3])
    o, (tok, nacc, fl) = compare_ragged(r2, eos=E, label="ragged greedy eos", greedy=True)
    assert fl[2] & oracle.FLAG_EOS and nacc[2] == 0 and tok[2].tolist() == [E] + [-1] * 8


def test_bad_spans_flagged_and_isolated():
    """Out-of-order, out-of-range and too-long spans: those requests emit
    nothing (SV_ROW_BAD_SPAN); the others are verified as usual."""
    _, r = _ragged("c3", gammas=[2, 3, 1, 0, 5, 2], B=6, V=9000)
    N = r.ids.shape[0]
    cu = _np(r.cu).astype(np.int32)  # [0, 2, 5, 6, 6, 11, 13]
    bad = cu.copy()
    bad[2] = 7       # request 1: [2, 7), valid (it overlaps its neighbours' data)
    bad[3] = 4       # request 2: [7, 4), out of order
    bad[6] = N + 3   # request 5: [11, 16), past n_draft
    cu_bad = torch.as_tensor(bad, device=DEV)
    o, (tok, nacc, fl) = compare_ragged(r, cu=cu_bad, label="ragged bad spans")
    assert fl[2] == oracle.FLAG_BAD_SPAN and fl[5] == oracle.FLAG_BAD_SPAN
    assert (tok[[2, 5]] == -1).all() and (nacc[[2, 5]] == 0).all()
    assert fl[1] != oracle.FLAG_BAD_SPAN and fl[3] != oracle.FLAG_BAD_SPAN
    # gamma_max smaller than the longest span
    r.gamma_max = 3
    o, (tok, nacc, fl) = compare_ragged(r, label="ragged span > gamma_max")
    assert fl[4] == oracle.FLAG_BAD_SPAN and tok.shape == (6, 4)
    o, (tok, nacc, fl) = compare_ragged(r, label="ragged greedy span > gamma_max", greedy=True)
    assert fl[4] == oracle.FLAG_BAD_SPAN


def test_long_gamma_max():
    """gamma_max + 1 > 64: the acceptance and the draw run as separate
    launches; spans from 0 to 70 drafts."""
    w = generate("c2", DEV, B=4, gamma=70, V=600)
    r = pack_ragged(w, [70, 0, 33, 64])
    compare_ragged(r, label="ragged gamma_max=70")
    compare_ragged(r, eos=int(_np(r.ids)[5]), label="ragged gamma_max=70 eos")
    w3 = generate("c3", DEV, B=3, gamma=70, V=3000)
    r3 = pack_ragged(w3, [70, 12, 0])
    compare_ragged(r3, label="ragged c3 gamma_max=70")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size(name):
    w = generate(name, DEV)
    g = ragged_gammas(w.cfg.B, w.ids.shape[1], 11)
    r = pack_ragged(w, g)
    del w
    req = np.sort(np.random.default_rng(0).choice(r.cu.shape[0] - 1, 16, replace=False))
    o, (tok, nacc, fl) = compare_ragged(r, requests=req, label=f"ragged {name} full")
    gam = r.gammas
    pos = np.arange(r.gamma_max + 1)[None, :]
    assert ((tok >= 0) == (pos <= nacc[:, None])).all()
    assert (nacc <= gam).all()
    assert (tok < r.logits.shape[1]).all()


def test_greedy_full_size():
    w = generate("c4", DEV)
    r = pack_ragged(w, ragged_gammas(w.cfg.B, w.ids.shape[1], 12))
    del w
    req = np.sort(np.random.default_rng(1).choice(r.cu.shape[0] - 1, 16, replace=False))
    compare_ragged(r, requests=req, label="ragged c4 full", greedy=True)


@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=7)),
    ("c3", dict(B=6)),
    ("c5", dict(B=5)),
    ("c3", dict(B=5, gamma=3, V=30011)),
    ("c5", dict(B=4, gamma=2, V=50001)),
])
def test_draft_logits(name, kw):
    """q formed from the packed draft logits; spans from gamma down to 0 drafts."""
    w = generate(name, DEV, **kw)
    G = w.ids.shape[1]
    r = pack_ragged(w, [G - (b % (G + 1)) for b in range(w.cfg.B)])
    compare_ragged(r, label=f"ragged dl {name} {kw} gammas={r.gammas.tolist()}", draft_logits=True)
    E = int(_np(r.ids)[0]) if r.ids.shape[0] else 0
    compare_ragged(r, eos=E, label=f"ragged dl eos {name}", draft_logits=True)


def test_draft_logits_all_zero_and_bad_span():
    _, r = _ragged("c3", gammas=[0] * 4, B=4, V=9000)
    compare_ragged(r, label="ragged dl all-zero", draft_logits=True)
    _, r = _ragged("c5", gammas=[2, 3, 1, 2], B=4, V=20000)
    cu = _np(r.cu).astype(np.int32)
    bad = cu.copy()
    bad[2] = cu[3] + 1  # request 1 ends past request 2's start; request 2 runs backwards
    o, (tok, nacc, fl) = compare_ragged(r, cu=torch.as_tensor(bad, device=DEV), label="ragged dl bad span",
                                        draft_logits=True)
    assert fl[2] == oracle.FLAG_BAD_SPAN


def test_draft_logits_full_size():
    w = generate("c5", DEV)
    r = pack_ragged(w, ragged_gammas(w.cfg.B, w.ids.shape[1], 13))
    del w
    req = np.sort(np.random.default_rng(2).choice(r.cu.shape[0] - 1, 8, replace=False))
    compare_ragged(r, requests=req, label="ragged dl c5 full", draft_logits=True)
