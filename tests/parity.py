"""Shared helpers for the GPU parity tests (HIP library vs the CPU oracle)."""

import numpy as np
import torch

import oracle
from oracle import pool as oracle_pool
import speculative_sampling_verification_sample_amd as sv


def widen(logits: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of GPU logits (bf16 through its bit pattern)."""
    t = logits.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy())
    return t.double().numpy()


def _np(t):
    return t.detach().cpu().numpy()


def _host(t):
    """Host copy for the oracle pool: bfloat16 as its int16 bit patterns."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def gpu_sample(w, draft_logits=False, lenience=None, **kw):
    """The library's sampling verify; with draft_logits, q is formed by the
    library from w.draft_logits; with lenience, the lenient call."""
    c = w.cfg
    prm = dict(temperature=c.temperature, top_k=c.top_k, top_p=c.top_p)
    prm.update(kw)
    if lenience is not None:
        tok, nacc, fl = sv.verify_sample_lenient(w.logits, w.q, w.ids, w.u_accept, w.u_resample, lenience=lenience,
                                                 **prm)
    elif draft_logits:
        tok, nacc, fl = sv.verify_sample_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                                      **prm)
    else:
        tok, nacc, fl = sv.verify_sample(w.logits, w.q, w.ids, w.u_accept, w.u_resample, **prm)
    torch.cuda.synchronize()
    return _np(tok), _np(nacc), _np(fl).astype(np.uint32)


def compare_sample(w, requests=None, label="", gpu=None, draft_logits=False, lenience=None, pool=False, **kw):
    """Run both sides; exact match required outside boundary rows.
    draft_logits: both sides form q from w.draft_logits; lenience: both
    sides use the lenient acceptance with that factor; pool: every request,
    the oracle spread over the host's cores (requests must be None)."""
    c = w.cfg
    prm = dict(T=c.temperature, top_k=c.top_k, top_p=c.top_p)
    if "temperature" in kw:
        prm["T"] = kw["temperature"]
    if "top_k" in kw:
        prm["top_k"] = kw["top_k"]
    if "top_p" in kw:
        prm["top_p"] = kw["top_p"]
    tok, nacc, fl = gpu if gpu is not None else gpu_sample(w, draft_logits=draft_logits, lenience=lenience, **kw)
    req = np.arange(c.B) if requests is None else np.asarray(requests)
    G = w.ids.shape[1]
    beta = 1.0 if lenience is None else float(np.float32(lenience))
    if pool:
        assert requests is None
        arrays = dict(logits=_host(w.logits), ids=_np(w.ids), u_accept=_np(w.u_accept), u_resample=_np(w.u_resample))
        if draft_logits:
            arrays["draft_logits"] = _host(w.draft_logits)
        else:
            arrays["q"] = _np(w.q)
        o = oracle_pool.run("sample_draft_logits" if draft_logits else "sample", arrays, dict(prm, beta=beta), c.B)
    else:
        ridx = torch.as_tensor(req, device=w.logits.device)
        lg = widen(w.logits.index_select(0, ridx))
        q = (_np(w.q.index_select(0, ridx)) if (w.q is not None and G > 0)
             else np.zeros((len(req), 0, lg.shape[2]), np.float32))
        ids = _np(w.ids.index_select(0, ridx))
        ua = _np(w.u_accept.index_select(0, ridx))
        ur = _np(w.u_resample.index_select(0, ridx))
        if draft_logits:
            dlg = widen(w.draft_logits.index_select(0, ridx)) if G > 0 else np.zeros((len(req), 0, lg.shape[2]))
            o = oracle.verify_sample_draft_logits(lg, dlg, ids, ua, ur, prm["T"], prm["top_k"], prm["top_p"])
        else:
            o = oracle.verify_sample(lg, q, ids, ua, ur, prm["T"], prm["top_k"], prm["top_p"], beta=beta)
    g_tok, g_nacc, g_fl = tok[req], nacc[req], fl[req]
    mism = (g_tok != o["tokens"]).any(axis=1) | (g_nacc != o["n_accepted"]) | (g_fl != o["flags"])
    boundary = o["accept_boundary"] | o["cdf_boundary"] | o["top_p_boundary"]
    hard = mism & ~boundary
    flagged = o["flags"] != 0
    print(f"[{label}] requests={len(req)} hard_mismatches={int(hard.sum())} boundary_rows={int(boundary.sum())} "
          f"(accept {int(o['accept_boundary'].sum())}, cdf {int(o['cdf_boundary'].sum())}, "
          f"top_p {int(o['top_p_boundary'].sum())}) boundary_mismatches={int((mism & boundary).sum())} "
          f"flag_rows={int(flagged.sum())} flag_row_mismatches={int((mism & flagged).sum())} "
          f"mean_accepted={g_nacc.mean():.3f} flags={np.unique(g_fl).tolist()}", flush=True)
    if hard.any():
        i = int(np.nonzero(hard)[0][0])
        raise AssertionError(
            f"[{label}] request {int(req[i])}: gpu tokens {g_tok[i].tolist()} n={g_nacc[i]} flags={g_fl[i]} vs "
            f"oracle {o['tokens'][i].tolist()} n={o['n_accepted'][i]} flags={o['flags'][i]}")
    return o, dict(mismatch=int(mism.sum()), boundary=int(boundary.sum()))


def compare_greedy(w, requests=None, label="", pool=False):
    """Greedy parity: bit-exact on every compared request (pool: all of
    them, the oracle spread over the host's cores)."""
    tok, nacc, fl = sv.verify_greedy(w.logits, w.ids)
    torch.cuda.synchronize()
    tok, nacc, fl = _np(tok), _np(nacc), _np(fl).astype(np.uint32)
    req = np.arange(w.cfg.B) if requests is None else np.asarray(requests)
    if pool:
        assert requests is None
        o = oracle_pool.run("greedy", dict(logits=_host(w.logits), ids=_np(w.ids)), {}, w.cfg.B)
    else:
        ridx = torch.as_tensor(req, device=w.logits.device)
        lg = widen(w.logits.index_select(0, ridx))
        ids = _np(w.ids.index_select(0, ridx))
        o = oracle.verify_greedy(lg, ids)
    ok = (tok[req] == o["tokens"]).all() and (nacc[req] == o["n_accepted"]).all() and (fl[req] == o["flags"]).all()
    print(f"[{label}] greedy requests={len(req)} mean_accepted={nacc[req].mean():.3f}", flush=True)
    if not ok:
        bad = np.nonzero((tok[req] != o["tokens"]).any(1) | (nacc[req] != o["n_accepted"]))[0]
        i = int(bad[0]) if bad.size else 0
        raise AssertionError(f"[{label}] request {int(req[i])}: gpu {tok[req][i].tolist()} vs oracle {o['tokens'][i].tolist()}")


def stats_floor(w, req, draft_logits=False):
    """Double precision floor of alpha, Z and Z' per position [B', gamma].

    Reading: the tolerance of 1e-5 relative holds above the resolution of
    the double arithmetic both sides compute in, not below it.  Each p (and
    a q formed from the draft's logits) is an exponential whose argument is
    of size up to m = max|z| / T over the row; the argument is rounded to
    double, so the library's and the oracle's p(x) differ by up to about
    m * 2^-53 relative, and their exact comparison of p(x) with q(x) may
    differ where the two agree that closely.  A sum over the vocabulary of
    such terms (a Z near 0, a Z' of one-hot rows) is therefore fixed only to
    about (1 + m) * 2^-53 times the total mass; the floor allows 2^-50
    (1 + m), the total mass of p and q being at most a few units."""
    c = w.cfg
    G = w.ids.shape[1]
    ridx = torch.as_tensor(np.asarray(req), device=w.logits.device)

    def row_max(t):
        t = t.index_select(0, ridx)[:, :G].float()
        return torch.where(torch.isfinite(t), t.abs(), torch.zeros_like(t)).amax(-1).double().cpu().numpy()

    m = row_max(w.logits)
    if draft_logits:
        m = np.maximum(m, row_max(w.draft_logits))
    return 2.0 ** -50 * (1.0 + m / float(np.float32(c.temperature)))


def compare_stats(w, requests=None, label="", rtol=1e-5, draft_logits=False, gpu=None, pool=False):
    """Statistics parity: every output within ``rtol`` relative of the
    oracle's value rounded to the outputs' float32 (or one float32 spacing
    there, which only differs in the subnormal range), NaN where the oracle
    has NaN.  Positions whose kept
    set the oracle decided within 1e-6 of top_p are boundary positions: they
    are counted and printed, and left out of the bound.  Below the double
    precision floor of the computation (``stats_floor``) the bound is that
    floor instead; the positions where it decides are counted and printed.
    The largest relative error is printed over all positions and over those
    with Z < 0.03.
    gpu: the four statistics outputs already computed (else the library's
    statistics call is run here).  pool: every request, the oracle spread
    over the host's cores.  Returns the largest relative error."""
    c = w.cfg
    if gpu is not None:
        al, zpq, zqp, acc = gpu
    elif draft_logits:
        al, zpq, zqp, acc = sv.accept_stats_draft_logits(w.logits, w.draft_logits, w.ids, c.temperature, c.top_k,
                                                         c.top_p)
    else:
        al, zpq, zqp, acc = sv.accept_stats(w.logits, w.q, w.ids, c.temperature, c.top_k, c.top_p)
    torch.cuda.synchronize()
    req = np.arange(c.B) if requests is None else np.asarray(requests)
    if pool:
        assert requests is None
        arrays = dict(logits=_host(w.logits), ids=_np(w.ids))
        if draft_logits:
            arrays["draft_logits"] = _host(w.draft_logits)
        else:
            arrays["q"] = _np(w.q)
        prm = dict(T=c.temperature, top_k=c.top_k, top_p=c.top_p)
        o = oracle_pool.run("stats_draft_logits" if draft_logits else "stats", arrays, prm, c.B)
    else:
        ridx = torch.as_tensor(req, device=w.logits.device)
        lg = widen(w.logits.index_select(0, ridx))
        ids = _np(w.ids.index_select(0, ridx))
        if draft_logits:
            dlg = widen(w.draft_logits.index_select(0, ridx))
            o = oracle.accept_stats_draft_logits(lg, dlg, ids, c.temperature, c.top_k, c.top_p, with_boundary=True)
        else:
            q = _np(w.q.index_select(0, ridx))
            o = oracle.accept_stats(lg, q, ids, c.temperature, c.top_k, c.top_p, with_boundary=True)
    boundary = o[4]
    small_z = np.abs(o[1]) < 0.03
    floor = stats_floor(w, req, draft_logits)
    worst = 0.0
    for name, g, ov in zip(("alpha", "z_pq", "z_qp", "accept_prob"), (al, zpq, zqp, acc), o[:4]):
        if g is None:  # an output left out
            continue
        g = _np(g)[req].astype(np.float64)
        # the outputs are float32: the oracle's value is taken rounded to
        # float32, and one float32 spacing at that value is allowed besides
        # the relative bound (it only matters below 1.2e-38, where float32
        # is subnormal; a value under 1.4e-45 reads as 0)
        ov = np.where(np.isnan(ov), ov, ov.astype(np.float32).astype(np.float64))
        ulp = np.spacing(np.abs(np.nan_to_num(ov)).astype(np.float32)).astype(np.float64)
        both_nan = np.isnan(g) & np.isnan(ov)
        err = np.where(both_nan, 0.0, np.abs(g - ov))
        rel = np.where(both_nan, 0.0, err / np.maximum(np.abs(ov), 1e-300))
        rel = np.where((err <= ulp) | both_nan, 0.0, rel)
        inside = ~boundary
        # the relative bound against the float32-rounded value; the fp64
        # floor where the value is itself at that floor (not for the
        # acceptance probability: a ratio of two probabilities)
        ok_rel = err <= np.maximum(rtol * np.abs(ov), ulp)
        fl = floor if name != "accept_prob" else 0.0
        at_floor = inside & ~both_nan & ~ok_rel & (err <= fl)
        bad = inside & ~(both_nan | ok_rel | at_floor)
        worst_here = float(np.nanmax(np.where(inside & ~at_floor, rel, 0.0))) if rel.size else 0.0
        worst_small = float(np.nanmax(np.where(inside & small_z & ~at_floor, rel, 0.0))) if rel.size else 0.0
        worst = max(worst, worst_here)
        print(f"[{label}] stats {name}: max_rel={worst_here:.3e} max_rel(Z<0.03, {int((inside & small_z).sum())} "
              f"positions)={worst_small:.3e} boundary_positions={int(boundary.sum())} "
              f"at_fp64_floor={int(at_floor.sum())}", flush=True)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"[{label}] {name}{i}: gpu {g[i]!r} oracle {ov[i]!r}")
    return worst
