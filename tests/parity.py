"""Shared helpers for the GPU parity tests (HIP library vs the CPU oracle)."""

import numpy as np
import torch

import oracle
import speculative_sampling_verification_sample_amd as sv


def widen(logits: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of GPU logits (bf16 through its bit pattern)."""
    t = logits.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy())
    return t.double().numpy()


def _np(t):
    return t.detach().cpu().numpy()


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


def compare_sample(w, requests=None, label="", gpu=None, draft_logits=False, lenience=None, **kw):
    """Run both sides; exact match required outside boundary rows.
    draft_logits: both sides form q from w.draft_logits; lenience: both
    sides use the lenient acceptance with that factor."""
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
    ridx = torch.as_tensor(req, device=w.logits.device)
    lg = widen(w.logits.index_select(0, ridx))
    G = w.ids.shape[1]
    q = _np(w.q.index_select(0, ridx)) if (w.q is not None and G > 0) else np.zeros((len(req), 0, lg.shape[2]), np.float32)
    ids = _np(w.ids.index_select(0, ridx))
    ua = _np(w.u_accept.index_select(0, ridx))
    ur = _np(w.u_resample.index_select(0, ridx))
    if draft_logits:
        dlg = widen(w.draft_logits.index_select(0, ridx)) if G > 0 else np.zeros((len(req), 0, lg.shape[2]))
        o = oracle.verify_sample_draft_logits(lg, dlg, ids, ua, ur, prm["T"], prm["top_k"], prm["top_p"])
    else:
        beta = 1.0 if lenience is None else float(np.float32(lenience))
        o = oracle.verify_sample(lg, q, ids, ua, ur, prm["T"], prm["top_k"], prm["top_p"], beta=beta)
    g_tok, g_nacc, g_fl = tok[req], nacc[req], fl[req]
    mism = (g_tok != o["tokens"]).any(axis=1) | (g_nacc != o["n_accepted"]) | (g_fl != o["flags"])
    boundary = o["accept_boundary"] | o["cdf_boundary"] | o["top_p_boundary"]
    hard = mism & ~boundary
    print(f"[{label}] requests={len(req)} mismatches={int(mism.sum())} boundary_rows={int(boundary.sum())} "
          f"boundary_mismatches={int((mism & boundary).sum())} mean_accepted={g_nacc.mean():.3f} "
          f"flags={np.unique(g_fl).tolist()}", flush=True)
    if hard.any():
        i = int(np.nonzero(hard)[0][0])
        raise AssertionError(
            f"[{label}] request {int(req[i])}: gpu tokens {g_tok[i].tolist()} n={g_nacc[i]} flags={g_fl[i]} vs "
            f"oracle {o['tokens'][i].tolist()} n={o['n_accepted'][i]} flags={o['flags'][i]}")
    return o, dict(mismatch=int(mism.sum()), boundary=int(boundary.sum()))


def compare_greedy(w, requests=None, label=""):
    tok, nacc, fl = sv.verify_greedy(w.logits, w.ids)
    torch.cuda.synchronize()
    tok, nacc, fl = _np(tok), _np(nacc), _np(fl).astype(np.uint32)
    req = np.arange(w.cfg.B) if requests is None else np.asarray(requests)
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


def compare_stats(w, requests=None, label="", rtol=1e-5, atol=2e-7, draft_logits=False, gpu=None):
    """gpu: the four statistics outputs already computed (else the library's
    statistics call is run here)."""
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
    ridx = torch.as_tensor(req, device=w.logits.device)
    lg = widen(w.logits.index_select(0, ridx))
    ids = _np(w.ids.index_select(0, ridx))
    if draft_logits:
        dlg = widen(w.draft_logits.index_select(0, ridx))
        o = oracle.accept_stats_draft_logits(lg, dlg, ids, c.temperature, c.top_k, c.top_p)
    else:
        q = _np(w.q.index_select(0, ridx))
        o = oracle.accept_stats(lg, q, ids, c.temperature, c.top_k, c.top_p)
    worst = 0.0
    for name, g, ov in zip(("alpha", "z_pq", "z_qp", "accept_prob"), (al, zpq, zqp, acc), o):
        if g is None:  # an output left out
            continue
        g = _np(g)[req].astype(np.float64)
        both_nan = np.isnan(g) & np.isnan(ov)
        err = np.where(both_nan, 0.0, np.abs(g - ov))
        rel = err / np.maximum(np.abs(ov), 1e-30)
        worst = max(worst, float(np.nanmax(np.where(both_nan, 0.0, rel))) if rel.size else 0.0)
        bad = ~(both_nan | (err <= rtol * np.abs(ov) + atol))
        print(f"[{label}] stats {name}: max_abs={np.nanmax(err) if err.size else 0:.3e} "
              f"max_rel={np.nanmax(np.where(both_nan, 0, rel)) if rel.size else 0:.3e}", flush=True)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"[{label}] {name}{i}: gpu {g[i]!r} oracle {ov[i]!r}")
    return worst
