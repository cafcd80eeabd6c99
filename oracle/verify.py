"""Plain float64 oracle of the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it and
for the page legend [WR] [AQ] [RL] [BS] [MN]).

Everything is computed one request and one row at a time in float64 NumPy.
Inputs are widened exactly first: bfloat16 bit patterns via
``bf16_bits_to_f64``, float32 values (q, uniforms, temperature, top_p) by a
plain float32 -> float64 conversion, so the oracle sees the very numbers the
library is given.

Conventions where the pages leave a step open (each one is listed, with its
reason, in the design notes of the repository):

* processing order: temperature, then top-k on the logits, then top-p on the
  renormalised top-k distribution, then renormalisation;
* top-k keeps every token whose logit is >= the k-th largest logit (ties at
  the cut are all kept);
* top-p keeps the smallest most-probable prefix whose mass reaches top_p plus
  every token tied (by logit) with the last one taken;
* acceptance is the strict comparison ``u < p(d)/q(d)``; q(d) = 0 accepts iff
  p(d) > 0 and raises FLAG_Q_ZERO;
* a sampled token is the first id (ascending) whose running sum of the
  weights exceeds ``u * W`` (no division by W); if rounding leaves none, the
  largest id with positive weight;
* an empty residual (Z = 0) raises FLAG_Z_DEGENERATE and samples from p of
  that position with the same uniform;
* a request whose logits hold NaN or +Inf (or a row that is all -Inf), or
  whose q(d_j) is NaN / negative / +Inf, raises FLAG_NONFINITE and emits no
  token (n_accepted = 0, every slot -1);
* a draft id outside [0, V) is rejected at its position and raises
  FLAG_BAD_ID;
* the residual weight is ``p - q`` where that difference is > 0 and 0
  otherwise (so a NaN q entry contributes no weight);
* with an end-of-sequence id (``eos >= 0``) nothing is committed after the
  first EOS: an accepted draft equal to EOS ends the request's output there
  (it becomes the last emitted token, so n_accepted counts the drafts before
  it and no token is drawn), and FLAG_EOS is raised whenever an EOS is
  emitted;
* in a ragged batch, a request whose draft span is out of order, out of
  range or longer than gamma_max raises FLAG_BAD_SPAN and emits nothing;
* lenient acceptance with factor beta in (0, 1] compares the target with the
  draft scaled to beta * q, in the acceptance (u < p / (beta q)) and in the
  residual ((p - beta q)_+); beta = 1 is the lossless rule.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Per-request status bits (same numeric values as the C header declares; the
# values are restated here, not imported, so the oracle shares nothing with
# the library).
FLAG_BAD_ID = 1
FLAG_Q_ZERO = 2
FLAG_Z_DEGENERATE = 4
FLAG_NONFINITE = 8
FLAG_EOS = 16
FLAG_BAD_SPAN = 32

# Half-width of the band around an acceptance, CDF or top-p boundary inside
# which float32 vs float64 rounding may legitimately flip a decision.
BOUNDARY_EPS = 1e-6


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (int16 / uint16) to float64.

    A bfloat16 value is the upper half of an IEEE float32, so shifting the 16
    bits into the top of a 32-bit word gives the float32 exactly.
    """
    b = np.ascontiguousarray(np.asarray(bits).astype(np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _f32(x) -> float:
    """The float64 value of x rounded to float32 (what the library is handed)."""
    return float(np.float32(x))


@dataclass
class ProcessedRow:
    """One position's processed target distribution."""

    p: np.ndarray  # float64 [V], exactly zero outside the kept set
    kept: np.ndarray  # bool [V]
    nonfinite: bool
    top_p_boundary: bool


def truncation_set(z: np.ndarray, T: float, top_k: int, top_p: float):
    """Kept set after top-k and top-p, plus the top-p boundary diagnostic.

    [WR] §7.3 (top-k / top-p zero out part of the vocabulary; the mass they
    leave is what p means) and [WR] §2.3 (p is the distribution after the
    production decoding rules).  The pages give no tie rule; ties at the cut
    are kept (see module docstring).
    Returns (kept, e, boundary) with e = exp(z/T - max) on the kept set.
    """
    V = z.size
    y = z / T
    kept = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        tau_k = np.sort(z)[::-1][top_k - 1]  # k-th largest, counted with multiplicity
        kept = z >= tau_k
    m = y[kept].max()
    e = np.where(kept, np.exp(y - m), 0.0)
    boundary = False
    if top_p < 1.0:
        p = e / e.sum()
        idx = np.nonzero(kept)[0]
        order = idx[np.argsort(-p[idx], kind="stable")]  # most probable first
        C = np.cumsum(p[order])
        hits = np.nonzero(C >= top_p)[0]
        n_star = int(hits[0]) if hits.size else len(order) - 1
        v_star = z[order[n_star]]
        boundary = abs(C[n_star] - top_p) < BOUNDARY_EPS or (
            n_star > 0 and abs(C[n_star - 1] - top_p) < BOUNDARY_EPS
        )
        kept = kept & (z >= v_star)
        e = np.where(kept, e, 0.0)
    return kept, e, boundary


def process_row(z, T: float, top_k: int = 0, top_p: float = 1.0) -> ProcessedRow:
    """Processed target distribution p of one position.

    [WR] §7.2 (temperature: p_T = softmax(z / T)), [WR] §7.3 and §2.3
    (truncation; p is the distribution actually sampled from), [MN] §二
    (notation table: p is the distribution after the sampling parameters).
    T and top_p are taken as the float32 values a caller hands the library.
    """
    z = np.asarray(z, dtype=np.float64)
    T = _f32(T)
    top_p = _f32(top_p)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return ProcessedRow(np.zeros_like(z), np.zeros(z.shape, bool), True, False)
    kept, e, boundary = truncation_set(z, T, int(top_k), top_p)
    p = e / e.sum()
    return ProcessedRow(p, kept, False, boundary)


def inverse_cdf(w: np.ndarray, u: float):
    """Draw one token from the non-negative weights w with the uniform u.

    The pages sample a discrete law without naming a method ([WR] §8 sample
    helper; [AQ] Python demo).  Reading used here: inverse CDF in ascending
    token id, strict ``C_x > u * W`` with C the running sum and W = sum(w).
    Returns (token, boundary) where boundary flags |C_x - t| < 1e-6 W at a
    token of positive weight.
    """
    C = np.cumsum(w)
    W = C[-1]
    t = float(u) * W
    over = np.nonzero(C > t)[0]
    pos = np.nonzero(w > 0)[0]
    if over.size:
        token = int(over[0])
    else:
        token = int(pos[-1])
    boundary = bool(pos.size) and float(np.min(np.abs(C[pos] - t))) < BOUNDARY_EPS * W
    return token, boundary


def residual_weights(p, q) -> np.ndarray:
    """Unnormalised residual (p - q)_+ of one position.

    [WR] §5 (r = max(0, p - q) / sum max(0, p - q)), [BS] §四 eq. (2),
    [RL] §2 (p'(x) = max(0, p - q) / Z).  Sampling by ``inverse_cdf`` needs
    no division by Z.  An entry counts only where p - q > 0.
    """
    diff = np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64)
    return np.where(diff > 0.0, diff, 0.0)


@dataclass
class RequestResult:
    tokens: np.ndarray  # int32 [gamma+1], -1 padded
    n_accepted: int
    flags: int
    accept_boundary: bool = False
    cdf_boundary: bool = False
    top_p_boundary: bool = False


def _no_output(gamma: int, flags: int) -> RequestResult:
    return RequestResult(np.full(gamma + 1, -1, np.int32), 0, flags)


def verify_from_processed(p_rows, q_rows, ids, u_accept, u_resample, top_p_boundary=False, eos=-1, beta=1.0):
    """Left-to-right verification of gamma drafts given processed p rows.

    [WR] §6 (verify d_1 with p_1 / q_1, stop at the first rejection, draw the
    replacement from that position's residual, or a bonus token from
    p_{gamma+1} when all gamma drafts pass), [WR] §4.1 (acceptance
    min(1, p/q), zero q handled explicitly), [WR] §5 and [BS] §四 eq. (2)
    (residual (p - q)_+ / Z), [RL] §1 steps 3-4, [WR] §10 (a round emits
    n_accepted + 1 tokens).  With ``eos >= 0``: [WR] §14.3 (runtime
    invariants: no token is committed after an EOS) -- an accepted draft
    equal to eos is the last emitted token and verification stops there.
    With ``beta < 1``: [MN] §八 (lenience) -- the draft distribution is
    scaled to beta * q before it is compared with the target, so a draft is
    accepted with min(1, p / (beta q)); the pages give no residual for this
    variant, and the plainest reading of "scale, then compare" keeps the
    rest of the step with beta * q in place of q: the replacement comes
    from (p - beta q)_+.
    """
    gamma = len(ids)
    V = p_rows[0].size
    ids = [int(d) for d in ids]
    # q(d_j) must be a valid probability wherever the id is valid.
    for j, d in enumerate(ids):
        if 0 <= d < V:
            qd = float(q_rows[j][d])
            if not (qd >= 0.0) or np.isinf(qd):
                return _no_output(gamma, FLAG_NONFINITE)
    if beta != 1.0:
        q_rows = [float(beta) * np.asarray(q, dtype=np.float64) for q in q_rows]
    flags = 0
    acc_boundary = False
    n_acc = gamma
    for j, d in enumerate(ids):
        if not (0 <= d < V):
            flags |= FLAG_BAD_ID
            n_acc = j
            break
        pd = float(p_rows[j][d])
        qd = float(q_rows[j][d])
        u = float(u_accept[j])
        if qd == 0.0:
            flags |= FLAG_Q_ZERO
            accept = pd > 0.0
        else:
            a = pd / qd
            accept = u < a
            if a < 1.0 and abs(u - a) < BOUNDARY_EPS:
                acc_boundary = True
        if not accept:
            n_acc = j
            break
        if d == eos:
            tokens = np.full(gamma + 1, -1, np.int32)
            tokens[: j + 1] = ids[: j + 1]
            return RequestResult(tokens, j, flags | FLAG_EOS, acc_boundary, False, top_p_boundary)
    if n_acc < gamma:
        w = residual_weights(p_rows[n_acc], q_rows[n_acc])
        if not (w.sum() > 0.0):
            flags |= FLAG_Z_DEGENERATE
            w = p_rows[n_acc]
    else:
        w = p_rows[gamma]
    token, cdf_boundary = inverse_cdf(w, float(u_resample[n_acc]))
    tokens = np.full(gamma + 1, -1, np.int32)
    tokens[:n_acc] = ids[:n_acc]
    tokens[n_acc] = token
    if eos >= 0 and token == eos:
        flags |= FLAG_EOS
    return RequestResult(tokens, n_acc, flags, acc_boundary, cdf_boundary, top_p_boundary)


def verify_request(z_rows, q_rows, ids, u_accept, u_resample, T, top_k=0, top_p=1.0, eos=-1, beta=1.0):
    """One request of the sampling verify step, from logits.

    Processes every position j = 0..gamma ([WR] §6: the target forward gives
    p_1 .. p_{gamma+1}; [BS] §三: the last one is the bonus distribution)
    and then verifies with ``verify_from_processed``.
    """
    gamma = len(ids)
    rows = [process_row(z_rows[j], T, top_k, top_p) for j in range(gamma + 1)]
    if any(r.nonfinite for r in rows):
        return _no_output(gamma, FLAG_NONFINITE)
    q64 = [np.asarray(q_rows[j], dtype=np.float64) for j in range(gamma)]
    return verify_from_processed(
        [r.p for r in rows], q64, ids, u_accept, u_resample,
        top_p_boundary=any(r.top_p_boundary for r in rows), eos=eos, beta=beta,
    )


def _batch_result(results, gamma):
    B = len(results)
    out = {
        "tokens": np.stack([r.tokens for r in results]) if B else np.zeros((0, gamma + 1), np.int32),
        "n_accepted": np.array([r.n_accepted for r in results], np.int32),
        "flags": np.array([r.flags for r in results], np.uint32),
        "accept_boundary": np.array([r.accept_boundary for r in results], bool),
        "cdf_boundary": np.array([r.cdf_boundary for r in results], bool),
        "top_p_boundary": np.array([r.top_p_boundary for r in results], bool),
    }
    return out


def verify_sample(logits, q, ids, u_accept, u_resample, T, top_k=0, top_p=1.0, requests=None, beta=1.0):
    """Batched sampling verify: loops ``verify_request`` over requests.

    logits: float64 [B, gamma+1, V] (already widened); q: [B, gamma, V];
    ids: [B, gamma]; u_accept: [B, gamma]; u_resample: [B, gamma+1].
    ``requests`` optionally restricts the loop to a list of request indices;
    ``beta`` is the lenience factor (1: lossless).
    """
    req = range(logits.shape[0]) if requests is None else requests
    gamma = ids.shape[1]
    res = [
        verify_request(logits[b], q[b], ids[b], u_accept[b], u_resample[b], T, top_k, top_p, beta=beta)
        for b in req
    ]
    return _batch_result(res, gamma)


def greedy_request(z_rows, ids, eos=-1) -> RequestResult:
    """Greedy verify: the longest draft prefix equal to the target argmax.

    [WR] §7.1 (accept d_i iff it is the target's most probable token,
    otherwise emit that token), [RL] §2 last paragraph (greedy keeps the
    longest matching prefix), [BS] §二 worked example (mat/and/the/dog vs
    the target's top-1).  Argmax ties go to the lowest id (first occurrence).
    A row holding NaN raises FLAG_NONFINITE and the request emits nothing.
    With ``eos >= 0`` a matching draft equal to eos ends the output there
    ([WR] §14.3), as in ``verify_from_processed``.
    """
    z_rows = np.asarray(z_rows, dtype=np.float64)
    gamma = len(ids)
    if np.isnan(z_rows).any():
        return _no_output(gamma, FLAG_NONFINITE)
    V = z_rows.shape[1]
    g = [int(np.argmax(z_rows[j])) for j in range(gamma + 1)]
    n_acc = gamma
    flags = 0
    tokens = np.full(gamma + 1, -1, np.int32)
    for j in range(gamma):
        if int(ids[j]) != g[j]:
            n_acc = j
            if not (0 <= int(ids[j]) < V):
                flags |= FLAG_BAD_ID
            break
        if g[j] == eos:
            tokens[: j + 1] = [int(d) for d in ids[: j + 1]]
            return RequestResult(tokens, j, flags | FLAG_EOS)
    tokens[:n_acc] = [int(d) for d in ids[:n_acc]]
    tokens[n_acc] = g[n_acc]
    if eos >= 0 and g[n_acc] == eos:
        flags |= FLAG_EOS
    return RequestResult(tokens, n_acc, flags)


def verify_greedy(logits, ids, requests=None):
    req = range(logits.shape[0]) if requests is None else requests
    res = [greedy_request(logits[b], ids[b]) for b in req]
    return _batch_result(res, ids.shape[1])


def stats_request(z_rows, q_rows, ids, T, top_k=0, top_p=1.0, boundary_out=None):
    """Per-position acceptance statistics of one request (positions j < gamma).

    alpha_j = sum_x min(p_j, q_j) ([WR] §4.2; [MN] §三, alpha = 1 - TV),
    Z_j = sum_x (p_j - q_j)_+ and Z'_j = sum_x (q_j - p_j)_+ ([RL] §2; [BS]
    §五: both equal the rejection probability when p and q are normalised),
    a_j = min(1, p_j(d_j) / q_j(d_j)) ([WR] §6).  q is used as given (not
    renormalised).  q_j(d_j) = 0 gives a_j = 1 if p_j(d_j) > 0 else 0; an id
    outside [0, V) gives a_j = NaN; a non-finite logits row gives NaN in all
    four outputs of that position.  ``boundary_out`` (a bool array of length
    gamma), when given, receives each position's top-p boundary diagnostic
    (``process_row``): a kept set decided within 1e-6 of top_p.
    """
    gamma = len(ids)
    out = np.full((4, gamma), np.nan)
    for j in range(gamma):
        r = process_row(z_rows[j], T, top_k, top_p)
        if boundary_out is not None:
            boundary_out[j] = r.top_p_boundary
        if r.nonfinite:
            continue
        p = r.p
        q = np.asarray(q_rows[j], dtype=np.float64)
        diff = p - q
        out[0, j] = np.minimum(p, q).sum()
        out[1, j] = np.where(diff > 0, diff, 0.0).sum()
        out[2, j] = np.where(diff < 0, -diff, 0.0).sum()
        d = int(ids[j])
        if 0 <= d < p.size:
            if q[d] == 0.0:
                out[3, j] = 1.0 if p[d] > 0 else 0.0
            else:
                out[3, j] = min(1.0, p[d] / q[d])
    return out


def accept_stats(logits, q, ids, T, top_k=0, top_p=1.0, requests=None, with_boundary=False):
    """Batched ``stats_request``; returns (alpha, z_pq, z_qp, accept_prob), each [B', gamma],
    and with ``with_boundary`` a fifth [B', gamma] bool array: the top-p boundary
    diagnostic of each position."""
    req = list(range(logits.shape[0]) if requests is None else requests)
    gamma = ids.shape[1]
    bnd = np.zeros((len(req), gamma), bool)
    res = [stats_request(logits[b], q[b], ids[b], T, top_k, top_p, boundary_out=bnd[i]) for i, b in enumerate(req)]
    if not res:
        out = tuple(np.zeros((0, gamma)) for _ in range(4))
    else:
        arr = np.stack(res)  # [B', 4, gamma]
        out = (arr[:, 0], arr[:, 1], arr[:, 2], arr[:, 3])
    return out + (bnd,) if with_boundary else out


# --------------------------------------------------------------------------
# q formed from the draft's logits
# --------------------------------------------------------------------------

def draft_q_rows(dz_rows, T, top_k=0, top_p=1.0):
    """The draft distributions q_j formed from the draft's logits.

    [WR] §2.3 and [MN] §二 (notation): q, like p, is the distribution after
    the decoding rules, so q_j is the draft's logits row put through exactly
    the processing of ``process_row`` with the same parameters.  A draft row
    holding NaN / +Inf (or all -Inf) has no q: its row is NaN.
    Returns (rows, top_p_boundary), the second flag as in ``process_row``.
    """
    rows = []
    boundary = False
    for z in dz_rows:
        r = process_row(z, T, top_k, top_p)
        rows.append(np.full(np.asarray(z).size, np.nan) if r.nonfinite else r.p)
        boundary = boundary or r.top_p_boundary
    return rows, boundary


def verify_request_draft_logits(z_rows, dz_rows, ids, u_accept, u_resample, T, top_k=0, top_p=1.0):
    """``verify_request`` with q_j = the processed draft logits row j."""
    q_rows, q_boundary = draft_q_rows(dz_rows, T, top_k, top_p)
    res = verify_request(z_rows, q_rows, ids, u_accept, u_resample, T, top_k, top_p)
    res.top_p_boundary = res.top_p_boundary or q_boundary
    return res


def verify_sample_draft_logits(logits, draft_logits, ids, u_accept, u_resample, T, top_k=0, top_p=1.0,
                               requests=None):
    """Batched ``verify_request_draft_logits``; draft_logits: float64 [B, gamma, V]."""
    req = range(logits.shape[0]) if requests is None else requests
    gamma = ids.shape[1]
    res = [
        verify_request_draft_logits(logits[b], draft_logits[b], ids[b], u_accept[b], u_resample[b], T, top_k,
                                    top_p)
        for b in req
    ]
    return _batch_result(res, gamma)


def stats_request_draft_logits(z_rows, dz_rows, ids, T, top_k=0, top_p=1.0, boundary_out=None):
    """``stats_request`` with q_j = the processed draft logits row j; a
    position whose draft row has no q gives NaN in all four outputs.
    ``boundary_out`` receives each position's top-p boundary diagnostic, of
    the target's or the draft's row."""
    q_rows = []
    qb = np.zeros(len(ids), bool)
    for j in range(len(ids)):
        rows, qb[j] = draft_q_rows(dz_rows[j:j + 1], T, top_k, top_p)
        q_rows.append(rows[0])
    out = stats_request(z_rows, q_rows, ids, T, top_k, top_p, boundary_out=boundary_out)
    if boundary_out is not None:
        boundary_out |= qb
    for j, q in enumerate(q_rows):
        if np.isnan(q).all():
            out[:, j] = np.nan
    return out


def accept_stats_draft_logits(logits, draft_logits, ids, T, top_k=0, top_p=1.0, requests=None,
                              with_boundary=False):
    """Batched ``stats_request_draft_logits``; returns (alpha, z_pq, z_qp, accept_prob)
    (plus the per-position top-p boundary diagnostic with ``with_boundary``)."""
    req = list(range(logits.shape[0]) if requests is None else requests)
    gamma = ids.shape[1]
    bnd = np.zeros((len(req), gamma), bool)
    res = [stats_request_draft_logits(logits[b], draft_logits[b], ids[b], T, top_k, top_p, boundary_out=bnd[i])
           for i, b in enumerate(req)]
    if not res:
        out = tuple(np.zeros((0, gamma)) for _ in range(4))
    else:
        arr = np.stack(res)
        out = (arr[:, 0], arr[:, 1], arr[:, 2], arr[:, 3])
    return out + (bnd,) if with_boundary else out


# --------------------------------------------------------------------------
# Ragged batches: request b drafted gamma_b tokens
# --------------------------------------------------------------------------

def ragged_span(cu, b, n_draft, gamma_max):
    """Draft positions [lo, hi) of request b in the packed arrays, or None
    when the span is out of order, out of range or longer than gamma_max.

    The packed layout: request b's gamma_b = cu[b+1] - cu[b] drafts are
    positions cu[b] .. cu[b+1]-1 of the draft arrays, and its gamma_b + 1
    target rows (and resampling uniforms) are rows cu[b] + b .. cu[b+1] + b
    ([WR] §11.2 and [MN] §九 point 3: no one draft length suits every
    request, so gamma is adapted per request and a batch holds different
    gamma_b).
    """
    lo, hi = int(cu[b]), int(cu[b + 1])
    if not (0 <= lo <= hi <= n_draft and hi - lo <= gamma_max):
        return None
    return lo, hi


def _pad_result(res, gamma_max):
    tokens = np.full(gamma_max + 1, -1, np.int32)
    tokens[: res.tokens.size] = res.tokens
    res.tokens = tokens
    return res


def verify_sample_ragged(logits, q, ids, cu, u_accept, u_resample, gamma_max, T, top_k=0, top_p=1.0, eos=-1,
                         requests=None):
    """Sampling verify of a ragged batch: ``verify_request`` on each
    request's own gamma_b rows (layout in ``ragged_span``).

    logits: float64 [N + B, V]; q: [N, V]; ids, u_accept: [N];
    u_resample: [N + B]; cu: [B + 1].  Tokens are returned padded to
    gamma_max + 1.
    """
    B = len(cu) - 1
    N = ids.shape[0]
    req = range(B) if requests is None else requests
    res = []
    for b in req:
        sp = ragged_span(cu, b, N, gamma_max)
        if sp is None:
            res.append(_no_output(gamma_max, FLAG_BAD_SPAN))
            continue
        lo, hi = sp
        r = verify_request(logits[lo + b: hi + b + 1], q[lo:hi], ids[lo:hi], u_accept[lo:hi],
                           u_resample[lo + b: hi + b + 1], T, top_k, top_p, eos)
        res.append(_pad_result(r, gamma_max))
    return _batch_result(res, gamma_max)


def verify_greedy_ragged(logits, ids, cu, gamma_max, eos=-1, requests=None):
    """Greedy verify of a ragged batch (``greedy_request`` per request)."""
    B = len(cu) - 1
    N = ids.shape[0]
    req = range(B) if requests is None else requests
    res = []
    for b in req:
        sp = ragged_span(cu, b, N, gamma_max)
        if sp is None:
            res.append(_no_output(gamma_max, FLAG_BAD_SPAN))
            continue
        lo, hi = sp
        res.append(_pad_result(greedy_request(logits[lo + b: hi + b + 1], ids[lo:hi], eos), gamma_max))
    return _batch_result(res, gamma_max)


def verify_sample_ragged_draft_logits(logits, draft_logits, ids, cu, u_accept, u_resample, gamma_max, T, top_k=0,
                                      top_p=1.0, eos=-1, requests=None):
    """``verify_sample_ragged`` with q formed from the draft's logits (packed
    [N, V], one row per draft position) by ``draft_q_rows``."""
    B = len(cu) - 1
    N = ids.shape[0]
    req = range(B) if requests is None else requests
    res = []
    for b in req:
        sp = ragged_span(cu, b, N, gamma_max)
        if sp is None:
            res.append(_no_output(gamma_max, FLAG_BAD_SPAN))
            continue
        lo, hi = sp
        q_rows, q_boundary = draft_q_rows(draft_logits[lo:hi], T, top_k, top_p)
        r = verify_request(logits[lo + b: hi + b + 1], q_rows, ids[lo:hi], u_accept[lo:hi],
                           u_resample[lo + b: hi + b + 1], T, top_k, top_p, eos)
        r.top_p_boundary = r.top_p_boundary or q_boundary
        res.append(_pad_result(r, gamma_max))
    return _batch_result(res, gamma_max)
