"""Build the inputs of one workload on a torch device from its seed."""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import CONFIGS, Config


@dataclass
class Workload:
    cfg: Config
    logits: torch.Tensor  # [B, gamma+1, V] float32 or bfloat16
    q: Optional[torch.Tensor]  # [B, gamma, V] float32 (None for greedy)
    ids: torch.Tensor  # [B, gamma] int32
    u_accept: torch.Tensor  # [B, gamma] float32
    u_resample: torch.Tensor  # [B, gamma+1] float32
    # [B, gamma, V] the draft's logits that q was formed from (None for greedy)
    draft_logits: Optional[torch.Tensor] = None

    @property
    def device(self):
        return self.logits.device


def _generators(seed: int, device) -> list:
    gens = []
    for child in np.random.SeedSequence(seed).spawn(4):
        g = torch.Generator(device=device)
        g.manual_seed(int(child.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
        gens.append(g)
    return gens


def _uniform24(shape, gen, device) -> torch.Tensor:
    """float32 uniforms k * 2^-24, k in [0, 2^24): exact in float32, never 1."""
    k = torch.randint(0, 1 << 24, shape, generator=gen, device=device, dtype=torch.int64)
    return k.to(torch.float32) * (2.0 ** -24)


def _draft_distribution(draft: torch.Tensor, T: float, top_k: int, top_p: float) -> torch.Tensor:
    """The draft model's own sampling distribution (draft-side recipe).

    softmax(draft / T) restricted to the draft's top-k (ties kept) and/or its
    nucleus of mass top_p (ties kept), renormalised, rounded to float32.  The
    verify step receives this q as input and never recomputes it.
    """
    x = draft.to(torch.float64)
    V = x.shape[-1]
    keep = torch.ones_like(x, dtype=torch.bool)
    if 0 < top_k < V:
        kth = torch.topk(x, top_k, dim=-1).values[..., -1:]
        keep = x >= kth
    logit = torch.where(keep, x / T, torch.full_like(x, -math.inf))
    prob = torch.softmax(logit, dim=-1)
    if top_p < 1.0:
        vals, order = torch.sort(prob, dim=-1, descending=True)
        csum = torch.cumsum(vals, dim=-1)
        n_star = torch.searchsorted(csum, torch.full_like(csum[..., :1], top_p), right=False)
        n_star = n_star.clamp(max=V - 1)
        cut_id = torch.gather(order, -1, n_star)
        cut_val = torch.gather(x, -1, cut_id)
        keep = keep & (x >= cut_val)
        del vals, order, csum
        prob = torch.where(keep, prob, torch.zeros_like(prob))
        prob = prob / prob.sum(dim=-1, keepdim=True)
    return prob.to(torch.float32)


def _sample_ids(q: torch.Tensor, gen, device) -> torch.Tensor:
    """Draft ids d ~ q by inverse CDF in float64 (only ids with q > 0 occur)."""
    lead = q.shape[:-1]
    V = q.shape[-1]
    cdf = torch.cumsum(q.to(torch.float64), dim=-1)
    u = _uniform24(lead + (1,), gen, device).to(torch.float64)
    t = u * cdf[..., -1:]
    ids = torch.searchsorted(cdf, t, right=True).clamp(max=V - 1)
    return ids.squeeze(-1).to(torch.int32)


def _finish(cfg, logits, q, ids, gens, device, draft=None) -> Workload:
    u = _uniform24((cfg.B, cfg.gamma + 1, 2), gens[3], device)
    u_accept = u[:, : cfg.gamma, 0].contiguous()
    u_resample = u[:, :, 1].contiguous()
    return Workload(cfg, logits.contiguous(), None if q is None else q.contiguous(),
                    ids.contiguous(), u_accept, u_resample, None if draft is None else draft.contiguous())


def generate(cfg, device="cpu", **override) -> Workload:
    """Inputs of workload ``cfg`` (a Config or its name) on ``device``.

    Keyword overrides (B, gamma, V, seed, temperature, top_k, top_p, ...)
    give smaller or edge-case variants built by the same recipe.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if override:
        cfg = cfg.with_(**override)
    device = torch.device(device)
    gens = _generators(cfg.seed, device)
    B, G, V = cfg.B, cfg.gamma, cfg.V
    T = float(np.float32(cfg.temperature))
    shape = (B, G + 1, V)

    if cfg.name.startswith("toy"):
        return _toy(cfg, gens, device)

    if cfg.name.startswith("c2"):
        z = 2.0 * torch.randn(shape, generator=gens[0], device=device)
        draft = z[:, :G] + 0.5 * torch.randn((B, G, V), generator=gens[1], device=device)
        q = _draft_distribution(draft, T, cfg.top_k, cfg.top_p)
        ids = _sample_ids(q, gens[2], device)
        return _finish(cfg, z.to(torch.float32), q, ids, gens, device, draft.to(torch.float32))

    if cfg.name.startswith("c3"):
        z = 3.0 * torch.randn(shape, generator=gens[0], device=device)
        n_boost = int(math.floor(0.01 * V))
        if n_boost > 0:
            flat = z.view(-1, V)
            pick = torch.rand(flat.shape, generator=gens[0], device=device).argsort(dim=1)[:, :n_boost]
            flat.scatter_add_(1, pick, torch.full(pick.shape, 6.0, device=device))
            del pick
        draft = (z[:, :G] + torch.randn((B, G, V), generator=gens[1], device=device)).to(torch.bfloat16)
        logits = z.to(torch.bfloat16)
        del z
        q = _draft_distribution(draft.to(torch.float32), T, cfg.top_k, cfg.top_p)
        ids = _sample_ids(q, gens[2], device)
        return _finish(cfg, logits, q, ids, gens, device, draft)

    if cfg.name.startswith("c4"):
        logits = (2.5 * torch.randn(shape, generator=gens[0], device=device)).to(torch.bfloat16)
        noisy = logits[:, :G].to(torch.float32) + 0.3 * torch.randn((B, G, V), generator=gens[1], device=device)
        ids = torch.argmax(noisy, dim=-1).to(torch.int32)  # first maximal index on ties
        del noisy
        return _finish(cfg, logits, None, ids, gens, device)

    if cfg.name.startswith("c5"):
        rows = B * (G + 1)
        rank = torch.rand((rows, V), generator=gens[0], device=device).argsort(dim=1).to(torch.float32) + 1.0
        z = (-1.1 * torch.log(rank)).view(shape)
        del rank
        z += 0.5 * torch.randn(shape, generator=gens[0], device=device)
        draft = (z[:, :G] + 0.8 * torch.randn((B, G, V), generator=gens[1], device=device)).to(torch.bfloat16)
        logits = z.to(torch.bfloat16)
        del z
        q = _draft_distribution(draft.to(torch.float32), T, cfg.top_k, cfg.top_p)
        ids = _sample_ids(q, gens[2], device)
        return _finish(cfg, logits, q, ids, gens, device, draft)

    raise ValueError(f"unknown workload {cfg.name}")


def _toy(cfg, gens, device) -> Workload:
    """Toy: one request's (p, q) rows replicated over B rounds.

    Target rows p_j ~ Dirichlet(1) (an Exponential(1) vector, normalised),
    logits = float32(ln p_j); draft q_j = float32(normalise(0.6 p_j + 0.4/V)).
    Each round draws fresh draft ids (from q) and fresh uniforms.  A config
    name ending in "const" replicates position 0 to every position, so the
    acceptance probability is the same at every position.
    """
    B, G, V = cfg.B, cfg.gamma, cfg.V
    e = -torch.log1p(-torch.rand((G + 1, V), generator=gens[0], device=device, dtype=torch.float64))
    P = e / e.sum(dim=-1, keepdim=True)
    if cfg.name.endswith("const"):
        P = P[:1].expand(G + 1, V).contiguous()
    Q = 0.6 * P[:G] + 0.4 / V
    Q = (Q / Q.sum(dim=-1, keepdim=True)).to(torch.float32)
    logits1 = torch.log(P).to(torch.float32)
    logits = logits1.unsqueeze(0).expand(B, G + 1, V)
    q = Q.unsqueeze(0).expand(B, G, V)
    ids = _sample_ids(q, gens[2], device)
    # draft logits whose processed distribution (T = 1, no truncation) is Q
    draft = torch.log(Q.to(torch.float64)).to(torch.float32).unsqueeze(0).expand(B, G, V)
    return _finish(cfg, logits, q, ids, gens, device, draft)


@dataclass
class RaggedWorkload:
    """A batch whose request b drafted gammas[b] tokens, in the packed layout:
    request b's drafts are positions cu[b] .. cu[b+1]-1 of ids / q /
    u_accept (/ draft_logits) and its gammas[b] + 1 target rows (and
    resampling uniforms) start at row cu[b] + b."""
    cfg: Config
    gamma_max: int
    gammas: np.ndarray              # [B] int
    cu: torch.Tensor                # [B + 1] int32
    logits: torch.Tensor            # [N + B, V]
    q: Optional[torch.Tensor]       # [N, V] float32 (None for greedy)
    ids: torch.Tensor               # [N] int32
    u_accept: torch.Tensor          # [N] float32
    u_resample: torch.Tensor        # [N + B] float32
    draft_logits: Optional[torch.Tensor] = None  # [N, V] (when the workload has them)


def ragged_gammas(B: int, gamma_max: int, seed: int) -> np.ndarray:
    """Per-request draft lengths, uniform on {0, .., gamma_max} (seeded)."""
    return np.random.default_rng(seed).integers(0, gamma_max + 1, B)


def pack_ragged(w: Workload, gammas) -> RaggedWorkload:
    """Keep the first gammas[b] drafts of each request of a uniform workload
    (and its first gammas[b] + 1 target rows), packed without padding."""
    gammas = np.asarray(gammas, dtype=np.int64)
    B, G1, V = w.logits.shape
    G = G1 - 1
    if gammas.shape != (B,) or gammas.min(initial=0) < 0 or gammas.max(initial=0) > G:
        raise ValueError("gammas must be [B] values in [0, gamma]")
    dev = w.logits.device
    rows = np.concatenate([b * G1 + np.arange(g + 1) for b, g in enumerate(gammas)]).astype(np.int64)
    drafts = np.concatenate([b * G + np.arange(g) for b, g in enumerate(gammas)] + [np.zeros(0, np.int64)])
    ri = torch.as_tensor(rows, device=dev)
    di = torch.as_tensor(drafts.astype(np.int64), device=dev)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(gammas)]).astype(np.int32), device=dev)
    return RaggedWorkload(
        w.cfg, G, gammas, cu,
        w.logits.reshape(B * G1, V).index_select(0, ri).contiguous(),
        None if w.q is None else w.q.reshape(B * G, V).index_select(0, di).contiguous(),
        w.ids.reshape(-1).index_select(0, di).contiguous(),
        w.u_accept.reshape(-1).index_select(0, di).contiguous(),
        w.u_resample.reshape(-1).index_select(0, ri).contiguous(),
        None if w.draft_logits is None else w.draft_logits.reshape(B * G, V).index_select(0, di).contiguous(),
    )
