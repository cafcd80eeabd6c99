"""More seeded random parity: ragged batches (dense q, q from the draft's
logits, greedy) with and without an end-of-sequence id; integer logits, so
that many tokens tie at the top-k and top-p cuts and at the argmax; batches
of 256 and more (the one-launch full-row sampler of untruncated rows);
drafts longer than 63 (the acceptance kernel for long drafts); top-k above
the fast path's limit (the exact selection).  Every request is compared with
the oracle."""

import numpy as np
import pytest
import torch

from parity import compare_greedy, compare_sample, compare_stats
from test_gpu_ragged import compare_ragged
from workloads import generate, pack_ragged

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _pick(rng, xs):
    return xs[int(rng.integers(0, len(xs)))]


def _ragged_cases(n=30, seed=5150):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        shape = ["c2", "c3", "c5", "toy"][i % 4]
        kw = dict(B=int(rng.integers(1, 9)), gamma=int(rng.integers(1, 9)), seed=50000 + i,
                  temperature=float(_pick(rng, [0.5, 0.7, 1.0, 1.3])))
        if shape != "toy":
            kw.update(V=int(_pick(rng, [9, 100, 2049, 7777, 30001])), top_k=int(_pick(rng, [0, 0, 3, 40])),
                      top_p=float(_pick(rng, [1.0, 1.0, 0.8, 0.97])))
        out.append((shape, kw, int(rng.integers(0, 2**31))))
    return out


RAGGED = _ragged_cases()


@pytest.mark.parametrize("shape,kw,gseed", RAGGED, ids=[f"{s}-{i}" for i, (s, _, _) in enumerate(RAGGED)])
def test_random_ragged(shape, kw, gseed):
    w = generate(shape, DEV, **kw)
    G = w.ids.shape[1]
    rng = np.random.default_rng(gseed)
    gammas = rng.integers(0, G + 1, size=w.cfg.B)
    r = pack_ragged(w, gammas)
    V = w.logits.shape[-1]
    eos = int(rng.integers(0, V)) if rng.random() < 0.5 else -1
    label = f"random ragged {shape} {kw} gammas={gammas.tolist()} eos={eos}"
    compare_ragged(r, eos=eos, label=label)
    compare_ragged(r, eos=eos, label=label + " draft logits", draft_logits=True)
    g = generate("c4", DEV, B=kw["B"], gamma=kw["gamma"], V=kw.get("V", 50), seed=kw["seed"])
    rg = pack_ragged(g, gammas)
    compare_ragged(rg, eos=eos, label=f"random ragged greedy {kw} eos={eos}", greedy=True)


def _integer_cases(n=15, seed=616):
    rng = np.random.default_rng(seed)
    return [(["c2", "c3", "c5"][i % 3],
             dict(B=int(rng.integers(1, 6)), gamma=int(rng.integers(1, 7)), V=int(_pick(rng, [50, 999, 5000])),
                  temperature=float(_pick(rng, [0.6, 1.0])), top_k=int(_pick(rng, [0, 1, 7, 60])),
                  top_p=float(_pick(rng, [1.0, 0.6, 0.9])), seed=60000 + i),
             float(_pick(rng, [1.0, 2.0, 4.0])))
            for i in range(n)]


INTEGER = _integer_cases()


@pytest.mark.parametrize("shape,kw,scale", INTEGER, ids=[f"{s}-{i}" for i, (s, _, _) in enumerate(INTEGER)])
def test_random_integer_logits(shape, kw, scale):
    """Logits rounded to multiples of 1/scale: ties everywhere."""
    w = generate(shape, DEV, **kw)
    lg = torch.round(w.logits.float() * scale) / scale
    w.logits = lg.to(w.logits.dtype).contiguous()
    label = f"integer logits {shape} {kw} scale={scale}"
    compare_sample(w, label=label)
    compare_stats(w, label=label)
    g = generate("c4", DEV, B=kw["B"], gamma=kw["gamma"], V=kw["V"], seed=kw["seed"])
    g.logits = (torch.round(g.logits.float() * scale) / scale).to(g.logits.dtype).contiguous()
    compare_greedy(g, label=f"integer logits greedy {kw} scale={scale}")


@pytest.mark.parametrize("shape,kw", [
    ("c2", dict(B=256, gamma=2, V=3001, seed=70001)),
    ("c2", dict(B=300, gamma=4, V=20000, seed=70002, temperature=0.7)),
    ("c5", dict(B=260, gamma=3, V=9000, seed=70003, top_p=1.0)),
    ("c3", dict(B=270, gamma=2, V=5000, seed=70004)),
])
def test_random_large_batches(shape, kw):
    w = generate(shape, DEV, **kw)
    compare_sample(w, label=f"large batch {shape} {kw}")
    compare_stats(w, label=f"large batch {shape} {kw}")


@pytest.mark.parametrize("shape,kw", [
    ("c2", dict(B=3, gamma=70, V=2000, seed=71001)),
    ("c2", dict(B=2, gamma=100, V=513, seed=71002, temperature=0.8)),
    ("c3", dict(B=2, gamma=66, V=4000, seed=71003)),
    ("c5", dict(B=2, gamma=64, V=3000, seed=71004)),
])
def test_random_long_drafts(shape, kw):
    w = generate(shape, DEV, **kw)
    compare_sample(w, label=f"long drafts {shape} {kw}")
    compare_sample(w, label=f"long drafts {shape} {kw} draft logits", draft_logits=True)


@pytest.mark.parametrize("top_k,top_p", [(257, 1.0), (400, 0.9), (1000, 0.5), (2500, 1.0)])
def test_random_large_top_k(top_k, top_p):
    w = generate("c3", DEV, B=3, gamma=3, V=20000, top_k=top_k, top_p=top_p, seed=72000 + top_k)
    compare_sample(w, label=f"top-k {top_k} top-p {top_p}")
    compare_stats(w, label=f"top-k {top_k} top-p {top_p}")


@pytest.mark.parametrize("shape,T,scale", [
    ("c2", 0.05, 1.0), ("c2", 5.0, 30.0), ("c2", 100.0, 1.0), ("c3", 0.05, 30.0),
    ("c3", 3.0, 0.01), ("c5", 0.1, 10.0), ("c5", 20.0, 1.0), ("c5", 0.7, 100.0),
])
def test_random_extreme_scales(shape, T, scale):
    """Sharp and flat distributions: small and large temperatures, logits
    scaled from 0.01x to 100x."""
    w = generate(shape, DEV, B=3, gamma=3, V=6000, temperature=T, seed=73000 + int(T * 100) + int(scale))
    w.logits = (w.logits.float() * scale).to(w.logits.dtype).contiguous()
    label = f"extreme {shape} T={T} scale={scale}"
    compare_sample(w, label=label)
    compare_stats(w, label=label)


@pytest.mark.parametrize("shape,factor", [("c2", 0.5), ("c3", 0.9), ("c5", 1.1), ("c2", 3.0), ("c5", 0.25),
                                          ("c3", 2.0)])
def test_random_unnormalised_q(shape, factor):
    """q as given, not summing to one (R11): the acceptance ratio, the
    residual (p - q)+ (which may vanish: Z_DEGENERATE) and the statistics
    all take it as it is."""
    w = generate(shape, DEV, B=5, gamma=4, V=7001, seed=74000 + int(factor * 100))
    w.q = (w.q * factor).contiguous()
    label = f"unnormalised q x{factor} {shape}"
    compare_sample(w, label=label)
    compare_sample(w, label=label + " lenient 0.7", lenience=0.7)
    compare_stats(w, label=label)
