"""Parity over a seeded spread of small configurations: the workloads' logit
shapes at random batch sizes, draft lengths, vocabulary sizes (most not a
multiple of 8), temperatures and top-k / top-p settings, including the
corners (top-k 1, top-k above the fast path's limit, top-k with top-p,
narrow nuclei).  Every request is compared with the oracle: sampling with a
dense q and with q formed from the draft's logits, lenient sampling on a
quarter of the cases, the statistics, and greedy."""

import numpy as np
import pytest
import torch

from parity import compare_greedy, compare_sample, compare_stats
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _configs(n=60, seed=20260):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        shape = ["c2", "c3", "c5"][i % 3]
        V = int(rng.choice([7, 33, 257, 1001, 4099, 12345, 32003, 40000]))
        top_k = int(rng.choice([0, 0, 1, 2, 5, 50, 300]))
        top_p = float(rng.choice([1.0, 1.0, 0.5, 0.9, 0.99]))
        kw = dict(B=int(rng.integers(1, 7)), gamma=int(rng.integers(0, 10)), V=V,
                  temperature=float(rng.choice([0.3, 0.7, 1.0, 1.7])), top_k=top_k if top_k < V else 0,
                  top_p=top_p, seed=30000 + i)
        out.append((shape, kw))
    return out


CASES = _configs()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("shape,kw", CASES, ids=[f"{s}-{i}" for i, (s, _) in enumerate(CASES)])
def test_random_config(shape, kw):
    w = generate(shape, DEV, **kw)
    label = f"random {shape} {kw}"
    compare_sample(w, label=label)
    if kw["seed"] % 4 == 0:
        compare_sample(w, label=label + " lenient 0.6", lenience=0.6)
    if kw["gamma"] > 0:
        compare_sample(w, label=label + " draft logits", draft_logits=True)
        compare_stats(w, label=label)
        compare_stats(w, label=label + " draft logits", draft_logits=True)


@pytest.mark.parametrize("i", range(6))
def test_random_greedy(i):
    rng = np.random.default_rng(777 + i)
    kw = dict(B=int(rng.integers(1, 9)), gamma=int(rng.integers(0, 12)),
              V=int(rng.choice([5, 63, 1000, 9999, 50001])), seed=40000 + i)
    compare_greedy(generate("c4", DEV, **kw), label=f"random greedy {kw}")
