"""A seeded sweep over every call form at once: each case draws a workload
shape, a vocabulary size from 2 to 300 001 (powers of two, one off them,
primes), a batch up to 400 requests, drafts up to 79 long, a temperature
from 0.2 to 3, and top-k / top-p from none to 1 and 0.3, then runs one call
form (sampling with a dense q, with q from the draft's logits, lenient,
statistics, ragged with and without an end-of-sequence id, greedy) and
compares every request with the oracle."""

import numpy as np
import pytest
import torch

from parity import compare_greedy, compare_sample, compare_stats
from test_gpu_ragged import compare_ragged
from workloads import generate, pack_ragged

pytestmark = pytest.mark.gpu

DEV = "cuda"
VOCABS = [2, 3, 8, 15, 16, 17, 31, 64, 255, 256, 257, 1000, 4096, 5003, 16385, 50000, 100003, 262144, 300001]
FORMS = ["sample", "draft_logits", "lenient", "stats", "ragged", "greedy"]


def _cases(n=150, seed=9090):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        shape = ["c2", "c3", "c5"][int(rng.integers(0, 3))]
        V = int(rng.choice(VOCABS))
        B = int(rng.integers(1, 9)) if V < 100000 else int(rng.integers(1, 4))
        if rng.random() < 0.1 and V <= 5003:
            B = int(rng.integers(200, 400))
        gamma = int(rng.integers(0, 12)) if rng.random() < 0.9 else int(rng.integers(60, 80))
        kw = dict(B=B, gamma=gamma, V=V, temperature=float(rng.choice([0.2, 0.5, 0.7, 0.8, 1.0, 1.5, 3.0])),
                  top_k=int(rng.choice([0, 0, 0, 1, 2, 3, 10, 64, 256, 257, 600])),
                  top_p=float(rng.choice([1.0, 1.0, 0.3, 0.7, 0.9, 0.95, 0.999])), seed=900000 + i)
        if kw["top_k"] >= V:
            kw["top_k"] = 0
        form = FORMS[i % len(FORMS)]
        out.append((shape, kw, form, int(rng.integers(0, 2**31))))
    return out


CASES = _cases()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("shape,kw,form,cseed", CASES, ids=[f"{f}-{s}-{i}" for i, (s, _, f, _) in enumerate(CASES)])
def test_sweep(shape, kw, form, cseed):
    rng = np.random.default_rng(cseed)
    label = f"sweep {shape} {kw} {form}"
    if form == "greedy":
        compare_greedy(generate("c4", DEV, B=kw["B"], gamma=kw["gamma"], V=kw["V"], seed=kw["seed"]), label=label)
        return
    w = generate(shape, DEV, **kw)
    if form == "sample":
        compare_sample(w, label=label)
    elif form == "draft_logits":
        # with no drafts there is no q to form: the call is plain sampling
        compare_sample(w, label=label, draft_logits=kw["gamma"] > 0)
    elif form == "lenient":
        compare_sample(w, label=label, lenience=float(rng.choice([0.3, 0.8])))
    elif form == "stats":
        if kw["gamma"] == 0:  # no drafted positions: nothing to measure, sample instead
            compare_sample(w, label=label)
            return
        compare_stats(w, label=label)
        compare_stats(w, label=label + " draft logits", draft_logits=True)
    else:
        gammas = rng.integers(0, kw["gamma"] + 1, size=kw["B"])
        r = pack_ragged(w, gammas)
        eos = int(rng.integers(0, kw["V"])) if rng.random() < 0.5 else -1
        compare_ragged(r, eos=eos, label=label + f" gammas={gammas.tolist()} eos={eos}")
        if kw["gamma"] > 0:
            compare_ragged(r, eos=eos, label=label + " draft logits", draft_logits=True)
