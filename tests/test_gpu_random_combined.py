"""Seeded random configurations through the combined sampling + statistics
calls (dense q and q from the draft's logits) and the allocation-free call:
the combined call's sampling outputs equal the sampling call's bit for bit,
its statistics meet the statistics bar, and the allocation-free call equals
the workspace call."""

import numpy as np
import pytest
import torch

import speculative_sampling_verification_sample_amd as sv
from test_gpu_random_configs import _configs
from test_gpu_sample_stats import _check
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [(s, kw) for s, kw in _configs(n=30, seed=90210) if kw["gamma"] > 0]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("shape,kw", CASES, ids=[f"{s}-{i}" for i, (s, _) in enumerate(CASES)])
def test_random_combined(shape, kw):
    w = generate(shape, DEV, **kw)
    label = f"random combined {shape} {kw}"
    _check(w, label)
    _check(w, label + " draft logits", draft_logits=True)


@pytest.mark.parametrize("shape,kw", CASES[:12], ids=[f"{s}-{i}" for i, (s, _) in enumerate(CASES[:12])])
def test_random_noalloc(shape, kw):
    w = generate(shape, DEV, **kw)
    c = w.cfg
    a = sv.verify_sample(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p)
    b = sv.verify_sample_noalloc(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
