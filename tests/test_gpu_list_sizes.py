"""Kept lists at the sizes where the top-k/top-p acceptance and the
statistics finish change how they read them:

- requests of at most 8 rows (gamma <= 7) have the first 64 entries of
  every row's list copied into LDS during the decision; gamma = 8 does not;
- a list of up to 64 entries is drawn from that copy, up to 256 from one
  read, longer ones in streamed steps of 256;
- the statistics finish loads the first 256 entries of p's (and q's) list
  with the row info and reads the rest afterwards;
- a kept set too long for a list is drawn by all four waves, which stay
  only in that case.

fp32 logits (no ties) keep exactly top_k tokens; every request is compared
with the oracle: sampling, lenient sampling and the statistics, with a
dense q and with q formed from the draft's logits."""

import pytest
import torch

from parity import compare_sample, compare_stats
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("gamma", [7, 8])
@pytest.mark.parametrize("top_k", [63, 64, 65, 255, 256, 257])
def test_list_sizes(gamma, top_k):
    w = generate("c2", DEV, B=6, gamma=gamma, V=4099, top_k=top_k, top_p=1.0, temperature=0.9,
                 seed=91000 + 10 * gamma + top_k)
    label = f"list sizes gamma={gamma} top_k={top_k}"
    compare_sample(w, label=label)
    compare_sample(w, label=label + " draft logits", draft_logits=True)
    compare_sample(w, label=label + " lenient 0.6", lenience=0.6)
    compare_stats(w, label=label)
    compare_stats(w, label=label + " draft logits", draft_logits=True)


@pytest.mark.parametrize("top_p", [0.5, 0.9])
def test_list_sizes_top_p_bf16(top_p):
    """bf16 rows under top-p (ties at the cut decided as the oracle does)."""
    w = generate("c3", DEV, B=5, gamma=6, V=6007, top_k=0, top_p=top_p, seed=92000 + int(top_p * 10))
    label = f"list sizes bf16 top_p={top_p}"
    compare_sample(w, label=label)
    compare_stats(w, label=label)
    compare_stats(w, label=label + " draft logits", draft_logits=True)


@pytest.mark.parametrize("gamma", [7, 9])
def test_oversized_kept_sets(gamma):
    """Flat-ish rows (T = 50, top-p 0.9) whose kept sets are too long for a
    list: the acceptance's four waves draw them from the whole row, with the
    list copy made during the decision (gamma = 7) and without it (gamma = 9)."""
    w = generate("c5", DEV, B=3, gamma=gamma, V=30000, temperature=50.0, top_p=0.9, seed=93000 + gamma)
    label = f"oversized kept sets gamma={gamma}"
    compare_sample(w, label=label)
    compare_sample(w, label=label + " draft logits", draft_logits=True)
