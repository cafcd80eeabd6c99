"""Statistics where p and q nearly agree: every term (p - q)_+ is tiny and
its sign is decided at the last bits of double precision, so a sign taken
from float approximations of p and q would move Z by as much as Z itself.

- q equal to the oracle's p rounded to float32: Z and Z' are sums of the
  rounding residues (about 1e-8 of the mass), on untruncated rows (the
  streamed statistics), top-k and top-p rows (the kept lists);
- q formed from draft logits equal to the target's: p = q term by term,
  on both sides, so Z = Z' = 0 and alpha = 1 up to the rounding of sum p;
- sharp rows (T = 0.2) in a large batch of short rows, where a Z of a few
  1e-12 holds only the double precision floor;
- the c2 and c3 workloads' full batches, every position.
"""

import numpy as np
import pytest
import torch

import oracle
import speculative_sampling_verification_sample_amd as sv
from parity import compare_stats, widen
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _q_from_oracle_p(w):
    """q[b, j] = the oracle's processed p of target row j, rounded to float32."""
    c = w.cfg
    lg = widen(w.logits)
    G = w.ids.shape[1]
    q = np.zeros((lg.shape[0], G, lg.shape[2]), np.float32)
    for b in range(lg.shape[0]):
        for j in range(G):
            q[b, j] = oracle.process_row(lg[b, j], c.temperature, c.top_k, c.top_p).p.astype(np.float32)
    return torch.from_numpy(q).to(w.logits.device).contiguous()


@pytest.mark.parametrize("shape,kw", [
    ("c2", dict(B=6, gamma=4, V=4099, seed=81001)),
    ("c2", dict(B=4, gamma=3, V=32000, seed=81002, temperature=0.3)),
    ("c3", dict(B=5, gamma=3, V=6001, seed=81003, top_k=0)),
    ("c3", dict(B=5, gamma=3, V=6001, seed=81004)),               # top-k 50
    ("c5", dict(B=4, gamma=3, V=9000, seed=81005)),               # top-p 0.95
    ("c5", dict(B=3, gamma=2, V=20000, seed=81006, top_p=1.0, temperature=2.0)),
])
def test_q_equal_to_p_rounded(shape, kw):
    w = generate(shape, DEV, **kw)
    w.q = _q_from_oracle_p(w)
    compare_stats(w, label=f"q = fl32(p) {shape} {kw}")


@pytest.mark.parametrize("shape,kw", [
    ("c2", dict(B=4, gamma=3, V=5003, seed=82001)),
    ("c3", dict(B=4, gamma=3, V=5003, seed=82002)),                # top-k 50
    ("c3", dict(B=4, gamma=3, V=5003, seed=82003, top_k=0)),
    ("c5", dict(B=3, gamma=3, V=12000, seed=82004)),               # top-p 0.95
])
def test_draft_logits_equal_to_target(shape, kw):
    w = generate(shape, DEV, **kw)
    G = w.ids.shape[1]
    w.draft_logits = w.logits[:, :G].contiguous()
    label = f"draft logits = target {shape} {kw}"
    compare_stats(w, label=label, draft_logits=True)
    c = w.cfg
    al, zpq, zqp, acc = sv.accept_stats_draft_logits(w.logits, w.draft_logits, w.ids, c.temperature, c.top_k,
                                                     c.top_p)
    torch.cuda.synchronize()
    # p and q come from the same logits by the same arithmetic: every term
    # of Z and Z' is exactly 0, and a(d) = min(1, p(d) / p(d)) = 1 (0 where
    # the draft's token lies outside the kept set: p(d) = q(d) = 0)
    assert torch.all(zpq == 0).item(), label
    assert torch.all(zqp == 0).item(), label
    assert torch.all((acc == 1) | (acc == 0)).item(), label
    assert torch.all((al - 1).abs() <= 1e-6).item(), label


@pytest.mark.parametrize("draft_logits", [False, True])
def test_sharp_short_rows(draft_logits):
    """341 requests x 11 positions of 255 tokens at T = 0.2: many Z of
    1e-14 to 1e-9."""
    w = generate("c3", DEV, B=341, gamma=11, V=255, temperature=0.2, top_k=0, top_p=1.0, seed=200246)
    compare_stats(w, label=f"sharp short rows draft_logits={draft_logits}", draft_logits=draft_logits)


@pytest.mark.parametrize("shape,draft_logits", [("c2", False), ("c2", True), ("c3", False), ("c3", True)])
def test_full_size_every_request(shape, draft_logits):
    """The workloads' full batches, every position against the oracle (in
    a pool of host processes): untruncated rows (c2: the S64 pass, streamed
    sums, for p and for a q formed from the draft's logits) and top-k lists
    (c3)."""
    w = generate(shape, DEV)
    compare_stats(w, label=f"{shape} full stats draft_logits={draft_logits}", draft_logits=draft_logits, pool=True)
