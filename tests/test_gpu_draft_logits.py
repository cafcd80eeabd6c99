"""GPU parity of the draft-logits calls (q formed in the library from the
draft's logits) against the CPU oracle's draft-logits functions, with the
same bar as the q-input calls: exact tokens / lengths / flags outside the
boundary band, statistics within 1e-5 relative (no absolute term)."""

import numpy as np
import pytest
import torch

import oracle
import speculative_sampling_verification_sample_amd as sv
from parity import compare_sample, compare_stats, gpu_sample
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=8)),
    ("c3", dict(B=6)),
    ("c5", dict(B=4)),
    ("c2", dict(B=6, gamma=3, V=10007)),
    ("c3", dict(B=5, gamma=2, V=40003)),
    ("c5", dict(B=3, gamma=3, V=70001)),
])
def test_sample_small_and_ragged(name, kw):
    w = generate(name, DEV, **kw)
    compare_sample(w, label=f"dl {name} {kw}", draft_logits=True)


def test_toy():
    w = generate("toy", DEV, B=20000)
    compare_sample(w, label="dl toy 2e4", draft_logits=True)


@pytest.mark.parametrize("name,kw", [
    ("c5", dict(B=4)),
    ("c3", dict(B=4)),
    ("c2", dict(B=6)),                      # untruncated: both rows streamed
    ("c2", dict(B=4, gamma=3, V=4001)),
    ("c3", dict(B=3, gamma=2, V=30011)),
])
def test_stats(name, kw):
    compare_stats(generate(name, DEV, **kw), label=f"dl stats {name} {kw}", draft_logits=True)


@pytest.mark.parametrize("gamma", [0, 1, 8])
def test_gamma_values(gamma):
    compare_sample(generate("c3", DEV, B=4, gamma=gamma, V=5000), label=f"dl gamma={gamma}", draft_logits=True)
    compare_sample(generate("c2", DEV, B=4, gamma=gamma, V=3000), label=f"dl c2 gamma={gamma}", draft_logits=True)


def test_long_gamma():
    """gamma + 1 > 64: the acceptance and the chunked draw run as separate launches."""
    compare_sample(generate("c2", DEV, B=3, gamma=70, V=600), label="dl gamma=70", draft_logits=True)


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_draft_rows_without_q(name):
    """NaN, +Inf and all -Inf draft rows; an invalid id on such a row; the
    statistics of those positions are NaN, the others are unaffected."""
    w = generate(name, DEV, B=6, gamma=3, V=9000)
    dz = w.draft_logits.clone()
    dz[0, 0, 17] = float("nan")
    dz[1, 2, :] = float("nan")
    dz[2, 1, 4000] = float("inf")
    dz[3, 0, :] = float("-inf")
    dz[4, 1, 5] = float("nan")
    ids = w.ids.clone()
    ids[4, 1] = 10 ** 6  # invalid id on the row without q
    w.draft_logits, w.ids = dz.contiguous(), ids.contiguous()
    o, _ = compare_sample(w, label=f"dl no-q {name}", draft_logits=True)
    for b in range(4):
        assert o["flags"][b] == oracle.FLAG_NONFINITE, (b, o["flags"][b])
    compare_stats(w, label=f"dl stats no-q {name}", draft_logits=True)


def test_ids_outside_the_drafts_kept_set():
    """A draft id the draft's own top-k excludes has q(d) = 0."""
    w = generate("c3", DEV, B=8, gamma=3, V=6000)
    dz = w.draft_logits.float()
    low = torch.argmin(dz, dim=-1).to(torch.int32)  # never in the draft's top-50
    ids = w.ids.clone()
    ids[::2, 0] = low[::2, 0]
    ids[1::2, 1] = low[1::2, 1]
    w.ids = ids.contiguous()
    o, _ = compare_sample(w, label="dl q(d)=0", draft_logits=True)
    assert (o["flags"] & oracle.FLAG_Q_ZERO).any()
    compare_stats(w, label="dl stats q(d)=0", draft_logits=True)


def test_flat_draft_rows():
    """Draft rows of one value: every token ties at the top-k cut, the draft
    rows take the exact path and q is uniform over the vocabulary."""
    w = generate("c3", DEV, B=3, gamma=2, V=5000)
    w.draft_logits = torch.zeros_like(w.draft_logits)
    compare_sample(w, label="dl flat draft", draft_logits=True)
    compare_stats(w, label="dl stats flat draft", draft_logits=True)


def test_fp32_draft_with_bf16_target():
    w = generate("c5", DEV, B=4, V=40000)
    w.draft_logits = w.draft_logits.float().contiguous()
    compare_sample(w, label="dl f32 draft", draft_logits=True)
    compare_stats(w, label="dl stats f32 draft", draft_logits=True)


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size(name):
    w = generate(name, DEV)
    gpu = gpu_sample(w, draft_logits=True)
    compare_sample(w, label=f"dl {name} full", gpu=gpu, draft_logits=True, pool=True)
    tok, nacc, fl = gpu
    pos = np.arange(w.cfg.gamma + 1)[None, :]
    assert ((tok >= 0) == (pos <= nacc[:, None])).all()
    assert (tok < w.cfg.V).all()


def test_full_size_stats():
    w = generate("c5", DEV)
    compare_stats(w, label="dl c5 full stats", draft_logits=True, pool=True)


def test_graph_replay_matches_eager():
    """The draft-logits call captured in a graph and replayed, with eager work
    and synchronisations between replays, gives the eager outputs every time."""
    w = generate("c5", DEV, B=4)
    c = w.cfg
    ws = torch.empty(sv.draft_logits_workspace_size(c.B, c.gamma, c.V, w.logits.dtype, w.draft_logits.dtype,
                                                    c.temperature, c.top_k, c.top_p), dtype=torch.uint8, device=DEV)
    outs = (torch.empty((c.B, c.gamma + 1), dtype=torch.int32, device=DEV),
            torch.empty((c.B,), dtype=torch.int32, device=DEV),
            torch.empty((c.B,), dtype=torch.int32, device=DEV))

    def call():
        sv.verify_sample_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample, c.temperature,
                                      c.top_k, c.top_p, workspace=ws, out=outs)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
