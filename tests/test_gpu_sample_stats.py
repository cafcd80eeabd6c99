"""The combined sampling + statistics calls: their sampling outputs are the
sampling call's, bit for bit, and their statistics match the oracle to the
statistics bar (1e-5 relative, no absolute term)."""

import numpy as np
import pytest
import torch

import speculative_sampling_verification_sample_amd as sv
from parity import compare_sample, compare_stats, gpu_sample
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _fused(w, draft_logits=False):
    c = w.cfg
    if draft_logits:
        out = sv.verify_sample_stats_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                                  c.temperature, c.top_k, c.top_p)
    else:
        out = sv.verify_sample_stats(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k,
                                     c.top_p)
    torch.cuda.synchronize()
    return out


def _check(w, label, draft_logits=False, pool=False):
    tok, nacc, fl, al, zpq, zqp, acc = _fused(w, draft_logits)
    sep = gpu_sample(w, draft_logits=draft_logits)
    for x, y in zip((tok, nacc, fl), sep):
        np.testing.assert_array_equal(x.cpu().numpy().astype(y.dtype), y)
    compare_sample(w, label=label, gpu=sep, draft_logits=draft_logits, pool=pool)
    compare_stats(w, label=label, draft_logits=draft_logits, gpu=(al, zpq, zqp, acc), pool=pool)


@pytest.mark.parametrize("dl", [False, True])
@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=6)),
    ("c3", dict(B=5)),
    ("c5", dict(B=4)),
    ("c2", dict(B=4, gamma=3, V=10007)),
    ("c3", dict(B=3, gamma=2, V=40003)),
    ("c5", dict(B=3, gamma=3, V=70001)),
])
def test_small(name, kw, dl):
    _check(generate(name, DEV, **kw), f"sample+stats {name} {kw} dl={dl}", draft_logits=dl)


def test_toy():
    _check(generate("toy", DEV, B=3000), "sample+stats toy")


@pytest.mark.parametrize("gamma", [0, 1, 70])
def test_gamma_values(gamma):
    V = 600 if gamma == 70 else 5000
    for name in ("c2", "c3"):
        w = generate(name, DEV, B=3, gamma=gamma, V=V)
        tok, nacc, fl, *st = _fused(w)
        sep = gpu_sample(w)
        for x, y in zip((tok, nacc, fl), sep):
            np.testing.assert_array_equal(x.cpu().numpy().astype(y.dtype), y)
        if gamma > 0:
            compare_stats(w, label=f"sample+stats {name} gamma={gamma}", gpu=st)


@pytest.mark.parametrize("dl", [False, True])
def test_full_size_c5(dl):
    """The headline workload (the bench's call), every request."""
    w = generate("c5", DEV)
    _check(w, f"sample+stats c5 full dl={dl}", draft_logits=dl, pool=True)


def test_graph_replay_matches_eager():
    w = generate("c5", DEV, B=4, V=50000)
    c = w.cfg
    ws = torch.empty(sv.workspace_size(c.B, c.gamma, c.V, w.logits.dtype, c.temperature, c.top_k, c.top_p),
                     dtype=torch.uint8, device=DEV)
    outs = (torch.empty((c.B, c.gamma + 1), dtype=torch.int32, device=DEV),
            torch.empty((c.B,), dtype=torch.int32, device=DEV),
            torch.empty((c.B,), dtype=torch.int32, device=DEV))
    souts = tuple(torch.empty((c.B, c.gamma), dtype=torch.float32, device=DEV) for _ in range(4))

    def call():
        sv.verify_sample_stats(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p,
                               workspace=ws, out=outs, stats_out=souts)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + souts]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs + souts:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs + souts, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dl", [False, True])
def test_calls_on_several_streams(dl):
    """The dense-q sums (and, with q from the draft's logits under top-p,
    the draft rows' passes) run on a side stream of the caller's stream:
    calls enqueued on three caller streams at once, each with its own
    workspace and outputs, give the default stream's results bit for bit."""
    w = generate("c5", DEV, B=4, V=50000)
    c = w.cfg

    def call():
        if dl:
            return sv.verify_sample_stats_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                                       c.temperature, c.top_k, c.top_p)
        return sv.verify_sample_stats(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k,
                                      c.top_p)

    ref = [t.clone() for t in call()]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    res = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            res.append(call())
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for r in res:
        for a, b in zip(r, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dl", [False, True])
@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=4)),
    ("c3", dict(B=4)),
    ("c5", dict(B=4)),
    ("c5", dict(B=3, gamma=3, V=70001)),
])
def test_without_z_qp(name, kw, dl):
    """Leaving Z' out (a null output) changes no other output, bit for bit,
    in the combined call and in the statistics-only call."""
    w = generate(name, DEV, **kw)
    c = w.cfg
    full = _fused(w, dl)
    if dl:
        part = sv.verify_sample_stats_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                                   c.temperature, c.top_k, c.top_p, z_qp=False)
        st_full = sv.accept_stats_draft_logits(w.logits, w.draft_logits, w.ids, c.temperature, c.top_k, c.top_p)
        st_part = sv.accept_stats_draft_logits(w.logits, w.draft_logits, w.ids, c.temperature, c.top_k, c.top_p,
                                               z_qp=False)
    else:
        part = sv.verify_sample_stats(w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k,
                                      c.top_p, z_qp=False)
        st_full = sv.accept_stats(w.logits, w.q, w.ids, c.temperature, c.top_k, c.top_p)
        st_part = sv.accept_stats(w.logits, w.q, w.ids, c.temperature, c.top_k, c.top_p, z_qp=False)
    torch.cuda.synchronize()
    assert part[5] is None and st_part[2] is None
    for k in (0, 1, 2, 3, 4, 6):
        np.testing.assert_array_equal(part[k].cpu().numpy(), full[k].cpu().numpy(), err_msg=f"output {k}")
    for k in (0, 1, 3):
        np.testing.assert_array_equal(st_part[k].cpu().numpy(), st_full[k].cpu().numpy(), err_msg=f"stats {k}")
