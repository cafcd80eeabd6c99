"""The Python binding checks every tensor it hands to the C ABI: inputs,
caller-supplied outputs and the workspace (device, dtype, shape, layout,
size), and raises before any launch."""

import pytest
import torch

import speculative_sampling_verification_sample_amd as sv
from workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _args(w):
    c = w.cfg
    return (w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p)


def test_rejects_bad_outputs_and_workspace():
    w = generate("c3", DEV, B=3, gamma=2, V=5000)
    B, G1 = w.cfg.B, w.cfg.gamma + 1
    ok = (torch.empty((B, G1), dtype=torch.int32, device=DEV), torch.empty((B,), dtype=torch.int32, device=DEV),
          torch.empty((B,), dtype=torch.int32, device=DEV))
    bad_outs = [
        (torch.empty((B - 1, G1), dtype=torch.int32, device=DEV), ok[1], ok[2]),   # too few requests
        (ok[0].to(torch.int64), ok[1], ok[2]),                                      # wrong dtype
        (ok[0], ok[1].cpu(), ok[2]),                                                 # host memory
        (torch.empty((G1, B), dtype=torch.int32, device=DEV).t(), ok[1], ok[2]),    # not contiguous
    ]
    for out in bad_outs:
        with pytest.raises(ValueError):
            sv.verify_sample(*_args(w), out=out)
    need = sv.workspace_size(B, G1 - 1, w.cfg.V, w.logits.dtype, w.cfg.temperature, w.cfg.top_k, w.cfg.top_p)
    for ws in (torch.empty(need, dtype=torch.uint8),                      # host memory
               torch.empty(need - 1, dtype=torch.uint8, device=DEV),      # too small
               torch.empty(need // 4 + 1, dtype=torch.float32, device=DEV),  # not bytes
               torch.empty(need + 16, dtype=torch.uint8, device=DEV)[1:]):  # misaligned
        with pytest.raises(ValueError):
            sv.verify_sample(*_args(w), workspace=ws)
    st = tuple(torch.empty((B, G1 - 1), dtype=torch.float32, device=DEV) for _ in range(4))
    with pytest.raises(ValueError):
        sv.verify_sample_stats(*_args(w), stats_out=(st[0], st[1], st[2][:1], st[3]))
    with pytest.raises(ValueError):
        sv.accept_stats(*((w.logits, w.q, w.ids) + _args(w)[5:]), out=(st[0].double(), st[1], st[2], st[3]))
    # the good ones run
    sv.verify_sample(*_args(w), out=ok, workspace=torch.empty(need, dtype=torch.uint8, device=DEV))
    sv.verify_sample_stats(*_args(w), stats_out=(st[0], st[1], None, st[3]))
    torch.cuda.synchronize()


def test_rejects_bad_inputs():
    w = generate("c2", DEV, B=2, gamma=2, V=1000)
    a = list(_args(w))
    for i, bad in ((1, w.q[:, :1]), (2, w.ids.long()), (3, w.u_accept.cpu()), (4, w.u_resample.double())):
        b = list(a)
        b[i] = bad
        with pytest.raises(ValueError):
            sv.verify_sample(*b)
    with pytest.raises(ValueError):
        sv.verify_sample(w.logits.half(), *a[1:])
