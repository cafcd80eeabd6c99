"""The allocation-free entry point (spec_verify_sample_noalloc, for callers
that cannot allocate device memory) gives exactly what spec_verify_sample
gives, on two calls in a row, the second smaller than the first, so its
static scratch carries the first call's contents into the second."""

import numpy as np
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


def _both(w):
    c = w.cfg
    args = (w.logits, w.q, w.ids, w.u_accept, w.u_resample, c.temperature, c.top_k, c.top_p)
    ref = sv.verify_sample(*args)
    out = (torch.full_like(ref[0], -7), torch.full_like(ref[1], -7), torch.full_like(ref[2], -7))
    got = sv.verify_sample_noalloc(*args, out=out)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    return ref


@pytest.mark.parametrize("big,small", [
    (("c5", dict(B=96)), ("c5", dict(B=5, V=70001))),     # top-p, kept lists
    (("c3", dict(B=128)), ("c3", dict(B=3, gamma=2))),    # top-k
    (("c2", dict(B=64)), ("c2", dict(B=4, V=10007))),     # untruncated full-row draws
])
def test_noalloc_matches_the_workspace_call(big, small):
    r1 = _both(generate(big[0], DEV, **big[1]))
    r2 = _both(generate(small[0], DEV, **small[1]))
    assert (r1[1].cpu().numpy() >= 0).all() and (r2[1].cpu().numpy() >= 0).all()


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    c5 = dict(temperature=0.7, top_k=0, top_p=0.95)
    assert sv.workspace_size(1024, 4, 256000, torch.bfloat16, **c5) > 64 * 1024 * 1024
    w = generate("c5", DEV, B=1024, V=4000)  # a small vocabulary keeps the inputs small
    # the refusal is decided from B, gamma and V alone: ask for the full vocabulary through the C ABI
    lib = sv.load_library()
    from speculative_sampling_verification_sample_amd._lib import SamplingParamsC
    code = lib.spec_verify_sample_noalloc(
        w.logits.data_ptr(), 1, w.q.data_ptr(), w.ids.data_ptr(), w.u_accept.data_ptr(), w.u_resample.data_ptr(),
        1024, 4, 256000, SamplingParamsC(0.7, 0, 0.95), w.ids.data_ptr(), w.ids.data_ptr(), w.ids.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert code == 2  # SV_ERR_UNSUPPORTED: nothing launched
