"""The pooled oracle (every request of a batch over several processes)
gives exactly what the single-process oracle gives."""

import numpy as np
import torch

import oracle
from oracle import pool as oracle_pool
from workloads import generate


def _host(t):
    t = t.contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _wide(t):
    return oracle_pool._wide(_host(t))


def test_pool_matches_single_process():
    w = generate("c3", "cpu", B=7, gamma=3, V=3001)
    c = w.cfg
    prm = dict(T=c.temperature, top_k=c.top_k, top_p=c.top_p)
    arrays = dict(logits=_host(w.logits), q=w.q.numpy(), ids=w.ids.numpy(), u_accept=w.u_accept.numpy(),
                  u_resample=w.u_resample.numpy())
    got = oracle_pool.run("sample", arrays, prm, c.B, workers=2)
    ref = oracle.verify_sample(_wide(w.logits), w.q.numpy(), w.ids.numpy(), w.u_accept.numpy(),
                               w.u_resample.numpy(), c.temperature, c.top_k, c.top_p)
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k])
    st = oracle_pool.run("stats", dict(logits=arrays["logits"], q=arrays["q"], ids=arrays["ids"]), prm, c.B,
                         workers=3)
    st_ref = oracle.accept_stats(_wide(w.logits), w.q.numpy(), w.ids.numpy(), c.temperature, c.top_k, c.top_p,
                                 with_boundary=True)
    for a, b in zip(st, st_ref):
        np.testing.assert_array_equal(a, b)


def test_pool_greedy_bf16():
    w = generate("c4", "cpu", B=5, gamma=2, V=999)
    got = oracle_pool.run("greedy", dict(logits=_host(w.logits), ids=w.ids.numpy()), {}, 5, workers=2)
    ref = oracle.verify_greedy(_wide(w.logits), w.ids.numpy())
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k])
