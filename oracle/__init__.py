"""CPU oracle for the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables); the only module both sides
use is the seeded input generator in ``workloads/``, which holds none of the
verify step's arithmetic: it builds what a caller hands over, among it the
draft's q, which it forms with its own softmax and truncation code (the
draft side's decoding rules); both sides take that q as an input.

It is a plain, slow, float64 NumPy implementation, one request and one row at
a time, written from the pages listed below.  Citations name the page and the
section / equation / table on it.

Pages (all on speculative decoding / speculative sampling):

* [WR]  wrblog.cn, "推测解码：草稿模型、接受率、正确性与加速边界"
        (Speculative decoding: draft model, acceptance rate, correctness and
        speed-up limits) -- numbered sections 1-19.
* [AQ]  aiqz.cc, "投机解码：草稿小模型 + 大模型并行验证的无损加速"
        (lossless acceleration with a small draft model and parallel
        verification) -- sections "并行验证机制", "Python 演示".
* [RL]  rainlin-net.pages.dev, "投机解码" notes -- §1 执行流程 (round),
        §2 分布等价性 (distribution equivalence), §3 加速条件 (speed-up).
* [BS]  baisen.site, "投机采样 / 投机解码（Speculative Decoding）" --
        sections 一 .. 十 (四 = accept/reject rule, 五 = proof,
        六 = greedy as a special case, 七 = expected output).
* [MN]  magicnetworld.com, "投机解码到底能加速多少：把接受率、草稿成本与墙钟收益算清楚"
        -- sections 一 .. 十 (三 = acceptance and residual, 四 = truncated
        geometric law and the E[T] table).

Parity status of every function is stated in its docstring; all functions
here are pinned by ``tests/test_oracle_*.py`` (worked examples, closed forms,
brute force on tiny inputs, chi-square of the output law).  One step is
"parity unpinned" by the pages: the replacement rule of the lenient
acceptance (``beta < 1``), which the pages do not give.  It is a reading
((p - beta q)_+), pinned only to the pages' 1/beta bound and to its own
closed-form law by exact enumeration.
"""

from .verify import (  # noqa: F401
    FLAG_BAD_ID,
    FLAG_Q_ZERO,
    FLAG_Z_DEGENERATE,
    FLAG_NONFINITE,
    FLAG_EOS,
    FLAG_BAD_SPAN,
    BOUNDARY_EPS,
    ProcessedRow,
    RequestResult,
    bf16_bits_to_f64,
    process_row,
    truncation_set,
    inverse_cdf,
    residual_weights,
    verify_request,
    verify_from_processed,
    verify_sample,
    greedy_request,
    verify_greedy,
    stats_request,
    accept_stats,
    draft_q_rows,
    verify_request_draft_logits,
    verify_sample_draft_logits,
    stats_request_draft_logits,
    accept_stats_draft_logits,
    ragged_span,
    verify_sample_ragged,
    verify_greedy_ragged,
    verify_sample_ragged_draft_logits,
)
