"""Seeded synthetic inputs for the speculative-sampling verify step.

This module is the only code the CPU oracle and the HIP library's callers
share.  It holds none of the verify step's arithmetic (acceptance, residual,
draws, statistics): it draws random numbers and builds what a *caller* of
the verify step hands over.  One piece of that is the draft side's own
decoding rules: q is formed from the draft logits by this module's own
softmax with temperature, top-k and top-p (written apart from the oracle's
processing of p), and both sides then take that q as an input --

* target logits for gamma+1 positions,
* the draft's own sampling distribution q for gamma positions, built by the
  draft-side recipe of each workload (the verify step takes q as given and
  never recomputes it),
* the draft token ids, sampled from q,
* float32 uniforms (integer * 2^-24, so exact and never 1.0).

Workloads (sizes B x (gamma+1) x V):

* ``toy``: 1e6 rounds x 5 x 5, float32.  Target rows ~ Dirichlet(1), logits =
  ln p; draft q = normalise(0.6 p + 0.4 / V); used for the chi-square law.
  ``generate("toy", name="toy_const")`` copies position 0 to every position
  (the same acceptance probability at every position).
* ``c2``: 64 x 5 x 32000, float32 logits ~ N(0, 2^2); draft logits = target +
  N(0, 0.5^2); T = 1, no truncation.
* ``c3``: 256 x 6 x 128256, bfloat16 logits ~ N(0, 3^2) with 1% of ids per
  row boosted by +6; draft = target + N(0, 1); T = 0.8, top-k = 50 on both.
* ``c4``: greedy, 512 x 9 x 152064, bfloat16 logits ~ N(0, 2.5^2); draft ids =
  argmax(target + N(0, 0.3^2)).
* ``c5``: 1024 x 5 x 256000, bfloat16 Zipf-shaped logits
  (-1.1 ln(rank) + N(0, 0.5^2), rank a random permutation per row); draft =
  target + N(0, 0.8^2); T = 0.7, top-p = 0.95 on both; also the acceptance
  statistics.

Ragged batches (a draft length per request): ``pack_ragged(w, gammas)``
keeps the first gammas[b] drafts of each request of a uniform workload and
packs them without padding; ``ragged_gammas`` draws gammas[b] uniformly from
{0, .., gamma} with its own seed.

Random streams: ``numpy.random.SeedSequence(seed).spawn(4)`` seeds four torch
generators on the chosen device: [0] target logits, [1] draft noise,
[2] draft-id sampling, [3] uniforms.  CPU and GPU generators give different
numbers for one seed; a test uses one device for both sides.
"""

from .configs import CONFIGS, Config  # noqa: F401
from .generate import RaggedWorkload, Workload, generate, pack_ragged, ragged_gammas  # noqa: F401
