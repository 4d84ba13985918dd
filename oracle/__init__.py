"""Float64 CPU oracle for query-dependent sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, helpers, tables or constants) and imports
nothing from it.

Every function computes the plain definition of one step, in numpy float64,
one row at a time, and cites the page and section it follows.  Where the pages
leave a step open, the docstring states the reading taken.

Parity status of each function (what pins it, from the tests in
``tests/test_oracle_pins.py``):

* ``round_to_bf16``      pinned: bit-equal to torch's fp32->bf16 rounding on
                         fp32-representable inputs, hand-made halfway cases.
* ``indexer_keys``, ``collapse_query``, ``token_scores``
                         pinned: brute-force loops on tiny inputs, group
                         semantics (a needle seen only by one group), linearity.
* ``page_stats``         pinned: closed forms (constant page, +/- pairs,
                         arithmetic progression).
* ``page_scores``        pinned: constant page equals the exact mean of
                         exp-scores; O(sigma^4) decay on axis-pair pages;
                         diagonal-vs-full covariance gap; Gaussian closed form.
* ``select_topp``/``select_topk``
                         pinned: hand-made dyadic distributions
                         (tests/golden/topp_dyadic.txt), brute-force subset
                         enumeration, p=1 / k>=n give everything.
* ``with_sink_window``, ``expand_pages``
                         pinned: hand-made cases.
* ``attend``             pinned: torch scaled_dot_product_attention in float64,
                         single-key support, key/value permutation invariance.
* ``prefill_*``          pinned: early blocks equal dense causal attention
                         (torch SDPA, is_causal), segment permutation
                         invariance, query covariance.
* ``rla_*``              pinned: single-token state is the outer product;
                         zero keys give the plain mean of the unselected
                         values; one unselected token returns its value; a
                         full support leaves nothing; the subtraction form
                         equals the direct sum; linear in V, invariant under
                         a joint key/value permutation.
* ``prefill_query_*``    pinned: a support of every causal key gives dense
                         causal attention (torch SDPA, is_causal); with one
                         head per group, or identical per-head channels, the
                         mean-of-probabilities ranking equals the logits
                         ranking; the probability mean is a distribution and
                         its top-k holds the largest mass (brute force); the
                         own token is always kept.
* ``prefill_oracle_*``   pinned: the block support is the top-k of the mean
                         of the block rows' causal torch SDPA weights over
                         earlier keys; the per-query support holds the
                         largest mass of all k-subsets (brute force) and the
                         own token; k covering every candidate gives dense
                         causal attention.
* ``pbs_*``              pinned: importance is a distribution and equals the
                         head/query mean of causal torch SDPA weights; the
                         permutation maps every segment onto itself, sorts by
                         importance and moves a planted key to its segment's
                         front; block scores are linear in the pooled means;
                         with every block selected the attention is dense
                         causal SDPA; on scattered heavy hitters the permuted
                         top block covers more attention mass than any
                         natural block (the method's purpose).
* ``head_mean_attention``, ``oracle_support``, ``support_coverage``,
  ``support_overlap``
                         pinned: the head-averaged distribution equals the
                         head mean of torch scaled_dot_product_attention
                         weights (float64, one-hot values); two-key logistic
                         closed form; equal keys give the uniform
                         distribution; the top-k oracle support has the
                         largest coverage of all k-subsets and the top-p one
                         the smallest size reaching p (brute force); hand-made
                         overlaps.

Parity unpinned (our readings, fixed only by our own written definitions, no
worked example on the pages): the indexer scale ``s_idx``, the mean over a
group's heads (and over a query block) of the projected query, the union of
the always-kept sink/window tokens after selection, the log-domain mean over a
group's heads of the page score, the partial-page term log(n/page), and the
residual linear attention's feature map on the raw (unscaled) query/key rows
with the unselected set taken as the complement of the final support; for the
segment permutation, the importance as the mean attention probability of the
last query block, the query's own segment kept in natural order, and top-k
block selection.
"""

from .sparse_attention import *  # noqa: F401,F403
from .sparse_attention import __all__  # noqa: F401
