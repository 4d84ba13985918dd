"""Plain float64 definitions of every step of query-dependent sparse attention.

Test infrastructure only (see the package docstring).  All arrays are numpy;
inputs are converted to float64 exactly (bf16 and fp32 values are exactly
representable in float64).  Loops stay simple so each step can be read
against the pages:

* "Full Attention Strikes Back" (RTPurbo) -- method section 1 (local heads keep
  an attention sink and a sliding window), section 2 (a low-rank r=16 projector
  applied to queries and keys before RoPE scores every cached token), section 3
  (dynamic top-p: take tokens until the accumulated attention mass of the
  low-rank scores reaches p; static top-k as the alternative).
* "Oracle-Guided Sparse Prefill for Full/GQA layers" -- section 2.1 (top-k
  support, attention recomputed with the original q, k, v restricted to the
  support; support shared by a block of b_sel = 64 consecutive queries) and
  section 2.2 (one head-collapsed scoring channel shared by the heads; the
  budget k is a runtime knob).
* "SPLA: Block Sparse Plus Linear Attention" -- section 2.1 (block score from a
  second-order Taylor expansion around the block mean, exp(q.kbar) times
  (1 + q^T Cov(k) q / 2), with the covariance replaced by its diagonal);
  section 2.2 (residual linear attention over the blocks left out of the
  support, with the parameter-free exponential feature map, computed by
  subtracting the selected blocks' linear-attention terms from a global
  state).
* "Sparser Block-Sparse Attention via Token Permutation" (PBS-Attn) -- section 1
  (attention output is invariant to a joint permutation of key/value pairs and
  covariant with a permutation of the queries); sections 2 to 4 (keys
  reordered inside fixed-size segments by a global importance taken from the
  last query block, block selection by mean pooling on the reordered keys).

Group convention (grouped-query attention): with G = H_q / H_kv, query head h
belongs to key/value group g = h // G.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "f64",
    "round_to_bf16",
    "indexer_keys",
    "collapse_query",
    "token_scores",
    "page_stats",
    "page_scores",
    "taylor_page_score",
    "candidate_order",
    "softmax_mass",
    "select_topp",
    "prefix_reaching",
    "select_topk",
    "with_sink_window",
    "expand_pages",
    "attend",
    "decode_row",
    "decode_row_pages",
    "prefill_block_rows",
    "prefill_block_query",
    "prefill_block_support",
    "prefill_block_attend",
    "prefill_query_scores",
    "prefill_query_support",
    "prefill_query_attend",
    "prefill_oracle_query_support",
    "prefill_oracle_block_support",
    "pbs_importance",
    "pbs_permutation",
    "pbs_block_keys",
    "pbs_block_scores",
    "pbs_block_support",
    "group_of_head",
    "heads_of_group",
    "rla_feature",
    "rla_state",
    "rla_unselected",
    "rla_by_subtraction",
    "head_mean_attention",
    "mass_scores",
    "oracle_support",
    "support_coverage",
    "support_overlap",
]


def f64(a) -> np.ndarray:
    """Exact conversion of an array (fp32 or bf16-valued fp32) to float64."""
    return np.asarray(a, dtype=np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the float32
    exponent range; its smallest subnormal step is 2**-133.  The value is
    returned as float64.  Used to model a bf16 store of a float64 result.
    """
    x = f64(x)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])  # |x| = m * 2**e with 0.5 <= m < 1
    step_exp = np.maximum(e - 8, -133)  # spacing of bf16 values near x
    q = np.rint(np.ldexp(x[nz], -step_exp))  # np.rint: half to even
    out[nz] = np.ldexp(q, step_exp)
    return out


def group_of_head(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    return h // (n_q_heads // n_kv_heads)


def heads_of_group(g: int, n_q_heads: int, n_kv_heads: int) -> list:
    G = n_q_heads // n_kv_heads
    return list(range(g * G, (g + 1) * G))


# ---------------------------------------------------------------------------
# Indexer (RTPurbo section 2; Oracle-Guided Sparse Prefill section 2.2)
# ---------------------------------------------------------------------------


def indexer_keys(k_pre, w_k) -> np.ndarray:
    """Low-rank indexer keys: row j is W_k^T k_j (k taken before RoPE).

    k_pre: [T, d], w_k: [d, r]  ->  [T, r]
    """
    return f64(k_pre) @ f64(w_k)


def collapse_query(q_heads, w_q_heads, s_idx: float) -> np.ndarray:
    """Head-collapsed indexer query of one group.

    Each head's pre-RoPE query is projected to rank r, q~_h = W_q[h]^T q_h,
    and the group keeps one scoring channel: the mean of q~_h over its heads,
    times the indexer scale s_idx.  Averaging the projected queries equals
    averaging the heads' low-rank logits (reading: the mean over the group's
    heads is how one shared channel serves them).

    q_heads: [G, d], w_q_heads: [G, d, r]  ->  [r]
    """
    q_heads, w_q_heads = f64(q_heads), f64(w_q_heads)
    G = q_heads.shape[0]
    acc = np.zeros(w_q_heads.shape[2])
    for h in range(G):
        acc += w_q_heads[h].T @ q_heads[h]
    return s_idx * acc / G


def token_scores(q_c, ktil) -> np.ndarray:
    """Indexer score of every cached token: x_j = q_c . K~_j.

    q_c: [r], ktil: [L, r]  ->  [L]
    """
    return f64(ktil) @ f64(q_c)


# ---------------------------------------------------------------------------
# Page statistics and the Taylor page score (SPLA section 2.1)
# ---------------------------------------------------------------------------


def page_stats(k, page_size: int = 64):
    """Per-page mean and diagonal (population) variance of the keys.

    k: [L, d] -> mean [P, d], var [P, d], n [P] with P = ceil(L / page_size);
    the last page may hold fewer than page_size tokens.  Variance divides by
    the number of tokens in the page (reading: the statistic of the block's
    own tokens, not an estimate of a wider population).
    """
    k = f64(k)
    L, d = k.shape
    P = (L + page_size - 1) // page_size
    mean = np.zeros((P, d))
    var = np.zeros((P, d))
    n = np.zeros(P, dtype=np.int64)
    for p in range(P):
        rows = k[p * page_size : min(L, (p + 1) * page_size)]
        n[p] = rows.shape[0]
        mu = rows.sum(axis=0) / n[p]
        dev = rows - mu
        mean[p] = mu
        var[p] = (dev * dev).sum(axis=0) / n[p]
    return mean, var, n


def taylor_page_score(qp, mean_p, var_p) -> float:
    """The printed block score exp(q.kbar) * (1 + q^T diag(var) q / 2).

    qp is the already-scaled query (s_att * q).  Diagonal covariance as the
    page prescribes to avoid O(d^2) storage.
    """
    qp, mean_p, var_p = f64(qp), f64(mean_p), f64(var_p)
    return math.exp(float(qp @ mean_p)) * (1.0 + 0.5 * float((qp * qp) @ var_p))


def page_scores(q_heads, mean, var, n_valid, s_att: float, page_size: int = 64):
    """Group page score x_p used for page selection.

    For head h with scaled query q'_h = s_att * q_h the log of the Taylor
    block score is  l_{h,p} = q'_h . kbar_p + log(1 + 0.5 * sum_i q'_{h,i}^2 var_{p,i}),
    plus log(n_p / page_size) for a partial page, so that the score keeps
    estimating the block's total exp-mass.  The group's score is the mean of
    l_{h,p} over its heads (reading: the log-domain analogue of the
    head-collapsed channel).  Ranking by the log score equals ranking by the
    score itself and cannot overflow.

    q_heads: [G, d], mean/var: [P, d], n_valid: [P] -> [P]
    """
    q_heads, mean, var = f64(q_heads), f64(mean), f64(var)
    qp = s_att * q_heads                      # [G, d]
    first = qp @ mean.T                       # [G, P]  q'_h . kbar_p
    second = np.log1p(0.5 * ((qp * qp) @ var.T))  # [G, P]
    ell = first + second
    partial = np.log(np.asarray(n_valid, dtype=np.float64) / page_size)
    return ell.mean(axis=0) + partial


# ---------------------------------------------------------------------------
# Support selection (RTPurbo section 3; Oracle-Guided Sparse Prefill 2.1/2.2)
# ---------------------------------------------------------------------------


def candidate_order(x) -> np.ndarray:
    """Candidates ranked by score descending; equal scores by index ascending."""
    x = f64(x)
    idx = np.arange(x.shape[0])
    return np.lexsort((idx, -x))


def softmax_mass(x) -> np.ndarray:
    """Attention mass of each candidate under the indexer scores."""
    x = f64(x)
    w = np.exp(x - x.max())
    return w / w.sum()


def select_topp(x, p: float) -> np.ndarray:
    """Dynamic top-p support: the shortest prefix of the candidate order whose
    accumulated mass reaches p (cumulative >= p).  p >= 1 keeps every
    candidate, as does a prefix sum that never reaches p in floating point.
    Returns the selected indices in ascending order.
    """
    x = f64(x)
    n = x.shape[0]
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if not p > 0:
        raise ValueError("p must be in (0, 1]")
    if p >= 1.0:
        return np.arange(n)
    order = candidate_order(x)
    take = prefix_reaching(softmax_mass(x)[order], p)
    return np.sort(order[:take])


def prefix_reaching(mass_in_order, p: float) -> int:
    """Length of the shortest prefix of the ordered masses whose running sum
    is >= p (all of them if the sum never gets there)."""
    n = len(mass_in_order)
    cum = 0.0
    for i in range(n):
        cum += float(mass_in_order[i])
        if cum >= p:
            return i + 1
    return n


def select_topk(x, k: int) -> np.ndarray:
    """Static top-k support: the first min(k, n) candidates of the order,
    returned in ascending index order."""
    if k < 1:
        raise ValueError("k must be >= 1")
    order = candidate_order(x)
    return np.sort(order[: min(k, order.shape[0])])


def with_sink_window(S, L: int, n_sink: int, n_window: int) -> np.ndarray:
    """Union of a support with the always-kept attention-sink tokens [0, n_sink)
    and the sliding window [L - n_window, L) (reading: the local tokens are
    added after selection and do not take part in the mass count)."""
    keep = set(int(j) for j in S)
    keep.update(range(0, min(n_sink, L)))
    keep.update(range(max(0, L - n_window), L))
    return np.array(sorted(keep), dtype=np.int64)


def expand_pages(pages, L: int, page_size: int = 64) -> np.ndarray:
    """Token indices of the selected pages (the last page may be partial)."""
    out = []
    for p in sorted(int(q) for q in pages):
        out.extend(range(p * page_size, min(L, (p + 1) * page_size)))
    return np.array(out, dtype=np.int64)


# ---------------------------------------------------------------------------
# Exact attention over the support (Oracle-Guided Sparse Prefill 2.1)
# ---------------------------------------------------------------------------


def attend(q_heads, K, V, s_att: float):
    """Softmax attention of each query head over the given keys/values,
    renormalised over them (the support).

    q_heads: [G, d], K/V: [n, d]  ->  o [G, d], lse [G]
    lse_h = log sum_j exp(s_att * q_h . k_j).
    """
    q_heads, K, V = f64(q_heads), f64(K), f64(V)
    G = q_heads.shape[0]
    o = np.zeros((G, V.shape[1]))
    lse = np.zeros(G)
    for h in range(G):
        logits = s_att * (K @ q_heads[h])
        m = logits.max()
        w = np.exp(logits - m)
        l = w.sum()
        o[h] = (w @ V) / l
        lse[h] = m + math.log(l)
    return o, lse


# ---------------------------------------------------------------------------
# Attention-mass oracle support (Oracle-Guided Sparse Prefill 2.1)
# ---------------------------------------------------------------------------


def head_mean_attention(q_heads, K, s_att: float) -> np.ndarray:
    """Token importance of one query position for one key/value group: the
    dense attention distribution of each of the group's query heads over all
    keys, averaged over those heads.

    q_heads: [G, d], K: [n, d]  ->  P [n] (P >= 0, sum 1 when n > 0).
    """
    q_heads, K = f64(q_heads), f64(K)
    G, n = q_heads.shape[0], K.shape[0]
    P = np.zeros(n)
    if n == 0:
        return P
    for h in range(G):
        logits = s_att * (K @ q_heads[h])
        w = np.exp(logits - logits.max())
        P += w / w.sum()
    return P / G


def mass_scores(P) -> np.ndarray:
    """log P: as candidate scores, the selection rules above rank by P and
    their softmax mass is P itself, so they return the oracle support."""
    with np.errstate(divide="ignore"):
        return np.log(f64(P))


def oracle_support(P, *, k=None, p=None) -> np.ndarray:
    """Attention-mass oracle support: the k tokens of largest P (the page's
    top-k rule), or the shortest prefix in that order whose P sum reaches p.
    Equal P values are taken lower index first; ascending indices."""
    if (p is None) == (k is None):
        raise ValueError("give exactly one of p, k")
    x = mass_scores(P)
    return select_topk(x, k) if k is not None else select_topp(x, p)


def support_coverage(P, S) -> float:
    """Dense attention mass a support covers: sum of P over the support."""
    P = f64(P)
    total = 0.0
    for j in S:
        total += P[int(j)]
    return total


def support_overlap(S, S_ref) -> int:
    """Number of tokens two supports have in common."""
    return len(set(int(j) for j in S) & set(int(j) for j in S_ref))


def decode_row(q_heads, w_q_heads, ktil, K, V, *, s_idx, s_att, p=None, k=None,
               n_sink=0, n_window=0):
    """One decode step of one key/value group: indexer scores, top-p (or
    top-k) support, sink/window union, exact attention over the support."""
    L = K.shape[0]
    q_c = collapse_query(q_heads, w_q_heads, s_idx)
    x = token_scores(q_c, ktil)
    if (p is None) == (k is None):
        raise ValueError("give exactly one of p, k")
    S = select_topp(x, p) if p is not None else select_topk(x, k)
    S = with_sink_window(S, L, n_sink, n_window)
    o, lse = attend(q_heads, f64(K)[S], f64(V)[S], s_att)
    return {"q_c": q_c, "x": x, "S": S, "o": o, "lse": lse}


def decode_row_pages(q_heads, mean, var, n_valid, K, V, *, s_att, k_pages,
                     page_size=64):
    """Page-granular decode of one group: Taylor page scores, top-k pages,
    expansion to tokens, exact attention over those tokens."""
    L = K.shape[0]
    x = page_scores(q_heads, mean, var, n_valid, s_att, page_size)
    pages = select_topk(x, k_pages)
    S = expand_pages(pages, L, page_size)
    o, lse = attend(q_heads, f64(K)[S], f64(V)[S], s_att)
    return {"x": x, "pages": pages, "S": S, "o": o, "lse": lse}


# ---------------------------------------------------------------------------
# Causal prefill with a support shared by a block of b_sel queries
# (Oracle-Guided Sparse Prefill 2.1 granularity, 2.2 inference)
# ---------------------------------------------------------------------------


def prefill_block_rows(blk: int, b_sel: int, N: int) -> range:
    return range(blk * b_sel, min(N, (blk + 1) * b_sel))


def prefill_block_query(Q_blk, w_q_heads, s_idx: float) -> np.ndarray:
    """Indexer query shared by a query block and a group: the mean over the
    block's queries and the group's heads of W_q[h]^T q_{i,h}, times s_idx.

    Q_blk: [n_rows, G, d], w_q_heads: [G, d, r] -> [r]
    """
    Q_blk, w_q_heads = f64(Q_blk), f64(w_q_heads)
    n_rows, G, _ = Q_blk.shape
    acc = np.zeros(w_q_heads.shape[2])
    for i in range(n_rows):
        for h in range(G):
            acc += w_q_heads[h].T @ Q_blk[i, h]
    return s_idx * acc / (n_rows * G)


def prefill_block_support(q_c, ktil, blk: int, b_sel: int, k: int) -> np.ndarray:
    """Shared support of query block blk: top-k of the indexer scores over the
    keys of all earlier blocks, j < b_sel * blk (all of them when there are at
    most k).  The block's own (diagonal) keys are always attended, causally,
    and are not part of this list."""
    n_cand = blk * b_sel
    if n_cand == 0:
        return np.zeros(0, dtype=np.int64)
    x = token_scores(q_c, f64(ktil)[:n_cand])
    return select_topk(x, k)


def prefill_block_attend(Q_blk, K, V, S, blk: int, b_sel: int, s_att: float):
    """Exact attention of each row of a query block: keys are the shared
    support S plus the block's own keys up to and including the row's
    position.

    Q_blk: [n_rows, G, d], K/V: [N, d] (keys of the group) -> o [n_rows, G, d],
    lse [n_rows, G]
    """
    Q_blk, K, V = f64(Q_blk), f64(K), f64(V)
    n_rows, G, d = Q_blk.shape
    base = blk * b_sel
    o = np.zeros((n_rows, G, d))
    lse = np.zeros((n_rows, G))
    S = [int(j) for j in S]
    for i in range(n_rows):
        keys = S + list(range(base, base + i + 1))
        oi, li = attend(Q_blk[i], K[keys], V[keys], s_att)
        o[i] = oi
        lse[i] = li
    return o, lse


def prefill_query_scores(q_i, w_q_heads, ktil, i: int, s_idx: float, aggregate: str = "logits"):
    """Per-query (b_sel = 1) scores of query position i for one group over
    its causal candidates j <= i (Oracle-Guided Sparse Prefill 2.1, per-query
    granularity: each query chooses its own support).

    aggregate = "logits": the head-collapsed channel, q_c = s_idx * mean_h
    W_q[h]^T q_{i,h}, scores q_c . Ktil_j (as in decode).
    aggregate = "probs": each head's own low-rank logits
    s_idx * (W_q[h]^T q_{i,h}) . Ktil_j turned into a softmax over the
    candidates, averaged over the heads; the score is the log of that mean
    (so the selection rules rank by the mean probability).

    q_i: [G, d], w_q_heads: [G, d, r], ktil: [>= i+1, r] -> [i + 1]
    """
    q_i, w_q_heads, kt = f64(q_i), f64(w_q_heads), f64(ktil)[: i + 1]
    if aggregate == "logits":
        return token_scores(collapse_query(q_i, w_q_heads, s_idx), kt)
    if aggregate != "probs":
        raise ValueError("aggregate must be 'logits' or 'probs'")
    G = q_i.shape[0]
    P = np.zeros(i + 1)
    for h in range(G):
        x = kt @ (s_idx * (w_q_heads[h].T @ q_i[h]))
        w = np.exp(x - x.max())
        P += w / w.sum()
    with np.errstate(divide="ignore"):
        return np.log(P / G)


def prefill_query_support(x, i: int, k: int) -> np.ndarray:
    """Support of query i: top-k of its scores over j <= i (all of them when
    there are at most k), plus the query's own token, which is always kept
    (the per-query counterpart of the always-attended diagonal block)."""
    return with_sink_window(select_topk(x, k), i + 1, 0, 1)


def prefill_query_attend(q_i, K, V, S, s_att: float):
    """Exact attention of query i (all heads of the group) over its support
    (which holds the query's own token)."""
    S = [int(j) for j in S]
    return attend(q_i, f64(K)[S], f64(V)[S], s_att)


def prefill_oracle_query_support(q_i, K, i: int, s_att: float, k: int) -> np.ndarray:
    """Attention-mass oracle support of query i (Oracle-Guided Sparse Prefill
    2.1, per-query granularity): the top k of the head-averaged causal dense
    distribution over j <= i, plus the query's own token (kept as in
    prefill_query_support)."""
    P = head_mean_attention(q_i, f64(K)[: i + 1], s_att)
    return with_sink_window(select_topk(mass_scores(P), k), i + 1, 0, 1)


def prefill_oracle_block_support(Q_blk, K, blk: int, b_sel: int, s_att: float, k: int) -> np.ndarray:
    """Attention-mass oracle support shared by query block blk (section 2.1,
    selection-block granularity): the causal dense distributions of the
    block's queries, averaged over its rows and the group's heads, ranked
    over the keys of earlier blocks j < b_sel * blk (the block's own keys are
    attended causally on top, as for every block support)."""
    n_cand = blk * b_sel
    if n_cand == 0:
        return np.zeros(0, dtype=np.int64)
    n_rows = f64(Q_blk).shape[0]
    imp = pbs_importance(Q_blk, f64(K)[: n_cand + n_rows], n_cand, s_att)
    return select_topk(mass_scores(imp[:n_cand]), k)


# ---------------------------------------------------------------------------
# Segment-permuted block selection (PBS-Attn, sections 2 to 4)
# ---------------------------------------------------------------------------


def pbs_importance(Q_last, K, first: int, s_att: float) -> np.ndarray:
    """Global key importance from the last query block (PBS-Attn section 3):
    each query i of the block (position first + i) and each head of the
    group attends causally to keys j <= first + i; the importance of key j is
    the mean over those (query, head) pairs of the attention probability
    (zero where the key is in a query's future).

    Q_last: [n_rows, G, d], K: [N, d] -> [N]
    """
    Q_last, K = f64(Q_last), f64(K)
    n_rows, G, _ = Q_last.shape
    imp = np.zeros(K.shape[0])
    for i in range(n_rows):
        L = first + i + 1
        for h in range(G):
            z = s_att * (K[:L] @ Q_last[i, h])
            w = np.exp(z - z.max())
            imp[:L] += w / w.sum()
    return imp / (n_rows * G)


def pbs_permutation(importance, seg: int) -> np.ndarray:
    """Segment permutation (PBS-Attn sections 2 and 3): the positions of each
    segment [s * seg, (s + 1) * seg) are reordered by importance, largest
    first (equal importance: lower position first); no key leaves its
    segment.  perm[p] = the position of the key placed at p."""
    imp = f64(importance)
    N = imp.shape[0]
    perm = np.arange(N)
    for s0 in range(0, N, seg):
        idx = np.arange(s0, min(N, s0 + seg))
        order = np.lexsort((idx, -imp[idx]))
        perm[s0:s0 + len(idx)] = idx[order]
    return perm


def pbs_block_keys(perm, blk: int, b_sel: int, seg: int, c: int) -> np.ndarray:
    """Keys of candidate block c of query block blk: a block of the permuted
    order in a segment that ends before the query block's segment, or, inside
    its own segment, a block in natural order (a permutation there would put
    later keys before earlier ones)."""
    own_seg_first_block = (blk * b_sel // seg) * seg // b_sel
    if c < own_seg_first_block:
        return np.asarray(perm[c * b_sel:(c + 1) * b_sel], dtype=np.int64)
    return np.arange(c * b_sel, (c + 1) * b_sel)


def pbs_block_scores(Q_blk, K, perm, blk: int, b_sel: int, seg: int) -> np.ndarray:
    """Mean-pooled block scores (PBS-Attn section 4): the mean of the block's
    queries over its rows and the group's heads, dotted with the mean of each
    candidate block's keys, for the blk earlier blocks.

    Q_blk: [n_rows, G, d], K: [N, d] -> [blk]
    """
    Q_blk, K = f64(Q_blk), f64(K)
    qbar = Q_blk.reshape(-1, Q_blk.shape[-1]).mean(axis=0)
    x = np.zeros(blk)
    for c in range(blk):
        kbar = K[pbs_block_keys(perm, blk, b_sel, seg, c)].mean(axis=0)
        x[c] = qbar @ kbar
    return x


def pbs_block_support(x, perm, blk: int, b_sel: int, seg: int, k_blocks: int) -> np.ndarray:
    """Keys of the top-k candidate blocks (ties lower block first), ascending;
    the query block's own keys are attended causally on top (as in
    prefill_block_attend)."""
    if blk == 0:
        return np.zeros(0, dtype=np.int64)
    blocks = select_topk(x, k_blocks)
    keys = np.concatenate([pbs_block_keys(perm, blk, b_sel, seg, int(c)) for c in blocks])
    return np.sort(keys)


# ---------------------------------------------------------------------------
# Residual linear attention over the unselected tokens (SPLA section 2.2)
# ---------------------------------------------------------------------------


def rla_feature(x) -> np.ndarray:
    """The parameter-free exponential feature map, applied elementwise:
    phi(x)_i = exp(x_i) (reading: on the raw query/key rows, no scale)."""
    return np.exp(f64(x))


def rla_state(K, V):
    """Global linear-attention state of one key/value group over all n
    cached tokens: S = sum_j phi(k_j) v_j^T  [d, d_v]  and  z = sum_j phi(k_j)
    [d].  (The recurrent state the page keeps; built here from scratch.)"""
    phk = rla_feature(K)
    return phk.T @ f64(V), phk.sum(axis=0)


def rla_unselected(q_heads, K, V, support):
    """Residual linear attention of each head over the tokens NOT in the
    support, as direct sums (the definition):
        num_h = sum_{j not in S} (phi(q_h) . phi(k_j)) v_j      [d_v]
        den_h = sum_{j not in S}  phi(q_h) . phi(k_j)
    and o_rla_h = num_h / den_h (the caller normalises; the page applies a
    learned RMS norm and gate on top, outside this path).
    q_heads [G, d], K/V [n, d], support: token indices -> (num [G, d_v], den [G])."""
    q_heads, K, V = f64(q_heads), f64(K), f64(V)
    n = K.shape[0]
    keep = np.ones(n, dtype=bool)
    keep[np.asarray(support, dtype=np.int64)] = False
    G = q_heads.shape[0]
    num = np.zeros((G, V.shape[1]))
    den = np.zeros(G)
    phq = rla_feature(q_heads)
    for h in range(G):
        for j in np.nonzero(keep)[0]:
            w = float(phq[h] @ rla_feature(K[j]))
            num[h] += w * V[j]
            den[h] += w
    return num, den


def rla_by_subtraction(q_heads, S_all, z_all, K_sel, V_sel):
    """The IO-efficient form of the same quantity: the global state's terms
    minus the selected tokens' terms, so unselected keys and values are never
    read again:  num_h = phi(q_h)^T S_all - sum_{j in S} (phi(q_h).phi(k_j)) v_j,
    den_h = phi(q_h) . z_all - sum_{j in S} phi(q_h) . phi(k_j)."""
    phq = rla_feature(q_heads)
    phk = rla_feature(K_sel)
    w = phq @ phk.T                       # [G, |S|]
    num = phq @ f64(S_all) - w @ f64(V_sel)
    den = phq @ f64(z_all) - w.sum(axis=1)
    return num, den
