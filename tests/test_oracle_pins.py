"""Pins of the float64 oracle to facts fixed outside the oracle itself:
hand-made distributions, brute force on tiny inputs, closed forms, library
routines (torch scaled_dot_product_attention in float64), and the invariants
the pages state.  CPU only."""

import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# bf16 rounding helper
# ---------------------------------------------------------------------------


def test_round_to_bf16_matches_torch_on_fp32_values():
    rng = _rng(0)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x32.astype(np.float64)), ref)


def test_round_to_bf16_halfway_cases():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even -> 1.
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6.
    assert O.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above halfway rounds up
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    assert O.round_to_bf16(np.array([-1 - 2.0 ** -8 - 2.0 ** -30]))[0] == -1 - 2.0 ** -7
    assert O.round_to_bf16(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# Selection rule: golden dyadic cases, brute force
# ---------------------------------------------------------------------------


def _golden_cases():
    cases = []
    with open(os.path.join(GOLDEN, "topp_dyadic.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, masses, param, expect = [s.strip() for s in line.split("|")]
            cases.append((kind, np.array([float(v) for v in masses.split()]),
                          float(param), [int(v) for v in expect.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"{c[0]}-{c[2]}-{len(c[1])}")
def test_golden_dyadic_rule(case):
    kind, masses, param, expect = case
    order = O.candidate_order(masses)  # order of masses == order of log-scores
    if kind == "topp":
        take = O.prefix_reaching(masses[order], param) if param < 1 else len(masses)
        got = sorted(order[:take].tolist())
    else:
        got = sorted(order[: min(int(param), len(masses))].tolist())
    assert got == expect


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"{c[0]}-{c[2]}-{len(c[1])}")
def test_golden_through_scores(case):
    """The score-level entry points reproduce the golden sets when scores are
    log-masses, except where p sits exactly on a running sum (there rounding
    of exp/log may decide, and the mass-level test above already pins it)."""
    kind, masses, param, expect = case
    x = np.log(masses)
    if kind == "topk":
        assert O.select_topk(x, int(param)).tolist() == expect
        return
    got = O.select_topp(x, param).tolist()
    cums = np.cumsum(np.sort(masses)[::-1])
    if not (param < 1 and np.any(np.abs(cums - param) < 1e-12)) or len(set(masses)) == 1:
        # p away from every running sum, or all masses equal (exp(0) = 1 each,
        # so the masses are exact): the rule decides
        assert got == expect
        return
    # p on an exact running sum of unequal masses: log and exp round, so the
    # sum at the boundary may land on either side of p; the expected set or
    # it plus the next candidate is accepted, and p -/+ 1e-9 (beyond any
    # float64 rounding here) gives exactly those two sets
    order = O.candidate_order(x)
    alt = sorted(expect + [int(order[len(expect)])])
    assert got in (expect, alt)
    assert O.select_topp(x, param - 1e-9).tolist() == expect
    assert O.select_topp(x, param + 1e-9).tolist() == alt


def test_softmax_mass_closed_form_and_shift():
    x = np.log(np.array([1.0, 2.0, 5.0]))
    np.testing.assert_allclose(O.softmax_mass(x), [1 / 8, 2 / 8, 5 / 8], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.softmax_mass(x + 700.0), [1 / 8, 2 / 8, 5 / 8], atol=1e-15)


@pytest.mark.parametrize("seed", range(12))
def test_topp_brute_force(seed):
    rng = _rng(100 + seed)
    n = int(rng.integers(1, 11))
    x = rng.standard_normal(n) * 2.0
    w = np.exp(x)
    for p in (0.3, 0.5, 0.77, 0.9, 0.99):
        S = O.select_topp(x, p)
        # brute force: minimum cardinality among subsets reaching p, then max mass
        best = None
        for c in range(1, n + 1):
            feas = []
            for sub in itertools.combinations(range(n), c):
                m = math.fsum(w[list(sub)]) / math.fsum(w)
                if m >= p:
                    feas.append((m, sub))
            if feas:
                best = (c, max(feas)[1])
                break
        assert best is not None
        assert len(S) == best[0]
        assert sorted(S.tolist()) == sorted(best[1])


@pytest.mark.parametrize("seed", range(8))
def test_topk_brute_force(seed):
    rng = _rng(200 + seed)
    n = int(rng.integers(1, 11))
    x = rng.standard_normal(n)
    for k in range(1, n + 2):
        S = O.select_topk(x, k)
        c = min(k, n)
        best = max(itertools.combinations(range(n), c), key=lambda s: math.fsum(x[list(s)]))
        assert sorted(S.tolist()) == sorted(best)


def test_ties_take_lower_index_and_all_at_p1():
    x = np.array([1.0, 3.0, 3.0, 3.0, 0.0])
    assert O.select_topk(x, 2).tolist() == [1, 2]
    assert O.select_topp(x, 1.0).tolist() == [0, 1, 2, 3, 4]
    # three tied maxima carry most of the mass; p just above 2/3 of their sum
    w = np.exp(x - 3.0)
    p = (2 * w[1]) / w.sum() + 1e-9
    assert O.select_topp(x, p).tolist() == [1, 2, 3]
    with pytest.raises(ValueError):
        O.select_topp(x, 0.0)
    with pytest.raises(ValueError):
        O.select_topk(x, 0)


def test_sink_window_and_page_expansion():
    S = np.array([10, 50, 97])
    assert O.with_sink_window(S, 100, 4, 5).tolist() == [0, 1, 2, 3, 10, 50, 95, 96, 97, 98, 99]
    assert O.with_sink_window(np.array([], dtype=int), 3, 4, 512).tolist() == [0, 1, 2]
    assert O.expand_pages([2, 0], 150, 64).tolist() == list(range(0, 64)) + list(range(128, 150))


# ---------------------------------------------------------------------------
# Indexer
# ---------------------------------------------------------------------------


def test_indexer_coordinate_projector_reduces_to_plain_dot():
    """With W = [I_r; 0] the low-rank channel is the first r coordinates, so
    the score is s_idx * (mean_h q_h[:r]) . k_j[:r]."""
    rng = _rng(1)
    d, r, G, L = 32, 16, 4, 50
    W = np.zeros((d, r))
    W[:r, :r] = np.eye(r)
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    s = 0.37
    x = O.token_scores(O.collapse_query(q, np.stack([W] * G), s), O.indexer_keys(K, W))
    expect = np.array([s * sum(q[:, i].mean() * K[j, i] for i in range(r)) for j in range(L)])
    np.testing.assert_allclose(x, expect, rtol=1e-13, atol=1e-13)


def test_indexer_collapse_is_mean_of_head_logits():
    rng = _rng(2)
    d, r, G, L = 64, 16, 8, 40
    Wq = rng.standard_normal((G, d, r)) / 8
    Wk = rng.standard_normal((d, r)) / 8
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    kt = O.indexer_keys(K, Wk)
    x = O.token_scores(O.collapse_query(q, Wq, 1.5), kt)
    per_head = np.stack([O.token_scores(O.collapse_query(q[h:h + 1], Wq[h:h + 1], 1.5), kt)
                         for h in range(G)])
    np.testing.assert_allclose(x, per_head.mean(axis=0), rtol=1e-12, atol=1e-12)


def test_indexer_group_semantics():
    """Two groups whose heads point at different planted keys: each group's
    top-1 is its own key, and the sign is right (aligned keys score high)."""
    rng = _rng(3)
    d, r, H_q, H_kv, L = 32, 16, 8, 2, 64
    G = H_q // H_kv
    W = rng.standard_normal((H_kv, d, r)) / math.sqrt(d)
    K = rng.standard_normal((L, H_kv, d)) * 0.1
    q = rng.standard_normal((H_q, d)) * 0.1
    targets = {0: 5, 1: 41}
    for g, j in targets.items():
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        for h in O.heads_of_group(g, H_q, H_kv):
            q[h] += 3 * u
        K[j, g] += 4 * u
        K[targets[1 - g], g] -= 4 * u  # the other group's needle is anti-aligned here
    for g, j in targets.items():
        hs = O.heads_of_group(g, H_q, H_kv)
        qc = O.collapse_query(q[hs], np.stack([W[g]] * G), 1.0)
        x = O.token_scores(qc, O.indexer_keys(K[:, g], W[g]))
        assert O.select_topk(x, 1).tolist() == [j]
        assert int(np.argmin(x)) == targets[1 - g]


# ---------------------------------------------------------------------------
# Page statistics and the Taylor page score
# ---------------------------------------------------------------------------


def test_page_stats_closed_forms():
    d = 8
    # page 0: constant rows; page 1: +/- sigma pairs around m; page 2: arithmetic
    # progression 0..63 in every dim; page 3 (partial, 10 rows): 0..9
    c = np.arange(d, dtype=float)
    m = np.linspace(-1, 1, d)
    sig = 0.75
    p1 = np.concatenate([m + sig * np.ones(d)] * 32 + [m - sig * np.ones(d)] * 32).reshape(64, d)
    p2 = np.repeat(np.arange(64, dtype=float)[:, None], d, axis=1)
    p3 = np.repeat(np.arange(10, dtype=float)[:, None], d, axis=1)
    K = np.concatenate([np.tile(c, (64, 1)), p1, p2, p3])
    mean, var, n = O.page_stats(K, 64)
    assert n.tolist() == [64, 64, 64, 10]
    np.testing.assert_allclose(mean[0], c, atol=0)
    np.testing.assert_allclose(var[0], 0, atol=0)
    np.testing.assert_allclose(mean[1], m, atol=1e-15)
    np.testing.assert_allclose(var[1], sig ** 2, rtol=1e-14)
    np.testing.assert_allclose(mean[2], 31.5, rtol=1e-15)
    np.testing.assert_allclose(var[2], (64 ** 2 - 1) / 12, rtol=1e-14)
    np.testing.assert_allclose(mean[3], 4.5, rtol=1e-15)
    np.testing.assert_allclose(var[3], (10 ** 2 - 1) / 12, rtol=1e-14)


def _axis_pair_page(kbar, sig, rng, npairs=32):
    """64 keys kbar +/- sig*z*e_a (pairs along coordinate axes): the empirical
    mean is exactly kbar and the empirical covariance exactly diagonal."""
    d = kbar.shape[0]
    rows = []
    for _ in range(npairs):
        a = int(rng.integers(d))
        z = float(rng.standard_normal())
        e = np.zeros(d)
        e[a] = sig * z
        rows += [kbar + e, kbar - e]
    return np.array(rows)


def test_taylor_constant_page_is_exact():
    rng = _rng(4)
    d = 16
    kb = rng.standard_normal(d)
    page = np.tile(kb, (64, 1))
    q = rng.standard_normal(d) * 0.3
    mean, var, _ = O.page_stats(page, 64)
    exact = np.mean(np.exp(page @ q))
    assert O.taylor_page_score(q, mean[0], var[0]) == pytest.approx(exact, rel=1e-14)


def test_taylor_axis_pairs_fourth_order_decay():
    """On axis-pair pages the Taylor score misses only 4th and higher moments:
    relative error ~ sigma^4 (log-log slope 4)."""
    rng = _rng(5)
    d = 16
    kb = rng.standard_normal(d) * 0.2
    q = rng.standard_normal(d) * 0.5
    base = _axis_pair_page(kb, 1.0, _rng(6)) - kb  # unit-scale deviations
    errs = []
    sigmas = [0.4, 0.2, 0.1, 0.05, 0.025]
    for s in sigmas:
        page = kb + s * base
        mean, var, _ = O.page_stats(page, 64)
        exact = np.mean(np.exp(page @ q))
        errs.append(abs(O.taylor_page_score(q, mean[0], var[0]) - exact) / exact)
    slopes = np.diff(np.log(errs)) / np.diff(np.log(sigmas))
    assert np.all(np.abs(slopes - 4.0) < 0.15), slopes


def test_taylor_diagonal_leaves_offdiagonal_term():
    """On general random pages the diagonal approximation leaves the
    off-diagonal covariance term, so the error is far larger than on
    axis-pair pages of the same scale (pins the diagonal, not the full
    covariance, being used)."""
    rng = _rng(7)
    d = 16
    q = rng.standard_normal(d) * 0.5
    kb = rng.standard_normal(d) * 0.2
    for s in (0.1, 0.025):
        gen = kb + s * rng.standard_normal((64, d))
        ax = kb + s * (_axis_pair_page(kb, 1.0, _rng(8)) - kb)
        errs = []
        for page in (gen, ax):
            mean, var, _ = O.page_stats(page, 64)
            exact = np.mean(np.exp(page @ q))
            errs.append(abs(O.taylor_page_score(q, mean[0], var[0]) - exact) / exact)
        assert errs[0] > 50 * errs[1]


def test_taylor_gaussian_closed_form():
    """For k ~ N(mu, diag(s2)), E exp(q.k) = exp(q.mu + q^T S q / 2); the
    Taylor score is its first-order expansion in t = q^T S q, so the relative
    gap approaches t^2/8."""
    rng = _rng(9)
    d = 16
    mu = rng.standard_normal(d) * 0.3
    s2 = rng.uniform(0.5, 1.5, d)
    for scale in (0.1, 0.05, 0.02):
        q = rng.standard_normal(d) * scale
        t = float((q * q) @ s2)
        exact = math.exp(float(q @ mu) + 0.5 * t)
        gap = (exact - O.taylor_page_score(q, mu, s2)) / exact
        assert gap == pytest.approx(t * t / 8, rel=0.05)


def test_page_scores_is_mean_of_log_taylor_scores():
    rng = _rng(10)
    d, G, P = 16, 4, 6
    q = rng.standard_normal((G, d))
    mean = rng.standard_normal((P, d))
    var = rng.uniform(0, 2, (P, d))
    n = np.array([64] * 5 + [20])
    s = 0.25
    x = O.page_scores(q, mean, var, n, s, 64)
    for p in range(P):
        logs = [math.log(O.taylor_page_score(s * q[h], mean[p], var[p])) for h in range(G)]
        assert x[p] == pytest.approx(np.mean(logs) + math.log(n[p] / 64), abs=1e-12)


# ---------------------------------------------------------------------------
# Attention over the support
# ---------------------------------------------------------------------------


def _sdpa(q, K, V, scale, causal=False):
    """torch SDPA in float64 on CPU (math backend), the library reference."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    Kt = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64))
    Vt = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, Kt, Vt, scale=scale, is_causal=causal)
    return out.numpy()


def test_dense_special_case_matches_sdpa():
    """p = 1 or k >= L (no sink/window) select every key, and the sparse
    decode equals dense attention."""
    rng = _rng(11)
    G, d, L, r = 4, 32, 200, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    Wq = rng.standard_normal((G, d, r)) / math.sqrt(d)
    Wk = rng.standard_normal((d, r)) / math.sqrt(d)
    kt = O.indexer_keys(K, Wk)
    s = 1 / math.sqrt(d)
    ref = _sdpa(q[None, :, None, :], K[None, None], V[None, None], s)[0, :, 0]
    for kw in ({"p": 1.0}, {"k": L}, {"k": L + 7}):
        out = O.decode_row(q, Wq, kt, K, V, s_idx=1.0, s_att=s, **kw)
        assert out["S"].tolist() == list(range(L))
        np.testing.assert_allclose(out["o"], ref, rtol=0, atol=1e-12)
    # lse against a direct logsumexp of the full logits
    o, lse = O.attend(q, K, V, s)
    logits = s * q @ K.T
    np.testing.assert_allclose(lse, np.log(np.exp(logits).sum(axis=1)), rtol=1e-13)


def test_single_key_support_returns_its_value():
    rng = _rng(12)
    q = rng.standard_normal((3, 16))
    K = rng.standard_normal((1, 16))
    V = rng.standard_normal((1, 16))
    o, lse = O.attend(q, K, V, 0.25)
    for h in range(3):
        np.testing.assert_array_equal(o[h], V[0])
    np.testing.assert_allclose(lse, 0.25 * q @ K[0], rtol=1e-15)


def test_gqa_heads_equal_single_head_attention():
    rng = _rng(13)
    q = rng.standard_normal((8, 32))
    K = rng.standard_normal((70, 32))
    V = rng.standard_normal((70, 32))
    o, lse = O.attend(q, K, V, 0.2)
    for h in range(8):
        oh, lh = O.attend(q[h:h + 1], K, V, 0.2)
        np.testing.assert_array_equal(oh[0], o[h])
        assert lh[0] == lse[h]


def test_kv_permutation_invariance_decode():
    """Jointly permuting (k_j, v_j, K~_j) leaves the output unchanged and maps
    the support through the permutation (scores have no ties here)."""
    rng = _rng(14)
    G, d, L, r = 4, 32, 300, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    W = rng.standard_normal((d, r)) / math.sqrt(d)
    Wq = np.stack([W] * G)
    kt = O.indexer_keys(K, W)
    perm = rng.permutation(L)
    for kw in ({"p": 0.8}, {"k": 40}):
        a = O.decode_row(q, Wq, kt, K, V, s_idx=2.0, s_att=0.2, **kw)
        b = O.decode_row(q, Wq, kt[perm], K[perm], V[perm], s_idx=2.0, s_att=0.2, **kw)
        assert sorted(perm[b["S"]].tolist()) == a["S"].tolist()
        np.testing.assert_allclose(b["o"], a["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b["lse"], a["lse"], rtol=0, atol=1e-12)


def test_head_permutation_covariance_decode():
    rng = _rng(15)
    G, d, L, r = 4, 16, 100, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    W = rng.standard_normal((d, r)) / 4
    Wq = np.stack([W] * G)
    kt = O.indexer_keys(K, W)
    perm = rng.permutation(G)
    a = O.decode_row(q, Wq, kt, K, V, s_idx=1.0, s_att=0.25, p=0.9)
    b = O.decode_row(q[perm], Wq[perm], kt, K, V, s_idx=1.0, s_att=0.25, p=0.9)
    assert a["S"].tolist() == b["S"].tolist()
    np.testing.assert_allclose(b["o"], a["o"][perm], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Causal prefill with block-shared supports
# ---------------------------------------------------------------------------


def _prefill_case(seed, N=320, G=2, d=16, r=16):
    rng = _rng(seed)
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    W = rng.standard_normal((d, r)) / math.sqrt(d)
    return Q, K, V, np.stack([W] * G), O.indexer_keys(K, W)


def test_early_prefill_blocks_equal_dense_causal():
    """While b_sel * blk <= k every earlier key is kept, so each row equals
    dense causal attention."""
    b_sel, k = 32, 96
    Q, K, V, Wq, kt = _prefill_case(16, N=224)
    s = 0.25
    N, G, d = Q.shape
    ref = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], V[None, None], s, causal=True)[0]
    for blk in range(0, k // b_sel + 1):
        rows = O.prefill_block_rows(blk, b_sel, N)
        qc = O.prefill_block_query(Q[rows.start:rows.stop], Wq, 1.0)
        S = O.prefill_block_support(qc, kt, blk, b_sel, k)
        assert S.tolist() == list(range(blk * b_sel))
        o, _ = O.prefill_block_attend(Q[rows.start:rows.stop], K, V, S, blk, b_sel, s)
        np.testing.assert_allclose(o, np.transpose(ref[:, rows.start:rows.stop], (1, 0, 2)),
                                   rtol=0, atol=1e-12)


def test_prefill_segment_permutation_invariance():
    """Permuting the keys strictly before the block (one segment, pairing of
    k, v and K~ kept) leaves the block's outputs unchanged."""
    b_sel, k, blk = 32, 40, 6
    Q, K, V, Wq, kt = _prefill_case(17)
    rng = _rng(18)
    base = blk * b_sel
    perm = np.concatenate([rng.permutation(base), np.arange(base, K.shape[0])])
    rows = O.prefill_block_rows(blk, b_sel, K.shape[0])
    Qb = Q[rows.start:rows.stop]
    qc = O.prefill_block_query(Qb, Wq, 1.0)
    S1 = O.prefill_block_support(qc, kt, blk, b_sel, k)
    S2 = O.prefill_block_support(qc, kt[perm], blk, b_sel, k)
    assert sorted(perm[S2].tolist()) == S1.tolist()
    o1, l1 = O.prefill_block_attend(Qb, K, V, S1, blk, b_sel, 0.25)
    o2, l2 = O.prefill_block_attend(Qb, K[perm], V[perm], S2, blk, b_sel, 0.25)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_prefill_block_query_permutation_invariant():
    Q, K, V, Wq, kt = _prefill_case(19)
    rng = _rng(20)
    Qb = Q[64:96]
    a = O.prefill_block_query(Qb, Wq, 0.7)
    b = O.prefill_block_query(Qb[rng.permutation(32)], Wq, 0.7)
    c = O.prefill_block_query(Qb[:, ::-1], Wq[::-1], 0.7)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a, c, rtol=1e-13, atol=1e-14)


def test_prefill_block_query_closed_form():
    """Value pins for the block query ("Oracle-Guided Sparse Prefill", section
    2.2 indexer shared by a block; the mean over the block's queries and the
    group's heads): with coordinate projectors W_q[h] = c_h [e_0 e_1] and
    queries q_{i,h} = (i, h, 5, ...), the block query is s_idx times the
    averages of c_h * i and c_h * h, which integer data give exactly."""
    n_rows, G, d, r = 64, 4, 8, 2
    c = np.array([1.0, 2.0, 3.0, 4.0])
    Wq = np.zeros((G, d, r))
    for h in range(G):
        Wq[h, 0, 0] = c[h]
        Wq[h, 1, 1] = c[h]
    Qb = np.full((n_rows, G, d), 5.0)
    for i in range(n_rows):
        for h in range(G):
            Qb[i, h, 0] = i
            Qb[i, h, 1] = h
    got = O.prefill_block_query(Qb, Wq, 0.5)
    mean_c_i = c.mean() * (n_rows - 1) / 2.0          # mean over (i, h) of c_h * i
    mean_c_h = float((c * np.arange(G)).mean())       # mean over (i, h) of c_h * h
    np.testing.assert_allclose(got, 0.5 * np.array([mean_c_i, mean_c_h]), rtol=0, atol=1e-13)
    # a one-row block is the decode step's head-collapsed query of that row,
    # and the block query is the mean of its rows' collapsed queries
    Q, K, V, Wq2, kt = _prefill_case(23)
    rows = [O.collapse_query(Q[i], Wq2, 0.7) for i in range(128, 192)]
    np.testing.assert_allclose(O.prefill_block_query(Q[128:129], Wq2, 0.7), rows[0],
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O.prefill_block_query(Q[128:192], Wq2, 0.7), np.mean(rows, axis=0),
                               rtol=1e-12, atol=1e-13)
    # linear in the queries: doubling one row shifts the mean by that row / n
    Qd = Q[128:192].copy()
    Qd[7] *= 2.0
    np.testing.assert_allclose(O.prefill_block_query(Qd, Wq2, 0.7),
                               np.mean(rows, axis=0) + rows[7] / 64.0, rtol=1e-12, atol=1e-13)


def test_prefill_support_excludes_own_block_and_is_topk():
    b_sel, k, blk = 32, 20, 5
    Q, K, V, Wq, kt = _prefill_case(21)
    rows = O.prefill_block_rows(blk, b_sel, K.shape[0])
    qc = O.prefill_block_query(Q[rows.start:rows.stop], Wq, 1.0)
    S = O.prefill_block_support(qc, kt, blk, b_sel, k)
    assert len(S) == k and S.max() < blk * b_sel
    x = kt[: blk * b_sel] @ qc
    assert x[S].min() > np.delete(x, S).max()


# ---------------------------------------------------------------------------
# Residual linear attention over the unselected tokens (SPLA section 2.2)
# ---------------------------------------------------------------------------


def _rla_case(seed, n=40, d=8, G=3, scale=0.5):
    rng = _rng(seed)
    q = rng.standard_normal((G, d)) * scale
    K = rng.standard_normal((n, d)) * scale
    V = rng.standard_normal((n, d))
    return q, K, V


def test_rla_state_single_token_is_outer_product():
    k = np.array([[0.5, -1.0, 0.0]])
    v = np.array([[2.0, 3.0, -1.0]])
    S, z = O.rla_state(k, v)
    e = np.exp(k[0])
    for i in range(3):
        for j in range(3):
            assert S[i, j] == e[i] * v[0, j]
    assert np.array_equal(z, e)


def test_rla_zero_keys_give_mean_of_unselected_values():
    """k = 0: every key's feature is all ones, so all weights are equal and
    num / den is the plain mean of the unselected values."""
    q, _, V = _rla_case(31)
    K = np.zeros((V.shape[0], q.shape[1]))
    support = [0, 3, 7, 8, 20]
    num, den = O.rla_unselected(q, K, V, support)
    rest = np.delete(V, support, axis=0)
    for h in range(q.shape[0]):
        np.testing.assert_allclose(num[h] / den[h], rest.mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(den[h], len(rest) * np.exp(q[h]).sum(), rtol=1e-13)


def test_rla_single_unselected_token_returns_its_value():
    q, K, V = _rla_case(32, n=6)
    support = [0, 1, 2, 4, 5]
    num, den = O.rla_unselected(q, K, V, support)
    for h in range(q.shape[0]):
        w = np.exp(q[h] + K[3]).sum()   # phi(q).phi(k) = sum_i exp(q_i + k_i)
        np.testing.assert_allclose(den[h], w, rtol=1e-13)
        np.testing.assert_allclose(num[h] / den[h], V[3], rtol=1e-12, atol=1e-13)


def test_rla_full_support_leaves_nothing():
    q, K, V = _rla_case(33)
    num, den = O.rla_unselected(q, K, V, np.arange(K.shape[0]))
    assert np.all(num == 0) and np.all(den == 0)
    S_all, z_all = O.rla_state(K, V)
    num2, den2 = O.rla_by_subtraction(q, S_all, z_all, K, V)
    np.testing.assert_allclose(num2, 0, atol=1e-12 * np.abs(q).max() * np.abs(S_all).max())
    np.testing.assert_allclose(den2, 0, atol=1e-12 * np.abs(z_all).max() * 10)


def test_rla_subtraction_equals_direct_sum():
    """The page's IO-efficient subtraction form and the definition agree (the
    identity the fused kernel relies on)."""
    q, K, V = _rla_case(34, n=60)
    rng = _rng(35)
    support = np.sort(rng.choice(60, 17, replace=False))
    num, den = O.rla_unselected(q, K, V, support)
    S_all, z_all = O.rla_state(K, V)
    num2, den2 = O.rla_by_subtraction(q, S_all, z_all, K[support], V[support])
    np.testing.assert_allclose(num2, num, rtol=1e-10, atol=1e-10 * np.abs(num).max())
    np.testing.assert_allclose(den2, den, rtol=1e-12)


def test_rla_linear_in_values_and_permutation_invariant():
    q, K, V = _rla_case(36, n=30)
    support = [2, 5, 11]
    num, den = O.rla_unselected(q, K, V, support)
    num2, den2 = O.rla_unselected(q, K, 2.0 * V, support)
    np.testing.assert_allclose(num2, 2.0 * num, rtol=1e-13)
    np.testing.assert_array_equal(den2, den)
    perm = _rng(37).permutation(30)
    inv = np.argsort(perm)
    num3, den3 = O.rla_unselected(q, K[perm], V[perm], inv[support])
    np.testing.assert_allclose(num3, num, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(den3, den, rtol=1e-12)


# ---------------------------------------------------------------------------
# Attention-mass oracle support (Oracle-Guided Sparse Prefill section 2.1)
# ---------------------------------------------------------------------------


def test_head_mean_attention_is_mean_of_sdpa_weights():
    """With one-hot values (V = I) torch's attention output is the weight
    row itself; averaging it over the group's heads gives P."""
    rng = _rng(40)
    G, d, n = 4, 16, 37
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d))
    s = 0.7 / math.sqrt(d)
    W = _sdpa(q[None, :, None, :], K[None, None], np.eye(n)[None, None], s)[0, :, 0]  # [G, n]
    P = O.head_mean_attention(q, K, s)
    np.testing.assert_allclose(P, W.mean(axis=0), rtol=1e-12, atol=1e-16)
    assert abs(P.sum() - 1.0) < 1e-13 and np.all(P >= 0)


def test_head_mean_attention_two_keys_logistic():
    q = np.array([[1.0, 2.0]])
    K = np.array([[0.5, 0.0], [0.0, 1.0]])
    s = 0.3
    a = s * (0.5 - 2.0)                 # logit difference of key 0 over key 1
    P = O.head_mean_attention(q, K, s)
    np.testing.assert_allclose(P, [1 / (1 + math.exp(-a)), 1 / (1 + math.exp(a))], rtol=1e-14)


def test_head_mean_attention_equal_keys_uniform_and_heads_symmetric():
    rng = _rng(41)
    q = rng.standard_normal((3, 8))
    K = np.tile(rng.standard_normal(8), (9, 1))
    np.testing.assert_allclose(O.head_mean_attention(q, K, 0.5), np.full(9, 1 / 9), rtol=1e-14)
    K = rng.standard_normal((20, 8))
    P = O.head_mean_attention(q, K, 0.5)
    np.testing.assert_allclose(O.head_mean_attention(q[::-1], K, 0.5), P, rtol=1e-13)
    perm = rng.permutation(20)
    np.testing.assert_allclose(O.head_mean_attention(q, K[perm], 0.5), P[perm], rtol=1e-13)
    # one head locked on key 5 gives it at least 1/G of the averaged mass
    u = K[5] / np.linalg.norm(K[5])
    K2, q2 = K.copy(), q.copy()
    K2[5] = 20.0 * u
    q2[1] = 5.0 * u                      # logit 100 on key 5, at most ~5|k| elsewhere
    assert O.head_mean_attention(q2, K2, 1.0)[5] >= 1 / 3 - 1e-9


@pytest.mark.parametrize("seed", range(6))
def test_oracle_support_brute_force(seed):
    rng = _rng(50 + seed)
    n = int(rng.integers(3, 10))
    P = rng.dirichlet(np.full(n, 0.5))
    for k in range(1, n + 1):
        S = O.oracle_support(P, k=k)
        best = max(sum(P[list(c)]) for c in itertools.combinations(range(n), k))
        assert len(S) == k and abs(O.support_coverage(P, S) - best) < 1e-15
    for p in (0.3, 0.5, 0.8, 0.95):
        S = O.oracle_support(P, p=p)
        assert O.support_coverage(P, S) >= p
        smaller = [sum(P[list(c)]) for c in itertools.combinations(range(n), len(S) - 1)]
        assert len(S) == 1 or max(smaller) < p


def test_oracle_support_ties_and_coverage_edges():
    P = np.array([0.25, 0.125, 0.25, 0.125, 0.25])
    assert O.oracle_support(P, k=2).tolist() == [0, 2]
    assert O.oracle_support(P, k=4).tolist() == [0, 1, 2, 4]
    assert O.oracle_support(P, p=0.5).tolist() == [0, 2]
    assert O.oracle_support(P, p=0.75).tolist() == [0, 2, 4]
    assert O.support_coverage(P, []) == 0.0
    assert O.support_coverage(P, range(5)) == 1.0
    assert O.support_overlap([1, 4, 7, 9], [0, 4, 9, 11]) == 2
    assert O.support_overlap([], [3]) == 0


# ---------------------------------------------------------------------------
# Per-query prefill supports (Oracle-Guided Sparse Prefill section 2.1, b_sel = 1)
# ---------------------------------------------------------------------------


def _pq_case(seed, N=40, G=3, d=8, r=4):
    rng = _rng(seed)
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    W = rng.standard_normal((G, d, r)) / math.sqrt(d)
    Kt = rng.standard_normal((N, r))
    return Q, K, V, W, Kt


def test_prefill_query_full_support_is_dense_causal():
    Q, K, V, W, Kt = _pq_case(60)
    N, G, d = Q.shape
    s = 1 / math.sqrt(d)
    ref = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], V[None, None], s, causal=True)[0]
    for i in (0, 1, 17, N - 1):
        for agg in ("logits", "probs"):
            x = O.prefill_query_scores(Q[i], W, Kt, i, 1.0, agg)
            S = O.prefill_query_support(x, i, k=N)
            assert S.tolist() == list(range(i + 1))
            o, _ = O.prefill_query_attend(Q[i], K, V, S, s)
            np.testing.assert_allclose(o, ref[:, i], rtol=1e-12, atol=1e-13)


def test_prefill_query_own_token_always_kept():
    Q, K, V, W, Kt = _pq_case(61)
    for agg in ("logits", "probs"):
        for i in range(6, 40):
            x = O.prefill_query_scores(Q[i], W, Kt, i, 1.0, agg)
            top = O.select_topk(x, 5)
            S = O.prefill_query_support(x, i, k=5)
            assert i in S and S.max() == i
            assert len(S) == (5 if i in top else 6)
            assert set(S.tolist()) - {i} <= set(top.tolist())


def test_prefill_query_probs_equal_logits_for_one_channel():
    """Softmax is monotone: with one head per group, or identical per-head
    projected queries, ranking by the probability mean is ranking by logits."""
    Q, K, V, W, Kt = _pq_case(62, G=1)
    for i in (5, 30):
        xl = O.prefill_query_scores(Q[i], W, Kt, i, 0.7, "logits")
        xp = O.prefill_query_scores(Q[i], W, Kt, i, 0.7, "probs")
        assert np.array_equal(O.candidate_order(xl), O.candidate_order(xp))
    Q, K, V, W, Kt = _pq_case(63, G=4)
    Q[:, :] = Q[:, :1]
    W[:] = W[:1]
    xl = O.prefill_query_scores(Q[33], W, Kt, 33, 0.7, "logits")
    xp = O.prefill_query_scores(Q[33], W, Kt, 33, 0.7, "probs")
    assert np.array_equal(O.candidate_order(xl), O.candidate_order(xp))


@pytest.mark.parametrize("seed", range(4))
def test_prefill_query_probs_topk_brute_force(seed):
    Q, K, V, W, Kt = _pq_case(70 + seed, N=9, G=3)
    i = 8
    x = O.prefill_query_scores(Q[i], W, Kt, i, 1.3, "probs")
    P = np.exp(x)
    assert abs(P.sum() - 1.0) < 1e-12
    for k in (1, 3, 6):
        S = O.select_topk(x, k)
        best = max(P[list(c)].sum() for c in itertools.combinations(range(i + 1), k))
        assert abs(P[S].sum() - best) < 1e-14


# ---------------------------------------------------------------------------
# Segment-permuted block selection (PBS-Attn sections 2 to 4)
# ---------------------------------------------------------------------------


def test_pbs_importance_is_mean_of_causal_sdpa_weights():
    rng = _rng(80)
    N, G, d, b = 50, 2, 8, 6
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    s = 0.4
    first = N - b
    imp = O.pbs_importance(Q[first:], K, first, s)
    W = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], np.eye(N)[None, None], s,
              causal=True)[0]                      # [G, N, N] weights
    np.testing.assert_allclose(imp, W[:, first:, :].mean(axis=(0, 1)), rtol=1e-12, atol=1e-16)
    assert abs(imp.sum() - 1.0) < 1e-12


def test_pbs_permutation_is_segmentwise_sort():
    rng = _rng(81)
    imp = rng.random(70)
    imp[[3, 4]] = 0.5                                  # a tie: lower position first
    perm = O.pbs_permutation(imp, 16)
    assert sorted(perm.tolist()) == list(range(70))
    for s0 in range(0, 70, 16):
        seg = perm[s0:s0 + 16]
        assert seg.min() >= s0 and seg.max() < s0 + 16
        assert np.all(np.diff(imp[seg]) <= 0)
    p0 = perm[:16].tolist()
    if imp[3] == imp[4]:
        assert p0.index(3) < p0.index(4)
    imp2 = np.zeros(40)
    imp2[29] = 1.0                                     # planted key goes to its segment's front
    assert O.pbs_permutation(imp2, 10)[20] == 29


def test_pbs_block_keys_and_scores_linear():
    rng = _rng(82)
    N, G, d, b_sel, seg = 256, 2, 8, 16, 64
    K = rng.standard_normal((N, d))
    Q = rng.standard_normal((N, G, d))
    perm = O.pbs_permutation(rng.random(N), seg)
    blk = 9                                            # own segment = blocks 8..11
    keys = [O.pbs_block_keys(perm, blk, b_sel, seg, c) for c in range(blk)]
    assert np.array_equal(np.sort(np.concatenate(keys)), np.arange(blk * b_sel))
    assert np.array_equal(keys[8], np.arange(128, 144))          # own segment: natural order
    assert np.array_equal(keys[3], perm[48:64])                  # earlier segment: permuted
    x = O.pbs_block_scores(Q[blk * b_sel:(blk + 1) * b_sel], K, perm, blk, b_sel, seg)
    qbar = Q[blk * b_sel:(blk + 1) * b_sel].reshape(-1, d).mean(axis=0)
    for c in (0, 5, 8):
        np.testing.assert_allclose(x[c], np.mean(K[keys[c]] @ qbar), rtol=1e-12)


def test_pbs_all_blocks_is_dense_causal():
    rng = _rng(83)
    N, G, d, b_sel, seg = 192, 2, 16, 32, 64
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    s = 1 / math.sqrt(d)
    perm = O.pbs_permutation(O.pbs_importance(Q[-b_sel:], K, N - b_sel, s), seg)
    ref = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], V[None, None], s, causal=True)[0]
    for blk in range(N // b_sel):
        rows = O.prefill_block_rows(blk, b_sel, N)
        x = O.pbs_block_scores(Q[rows.start:rows.stop], K, perm, blk, b_sel, seg)
        S_ = O.pbs_block_support(x, perm, blk, b_sel, seg, k_blocks=100)
        assert np.array_equal(S_, np.arange(blk * b_sel))
        o, _ = O.prefill_block_attend(Q[rows.start:rows.stop], K, V, S_, blk, b_sel, s)
        np.testing.assert_allclose(o, np.transpose(ref[:, rows.start:rows.stop], (1, 0, 2)),
                                   rtol=1e-11, atol=1e-12)


def test_pbs_permutation_concentrates_scattered_heavy_hitters():
    """Four heavy-hitter keys scattered over each segment: after the
    segment permutation one block of each earlier segment holds all of them,
    and the top block per segment covers more attention mass than the best
    natural block (the gain the page reports, on a constructed input)."""
    rng = _rng(84)
    N, G, d, b_sel, seg = 512, 1, 16, 16, 128
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    K = rng.standard_normal((N, d)) * 0.3
    Q = rng.standard_normal((N, G, d)) * 0.3 + 2.0 * u
    hh = [s0 + o for s0 in range(0, N, seg) for o in (5, 37, 70, 101)]
    K[hh] += 4.0 * u
    s = 1 / math.sqrt(d)
    imp = O.pbs_importance(Q[-b_sel:], K, N - b_sel, s)
    perm = O.pbs_permutation(imp, seg)
    for s0 in range(0, N - seg, seg):
        assert set(perm[s0:s0 + 4].tolist()) == {s0 + 5, s0 + 37, s0 + 70, s0 + 101}
    blk = N // b_sel - 1
    P = O.head_mean_attention(Q[blk * b_sel], K[:blk * b_sel], s)
    x = O.pbs_block_scores(Q[blk * b_sel:], K, perm, blk, b_sel, seg)
    n_perm_blocks = (blk * b_sel // seg) * seg // b_sel
    best_perm = max(P[O.pbs_block_keys(perm, blk, b_sel, seg, c)].sum() for c in range(n_perm_blocks))
    best_nat = max(P[c * b_sel:(c + 1) * b_sel].sum() for c in range(n_perm_blocks))
    assert best_perm > 2 * best_nat
    top = O.select_topk(x[:n_perm_blocks], 3)
    assert all(perm[c * b_sel] in hh for c in top)      # the chosen blocks lead with heavy hitters


# ---------------------------------------------------------------------------
# Prefill attention-mass oracle supports (Oracle-Guided Sparse Prefill 2.1)
# ---------------------------------------------------------------------------


def test_prefill_oracle_block_support_from_sdpa_weights():
    rng = _rng(90)
    N, G, d, b_sel = 96, 2, 8, 16
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    s = 0.6
    W = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], np.eye(N)[None, None], s,
              causal=True)[0]                                  # [G, N, N]
    for blk in (1, 3, 5):
        rows = O.prefill_block_rows(blk, b_sel, N)
        S_ = O.prefill_oracle_block_support(Q[rows.start:rows.stop], K, blk, b_sel, s, k=7)
        P = W[:, rows.start:rows.stop, : blk * b_sel].mean(axis=(0, 1))
        ref = np.sort(np.argsort(-P, kind="stable")[:7])
        assert np.array_equal(S_, ref)
    assert len(O.prefill_oracle_block_support(Q[:16], K, 0, b_sel, s, k=7)) == 0


@pytest.mark.parametrize("seed", range(3))
def test_prefill_oracle_query_support_brute_force(seed):
    rng = _rng(91 + seed)
    G, d, i = 3, 6, 8
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((12, d))
    P = O.head_mean_attention(q, K[: i + 1], 0.8)
    for k in (1, 3, 5):
        S_ = O.prefill_oracle_query_support(q, K, i, 0.8, k)
        assert i in S_
        top = set(S_.tolist()) - ({i} if len(S_) > k else set())
        best = max(P[list(c)].sum() for c in itertools.combinations(range(i + 1), k))
        assert abs(P[sorted(top)].sum() - best) < 1e-14


def test_prefill_oracle_full_budget_is_dense_causal():
    rng = _rng(94)
    N, G, d, b_sel = 64, 2, 8, 16
    Q = rng.standard_normal((N, G, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    s = 1 / math.sqrt(d)
    ref = _sdpa(np.transpose(Q, (1, 0, 2))[None], K[None, None], V[None, None], s, causal=True)[0]
    for blk in range(N // b_sel):
        rows = O.prefill_block_rows(blk, b_sel, N)
        S_ = O.prefill_oracle_block_support(Q[rows.start:rows.stop], K, blk, b_sel, s, k=N)
        o, _ = O.prefill_block_attend(Q[rows.start:rows.stop], K, V, S_, blk, b_sel, s)
        np.testing.assert_allclose(o, np.transpose(ref[:, rows.start:rows.stop], (1, 0, 2)),
                                   rtol=1e-11, atol=1e-12)
    for i in (0, 17, 63):
        S_ = O.prefill_oracle_query_support(Q[i], K, i, s, k=N)
        o, _ = O.prefill_query_attend(Q[i], K, V, S_, s)
        np.testing.assert_allclose(o, ref[:, i], rtol=1e-11, atol=1e-12)
