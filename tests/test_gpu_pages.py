"""GPU parity of the page-granular decode path against the float64 oracle:
page statistics (mean, diagonal variance), Taylor page scores, top-k page
selection expanded to tokens, and sparse decode over those tokens; the 1M-token
page workload at full size."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests import _support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PAGE = synth.PAGE


def ops():
    from dynamic_sparse_attention_02_amd import ops as _ops
    return _ops


def seq_pages(inp, b):
    L = inp.seq_lens[b]
    npg = (L + PAGE - 1) // PAGE
    n_valid = [min(PAGE, L - p * PAGE) for p in range(npg)]
    return inp.page_table[b, :npg].long(), n_valid


def oracle_stats(inp, b, g):
    """Oracle page statistics of sequence b, group g (float64)."""
    return O.page_stats(S.to_np(inp.seq_keys(b, g)), PAGE)


def oracle_stats_pool(inp, groups=None):
    """Statistics pool [n_pages][H_kv][2][d] holding the oracle's values,
    rounded once to the cache dtype; also returns the float64 values as read
    back from that pool, per (b, g)."""
    pool = torch.zeros((inp.n_pages, inp.H_kv, 2, inp.d), dtype=inp.dtype, device=inp.device)
    rows = {}
    groups = range(inp.H_kv) if groups is None else groups
    for b in range(inp.B):
        if inp.seq_lens[b] == 0:
            continue
        pids, _ = seq_pages(inp, b)
        for g in groups:
            mean, var, n = oracle_stats(inp, b, g)
            st = np.stack([S.store_round(mean, inp.dtype), S.store_round(var, inp.dtype)], axis=1)
            pool[pids.to(inp.device), g] = torch.from_numpy(st).to(inp.dtype).to(inp.device)
            rows[(b, g)] = (st[:, 0], st[:, 1], n)
    return pool, rows


def bf16_ulp(v):
    """One unit in the last place of bfloat16 at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_page_stats_matches_oracle(dtype):
    """Every page of ragged sequences (full pages, a 40-token and a 2-token
    tail, a single-token sequence), all groups."""
    o = ops()
    inp = synth.make_decode_custom(B=3, H_q=8, H_kv=2, d=128, seq_lens=[1000, 130, 1],
                                   dtype=dtype, device="cuda", seed=21, hh_frac=0.01, alpha=10.0,
                                   shuffle=True)
    shape = S.shape_of(inp)
    pid, nval = [], []
    for b in range(inp.B):
        p, n = seq_pages(inp, b)
        pid += p.tolist()
        nval += n
    pid_t = torch.tensor(pid, dtype=torch.int32, device="cuda")
    nval_t = torch.tensor(nval, dtype=torch.int32, device="cuda")
    stats = torch.full((inp.n_pages, inp.H_kv, 2, inp.d), float("nan"), dtype=dtype, device="cuda")
    o.sa_page_stats(shape, inp.k_pool, pid_t, nval_t, stats)
    torch.cuda.synchronize()
    for b in range(inp.B):
        pids, _ = seq_pages(inp, b)
        for g in range(inp.H_kv):
            mean, var, n = oracle_stats(inp, b, g)
            got = S.to_np(stats[pids.cuda(), g])
            for j, ref in ((0, mean), (1, var)):
                if dtype == torch.float32:
                    tol = 1e-5 * np.maximum(1.0, np.abs(ref))
                else:  # fp32 accumulation, one rounding to bf16: at most 1 ulp apart
                    tol = bf16_ulp(ref) + 1e-30
                err = np.abs(got[:, j] - ref)
                assert np.all(err <= tol), (b, g, j, float(err.max()))
            if n[-1] == 1:
                assert np.all(got[-1, 1] == 0.0)  # one token: zero variance


@pytest.mark.parametrize("G,d,dtype", [(1, 128, torch.float32), (4, 128, torch.bfloat16),
                                       (8, 128, torch.bfloat16), (16, 128, torch.bfloat16),
                                       (2, 64, torch.bfloat16), (16, 64, torch.float32)])
def test_page_scores_matches_oracle(G, d, dtype):
    """Taylor page scores of every page of ragged rows (an empty row is left
    untouched) from oracle statistics stored in the cache dtype."""
    o = ops()
    inp = synth.make_decode_custom(B=4, H_q=2 * G, H_kv=2, d=d, seq_lens=[5000, 0, 100, 64],
                                   dtype=dtype, device="cuda", seed=30 + G, hh_frac=0.01,
                                   alpha=10.0, shuffle=True)
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    pool, rows = oracle_stats_pool(inp)
    x = torch.full((inp.B * inp.H_kv, inp.max_pages), float("nan"), dtype=torch.float32,
                   device="cuda")
    o.sa_page_scores(shape, pages, inp.q, pool, inp.s_att, x)
    torch.cuda.synchronize()
    for b in range(inp.B):
        for g in range(inp.H_kv):
            r = b * inp.H_kv + g
            if inp.seq_lens[b] == 0:
                assert torch.all(torch.isnan(x[r]))
                continue
            mean, var, n = rows[(b, g)]
            ref = O.page_scores(S.to_np(inp.q[b, inp.heads(g)]), mean, var, n, inp.s_att, PAGE)
            got = x[r, :len(n)].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(ref).max()))
            assert torch.all(torch.isnan(x[r, len(n):]))


def run_page_decode(inp, pool, k_pages, out_dtype=torch.float32):
    """sa_page_scores, sa_select_topk over pages, sa_sparse_decode."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    rows = inp.B * inp.H_kv
    cap = min(k_pages * PAGE, max(max(inp.seq_lens), 1))
    x = torch.full((rows, inp.max_pages), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((rows, cap), -7, dtype=torch.int32, device="cuda")
    count = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((inp.B, inp.H_q, inp.d), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((inp.B, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    ws_s = o.alloc_workspace(o.workspace_size(L.SA_OP_SELECT, shape, inp.max_pages))
    ws_d = o.alloc_workspace(o.workspace_size(L.SA_OP_SPARSE_DECODE, shape, cap))
    o.sa_page_scores(shape, pages, inp.q, pool, inp.s_att, x)
    o.sa_select_topk(shape, pages, x, k_pages, PAGE, 0, 0, idx, count, ws_s)
    o.sa_sparse_decode(shape, pages, inp.q, inp.k_pool, inp.v_pool, idx, count, inp.s_att, out,
                       lse, ws_d)
    torch.cuda.synchronize()
    return x, idx, count, out, lse


def check_page_rows(inp, rows, x, idx, count, out, lse, k_pages, groups, tol):
    n_diff = 0
    for b in range(inp.B):
        L = inp.seq_lens[b]
        for g in groups:
            r = b * inp.H_kv + g
            hs = inp.heads(g)
            if L == 0:
                assert int(count[r]) == 0
                assert torch.all(out[b, hs] == 0) and torch.all(torch.isneginf(lse[b, hs]))
                continue
            mean, var, n = rows[(b, g)]
            q = S.to_np(inp.q[b, hs])
            xo = O.page_scores(q, mean, var, n, inp.s_att, PAGE)
            core = O.select_topk(xo, k_pages)
            toks = S.gpu_support(idx, count, r)
            gp = np.unique(toks // PAGE)
            # the token list is exactly the expansion of its pages
            assert toks.tolist() == O.expand_pages(gp, L, PAGE).tolist()
            n_diff += S.check_support(gp, xo, core, L=len(n), k=k_pages)
            K = S.to_np(inp.seq_keys(b, g))
            V = S.to_np(inp.seq_values(b, g))
            o_ref, l_ref = O.attend(q, K[toks], V[toks], inp.s_att)
            assert S.max_abs(S.to_np(out[b, hs]), o_ref) <= tol, (b, g)
            assert S.max_abs(lse[b, hs].cpu().numpy(), l_ref) <= max(tol, 1e-5) * max(
                1.0, np.abs(l_ref).max())
            if np.array_equal(gp, core):
                ref = O.decode_row_pages(q, mean, var, n, K, V, s_att=inp.s_att, k_pages=k_pages,
                                         page_size=PAGE)
                assert S.max_abs(S.to_np(out[b, hs]), ref["o"]) <= tol
    return n_diff


@pytest.mark.parametrize("k_pages", [1, 6, 40])
def test_page_decode_ragged(k_pages):
    """Top-k pages on ragged rows (partial last pages, an empty row, a row
    with fewer pages than k) through decode, fp32 and bf16."""
    for dtype in (torch.float32, torch.bfloat16):
        inp = synth.make_decode_custom(B=4, H_q=16, H_kv=2, d=128,
                                       seq_lens=[64 * 40 + 17, 0, 64 * 3, 2500], dtype=dtype,
                                       device="cuda", seed=k_pages, hh_frac=0.01, alpha=10.0,
                                       shuffle=True)
        pool, rows = oracle_stats_pool(inp)
        x, idx, count, out, lse = run_page_decode(inp, pool, k_pages)
        check_page_rows(inp, rows, x, idx, count, out, lse, k_pages, range(inp.H_kv),
                        S.TOL[dtype])


def test_decode1m_workload():
    """The 1M-token page workload (one sequence, 32/4 heads, d=128, bf16,
    16384 pages, top-32 pages): GPU page statistics against the oracle on a
    seeded sample of pages, then page scores, selection and decode from the
    oracle's statistics against the oracle, every group; the planted pages
    are reported."""
    o = ops()
    inp = synth.make_decode1m(device="cuda")
    k_pages = inp.select["k_pages"]
    shape = S.shape_of(inp)
    n_pages = inp.max_pages
    pid = inp.page_table[0].contiguous()
    nval = torch.full((n_pages,), PAGE, dtype=torch.int32, device="cuda")
    stats = torch.empty((inp.n_pages, inp.H_kv, 2, inp.d), dtype=inp.dtype, device="cuda")
    o.sa_page_stats(shape, inp.k_pool, pid, nval, stats)
    torch.cuda.synchronize()
    pool, rows = oracle_stats_pool(inp)
    rng = np.random.default_rng(11)
    for g in range(inp.H_kv):
        mean, var, _ = rows[(0, g)]
        sample = np.union1d(rng.choice(n_pages, 256, replace=False),
                            inp.planted[(0, g)].numpy())
        got = S.to_np(stats[pid[torch.from_numpy(sample).cuda()].long(), g])
        # the pool holds round(oracle); the GPU's fp32 statistic rounds to
        # within one bf16 ulp of it
        for j, ref in ((0, mean[sample]), (1, var[sample])):
            assert np.all(np.abs(got[:, j] - ref) <= 2 * bf16_ulp(ref) + 1e-30), (g, j)
    x, idx, count, out, lse = run_page_decode(inp, pool, k_pages, out_dtype=torch.bfloat16)
    n_diff = check_page_rows(inp, rows, x, idx, count, out, lse, k_pages, range(inp.H_kv),
                             S.TOL[torch.bfloat16])
    found = []
    for g in range(inp.H_kv):
        gp = set((S.gpu_support(idx, count, g) // PAGE).tolist())
        found.append(len(gp & set(inp.planted[(0, g)].tolist())))
    print(f"decode1m: planted pages selected per group {found} of 16, "
          f"tolerated support differences {n_diff}")


def run_step_pages(inp, pool, k_pages, out_dtype=torch.float32, ws=None):
    """sa_decode_step_pages: the whole page-level step in one call."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    rows = inp.B * inp.H_kv
    cap = min(k_pages * PAGE, max(max(inp.seq_lens), 1))
    x = torch.full((rows, inp.max_pages), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((rows, cap), -7, dtype=torch.int32, device="cuda")
    count = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((inp.B, inp.H_q, inp.d), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((inp.B, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = o.alloc_workspace(o.workspace_size(L.SA_OP_DECODE_STEP_PAGES, shape, cap))
    o.sa_decode_step_pages(shape, pages, inp.q, pool, inp.k_pool, inp.v_pool, inp.s_att, k_pages,
                           x, idx, count, out, lse, ws)
    torch.cuda.synchronize()
    return x, idx, count, out, lse


def assert_same_step(inp, a, b, tol):
    """Same page scores, index lists and counts; outputs within tol (the two
    paths sum the softmax in different orders)."""
    xa, ia, ca, oa, la = a
    xb, ib, cb, ob, lb = b
    for r in range(inp.B * inp.H_kv):
        L = inp.seq_lens[r // inp.H_kv]
        npg = (L + PAGE - 1) // PAGE
        assert torch.equal(xa[r, :npg], xb[r, :npg]), r
    assert torch.equal(ca, cb)
    assert torch.equal(ia, ib)
    assert S.max_abs(S.to_np(oa), S.to_np(ob)) <= tol
    fin = torch.isfinite(lb)
    assert torch.equal(fin, torch.isfinite(la))
    assert S.max_abs(la[fin].cpu().numpy(), lb[fin].cpu().numpy()) <= max(tol, 1e-5) * max(
        1.0, float(lb[fin].abs().max()) if fin.any() else 1.0)


@pytest.mark.parametrize("G,d,k_pages,seq_lens,hkv", [
    (4, 128, 6, [64 * 40 + 17, 0, 64 * 3, 2500], 2),
    (8, 128, 32, [64 * 700 + 1, 64 * 31, 64 * 500], 2),
    (16, 128, 1, [100000, 65], 2),
    (8, 64, 17, [64 * 900, 64 * 2000 + 63], 2),
    (8, 128, 20, [64 * 3000 + 5], 1),
])
def test_decode_step_pages_fused_matches_calls(G, d, k_pages, seq_lens, hkv):
    """The one-launch page-level step (bf16, few rows, top-k <= 32 pages)
    against the three separate calls and against the oracle: ragged rows with
    partial last pages, an empty row, rows with fewer pages than k, and one
    row served by every compute unit."""
    inp = synth.make_decode_custom(B=len(seq_lens), H_q=hkv * G, H_kv=hkv, d=d, seq_lens=seq_lens,
                                   dtype=torch.bfloat16, device="cuda", seed=40 + G + k_pages,
                                   hh_frac=0.01, alpha=10.0, shuffle=True)
    pool, rows = oracle_stats_pool(inp)
    tol = S.TOL[torch.bfloat16]
    ref = run_page_decode(inp, pool, k_pages)
    got = run_step_pages(inp, pool, k_pages)
    assert_same_step(inp, got, ref, tol)
    check_page_rows(inp, rows, *got, k_pages, range(inp.H_kv), tol)


@pytest.mark.parametrize("dtype,G,k_pages", [(torch.float32, 8, 6), (torch.bfloat16, 2, 6),
                                             (torch.bfloat16, 8, 40)])
def test_decode_step_pages_separate_path(dtype, G, k_pages):
    """Problems outside the one-launch plan (fp32, group size 2, more than 32
    pages) run as the three calls, with the same results."""
    inp = synth.make_decode_custom(B=3, H_q=2 * G, H_kv=2, d=128,
                                   seq_lens=[64 * 60 + 5, 64 * 3, 3000], dtype=dtype,
                                   device="cuda", seed=60 + G, hh_frac=0.01, alpha=10.0,
                                   shuffle=True)
    pool, rows = oracle_stats_pool(inp)
    ref = run_page_decode(inp, pool, k_pages)
    got = run_step_pages(inp, pool, k_pages)
    assert_same_step(inp, got, ref, S.TOL[dtype])
    check_page_rows(inp, rows, *got, k_pages, range(inp.H_kv), S.TOL[dtype])


@pytest.mark.parametrize("hkv,lens", [(2, [64 * 3000 + 9, 64 * 777]), (1, [64 * 3000 + 9])])
def test_decode_step_pages_ties(hkv, lens):
    """Exact ties spread over workgroups (four rows, or one row served by
    every compute unit): every 100th page of a row has zero
    mean and unit variance, every other page zero statistics, so the scores
    take two values (and the length term of a partial last page).  Row 0 has
    30 tied high pages for 20 places: the 20 lowest indices win; row 1 has 8
    high pages and 12 places among the tied low pages.  Two calls on one
    workspace, both equal to the three separate calls."""
    from dynamic_sparse_attention_02_amd import _lib as L
    o = ops()
    inp = synth.make_decode_custom(B=len(lens), H_q=8 * hkv, H_kv=hkv, d=128, seq_lens=lens,
                                   dtype=torch.bfloat16, device="cuda", seed=71, shuffle=True)
    pool = torch.zeros((inp.n_pages, inp.H_kv, 2, inp.d), dtype=inp.dtype, device="cuda")
    for b in range(inp.B):
        pids, _ = seq_pages(inp, b)
        pool[pids[::100].cuda(), :, 1] = 1.0
    k_pages = 20
    shape = S.shape_of(inp)
    ws = o.alloc_workspace(o.workspace_size(L.SA_OP_DECODE_STEP_PAGES, shape, k_pages * PAGE))
    ref = run_page_decode(inp, pool, k_pages)
    want = {0: list(range(0, 2000, 100)),
            1: sorted(list(range(0, 777, 100)) + list(range(1, 13)))}
    for _ in range(2):
        got = run_step_pages(inp, pool, k_pages, ws=ws)
        assert_same_step(inp, got, ref, S.TOL[torch.bfloat16])
        idx, count = got[1], got[2]
        for r in range(inp.B * inp.H_kv):
            b = r // inp.H_kv
            toks = S.gpu_support(idx, count, r)
            assert toks.tolist() == O.expand_pages(np.array(want[b]), inp.seq_lens[b],
                                                   PAGE).tolist(), r


def test_decode_step_pages_decode1m():
    """The 1M-token page workload through the one-launch step: the same
    scores, lists and counts as the three calls and outputs within the bf16
    bound, twice on one workspace; then against the oracle."""
    from dynamic_sparse_attention_02_amd import _lib as L
    o = ops()
    inp = synth.make_decode1m(device="cuda")
    k_pages = inp.select["k_pages"]
    pool, rows = oracle_stats_pool(inp)
    shape = S.shape_of(inp)
    ws = o.alloc_workspace(o.workspace_size(L.SA_OP_DECODE_STEP_PAGES, shape, k_pages * PAGE))
    ref = run_page_decode(inp, pool, k_pages, out_dtype=torch.bfloat16)
    for _ in range(2):
        got = run_step_pages(inp, pool, k_pages, out_dtype=torch.bfloat16, ws=ws)
        assert_same_step(inp, got, ref, S.TOL[torch.bfloat16])
    check_page_rows(inp, rows, *got, k_pages, range(inp.H_kv), S.TOL[torch.bfloat16])
