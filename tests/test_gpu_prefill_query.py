"""GPU parity of per-query (b_sel = 1) prefill against the float64 oracle:
supports by the head-collapsed indexer (sa_select_prefill_topk, b_sel = 1) or
by the mean of the heads' probabilities (sa_select_prefill_topk_probs), and
attention of every query over its own list (sa_sparse_prefill_query)."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests import _support as S
from tests.test_gpu_prefill import oracle_kidx, prefill_shape

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def ops():
    from dynamic_sparse_attention_02_amd import ops as _ops
    return _ops


def _lib():
    from dynamic_sparse_attention_02_amd import _lib as L
    return L


def run_query_prefill(inp, kidx, k, probs=False, out_dtype=None):
    o = ops()
    L_ = _lib()
    shape = prefill_shape(inp)
    pages = o.make_pages(inp.page_table, None)
    cap = min(k + 1, inp.N)
    rows = inp.N * inp.H_kv
    idx = torch.full((rows, cap), -7, dtype=torch.int32, device="cuda")
    count = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    ws = o.alloc_workspace(o.workspace_size(L_.SA_OP_PREFILL_SELECT, shape, inp.N))
    sel = o.sa_select_prefill_topk_probs if probs else o.sa_select_prefill_topk
    sel(shape, pages, inp.N, inp.q, inp.w_q, kidx, inp.s_idx, 1, k, idx, count, ws)
    out = torch.full((inp.N, inp.H_q, inp.d), float("nan"), dtype=out_dtype or inp.dtype,
                     device="cuda")
    lse = torch.full((inp.N, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    ws_a = o.alloc_workspace(o.workspace_size(L_.SA_OP_PREFILL_QUERY, shape, cap))
    o.sa_sparse_prefill_query(shape, pages, inp.N, inp.q, inp.k_pool, inp.v_pool, idx, count,
                              inp.s_att, out, lse, ws_a)
    torch.cuda.synchronize()
    return idx, count, out, lse


def check_queries(inp, kt_rows, idx, count, out, lse, k, queries, groups, probs=False):
    tol = S.TOL[inp.dtype]
    n_diff = 0
    agg = "probs" if probs else "logits"
    for g in groups:
        hs = inp.heads(g)
        K = S.to_np(inp.keys(g))
        V = S.to_np(inp.values(g))
        wq = S.to_np(inp.w_q[hs])
        for i in queries:
            qi = S.to_np(inp.q[i, hs])
            x = O.prefill_query_scores(qi, wq, kt_rows[g], i, inp.s_idx, agg)
            core = O.select_topk(x, k)
            gsup = S.gpu_support(idx, count, i * inp.H_kv + g)
            n_diff += S.check_support(gsup, x, core, L=i + 1, k=k, n_window=1)
            assert i in gsup
            o_ref, l_ref = O.prefill_query_attend(qi, K, V, gsup, inp.s_att)
            go = S.to_np(out[i, hs])
            gl = lse[i, hs].cpu().numpy().astype(np.float64)
            assert S.max_abs(go, o_ref) <= tol, (i, g, S.max_abs(go, o_ref))
            assert S.max_abs(gl, l_ref) <= 1e-4 * max(1.0, np.abs(l_ref).max()), (i, g)
            if len(gsup) == len(O.with_sink_window(core, i + 1, 0, 1)) and \
                    set(gsup.tolist()) == set(O.with_sink_window(core, i + 1, 0, 1).tolist()):
                o2, _ = O.prefill_query_attend(qi, K, V, O.with_sink_window(core, i + 1, 0, 1),
                                               inp.s_att)
                assert S.max_abs(go, o2) <= tol
    return n_diff


@pytest.mark.parametrize("N,k,dtype,probs", [
    (700, 64, torch.bfloat16, False),
    (700, 64, torch.bfloat16, True),
    (333, 40, torch.float32, False),
    (333, 40, torch.float32, True),
    (150, 500, torch.bfloat16, False),     # k above every row: all causal keys
])
def test_query_prefill_matches_oracle(N, k, dtype, probs):
    inp = synth.make_prefill_custom(N=N, H_q=8, H_kv=2, d=128, dtype=dtype, device="cuda",
                                    seed=N + 3 * probs, n_hh=8)
    kidx, kt_rows = oracle_kidx(inp)
    idx, count, out, lse = run_query_prefill(inp, kidx, k, probs=probs)
    expect = np.minimum(np.arange(N) + 1, k + 1)  # top-k plus the own token (or all)
    cnt = count.view(N, inp.H_kv).cpu().numpy()
    for g in range(inp.H_kv):
        assert np.all((cnt[:, g] == expect) | (cnt[:, g] == expect - 1))
    queries = sorted(set([0, 1, 2, k - 1, k, k + 1, N // 2, N - 2, N - 1]) & set(range(N)))
    check_queries(inp, kt_rows, idx, count, out, lse, k, queries, range(inp.H_kv), probs=probs)


@pytest.mark.parametrize("H_q,H_kv,d", [(4, 4, 64), (16, 1, 128), (8, 4, 64)])
def test_query_prefill_group_sizes(H_q, H_kv, d):
    inp = synth.make_prefill_custom(N=300, H_q=H_q, H_kv=H_kv, d=d, dtype=torch.bfloat16,
                                    device="cuda", seed=H_q + 7 * H_kv, n_hh=4)
    kidx, kt_rows = oracle_kidx(inp)
    for probs in (False, True):
        idx, count, out, lse = run_query_prefill(inp, kidx, 32, probs=probs)
        check_queries(inp, kt_rows, idx, count, out, lse, 32, [0, 31, 32, 33, 150, 299],
                      range(inp.H_kv), probs=probs)


def test_query_prefill_dense_when_k_covers_everything():
    """k >= N: every query attends to all its causal keys: dense causal
    attention (torch SDPA in float64 on the CPU)."""
    inp = synth.make_prefill_custom(N=260, H_q=4, H_kv=1, d=128, dtype=torch.float32,
                                    device="cuda", seed=5, n_hh=3)
    kidx, _ = oracle_kidx(inp)
    idx, count, out, lse = run_query_prefill(inp, kidx, 1000, out_dtype=torch.float32)
    assert torch.equal(count.cpu(), torch.arange(1, 261, dtype=torch.int32))
    q = inp.q.double().cpu().permute(1, 0, 2)[None]
    K = inp.keys(0).double().cpu()[None, None]
    V = inp.values(0).double().cpu()[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=inp.s_att,
                                                           is_causal=True)[0].permute(1, 0, 2)
    assert S.max_abs(out.double().cpu().numpy(), ref.numpy()) <= 1e-5


def test_query_prefill_deterministic():
    inp = synth.make_prefill_custom(N=900, H_q=8, H_kv=2, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=9, n_hh=10)
    kidx, _ = oracle_kidx(inp)
    a = run_query_prefill(inp, kidx, 100, probs=True)
    b = run_query_prefill(inp, kidx, 100, probs=True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("probs", [False, True])
def test_query_prefill_32k_workload_sampled(probs):
    """The per-query 32K workload as the bench runs it (32/8 heads, d=128,
    bf16, top-2048 per query): sampled (query, group) rows against the
    oracle, early, boundary and late queries."""
    inp = synth.make_prefill_query32k(device="cuda")
    groups = [0, 5]
    kidx, kt_rows = oracle_kidx(inp, groups=groups)
    idx, count, out, lse = run_query_prefill(inp, kidx, inp.top_k, probs=probs)
    queries = [0, 2047, 2048, 2049, 9000, 20000, 32767]
    n_diff = check_queries(inp, kt_rows, idx, count, out, lse, inp.top_k, queries, groups,
                           probs=probs)
    print(f"prefill32k_query probs={probs}: tolerated support differences {n_diff}")


def test_query_prefill_long_tie_groups():
    """Per-query top-k over indexer keys drawn from three fixed vectors (long
    exact tie groups across the threshold): lists exactly the oracle's, ties
    lowest index first, the own token always kept."""
    from tests.test_gpu_prefill import quantised_kidx
    inp = synth.make_prefill_custom(N=6000, H_q=4, H_kv=1, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=23, n_hh=4)
    kidx, kt_rows = quantised_kidx(inp, 5, probs=(0.7, 0.2, 0.1))
    k = 700
    idx, count, out, lse = run_query_prefill(inp, kidx, k)
    queries = [0, 699, 700, 2500, 5999]
    check_queries(inp, kt_rows, idx, count, out, lse, k, queries, [0])
    wq = S.to_np(inp.w_q[inp.heads(0)])
    for i in queries:
        x = O.prefill_query_scores(S.to_np(inp.q[i, inp.heads(0)]), wq, kt_rows[0], i, inp.s_idx, "logits")
        expect = O.with_sink_window(O.select_topk(x, k), i + 1, 0, 1)
        assert S.gpu_support(idx, count, i).tolist() == expect.tolist(), i
