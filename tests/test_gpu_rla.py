"""GPU parity of the residual linear attention tail ("SPLA", section 2.2)
against the float64 oracle: the global state built by sa_rla_state, and the
unselected-token terms sa_sparse_decode_rla and sa_decode_step_rla form by
subtraction while they compute the exact attention over the support."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests import _support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def ops():
    from dynamic_sparse_attention_02_amd import ops as _ops
    return _ops


def _inputs(lens, dtype, d, G=4, H_kv=2, seed=0):
    return synth.make_decode_custom(B=len(lens), H_q=G * H_kv, H_kv=H_kv, d=d, seq_lens=lens,
                                    dtype=dtype, device="cuda", seed=seed, hh_frac=0.01,
                                    alpha=10.0, shuffle=True)


def gpu_state(inp, first=0, lens=None, state=None):
    o = ops()
    shape = S.shape_of(inp)
    lens_t = inp.seq_lens_tensor() if lens is None else torch.tensor(lens, dtype=torch.int32,
                                                                      device="cuda")
    pages = o.make_pages(inp.page_table, lens_t)
    if state is None:
        state = torch.zeros((inp.B, inp.H_kv, inp.d + 1, inp.d), dtype=torch.float32,
                            device="cuda")
    o.sa_rla_state(shape, pages, inp.k_pool, inp.v_pool, first, state)
    torch.cuda.synchronize()
    return state


def oracle_state(inp):
    st = np.zeros((inp.B, inp.H_kv, inp.d + 1, inp.d))
    for b in range(inp.B):
        for g in range(inp.H_kv):
            if inp.seq_lens[b] == 0:
                continue
            Sm, z = O.rla_state(S.to_np(inp.seq_keys(b, g)), S.to_np(inp.seq_values(b, g)))
            st[b, g, :inp.d] = Sm
            st[b, g, inp.d] = z
    return st


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_rla_state_matches_oracle(dtype, d):
    inp = _inputs([1000, 130, 0], dtype, d, seed=3)
    got = gpu_state(inp).cpu().numpy().astype(np.float64)
    ref = oracle_state(inp)
    np.testing.assert_allclose(got, ref, rtol=2e-5, atol=2e-5 * np.abs(ref).max())
    assert np.all(got[2] == 0)  # empty sequence adds nothing


def test_rla_state_extends_in_place():
    """Building [0, 600) then adding [600, L) equals one build over [0, L)."""
    inp = _inputs([1000, 700], torch.bfloat16, 128, seed=4)
    full = gpu_state(inp).cpu().numpy()
    part = gpu_state(inp, lens=[600, 600])
    both = gpu_state(inp, first=600, state=part).cpu().numpy()
    np.testing.assert_allclose(both, full, rtol=1e-5, atol=1e-5 * np.abs(full).max())


def _unselected_scale(q, K, V):
    """Magnitudes the subtraction works at: sum over all tokens of the
    weights and of weight * |v| (float64)."""
    w = O.rla_feature(q) @ O.rla_feature(K).T   # [G, n]
    return w.sum(axis=1), w @ np.abs(V)         # [G], [G, d]


@pytest.mark.parametrize("rule,dtype,d", [({"p": 0.9}, torch.bfloat16, 128), ({"k": 50}, torch.float32, 64),
                                          ({"p": 1.0}, torch.bfloat16, 128)])
def test_decode_rla_matches_oracle(rule, dtype, d):
    """Exact attention equal to sa_sparse_decode's; unselected-token terms
    (numerator and denominator) against the oracle's direct sums over the
    tokens outside the GPU's support, given the oracle's state."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    inp = _inputs([3000, 0, 777], dtype, d, seed=5)
    kidx = S.oracle_kidx_pool(inp)
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    cap = max(inp.seq_lens)
    x, idx, count, out, lse = S.empty_like_outputs(inp, cap)
    ws_i = o.alloc_workspace(o.workspace_size(L.SA_OP_INDEX_SCORES, shape, 0))
    ws_s = o.alloc_workspace(o.workspace_size(L.SA_OP_SELECT, shape, cap))
    o.sa_index_scores(shape, pages, inp.q, inp.w_q, kidx, inp.s_idx, x, ws_i)
    p = S.f32(rule["p"]) if "p" in rule else None
    if p is not None:
        o.sa_select_topp(shape, pages, x, p, 4, 16, idx, count, ws_s)
    else:
        o.sa_select_topk(shape, pages, x, rule["k"], 1, 4, 16, idx, count, ws_s)
    state = torch.from_numpy(oracle_state(inp)).float().cuda()
    ws_d = o.alloc_workspace(o.workspace_size(L.SA_OP_SPARSE_DECODE, shape, cap))
    ws_r = o.alloc_workspace(o.workspace_size(L.SA_OP_SPARSE_DECODE_RLA, shape, cap))
    o.sa_sparse_decode(shape, pages, inp.q, inp.k_pool, inp.v_pool, idx, count, inp.s_att, out,
                       lse, ws_d)
    out2, lse2 = torch.full_like(out, float("nan")), torch.full_like(lse, float("nan"))
    num = torch.full((inp.B, inp.H_q, inp.d), float("nan"), dtype=torch.float32, device="cuda")
    den = torch.full((inp.B, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    o.sa_sparse_decode_rla(shape, pages, inp.q, inp.k_pool, inp.v_pool, idx, count, inp.s_att,
                           out2, lse2, state, num, den, ws_r)
    torch.cuda.synchronize()
    # same attention as sa_sparse_decode (which may run it on the matrix cores:
    # equal within rounding)
    torch.testing.assert_close(out, out2, rtol=1e-4, atol=1e-5)
    torch.testing.assert_close(lse, lse2, rtol=0, atol=1e-4)
    for b in range(inp.B):
        for g in range(inp.H_kv):
            hs = inp.heads(g)
            gn, gd = S.to_np(num[b, hs]), S.to_np(den[b, hs])
            if inp.seq_lens[b] == 0:
                assert np.all(gn == 0) and np.all(gd == 0)
                continue
            q = S.to_np(inp.q[b, hs])
            K = S.to_np(inp.seq_keys(b, g))
            V = S.to_np(inp.seq_values(b, g))
            sup = S.gpu_support(idx, count, b * inp.H_kv + g)
            rn, rd = O.rla_unselected(q, K, V, sup)
            wsum, wabs = _unselected_scale(q, K, V)
            assert np.all(np.abs(gd - rd) <= 3e-5 * wsum), (b, g, gd, rd)
            assert np.all(np.abs(gn - rn) <= 3e-5 * wabs.max(axis=1, keepdims=True)), (b, g)
            if len(sup) == inp.seq_lens[b]:  # nothing left out: only rounding remains
                assert np.all(np.abs(gd) <= 3e-5 * wsum)


def test_rla_decode64k_full_size():
    """The 64K decode workload with the residual linear attention tail, as
    the bench runs it: the state of the whole 65536-token cache by
    sa_rla_state, then indexer scores, top-p 0.9 with sink 4 and window 512,
    and sa_sparse_decode_rla; every group against the oracle (state element
    by element, unselected-token terms against the direct sums)."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    inp = synth.make_decode64k(device="cpu").to("cuda")
    kidx = S.oracle_kidx_pool(inp)
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    cap = max(inp.seq_lens)
    state = gpu_state(inp)
    st = state.cpu().numpy().astype(np.float64)
    x, idx, count, out, lse = S.empty_like_outputs(inp, cap)
    out = out.to(torch.bfloat16)
    ws_i = o.alloc_workspace(o.workspace_size(L.SA_OP_INDEX_SCORES, shape, 0))
    ws_s = o.alloc_workspace(o.workspace_size(L.SA_OP_SELECT, shape, cap))
    ws_r = o.alloc_workspace(o.workspace_size(L.SA_OP_SPARSE_DECODE_RLA, shape, cap))
    p = S.f32(0.9)
    o.sa_index_scores(shape, pages, inp.q, inp.w_q, kidx, inp.s_idx, x, ws_i)
    o.sa_select_topp(shape, pages, x, p, 4, 512, idx, count, ws_s)
    num = torch.full((inp.B, inp.H_q, inp.d), float("nan"), dtype=torch.float32, device="cuda")
    den = torch.full((inp.B, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    o.sa_sparse_decode_rla(shape, pages, inp.q, inp.k_pool, inp.v_pool, idx, count, inp.s_att,
                           out, lse, state, num, den, ws_r)
    torch.cuda.synchronize()
    worst = 0.0
    for g in range(inp.H_kv):
        hs = inp.heads(g)
        K = S.to_np(inp.seq_keys(0, g))
        V = S.to_np(inp.seq_values(0, g))
        # state: each term carries the fp32 exponential's relative error (a
        # few 1e-7 for these keys) and the compensated sum adds a few fp32
        # rounding units, so an element stays within 2e-6 of the sum of the
        # magnitudes of its terms, however long the cache
        Sm, z = O.rla_state(K, V)
        mag = O.rla_feature(K).T @ np.abs(V)
        assert np.all(np.abs(st[0, g, :inp.d] - Sm) <= 2e-6 * mag + 1e-30), g
        assert np.all(np.abs(st[0, g, inp.d] - z) <= 2e-6 * z), g
        q = S.to_np(inp.q[0, hs])
        sup = S.gpu_support(idx, count, g)
        rn, rd = O.rla_unselected(q, K, V, sup)
        wsum, wabs = _unselected_scale(q, K, V)
        gn, gd = S.to_np(num[0, hs]), S.to_np(den[0, hs])
        assert np.all(np.abs(gd - rd) <= 3e-5 * wsum), (g, gd, rd)
        assert np.all(np.abs(gn - rn) <= 3e-5 * wabs.max(axis=1, keepdims=True)), g
        worst = max(worst, float((np.abs(gd - rd) / wsum).max()))
        o_ref, _ = O.attend(q, K[sup], V[sup], inp.s_att)
        assert S.max_abs(S.to_np(out[0, hs]), o_ref) <= 2e-2, g
    print(f"rla decode64k: worst denominator error {worst:.2e} of the summed weights")


def _check_unselected(inp, idx, count, num, den, tol=3e-5):
    """Every group's unselected-token terms against the oracle's direct sums
    over the tokens outside the GPU's support; returns the worst denominator
    error relative to the summed weights."""
    worst = 0.0
    for b in range(inp.B):
        for g in range(inp.H_kv):
            hs = inp.heads(g)
            gn, gd = S.to_np(num[b, hs]), S.to_np(den[b, hs])
            if inp.seq_lens[b] == 0:
                assert np.all(gn == 0) and np.all(gd == 0), (b, g)
                continue
            q = S.to_np(inp.q[b, hs])
            K = S.to_np(inp.seq_keys(b, g))
            V = S.to_np(inp.seq_values(b, g))
            sup = S.gpu_support(idx, count, b * inp.H_kv + g)
            rn, rd = O.rla_unselected(q, K, V, sup)
            wsum, wabs = _unselected_scale(q, K, V)
            assert np.all(np.abs(gd - rd) <= tol * wsum), (b, g, gd, rd)
            assert np.all(np.abs(gn - rn) <= tol * wabs.max(axis=1, keepdims=True)), (b, g)
            worst = max(worst, float((np.abs(gd - rd) / wsum).max()))
    return worst


def _same(a, b):
    """Bit-for-bit equal, NaN (never written) matching NaN."""
    torch.testing.assert_close(a, b, rtol=0, atol=0, equal_nan=True)


def _step(o, inp, kidx, ws, p, top_k, n_sink, n_window, state=None, out_dtype=None):
    """sa_decode_step (state None) or sa_decode_step_rla; returns x, idx,
    count, out, lse (and num, den)."""
    shape = S.shape_of(inp)
    pages = o.make_pages(inp.page_table, inp.seq_lens_tensor())
    cap = max(inp.seq_lens)
    x, idx, count, out, lse = S.empty_like_outputs(inp, cap)
    if out_dtype is not None:
        out = out.to(out_dtype)
    if state is None:
        o.sa_decode_step(shape, pages, inp.q, inp.w_q, kidx, inp.k_pool, inp.v_pool, inp.s_idx,
                         inp.s_att, p, top_k, n_sink, n_window, x, idx, count, out, lse, ws)
        torch.cuda.synchronize()
        return x, idx, count, out, lse
    num = torch.full((inp.B, inp.H_q, inp.d), float("nan"), dtype=torch.float32, device="cuda")
    den = torch.full((inp.B, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    o.sa_decode_step_rla(shape, pages, inp.q, inp.w_q, kidx, inp.k_pool, inp.v_pool, inp.s_idx,
                         inp.s_att, p, top_k, n_sink, n_window, x, idx, count, out, lse, state,
                         num, den, ws)
    torch.cuda.synchronize()
    return x, idx, count, out, lse, num, den


# (lengths, kv heads, group size, dtype, head dim): the first four take the
# persistent single launch (few rows, bf16: G = 4, 8, 16 and d = 64), the
# last two the separate calls (fp32; more than 16 rows)
_STEP_CASES = [([3000, 0, 777], 2, 4, torch.bfloat16, 128),
               ([2500, 64], 2, 8, torch.bfloat16, 128),
               ([1900], 1, 16, torch.bfloat16, 128),
               ([1200, 333], 4, 4, torch.bfloat16, 64),
               ([1500, 0, 640], 2, 4, torch.float32, 64),
               ([900, 1300, 70], 6, 4, torch.bfloat16, 128)]


@pytest.mark.parametrize("case", range(len(_STEP_CASES)))
def test_decode_step_rla_matches_step_and_oracle(case):
    """sa_decode_step_rla: the scores, lists, counts, outputs and lse of
    sa_decode_step (identical where both run the same launches), and the
    unselected-token terms against the oracle; one workspace of the RLA op's
    size serves both entry points, called alternately."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    lens, H_kv, G, dtype, d = _STEP_CASES[case]
    inp = _inputs(lens, dtype, d, G=G, H_kv=H_kv, seed=40 + case)
    kidx = S.oracle_kidx_pool(inp)
    shape = S.shape_of(inp)
    cap = max(inp.seq_lens)
    state = torch.from_numpy(oracle_state(inp)).float().cuda()
    ws = o.alloc_workspace(o.workspace_size(L.SA_OP_DECODE_STEP_RLA, shape, cap))
    assert o.workspace_size(L.SA_OP_DECODE_STEP_RLA, shape, cap) > \
        o.workspace_size(L.SA_OP_DECODE_STEP, shape, cap)
    p = S.f32(0.9)
    ref = _step(o, inp, kidx, ws, p, 0, 4, 16)
    got = _step(o, inp, kidx, ws, p, 0, 4, 16, state=state)
    again = _step(o, inp, kidx, ws, p, 0, 4, 16)
    for r, a_ in zip(ref, again):
        _same(r, a_)  # the shared workspace leaves the plain step unchanged
    # same scores and lists whichever path runs (same arithmetic)
    assert torch.equal(ref[1], got[1]) and torch.equal(ref[2], got[2])
    for b in range(inp.B):
        rs = slice(b * H_kv, (b + 1) * H_kv)
        assert torch.equal(ref[0][rs, :lens[b]], got[0][rs, :lens[b]])
    # the attention may be split over a different number of workgroups:
    # equal within rounding
    torch.testing.assert_close(ref[3], got[3], rtol=0, atol=1e-5)
    torch.testing.assert_close(ref[4], got[4], rtol=0, atol=1e-4)  # -inf for empty rows
    _check_unselected(inp, got[1], got[2], got[5], got[6])


def test_decode_step_rla_decode64k_full_size():
    """The 64K decode workload through sa_decode_step_rla as the bench times
    it (persistent launch with the residual tail): lists and outputs equal to
    sa_decode_step's, unselected-token terms of every group against the
    oracle given the GPU-built state."""
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    inp = synth.make_decode64k(device="cpu").to("cuda")
    kidx = S.oracle_kidx_pool(inp)
    shape = S.shape_of(inp)
    cap = max(inp.seq_lens)
    state = gpu_state(inp)
    ws = o.alloc_workspace(o.workspace_size(L.SA_OP_DECODE_STEP_RLA, shape, cap))
    p = S.f32(0.9)
    ref = _step(o, inp, kidx, ws, p, 0, 4, 512, out_dtype=torch.bfloat16)
    got = _step(o, inp, kidx, ws, p, 0, 4, 512, state=state, out_dtype=torch.bfloat16)
    for r, g_ in zip(ref[:3], got[:3]):  # scores, lists, counts
        _same(r, g_)
    # outputs equal within rounding (bf16: a unit in the last place)
    torch.testing.assert_close(ref[3].float(), got[3].float(), rtol=8e-3, atol=1e-5)
    torch.testing.assert_close(ref[4], got[4], rtol=0, atol=1e-4)
    assert np.all(S.to_np(got[2]) > 0)
    worst = _check_unselected(inp, got[1], got[2], got[5], got[6])
    print(f"decode step rla 64k: worst denominator error {worst:.2e} of the summed weights")
