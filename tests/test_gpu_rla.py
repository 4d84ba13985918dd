"""GPU parity of the residual linear attention tail ("SPLA", section 2.2)
against the float64 oracle: the global state built by sa_rla_state, and the
unselected-token terms sa_sparse_decode_rla forms by subtraction while it
computes the exact attention over the support."""

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
    """Exact attention identical to sa_sparse_decode; unselected-token terms
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
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
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
