"""GPU parity of the causal block-sparse prefill against the float64 oracle:
block supports (top-k over earlier blocks' keys, b_sel = 64) and MFMA
attention over support + causal diagonal block."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests import _support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

B_SEL = 64


def ops():
    from dynamic_sparse_attention_02_amd import ops as _ops
    return _ops


def prefill_shape(inp):
    o = ops()
    return o.make_shape(batch=1, n_q_heads=inp.H_q, n_kv_heads=inp.H_kv, head_dim=inp.d,
                        max_pages=inp.page_table.shape[1], max_len=inp.N,
                        n_pool_pages=inp.k_pool.shape[0])


def oracle_kidx(inp, groups=None):
    """Oracle indexer keys per group (rounded to the cache dtype) and the pool."""
    rows = {}
    pool = torch.zeros((inp.k_pool.shape[0], inp.H_kv, 64, 16), dtype=inp.dtype, device=inp.device)
    for g in range(inp.H_kv):
        K = S.to_np(inp.keys(g))
        kt = S.store_round(O.indexer_keys(K, S.to_np(inp.w_k[g])), inp.dtype)
        if groups is None or g in groups:
            rows[g] = kt
        full = torch.zeros((pool.shape[0] * 64, 16), dtype=inp.dtype)
        full[: inp.N] = torch.from_numpy(kt).to(inp.dtype)
        pool[:, g] = full.view(pool.shape[0], 64, 16).to(inp.device)
    return pool, rows


def run_prefill(inp, kidx, k, out_dtype=torch.bfloat16):
    o = ops()
    from dynamic_sparse_attention_02_amd import _lib as L
    shape = prefill_shape(inp)
    pages = o.make_pages(inp.page_table, None)
    nblk = inp.n_blocks
    cap = min(k, inp.N)
    idx = torch.full((nblk * inp.H_kv, cap), -7, dtype=torch.int32, device="cuda")
    count = torch.full((nblk * inp.H_kv,), -7, dtype=torch.int32, device="cuda")
    ws = o.alloc_workspace(o.workspace_size(L.SA_OP_PREFILL_SELECT, shape, inp.N))
    o.sa_select_prefill_topk(shape, pages, inp.N, inp.q, inp.w_q, kidx, inp.s_idx, B_SEL, k, idx,
                             count, ws)
    out = torch.full((inp.N, inp.H_q, inp.d), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((inp.N, inp.H_q), float("nan"), dtype=torch.float32, device="cuda")
    o.sa_sparse_prefill(shape, pages, inp.N, inp.q, inp.k_pool, inp.v_pool, idx, count, B_SEL,
                        inp.s_att, out, lse)
    torch.cuda.synchronize()
    return idx, count, out, lse


def check_blocks(inp, kt_rows, idx, count, out, lse, k, blocks, groups, tol=2e-2):
    n_diff = 0
    for g in groups:
        hs = inp.heads(g)
        K = S.to_np(inp.keys(g))
        V = S.to_np(inp.values(g))
        wq = S.to_np(inp.w_q[hs])
        for blk in blocks:
            rows = O.prefill_block_rows(blk, B_SEL, inp.N)
            Qb = S.to_np(inp.q[rows.start:rows.stop][:, hs])
            qc = O.prefill_block_query(Qb, wq, inp.s_idx)
            core = O.prefill_block_support(qc, kt_rows[g], blk, B_SEL, k)
            r = blk * inp.H_kv + g
            gsup = S.gpu_support(idx, count, r)
            n_cand = blk * B_SEL
            if n_cand:
                x = O.token_scores(qc, kt_rows[g][:n_cand])
                n_diff += S.check_support(gsup, x, core, L=n_cand, k=k)
            else:
                assert len(gsup) == 0
            o_ref, l_ref = O.prefill_block_attend(Qb, K, V, gsup, blk, B_SEL, inp.s_att)
            go = S.to_np(out[rows.start:rows.stop][:, hs])
            gl = lse[rows.start:rows.stop][:, hs].cpu().numpy().astype(np.float64)
            err = S.max_abs(go, o_ref)
            assert err <= tol, (blk, g, err)
            assert S.max_abs(gl, l_ref) <= 1e-2 * max(1.0, np.abs(l_ref).max()), (blk, g)
    return n_diff


@pytest.mark.parametrize("N,k", [(1000, 128), (777, 64), (640, 2048)])
def test_prefill_small(N, k):
    inp = synth.make_prefill_custom(N=N, H_q=8, H_kv=2, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=N, n_hh=12)
    kidx, kt_rows = oracle_kidx(inp)
    idx, count, out, lse = run_prefill(inp, kidx, k)
    check_blocks(inp, kt_rows, idx, count, out, lse, k, range(inp.n_blocks), range(inp.H_kv))


def test_prefill_late_maximum_raises():
    """Planted keys with logits about 13 log2 units above the rest (q += 4u,
    k += 25u): in many (block, query) rows a later tile of the list, or the
    diagonal tile, holds a key far above the running maximum, so the
    attention's lazily raised maximum moves after the first tile (147 such
    raises in this input, counted on the CPU from the oracle's supports)."""
    inp = synth.make_prefill_custom(N=1200, H_q=8, H_kv=2, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=5, n_hh=6, q_shift=4.0, k_shift=25.0)
    kidx, kt_rows = oracle_kidx(inp)
    idx, count, out, lse = run_prefill(inp, kidx, 96)
    check_blocks(inp, kt_rows, idx, count, out, lse, 96, range(inp.n_blocks), range(inp.H_kv))


@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (4, 2), (8, 1), (16, 1)])
def test_prefill_group_sizes(H_q, H_kv):
    """G = 1, 2, 8, 16 (a group of more than 4 heads is split over several
    workgroups that gather the same keys)."""
    inp = synth.make_prefill_custom(N=450, H_q=H_q, H_kv=H_kv, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=H_q * 10 + H_kv, n_hh=6)
    kidx, kt_rows = oracle_kidx(inp)
    idx, count, out, lse = run_prefill(inp, kidx, 96)
    check_blocks(inp, kt_rows, idx, count, out, lse, 96, range(inp.n_blocks), range(inp.H_kv))


def test_prefill_dense_when_k_covers_everything():
    """k >= N: every block attends to all earlier keys, i.e. dense causal
    attention (torch SDPA, float64 CPU)."""
    inp = synth.make_prefill_custom(N=300, H_q=4, H_kv=1, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=7)
    kidx, _ = oracle_kidx(inp)
    idx, count, out, lse = run_prefill(inp, kidx, 4096, out_dtype=torch.float32)
    q = S.to_np(inp.q).transpose(1, 0, 2)  # [H, N, d]
    K = S.to_np(inp.keys(0))
    V = S.to_np(inp.values(0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        scale=inp.s_att, is_causal=True)[0].numpy().transpose(1, 0, 2)
    assert S.max_abs(S.to_np(out), ref) <= 2e-2


def test_prefill128k_sampled_blocks():
    """The 128K prefill workload (32/8 heads, d=128, bf16, 0.5% column heavy
    hitters, top-k 2048 + diagonal); a seeded sample of 64 query blocks
    (including the first blocks, the k boundary and the last block) checked
    for every group."""
    inp = synth.make_prefill128k(device="cuda")
    rng = np.random.default_rng(4)
    rng.choice(inp.H_kv, 2, replace=False)  # (keeps the seeded block sample)
    groups = list(range(inp.H_kv))
    kidx, kt_rows = oracle_kidx(inp, groups)
    k = inp.top_k
    idx, count, out, lse = run_prefill(inp, kidx, k)
    nblk = inp.n_blocks
    fixed = [0, 31, 32, 33, nblk - 1]
    others = rng.choice(np.setdiff1d(np.arange(nblk), fixed), 59, replace=False).tolist()
    blocks = sorted(fixed + others)
    n_diff = check_blocks(inp, kt_rows, idx, count, out, lse, k, blocks, groups)
    print(f"prefill128k: groups {groups}, tolerated support differences {n_diff}")


def quantised_kidx(inp, seed, probs=(0.8, 0.15, 0.05)):
    """Indexer keys drawn from three fixed 16-vectors (rounded to the cache
    dtype): every block's scores take three values, in long tie groups."""
    rng = np.random.default_rng(seed)
    vecs = S.store_round(rng.standard_normal((len(probs), 16)), inp.dtype)
    kt = vecs[rng.choice(len(probs), size=inp.N, p=list(probs))]
    pool = torch.zeros((inp.k_pool.shape[0], inp.H_kv, 64, 16), dtype=inp.dtype)
    full = torch.zeros((pool.shape[0] * 64, 16), dtype=inp.dtype)
    full[: inp.N] = torch.from_numpy(kt).to(inp.dtype)
    for g in range(inp.H_kv):
        pool[:, g] = full.view(pool.shape[0], 64, 16)
    return pool.to(inp.device), {g: kt for g in range(inp.H_kv)}


def test_prefill_select_long_tie_groups():
    """Top-2048 over rows of up to 20K candidates whose scores take three
    values: the threshold falls inside a tie group of thousands of candidates
    (more than the selection keeps per wave for its exact second pass), and
    the lists must be exactly the oracle's, ties lowest index first."""
    inp = synth.make_prefill_custom(N=20000, H_q=4, H_kv=1, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=21, n_hh=4)
    kidx, kt_rows = quantised_kidx(inp, 3)
    k = 2048
    idx, count, out, lse = run_prefill(inp, kidx, k)
    blocks = [1, 33, 40, 150, inp.n_blocks - 1]
    check_blocks(inp, kt_rows, idx, count, out, lse, k, blocks, [0])
    wq = S.to_np(inp.w_q[inp.heads(0)])
    for blk in blocks:
        rows = O.prefill_block_rows(blk, B_SEL, inp.N)
        qc = O.prefill_block_query(S.to_np(inp.q[rows.start:rows.stop][:, inp.heads(0)]), wq, inp.s_idx)
        core = O.prefill_block_support(qc, kt_rows[0], blk, B_SEL, k)
        assert S.gpu_support(idx, count, blk).tolist() == core.tolist(), blk


def periodic_kidx(inp, seed, on_high):
    """Indexer keys s_j * v plus small noise, with s_j near +3 on the keys of
    every eighth 16-key tile and near -3 elsewhere (on_high), or the other
    way round: the scores of a row are bimodal with a mode that only every
    eighth tile holds."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(16)
    on = (np.arange(inp.N) // 16) % 8 == 0
    sj = np.where(on == on_high, 3.0, -3.0) + rng.uniform(-0.5, 0.5, inp.N)
    kt = S.store_round(sj[:, None] * v[None, :] + 0.05 * rng.standard_normal((inp.N, 16)), inp.dtype)
    pool = torch.zeros((inp.k_pool.shape[0], inp.H_kv, 64, 16), dtype=inp.dtype)
    full = torch.zeros((pool.shape[0] * 64, 16), dtype=inp.dtype)
    full[: inp.N] = torch.from_numpy(kt).to(inp.dtype)
    for g in range(inp.H_kv):
        pool[:, g] = full.view(pool.shape[0], 64, 16)
    return pool.to(inp.device), {g: kt for g in range(inp.H_kv)}


@pytest.mark.parametrize("on_high", [True, False])
def test_prefill_select_periodic_keys(on_high):
    """Top-2048 over rows of 4K-40K candidates whose scores follow a pattern
    with period 128 keys (a threshold estimated from a regular sample of the
    row can be far off); the supports must still be the oracle's."""
    inp = synth.make_prefill_custom(N=40000, H_q=4, H_kv=1, d=128, dtype=torch.bfloat16,
                                    device="cuda", seed=23, n_hh=0)
    kidx, kt_rows = periodic_kidx(inp, 5, on_high)
    k = 2048
    idx, count, out, lse = run_prefill(inp, kidx, k)
    blocks = [2, 40, 64, 65, 70, 200, 400, inp.n_blocks - 1]
    check_blocks(inp, kt_rows, idx, count, out, lse, k, blocks, [0])
