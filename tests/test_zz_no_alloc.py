"""The allocation-free decode step (sa_decode_step_noalloc) against
sa_decode_step on the same inputs, through the C ABI.  Both run the same
kernels, so lists, counts, scores and outputs must be identical.  The calls
follow one another on the library's one scratch array, with shapes that
shrink and grow again and that switch between the single persistent launch,
the persistent few-row selection and the separate launches, so each call
depends on the previous one having left the scratch's zero state clean."""

import pytest
import torch

import synth
from tests import _support as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (inputs, rule): in call order
CASES = [
    # 8 rows, group of 8: the single persistent launch
    (dict(B=2, H_q=32, H_kv=4, d=128, seq_lens=[20000, 9000], dtype=torch.bfloat16, seed=41),
     dict(p=0.9, n_sink=4, n_window=512)),
    # group of 2: separate launches, the long rows' selection as one persistent launch
    (dict(B=1, H_q=8, H_kv=4, d=64, seq_lens=[40000], dtype=torch.float32, seed=42),
     dict(p=0.9, n_sink=4, n_window=64)),
    # smaller input, persistent launch, top-k
    (dict(B=1, H_q=16, H_kv=2, d=128, seq_lens=[3000], dtype=torch.bfloat16, seed=43),
     dict(top_k=64, n_sink=4, n_window=64)),
    # 20 rows: separate launches with one block per row
    (dict(B=5, H_q=16, H_kv=4, d=64, seq_lens=[700, 1500, 0, 64, 2000], dtype=torch.float32, seed=44),
     dict(p=0.8, n_sink=4, n_window=32)),
    # the smallest, persistent launch
    (dict(B=1, H_q=8, H_kv=2, d=64, seq_lens=[500], dtype=torch.float32, seed=45),
     dict(p=0.9)),
    # the first shape again, after all the smaller ones
    (dict(B=2, H_q=32, H_kv=4, d=128, seq_lens=[20000, 9000], dtype=torch.bfloat16, seed=41),
     dict(p=0.9, n_sink=4, n_window=512)),
]


def _call(entry, inp, pool, rule, ws=None):
    from dynamic_sparse_attention_02_amd import ops
    shape = S.shape_of(inp)
    pages = ops.make_pages(inp.page_table, inp.seq_lens_tensor())
    cap = max(max(inp.seq_lens), 1)
    x, idx, count, out, lse = S.empty_like_outputs(inp, cap)
    args = (shape, pages, inp.q, inp.w_q, pool, inp.k_pool, inp.v_pool, inp.s_idx, inp.s_att,
            S.f32(rule.get("p", 0.0)), rule.get("top_k", 0), rule.get("n_sink", 0),
            rule.get("n_window", 0), x, idx, count, out, lse)
    if entry == "step":
        ops.sa_decode_step(*args, ws)
    else:
        ops.sa_decode_step_noalloc(*args)
    return x, idx, count, out, lse


def test_noalloc_matches_decode_step_over_consecutive_calls():
    from dynamic_sparse_attention_02_amd import _lib as L
    from dynamic_sparse_attention_02_amd import ops
    inputs = []
    for kw, rule in CASES:
        inp = synth.make_decode_custom(device="cuda", hh_frac=0.01, alpha=12.0, shuffle=True, **kw)
        inputs.append((inp, S.oracle_kidx_pool(inp), rule))
    # the existing entry point, each call on a workspace of its own
    refs = []
    for inp, pool, rule in inputs:
        shape = S.shape_of(inp)
        cap = max(max(inp.seq_lens), 1)
        ws = ops.alloc_workspace(ops.workspace_size(L.SA_OP_DECODE_STEP, shape, cap))
        refs.append(_call("step", inp, pool, rule, ws))
        torch.cuda.synchronize()
    # the allocation-free entry point, the calls back to back on its scratch
    got = [_call("noalloc", inp, pool, rule) for inp, pool, rule in inputs]
    torch.cuda.synchronize()
    for c, ((inp, _, rule), r, g) in enumerate(zip(inputs, refs, got)):
        rx, ridx, rcnt, rout, rlse = r
        gx, gidx, gcnt, gout, glse = g
        assert torch.all(rcnt >= 0) and torch.equal(rcnt, gcnt), c
        assert torch.equal(ridx, gidx), c
        for b, L_ in enumerate(inp.seq_lens):
            rows = slice(b * inp.H_kv, (b + 1) * inp.H_kv)
            assert torch.equal(rx[rows, :L_], gx[rows, :L_]), (c, b)
        assert torch.equal(rout, gout) and torch.equal(rlse, glse), c
