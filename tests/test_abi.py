"""The C-ABI library loads and exports every entry point include/sa.h declares,
and rejects bad arguments on the host (before any launch, so no GPU is
touched).  CPU only."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")
LIB = os.path.join(ROOT, "dynamic_sparse_attention_02_amd", "libsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB),
                                reason="libsa.so not built (python -m dynamic_sparse_attention_02_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def lib():
    from dynamic_sparse_attention_02_amd import _lib as L
    return L, L.load()


def test_every_declared_symbol_is_exported_and_bound():
    L, so = lib()
    names = declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(so, n), f"{n} declared in sa.h but not exported"
        assert n in L.SIGNATURES, f"{n} has no ctypes signature in the binding"
    assert set(L.SIGNATURES) == set(names)
    from dynamic_sparse_attention_02_amd import ops
    for n in names:
        if n.startswith("sa_") and n not in ("sa_workspace_size", "sa_status_string",
                                              "sa_last_error", "sa_version"):
            assert hasattr(ops, n), f"binding lacks {n}"


def test_status_strings_and_version():
    L, so = lib()
    assert so.sa_status_string(0) == b"SA_OK"
    assert so.sa_status_string(3) == b"SA_ERR_CAPACITY"
    assert so.sa_status_string(99) == b"SA_ERR_UNKNOWN"
    assert b"gfx950" in so.sa_version()


def _shape(L, **kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=4, head_dim=128, idx_rank=16, page_size=64,
                max_pages=1024, max_len=65536, n_pool_pages=1024)
    base.update(kw)
    return L.SaShape(*[base[f] for f, _ in L.SaShape._fields_])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


def test_workspace_sizes():
    L, so = lib()
    s = _shape(L)
    ws = lambda op, prm: so.sa_workspace_size(op, ctypes.byref(s), prm)
    assert ws(L.SA_OP_INDEX_SCORES, 0) >= 4 * 16 * 4
    # few rows: room for the persistent selection too (its size does not
    # depend on the candidates); many rows: grows with the candidates
    assert ws(L.SA_OP_SELECT, 1 << 22) >= ws(L.SA_OP_SELECT, 1024) > 0
    s32 = _shape(L, batch=8)
    assert (so.sa_workspace_size(L.SA_OP_SELECT, ctypes.byref(s32), 1 << 22)
            > so.sa_workspace_size(L.SA_OP_SELECT, ctypes.byref(s32), 1024) > 0)
    assert ws(L.SA_OP_SPARSE_DECODE, 65536) > ws(L.SA_OP_SPARSE_DECODE, 64) > 0
    assert ws(L.SA_OP_DECODE_STEP, 65536) >= ws(L.SA_OP_SELECT, 65536) + ws(L.SA_OP_SPARSE_DECODE, 65536)
    bad = _shape(L, head_dim=96)
    assert so.sa_workspace_size(L.SA_OP_SELECT, ctypes.byref(bad), 10) == 0


def _pages(L):
    return L.SaPages(FAKE, FAKE)


def test_validation_codes():
    L, so = lib()
    s = _shape(L)
    pg = _pages(L)
    B = ctypes.byref
    # select: bad p, capacity, workspace, NULL buffer
    assert so.sa_select_topp(B(s), B(pg), FAKE, 65536, 0.0, 0, 0, FAKE, FAKE, 65536, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert b"p=" in so.sa_last_error()
    assert so.sa_select_topp(B(s), B(pg), FAKE, 65536, 1.5, 0, 0, FAKE, FAKE, 65536, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_select_topp(B(s), B(pg), FAKE, 65536, 0.9, 0, 0, FAKE, FAKE, 1000, FAKE, 1 << 30, None) == L.SA_ERR_CAPACITY
    assert so.sa_select_topp(B(s), B(pg), FAKE, 65536, 0.9, 0, 0, FAKE, FAKE, 65536, FAKE, 16, None) == L.SA_ERR_WORKSPACE
    assert so.sa_select_topp(B(s), B(pg), FAKE, 65536, 0.9, 0, 0, FAKE, FAKE, 65536, None, 1 << 30, None) == L.SA_ERR_WORKSPACE
    assert so.sa_select_topp(B(s), B(pg), None, 65536, 0.9, 0, 0, FAKE, FAKE, 65536, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_select_topp(B(s), B(pg), FAKE, 100, 0.9, 0, 0, FAKE, FAKE, 65536, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_select_topp(None, B(pg), FAKE, 65536, 0.9, 0, 0, FAKE, FAKE, 65536, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    # top-k: k < 1, capacity, pages with sink, unit
    assert so.sa_select_topk(B(s), B(pg), FAKE, 65536, 0, 1, 0, 0, FAKE, FAKE, 100, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_select_topk(B(s), B(pg), FAKE, 65536, 64, 1, 4, 512, FAKE, FAKE, 579, FAKE, 1 << 30, None) == L.SA_ERR_CAPACITY
    assert so.sa_select_topk(B(s), B(pg), FAKE, 65536, 32, 64, 4, 0, FAKE, FAKE, 2048, FAKE, 1 << 30, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_select_topk(B(s), B(pg), FAKE, 65536, 32, 7, 0, 0, FAKE, FAKE, 2048, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_select_topk(B(s), B(pg), FAKE, 65536, 32, 64, 0, 0, FAKE, FAKE, 2047, FAKE, 1 << 30, None) == L.SA_ERR_CAPACITY
    # shapes
    for kw, code in ((dict(head_dim=96), L.SA_ERR_UNSUPPORTED), (dict(idx_rank=8), L.SA_ERR_UNSUPPORTED),
                     (dict(page_size=32), L.SA_ERR_UNSUPPORTED), (dict(n_kv_heads=5), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(n_q_heads=96, n_kv_heads=4), L.SA_ERR_UNSUPPORTED),
                     (dict(max_len=65537), L.SA_ERR_INVALID_ARGUMENT), (dict(batch=0), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(n_pool_pages=0), L.SA_ERR_INVALID_ARGUMENT)):
        bad = _shape(L, **kw)
        assert so.sa_index_scores(B(bad), B(pg), FAKE, FAKE, FAKE, L.SA_BF16, 1.0, FAKE, 65536, FAKE, 1 << 20, None) == code, kw
    # decode: workspace too small, bad dtype, NULL count
    assert so.sa_sparse_decode(B(s), B(pg), FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 65536, 0.1, FAKE, L.SA_F32, None, FAKE, 100, None) == L.SA_ERR_WORKSPACE
    assert so.sa_sparse_decode(B(s), B(pg), FAKE, FAKE, FAKE, 7, FAKE, FAKE, 65536, 0.1, FAKE, L.SA_F32, None, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_sparse_decode(B(s), B(pg), FAKE, FAKE, FAKE, L.SA_BF16, FAKE, None, 65536, 0.1, FAKE, L.SA_F32, None, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    # decode with the residual linear attention tail: workspace covers the
    # extra partials, NULL state; state build: negative first token
    ws_plain = so.sa_workspace_size(L.SA_OP_SPARSE_DECODE, B(s), 65536)
    assert so.sa_workspace_size(L.SA_OP_SPARSE_DECODE_RLA, B(s), 65536) > ws_plain
    assert so.sa_sparse_decode_rla(B(s), B(pg), FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 65536, 0.1, FAKE, L.SA_F32, None, FAKE, FAKE, FAKE, FAKE, ws_plain, None) == L.SA_ERR_WORKSPACE
    assert so.sa_sparse_decode_rla(B(s), B(pg), FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 65536, 0.1, FAKE, L.SA_F32, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_rla_state(B(s), B(pg), FAKE, FAKE, L.SA_BF16, -1, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_rla_state(B(s), B(pg), FAKE, FAKE, L.SA_BF16, 0, None, None) == L.SA_ERR_INVALID_ARGUMENT
    # attention mass and coverage
    ws_mass = so.sa_workspace_size(L.SA_OP_ATTENTION_MASS, B(s), 0)
    assert ws_mass >= 32 * 65536 * 4  # [rows][G][max_len] fp32 logits
    assert so.sa_attention_mass(B(s), B(pg), FAKE, FAKE, L.SA_BF16, 0.1, FAKE, 65535, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_attention_mass(B(s), B(pg), FAKE, FAKE, L.SA_BF16, 0.1, FAKE, 65536, FAKE, ws_mass - 1, None) == L.SA_ERR_WORKSPACE
    assert so.sa_attention_mass(B(s), B(pg), None, FAKE, L.SA_BF16, 0.1, FAKE, 65536, FAKE, ws_mass, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_attention_mass(B(s), B(pg), FAKE, FAKE, 7, 0.1, FAKE, 65536, FAKE, ws_mass, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_support_coverage(B(s), B(pg), FAKE, 65536, FAKE, FAKE, 0, None, None, 0, FAKE, None, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_support_coverage(B(s), B(pg), FAKE, 65536, FAKE, FAKE, 64, FAKE, None, 64, FAKE, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_support_coverage(B(s), B(pg), FAKE, 65536, FAKE, FAKE, 64, FAKE, FAKE, 0, FAKE, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_support_coverage(B(s), B(pg), FAKE, 65536, FAKE, FAKE, 64, None, None, 0, None, None, None) == L.SA_ERR_INVALID_ARGUMENT
    # decode step: capacity and p
    assert so.sa_decode_step(B(s), B(pg), FAKE, FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 0.1, 0.9, 0, 4, 512, FAKE, 65536, FAKE, FAKE, 60000, FAKE, L.SA_F32, None, FAKE, 1 << 30, None) == L.SA_ERR_CAPACITY
    assert so.sa_decode_step(B(s), B(pg), FAKE, FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 0.1, 0.0, 0, 4, 512, FAKE, 65536, FAKE, FAKE, 65536, FAKE, L.SA_F32, None, FAKE, 1 << 30, None) == L.SA_ERR_INVALID_ARGUMENT
    # page-level decode step: top_k, score row width, capacity, workspace,
    # NULL statistics (shape: 1024 pages of 64 tokens, so cap >= k * 64)
    ws_pg = so.sa_workspace_size(L.SA_OP_DECODE_STEP_PAGES, B(s), 2048)
    assert ws_pg >= so.sa_workspace_size(L.SA_OP_SPARSE_DECODE, B(s), 2048)
    step_pg = lambda *a: so.sa_decode_step_pages(B(s), B(pg), *a)
    assert step_pg(FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 0.1, 0, FAKE, 1024, FAKE, FAKE, 2048, FAKE, L.SA_F32, None, FAKE, ws_pg, None) == L.SA_ERR_INVALID_ARGUMENT
    assert step_pg(FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 0.1, 32, FAKE, 1023, FAKE, FAKE, 2048, FAKE, L.SA_F32, None, FAKE, ws_pg, None) == L.SA_ERR_INVALID_ARGUMENT
    assert step_pg(FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 0.1, 32, FAKE, 1024, FAKE, FAKE, 2047, FAKE, L.SA_F32, None, FAKE, ws_pg, None) == L.SA_ERR_CAPACITY
    assert step_pg(FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 0.1, 32, FAKE, 1024, FAKE, FAKE, 2048, FAKE, L.SA_F32, None, FAKE, ws_pg - 1, None) == L.SA_ERR_WORKSPACE
    assert step_pg(FAKE, None, FAKE, FAKE, L.SA_BF16, 0.1, 32, FAKE, 1024, FAKE, FAKE, 2048, FAKE, L.SA_F32, None, FAKE, ws_pg, None) == L.SA_ERR_INVALID_ARGUMENT
    # prefill: batch, b_sel, dtype, n_tokens
    s1 = _shape(L, n_q_heads=32, n_kv_heads=8, max_pages=2048, max_len=131072, n_pool_pages=2048)
    assert so.sa_sparse_prefill(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 2048, 32, 0.1, FAKE, L.SA_BF16, None, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_sparse_prefill(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_F32, FAKE, FAKE, 2048, 64, 0.1, FAKE, L.SA_BF16, None, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_sparse_prefill(B(s1), B(pg), 131073, FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 2048, 64, 0.1, FAKE, L.SA_BF16, None, None) == L.SA_ERR_INVALID_ARGUMENT
    s2 = _shape(L, batch=2)
    assert so.sa_select_prefill_topk(B(s2), B(pg), 100, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 64, 2048, FAKE, FAKE, 2048, FAKE, 1 << 30, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_select_prefill_topk(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 64, 2048, FAKE, FAKE, 2000, FAKE, 1 << 30, None) == L.SA_ERR_CAPACITY
    # per-query prefill: b_sel, capacity (k + 1 with the own token), workspace
    assert so.sa_select_prefill_topk(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 1, 2048, FAKE, FAKE, 2048, FAKE, 1 << 40, None) == L.SA_ERR_CAPACITY
    assert so.sa_select_prefill_topk(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 2, 2048, FAKE, FAKE, 2049, FAKE, 1 << 40, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_select_prefill_topk_probs(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 64, 2048, FAKE, FAKE, 2049, FAKE, 1 << 40, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_select_prefill_topk_probs(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 1, 0, FAKE, FAKE, 2049, FAKE, 1 << 40, None) == L.SA_ERR_INVALID_ARGUMENT
    ws_q = so.sa_workspace_size(L.SA_OP_PREFILL_QUERY, B(s1), 2049)
    assert ws_q > 131072 * 4
    assert so.sa_sparse_prefill_query(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 2049, 0.1, FAKE, L.SA_BF16, None, FAKE, ws_q - 1, None) == L.SA_ERR_WORKSPACE
    assert so.sa_sparse_prefill_query(B(s1), B(pg), 0, FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 2049, 0.1, FAKE, L.SA_BF16, None, FAKE, ws_q, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_sparse_prefill(B(s1), B(pg), 131072, FAKE, FAKE, FAKE, L.SA_BF16, FAKE, FAKE, 2048, 1, 0.1, FAKE, L.SA_BF16, None, None) == L.SA_ERR_UNSUPPORTED
    # segment permutation: segment length, sizes, capacity
    assert so.sa_pbs_permutation(B(s1), FAKE, 131072, 100, FAKE, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_pbs_permutation(B(s1), FAKE, 131072, 8192, FAKE, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_pbs_permutation(B(s1), None, 131072, 2048, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    ws_pi = so.sa_workspace_size(L.SA_OP_PBS_IMPORTANCE, B(s1), 64)
    assert so.sa_pbs_importance(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 0, FAKE, FAKE, ws_pi, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_pbs_importance(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 64, FAKE, FAKE, ws_pi - 1, None) == L.SA_ERR_WORKSPACE
    assert so.sa_pbs_importance(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 1000, FAKE, FAKE, 1 << 40, None) == L.SA_ERR_UNSUPPORTED
    ws_ps = so.sa_workspace_size(L.SA_OP_PBS_SELECT, B(s1), 32)
    assert so.sa_pbs_select(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, FAKE, 2048, 64, 32, FAKE, FAKE, 2047, FAKE, ws_ps, None) == L.SA_ERR_CAPACITY
    assert so.sa_pbs_select(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, FAKE, 2048, 32, 32, FAKE, FAKE, 2048, FAKE, ws_ps, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_pbs_select(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, FAKE, 2048, 64, 32, FAKE, FAKE, 2048, FAKE, ws_ps - 1, None) == L.SA_ERR_WORKSPACE
    # prefill attention-mass oracle: b_sel, capacity
    ws_po = so.sa_workspace_size(L.SA_OP_PREFILL_ORACLE, B(s1), 0)
    assert so.sa_select_prefill_oracle(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 32, 2048, FAKE, FAKE, 2048, FAKE, ws_po, None) == L.SA_ERR_UNSUPPORTED
    assert so.sa_select_prefill_oracle(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 1, 2048, FAKE, FAKE, 2048, FAKE, ws_po, None) == L.SA_ERR_CAPACITY
    assert so.sa_select_prefill_oracle(B(s1), B(pg), 131072, FAKE, FAKE, L.SA_BF16, 0.1, 64, 2048, FAKE, FAKE, 2048, FAKE, ws_po - 1, None) == L.SA_ERR_WORKSPACE
    # maintenance calls
    assert so.sa_index_append(B(s), None, FAKE, L.SA_BF16, FAKE, 5, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_index_append(B(s), FAKE, FAKE, L.SA_BF16, FAKE, -1, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_page_stats(B(s), FAKE, 9, FAKE, FAKE, 3, FAKE, None) == L.SA_ERR_INVALID_ARGUMENT
    assert so.sa_page_scores(B(s), B(pg), FAKE, FAKE, L.SA_BF16, 0.1, FAKE, 10, None) == L.SA_ERR_INVALID_ARGUMENT


def test_zero_work_calls_return_ok_without_launch():
    L, so = lib()
    s = _shape(L)
    assert so.sa_index_append(ctypes.byref(s), None, None, L.SA_BF16, None, 0, None, None) == L.SA_OK
    assert so.sa_page_stats(ctypes.byref(s), None, L.SA_BF16, None, None, 0, None, None) == L.SA_OK
    assert so.sa_last_error() == b""


def test_decode_step_noalloc_rejects_before_touching_the_device():
    """The allocation-free decode step checks its arguments, and whether the
    shape fits the library's scratch, before it sets up anything on a device:
    these calls return on the host."""
    L, so = lib()
    s = _shape(L)
    pg = L.SaPages(FAKE, FAKE)
    B = ctypes.byref
    call = lambda sh, p, cap, **kw: so.sa_decode_step_noalloc(
        B(sh), B(pg), FAKE, FAKE, FAKE, FAKE, FAKE, L.SA_BF16, 1.0, 0.1, p, 0, 4, 512, FAKE,
        sh.max_len, FAKE, FAKE, cap, FAKE, L.SA_F32, None, None)
    assert call(s, 0.9, 60000) == L.SA_ERR_CAPACITY
    assert call(s, 0.0, 65536) == L.SA_ERR_INVALID_ARGUMENT
    # 32 sequences of up to 128K tokens need far more than the 64 MiB scratch
    big = _shape(L, batch=32, n_kv_heads=8, max_pages=2048, max_len=131072, n_pool_pages=65536)
    assert call(big, 0.9, 131072) == L.SA_ERR_WORKSPACE
    assert b"scratch" in so.sa_last_error()
