"""Torch-facing binding of libsa: one function per C entry point, same names.

Each function only marshals arguments (tensor -> device pointer, current
stream -> hipStream_t) and raises SAError on a non-OK status; all computation
happens in the HIP kernels.  Tensors must already live on the GPU in the
layouts documented in include/sa.h.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L

__all__ = [
    "SAError",
    "make_shape",
    "make_pages",
    "workspace_size",
    "alloc_workspace",
    "sa_index_append",
    "sa_page_stats",
    "sa_index_scores",
    "sa_page_scores",
    "sa_select_topp",
    "sa_select_topk",
    "sa_sparse_decode",
    "sa_sparse_decode_rla",
    "sa_rla_state",
    "sa_attention_mass",
    "sa_support_coverage",
    "sa_decode_step",
    "sa_decode_step_rla",
    "sa_decode_step_pages",
    "sa_select_prefill_topk",
    "sa_sparse_prefill",
    "sa_select_prefill_topk_probs",
    "sa_sparse_prefill_query",
    "sa_select_prefill_oracle",
    "sa_pbs_importance",
    "sa_pbs_permutation",
    "sa_pbs_select",
    "version",
]

SAError = L.SAError


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.SA_BF16
    if t.dtype == torch.float32:
        return L.SA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libsa takes GPU tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(*, batch, n_q_heads, n_kv_heads, head_dim, max_pages, max_len, n_pool_pages,
               idx_rank=16, page_size=64) -> L.SaShape:
    return L.SaShape(batch, n_q_heads, n_kv_heads, head_dim, idx_rank, page_size, max_pages,
                     max_len, n_pool_pages)


def make_pages(page_table: torch.Tensor, seq_lens: torch.Tensor | None) -> L.SaPages:
    """Paging descriptor (holds references to both tensors)."""
    if page_table.dtype != torch.int32 or (seq_lens is not None and seq_lens.dtype != torch.int32):
        raise TypeError("page_table and seq_lens must be int32")
    pg = L.SaPages(_dev(page_table), _dev(seq_lens) if seq_lens is not None else None)
    pg._keep = (page_table, seq_lens)  # the descriptor keeps its tensors alive
    return pg


def workspace_size(op: int, shape: L.SaShape, param: int = 0) -> int:
    return int(L.load().sa_workspace_size(op, ctypes.byref(shape), int(param)))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of at least nbytes (the library leaves it zeroed)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev(ws), ws.numel() * ws.element_size()


def version() -> str:
    return L.load().sa_version().decode()


def sa_index_append(shape, k_pre, w_k, slot, kidx_pool, stream=None):
    st = L.load().sa_index_append(ctypes.byref(shape), _dev(k_pre), _dev(w_k), _dt(k_pre),
                                  _dev(slot), int(slot.numel()), _dev(kidx_pool), _stream(stream))
    L.check(st, "sa_index_append")


def sa_page_stats(shape, k_pool, pages, n_valid, stats_pool, stream=None):
    st = L.load().sa_page_stats(ctypes.byref(shape), _dev(k_pool), _dt(k_pool), _dev(pages),
                                _dev(n_valid), int(pages.numel()), _dev(stats_pool), _stream(stream))
    L.check(st, "sa_page_stats")


def sa_index_scores(shape, pages, q, w_q, kidx_pool, s_idx, x, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_index_scores(ctypes.byref(shape), ctypes.byref(pages), _dev(q), _dev(w_q),
                                  _dev(kidx_pool), _dt(q), float(s_idx), _dev(x), int(x.stride(0)),
                                  wp, wn, _stream(stream))
    L.check(st, "sa_index_scores")


def sa_page_scores(shape, pages, q, stats_pool, s_att, x, stream=None):
    st = L.load().sa_page_scores(ctypes.byref(shape), ctypes.byref(pages), _dev(q),
                                 _dev(stats_pool), _dt(q), float(s_att), _dev(x), int(x.stride(0)),
                                 _stream(stream))
    L.check(st, "sa_page_scores")


def sa_select_topp(shape, pages, x, p, n_sink, n_window, idx, count, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_select_topp(ctypes.byref(shape), ctypes.byref(pages), _dev(x),
                                 int(x.stride(0)), float(p), int(n_sink), int(n_window), _dev(idx),
                                 _dev(count), int(idx.shape[-1]), wp, wn, _stream(stream))
    L.check(st, "sa_select_topp")


def sa_select_topk(shape, pages, x, k, unit, n_sink, n_window, idx, count, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_select_topk(ctypes.byref(shape), ctypes.byref(pages), _dev(x),
                                 int(x.stride(0)), int(k), int(unit), int(n_sink), int(n_window),
                                 _dev(idx), _dev(count), int(idx.shape[-1]), wp, wn,
                                 _stream(stream))
    L.check(st, "sa_select_topk")


def sa_sparse_decode(shape, pages, q, k_pool, v_pool, idx, count, s_att, out, lse, ws,
                     stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_sparse_decode(ctypes.byref(shape), ctypes.byref(pages), _dev(q), _dev(k_pool),
                                   _dev(v_pool), _dt(q), _dev(idx), _dev(count),
                                   int(idx.shape[-1]), float(s_att), _dev(out), _dt(out), _dev(lse),
                                   wp, wn, _stream(stream))
    L.check(st, "sa_sparse_decode")


def sa_sparse_decode_rla(shape, pages, q, k_pool, v_pool, idx, count, s_att, out, lse, rla_state,
                         rla_num, rla_den, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_sparse_decode_rla(ctypes.byref(shape), ctypes.byref(pages), _dev(q),
                                       _dev(k_pool), _dev(v_pool), _dt(q), _dev(idx), _dev(count),
                                       int(idx.shape[-1]), float(s_att), _dev(out), _dt(out),
                                       _dev(lse), _dev(rla_state), _dev(rla_num), _dev(rla_den),
                                       wp, wn, _stream(stream))
    L.check(st, "sa_sparse_decode_rla")


def sa_rla_state(shape, pages, k_pool, v_pool, first_token, state, stream=None):
    st = L.load().sa_rla_state(ctypes.byref(shape), ctypes.byref(pages), _dev(k_pool),
                               _dev(v_pool), _dt(k_pool), int(first_token), _dev(state),
                               _stream(stream))
    L.check(st, "sa_rla_state")


def sa_attention_mass(shape, pages, q, k_pool, s_att, x, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_attention_mass(ctypes.byref(shape), ctypes.byref(pages), _dev(q),
                                    _dev(k_pool), _dt(q), float(s_att), _dev(x), int(x.stride(0)),
                                    wp, wn, _stream(stream))
    L.check(st, "sa_attention_mass")


def sa_support_coverage(shape, pages, x, idx, count, mass, ref_idx=None, ref_count=None,
                        overlap=None, stream=None):
    st = L.load().sa_support_coverage(ctypes.byref(shape), ctypes.byref(pages), _dev(x),
                                      int(x.stride(0)), _dev(idx), _dev(count), int(idx.shape[-1]),
                                      _dev(ref_idx), _dev(ref_count),
                                      int(ref_idx.shape[-1]) if ref_idx is not None else 0,
                                      _dev(mass), _dev(overlap), _stream(stream))
    L.check(st, "sa_support_coverage")


def sa_decode_step(shape, pages, q, w_q, kidx_pool, k_pool, v_pool, s_idx, s_att, p, top_k,
                   n_sink, n_window, x, idx, count, out, lse, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_decode_step(ctypes.byref(shape), ctypes.byref(pages), _dev(q), _dev(w_q),
                                 _dev(kidx_pool), _dev(k_pool), _dev(v_pool), _dt(q), float(s_idx),
                                 float(s_att), float(p), int(top_k), int(n_sink), int(n_window),
                                 _dev(x), int(x.stride(0)), _dev(idx), _dev(count),
                                 int(idx.shape[-1]), _dev(out), _dt(out), _dev(lse), wp, wn,
                                 _stream(stream))
    L.check(st, "sa_decode_step")


def sa_decode_step_rla(shape, pages, q, w_q, kidx_pool, k_pool, v_pool, s_idx, s_att, p, top_k,
                       n_sink, n_window, x, idx, count, out, lse, rla_state, rla_num, rla_den, ws,
                       stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_decode_step_rla(ctypes.byref(shape), ctypes.byref(pages), _dev(q), _dev(w_q),
                                     _dev(kidx_pool), _dev(k_pool), _dev(v_pool), _dt(q),
                                     float(s_idx), float(s_att), float(p), int(top_k), int(n_sink),
                                     int(n_window), _dev(x), int(x.stride(0)), _dev(idx),
                                     _dev(count), int(idx.shape[-1]), _dev(out), _dt(out),
                                     _dev(lse), _dev(rla_state), _dev(rla_num), _dev(rla_den), wp,
                                     wn, _stream(stream))
    L.check(st, "sa_decode_step_rla")


def sa_decode_step_noalloc(shape, pages, q, w_q, kidx_pool, k_pool, v_pool, s_idx, s_att, p,
                           top_k, n_sink, n_window, x, idx, count, out, lse, stream=None):
    st = L.load().sa_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(pages), _dev(q),
                                         _dev(w_q), _dev(kidx_pool), _dev(k_pool), _dev(v_pool),
                                         _dt(q), float(s_idx), float(s_att), float(p), int(top_k),
                                         int(n_sink), int(n_window), _dev(x), int(x.stride(0)),
                                         _dev(idx), _dev(count), int(idx.shape[-1]), _dev(out),
                                         _dt(out), _dev(lse), _stream(stream))
    L.check(st, "sa_decode_step_noalloc")


def sa_decode_step_pages(shape, pages, q, stats_pool, k_pool, v_pool, s_att, top_k, x, idx, count,
                         out, lse, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_decode_step_pages(ctypes.byref(shape), ctypes.byref(pages), _dev(q),
                                       _dev(stats_pool), _dev(k_pool), _dev(v_pool), _dt(q),
                                       float(s_att), int(top_k), _dev(x), int(x.stride(0)),
                                       _dev(idx), _dev(count), int(idx.shape[-1]), _dev(out),
                                       _dt(out), _dev(lse), wp, wn, _stream(stream))
    L.check(st, "sa_decode_step_pages")


def sa_select_prefill_topk(shape, pages, n_tokens, q, w_q, kidx_pool, s_idx, b_sel, k, idx,
                           count, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_select_prefill_topk(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens),
                                         _dev(q), _dev(w_q), _dev(kidx_pool), _dt(q), float(s_idx),
                                         int(b_sel), int(k), _dev(idx), _dev(count),
                                         int(idx.shape[-1]), wp, wn, _stream(stream))
    L.check(st, "sa_select_prefill_topk")


def sa_sparse_prefill(shape, pages, n_tokens, q, k_pool, v_pool, idx, count, b_sel, s_att, out,
                      lse, stream=None):
    st = L.load().sa_sparse_prefill(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens),
                                    _dev(q), _dev(k_pool), _dev(v_pool), _dt(q), _dev(idx),
                                    _dev(count), int(idx.shape[-1]), int(b_sel), float(s_att),
                                    _dev(out), _dt(out), _dev(lse), _stream(stream))
    L.check(st, "sa_sparse_prefill")


def sa_select_prefill_topk_probs(shape, pages, n_tokens, q, w_q, kidx_pool, s_idx, b_sel, k, idx,
                                 count, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_select_prefill_topk_probs(ctypes.byref(shape), ctypes.byref(pages),
                                               int(n_tokens), _dev(q), _dev(w_q), _dev(kidx_pool),
                                               _dt(q), float(s_idx), int(b_sel), int(k), _dev(idx),
                                               _dev(count), int(idx.shape[-1]), wp, wn,
                                               _stream(stream))
    L.check(st, "sa_select_prefill_topk_probs")


def sa_sparse_prefill_query(shape, pages, n_tokens, q, k_pool, v_pool, idx, count, s_att, out, lse,
                            ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_sparse_prefill_query(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens),
                                          _dev(q), _dev(k_pool), _dev(v_pool), _dt(q), _dev(idx),
                                          _dev(count), int(idx.shape[-1]), float(s_att), _dev(out),
                                          _dt(out), _dev(lse), wp, wn, _stream(stream))
    L.check(st, "sa_sparse_prefill_query")


def sa_pbs_importance(shape, pages, n_tokens, q, k_pool, s_att, n_rows, importance, ws, stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_pbs_importance(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens), _dev(q),
                                    _dev(k_pool), _dt(q), float(s_att), int(n_rows),
                                    _dev(importance), wp, wn, _stream(stream))
    L.check(st, "sa_pbs_importance")


def sa_pbs_permutation(shape, importance, n_tokens, seg, perm, stream=None):
    st = L.load().sa_pbs_permutation(ctypes.byref(shape), _dev(importance), int(n_tokens), int(seg),
                                     _dev(perm), _stream(stream))
    L.check(st, "sa_pbs_permutation")


def sa_pbs_select(shape, pages, n_tokens, q, k_pool, perm, seg, b_sel, k_blocks, idx, count, ws,
                  stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_pbs_select(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens), _dev(q),
                                _dev(k_pool), _dt(q), _dev(perm), int(seg), int(b_sel),
                                int(k_blocks), _dev(idx), _dev(count), int(idx.shape[-1]), wp, wn,
                                _stream(stream))
    L.check(st, "sa_pbs_select")


def sa_select_prefill_oracle(shape, pages, n_tokens, q, k_pool, s_att, b_sel, k, idx, count, ws,
                             stream=None):
    wp, wn = _ws(ws)
    st = L.load().sa_select_prefill_oracle(ctypes.byref(shape), ctypes.byref(pages), int(n_tokens),
                                           _dev(q), _dev(k_pool), _dt(q), float(s_att), int(b_sel),
                                           int(k), _dev(idx), _dev(count), int(idx.shape[-1]), wp,
                                           wn, _stream(stream))
    L.check(st, "sa_select_prefill_oracle")
