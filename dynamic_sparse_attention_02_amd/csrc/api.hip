// C ABI of libsa: host-side argument validation, workspace sizing and
// dispatch to the kernel launchers.  Every check happens before any launch so
// a rejected call has no side effect.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "sa_internal.h"

namespace {

constexpr int kMaxDecodeRows = 4096;  // (sequence, group) rows of one decode call

thread_local std::string g_err;

sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sa_status ok() {
  g_err.clear();
  return SA_OK;
}

sa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNotSupported) return fail(SA_ERR_UNSUPPORTED, "%s: not implemented", what);
  return fail(SA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool valid_dtype(sa_dtype d) { return d == SA_F32 || d == SA_BF16; }

// Shape checks shared by all calls.
sa_status check_shape(const sa_shape* s, const char* fn) {
  if (!s) return fail(SA_ERR_INVALID_ARGUMENT, "%s: shape is NULL", fn);
  if (s->batch < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: batch=%d must be >= 1", fn, s->batch);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: head counts must be >= 1", fn);
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_kv_heads=%d does not divide n_q_heads=%d", fn,
                s->n_kv_heads, s->n_q_heads);
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(SA_ERR_UNSUPPORTED, "%s: group size %d not in {1,2,4,8,16}", fn, G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "%s: head_dim=%d not in {64,128}", fn, s->head_dim);
  if (s->idx_rank != sa::kRank)
    return fail(SA_ERR_UNSUPPORTED, "%s: idx_rank=%d must be %d", fn, s->idx_rank, sa::kRank);
  if (s->page_size != sa::kPage)
    return fail(SA_ERR_UNSUPPORTED, "%s: page_size=%d must be %d", fn, s->page_size, sa::kPage);
  if (s->max_pages < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: max_pages must be >= 1", fn);
  if (s->max_len < 0 || (int64_t)s->max_len > (int64_t)s->max_pages * s->page_size)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: max_len=%d outside [0, max_pages*page_size=%lld]",
                fn, s->max_len, (long long)s->max_pages * s->page_size);
  if (s->max_len > (1 << 24))
    return fail(SA_ERR_UNSUPPORTED, "%s: max_len=%d above 2^24", fn, s->max_len);
  if (s->n_pool_pages < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_pool_pages must be >= 1", fn);
  return SA_OK;
}

sa::Shape to_shape(const sa_shape* s) {
  sa::Shape r;
  r.B = s->batch;
  r.Hq = s->n_q_heads;
  r.Hkv = s->n_kv_heads;
  r.D = s->head_dim;
  r.R = s->idx_rank;
  r.page = s->page_size;
  r.max_pages = s->max_pages;
  r.max_len = s->max_len;
  r.n_pool_pages = s->n_pool_pages;
  return r;
}

sa_status check_pages(const sa_pages* pg, bool need_lens, const char* fn) {
  if (!pg) return fail(SA_ERR_INVALID_ARGUMENT, "%s: pages is NULL", fn);
  if (!pg->page_table) return fail(SA_ERR_INVALID_ARGUMENT, "%s: page_table is NULL", fn);
  if (need_lens && !pg->seq_lens) return fail(SA_ERR_INVALID_ARGUMENT, "%s: seq_lens is NULL", fn);
  return SA_OK;
}

sa_status check_ws(void* ws, size_t have, size_t need, const char* fn) {
  if (need == 0) return SA_OK;
  if (!ws) return fail(SA_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (have < need)
    return fail(SA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, have, need);
  return SA_OK;
}

size_t index_ws(const sa_shape* s) {
  return sa::align_up((size_t)s->batch * s->n_kv_heads * sa::kRank * sizeof(float), 256);
}

size_t select_ws(const sa_shape* s, int64_t max_cand) {
  if (max_cand < 1) max_cand = 1;
  return sa::align_up(sa::select_workspace_bytes(s->batch * s->n_kv_heads, (int32_t)max_cand), 256);
}

size_t decode_ws(const sa_shape* s, int64_t cap, bool rla = false) {
  if (cap < 1) cap = 1;
  sa::Shape sh = to_shape(s);
  return sa::align_up(sa::decode_workspace_bytes(sh, (int32_t)cap, rla), 256);
}

size_t mass_ws(const sa_shape* s) {
  return sa::align_up(sa::mass_workspace_bytes(to_shape(s)), 256);
}

#define SA_TRY(expr)            \
  do {                          \
    sa_status _st = (expr);     \
    if (_st != SA_OK) return _st; \
  } while (0)

// Region of the persistent single-launch step, placed after the separate
// calls' regions so that a workspace shared by calls that take different
// paths (the plan depends on n_sink / n_window, not on the shape alone) never
// lets one path's state alias the other's.
size_t fused_region(const sa_shape* s) {
  const int rows = s->batch * s->n_kv_heads;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (rows > 16 || G < 4) return 0;
  return sa::align_up(sa::fused_workspace_bytes(rows, 256, G, s->head_dim), 256);
}

// Decode-step workspace: index | select | decode | fused step.
size_t step_ws(const sa_shape* s, int64_t cap) {
  return index_ws(s) + select_ws(s, s->max_len) + decode_ws(s, cap) + fused_region(s);
}

// The residual linear attention's sums in a decode step, after step_ws:
// room for either path's (per chunk, or per row, workgroup and head).
size_t step_rla_ws(const sa_shape* s, int64_t cap) {
  if (cap < 1) cap = 1;
  const sa::Shape sh = to_shape(s);
  size_t b = sa::decode_rla_part_bytes(sh, (int32_t)cap);
  if (fused_region(s)) {
    const size_t f = sa::fused_rla_bytes(s->batch * s->n_kv_heads, 256, s->n_q_heads / s->n_kv_heads,
                                         s->head_dim);
    if (f > b) b = f;
  }
  return sa::align_up(b, 256);
}

// Page-level step workspace: select | decode | fused step.
size_t step_pages_ws(const sa_shape* s, int64_t cap) {
  const int64_t n_cand = (s->max_len + s->page_size - 1) / s->page_size;
  return select_ws(s, n_cand) + decode_ws(s, cap) + fused_region(s);
}

int64_t topk_cap_needed(const sa_shape* s, int32_t k, int32_t unit, int32_t n_sink,
                        int32_t n_window) {
  int64_t need;
  if (unit == 1) need = (int64_t)(k < s->max_len ? k : s->max_len) + n_sink + n_window;
  else need = (int64_t)k * unit;
  return need < s->max_len ? need : s->max_len;
}

}  // namespace

extern "C" {

const char* sa_version(void) { return "sa 0.1 (gfx950)"; }

const char* sa_status_string(sa_status st) {
  switch (st) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARGUMENT: return "SA_ERR_INVALID_ARGUMENT";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_CAPACITY: return "SA_ERR_CAPACITY";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
  }
  return "SA_ERR_UNKNOWN";
}

const char* sa_last_error(void) { return g_err.c_str(); }

size_t sa_workspace_size(sa_op op, const sa_shape* s, int64_t param) {
  if (check_shape(s, "sa_workspace_size") != SA_OK) return 0;
  switch (op) {
    case SA_OP_INDEX_SCORES: return index_ws(s);
    case SA_OP_SELECT: return select_ws(s, param);
    case SA_OP_SPARSE_DECODE: return decode_ws(s, param);
    case SA_OP_PREFILL_SELECT: {
      sa::Shape sh = to_shape(s);
      return sa::align_up(sa::prefill_select_workspace_bytes(sh, (int32_t)param), 256);
    }
    case SA_OP_DECODE_STEP:
      return step_ws(s, param);
    case SA_OP_DECODE_STEP_PAGES:
      return step_pages_ws(s, param);
    case SA_OP_DECODE_STEP_RLA:
      return step_ws(s, param) + step_rla_ws(s, param);
    case SA_OP_SPARSE_DECODE_RLA:
      return decode_ws(s, param, true);
    case SA_OP_ATTENTION_MASS:
      return mass_ws(s);
    case SA_OP_PREFILL_ORACLE: {
      sa::Shape sh = to_shape(s);
      return sa::align_up(sa::prefill_oracle_workspace_bytes(sh, s->max_len), 256);
    }
    case SA_OP_PBS_IMPORTANCE: {
      sa::Shape sh = to_shape(s);
      return sa::align_up(sa::pbs_importance_workspace_bytes(sh, s->max_len, param < 1 ? 1 : (int32_t)param), 256);
    }
    case SA_OP_PBS_SELECT: {
      sa::Shape sh = to_shape(s);
      return sa::align_up(sa::pbs_select_workspace_bytes(sh, s->max_len, param < 1 ? 1 : (int32_t)param), 256);
    }
    case SA_OP_PREFILL_QUERY: {
      sa::Shape sh = to_shape(s);
      return sa::align_up(sa::prefill_query_workspace_bytes(sh, s->max_len, param < 1 ? 1 : (int32_t)param), 256);
    }
  }
  return 0;
}

sa_status sa_index_append(const sa_shape* s, const void* k_pre, const void* w_k, sa_dtype dt,
                          const int64_t* slot, int32_t T, void* kidx_pool, hipStream_t st) {
  const char* fn = "sa_index_append";
  SA_TRY(check_shape(s, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (T < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: T=%d < 0", fn, T);
  if (T > 0 && (!k_pre || !w_k || !slot || !kidx_pool))
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  return hip_status(sa::launch_index_append(to_shape(s), k_pre, w_k, dt, slot, T, kidx_pool, st), fn);
}

sa_status sa_page_stats(const sa_shape* s, const void* k_pool, sa_dtype dt, const int32_t* pages,
                        const int32_t* n_valid, int32_t n, void* stats_pool, hipStream_t st) {
  const char* fn = "sa_page_stats";
  SA_TRY(check_shape(s, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (n < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: n=%d < 0", fn, n);
  if (n > 0 && (!k_pool || !pages || !n_valid || !stats_pool))
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  return hip_status(sa::launch_page_stats(to_shape(s), k_pool, dt, pages, n_valid, n, stats_pool, st), fn);
}

sa_status sa_index_scores(const sa_shape* s, const sa_pages* pg, const void* q, const void* w_q,
                          const void* kidx_pool, sa_dtype dt, float s_idx, float* x, int64_t ldx,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_index_scores";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !w_q || !kidx_pool || !x) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ldx < s->max_len) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < max_len=%d", fn, (long long)ldx, s->max_len);
  if (!(s_idx == s_idx)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_idx is NaN", fn);
  SA_TRY(check_ws(ws, ws_bytes, index_ws(s), fn));
  return hip_status(sa::launch_index_scores(to_shape(s), *pg, q, w_q, kidx_pool, dt, s_idx, x, ldx,
                                            (float*)ws, st), fn);
}

sa_status sa_page_scores(const sa_shape* s, const sa_pages* pg, const void* q,
                         const void* stats_pool, sa_dtype dt, float s_att, float* x, int64_t ldx,
                         hipStream_t st) {
  const char* fn = "sa_page_scores";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !stats_pool || !x) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ldx < s->max_pages) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < max_pages=%d", fn, (long long)ldx, s->max_pages);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  return hip_status(sa::launch_page_scores(to_shape(s), *pg, q, stats_pool, dt, s_att, x, ldx, st), fn);
}

static sa_status select_common(const char* fn, const sa_shape* s, const sa_pages* pg,
                               const float* x, int64_t ldx, int32_t unit, int32_t n_sink,
                               int32_t n_window, int32_t* idx, int32_t* count, int32_t cap,
                               void* ws, size_t ws_bytes, int64_t cap_needed,
                               sa::SelectArgs& a) {
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!x || !idx || !count) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (unit != 1 && unit != s->page_size)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: unit=%d must be 1 or page_size", fn, unit);
  const int64_t max_cand = unit == 1 ? s->max_len : (s->max_len + unit - 1) / unit;
  if (ldx < max_cand) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < %lld candidates", fn, (long long)ldx, (long long)max_cand);
  if (n_sink < 0 || n_window < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_sink/n_window < 0", fn);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (cap < cap_needed)
    return fail(SA_ERR_CAPACITY, "%s: cap=%d below the worst-case support %lld", fn, cap, (long long)cap_needed);
  SA_TRY(check_ws(ws, ws_bytes, select_ws(s, max_cand), fn));
  a.x = x;
  a.ldx = ldx;
  a.seq_lens = pg->seq_lens;
  a.rows = s->batch * s->n_kv_heads;
  a.Hkv = s->n_kv_heads;
  a.max_len = s->max_len;
  a.unit = unit;
  a.max_cand = (int32_t)max_cand;
  a.n_sink = n_sink;
  a.n_window = n_window;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  return SA_OK;
}

sa_status sa_select_topp(const sa_shape* s, const sa_pages* pg, const float* x, int64_t ldx,
                         float p, int32_t n_sink, int32_t n_window, int32_t* idx, int32_t* count,
                         int32_t cap, void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_select_topp";
  if (!(p > 0.f && p <= 1.f)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: p=%g outside (0, 1]", fn, (double)p);
  sa::SelectArgs a{};
  SA_TRY(select_common(fn, s, pg, x, ldx, 1, n_sink, n_window, idx, count, cap, ws, ws_bytes,
                       s ? s->max_len : 0, a));
  a.is_topk = 0;
  a.p = p;
  a.k = 0;
  return hip_status(sa::launch_select(a, ws, st), fn);
}

sa_status sa_select_topk(const sa_shape* s, const sa_pages* pg, const float* x, int64_t ldx,
                         int32_t k, int32_t unit, int32_t n_sink, int32_t n_window, int32_t* idx,
                         int32_t* count, int32_t cap, void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_select_topk";
  if (k < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: k=%d < 1", fn, k);
  if (unit != 1 && (n_sink != 0 || n_window != 0))
    return fail(SA_ERR_UNSUPPORTED, "%s: sink/window tokens need unit=1", fn);
  SA_TRY(check_shape(s, fn));
  sa::SelectArgs a{};
  SA_TRY(select_common(fn, s, pg, x, ldx, unit, n_sink, n_window, idx, count, cap, ws, ws_bytes,
                       topk_cap_needed(s, k, unit, n_sink, n_window), a));
  a.is_topk = 1;
  a.p = 0.f;
  a.k = k;
  return hip_status(sa::launch_select(a, ws, st), fn);
}

sa_status sa_sparse_decode(const sa_shape* s, const sa_pages* pg, const void* q,
                           const void* k_pool, const void* v_pool, sa_dtype dt,
                           const int32_t* idx, const int32_t* count, int32_t cap, float s_att,
                           void* out, sa_dtype out_dt, float* lse, void* ws, size_t ws_bytes,
                           hipStream_t st) {
  const char* fn = "sa_sparse_decode";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !v_pool || !idx || !count || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  SA_TRY(check_ws(ws, ws_bytes, decode_ws(s, cap), fn));
  return hip_status(sa::launch_sparse_decode(to_shape(s), *pg, q, k_pool, v_pool, dt, idx, count,
                                             cap, s_att, out, out_dt, lse, ws, st), fn);
}

sa_status sa_sparse_decode_rla(const sa_shape* s, const sa_pages* pg, const void* q,
                               const void* k_pool, const void* v_pool, sa_dtype dt,
                               const int32_t* idx, const int32_t* count, int32_t cap, float s_att,
                               void* out, sa_dtype out_dt, float* lse, const float* rla_state,
                               float* rla_num, float* rla_den, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  const char* fn = "sa_sparse_decode_rla";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !v_pool || !idx || !count || !out || !rla_state || !rla_num || !rla_den)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  SA_TRY(check_ws(ws, ws_bytes, decode_ws(s, cap, true), fn));
  return hip_status(sa::launch_sparse_decode_rla(to_shape(s), *pg, q, k_pool, v_pool, dt, idx,
                                                 count, cap, s_att, out, out_dt, lse, rla_state,
                                                 rla_num, rla_den, ws, nullptr, st), fn);
}

sa_status sa_rla_state(const sa_shape* s, const sa_pages* pg, const void* k_pool,
                       const void* v_pool, sa_dtype dt, int32_t first_token, float* state,
                       hipStream_t st) {
  const char* fn = "sa_rla_state";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!k_pool || !v_pool || !state) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (first_token < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: first_token=%d < 0", fn, first_token);
  return hip_status(sa::launch_rla_state(to_shape(s), *pg, k_pool, v_pool, dt, first_token, state, st), fn);
}

sa_status sa_attention_mass(const sa_shape* s, const sa_pages* pg, const void* q,
                            const void* k_pool, sa_dtype dt, float s_att, float* x, int64_t ldx,
                            void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_attention_mass";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !x) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ldx < s->max_len) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < max_len=%d", fn, (long long)ldx, s->max_len);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  SA_TRY(check_ws(ws, ws_bytes, mass_ws(s), fn));
  return hip_status(sa::launch_attention_mass(to_shape(s), *pg, q, k_pool, dt, s_att, x, ldx, ws, st), fn);
}

sa_status sa_support_coverage(const sa_shape* s, const sa_pages* pg, const float* x, int64_t ldx,
                              const int32_t* idx, const int32_t* count, int32_t cap,
                              const int32_t* ref_idx, const int32_t* ref_count, int32_t ref_cap,
                              float* mass, int32_t* overlap, hipStream_t st) {
  const char* fn = "sa_support_coverage";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!x || !idx || !count || !mass) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ref_idx && (!ref_count || !overlap))
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: ref_idx given without ref_count/overlap", fn);
  if (ldx < s->max_len) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < max_len=%d", fn, (long long)ldx, s->max_len);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (ref_idx && ref_cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ref_cap=%d < 1", fn, ref_cap);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  return hip_status(sa::launch_coverage(to_shape(s), *pg, x, ldx, idx, count, cap, ref_idx,
                                        ref_idx ? ref_count : nullptr, ref_cap, mass,
                                        ref_idx ? overlap : nullptr, st), fn);
}

}  // extern "C"

namespace {

// Scratch of sa_decode_step_noalloc: one copy per device, held until the
// process ends.  Its front holds the persistent launches' zero part laid out
// for the most rows they serve, so every call finds it zero whatever its
// shape; the rest is the workspace of one call.  Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void k_zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Device address of this device's scratch; set up on the first call on a
// device (its zero part cleared once, by a fill kernel on the caller's
// stream).  NULL on failure.
void* scratch_on_device(hipStream_t st, hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !ptr) return nullptr;
  const size_t words = sa::fused_zero_bytes(sa::kFusedMaxRows) / 4;
  k_zero_words<<<256, 256, 0, st>>>((uint32_t*)ptr, words);
  *err = hipGetLastError();
  if (*err != hipSuccess) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

// sa_decode_step on the caller's workspace, or (use_scratch) on this
// device's scratch, whose front is the persistent launches' zero part; every
// argument is checked before the scratch is set up or anything launched.
sa_status decode_step_impl(const char* fn, const sa_shape* s, const sa_pages* pg, const void* q,
                           const void* w_q, const void* kidx_pool, const void* k_pool,
                           const void* v_pool, sa_dtype dt, float s_idx, float s_att, float p,
                           int32_t top_k, int32_t n_sink, int32_t n_window, float* x, int64_t ldx,
                           int32_t* idx, int32_t* count, int32_t cap, void* out, sa_dtype out_dt,
                           float* lse, void* ws, size_t ws_bytes, bool use_scratch,
                           const float* rla_state, float* rla_num, float* rla_den, hipStream_t st) {
  const bool rla = rla_state != nullptr;
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !w_q || !kidx_pool || !k_pool || !v_pool || !x || !idx || !count || !out ||
      (rla && (!rla_num || !rla_den)))
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ldx < s->max_len) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx < max_len", fn);
  if (top_k < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: top_k=%d < 0", fn, top_k);
  if (top_k == 0 && !(p > 0.f && p <= 1.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: p=%g outside (0, 1]", fn, (double)p);
  if (n_sink < 0 || n_window < 0) return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_sink/n_window < 0", fn);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  const int64_t cap_needed = top_k > 0 ? topk_cap_needed(s, top_k, 1, n_sink, n_window) : s->max_len;
  if (cap < 1 || cap < cap_needed)
    return fail(SA_ERR_CAPACITY, "%s: cap=%d below the worst-case support %lld", fn, cap, (long long)cap_needed);
  const size_t w_i = index_ws(s), w_s = select_ws(s, s->max_len), w_d = decode_ws(s, cap);
  void* zero = nullptr;
  if (use_scratch) {
    const size_t zb = sa::fused_zero_bytes(sa::kFusedMaxRows);
    const size_t need = zb + step_ws(s, cap);
    if (need > kScratchBytes)
      return fail(SA_ERR_WORKSPACE, "%s: this shape needs %zu bytes of scratch, above the %zu the "
                  "library holds per device (use sa_decode_step with a workspace)", fn, need,
                  kScratchBytes);
    hipError_t e = hipSuccess;
    char* sc = (char*)scratch_on_device(st, &e);
    if (!sc) return hip_status(e == hipSuccess ? hipErrorInvalidValue : e, fn);
    zero = sc;
    ws = sc + zb;
    ws_bytes = kScratchBytes - zb;
  }
  SA_TRY(check_ws(ws, ws_bytes, step_ws(s, cap) + (rla ? step_rla_ws(s, cap) : 0), fn));
  char* base = (char*)ws;
  char* rla_part = base + step_ws(s, cap);
  const sa::Shape sh = to_shape(s);
  int32_t nb = 0, tpb = 0;
  if ((!rla || dt == SA_BF16) && sa::fused_plan(sh, n_sink, n_window, dt, rla ? 3 : 0, &nb, &tpb)) {
    const sa::FusedRla fr{rla_state, rla_num, rla_den, rla_part};
    return hip_status(sa::launch_decode_fused(sh, *pg, q, w_q, kidx_pool, k_pool, v_pool, dt, s_idx,
                                              s_att, p, top_k, n_sink, n_window, x, ldx, idx, count,
                                              cap, out, out_dt, lse, base + w_i + w_s + w_d, zero, nb,
                                              tpb, rla ? &fr : nullptr, st), fn);
  }
  hipError_t e = sa::launch_index_scores(sh, *pg, q, w_q, kidx_pool, dt, s_idx, x, ldx, (float*)base, st);
  if (e != hipSuccess) return hip_status(e, fn);
  sa::SelectArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.seq_lens = pg->seq_lens;
  a.rows = s->batch * s->n_kv_heads;
  a.Hkv = s->n_kv_heads;
  a.max_len = s->max_len;
  a.unit = 1;
  a.max_cand = s->max_len;
  a.is_topk = top_k > 0;
  a.p = p;
  a.k = top_k;
  a.n_sink = n_sink;
  a.n_window = n_window;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  a.fused_zero = zero;
  e = sa::launch_select(a, base + w_i, st);
  if (e != hipSuccess) return hip_status(e, fn);
  if (rla)
    e = sa::launch_sparse_decode_rla(sh, *pg, q, k_pool, v_pool, dt, idx, count, cap, s_att, out,
                                     out_dt, lse, rla_state, rla_num, rla_den, base + w_i + w_s,
                                     rla_part, st);
  else
    e = sa::launch_sparse_decode(sh, *pg, q, k_pool, v_pool, dt, idx, count, cap, s_att, out,
                                 out_dt, lse, base + w_i + w_s, st);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

sa_status sa_decode_step(const sa_shape* s, const sa_pages* pg, const void* q, const void* w_q,
                         const void* kidx_pool, const void* k_pool, const void* v_pool,
                         sa_dtype dt, float s_idx, float s_att, float p, int32_t top_k,
                         int32_t n_sink, int32_t n_window, float* x, int64_t ldx, int32_t* idx,
                         int32_t* count, int32_t cap, void* out, sa_dtype out_dt, float* lse,
                         void* ws, size_t ws_bytes, hipStream_t st) {
  return decode_step_impl("sa_decode_step", s, pg, q, w_q, kidx_pool, k_pool, v_pool, dt, s_idx,
                          s_att, p, top_k, n_sink, n_window, x, ldx, idx, count, cap, out, out_dt,
                          lse, ws, ws_bytes, false, nullptr, nullptr, nullptr, st);
}

sa_status sa_decode_step_rla(const sa_shape* s, const sa_pages* pg, const void* q,
                             const void* w_q, const void* kidx_pool, const void* k_pool,
                             const void* v_pool, sa_dtype dt, float s_idx, float s_att, float p,
                             int32_t top_k, int32_t n_sink, int32_t n_window, float* x, int64_t ldx,
                             int32_t* idx, int32_t* count, int32_t cap, void* out, sa_dtype out_dt,
                             float* lse, const float* rla_state, float* rla_num, float* rla_den,
                             void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_decode_step_rla";
  if (!rla_state) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  return decode_step_impl(fn, s, pg, q, w_q, kidx_pool, k_pool, v_pool, dt, s_idx, s_att, p,
                          top_k, n_sink, n_window, x, ldx, idx, count, cap, out, out_dt, lse, ws,
                          ws_bytes, false, rla_state, rla_num, rla_den, st);
}

sa_status sa_decode_step_noalloc(const sa_shape* s, const sa_pages* pg, const void* q,
                                 const void* w_q, const void* kidx_pool, const void* k_pool,
                                 const void* v_pool, sa_dtype dt, float s_idx, float s_att, float p,
                                 int32_t top_k, int32_t n_sink, int32_t n_window, float* x,
                                 int64_t ldx, int32_t* idx, int32_t* count, int32_t cap, void* out,
                                 sa_dtype out_dt, float* lse, hipStream_t st) {
  return decode_step_impl("sa_decode_step_noalloc", s, pg, q, w_q, kidx_pool, k_pool, v_pool, dt,
                          s_idx, s_att, p, top_k, n_sink, n_window, x, ldx, idx, count, cap, out,
                          out_dt, lse, nullptr, 0, true, nullptr, nullptr, nullptr, st);
}

sa_status sa_decode_step_pages(const sa_shape* s, const sa_pages* pg, const void* q,
                               const void* stats_pool, const void* k_pool, const void* v_pool,
                               sa_dtype dt, float s_att, int32_t top_k, float* x, int64_t ldx,
                               int32_t* idx, int32_t* count, int32_t cap, void* out,
                               sa_dtype out_dt, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  const char* fn = "sa_decode_step_pages";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, true, fn));
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !stats_pool || !k_pool || !v_pool || !x || !idx || !count || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (ldx < s->max_pages) return fail(SA_ERR_INVALID_ARGUMENT, "%s: ldx=%lld < max_pages=%d", fn, (long long)ldx, s->max_pages);
  if (top_k < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: top_k=%d < 1", fn, top_k);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  if ((int64_t)s->batch * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: batch * n_kv_heads above %d", fn, kMaxDecodeRows);
  const int64_t cap_needed = topk_cap_needed(s, top_k, s->page_size, 0, 0);
  if (cap < 1 || cap < cap_needed)
    return fail(SA_ERR_CAPACITY, "%s: cap=%d below the worst-case support %lld", fn, cap, (long long)cap_needed);
  SA_TRY(check_ws(ws, ws_bytes, step_pages_ws(s, cap), fn));
  const sa::Shape sh = to_shape(s);
  const int64_t n_cand = (s->max_len + s->page_size - 1) / s->page_size;
  const size_t w_s = select_ws(s, n_cand);
  char* base = (char*)ws;
  int32_t nb = 0, tpb = 0;
  if (dt == SA_BF16 && sa::fused_plan_pages(sh, top_k, &nb, &tpb))
    return hip_status(sa::launch_decode_fused_pages(sh, *pg, q, stats_pool, k_pool, v_pool, s_att,
                                                    top_k, x, ldx, idx, count, cap, out, out_dt,
                                                    lse, base + w_s + decode_ws(s, cap), nullptr,
                                                    nb, tpb, st), fn);
  hipError_t e = sa::launch_page_scores(sh, *pg, q, stats_pool, dt, s_att, x, ldx, st);
  if (e != hipSuccess) return hip_status(e, fn);
  sa::SelectArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.seq_lens = pg->seq_lens;
  a.rows = s->batch * s->n_kv_heads;
  a.Hkv = s->n_kv_heads;
  a.max_len = s->max_len;
  a.unit = s->page_size;
  a.max_cand = (int32_t)n_cand;
  a.is_topk = 1;
  a.p = 0.f;
  a.k = top_k;
  a.n_sink = 0;
  a.n_window = 0;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  e = sa::launch_select(a, base, st);
  if (e != hipSuccess) return hip_status(e, fn);
  e = sa::launch_sparse_decode(sh, *pg, q, k_pool, v_pool, dt, idx, count, cap, s_att, out, out_dt,
                               lse, base + w_s, st);
  return hip_status(e, fn);
}

static sa_status prefill_select_common(const char* fn, const sa_shape* s, const sa_pages* pg,
                                       int32_t n_tokens, const void* q, const void* w_q,
                                       const void* kidx_pool, sa_dtype dt, float s_idx,
                                       int32_t b_sel, int32_t k, int32_t* idx, int32_t* count,
                                       int32_t cap, void* ws, size_t ws_bytes, hipStream_t st,
                                       bool probs) {
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, false, fn));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (s->batch != 1) return fail(SA_ERR_UNSUPPORTED, "%s: prefill takes batch=1", fn);
  if (!q || !w_q || !kidx_pool || !idx || !count) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (n_tokens < 1 || n_tokens > s->max_len)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_tokens=%d outside [1, max_len=%d]", fn, n_tokens, s->max_len);
  if (probs ? b_sel != 1 : (b_sel != 64 && b_sel != 1))
    return fail(SA_ERR_UNSUPPORTED, "%s: b_sel=%d must be %s", fn, b_sel, probs ? "1" : "1 or 64");
  if (k < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: k=%d < 1", fn, k);
  const int64_t kk = b_sel == 1 ? (int64_t)k + 1 : (int64_t)k;  // per query: plus the own token
  const int64_t need = kk < n_tokens ? kk : n_tokens;
  if (cap < 1 || cap < need) return fail(SA_ERR_CAPACITY, "%s: cap=%d below %lld", fn, cap, (long long)need);
  const sa::Shape sh = to_shape(s);
  SA_TRY(check_ws(ws, ws_bytes, sa::align_up(sa::prefill_select_workspace_bytes(sh, n_tokens), 256), fn));
  return hip_status(sa::launch_prefill_select(sh, *pg, n_tokens, q, w_q, kidx_pool, dt, s_idx, b_sel,
                                              k, idx, count, cap, ws, st, probs), fn);
}

sa_status sa_select_prefill_topk(const sa_shape* s, const sa_pages* pg, int32_t n_tokens,
                                 const void* q, const void* w_q, const void* kidx_pool,
                                 sa_dtype dt, float s_idx, int32_t b_sel, int32_t k, int32_t* idx,
                                 int32_t* count, int32_t cap, void* ws, size_t ws_bytes,
                                 hipStream_t st) {
  return prefill_select_common("sa_select_prefill_topk", s, pg, n_tokens, q, w_q, kidx_pool, dt,
                               s_idx, b_sel, k, idx, count, cap, ws, ws_bytes, st, false);
}

sa_status sa_select_prefill_topk_probs(const sa_shape* s, const sa_pages* pg, int32_t n_tokens,
                                       const void* q, const void* w_q, const void* kidx_pool,
                                       sa_dtype dt, float s_idx, int32_t b_sel, int32_t k,
                                       int32_t* idx, int32_t* count, int32_t cap, void* ws,
                                       size_t ws_bytes, hipStream_t st) {
  return prefill_select_common("sa_select_prefill_topk_probs", s, pg, n_tokens, q, w_q, kidx_pool,
                               dt, s_idx, b_sel, k, idx, count, cap, ws, ws_bytes, st, true);
}

sa_status sa_sparse_prefill_query(const sa_shape* s, const sa_pages* pg, int32_t n_tokens,
                                  const void* q, const void* k_pool, const void* v_pool,
                                  sa_dtype dt, const int32_t* idx, const int32_t* count,
                                  int32_t cap, float s_att, void* out, sa_dtype out_dt, float* lse,
                                  void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_sparse_prefill_query";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, false, fn));
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (s->batch != 1) return fail(SA_ERR_UNSUPPORTED, "%s: prefill takes batch=1", fn);
  if (!q || !k_pool || !v_pool || !idx || !count || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (n_tokens < 1 || n_tokens > s->max_len)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_tokens=%d outside [1, max_len=%d]", fn, n_tokens, s->max_len);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  if (s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: n_kv_heads above %d", fn, kMaxDecodeRows);
  const sa::Shape sh = to_shape(s);
  SA_TRY(check_ws(ws, ws_bytes, sa::align_up(sa::prefill_query_workspace_bytes(sh, n_tokens, cap), 256), fn));
  return hip_status(sa::launch_sparse_prefill_query(sh, *pg, n_tokens, q, k_pool, v_pool, dt, idx,
                                                    count, cap, s_att, out, out_dt, lse, ws, st), fn);
}

static sa_status pbs_common(const char* fn, const sa_shape* s, const sa_pages* pg, int32_t n_tokens) {
  SA_TRY(check_shape(s, fn));
  if (pg) SA_TRY(check_pages(pg, false, fn));
  if (s->batch != 1) return fail(SA_ERR_UNSUPPORTED, "%s: prefill takes batch=1", fn);
  if (n_tokens < 1 || n_tokens > s->max_len)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_tokens=%d outside [1, max_len=%d]", fn, n_tokens, s->max_len);
  return SA_OK;
}

sa_status sa_select_prefill_oracle(const sa_shape* s, const sa_pages* pg, int32_t n_tokens,
                                  const void* q, const void* k_pool, sa_dtype dt, float s_att,
                                  int32_t b_sel, int32_t k, int32_t* idx, int32_t* count,
                                  int32_t cap, void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_select_prefill_oracle";
  if (!pg) return fail(SA_ERR_INVALID_ARGUMENT, "%s: pages is NULL", fn);
  SA_TRY(pbs_common(fn, s, pg, n_tokens));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !idx || !count) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (b_sel != 1 && b_sel != 64) return fail(SA_ERR_UNSUPPORTED, "%s: b_sel=%d must be 1 or 64", fn, b_sel);
  if (k < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: k=%d < 1", fn, k);
  if (s->n_kv_heads > 64) return fail(SA_ERR_UNSUPPORTED, "%s: n_kv_heads above 64", fn);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  const int64_t kk = b_sel == 1 ? (int64_t)k + 1 : (int64_t)k;
  const int64_t need = kk < n_tokens ? kk : n_tokens;
  if (cap < 1 || cap < need) return fail(SA_ERR_CAPACITY, "%s: cap=%d below %lld", fn, cap, (long long)need);
  const sa::Shape sh = to_shape(s);
  SA_TRY(check_ws(ws, ws_bytes, sa::align_up(sa::prefill_oracle_workspace_bytes(sh, n_tokens), 256), fn));
  return hip_status(sa::launch_prefill_oracle_select(sh, *pg, n_tokens, q, k_pool, dt, s_att, b_sel,
                                                     k, idx, count, cap, ws, st), fn);
}

sa_status sa_pbs_importance(const sa_shape* s, const sa_pages* pg, int32_t n_tokens, const void* q,
                            const void* k_pool, sa_dtype dt, float s_att, int32_t n_rows,
                            float* importance, void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_pbs_importance";
  if (!pg) return fail(SA_ERR_INVALID_ARGUMENT, "%s: pages is NULL", fn);
  SA_TRY(pbs_common(fn, s, pg, n_tokens));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !importance) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (n_rows < 1 || n_rows > n_tokens)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_rows=%d outside [1, n_tokens=%d]", fn, n_rows, n_tokens);
  if ((int64_t)n_rows * s->n_kv_heads > kMaxDecodeRows)
    return fail(SA_ERR_UNSUPPORTED, "%s: n_rows * n_kv_heads above %d", fn, kMaxDecodeRows);
  if (!(s_att == s_att)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: s_att is NaN", fn);
  const sa::Shape sh = to_shape(s);
  SA_TRY(check_ws(ws, ws_bytes, sa::align_up(sa::pbs_importance_workspace_bytes(sh, n_tokens, n_rows), 256), fn));
  return hip_status(sa::launch_pbs_importance(sh, *pg, n_tokens, q, k_pool, dt, s_att, n_rows,
                                              importance, ws, st), fn);
}

sa_status sa_pbs_permutation(const sa_shape* s, const float* importance, int32_t n_tokens,
                             int32_t seg, int32_t* perm, hipStream_t st) {
  const char* fn = "sa_pbs_permutation";
  SA_TRY(pbs_common(fn, s, nullptr, n_tokens));
  if (!importance || !perm) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (seg < 64 || seg > 4096 || seg % 64 != 0)
    return fail(SA_ERR_UNSUPPORTED, "%s: seg=%d must be a multiple of 64 in [64, 4096]", fn, seg);
  return hip_status(sa::launch_pbs_permutation(to_shape(s), importance, n_tokens, seg, perm, st), fn);
}

sa_status sa_pbs_select(const sa_shape* s, const sa_pages* pg, int32_t n_tokens, const void* q,
                        const void* k_pool, sa_dtype dt, const int32_t* perm, int32_t seg,
                        int32_t b_sel, int32_t k_blocks, int32_t* idx, int32_t* count, int32_t cap,
                        void* ws, size_t ws_bytes, hipStream_t st) {
  const char* fn = "sa_pbs_select";
  if (!pg) return fail(SA_ERR_INVALID_ARGUMENT, "%s: pages is NULL", fn);
  SA_TRY(pbs_common(fn, s, pg, n_tokens));
  if (!valid_dtype(dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad dtype", fn);
  if (!q || !k_pool || !perm || !idx || !count) return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (b_sel != 64) return fail(SA_ERR_UNSUPPORTED, "%s: b_sel=%d must be 64", fn, b_sel);
  if (seg < 64 || seg > 4096 || seg % 64 != 0)
    return fail(SA_ERR_UNSUPPORTED, "%s: seg=%d must be a multiple of 64 in [64, 4096]", fn, seg);
  if (k_blocks < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: k_blocks=%d < 1", fn, k_blocks);
  const int64_t nblk = (n_tokens + 63) / 64;
  const int64_t kb = k_blocks < nblk - 1 ? k_blocks : (nblk - 1 > 0 ? nblk - 1 : 0);
  if (cap < 1 || cap < kb * 64) return fail(SA_ERR_CAPACITY, "%s: cap=%d below %lld", fn, cap, (long long)(kb * 64));
  const sa::Shape sh = to_shape(s);
  SA_TRY(check_ws(ws, ws_bytes, sa::align_up(sa::pbs_select_workspace_bytes(sh, n_tokens, k_blocks), 256), fn));
  return hip_status(sa::launch_pbs_select(sh, *pg, n_tokens, q, k_pool, dt, perm, seg, k_blocks, idx,
                                          count, cap, ws, st), fn);
}

sa_status sa_sparse_prefill(const sa_shape* s, const sa_pages* pg, int32_t n_tokens, const void* q,
                            const void* k_pool, const void* v_pool, sa_dtype dt, const int32_t* idx,
                            const int32_t* count, int32_t cap, int32_t b_sel, float s_att, void* out,
                            sa_dtype out_dt, float* lse, hipStream_t st) {
  const char* fn = "sa_sparse_prefill";
  SA_TRY(check_shape(s, fn));
  SA_TRY(check_pages(pg, false, fn));
  if (dt != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "%s: inputs must be bf16", fn);
  if (!valid_dtype(out_dt)) return fail(SA_ERR_INVALID_ARGUMENT, "%s: bad out dtype", fn);
  if (s->batch != 1) return fail(SA_ERR_UNSUPPORTED, "%s: prefill takes batch=1", fn);
  if (!q || !k_pool || !v_pool || !idx || !count || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
  if (n_tokens < 1 || n_tokens > s->max_len)
    return fail(SA_ERR_INVALID_ARGUMENT, "%s: n_tokens=%d outside [1, max_len=%d]", fn, n_tokens, s->max_len);
  if (b_sel != 64)
    return fail(SA_ERR_UNSUPPORTED, "%s: b_sel=%d must be 64 (per query: sa_sparse_prefill_query)", fn, b_sel);
  if (cap < 1) return fail(SA_ERR_INVALID_ARGUMENT, "%s: cap=%d < 1", fn, cap);
  if (cap > 2048) return fail(SA_ERR_UNSUPPORTED, "%s: cap=%d above 2048 listed keys", fn, cap);
  if (s->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "%s: head_dim must be 128", fn);
  return hip_status(sa::launch_sparse_prefill(to_shape(s), *pg, n_tokens, q, k_pool, v_pool, idx,
                                              count, cap, b_sel, s_att, out, out_dt, lse, st), fn);
}

}  // extern "C"
