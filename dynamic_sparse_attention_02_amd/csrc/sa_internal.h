// Internal declarations shared by the HIP translation units of libsa.
// Device helpers (dtype conversion, order-preserving score keys, wave and
// block reductions) and the host-side launch entry points each kernel file
// provides to the C ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa.h"

namespace sa {

constexpr int kPage = 64;   // tokens per page
constexpr int kRank = 16;   // indexer rank r
constexpr int kWave = 64;   // CDNA wavefront width

// bf16 values are stored as raw 16-bit patterns.
typedef uint16_t bf16_raw;

__device__ __forceinline__ float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// Round-to-nearest-even fp32 -> bf16 (quiet NaN kept).
__device__ __forceinline__ bf16_raw f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_raw)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_raw)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_raw>(bf16_raw v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_raw from_f32<bf16_raw>(float v) { return f32_to_bf16(v); }

// Order-preserving map of an fp32 score to uint32: a < b  <=>  key(a) < key(b);
// -0 and +0 map to the same key (adding +0 turns -0 into +0).  Negative
// scores have every bit flipped, the others only the sign bit.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Cross-lane helpers on DPP row operations (16-lane rows) and readlane; no
// LDS round trips.  Reductions return the same value in every lane (taken
// from lanes 0, 16, 32, 48 in a fixed order, so the result is uniform).
#define SA_DPP(v, ctrl) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), 0xF, 0xF, true))
#define SA_DPP_ROWS(v, ctrl, rows) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), (rows), 0xF, true))
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <typename Op>
__device__ __forceinline__ uint32_t row_allreduce_bits(uint32_t v, Op op) {
  v = op(v, SA_DPP(v, kDppXor1));
  v = op(v, SA_DPP(v, kDppXor2));
  v = op(v, SA_DPP(v, kDppHalfMirror));
  v = op(v, SA_DPP(v, kDppMirror));
  return v;
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_bits(uint32_t v, Op op) {
  v = row_allreduce_bits(v, op);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_allreduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_allreduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_allreduce_bits(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_allreduce_bits(v, [](uint32_t a, uint32_t b) { return a + b; });
}
// Inclusive prefix sum across the wave: Kogge-Stone inside each row, then
// the row totals carried into the rows above (row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += SA_DPP(v, kDppShr1);
  v += SA_DPP(v, kDppShr2);
  v += SA_DPP(v, kDppShr4);
  v += SA_DPP(v, kDppShr8);
  v += SA_DPP_ROWS(v, kDppBcast15, 0xA);
  v += SA_DPP_ROWS(v, kDppBcast31, 0xC);
  return v;
}

__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v) {
  return wave_incl_scan(v) - v;
}

// Maximum over the four lanes i, i ^ 16, i ^ 32, i ^ 48 (the same position
// in each 16-lane row), by the gfx950 row swaps (no LDS round trip); every
// lane receives the result.
__device__ __forceinline__ float row4_max(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Sum / maximum over each aligned group of 16 lanes (a DPP row); every lane
// of the row receives its row's value.
__device__ __forceinline__ float row16_sum(float v) {
  return __uint_as_float(row_allreduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ float row16_max(float v) {
  return __uint_as_float(row_allreduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
// ---------------------------------------------------------------------------
// Taylor page scores ("SPLA", section 2.1, diagonal covariance), shared by
// the page-score kernel and the fused page step so
// both form every score with the same operations in the same order: a page
// is spread over D / 8 lanes, 8 dimensions each.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16_raw>(const bf16_raw* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Sum over aligned groups of N lanes (N = 8 or 16) with DPP row operations;
// every lane of the group receives the total.
template <int N>
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
  if (N == 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

// The group's scaled query q'_h = s_att q_h in LDS: the sum over heads
// s_qs[e] = sum_h q'_h[e] and the squares s_qq[h][e] = q'_h[e]^2 (nt threads
// of the block take part; the caller synchronises).
template <typename T, int D, int G>
__device__ __forceinline__ void stage_page_query(const T* qg, float s_att, float* s_qs,
                                                 float (*s_qq)[D], int nt) {
  for (int e = threadIdx.x; e < D; e += nt) {
    float sum = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qp = s_att * to_f32<T>(qg[h * D + e]);
      sum += qp;
      s_qq[h][e] = qp * qp;
    }
    s_qs[e] = sum;
  }
}
// This lane's 8 dimensions (sub = lane within the page's lanes) of them.
template <int D, int G>
__device__ __forceinline__ void page_query_lane(const float* s_qs, const float (*s_qq)[D], int sub,
                                                float (&qs)[8], float (&qq)[G][8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) qs[e] = s_qs[sub * 8 + e];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qq[h][e] = s_qq[h][sub * 8 + e];
}
// One step of a reduce-scatter over the lanes of a page: the lanes split in
// two halves by the DPP pairing CTRL (each lane's partner sits in the other
// half); a lane keeps half of its N partial sums (the lower half the first
// N / 2, the upper half the rest), adding its partner's partials of those.
// With one sum left the step adds the partner's whole sum instead.
template <int N, int CTRL>
__device__ __forceinline__ void page_reduce_step(float* v, int sub, int bit) {
  if constexpr (N > 1) {
    const bool upper = (sub & bit) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = upper ? v[N / 2 + i] : v[i];
      const float send = upper ? v[i] : v[N / 2 + i];
      v[i] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xF, 0xF, true));
    }
  } else {
    v[0] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[0]), CTRL, 0xF, 0xF, true));
  }
}
// sum_h [q'_h . mean + log(1 + 0.5 q'_h^2 . var)] of the page whose 8 mean and
// variance dimensions of this lane are mu, va; every lane of the page gets it.
// The G per-head variance sums are reduce-scattered over the page's lanes
// (widest pairing first), so each lane ends holding whole sums of
// max(1, G / LPP) heads, each head held by max(1, LPP / G) lanes; every lane
// takes the logarithm of its own, and one row sum adds them (scaled by the
// repetition) to the mean term.
template <int LPP, int G>
__device__ __forceinline__ float page_score_sum(const float (&mu)[8], const float (&va)[8],
                                                const float (&qs)[8], const float (&qq)[G][8],
                                                int sub) {
  static_assert(LPP == 8 || LPP == 16, "a page spreads over 8 or 16 lanes");
  float first = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) first = fmaf(qs[e], mu[e], first);
  float v[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float c = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) c = fmaf(qq[h][e], va[e], c);
    v[h] = c;
  }
  constexpr int N0 = G;
  constexpr int N1 = LPP == 16 ? (N0 > 1 ? N0 / 2 : 1) : N0;
  constexpr int N2 = N1 > 1 ? N1 / 2 : 1;
  constexpr int N3 = N2 > 1 ? N2 / 2 : 1;
  constexpr int N4 = N3 > 1 ? N3 / 2 : 1;
  if constexpr (LPP == 16) page_reduce_step<N0, kDppMirror>(v, sub, 8);
  page_reduce_step<N1, kDppHalfMirror>(v, sub, 4);
  page_reduce_step<N2, kDppXor2>(v, sub, 2);
  page_reduce_step<N3, kDppXor1>(v, sub, 1);
  constexpr int DUP = LPP / G > 1 ? LPP / G : 1;  // lanes holding each head's sum
  float lp = 0.f;
#pragma unroll
  for (int i = 0; i < N4; ++i) lp += __logf(1.0f + 0.5f * v[i]);
  return row_sum<LPP>(first + lp * (1.0f / (float)DUP));
}
// The page score: the head mean plus log(valid tokens / page size).
template <int G>
__device__ __forceinline__ float page_score_final(float sum, int32_t L, int32_t page) {
  const int nv = (L - page * kPage) < kPage ? (L - page * kPage) : kPage;
  return sum * (1.0f / (float)G) + (nv < kPage ? __logf((float)nv * (1.0f / (float)kPage)) : 0.f);
}

// Value of a lane chosen by a wave-uniform index.
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int src) {
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), src) << 32) | lane_u32((uint32_t)v, src);
}

// 64-bit sums on the same DPP patterns, as (lo, hi) halves with a carry.
__device__ __forceinline__ void add_u64_parts(uint32_t& lo, uint32_t& hi, uint32_t lo2, uint32_t hi2) {
  const uint32_t nl = lo + lo2;
  hi = hi + hi2 + (nl < lo ? 1u : 0u);
  lo = nl;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  add_u64_parts(lo, hi, SA_DPP(lo, kDppXor1), SA_DPP(hi, kDppXor1));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppXor2), SA_DPP(hi, kDppXor2));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppHalfMirror), SA_DPP(hi, kDppHalfMirror));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppMirror), SA_DPP(hi, kDppMirror));
  uint64_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * i) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * i);
  return (r[0] + r[1]) + (r[2] + r[3]);
}
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  add_u64_parts(lo, hi, SA_DPP(lo, kDppShr1), SA_DPP(hi, kDppShr1));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppShr2), SA_DPP(hi, kDppShr2));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppShr4), SA_DPP(hi, kDppShr4));
  add_u64_parts(lo, hi, SA_DPP(lo, kDppShr8), SA_DPP(hi, kDppShr8));
  add_u64_parts(lo, hi, SA_DPP_ROWS(lo, kDppBcast15, 0xA), SA_DPP_ROWS(hi, kDppBcast15, 0xA));
  add_u64_parts(lo, hi, SA_DPP_ROWS(lo, kDppBcast31, 0xC), SA_DPP_ROWS(hi, kDppBcast31, 0xC));
  return ((uint64_t)hi << 32) | lo;
}

// Clamp helpers for caller-provided paging data (never fault on bad input).
__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}
__device__ __forceinline__ int64_t clamp_page(int32_t p, int64_t n_pool_pages) {
  return (p < 0) ? 0 : ((int64_t)p >= n_pool_pages ? n_pool_pages - 1 : (int64_t)p);
}

// Plain-old-data copy of sa_shape for kernel arguments.
struct Shape {
  int32_t B, Hq, Hkv, D, R, page, max_pages, max_len;
  int64_t n_pool_pages;
};

// ---------------------------------------------------------------------------
// Host launchers (each defined in the kernel's own translation unit).
// They assume validated arguments and return the launch status.
// ---------------------------------------------------------------------------

hipError_t launch_index_append(const Shape& s, const void* k_pre, const void* w_k, sa_dtype dt,
                               const int64_t* slot, int32_t T, void* kidx_pool,
                               hipStream_t st);
hipError_t launch_page_stats(const Shape& s, const void* k_pool, sa_dtype dt,
                             const int32_t* pages, const int32_t* n_valid, int32_t n,
                             void* stats_pool, hipStream_t st);
hipError_t launch_index_scores(const Shape& s, const sa_pages& pg, const void* q,
                               const void* w_q, const void* kidx_pool, sa_dtype dt,
                               float s_idx, float* x, int64_t ldx, float* qc_ws,
                               hipStream_t st);
hipError_t launch_page_scores(const Shape& s, const sa_pages& pg, const void* q,
                              const void* stats_pool, sa_dtype dt, float s_att, float* x,
                              int64_t ldx, hipStream_t st);

// Selection.  mode: 0 = top-p (param_p), 1 = top-k (param_k).
struct SelectArgs {
  const float* x;
  int64_t ldx;
  const int32_t* seq_lens;  // candidates per row derive from seq_lens[b]
  int32_t rows, Hkv, max_len;
  int32_t unit;             // 1 = tokens, page = pages expanded to tokens
  int32_t max_cand;         // upper bound on candidates per row
  int32_t is_topk;
  float p;
  int32_t k;
  int32_t n_sink, n_window;
  int32_t* idx;
  int32_t* count;
  int32_t cap;
  // prefill rows: row r (= (blk - prefill_blk0) * Hkv + g) has
  // prefill_bsel * blk candidates; 0 for decode rows
  int32_t prefill_bsel;
  int32_t prefill_blk0;
  int32_t prefill_self;     // per-query rows: the own token is a candidate too
  // 16-bit key rows (prefill top-k, rows of at most kSelectRowMax candidates):
  // x then holds ldx 32-bit words per row, candidate c's top 16 key bits in
  // word (c / 128) * 64 + c % 64 (low half for c % 128 < 64, else high), and
  // the threshold bin's exact scores are recomputed from qcb and kidx.
  int32_t key16;
  const float* qcb;         // [blocks][Hkv][16] block-mean low-rank queries
  const void* kidx;         // indexer key pool [pages][Hkv][64][16]
  int32_t kidx_bf16;
  const int32_t* pt;        // the sequence's page-table row
  int64_t n_pool_pages;
  // host side: the zero part the persistent few-row launch uses instead of
  // the one in its workspace region (NULL: its own)
  void* fused_zero;
};
constexpr int kSelectRowMax = 131072;  // longest row the one-block-per-row selection takes
size_t select_workspace_bytes(int32_t rows, int32_t max_cand);
hipError_t launch_select(const SelectArgs& a, void* ws, hipStream_t st);

size_t decode_workspace_bytes(const Shape& s, int32_t cap, bool rla = false);
// the residual linear attention's per-chunk sums, the part of
// decode_workspace_bytes(rla = true) beyond decode_workspace_bytes(rla = false)
size_t decode_rla_part_bytes(const Shape& s, int32_t cap);
// rla_part: where the per-chunk sums go, or NULL for their place after the
// other partials in ws
hipError_t launch_sparse_decode_rla(const Shape& s, const sa_pages& pg, const void* q,
                                    const void* k_pool, const void* v_pool, sa_dtype dt,
                                    const int32_t* idx, const int32_t* count, int32_t cap,
                                    float s_att, void* out, sa_dtype out_dt, float* lse,
                                    const float* rla_state, float* rla_num, float* rla_den,
                                    void* ws, void* rla_part, hipStream_t st);
hipError_t launch_rla_state(const Shape& s, const sa_pages& pg, const void* k_pool,
                            const void* v_pool, sa_dtype dt, int32_t first, float* state,
                            hipStream_t st);
hipError_t launch_sparse_decode(const Shape& s, const sa_pages& pg, const void* q,
                                const void* k_pool, const void* v_pool, sa_dtype dt,
                                const int32_t* idx, const int32_t* count, int32_t cap,
                                float s_att, void* out, sa_dtype out_dt, float* lse,
                                void* ws, hipStream_t st);

size_t prefill_select_workspace_bytes(const Shape& s, int32_t n_tokens);
hipError_t launch_prefill_select(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* w_q, const void* kidx_pool,
                                 sa_dtype dt, float s_idx, int32_t b_sel, int32_t k,
                                 int32_t* idx, int32_t* count, int32_t cap, void* ws,
                                 hipStream_t st, bool probs = false);
constexpr int32_t kPrefillQuerySlab = 512;  // query rows per per-query attention launch
size_t prefill_query_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t cap);
hipError_t launch_sparse_prefill_query(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       sa_dtype dt, const int32_t* idx, const int32_t* count,
                                       int32_t cap, float s_att, void* out, sa_dtype out_dt,
                                       float* lse, void* ws, hipStream_t st);
hipError_t launch_sparse_prefill(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* idx, const int32_t* count, int32_t cap,
                                 int32_t b_sel, float s_att, void* out, sa_dtype out_dt,
                                 float* lse, hipStream_t st);

constexpr int kFusedMaxRows = 16;  // rows a persistent launch serves at most
size_t fused_workspace_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D);
// the persistent step's residual linear attention sums (per row, workgroup
// and head), a region of their own
size_t fused_rla_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D);
struct FusedRla {
  const float* state;  // [B][Hkv][D + 1][D]
  float* num;          // [B][Hq][D]
  float* den;          // [B][Hq]
  void* part;          // fused_rla_bytes
};
size_t fused_zero_bytes(int32_t rows_cap);
// mode 0: token step, 1: page step, 2: selection only, 3: token step with
// the residual linear attention (bf16)
bool fused_plan(const Shape& s, int32_t n_sink, int32_t n_window, sa_dtype dt, int mode,
                int32_t* nb, int32_t* tpb);
bool fused_plan_pages(const Shape& s, int32_t top_k, int32_t* nb, int32_t* tpb);
bool select_fused_plan(const SelectArgs& sa, int32_t* nb, int32_t* tpb);
hipError_t launch_select_fused(const SelectArgs& sa, void* ws, int32_t nb, int32_t tpb,
                               hipStream_t st);
hipError_t launch_decode_fused_pages(const Shape& s, const sa_pages& pg, const void* q,
                                     const void* stats_pool, const void* k_pool, const void* v_pool,
                                     float s_att, int32_t top_k, float* x, int64_t ldx,
                                     int32_t* idx, int32_t* count, int32_t cap, void* out,
                                     sa_dtype out_dt, float* lse, void* ws, void* zero, int32_t nb,
                                     int32_t tpb, hipStream_t st);
hipError_t launch_decode_fused(const Shape& s, const sa_pages& pg, const void* q, const void* w_q,
                               const void* kidx_pool, const void* k_pool, const void* v_pool,
                               sa_dtype dt, float s_idx, float s_att, float p, int32_t top_k,
                               int32_t n_sink, int32_t n_window, float* x, int64_t ldx,
                               int32_t* idx, int32_t* count, int32_t cap, void* out,
                               sa_dtype out_dt, float* lse, void* ws, void* zero, int32_t nb,
                               int32_t tpb, const FusedRla* rla, hipStream_t st);

size_t mass_workspace_bytes(const Shape& s);
hipError_t launch_attention_mass(const Shape& s, const sa_pages& pg, const void* q,
                                 const void* k_pool, sa_dtype dt, float s_att, float* x,
                                 int64_t ldx, void* ws, hipStream_t st, bool rows_fast = false);
hipError_t launch_coverage(const Shape& s, const sa_pages& pg, const float* x, int64_t ldx,
                           const int32_t* idx, const int32_t* count, int32_t cap,
                           const int32_t* ridx, const int32_t* rcount, int32_t rcap, float* mass,
                           int32_t* overlap, hipStream_t st);

size_t prefill_oracle_workspace_bytes(const Shape& s, int32_t n_tokens);
hipError_t launch_prefill_oracle_select(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                        const void* q, const void* k_pool, sa_dtype dt,
                                        float s_att, int32_t b_sel, int32_t k, int32_t* idx,
                                        int32_t* count, int32_t cap, void* ws, hipStream_t st);
size_t pbs_importance_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t n_rows);
size_t pbs_select_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t k_blocks);
hipError_t launch_pbs_importance(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* k_pool, sa_dtype dt, float s_att,
                                 int32_t n_rows, float* imp, void* ws, hipStream_t st);
hipError_t launch_pbs_permutation(const Shape& s, const float* imp, int32_t n_tokens, int32_t seg,
                                  int32_t* perm, hipStream_t st);
hipError_t launch_pbs_select(const Shape& s, const sa_pages& pg, int32_t n_tokens, const void* q,
                             const void* k_pool, sa_dtype dt, const int32_t* perm, int32_t seg,
                             int32_t k_blocks, int32_t* idx, int32_t* count, int32_t cap,
                             void* ws, hipStream_t st);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace sa
