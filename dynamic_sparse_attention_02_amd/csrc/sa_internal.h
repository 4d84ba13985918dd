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
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum across the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t w = __shfl_up(v, o, kWave);
    if (lane >= o) v += w;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v) {
  return wave_incl_scan(v) - v;
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
};
size_t select_workspace_bytes(int32_t rows, int32_t max_cand);
hipError_t launch_select(const SelectArgs& a, void* ws, hipStream_t st);

size_t decode_workspace_bytes(const Shape& s, int32_t cap);
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
                                 hipStream_t st);
hipError_t launch_sparse_prefill(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* idx, const int32_t* count, int32_t cap,
                                 int32_t b_sel, float s_att, void* out, sa_dtype out_dt,
                                 float* lse, hipStream_t st);

size_t fused_workspace_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D);
bool fused_plan(const Shape& s, int32_t n_sink, int32_t n_window, int32_t* nb, int32_t* tpb);
hipError_t launch_decode_fused(const Shape& s, const sa_pages& pg, const void* q, const void* w_q,
                               const void* kidx_pool, const void* k_pool, const void* v_pool,
                               sa_dtype dt, float s_idx, float s_att, float p, int32_t top_k,
                               int32_t n_sink, int32_t n_window, float* x, int64_t ldx,
                               int32_t* idx, int32_t* count, int32_t cap, void* out,
                               sa_dtype out_dt, float* lse, void* ws, int32_t nb, int32_t tpb,
                               hipStream_t st);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace sa
