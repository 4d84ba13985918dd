// Indexer kernels: low-rank indexer keys and token scores ("Full Attention
// Strikes Back", method section 2; head-collapsed query, "Oracle-Guided Sparse
// Prefill", section 2.2) and page statistics / Taylor page scores ("SPLA",
// section 2.1, diagonal covariance).
//
// All four are HBM-streaming kernels: each element of the cached rows is read
// once, with consecutive lanes on consecutive rows of a page so every wave
// load covers whole 64-byte segments.
#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------------------
// Indexer keys of appended tokens: kidx[slot] = W_k[g]^T k_pre[t][g].
// 16 lanes per (token, group) pair, one lane per output column.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_index_append(const T* __restrict__ k_pre, const T* __restrict__ w_k,
               const int64_t* __restrict__ slot, int32_t n_tok, int32_t Hkv, int32_t D,
               int64_t n_pool_pages, T* __restrict__ kidx) {
  const int pair = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (pair >= n_tok * Hkv) return;
  const int t = pair / Hkv, g = pair % Hkv;
  const T* kr = k_pre + ((int64_t)t * Hkv + g) * D;
  const T* w = w_k + (int64_t)g * D * kRank + c;
  float acc = 0.f;
  for (int i = 0; i < D; ++i) acc = fmaf(to_f32<T>(kr[i]), to_f32<T>(w[i * kRank]), acc);
  int64_t s = slot[t];
  int64_t page = s / kPage, off = s % kPage;
  if (s < 0 || page >= n_pool_pages) return;  // out-of-pool slot: skipped
  kidx[((page * Hkv + g) * kPage + off) * kRank + c] = from_f32<T>(acc);
}

hipError_t launch_index_append(const Shape& s, const void* k_pre, const void* w_k, sa_dtype dt,
                               const int64_t* slot, int32_t T_, void* kidx_pool,
                               hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  dim3 grid((T_ * s.Hkv + 15) / 16);
  if (dt == SA_BF16)
    k_index_append<bf16_raw><<<grid, 256, 0, st>>>((const bf16_raw*)k_pre, (const bf16_raw*)w_k,
                                                   slot, T_, s.Hkv, s.D, s.n_pool_pages,
                                                   (bf16_raw*)kidx_pool);
  else
    k_index_append<float><<<grid, 256, 0, st>>>((const float*)k_pre, (const float*)w_k, slot, T_,
                                                s.Hkv, s.D, s.n_pool_pages, (float*)kidx_pool);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Head-collapsed indexer query: qc[b][g][c] = s_idx / G * sum_{h in g} sum_i
// W_q[h][i][c] q[b][h][i].  One block per (g, b); thread t takes the (h, i)
// pairs t, t + 256, ... and loads each W row of r = 16 values at once; the 16
// partial sums are reduced across the block in a fixed order.
// ---------------------------------------------------------------------------
// One row of r = 16 values (bf16 or fp32) as floats, with 16-byte loads.
template <typename T>
__device__ __forceinline__ void load_row16(const T* p, float (&w)[kRank]);
template <>
__device__ __forceinline__ void load_row16<bf16_raw>(const bf16_raw* p, float (&w)[kRank]) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  const uint4 a = v[0], b = v[1];
  const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[2 * i] = __uint_as_float(u[i] << 16);
    w[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load_row16<float>(const float* p, float (&w)[kRank]) {
  const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = v[i];
    w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
k_collapse(const T* __restrict__ q, const T* __restrict__ w_q, int32_t Hq, int32_t Hkv,
           int32_t D, float s_idx, float* __restrict__ qc) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) acc[c] = 0.f;
  const int n_pairs = G * D;
  for (int pi = threadIdx.x; pi < n_pairs; pi += 256) {
    const int h = g * G + pi / D, i = pi % D;
    float w[kRank];
    load_row16<T>(w_q + ((int64_t)h * D + i) * kRank, w);
    const float qv = to_f32<T>(q[((int64_t)b * Hq + h) * D + i]);
#pragma unroll
    for (int c = 0; c < kRank; ++c) acc[c] = fmaf(w[c], qv, acc[c]);
  }
  __shared__ float red[4][kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) {
    const float v = wave_sum(acc[c]);
    if (lane == 0) red[wave][c] = v;
  }
  __syncthreads();
  if (threadIdx.x < kRank) {
    const float v = (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
    qc[((int64_t)b * Hkv + g) * kRank + threadIdx.x] = v * (s_idx / (float)G);
  }
}

// ---------------------------------------------------------------------------
// Token scores x[b][g][j] = qc[b][g] . Kidx[b][g][j].  Each block streams
// 1024 tokens of one (b, g): lane -> token, 4 tokens per lane.
// ---------------------------------------------------------------------------
constexpr int kScoreTile = 1024;

template <typename T>
__global__ void __launch_bounds__(256)
k_token_scores(const T* __restrict__ kidx, const int32_t* __restrict__ page_table,
               const int32_t* __restrict__ seq_lens, const float* __restrict__ qc, Shape s,
               float* __restrict__ x, int64_t ldx) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int32_t L = clamp_len(seq_lens[b], s.max_len);
  const int32_t j0 = blockIdx.x * kScoreTile;
  if (j0 >= L) return;
  float qv[kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) qv[c] = qc[((int64_t)b * s.Hkv + g) * kRank + c];
  const int32_t* pt = page_table + (int64_t)b * s.max_pages;
  float* xr = x + ((int64_t)b * s.Hkv + g) * ldx;
#pragma unroll
  for (int u = 0; u < kScoreTile / 256; ++u) {
    const int32_t j = j0 + u * 256 + threadIdx.x;
    if (j < L) {
      const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
      const T* row = kidx + ((page * s.Hkv + g) * kPage + (j & 63)) * kRank;
      float k[kRank];
      load_row16<T>(row, k);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kRank; ++c) acc = fmaf(qv[c], k[c], acc);
      xr[j] = acc;
    }
  }
}

hipError_t launch_index_scores(const Shape& s, const sa_pages& pg, const void* q,
                               const void* w_q, const void* kidx_pool, sa_dtype dt,
                               float s_idx, float* x, int64_t ldx, float* qc_ws,
                               hipStream_t st) {
  if (s.max_len == 0 || s.B == 0) return hipSuccess;
  dim3 g1(s.Hkv, s.B);
  dim3 g2((s.max_len + kScoreTile - 1) / kScoreTile, s.Hkv, s.B);
  if (dt == SA_BF16) {
    k_collapse<bf16_raw><<<g1, 256, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)w_q, s.Hq,
                                             s.Hkv, s.D, s_idx, qc_ws);
    k_token_scores<bf16_raw><<<g2, 256, 0, st>>>((const bf16_raw*)kidx_pool, pg.page_table,
                                                 pg.seq_lens, qc_ws, s, x, ldx);
  } else {
    k_collapse<float><<<g1, 256, 0, st>>>((const float*)q, (const float*)w_q, s.Hq, s.Hkv, s.D,
                                          s_idx, qc_ws);
    k_token_scores<float><<<g2, 256, 0, st>>>((const float*)kidx_pool, pg.page_table,
                                              pg.seq_lens, qc_ws, s, x, ldx);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Page statistics: mean and population variance of the first n_valid tokens
// of a pool page, per group.  One block of D threads per (listed page, g):
// lane i owns dimension i; rows are read twice (mean, then squared
// deviations), both passes from L1/L2 after the first touch.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(128)
k_page_stats(const T* __restrict__ k_pool, const int32_t* __restrict__ pages,
             const int32_t* __restrict__ n_valid, int32_t Hkv, int32_t D, int64_t n_pool_pages,
             T* __restrict__ stats) {
  const int i = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t page = clamp_page(pages[blockIdx.x], n_pool_pages);
  int n = n_valid[blockIdx.x];
  n = n < 1 ? 1 : (n > kPage ? kPage : n);
  if (i >= D) return;
  const T* base = k_pool + (page * Hkv + g) * kPage * (int64_t)D + i;
  float s = 0.f;
  for (int t = 0; t < n; ++t) s += to_f32<T>(base[(int64_t)t * D]);
  const float mean = s / (float)n;
  float ss = 0.f;
  for (int t = 0; t < n; ++t) {
    const float dv = to_f32<T>(base[(int64_t)t * D]) - mean;
    ss = fmaf(dv, dv, ss);
  }
  T* out = stats + (page * Hkv + g) * 2 * (int64_t)D;
  out[i] = from_f32<T>(mean);
  out[D + i] = from_f32<T>(ss / (float)n);
}

hipError_t launch_page_stats(const Shape& s, const void* k_pool, sa_dtype dt,
                             const int32_t* pages, const int32_t* n_valid, int32_t n,
                             void* stats_pool, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dim3 grid(n, s.Hkv);
  if (dt == SA_BF16)
    k_page_stats<bf16_raw><<<grid, 128, 0, st>>>((const bf16_raw*)k_pool, pages, n_valid, s.Hkv,
                                                 s.D, s.n_pool_pages, (bf16_raw*)stats_pool);
  else
    k_page_stats<float><<<grid, 128, 0, st>>>((const float*)k_pool, pages, n_valid, s.Hkv, s.D,
                                              s.n_pool_pages, (float*)stats_pool);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Taylor page scores.  A page's statistics row (mean then variance, 2*D
// values) is spread over D/8 lanes holding 8 dimensions each (16-byte loads
// for bf16), so a wave covers 512/D pages per load instruction.
//   x = mean_h [ q'_h.mean + log1p(0.5 * q'_h^2.var) ] + log(n / page)
// The first term is (sum_h q'_h).mean / G, one dot product per page.  The
// per-head variance sums are reduced over the page's lanes with DPP row
// operations, each lane keeps the heads h = sub (mod lanes per page), takes
// log1p of those, and one more reduction sums them.
// ---------------------------------------------------------------------------
// pages per lane: one (small blocks, many of them, outrun a few large ones:
// the group's scaled query is staged once per block in LDS)
constexpr int kPSRounds = 1;

template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
k_page_scores(const T* __restrict__ q, const T* __restrict__ stats,
              const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
              Shape s, float s_att, float* __restrict__ x, int64_t ldx) {
  constexpr int LPP = D / 8;            // lanes per page
  constexpr int PPW = kWave / LPP;      // pages per wave and round
  constexpr int PPB = 4 * PPW * kPSRounds;
  constexpr int HPL = (G + LPP - 1) / LPP;  // heads kept per lane
  static_assert(LPP == 8 || LPP == 16, "head_dim 64 or 128");
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPP, slot = lane / LPP;
  const int32_t L = clamp_len(seq_lens[b], s.max_len);
  const int32_t n_pages = (L + kPage - 1) / kPage;
  const int32_t p0 = blockIdx.x * PPB;
  if (p0 >= n_pages) return;
  const int32_t* pt = page_table + (int64_t)b * s.max_pages;
  float mu[kPSRounds][8], va[kPSRounds][8];
  int32_t pg[kPSRounds];
#pragma unroll
  for (int r = 0; r < kPSRounds; ++r) {
    pg[r] = p0 + (r * 4 + wave) * PPW + slot;
    if (pg[r] < n_pages) {
      const int64_t page = clamp_page(pt[pg[r]], s.n_pool_pages);
      const T* row = stats + (page * s.Hkv + g) * 2 * (int64_t)D;
      load8<T>(row + sub * 8, mu[r]);
      load8<T>(row + D + sub * 8, va[r]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mu[r][e] = 0.f;
        va[r][e] = 0.f;
      }
    }
  }
  // scaled query of the group's heads, formed once per block in LDS (every
  // page of the block reuses it), then this lane's 8 dimensions in registers
  __shared__ __align__(16) float s_qs[D];
  __shared__ __align__(16) float s_qq[G][D];
  stage_page_query<T, D, G>(q + ((int64_t)b * s.Hq + g * G) * D, s_att, s_qs, s_qq, 256);
  __syncthreads();
  float qs[8], qq[G][8];
  page_query_lane<D, G>(s_qs, s_qq, sub, qs, qq);
#pragma unroll
  for (int r = 0; r < kPSRounds; ++r) {
    const float acc = page_score_sum<LPP, G>(mu[r], va[r], qs, qq, sub);
    if (sub == 0 && pg[r] < n_pages)
      x[((int64_t)b * s.Hkv + g) * ldx + pg[r]] = page_score_final<G>(acc, L, pg[r]);
  }
}

template <typename T, int D>
static void page_scores_g(const Shape& s, const sa_pages& pg, const void* q, const void* st_pool,
                          float s_att, float* x, int64_t ldx, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  constexpr int PPB = 4 * (kWave / (D / 8)) * kPSRounds;
  dim3 grid((s.max_pages + PPB - 1) / PPB, s.Hkv, s.B);
#define SA_PS(GG)                                                                          \
  k_page_scores<T, D, GG><<<grid, 256, 0, st>>>((const T*)q, (const T*)st_pool,           \
                                                pg.page_table, pg.seq_lens, s, s_att, x, ldx)
  switch (G) {
    case 1: SA_PS(1); break;
    case 2: SA_PS(2); break;
    case 4: SA_PS(4); break;
    case 8: SA_PS(8); break;
    default: SA_PS(16); break;
  }
#undef SA_PS
}

hipError_t launch_page_scores(const Shape& s, const sa_pages& pg, const void* q,
                              const void* stats_pool, sa_dtype dt, float s_att, float* x,
                              int64_t ldx, hipStream_t st) {
  if (s.max_len == 0 || s.B == 0) return hipSuccess;
  if (dt == SA_BF16) {
    if (s.D == 128) page_scores_g<bf16_raw, 128>(s, pg, q, stats_pool, s_att, x, ldx, st);
    else page_scores_g<bf16_raw, 64>(s, pg, q, stats_pool, s_att, x, ldx, st);
  } else {
    if (s.D == 128) page_scores_g<float, 128>(s, pg, q, stats_pool, s_att, x, ldx, st);
    else page_scores_g<float, 64>(s, pg, q, stats_pool, s_att, x, ldx, st);
  }
  return hipGetLastError();
}

}  // namespace sa
