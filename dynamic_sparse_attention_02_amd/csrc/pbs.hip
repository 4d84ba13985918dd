// Segment-permuted block selection for causal prefill ("Sparser Block-Sparse
// Attention via Token Permutation", sections 2 to 4): keys are reordered
// inside fixed-size segments so that the keys that draw attention cluster in
// a few blocks, and query blocks then pick whole blocks of the reordered keys.
//
//   importance  mean over the last query block's queries and the group's heads
//               of their causal dense attention distribution (the
//               attention-mass kernels, each query row a sequence of its own
//               causal length on page-table row 0), then a mean over rows;
//   permutation per (segment, group) a bitonic sort in LDS of 64-bit keys
//               (importance descending, position ascending);
//   selection   pooled means: q over a query block's rows and the group's
//               heads, k over each 64-key block of the permuted order (and of
//               the natural order, for the query's own segment); a block's
//               score is their dot product; the row-resident radix select keeps
//               the top k blocks; the selected blocks expand through the
//               permutation into key lists for the block-sparse prefill
//               attention, which gathers listed rows in any order (the
//               permuted attention needs no data movement and, queries keeping
//               their order, no inverse permutation).
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kBlk = 64;          // query and key block (b_sel)
constexpr int kMaxSeg = 4096;     // segment length limit (one LDS sort)

// imp[g][j] = (1 / n_rows) sum_i exp(x[(i, g)][j]) over rows i whose causal
// length first + i + 1 exceeds j.
__global__ void __launch_bounds__(256)
k_pbs_importance(const float* __restrict__ x, int64_t ldx, int32_t n_rows, int32_t first,
                 int32_t Hkv, int32_t N, float* __restrict__ imp) {
  const int g = blockIdx.y;
  const int32_t j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  float acc = 0.f;
  for (int i = 0; i < n_rows; ++i)
    if (j < first + i + 1) acc += expf(x[((int64_t)i * Hkv + g) * ldx + j]);
  imp[(int64_t)g * N + j] = acc / (float)n_rows;
}

__global__ void k_pbs_lens(int32_t* __restrict__ lens, int32_t n, int32_t first) {
  const int32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) lens[i] = first + i + 1;
}

// One workgroup per (segment, group): sort (importance desc, position asc).
// Importance is >= 0, so its bit pattern orders like the value; the key
// (~bits << 32 | position) sorts ascending into the wanted order.  Padding
// past the sequence gets the largest key.
__global__ void __launch_bounds__(1024)
k_pbs_sort(const float* __restrict__ imp, int32_t N, int32_t seg, int32_t* __restrict__ perm) {
  const int s = blockIdx.x, g = blockIdx.y;
  const int32_t s0 = s * seg;
  const int32_t len = min(seg, N - s0);
  int P = 1;
  while (P < seg) P <<= 1;
  __shared__ uint64_t k[kMaxSeg];
  for (int i = threadIdx.x; i < P; i += 1024) {
    uint64_t v = ~0ull;
    if (i < len) {
      const uint32_t bits = __float_as_uint(fmaxf(imp[(int64_t)g * N + s0 + i], 0.f));
      v = ((uint64_t)(~bits) << 32) | (uint32_t)(s0 + i);
    }
    k[i] = v;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += 1024) {
        const int lo = 2 * i - (i & (stride - 1));  // first of the pair
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = k[lo], b = k[hi];
        if ((a > b) == up) {
          k[lo] = b;
          k[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < len; i += 1024)
    perm[(int64_t)g * N + s0 + i] = (int32_t)(uint32_t)k[i];
}

// qbar[blk][g][d] = mean over the block's rows i and the group's heads h of
// q[i][h][d] (fp32).  One workgroup per (block, group): thread t sums 8 dims
// (chunk t % (D / 8)) over the (row, head) pairs t / (D / 8), + 256 / (D / 8),
// ... with 16-byte loads issued together; the shares meet in LDS.
template <typename T>
__global__ void __launch_bounds__(256)
k_pbs_qbar(const T* __restrict__ q, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
           float* __restrict__ qbar) {
  const int blk = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int G = Hq / Hkv;
  const int32_t r0 = blk * kBlk, nr = min(kBlk, N - r0);
  const int nch = D / 8;             // 8-dim chunks: 8 or 16
  const int sh = 256 / nch;          // shares
  const int c = t % nch, share = t / nch;
  const int pairs = nr * G;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int p0 = share; p0 < pairs; p0 += 4 * sh) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u * sh;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
      if (p < pairs) {
        const T* src = q + ((int64_t)(r0 + p / G) * Hq + g * G + p % G) * D + c * 8;
        if constexpr (sizeof(T) == 2) {
          const uint4 w = *reinterpret_cast<const uint4*>(src);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[u][2 * e] = __uint_as_float(ww[e] << 16);
            v[u][2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = src[e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
  }
  __shared__ float part[256][9];
#pragma unroll
  for (int e = 0; e < 8; ++e) part[t][e] = acc[e];
  __syncthreads();
  if (t < D) {
    const int cc = t / 8, e = t % 8;
    float s = 0.f;
    for (int j = 0; j < sh; ++j) s += part[j * nch + cc][e];
    qbar[((int64_t)blk * Hkv + g) * D + t] = s / (float)pairs;
  }
}

// kbar[0][g][c][d]: mean of the keys of natural block c; kbar[1][g][c][d]:
// mean of the keys perm[g][64c .. 64c + 63] (complete blocks only).
template <typename T>
__global__ void __launch_bounds__(128)
k_pbs_kbar(const T* __restrict__ k_pool, const int32_t* __restrict__ pt, Shape s, int32_t N,
           const int32_t* __restrict__ perm, float* __restrict__ kbar) {
  const int c = blockIdx.x, g = blockIdx.y, which = blockIdx.z, d = threadIdx.x;
  const int D = s.D;
  if (d >= D) return;
  const int nkb = N / kBlk;
  float acc = 0.f;
  for (int t = 0; t < kBlk; ++t) {
    int32_t j = c * kBlk + t;
    if (which) j = perm[(int64_t)g * N + j];
    j = j < 0 ? 0 : (j >= N ? N - 1 : j);
    const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
    acc += to_f32<T>(k_pool[((page * s.Hkv + g) * kPage + (j & 63)) * D + d]);
  }
  kbar[(((int64_t)which * s.Hkv + g) * nkb + c) * D + d] = acc / (float)kBlk;
}

// x[(blk, g)][c] = qbar[blk][g] . kbar[c < own segment's first block ? 1 : 0][g][c]
// for c < blk: a 64 x 64 tile of (query block, candidate block) per
// workgroup, both key variants accumulated side by side (fp32, dims in
// order), 4 x 4 outputs per thread, 16-dim steps staged in LDS.
__global__ void __launch_bounds__(256)
k_pbs_scores(const float* __restrict__ qbar, const float* __restrict__ kbar, int32_t nblk,
             int32_t nkb, int32_t Hkv, int32_t D, int32_t seg_blocks, float* __restrict__ x,
             int64_t ldx) {
  const int g = blockIdx.z;
  const int b0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (c0 >= min(nblk, b0 + 64) - 1 || c0 >= nkb) return;  // no candidate of any row in the tile
  const int t = threadIdx.x, tr = t / 16, tc = t % 16;
  __shared__ float qs[16][65];
  __shared__ float kp[16][65];
  __shared__ float kn[16][65];
  float ap[4][4], an[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) ap[i][j] = an[i][j] = 0.f;
  const float* kb_nat = kbar + (int64_t)g * nkb * D;
  const float* kb_perm = kbar + ((int64_t)Hkv + g) * nkb * D;
  for (int d0 = 0; d0 < D; d0 += 16) {
    __syncthreads();
    for (int e = t; e < 64 * 16; e += 256) {
      const int r = e / 16, dd = e % 16;
      const int blk = b0 + r, c = c0 + r;
      qs[dd][r] = blk < nblk ? qbar[((int64_t)blk * Hkv + g) * D + d0 + dd] : 0.f;
      kn[dd][r] = c < nkb ? kb_nat[(int64_t)c * D + d0 + dd] : 0.f;
      kp[dd][r] = c < nkb ? kb_perm[(int64_t)c * D + d0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int dd = 0; dd < 16; ++dd) {
      float a[4], bp[4], bn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = qs[dd][tr * 4 + i];
        bp[i] = kp[dd][tc * 4 + i];
        bn[i] = kn[dd][tc * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ap[i][j] = fmaf(a[i], bp[j], ap[i][j]);
          an[i][j] = fmaf(a[i], bn[j], an[i][j]);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = b0 + tr * 4 + i;
    if (blk >= nblk) continue;
    const int own_first = (blk / seg_blocks) * seg_blocks;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tc * 4 + j;
      if (c < blk && c < nkb) x[((int64_t)blk * Hkv + g) * ldx + c] = c < own_first ? ap[i][j] : an[i][j];
    }
  }
}

// Key lists: selected block c (ascending block order) contributes
// perm[g][64c ..] (earlier segment) or 64c .. (own segment).  One workgroup
// per (block, group) row.
__global__ void __launch_bounds__(256)
k_pbs_expand(const int32_t* __restrict__ bsel_idx, const int32_t* __restrict__ bsel_cnt,
             int32_t kb_cap, const int32_t* __restrict__ perm, int32_t N, int32_t Hkv,
             int32_t seg_blocks, int32_t* __restrict__ idx, int32_t* __restrict__ count,
             int32_t cap) {
  const int row = blockIdx.x;
  const int blk = row / Hkv, g = row % Hkv;
  int32_t nb = bsel_cnt[row];
  nb = nb < 0 ? 0 : (nb > kb_cap ? kb_cap : nb);
  const int64_t nk = (int64_t)nb * kBlk < cap ? (int64_t)nb * kBlk : cap;
  const int own_first = (blk / seg_blocks) * seg_blocks;
  int32_t* out = idx + (int64_t)row * cap;
  for (int64_t o = threadIdx.x; o < cap; o += 256) {
    int32_t v = -1;
    if (o < nk) {
      const int32_t c = bsel_idx[(int64_t)row * kb_cap + o / kBlk];
      const int32_t j = c * kBlk + (int32_t)(o % kBlk);
      v = c < own_first ? perm[(int64_t)g * N + j] : j;
    }
    out[o] = v;
  }
  if (threadIdx.x == 0) count[row] = (int32_t)nk;
}

struct PbsImpLayout {
  size_t off_lens, off_x, off_mass, total;
  int64_t ldx;
};

PbsImpLayout pbs_imp_layout(const Shape& s, int32_t n_tokens, int32_t n_rows) {
  PbsImpLayout L;
  L.ldx = n_tokens;
  Shape s2 = s;
  s2.B = n_rows;
  s2.max_len = n_tokens;
  size_t off = 0;
  L.off_lens = off;
  off += align_up((size_t)n_rows * sizeof(int32_t), 256);
  L.off_x = off;
  off += align_up((size_t)n_rows * s.Hkv * (size_t)n_tokens * sizeof(float), 256);
  L.off_mass = off;
  off += align_up(mass_workspace_bytes(s2), 256);
  L.total = off;
  return L;
}

struct PbsSelLayout {
  size_t off_qbar, off_kbar, off_x, off_bidx, off_bcnt, off_sel, total;
  int32_t nblk, nkb;
};

PbsSelLayout pbs_sel_layout(const Shape& s, int32_t n_tokens, int32_t k_blocks) {
  PbsSelLayout L;
  L.nblk = (n_tokens + kBlk - 1) / kBlk;
  L.nkb = n_tokens / kBlk;
  const int64_t rows = (int64_t)L.nblk * s.Hkv;
  const int64_t ldx = L.nblk > 1 ? L.nblk : 1;
  size_t off = 0;
  L.off_qbar = off;
  off += align_up((size_t)rows * s.D * sizeof(float), 256);
  L.off_kbar = off;
  off += align_up((size_t)2 * s.Hkv * (L.nkb > 0 ? L.nkb : 1) * s.D * sizeof(float), 256);
  L.off_x = off;
  off += align_up((size_t)rows * ldx * sizeof(float), 256);
  L.off_bidx = off;
  off += align_up((size_t)rows * (k_blocks > 0 ? k_blocks : 1) * sizeof(int32_t), 256);
  L.off_bcnt = off;
  off += align_up((size_t)rows * sizeof(int32_t), 256);
  L.off_sel = off;
  off += align_up(select_workspace_bytes((int32_t)rows, (int32_t)ldx), 256);
  L.total = off;
  return L;
}

}  // namespace

size_t pbs_importance_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t n_rows) {
  return pbs_imp_layout(s, n_tokens, n_rows).total;
}

size_t pbs_select_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t k_blocks) {
  return pbs_sel_layout(s, n_tokens, k_blocks).total;
}

hipError_t launch_pbs_importance(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* k_pool, sa_dtype dt, float s_att,
                                 int32_t n_rows, float* imp, void* ws, hipStream_t st) {
  const PbsImpLayout L = pbs_imp_layout(s, n_tokens, n_rows);
  char* base = (char*)ws;
  int32_t* lens = (int32_t*)(base + L.off_lens);
  float* x = (float*)(base + L.off_x);
  const int32_t first = n_tokens - n_rows;
  k_pbs_lens<<<(n_rows + 255) / 256, 256, 0, st>>>(lens, n_rows, first);
  Shape s2 = s;
  s2.B = n_rows;
  s2.max_len = n_tokens;
  s2.max_pages = 0;  // every query row reads page-table row 0
  sa_pages p2;
  p2.page_table = pg.page_table;
  p2.seq_lens = lens;
  const size_t qe = dt == SA_BF16 ? 2 : 4;
  hipError_t e = launch_attention_mass(s2, p2, (const char*)q + (size_t)first * s.Hq * s.D * qe,
                                       k_pool, dt, s_att, x, L.ldx, base + L.off_mass, st,
                                       /*rows_fast=*/true);
  if (e != hipSuccess) return e;
  dim3 grid((n_tokens + 255) / 256, s.Hkv);
  k_pbs_importance<<<grid, 256, 0, st>>>(x, L.ldx, n_rows, first, s.Hkv, n_tokens, imp);
  return hipGetLastError();
}

hipError_t launch_pbs_permutation(const Shape& s, const float* imp, int32_t n_tokens, int32_t seg,
                                  int32_t* perm, hipStream_t st) {
  dim3 grid((n_tokens + seg - 1) / seg, s.Hkv);
  k_pbs_sort<<<grid, 1024, 0, st>>>(imp, n_tokens, seg, perm);
  return hipGetLastError();
}

hipError_t launch_pbs_select(const Shape& s, const sa_pages& pg, int32_t n_tokens, const void* q,
                             const void* k_pool, sa_dtype dt, const int32_t* perm, int32_t seg,
                             int32_t k_blocks, int32_t* idx, int32_t* count, int32_t cap,
                             void* ws, hipStream_t st) {
  const PbsSelLayout L = pbs_sel_layout(s, n_tokens, k_blocks);
  char* base = (char*)ws;
  float* qbar = (float*)(base + L.off_qbar);
  float* kbar = (float*)(base + L.off_kbar);
  float* x = (float*)(base + L.off_x);
  int32_t* bidx = (int32_t*)(base + L.off_bidx);
  int32_t* bcnt = (int32_t*)(base + L.off_bcnt);
  const int64_t ldx = L.nblk > 1 ? L.nblk : 1;
  const int seg_blocks = seg / kBlk;
  dim3 gq(L.nblk, s.Hkv);
  if (dt == SA_BF16) k_pbs_qbar<bf16_raw><<<gq, 256, 0, st>>>((const bf16_raw*)q, n_tokens, s.Hq, s.Hkv, s.D, qbar);
  else k_pbs_qbar<float><<<gq, 256, 0, st>>>((const float*)q, n_tokens, s.Hq, s.Hkv, s.D, qbar);
  if (L.nkb > 0) {
    dim3 gk(L.nkb, s.Hkv, 2);
    if (dt == SA_BF16)
      k_pbs_kbar<bf16_raw><<<gk, 128, 0, st>>>((const bf16_raw*)k_pool, pg.page_table, s, n_tokens, perm, kbar);
    else
      k_pbs_kbar<float><<<gk, 128, 0, st>>>((const float*)k_pool, pg.page_table, s, n_tokens, perm, kbar);
    dim3 gs((unsigned)((L.nkb + 63) / 64), (L.nblk + 63) / 64, s.Hkv);
    k_pbs_scores<<<gs, 256, 0, st>>>(qbar, kbar, L.nblk, L.nkb, s.Hkv, s.D, seg_blocks, x, ldx);
  }
  SelectArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.seq_lens = nullptr;
  a.rows = L.nblk * s.Hkv;
  a.Hkv = s.Hkv;
  a.max_len = n_tokens;
  a.unit = 1;
  a.max_cand = (int32_t)ldx;
  a.is_topk = 1;
  a.p = 0.f;
  a.k = k_blocks;
  a.n_sink = 0;
  a.n_window = 0;
  a.idx = bidx;
  a.count = bcnt;
  a.cap = k_blocks;
  a.prefill_bsel = 1;  // query block blk has blk candidate blocks
  a.prefill_blk0 = 0;
  a.prefill_self = 0;
  hipError_t e = launch_select(a, base + L.off_sel, st);
  if (e != hipSuccess) return e;
  k_pbs_expand<<<L.nblk * s.Hkv, 256, 0, st>>>(bidx, bcnt, k_blocks, perm, n_tokens, s.Hkv,
                                               seg_blocks, idx, count, cap);
  return hipGetLastError();
}

}  // namespace sa
