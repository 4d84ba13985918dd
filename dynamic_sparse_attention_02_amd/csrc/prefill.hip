// Causal prefill with supports shared by blocks of b_sel = 64 queries
// ("Oracle-Guided Sparse Prefill", section 2.1: top-k support per selection
// block, attention recomputed with the original q, k, v over the support;
// section 2.2: one head-collapsed indexer channel).
//
// Selection: per (query block, group) the block-collapsed indexer query is
// formed (sum of the block's queries per head, then projected), scores over
// the keys of all earlier blocks are written for a slab of query blocks, and
// the row-resident radix select keeps the top k of each row.
//
// Attention: one workgroup per (query block, group); each wave owns one query
// head and 32 of the block's 64 queries (two waves per head, so a wave needs
// few enough registers for two waves to share each SIMD and overlap one's
// matrix-core products with the other's softmax); the heads of a group share
// every gathered K/V tile.  Per 64-key tile the wave computes S^T = K Q^T and
// O^T += V^T P^T on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulate).  In this transposed form a lane holds one query's scores, so
// the online softmax needs one cross-lane exchange per row, and the fp32 S^T
// accumulator already has the lane layout of the P^T operand once the keys of
// each 16-key step are taken in the order the accumulator holds them; V is
// written to LDS transposed so V^T operands are two 8-byte reads.  K/V tiles
// are double-buffered in LDS with the next tile's rows in flight during the
// current tile's products.
#include "sa_internal.h"

namespace sa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kQB = 64;     // queries per selection block
constexpr int kSlab = 256;  // query blocks per score slab

__global__ void k_iota1(int32_t* __restrict__ v, int32_t n) {
  const int32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) v[i] = i + 1;
}

// ---------------------------------------------------------------------------
// Block-collapsed indexer query: qcb[blk][g][c] = s_idx / (rows * G) *
// sum_{h in g} sum_d W_q[h][d][c] * (sum_{i in blk} q[i][h][d]).
// Thread t sums 8 consecutive dims (one 16-byte load for bf16) of one head
// over a share of the block's rows; the shares are added in LDS, then each
// thread projects its (head, dims) chunk and the block reduces the rank-16
// result.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
k_prefill_qc(const T* __restrict__ q, const T* __restrict__ w_q, int32_t N, int32_t Hq,
             int32_t Hkv, int32_t D, int32_t bsel, float s_idx, float* __restrict__ qcb) {
  const int blk = blockIdx.x, g = blockIdx.y;
  const int G = Hq / Hkv;
  const int r0 = blk * bsel;
  const int nr = min(bsel, N - r0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = G * D / 8;              // (head, 8 dims) chunks: <= 256
  const int parts = 256 / chunks;            // row shares per chunk
  const int ch = threadIdx.x % chunks, part = threadIdx.x / chunks;
  const int h = g * G + (ch * 8) / D, d0 = (ch * 8) % D;
  __shared__ float qs[256][8];               // each thread's partial sums
  float acc8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  if (part < parts) {
    for (int i = part; i < nr; i += parts) {
      const T* src = q + ((int64_t)(r0 + i) * Hq + h) * D + d0;
      if constexpr (sizeof(T) == 2) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc8[2 * e] += __uint_as_float(w[e] << 16);
          acc8[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] += to_f32<T>(src[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) qs[threadIdx.x][e] = acc8[e];
  __syncthreads();
  // projection of this thread's chunk (first `chunks` threads)
  float acc[kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) acc[c] = 0.f;
  if (threadIdx.x < chunks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.f;
      for (int pp = 0; pp < parts; ++pp) v += qs[pp * chunks + ch][e];
      const T* wr = w_q + ((int64_t)h * D + d0 + e) * kRank;
#pragma unroll
      for (int c = 0; c < kRank; ++c) acc[c] = fmaf(to_f32<T>(wr[c]), v, acc[c]);
    }
  }
  __shared__ float red[4][kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) {
    const float v = wave_sum(acc[c]);
    if (lane == 0) red[wave][c] = v;
  }
  __syncthreads();
  if (threadIdx.x < kRank) {
    const int c = threadIdx.x;
    const float v = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    qcb[((int64_t)blk * Hkv + g) * kRank + c] = v * (s_idx / (float)(nr * G));
  }
}

// ---------------------------------------------------------------------------
// Scores of a slab of query blocks: x[(blk - blk0) * Hkv + g][j] =
// qcb[blk][g] . Kidx[g][j] for j < bsel * blk + self (the keys of earlier
// blocks; per query, bsel = 1 and self = 1: the keys up to and including the
// query's own).  A workgroup covers 256 candidates and kRowsT query blocks of
// one group: each key row is loaded once and scored against every block's
// query.
// ---------------------------------------------------------------------------
constexpr int kRowsT = 32;

// K16: instead of the fp32 score, the top 16 bits of its order-preserving key,
// two candidates per 32-bit word (ldx then counts words): candidate j in
// word (j / 128) * 64 + j % 64, low half for j % 128 < 64, else high.
template <typename T, bool K16>
__global__ void __launch_bounds__(256)
k_prefill_scores(const T* __restrict__ kidx, const int32_t* __restrict__ pt,
                 const float* __restrict__ qcb, int32_t blk0, int32_t blk1, int32_t bsel,
                 int32_t self, Shape s, float* __restrict__ x, int64_t ldx) {
  const int g = blockIdx.z;
  const int b_lo = blk0 + blockIdx.y * kRowsT;
  const int b_hi = min(blk1, b_lo + kRowsT);
  const int32_t j = blockIdx.x * 256 + threadIdx.x;
  const int32_t lim_hi = bsel * (b_hi - 1) + self;  // candidates of the slab's last row
  if ((int64_t)blockIdx.x * 256 >= (int64_t)lim_hi) return;  // above every row
  __shared__ float qs[kRowsT][kRank];
  for (int i = threadIdx.x; i < kRowsT * kRank; i += 256) {
    const int bb = b_lo + i / kRank;
    qs[i / kRank][i % kRank] = bb < b_hi ? qcb[((int64_t)bb * s.Hkv + g) * kRank + i % kRank] : 0.f;
  }
  __syncthreads();
  if (j >= lim_hi) return;
  const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
  const T* row = kidx + ((page * s.Hkv + g) * kPage + (j & 63)) * kRank;
  float k[kRank];
  if constexpr (sizeof(T) == 2) {
    const uint4* v = reinterpret_cast<const uint4*>(row);
    const uint4 a = v[0], b = v[1];
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k[2 * i] = __uint_as_float(u[i] << 16);
      k[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRank; ++i) k[i] = to_f32<T>(row[i]);
  }
  for (int bb = b_lo; bb < b_hi; ++bb) {
    if (j >= bsel * bb + self) continue;
    const float* qv = qs[bb - b_lo];
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < kRank; ++c) a = fmaf(qv[c], k[c], a);
    const int64_t r = (int64_t)(bb - blk0) * s.Hkv + g;
    if (K16)
      reinterpret_cast<uint16_t*>(x)[r * 2 * ldx + 2 * ((j >> 7) * 64 + (j & 63)) + ((j >> 6) & 1)] =
          (uint16_t)(score_key(a) >> 16);
    else
      x[r * ldx + j] = a;
  }
}

// ---------------------------------------------------------------------------
// Per-query selection by the mean of the heads' probabilities (the
// aggregation the attention-mass oracle uses, applied to the low-rank
// channels): each head keeps its own projected query, its logits over the
// candidates j <= i become a softmax, and the score of j is the log of the
// mean over the group's heads of those probabilities.
// ---------------------------------------------------------------------------

// qh[i][h][c] = s_idx * sum_d W_q[h][d][c] q[i][h][d].  One workgroup per
// (query, group); thread = (head, D/16 dims), so a head's 16 threads are one
// DPP row.
template <typename T>
__global__ void __launch_bounds__(256)
k_prefill_qh(const T* __restrict__ q, const T* __restrict__ w_q, int32_t Hq, int32_t Hkv,
             int32_t D, float s_idx, float* __restrict__ qh) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int G = Hq / Hkv;
  const int t = threadIdx.x;
  if (t >= G * 16) return;  // whole 16-lane rows leave together
  const int h = g * G + (t >> 4), part = t & 15;
  const int dpt = D / 16;
  float acc[kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) acc[c] = 0.f;
  for (int e = 0; e < dpt; ++e) {
    const int d = part * dpt + e;
    const float v = to_f32<T>(q[((int64_t)i * Hq + h) * D + d]);
    const T* wr = w_q + ((int64_t)h * D + d) * kRank;
#pragma unroll
    for (int c = 0; c < kRank; ++c) acc[c] = fmaf(to_f32<T>(wr[c]), v, acc[c]);
  }
#pragma unroll
  for (int c = 0; c < kRank; ++c) {
    const float v = row16_sum(acc[c]);
    if (part == 0) qh[((int64_t)i * Hq + h) * kRank + c] = v * s_idx;
  }
}

constexpr int kRowsQ = 8;     // query rows per workgroup in the per-head passes
constexpr float kLog2eP = 1.4426950408889634f;

// MODE 0: per (256-candidate tile, query, head) and wave, the max and the sum
// of 2^(x - max) of the head's base-2 logits over the wave's candidates
// j <= i.  MODE 1: the scores x[row][j] = ln((1/G) sum_h 2^(x_h - lse2_h)).
template <typename T, int G, int MODE>
__global__ void __launch_bounds__(256)
k_prefill_hprob(const T* __restrict__ kidx, const int32_t* __restrict__ pt,
                const float* __restrict__ qh, const float* __restrict__ lse2, int32_t q0,
                int32_t q1, Shape s, float2* __restrict__ part, int32_t nparts,
                float* __restrict__ x, int64_t ldx) {
  const int g = blockIdx.z;
  const int b_lo = q0 + blockIdx.y * kRowsQ;
  const int b_hi = min(q1, b_lo + kRowsQ);
  const int tile = blockIdx.x;
  const int32_t j = tile * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int64_t)tile * 256 >= (int64_t)b_hi) return;  // past the last row's candidates (j <= b_hi - 1)
  __shared__ float qs[kRowsQ][G][kRank];
  for (int e = threadIdx.x; e < kRowsQ * G * kRank; e += 256) {
    const int r = e / (G * kRank), hc = e % (G * kRank);
    const int bb = b_lo + r;
    qs[r][hc / kRank][hc % kRank] =
        bb < b_hi ? qh[((int64_t)bb * s.Hq + g * G) * kRank + hc] * kLog2eP : 0.f;
  }
  __syncthreads();
  float k[kRank];
  if (j < b_hi) {
    const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
    const T* row = kidx + ((page * s.Hkv + g) * kPage + (j & 63)) * kRank;
#pragma unroll
    for (int c = 0; c < kRank; ++c) k[c] = to_f32<T>(row[c]);
  } else {
#pragma unroll
    for (int c = 0; c < kRank; ++c) k[c] = 0.f;
  }
  for (int bb = b_lo; bb < b_hi; ++bb) {
    if ((int64_t)tile * 256 > bb) continue;  // whole tile past row bb (uniform)
    const bool ok = j <= bb;
    const int64_t r = (int64_t)(bb - q0) * s.Hkv + g;
    if (MODE == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < kRank; ++c) a = fmaf(qs[bb - b_lo][h][c], k[c], a);
        const float m = wave_max(ok ? a : -INFINITY);
        const float l = wave_sum(ok ? exp2f(a - m) : 0.f);
        if (lane == 0) part[(r * nparts + tile * 4 + wave) * G + h] = make_float2(m, l);
      }
    } else {
      if (!ok) continue;
      float u[G];
      float M = -INFINITY;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < kRank; ++c) a = fmaf(qs[bb - b_lo][h][c], k[c], a);
        u[h] = a - lse2[((int64_t)bb * s.Hq + g * G) + h];
        M = fmaxf(M, u[h]);
      }
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) sum += exp2f(u[h] - M);
      x[r * ldx + j] = 0.6931471805599453f * (M + log2f(sum)) - logf((float)G);
    }
  }
}

// lse2[i][h] = log2 sum_{j <= i} 2^(x_h): the wave partials of query i merged
// in order; one wave per head.
template <int G>
__global__ void __launch_bounds__(256)
k_prefill_hnorm(const float2* __restrict__ part, int32_t nparts, int32_t q0, int32_t Hq,
                int32_t Hkv, float* __restrict__ lse2) {
  const int r = blockIdx.x;  // (query - q0) * Hkv + g
  const int i = q0 + r / Hkv, g = r % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int np = min(nparts, ((i + 1) + 63) / 64);  // waves that saw candidates of row i
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY, l = 0.f;
    for (int c = lane; c < np; c += 64) {
      const float2 v = part[((int64_t)r * nparts + c) * G + h];
      const float mn = fmaxf(m, v.x);
      l = (mn == -INFINITY) ? 0.f : l * exp2f(m - mn) + v.y * exp2f(v.x - mn);
      m = mn;
    }
    const float M = wave_max(m);
    const float Ls = wave_sum(m == -INFINITY ? 0.f : l * exp2f(m - M));
    if (lane == 0) lse2[(int64_t)i * Hq + g * G + h] = M + log2f(Ls);
  }
}

// ---------------------------------------------------------------------------
// Block-sparse causal attention.
// ---------------------------------------------------------------------------
constexpr int kKT = 64;                 // keys per tile
constexpr int kKPitch = 128 * 2 + 16;   // K tile row pitch in bytes (d = 128 bf16)
constexpr int kVPitch = kKT * 2 + 8;    // V^T row pitch in bytes (64 keys bf16; 34 dwords)
constexpr int kMaxListed = 2048;        // listed keys per block the attention kernel takes
constexpr float kLazy = 8.f;            // log2 headroom of the lazily raised softmax maximum

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// HB query heads of one group per workgroup (two waves each, 32 queries per
// wave); a group of G > HB heads takes G / HB workgroups.
template <int HB>
__global__ void __launch_bounds__(HB * 2 * 64)
k_prefill_attn(const bf16_raw* __restrict__ q, const bf16_raw* __restrict__ k_pool,
               const bf16_raw* __restrict__ v_pool, const int32_t* __restrict__ pt,
               const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int32_t cap,
               int32_t N, Shape s, float s_att, void* __restrict__ out, int32_t out_bf16,
               float* __restrict__ lse) {
  constexpr int D = 128;
  constexpr int NBQ = 1;        // 32-query blocks per wave
  constexpr int WPH = 2 / NBQ;  // waves per head
  constexpr int NT = HB * WPH * 64;
  constexpr int PIECES = kKT * (D * 2 / 16);  // 16-byte pieces per tile per tensor
  constexpr int LPT = (PIECES + NT - 1) / NT;
  const int nblk = (N + kQB - 1) / kQB;
  const int G = s.Hq / s.Hkv, n_sub = G / HB;
  // heaviest items (late blocks, full supports) first; workgroups of one
  // block and group run side by side
  const int item = blockIdx.x / n_sub, sub = blockIdx.x % n_sub;
  const int blk = nblk - 1 - item / s.Hkv;
  const int g = item % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = g * G + sub * HB + wave / WPH;
  const int qpart = wave % WPH;
  const int half = lane >> 5, l32 = lane & 31;
  const int row = blk * s.Hkv + g;
  int32_t nl = count[row];
  nl = nl < 0 ? 0 : (nl > cap ? cap : nl);
  const int32_t q0 = blk * kQB;
  const int32_t nq = min(kQB, N - q0);
  const int n_list_tiles = (nl + kKT - 1) / kKT;
  const int n_tiles = n_list_tiles + 1;  // + the diagonal tile
  const int32_t* list = idx + (int64_t)row * cap;

  __shared__ __align__(16) char Ks[2][kKT * kKPitch];
  __shared__ __align__(16) char Vt[2][D * kVPitch];
  // pool row (page * Hkv + g) * 64 + slot of every key the item visits, in
  // tile order (listed keys, then the diagonal block); -1 marks padding
  __shared__ int32_t rows_lds[kMaxListed + kKT];

  // Q as the B operand of S^T = K Q^T: Qb[nb][ks] holds query nb*32 + l32,
  // dims ks*16 + 8*half .. +7
  bf16x8_t Qb[NBQ][8];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    const int32_t qi = q0 + (qpart * NBQ + nb) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qi < N)
        v = *reinterpret_cast<const uint4*>(q + ((int64_t)qi * s.Hq + h) * D + ks * 16 + 8 * half);
      Qb[nb][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // resolve every key's pool row once (list entry -> page table -> row)
  const int n_rows_total = n_list_tiles * kKT + kKT;
  for (int t = tid; t < n_rows_total; t += NT) {
    int32_t j = -1;
    if (t < n_list_tiles * kKT) {
      if (t < nl) j = list[t];
    } else if (t - n_list_tiles * kKT < nq) {
      j = q0 + (t - n_list_tiles * kKT);
    }
    int32_t rw = -1;
    if (j >= 0) {
      j = j >= N ? N - 1 : j;
      const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
      rw = (int32_t)((page * s.Hkv + g) * kPage + (j & 63));
    }
    rows_lds[t] = rw;
  }
  __syncthreads();
  // Gather: piece pc moves 16 bytes (8 head dims, chunk col = pc / 64) of
  // key row r = pc % 64, so the 64 lanes of a wave hold one chunk of all 64
  // keys: the transposed V^T stores of a wave then fill one LDS row.
  uint4 kr[LPT], vr[LPT];
  auto gather = [&](int tile) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int pc = i * NT + tid;
      const int r = pc & 63, col = pc >> 6;
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (pc < PIECES) {
        const int32_t rw = rows_lds[tile * kKT + r];
        if (rw >= 0) {
          const int64_t off = (int64_t)rw * D + col * 8;
          kr[i] = *reinterpret_cast<const uint4*>(k_pool + off);
          vr[i] = *reinterpret_cast<const uint4*>(v_pool + off);
        }
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int pc = i * NT + tid;
      if (pc < PIECES) {
        const int r = pc & 63, col = pc >> 6;
        *reinterpret_cast<uint4*>(Ks[buf] + r * kKPitch + col * 16) = kr[i];
        const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint16_t*>(Vt[buf] + (col * 8 + 2 * e) * kVPitch + r * 2) = (uint16_t)(w[e] & 0xffffu);
          *reinterpret_cast<uint16_t*>(Vt[buf] + (col * 8 + 2 * e + 1) * kVPitch + r * 2) = (uint16_t)(w[e] >> 16);
        }
      }
    }
  };

  f32x16_t acc[4][NBQ];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
  float m_run[NBQ], l_run[NBQ];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }
  const float sl2 = s_att * 1.4426950408889634f;  // scores in log2 units

  gather(0);
  stage(0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) gather(tile + 1);
    const bool diag = tile == n_list_tiles;
    const int nt = diag ? nq : min(kKT, nl - tile * kKT);

    // S^T[key][query] for the 64 keys x 64 queries of this wave's head
    f32x16_t S[2][NBQ];
#pragma unroll
    for (int mk = 0; mk < 2; ++mk)
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) S[mk][nb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
        const uint4 a = *reinterpret_cast<const uint4*>(Ks[buf] + (mk * 32 + l32) * kKPitch + ks * 32 + half * 16);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
          S[mk][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, Qb[nb][ks], S[mk][nb], 0, 0, 0);
      }
    }
    // online softmax per query (lane's query nb*32 + l32; keys spread over
    // this lane's 32 accumulator values and the partner lane's), in log2
    // units.  The running maximum is raised only when a tile's maximum
    // exceeds it by more than kLazy (so P stays below 2^kLazy): the output
    // accumulator is rescaled on those tiles only.
    const bool masked = diag || nt < kKT;
    float mt[NBQ];
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      const int qloc = (qpart * NBQ + nb) * 32 + l32;
      if (masked) {
#pragma unroll
        for (int mk = 0; mk < 2; ++mk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kloc = mk * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (!(kloc < nt && (!diag || kloc <= qloc))) S[mk][nb][v] = -INFINITY;
          }
      }
      float m = -INFINITY;
#pragma unroll
      for (int mk = 0; mk < 2; ++mk)
#pragma unroll
        for (int v = 0; v < 16; ++v) m = fmaxf(m, S[mk][nb][v]);
      mt[nb] = fmaxf(m, __shfl_xor(m, 32, 64)) * sl2;
    }
    bool raise[NBQ], any_raise = false;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      raise[nb] = mt[nb] > m_run[nb] + kLazy;
      any_raise = any_raise || raise[nb];
    }
    if (__ballot(any_raise)) {
      float alpha[NBQ];
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        const bool r = raise[nb];
        const float m_new = r ? mt[nb] : m_run[nb];
        alpha[nb] = r ? __builtin_amdgcn_exp2f(m_run[nb] - m_new) : 1.f;  // 0 on the first raise
        l_run[nb] *= alpha[nb];
        m_run[nb] = m_new;
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mb][nb][v] *= alpha[nb];
    }
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      const float m_use = m_run[nb] == -INFINITY ? 0.f : m_run[nb];
      float lt = 0.f;
#pragma unroll
      for (int mk = 0; mk < 2; ++mk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[mk][nb][v], sl2, -m_use));
          S[mk][nb][v] = p;
          lt += p;
        }
      l_run[nb] += lt + __shfl_xor(lt, 32, 64);
    }
    // O^T[d][query] += V^T[d][key] P^T[key][query], 16 keys per step in the
    // accumulator's key order
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int mk = st >> 1, hv = (st & 1) * 8;
      bf16x8_t Pb[NBQ];
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        uint4 pw;
        pw.x = pack_bf16x2(S[mk][nb][hv + 0], S[mk][nb][hv + 1]);
        pw.y = pack_bf16x2(S[mk][nb][hv + 2], S[mk][nb][hv + 3]);
        pw.z = pack_bf16x2(S[mk][nb][hv + 4], S[mk][nb][hv + 5]);
        pw.w = pack_bf16x2(S[mk][nb][hv + 6], S[mk][nb][hv + 7]);
        Pb[nb] = __builtin_bit_cast(bf16x8_t, pw);
      }
      const int kbase = mk * 32 + (st & 1) * 16 + 4 * half;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const char* vrow = Vt[buf] + (mb * 32 + l32) * kVPitch;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kbase * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (kbase + 8) * 2);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, Pb[nb], acc[mb][nb], 0, 0, 0);
      }
    }
    // the other buffer was released by the barrier that ended the previous tile
    if (tile + 1 < n_tiles) stage(buf ^ 1);
    __syncthreads();
  }
  // normalise and store: lane holds d = mb*32 + 8*(v/4) + 4*half + v%4 of
  // query nb*32 + l32
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    const int32_t qi = q0 + (qpart * NBQ + nb) * 32 + l32;
    if (qi >= N) continue;
    const float inv = l_run[nb] > 0.f ? 1.f / l_run[nb] : 0.f;
    const int64_t obase = ((int64_t)qi * s.Hq + h) * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = mb * 32 + 8 * grp + 4 * half;
        const float o0 = acc[mb][nb][grp * 4 + 0] * inv, o1 = acc[mb][nb][grp * 4 + 1] * inv;
        const float o2 = acc[mb][nb][grp * 4 + 2] * inv, o3 = acc[mb][nb][grp * 4 + 3] * inv;
        if (out_bf16) {
          uint2 w;
          w.x = pack_bf16x2(o0, o1);
          w.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>((bf16_raw*)out + obase + d0) = w;
        } else {
          *reinterpret_cast<float4*>((float*)out + obase + d0) = make_float4(o0, o1, o2, o3);
        }
      }
    if (lse && half == 0)
      lse[(int64_t)qi * s.Hq + h] = l_run[nb] > 0.f ? (m_run[nb] + log2f(l_run[nb])) * 0.6931471805599453f : -INFINITY;
  }
}

// Selection plan: rows of query blocks (bsel = 64) or of queries (bsel = 1)
// are scored and selected a slab at a time.
struct PrefillSelPlan {
  int32_t nblk;      // query blocks (or queries)
  int64_t slab;      // blocks per slab
  int32_t self;      // the own token is a candidate (per query)
  int64_t ldx;       // score row stride (candidates of the last row)
  int32_t nparts;    // per-head passes: wave partials per row
  size_t off_x, off_part, off_lse, off_sel, total;
};

PrefillSelPlan prefill_sel_plan(const Shape& s, int32_t n_tokens, int32_t bsel, bool probs) {
  PrefillSelPlan p;
  p.nblk = (n_tokens + bsel - 1) / bsel;
  p.self = bsel == 1 ? 1 : 0;
  if (bsel == 1) {  // query slabs of about 512 MB of scores, 256 .. 4096 queries
    int64_t q = ((int64_t)512 << 20) / ((int64_t)s.Hkv * n_tokens * 4);
    q = q < 256 ? 256 : (q > 4096 ? 4096 : q);
    p.slab = p.nblk < q ? p.nblk : q;
  } else {
    p.slab = p.nblk < kSlab ? p.nblk : kSlab;
  }
  p.ldx = n_tokens > 1 ? n_tokens : 1;
  p.nparts = probs ? (int32_t)(((n_tokens + 255) / 256) * 4) : 0;
  const int G = s.Hq / s.Hkv;
  size_t off = probs ? align_up((size_t)n_tokens * s.Hq * kRank * sizeof(float), 256)
                     : align_up((size_t)p.nblk * s.Hkv * kRank * sizeof(float), 256);
  p.off_x = off;
  off += align_up((size_t)p.slab * s.Hkv * (size_t)p.ldx * sizeof(float), 256);
  p.off_part = off;
  if (probs) off += align_up((size_t)p.slab * s.Hkv * p.nparts * G * sizeof(float2), 256);
  p.off_lse = off;
  if (probs) off += align_up((size_t)n_tokens * s.Hq * sizeof(float), 256);
  p.off_sel = off;
  off += align_up(select_workspace_bytes((int32_t)(p.slab * s.Hkv), n_tokens), 256);
  p.total = off;
  return p;
}

}  // namespace

// Workspace of the prefill selection: the larger of the three plans (block
// supports; per-query with logits; per-query with probabilities).
size_t prefill_select_workspace_bytes(const Shape& s, int32_t n_tokens) {
  size_t a = prefill_sel_plan(s, n_tokens, kQB, false).total;
  const size_t b = prefill_sel_plan(s, n_tokens, 1, false).total;
  const size_t c = prefill_sel_plan(s, n_tokens, 1, true).total;
  a = a > b ? a : b;
  return a > c ? a : c;
}

hipError_t launch_prefill_select(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* w_q, const void* kidx_pool,
                                 sa_dtype dt, float s_idx, int32_t b_sel, int32_t k,
                                 int32_t* idx, int32_t* count, int32_t cap, void* ws,
                                 hipStream_t st, bool probs) {
  const PrefillSelPlan P = prefill_sel_plan(s, n_tokens, b_sel, probs);
  const int G = s.Hq / s.Hkv;
  char* base = (char*)ws;
  float* qv = (float*)base;  // qcb [nblk][Hkv][16] or, per head, qh [n][Hq][16]
  float* xs = (float*)(base + P.off_x);
  float2* part = (float2*)(base + P.off_part);
  float* lse2 = (float*)(base + P.off_lse);
  void* sel_ws = base + P.off_sel;
  const bool bf = dt == SA_BF16;
  if (probs) {
    dim3 g1(n_tokens, s.Hkv);
    if (bf) k_prefill_qh<bf16_raw><<<g1, 256, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)w_q,
                                                      s.Hq, s.Hkv, s.D, s_idx, qv);
    else k_prefill_qh<float><<<g1, 256, 0, st>>>((const float*)q, (const float*)w_q, s.Hq, s.Hkv,
                                                 s.D, s_idx, qv);
  } else {
    dim3 g1(P.nblk, s.Hkv);
    if (bf) k_prefill_qc<bf16_raw><<<g1, 256, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)w_q,
                                                      n_tokens, s.Hq, s.Hkv, s.D, b_sel, s_idx, qv);
    else k_prefill_qc<float><<<g1, 256, 0, st>>>((const float*)q, (const float*)w_q, n_tokens, s.Hq,
                                                 s.Hkv, s.D, b_sel, s_idx, qv);
  }
  for (int b0 = 0; b0 < P.nblk; b0 += (int)P.slab) {
    const int b1 = b0 + (int)P.slab < P.nblk ? b0 + (int)P.slab : P.nblk;
    const int64_t cand_hi = (int64_t)b_sel * (b1 - 1) + P.self;  // candidates of the last row
    const int64_t ldx = cand_hi > 0 ? cand_hi : 1;
    // logit scores go to the selection as 16-bit keys (exact scores of the
    // threshold bin are recomputed there) when its one-block rows take them
    const bool key16 = !probs && ldx <= kSelectRowMax;
    if (probs) {
      const int ntile = (int)((cand_hi + 255) / 256);
      dim3 g2(ntile > 0 ? ntile : 1, (b1 - b0 + kRowsQ - 1) / kRowsQ, s.Hkv);
#define SA_HP(GG)                                                                               \
  case GG:                                                                                      \
    if (bf) {                                                                                   \
      k_prefill_hprob<bf16_raw, GG, 0><<<g2, 256, 0, st>>>((const bf16_raw*)kidx_pool,          \
          pg.page_table, qv, lse2, b0, b1, s, part, P.nparts, xs, ldx);                         \
      k_prefill_hnorm<GG><<<(b1 - b0) * s.Hkv, 256, 0, st>>>(part, P.nparts, b0, s.Hq, s.Hkv, lse2); \
      k_prefill_hprob<bf16_raw, GG, 1><<<g2, 256, 0, st>>>((const bf16_raw*)kidx_pool,          \
          pg.page_table, qv, lse2, b0, b1, s, part, P.nparts, xs, ldx);                         \
    } else {                                                                                    \
      k_prefill_hprob<float, GG, 0><<<g2, 256, 0, st>>>((const float*)kidx_pool,                \
          pg.page_table, qv, lse2, b0, b1, s, part, P.nparts, xs, ldx);                         \
      k_prefill_hnorm<GG><<<(b1 - b0) * s.Hkv, 256, 0, st>>>(part, P.nparts, b0, s.Hq, s.Hkv, lse2); \
      k_prefill_hprob<float, GG, 1><<<g2, 256, 0, st>>>((const float*)kidx_pool,                \
          pg.page_table, qv, lse2, b0, b1, s, part, P.nparts, xs, ldx);                         \
    }                                                                                           \
    break;
      switch (G) {
        SA_HP(1)
        SA_HP(2)
        SA_HP(4)
        SA_HP(8)
        SA_HP(16)
        default: return hipErrorNotSupported;
      }
#undef SA_HP
    } else {
      dim3 g2((unsigned)((ldx + 255) / 256), (b1 - b0 + kRowsT - 1) / kRowsT, s.Hkv);
      const int64_t ldw = ((ldx + 127) / 128) * 64;  // 16-bit keys: words per row
      if (key16) {
        if (bf)
          k_prefill_scores<bf16_raw, true><<<g2, 256, 0, st>>>((const bf16_raw*)kidx_pool,
              pg.page_table, qv, b0, b1, b_sel, P.self, s, xs, ldw);
        else
          k_prefill_scores<float, true><<<g2, 256, 0, st>>>((const float*)kidx_pool,
              pg.page_table, qv, b0, b1, b_sel, P.self, s, xs, ldw);
      } else {
        if (bf)
          k_prefill_scores<bf16_raw, false><<<g2, 256, 0, st>>>((const bf16_raw*)kidx_pool,
              pg.page_table, qv, b0, b1, b_sel, P.self, s, xs, ldx);
        else
          k_prefill_scores<float, false><<<g2, 256, 0, st>>>((const float*)kidx_pool,
              pg.page_table, qv, b0, b1, b_sel, P.self, s, xs, ldx);
      }
    }
    SelectArgs a{};
    a.x = xs;
    a.ldx = key16 ? ((ldx + 127) / 128) * 64 : ldx;
    a.seq_lens = nullptr;
    a.rows = (b1 - b0) * s.Hkv;
    if (key16) {
      a.key16 = 1;
      a.qcb = qv;
      a.kidx = kidx_pool;
      a.kidx_bf16 = bf ? 1 : 0;
      a.pt = pg.page_table;
      a.n_pool_pages = s.n_pool_pages;
    }
    a.Hkv = s.Hkv;
    a.max_len = n_tokens;
    a.unit = 1;
    a.max_cand = (int32_t)ldx;
    a.is_topk = 1;
    a.p = 0.f;
    a.k = k;
    a.n_sink = 0;
    a.n_window = P.self;  // per query: the own token is always kept
    a.idx = idx + (int64_t)b0 * s.Hkv * cap;
    a.count = count + (int64_t)b0 * s.Hkv;
    a.cap = cap;
    a.prefill_bsel = b_sel;
    a.prefill_blk0 = b0;
    a.prefill_self = P.self;
    hipError_t e = launch_select(a, sel_ws, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

// Per-query attention: the split-KV decode kernels with every query row as a
// "sequence" of length i + 1 that shares the one page table row.
size_t prefill_query_workspace_bytes(const Shape& s, int32_t n_tokens, int32_t cap) {
  Shape s2 = s;
  s2.B = kPrefillQuerySlab;
  return align_up((size_t)n_tokens * sizeof(int32_t), 256) + decode_workspace_bytes(s2, cap);
}

hipError_t launch_sparse_prefill_query(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       sa_dtype dt, const int32_t* idx, const int32_t* count,
                                       int32_t cap, float s_att, void* out, sa_dtype out_dt,
                                       float* lse, void* ws, hipStream_t st) {
  int32_t* lens = (int32_t*)ws;
  void* dws = (char*)ws + align_up((size_t)n_tokens * sizeof(int32_t), 256);
  k_iota1<<<(n_tokens + 255) / 256, 256, 0, st>>>(lens, n_tokens);
  const size_t qe = dt == SA_BF16 ? 2 : 4, oe = out_dt == SA_BF16 ? 2 : 4;
  // the decode kernels plan at most 4096 (row, group) pairs per launch
  const int32_t qslab = kPrefillQuerySlab < 4096 / s.Hkv ? kPrefillQuerySlab : 4096 / s.Hkv;
  for (int32_t q0 = 0; q0 < n_tokens; q0 += qslab) {
    const int32_t nq = n_tokens - q0 < qslab ? n_tokens - q0 : qslab;
    Shape s2 = s;
    s2.B = nq;
    s2.max_pages = 0;  // every query row reads page-table row 0
    sa_pages p2;
    p2.page_table = pg.page_table;
    p2.seq_lens = lens + q0;
    hipError_t e = launch_sparse_decode(
        s2, p2, (const char*)q + (size_t)q0 * s.Hq * s.D * qe, k_pool, v_pool, dt,
        idx + (int64_t)q0 * s.Hkv * cap, count + (int64_t)q0 * s.Hkv, cap, s_att,
        (char*)out + (size_t)q0 * s.Hq * s.D * oe, out_dt, lse ? lse + (int64_t)q0 * s.Hq : nullptr,
        dws, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* idx, const int32_t* count, int32_t cap,
                                 int32_t b_sel, float s_att, void* out, sa_dtype out_dt,
                                 float* lse, hipStream_t st) {
  const int nblk = (n_tokens + kQB - 1) / kQB;
  const int G = s.Hq / s.Hkv;
  const int HB = G < 4 ? G : 4;
  dim3 grid(nblk * s.Hkv * (G / HB));
#define SA_PA(HH)                                                                           \
  k_prefill_attn<HH><<<grid, HH * 2 * 64, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)k_pool, \
                                                   (const bf16_raw*)v_pool, pg.page_table, idx, \
                                                   count, cap, n_tokens, s, s_att, out,         \
                                                   out_dt == SA_BF16, lse)
  switch (HB) {
    case 1: SA_PA(1); break;
    case 2: SA_PA(2); break;
    default: SA_PA(4); break;
  }
#undef SA_PA
  return hipGetLastError();
}

}  // namespace sa
