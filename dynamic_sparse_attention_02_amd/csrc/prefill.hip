// Causal prefill with supports shared by blocks of b_sel = 64 queries
// ("Oracle-Guided Sparse Prefill", section 2.1: top-k support per selection
// block, attention recomputed with the original q, k, v over the support;
// section 2.2: one head-collapsed indexer channel).
//
// Selection: per (query block, group) the block-collapsed indexer query is
// formed (sum of the block's queries per head, then projected).  With bf16
// indexer keys the scores over the keys of all earlier blocks are formed on
// the matrix cores against a sampled per-row threshold, and only the hits
// (a few thousand per row) reach the exact top-k; otherwise the scores of a
// slab of query blocks are written and the row-resident radix select keeps
// the top k of each row.
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
// Query blocks per score slab.  One slab holds the whole 128K prefill (2048
// blocks): a single launch of each selection kernel balances the rows'
// uneven work over the chip, where eight slabs paid eight launch tails
// (1.52 -> 1.38 ms).  The slab's fp32 score rows (8.6 GB at 128K, used only
// when a row leaves the hit path) are sized for a GPU with hundreds of GB.
constexpr int kSlab = 2048;

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
constexpr int kQcNT = 256;  // threads of k_prefill_qc
template <typename T>
__global__ void __launch_bounds__(kQcNT)
k_prefill_qc(const T* __restrict__ q, const T* __restrict__ w_q, int32_t N, int32_t Hq,
             int32_t Hkv, int32_t D, int32_t bsel, float s_idx, float* __restrict__ qcb) {
  const int blk = blockIdx.x, g = blockIdx.y;
  const int G = Hq / Hkv;
  const int r0 = blk * bsel;
  const int nr = min(bsel, N - r0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = G * D / 8;              // (head, 8 dims) chunks: <= 256
  const int parts = kQcNT / chunks;          // row shares per chunk
  const int ch = threadIdx.x % chunks, part = threadIdx.x / chunks;
  const int h = g * G + (ch * 8) / D, d0 = (ch * 8) % D;
  __shared__ float qs[kQcNT][8];             // each thread's partial sums
  float acc8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  if (part < parts) {
    int i = part;
    if constexpr (sizeof(T) == 2) {
      auto add = [&](const uint4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc8[2 * e] += __uint_as_float(w[e] << 16);
          acc8[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
        }
      };
      // eight rows' loads in flight at a time (the sum order is the same)
      for (; i + 7 * parts < nr; i += 8 * parts) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = *reinterpret_cast<const uint4*>(q + ((int64_t)(r0 + i + u * parts) * Hq + h) * D + d0);
#pragma unroll
        for (int u = 0; u < 8; ++u) add(v[u]);
      }
      for (; i < nr; i += parts) add(*reinterpret_cast<const uint4*>(q + ((int64_t)(r0 + i) * Hq + h) * D + d0));
    } else {
      for (; i < nr; i += parts) {
        const T* src = q + ((int64_t)(r0 + i) * Hq + h) * D + d0;
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
  __shared__ float red[kQcNT / 64][kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) {
    const float v = wave_sum(acc[c]);
    if (lane == 0) red[wave][c] = v;
  }
  __syncthreads();
  if (threadIdx.x < kRank) {
    const int c = threadIdx.x;
    static_assert(kQcNT == 256, "four waves' sums");
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
constexpr int kTileBytes = kKT * 128 * 2;  // one 64-key tile of K or V (d = 128 bf16)
constexpr int kMaxListed = 2048;        // listed keys per block the attention kernel takes
constexpr float kLazy = 8.f;            // log2 headroom of the lazily raised softmax maximum

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// a.x * b.x + a.y * b.y + c over bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
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

  // K and V tiles, three of each (tile t in buffer t mod 3).  A tile is
  // chunk-major: chunk c (dims 8c .. 8c + 7, 16 bytes per key) of the 64
  // keys fills 1 KB, key r at slot r ^ 4 (c & 1) ^ 8 ((c >> 1) & 1), so
  // that the K operand reads and the transposing V reads below are free of
  // conflicts on the 64 LDS banks (each 256-byte access phase covers every
  // bank once).
  __shared__ __align__(16) char K0[kTileBytes], K1[kTileBytes], K2[kTileBytes];
  __shared__ __align__(16) char V0[kTileBytes], V1[kTileBytes], V2[kTileBytes];
  // pool row (page * Hkv + g) * 64 + slot of every key the item visits, in
  // tile order (listed keys, then the diagonal block); -1 marks padding
  __shared__ int32_t rows_lds[kMaxListed + kKT];

  // Q as the B operand of S^T = K Q^T: Qb[nb][ks] holds query nb*32 + l32,
  // dims ks*16 + 8*half .. +7
  // The query is stored pre-scaled by s_att * log2(e) (rounded once to
  // bf16), so the products are the logits in log2 units.
  const float sl2 = s_att * 1.4426950408889634f;
  bf16x8_t Qb[NBQ][8];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    const int32_t qi = q0 + (qpart * NBQ + nb) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qi < N)
        v = *reinterpret_cast<const uint4*>(q + ((int64_t)qi * s.Hq + h) * D + ks * 16 + 8 * half);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(__uint_as_float(w[e] << 16) * sl2, __uint_as_float(w[e] & 0xffff0000u) * sl2);
      Qb[nb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }

  // resolve every key's pool row once (list entry -> page table -> row)
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const kb0 = (lds_char*)K0;
  lds_char* const kb1 = (lds_char*)K1;
  lds_char* const kb2 = (lds_char*)K2;
  lds_char* const vb0 = (lds_char*)V0;
  lds_char* const vb1 = (lds_char*)V1;
  lds_char* const vb2 = (lds_char*)V2;
  // every slot starts at zero: a slot that no key fills keeps finite values
  // (zero, or an earlier tile's key), which the mask turns into P = 0
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  for (int o = tid * 16; o < kTileBytes; o += NT * 16) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    *(lds_u32x4*)(kb0 + o) = z;
    *(lds_u32x4*)(kb1 + o) = z;
    *(lds_u32x4*)(kb2 + o) = z;
    *(lds_u32x4*)(vb0 + o) = z;
    *(lds_u32x4*)(vb1 + o) = z;
    *(lds_u32x4*)(vb2 + o) = z;
  }
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
  // Gather straight into LDS (global_load_lds_dwordx4): instruction i of a
  // wave moves chunk c = i * NT / 64 + wave of the tile's 64 keys, lane p
  // loading the key of slot p.  No registers hold the tile and
  // no LDS stores are issued; the barrier that precedes a tile's first use
  // waits for its loads.
  typedef __attribute__((address_space(3))) void lds_void;
  // s_waitcnt vmcnt(0): this wave's loads into LDS have landed.  Issued
  // before every barrier that publishes a tile, so that after the barrier
  // every wave's part of it is there (the compiler's own waits are not
  // relied on for this).
  auto wait_loads = []() { __builtin_amdgcn_s_waitcnt(0x0F70); };
  auto gather = [&](int tile, lds_char* dk, lds_char* dv) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = (i * NT + tid) >> 6;
      if (c < 16) {
        const int r = lane ^ (4 * (c & 1)) ^ (8 * ((c >> 1) & 1));
        const int32_t rw = rows_lds[tile * kKT + r];
        if (rw >= 0) {
          const int64_t off = (int64_t)rw * D + c * 8;
          __builtin_amdgcn_global_load_lds((const void*)(k_pool + off), (lds_void*)(dk + c * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(v_pool + off), (lds_void*)(dv + c * 1024), 16, 0, 0);
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
  // m_run: running maximum (log2 units, -inf before the first key);
  // negm: -m_run (0 before the first key) in every accumulator slot, the
  // C operand of each tile's first product, so the products come out as
  // logit - m_run and feed the exponential directly.
  float m_run[NBQ], l_run[NBQ];
  f32x16_t negm[NBQ];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) negm[nb][v] = 0.f;
  }
  const uint32_t ones2 = 0x3f803f80u;  // bf16 pair (1, 1)

  // K Q^T of a tile: S^T[key][query] for the 64 keys x 32 queries of this
  // wave, minus the running maximum.  ka: this lane's K operand address in
  // the tile (key mk * 32 + l32, chunk 2 ks + half, in its swizzled slot)
  // for even ks; odd ks flip the slot's bit 3 (ka1 = address ^ 128).
  f32x16_t S[2][NBQ];
  const int klane = half * 1024 + (l32 ^ (4 * half)) * 16;
  auto score_mfma = [&](lds_char* ka, lds_char* ka1, int ks, int mk) {
    const u32x4_t a = *(const lds_u32x4*)(((ks & 1) ? ka1 : ka) + (ks * 2048 + mk * 512));
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb)
      S[mk][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, Qb[nb][ks], ks == 0 ? negm[nb] : S[mk][nb], 0, 0, 0);
  };
  // O^T[d][query] += V^T[d][key] P^T[key][query] for one 16-key step st of
  // a tile and one 32-row block mb of d (keys in the score accumulator's
  // order).  The V^T operand comes through the transposing LDS read
  // (ds_read_b64_tr_b16): in each 16-lane group, lane 4k + t points at dims
  // 4t .. 4t + 3 of key k, and lane j then receives dim j of the four keys.
  // Group g = lane / 16 takes dims (g & 1) * 16 .. + 15 of the block and
  // keys 4 (g >> 1) + 0..3 (then + 8), which is the operand's layout: lane
  // (l32, half) holds d = l32 of keys 4 half + 0..3 and 8 + 4 half + 0..3
  // of the step.  va: this lane's address in the tile for st = mb = 0 (its
  // first four keys); va1 = va ^ 128, the next four (slot bit 3 flipped).
  bf16x8_t Pb[4][NBQ];
  const int vg = lane >> 4, vs = lane & 15;
  const int vlane = ((vg & 1) * 2 + ((vs >> 1) & 1)) * 1024 +
                    ((4 * (vg >> 1) + (vs >> 2)) ^ (4 * ((vs >> 1) & 1)) ^ (8 * (vg & 1))) * 16 + (vs & 1) * 8;
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
  auto pv_mfma = [&](lds_char* va, lds_char* va1, int st, int mb) {
    const int kb = (st >> 1) * 32 + (st & 1) * 16;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va + (mb * 4096 + kb * 16)));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va1 + (mb * 4096 + kb * 16)));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, Pb[st][nb], acc[mb][nb], 0, 0, 0);
  };
  // a lane offset made opaque to the optimiser (per use), so that the reads
  // of a tile add their constant offsets to one register instead of each
  // keeping its own precomputed address; the buffer itself stays visible,
  // so the compiler knows that these reads do not touch the buffers whose
  // loads are in flight
  auto opaque = [](int v) {
    asm volatile("" : "+v"(v));
    return v;
  };

  // Tiles cycle through the three buffers, loaded two tiles ahead of their
  // products, so after the single barrier of iteration t the products of
  // tile t (P V) and the scores of tile t + 1 (K Q^T) are independent and
  // interleave.  The buffers loaded in iteration t last held tile t - 1,
  // which every wave finished before that barrier.  The loop is unrolled by
  // three so that each buffer is a distinct LDS object in every iteration
  // (the compiler then need not wait for the loads in flight before each
  // read).  The last iteration scores a stale buffer (in bounds, result
  // unused) so that its body has no branch between the two product chains.
  gather(0, kb0, vb0);
  if (n_tiles > 1) gather(1, kb1, vb1);
  wait_loads();
  __syncthreads();
  {
    lds_char* ka = kb0 + opaque(klane);
    lds_char* ka1 = kb0 + opaque(klane ^ 128);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) score_mfma(ka, ka1, ks, mk);
  }
  auto body = [&](lds_char* vcur, lds_char* knext, lds_char* dk, lds_char* dv, int tile) {
    const bool diag = tile == n_list_tiles;
    const int nt = diag ? nq : min(kKT, nl - tile * kKT);

    // online softmax per query (lane's query nb*32 + l32; keys spread over
    // this lane's 32 accumulator values and the partner lane's); S holds
    // logit - m_run in log2 units.  The running maximum is raised only when
    // a tile's maximum exceeds it by more than kLazy (so P stays below
    // 2^kLazy): the output accumulator is rescaled on those tiles only.
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
      mt[nb] = fmaxf(m, __shfl_xor(m, 32, 64));
    }
    bool raise[NBQ], any_raise = false;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      raise[nb] = m_run[nb] == -INFINITY ? mt[nb] > -INFINITY : mt[nb] > kLazy;
      any_raise = any_raise || raise[nb];
    }
    if (__ballot(any_raise)) {
      float alpha[NBQ];
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        const bool r = raise[nb];
        const float shift = r ? mt[nb] : 0.f;
        const float m_new = r ? (m_run[nb] == -INFINITY ? 0.f : m_run[nb]) + mt[nb] : m_run[nb];
        alpha[nb] = r ? __builtin_amdgcn_exp2f(m_run[nb] - m_new) : 1.f;  // 0 on the first raise
        l_run[nb] *= alpha[nb];
        m_run[nb] = m_new;
#pragma unroll
        for (int mk = 0; mk < 2; ++mk)
#pragma unroll
          for (int v = 0; v < 16; ++v) S[mk][nb][v] -= shift;
        const float nm = m_new == -INFINITY ? 0.f : -m_new;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[nb][v] = nm;
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mb][nb][v] *= alpha[nb];
    }
    // P = 2^S as bf16 (the B operand of the P V products, keys in the
    // accumulator's order) and its row sum from the same bf16 values
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      float lt = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int mk = st >> 1, hv = (st & 1) * 8;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = pack_bf16x2(__builtin_amdgcn_exp2f(S[mk][nb][hv + 2 * e]),
                             __builtin_amdgcn_exp2f(S[mk][nb][hv + 2 * e + 1]));
          lt = dot2_bf16(w[e], ones2, lt);
        }
        Pb[st][nb] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
      l_run[nb] += lt + __shfl_xor(lt, 32, 64);
    }
    wait_loads();
    __syncthreads();
    if (tile + 2 < n_tiles) gather(tile + 2, dk, dv);
    lds_char* va = vcur + opaque(vlane);
    lds_char* va1 = vcur + opaque(vlane ^ 128);
    lds_char* ka = knext + opaque(klane);
    lds_char* ka1 = knext + opaque(klane ^ 128);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pv_mfma(va, va1, i >> 2, i & 3);
      score_mfma(ka, ka1, i >> 1, i & 1);
    }
  };
  for (int t0 = 0;; t0 += 3) {
    body(vb0, kb1, kb2, vb2, t0);
    if (t0 + 1 >= n_tiles) break;
    body(vb1, kb2, kb0, vb0, t0 + 1);
    if (t0 + 2 >= n_tiles) break;
    body(vb2, kb0, kb1, vb1, t0 + 2);
    if (t0 + 3 >= n_tiles) break;
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

// ---------------------------------------------------------------------------
// Top-k rows with bf16 indexer keys (k <= kHitMaxK): three launches per slab
// instead of one fp32 score per candidate written and read back.
//   k_pf_thresh (one launch for every row): per row, a threshold lo from a sample of the row (the scores
//     of every stride-th 16-candidate tile): the 24-bit key floor at which ks
//     sampled keys are reached from the top, ks set so that the whole row
//     holds between k and kHitCap keys >= lo except with negligible
//     probability.  Rows of at most kHitCap candidates take lo = 0.
//   k_pf_hits: the scores of 64 rows x 256 candidates per workgroup on the
//     matrix cores, written as a hit bitmap (key >= lo) plus the keys of the
//     first kSlotCap hits of each (row, 256-candidate tile).
//   k_pf_select: per row, the exact top k among the hits: the hit list from
//     the bitmap and the stored keys (a tile with more hits has its keys
//     recomputed), then the radix levels over the list.  A row whose hits do
//     not bracket k (fewer than k, or more than kHitCap) is resolved over all
//     its candidates, the keys recomputed tile by tile.
// A score is one matrix-core product (v_mfma_f32_16x16x32_bf16, fp32
// accumulate) wherever it is formed: the block's indexer query, split into a
// bf16 high part and the bf16 rounding of the remainder (16 significant
// bits), sits in row (blk - blk0) mod 16 of the A operand and the candidate's
// key in column c mod 16 of the B operand, with the same k order (high part
// against the 16 key values, then low part), in both k_pf_hits and
// k_pf_select, so both see the same float for every candidate.
// ---------------------------------------------------------------------------
constexpr int kHitCap = 4096;      // hits a row's exact selection holds in LDS
constexpr int kSlotCap = 128;      // keys stored per (row, 256-candidate tile)
constexpr int kHitSample = 16384;  // sampled candidates per row at most
constexpr int kSelNT = 512;        // threads of k_pf_thresh and k_pf_select
constexpr int kHitMaxK = 2048;     // largest k the hit path takes
typedef __attribute__((ext_vector_type(8))) float f32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// A operand of the score product: lane l holds row l % 16's k-slice
// 8 (l / 16) .. + 8, i.e. q[0..8) and q[8..16) of the high part for slices 0
// and 1, of the low part for slices 2 and 3 (zero when !valid).
__device__ __forceinline__ bf16x8_t split_query(const float* __restrict__ q16, int lane, bool valid) {
  const int lg = lane >> 4;
  f32x8_t f = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float4 a = *reinterpret_cast<const float4*>(q16 + 8 * (lg & 1));
    const float4 b = *reinterpret_cast<const float4*>(q16 + 8 * (lg & 1) + 4);
    f = f32x8_t{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
  const bf16x8_t hi = __builtin_convertvector(f, bf16x8_t);
  if (lg < 2) return hi;
  return __builtin_convertvector(f - __builtin_convertvector(hi, f32x8_t), bf16x8_t);
}

// The U 16-candidate tiles from cb (a multiple of 16) against the A
// operand: acc[u] holds the products of candidate cb + 16 u + (lane % 16)
// with rows 4 (lane / 16) + i.  A tile's 16 candidates share one page, so
// its page id is one uniform load; the key loads are branch-free (a tile
// past lim reads the last valid page, a candidate past lim its page's row)
// and zeroed afterwards, so all U of them are in flight together.
template <int U>
__device__ __forceinline__ void load_tiles(const bf16_raw* __restrict__ kidx,
                                           const int32_t* __restrict__ pt, const Shape& s, int g,
                                           int32_t cb, int32_t lim, int lane, uint4 (&kv)[U]) {
  const int col = lane & 15;
  const int32_t plast = lim > 0 ? (lim - 1) >> 6 : 0;
  int64_t page[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t pi = (cb + 16 * u) >> 6;
    page[u] = clamp_page(pt[pi < plast ? pi : plast], s.n_pool_pages);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t c = cb + 16 * u + col;
    kv[u] = *reinterpret_cast<const uint4*>(kidx + ((page[u] * s.Hkv + g) * kPage + (c & 63)) * kRank +
                                            8 * ((lane >> 4) & 1));
  }
}
template <int U>
__device__ __forceinline__ void product_tiles(int32_t cb, int32_t lim, bf16x8_t qa, int lane,
                                              const uint4 (&kv)[U], f32x4_t (&acc)[U]) {
  const int col = lane & 15;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = cb + 16 * u + col < lim;
    const uint4 w = ok ? kv[u] : make_uint4(0u, 0u, 0u, 0u);
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, __builtin_bit_cast(bf16x8_t, w),
                                                     f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
}
template <int U>
__device__ __forceinline__ void score_tiles(const bf16_raw* __restrict__ kidx,
                                            const int32_t* __restrict__ pt, const Shape& s, int g,
                                            int32_t cb, int32_t lim, bf16x8_t qa, int lane,
                                            f32x4_t (&acc)[U]) {
  uint4 kv[U];
  load_tiles<U>(kidx, pt, s, g, cb, lim, lane, kv);
  product_tiles<U>(cb, lim, qa, lane, kv, acc);
}

// Exclusive scan over the kSelNT threads.
__device__ __forceinline__ uint32_t sel_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  constexpr int NW = kSelNT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) red[w] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t x = red[i];
    off += i < w ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// The bin of hc[0, nb) where the count from the top bin down reaches need
// (1 <= need): *bin (0xffffffff if the bins hold fewer) and *before, the
// count of the bins above it.
__device__ __forceinline__ void top_bin(const uint32_t* hc, int nb, uint32_t need, uint32_t* red,
                                        uint32_t* bin, uint32_t* before) {
  const int t = threadIdx.x;
  const int per = nb / kSelNT > 0 ? nb / kSelNT : 1;
  const bool owns = t * per < nb;
  uint32_t c = 0;
  if (owns)
    for (int e = 0; e < per; ++e) c += hc[nb - 1 - (t * per + e)];
  if (t == 0) *bin = 0xffffffffu;
  uint32_t tot;
  uint32_t cb = sel_scan(c, red, tot);
  if (owns)
    for (int e = 0; e < per; ++e) {
      const int b = nb - 1 - (t * per + e);
      const uint32_t v = hc[b];
      if (cb < need && cb + v >= need) {
        *bin = (uint32_t)b;
        *before = cb;
      }
      cb += v;
    }
  __syncthreads();
}

// The sampled thresholds of rows (blk, g) and (blk + 1, g), blk = 2 (w /
// Hkv), g = w % Hkv for workgroup w, over all query blocks (or queries): lo
// such that the row holds between k and kHitCap keys >= lo except with
// negligible probability; rows of at most kHitCap candidates take 0.  The
// two rows share the sampled key rows (one load scores both queries).
constexpr int kThrPer = 24;  // sampled candidates per thread (stride >= 11)
__global__ void __launch_bounds__(kSelNT, 4)
k_pf_thresh(const bf16_raw* __restrict__ kidx, const int32_t* __restrict__ pt,
            const float* __restrict__ qcb, int32_t nblk, int32_t bsel, int32_t self, Shape s,
            int32_t k, int32_t stride, uint32_t* __restrict__ lo_all) {
  const int t = threadIdx.x;
  const int g = blockIdx.x % s.Hkv;
  const int32_t blk0 = 2 * (int32_t)(blockIdx.x / s.Hkv);
  __shared__ float qs[2][kRank];
  __shared__ uint32_t hc[2][4096];
  __shared__ int32_t s_pg[kThrPer * kSelNT / 16];  // pool page of each sampled tile
  __shared__ uint32_t red[kSelNT / 64];
  __shared__ uint32_t s_bin, s_bef;
  // per row: candidates, sampled tiles and candidates, the sample count ks
  // the threshold must reach (0: the row takes lo = 0)
  int32_t n[2], nst[2];
  uint32_t ks[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int32_t blk = blk0 + r;
    n[r] = blk < nblk ? bsel * blk + self : 0;
    nst[r] = 0;
    ks[r] = 0u;
    if (n[r] > kHitCap) {
      const int32_t ntl = (n[r] + 15) >> 4;  // 16-candidate tiles
      nst[r] = (ntl + stride - 1) / stride;   // sampled tiles: 16 nst <= kThrPer kSelNT
      const int32_t last = (nst[r] - 1) * stride;
      const int32_t m = nst[r] * 16 - (last == ntl - 1 ? ntl * 16 - n[r] : 0);
      const float kf = (float)k * (float)m / (float)n[r];
      const uint32_t kk = (uint32_t)ceilf(kf + 5.5f * sqrtf(kf) + 6.f);
      ks[r] = kk < (uint32_t)m ? kk : 0u;
    }
  }
  if (ks[0] == 0u && ks[1] == 0u) {
    if (t < 2 && blk0 + t < nblk) lo_all[(int64_t)(blk0 + t) * s.Hkv + g] = 0u;
    return;
  }
  const int32_t nsa = nst[0] > nst[1] ? nst[0] : nst[1];  // the sample of the longer row
  for (int j = t; j < nsa; j += kSelNT) s_pg[j] = (int32_t)clamp_page(pt[(j * stride) >> 2], s.n_pool_pages);
  for (int i = t; i < 2 * 4096; i += kSelNT) (&hc[0][0])[i] = 0u;
  if (t < 2 * kRank) {
    const int r = t / kRank;
    qs[r][t % kRank] = blk0 + r < nblk ? qcb[((int64_t)(blk0 + r) * s.Hkv + g) * kRank + t % kRank] : 0.f;
  }
  __syncthreads();
  uint32_t key0[kThrPer], key1[kThrPer];
  uint32_t v0 = 0u, v1 = 0u;  // bit e: sample e is a candidate of row 0 / 1 with ks != 0
#pragma unroll
  for (int e = 0; e < kThrPer; ++e) key0[e] = key1[e] = 0u;
#pragma unroll
  for (int e0 = 0; e0 < kThrPer; e0 += 4) {
    if (e0 * kSelNT >= nsa * 16) break;  // (uniform) past the sample
    // branch-free loads (a position past the sample reads the first
    // sampled candidate); a sampled tile's 16 candidates share a page
    uint4 va[4], vb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t i = (e0 + e) * kSelNT + t;  // sample position
      const int32_t c = (((i >> 4) * stride) << 4) + (i & 15);
      const bool ok = i < nsa * 16;
      v0 |= (ok && ks[0] != 0u && i < nst[0] * 16 && c < n[0]) ? 1u << (e0 + e) : 0u;
      v1 |= (ok && ks[1] != 0u && i < nst[1] * 16 && c < n[1]) ? 1u << (e0 + e) : 0u;
      const int64_t page = s_pg[ok ? i >> 4 : 0];
      const uint4* v = reinterpret_cast<const uint4*>(kidx + ((page * s.Hkv + g) * kPage + ((ok ? c : 0) & 63)) * kRank);
      va[e] = v[0];
      vb[e] = v[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u[8] = {va[e].x, va[e].y, va[e].z, va[e].w, vb[e].x, vb[e].y, vb[e].z, vb[e].w};
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lo16 = __uint_as_float(u[j] << 16), hi16 = __uint_as_float(u[j] & 0xffff0000u);
        a0 = fmaf(qs[0][2 * j], lo16, a0);
        a0 = fmaf(qs[0][2 * j + 1], hi16, a0);
        a1 = fmaf(qs[1][2 * j], lo16, a1);
        a1 = fmaf(qs[1][2 * j + 1], hi16, a1);
      }
      key0[e0 + e] = score_key(a0);
      key1[e0 + e] = score_key(a1);
      if ((v0 >> (e0 + e)) & 1u) atomicAdd(&hc[0][key0[e0 + e] >> 20], 1u);
      if ((v1 >> (e0 + e)) & 1u) atomicAdd(&hc[1][key1[e0 + e] >> 20], 1u);
    }
  }
  __syncthreads();
  // level 1 of both rows, then level 2 inside each row's crossing bin
  uint32_t b1[2] = {0xffffffffu, 0xffffffffu}, bef[2] = {0u, 0u};
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (ks[r] == 0u) continue;  // (uniform)
    top_bin(hc[r], 4096, ks[r], red, &s_bin, &s_bef);
    b1[r] = s_bin;
    bef[r] = s_bef;
  }
  for (int i = t; i < 2 * 4096; i += kSelNT) (&hc[0][0])[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kThrPer; ++e) {
    if (((v0 >> e) & 1u) && (key0[e] >> 20) == b1[0]) atomicAdd(&hc[0][(key0[e] >> 8) & 0xfffu], 1u);
    if (((v1 >> e) & 1u) && (key1[e] >> 20) == b1[1]) atomicAdd(&hc[1][(key1[e] >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint32_t lo = 0u;
    if (ks[r] != 0u && b1[r] != 0xffffffffu) {  // (uniform)
      top_bin(hc[r], 4096, ks[r] - bef[r], red, &s_bin, &s_bef);
      lo = (b1[r] << 20) | ((s_bin == 0xffffffffu ? 0u : s_bin) << 8);
    }
    if (t == 0 && blk0 + r < nblk) lo_all[(int64_t)(blk0 + r) * s.Hkv + g] = lo;
  }
}

constexpr int kHitWaves = 2;  // waves (16 rows each) per k_pf_hits workgroup
__global__ void __launch_bounds__(64 * kHitWaves)
k_pf_hits(const bf16_raw* __restrict__ kidx, const int32_t* __restrict__ pt,
          const float* __restrict__ qcb, const uint32_t* __restrict__ lo_in, int32_t blk0,
          int32_t blk1, int32_t bsel, int32_t self, Shape s, int32_t tpr,
          uint32_t* __restrict__ bits, uint32_t* __restrict__ slots) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar row and page arithmetic
  const int col = lane & 15, lg = lane >> 4;
  const int g = blockIdx.z;
  const int32_t bfirst = blk0 + (int32_t)blockIdx.y * (16 * kHitWaves) + wave * 16;  // this wave's 16 rows
  if (bfirst >= blk1) return;
  const int32_t blast = min(blk1, bfirst + 16) - 1;
  const int32_t nmax = bsel * blast + self;  // candidates of the wave's last row
  const int32_t x = (int32_t)blockIdx.x;  // the 256-candidate tile
  const int32_t cb0 = 256 * x;
  if (cb0 >= nmax) return;  // no row of the wave has candidates here
  __shared__ uint32_t stage[kHitWaves][16][128];  // the keys of one half tile, [row][candidate - cb]
  __shared__ uint64_t msk[kHitWaves][8][4];       // hit ballots, [16-candidate tile][i]: bit 16 q + col = row 4 q + i
  const int32_t bq = bfirst + col;
  const bf16x8_t qa = split_query(qcb + ((int64_t)(bq < blk1 ? bq : bfirst) * s.Hkv + g) * kRank, lane, bq < blk1);
  // the rows' thresholds as floats: for a finite score f, key(f) >= lo
  // exactly when f >= key_score(lo), and every finite f passes when lo is at
  // most the key of -inf
  int32_t n_i[4];
  float lof[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t bb = bfirst + 4 * lg + i;
    const uint32_t lv = lo_in[(int64_t)((bb < blk1 ? bb : blast) - blk0) * s.Hkv + g];
    n_i[i] = bb < blk1 ? bsel * bb + self : 0;
    lof[i] = bb >= blk1 ? INFINITY : (lv <= 0x007fffffu ? -INFINITY : key_score(lv));
  }
  // lane L finishes bitmap word 4 hf + (L % 4) of row L / 4
  const int R = lane >> 2, q = lane & 3;
  const int32_t bR = bfirst + R;
  const bool rowok = bR < blk1 && cb0 < bsel * bR + self;
  const int64_t r = (int64_t)(bR - blk0) * s.Hkv + g;
  uint32_t carry = 0u;  // hits of this row in the first half
  uint4 kv[16];  // both halves' key rows in flight together
  load_tiles<16>(kidx, pt, s, g, cb0, nmax, lane, kv);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int32_t cb = cb0 + 128 * hf;
    f32x4_t acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 w = cb + 16 * u + col < nmax ? kv[8 * hf + u] : make_uint4(0u, 0u, 0u, 0u);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, __builtin_bit_cast(bf16x8_t, w),
                                                       f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    // the scores are staged as floats (keys only for the hits, below);
    // every lane stores the same (uniform) ballot, and when every row of
    // the wave holds all of these candidates the bound check drops out
    if (cb + 128 <= bsel * bfirst + self) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          stage[wave][4 * lg + i][16 * u + col] = __float_as_uint(acc[u][i]);
          msk[wave][u][i] = __builtin_amdgcn_ballot_w64(acc[u][i] >= lof[i]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          stage[wave][4 * lg + i][16 * u + col] = __float_as_uint(acc[u][i]);
          msk[wave][u][i] = __builtin_amdgcn_ballot_w64(cb + 16 * u + col < n_i[i] && acc[u][i] >= lof[i]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // word 4 hf + q of row R: 16-candidate tiles 2q (low half) and 2q + 1
    const uint64_t a = msk[wave][2 * q][R & 3], b = msk[wave][2 * q + 1][R & 3];
    const int sh = 16 * (R >> 2);
    const uint32_t w = (uint32_t)((a >> sh) & 0xffffu) | ((uint32_t)((b >> sh) & 0xffffu) << 16);
    // hits of this row before this word: the first half plus the row's earlier lanes
    const uint32_t pc = (uint32_t)__popc(w);
    uint32_t inc = pc;
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) {
      const uint32_t v = (uint32_t)__shfl_up((int)inc, d, 4);
      if (q >= d) inc += v;
    }
    if (rowok) {
      bits[(r * tpr + x) * 8 + 4 * hf + q] = w;
      uint32_t e = carry + inc - pc, ww = w;
      uint32_t* sl = slots + (r * tpr + x) * kSlotCap;
      while (ww != 0u && e < (uint32_t)kSlotCap) {
        const int bt = __ffs(ww) - 1;
        ww &= ww - 1u;
        sl[e++] = score_key(__uint_as_float(stage[wave][R][32 * q + bt]));
      }
    }
    carry += (uint32_t)__shfl((int)inc, (lane & ~3) + 3);  // the row's total in this half
    // the next half rewrites stage and msk: this wave's reads come first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

__global__ void __launch_bounds__(kSelNT, 6)
k_pf_select(const bf16_raw* __restrict__ kidx, const int32_t* __restrict__ pt,
            const float* __restrict__ qcb, const uint32_t* __restrict__ bits,
            const uint32_t* __restrict__ slots, int32_t blk0, int32_t bsel, int32_t self, Shape s,
            int32_t tpr, int32_t k, int32_t n_window, int32_t* __restrict__ idx_out,
            int32_t* __restrict__ count_out, int32_t cap) {
  constexpr int NT = kSelNT, NW = NT / 64;
  constexpr uint32_t kSearchM = 0, kGEM = 1, kTiesM = 2;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const int g = row % s.Hkv;
  const int32_t blk = blk0 + row / s.Hkv;
  const int32_t n = bsel * blk + self;  // <= 256 kSelNT (host-checked)
  const int pr = (blk - blk0) & 15;     // the block's row in the score product
  const int32_t ntr = (n + 255) >> 8;   // 256-candidate tiles of the row: thread t owns tile t
  __shared__ uint32_t l_key[kHitCap];  // hit keys in candidate order (tile t's at toff[t])
  __shared__ uint32_t hc[4096];
  __shared__ uint32_t sel[NT * 8];  // selection bitmap, words [8 t, 8 t + 8) = tile t
  __shared__ uint32_t toff[NT], ovf[NT];
  __shared__ uint32_t red[NW];
  __shared__ uint32_t s_novf, s_mode, s_pre, s_need, s_thr, s_neq, s_bin, s_bef;
  uint32_t* const tie = l_key;  // all-candidate path: tie bitmap over the list arrays
#pragma unroll
  for (int e = 0; e < 8; ++e) sel[8 * t + e] = 0u;
  if (t == 0) {
    s_novf = 0u;
    s_mode = kSearchM;
    s_pre = 0u;
    s_need = (uint32_t)k;
    s_thr = 0u;
    s_neq = 0u;
  }
  for (int i = t; i < 4096; i += NT) hc[i] = 0u;  // level-1 counts, added while the list is built
  uint32_t w[8];
  uint32_t cnt = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = 0u;
  if (t < ntr) {
    const uint4* bp = reinterpret_cast<const uint4*>(bits + ((int64_t)row * tpr + t) * 8);
    const uint4 a = bp[0], b = bp[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) cnt += (uint32_t)__popc(w[e]);
  }
  // the first 32 stored keys of the tile, in flight across the scan
  uint4 sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sv[j] = make_uint4(0u, 0u, 0u, 0u);
  const uint4* slp = reinterpret_cast<const uint4*>(slots + ((int64_t)row * tpr + (t < ntr ? t : 0)) * kSlotCap);
  if (t < ntr && cnt != 0u && cnt <= (uint32_t)kSlotCap) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = slp[j];
  }
  uint32_t H;
  const uint32_t off = sel_scan(cnt, red, H);  // (its barriers publish the set-up above)
  const bool take_all = k >= n;
  const bool fast = !take_all && H >= (uint32_t)k && H <= (uint32_t)kHitCap;
  const bf16x8_t qa = split_query(qcb + ((int64_t)blk * s.Hkv + g) * kRank, lane, col == pr);
  // keys of the row's candidates recomputed, tile by tile over the waves:
  // fn(candidate, key) in the lanes that hold the block's row
  auto for_all_keys = [&](auto&& fn) {
    for (int32_t th = wave; th < 2 * ntr; th += NW) {  // half tiles of 128 candidates
      f32x4_t acc[8];
      score_tiles<8>(kidx, pt, s, g, 128 * th, n, qa, lane, acc);
      if (lg == (pr >> 2)) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int32_t c = 128 * th + 16 * u + col;
          const float v = (pr & 3) == 0 ? acc[u][0] : ((pr & 3) == 1 ? acc[u][1] : ((pr & 3) == 2 ? acc[u][2] : acc[u][3]));
          if (c < n) fn(c, score_key(v));
        }
      }
    }
  };
  if (fast) {
    // ---- the hit list, in candidate order ----
    if (t < ntr) {
      toff[t] = off;
      const bool stored = cnt <= (uint32_t)kSlotCap;
      if (stored) {  // the stored keys (the first 32 already loaded)
        auto put = [&](uint32_t e, uint32_t key) {
          if (e < cnt) {
            l_key[off + e] = key;
            atomicAdd(&hc[key >> 20], 1u);
          }
        };
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          put(4u * j, sv[j].x);
          put(4u * j + 1, sv[j].y);
          put(4u * j + 2, sv[j].z);
          put(4u * j + 3, sv[j].w);
        }
        for (uint32_t e0 = 32u; e0 < cnt; e0 += 32u) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = slp[e0 / 4u + j];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            put(e0 + 4u * j, sv[j].x);
            put(e0 + 4u * j + 1, sv[j].y);
            put(e0 + 4u * j + 2, sv[j].z);
            put(e0 + 4u * j + 3, sv[j].w);
          }
        }
      }
      if (!stored) ovf[atomicAdd(&s_novf, 1u)] = (uint32_t)t;
    }
    __syncthreads();
    // tiles with more hits than stored keys: recompute their keys
    for (uint32_t o = (uint32_t)wave; o < s_novf; o += NW) {
      const int32_t tt = (int32_t)ovf[o];
      const uint4* bp = reinterpret_cast<const uint4*>(bits + ((int64_t)row * tpr + tt) * 8);
      const uint4 a = bp[0], b = bp[1];
      const uint32_t tw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      for (int hf = 0; hf < 2; ++hf) {
      f32x4_t acc[8];
      score_tiles<8>(kidx, pt, s, g, 256 * tt + 128 * hf, n, qa, lane, acc);
      if (lg == (pr >> 2)) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = 128 * hf + 16 * u + col;  // candidate within the tile
          if ((tw[q >> 5] >> (q & 31)) & 1u) {
            uint32_t rank = (uint32_t)__popc(tw[q >> 5] & ((1u << (q & 31)) - 1u));
#pragma unroll
            for (int wi = 0; wi < 8; ++wi) rank += wi < (q >> 5) ? (uint32_t)__popc(tw[wi]) : 0u;
            const float v = (pr & 3) == 0 ? acc[u][0] : ((pr & 3) == 1 ? acc[u][1] : ((pr & 3) == 2 ? acc[u][2] : acc[u][3]));
            const uint32_t key = score_key(v);
            l_key[toff[tt] + rank] = key;
            atomicAdd(&hc[key >> 20], 1u);
          }
        }
      }
      }
    }
    __syncthreads();
  }
  // ---- radix levels (12 + 12 + 8 bits, counts from the top) ----
  if (!take_all) {
    for (int level = 1; level <= 3; ++level) {
      if (s_mode != kSearchM) break;  // block-uniform (read after a barrier)
      const int NB = level == 3 ? 256 : 4096;
      const uint32_t pre = s_pre;
      const bool have = fast && level == 1;  // the list build made the level-1 counts
      if (!have) {
        for (int i = t; i < NB; i += NT) hc[i] = 0u;
        __syncthreads();
      }
      auto add = [&](int32_t, uint32_t key) {
        if (level == 1) atomicAdd(&hc[key >> 20], 1u);
        else if (level == 2) { if ((key >> 20) == pre) atomicAdd(&hc[(key >> 8) & 0xfffu], 1u); }
        else if ((key >> 8) == pre) atomicAdd(&hc[key & 0xffu], 1u);
      };
      if (!have) {
        if (fast) {
          for (uint32_t j = (uint32_t)t; j < H; j += NT) add(0, l_key[j]);
        } else {
          for_all_keys(add);
        }
        __syncthreads();
      }
      top_bin(hc, NB, s_need, red, &s_bin, &s_bef);
      if (t == 0) {
        const uint32_t bin = s_bin;
        if (bin == 0xffffffffu) {  // fewer candidates than k: cannot happen (k < n), take all
          s_mode = kGEM;
          s_thr = 0u;
        } else {
          const uint32_t np = level == 1 ? bin : (level == 2 ? ((pre << 12) | bin) : ((pre << 8) | bin));
          const uint32_t floor_key = level == 1 ? (np << 20) : (level == 2 ? (np << 8) : np);
          const uint32_t nd = s_need - s_bef;
          if (nd == hc[bin]) {
            s_mode = kGEM;
            s_thr = floor_key;
          } else if (level < 3) {
            s_pre = np;
            s_need = nd;
          } else {
            s_mode = kTiesM;
            s_thr = floor_key;
            s_neq = nd;
          }
        }
      }
      __syncthreads();
    }
    // ---- marking ----
    const uint32_t mode = s_mode, thr = s_thr, neq = s_neq;
    if (fast) {
      // thread t walks its tile's hits in candidate order (list positions
      // off, off + 1, ...) and sets its own selection words
      uint32_t neq_t = 0u;
      {
        uint32_t e = off;
#pragma unroll
        for (int wi = 0; wi < 8; ++wi) {
          uint32_t ww = w[wi], m = 0u;
          while (ww != 0u) {
            const uint32_t bit = ww & (0u - ww);
            ww &= ww - 1u;
            const uint32_t key = l_key[e++];
            if (key > thr || (mode == kGEM && key == thr)) m |= bit;
            neq_t += key == thr ? 1u : 0u;
          }
          sel[8 * t + wi] |= m;
        }
      }
      if (mode == kTiesM) {  // the neq lowest-index keys equal to thr
        uint32_t tot;
        const uint32_t before = sel_scan(neq_t, red, tot);
        uint32_t left = before < neq ? neq - before : 0u;
        uint32_t e = off;
#pragma unroll
        for (int wi = 0; wi < 8; ++wi) {
          uint32_t ww = w[wi], m = 0u;
          while (ww != 0u) {
            const uint32_t bit = ww & (0u - ww);
            ww &= ww - 1u;
            if (l_key[e++] == thr && left != 0u) {
              m |= bit;
              --left;
            }
          }
          sel[8 * t + wi] |= m;
        }
      }
    } else {
      if (mode == kTiesM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tie[8 * t + e] = 0u;
      }
      __syncthreads();
      for_all_keys([&](int32_t c, uint32_t key) {
        if (key > thr || (mode == kGEM && key == thr)) atomicOr(&sel[c >> 5], 1u << (c & 31));
        else if (mode == kTiesM && key == thr) atomicOr(&tie[c >> 5], 1u << (c & 31));
      });
      __syncthreads();
      if (mode == kTiesM) {
        uint32_t tw[8], c = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tw[e] = tie[8 * t + e];
          c += (uint32_t)__popc(tw[e]);
        }
        uint32_t tot;
        const uint32_t before = sel_scan(c, red, tot);
        uint32_t left = before < neq ? neq - before : 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t b = tw[e], keep = 0u;
          while (b != 0u && left != 0u) {
            keep |= b & (0u - b);
            b &= b - 1u;
            --left;
          }
          sel[8 * t + e] |= keep;
        }
      }
    }
    __syncthreads();
  }
  // ---- ordered compaction: thread t owns candidates [256 t, 256 t + 256) ----
  uint32_t sw[8], c = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int32_t lo = 256 * t + 32 * e;
    uint32_t m = 0u;
    if (lo < n) {
      const uint32_t vm = n - lo >= 32 ? ~0u : ((1u << (n - lo)) - 1u);
      const int32_t ws = n - n_window;  // always-kept window [n - n_window, n)
      uint32_t fm = 0u;
      if (ws < lo + 32) fm = ws <= lo ? ~0u : (~0u << (ws - lo));
      m = ((take_all ? ~0u : sel[8 * t + e]) | fm) & vm;
    }
    sw[e] = m;
    c += (uint32_t)__popc(m);
  }
  uint32_t total;
  uint32_t rank = sel_scan(c, red, total);
  // every word's mask and output offset to LDS (the offsets over hc), then
  // word j written by thread j mod NT: a short dense row spreads over all
  // threads instead of the few that own its words
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sel[8 * t + e] = sw[e];
    hc[8 * t + e] = rank;
    rank += (uint32_t)__popc(sw[e]);
  }
  __syncthreads();
  int32_t* out = idx_out + (int64_t)row * cap;
  const uint32_t T = total < (uint32_t)cap ? total : (uint32_t)cap;
  for (int32_t j = t; j < ((n + 31) >> 5); j += NT) {
    uint32_t b = sel[j], o = hc[j];
    while (b != 0u) {
      const int jj = __ffs(b) - 1;
      b &= b - 1u;
      if (o < (uint32_t)cap) out[o] = 32 * j + jj;
      ++o;
    }
  }
  for (int64_t o = (int64_t)T + t; o < cap; o += NT) out[o] = -1;
  if (t == 0) count_out[row] = (int32_t)T;
}

// Selection plan: rows of query blocks (bsel = 64) or of queries (bsel = 1)
// are scored and selected a slab at a time.
struct PrefillSelPlan {
  int32_t nblk;      // query blocks (or queries)
  int64_t slab;      // blocks per slab
  int32_t self;      // the own token is a candidate (per query)
  int64_t ldx;       // score row stride (candidates of the last row)
  int32_t nparts;    // per-head passes: wave partials per row
  size_t off_lo, off_x, off_part, off_lse, off_sel, total;
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
  p.off_lo = off;  // sampled top-k thresholds of every row
  if (!probs) off += align_up((size_t)p.nblk * s.Hkv * sizeof(uint32_t), 256);
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
  // every row's sampled threshold when the slabs may take the hit path
  uint32_t* hit_lo = (bf && !probs && k <= kHitMaxK) ? (uint32_t*)(base + P.off_lo) : nullptr;
  if (probs) {
    dim3 g1(n_tokens, s.Hkv);
    if (bf) k_prefill_qh<bf16_raw><<<g1, 256, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)w_q,
                                                      s.Hq, s.Hkv, s.D, s_idx, qv);
    else k_prefill_qh<float><<<g1, 256, 0, st>>>((const float*)q, (const float*)w_q, s.Hq, s.Hkv,
                                                 s.D, s_idx, qv);
  } else {
    dim3 g1(P.nblk, s.Hkv);
    if (bf) k_prefill_qc<bf16_raw><<<g1, kQcNT, 0, st>>>((const bf16_raw*)q, (const bf16_raw*)w_q,
                                                        n_tokens, s.Hq, s.Hkv, s.D, b_sel, s_idx, qv);
    else k_prefill_qc<float><<<g1, kQcNT, 0, st>>>((const float*)q, (const float*)w_q, n_tokens, s.Hq,
                                                   s.Hkv, s.D, b_sel, s_idx, qv);
    // sampled thresholds of every row (every stride-th 16-candidate tile)
    if (hit_lo != nullptr)
      k_pf_thresh<<<(unsigned)(((P.nblk + 1) / 2) * s.Hkv), kSelNT, 0, st>>>((const bf16_raw*)kidx_pool,
                                                                            pg.page_table, qv, P.nblk, b_sel,
                                                                            P.self, s, k, k <= 1024 ? 16 : 12,
                                                                            hit_lo);
  }
  for (int b0 = 0; b0 < P.nblk; b0 += (int)P.slab) {
    const int b1 = b0 + (int)P.slab < P.nblk ? b0 + (int)P.slab : P.nblk;
    const int64_t cand_hi = (int64_t)b_sel * (b1 - 1) + P.self;  // candidates of the last row
    const int64_t ldx = cand_hi > 0 ? cand_hi : 1;
    // logit scores go to the selection as 16-bit keys (exact scores of the
    // threshold bin are recomputed there) when its one-block rows take them
    const bool key16 = !probs && ldx <= kSelectRowMax;
    // bf16 indexer keys and k <= kHitMaxK: sampled thresholds, hit bitmaps
    // from the matrix cores and the exact top k over the hits
    if (key16 && hit_lo != nullptr && ldx >= 256) {
      const int64_t rows = (int64_t)(b1 - b0) * s.Hkv;
      const int32_t tpr = (int32_t)((ldx + 255) / 256);
      const size_t need = (size_t)rows * tpr * (8 + kSlotCap) * 4;
      if (need > (size_t)P.slab * s.Hkv * (size_t)P.ldx * sizeof(float)) return hipErrorInvalidValue;
      const uint32_t* lo = hit_lo + (int64_t)b0 * s.Hkv;
      uint32_t* bits = (uint32_t*)xs;
      uint32_t* slots = bits + (size_t)rows * tpr * 8;
      dim3 gh((unsigned)tpr, (unsigned)((b1 - b0 + 16 * kHitWaves - 1) / (16 * kHitWaves)), (unsigned)s.Hkv);
      k_pf_hits<<<gh, 64 * kHitWaves, 0, st>>>((const bf16_raw*)kidx_pool, pg.page_table, qv, lo, b0, b1, b_sel,
                                    P.self, s, tpr, bits, slots);
      k_pf_select<<<(unsigned)rows, kSelNT, 0, st>>>((const bf16_raw*)kidx_pool, pg.page_table, qv, bits,
                                                     slots, b0, b_sel, P.self, s, tpr, k, P.self,
                                                     idx + (int64_t)b0 * s.Hkv * cap,
                                                     count + (int64_t)b0 * s.Hkv, cap);
      continue;
    }
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
