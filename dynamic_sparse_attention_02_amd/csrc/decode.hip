// Split-KV sparse decode: exact softmax attention of each query head over the
// listed support of its key/value group ("Oracle-Guided Sparse Prefill",
// section 2.1: attention recomputed with the original q, k, v restricted to
// the support; one support per group shared by its query heads).
//
// The support lists are cut into chunks of a multiple of 64 listed tokens,
// one size for all rows, chosen at run time from the total list length; a
// persistent grid of blocks takes the (row, chunk) items in turn.  A block
// gathers the K and V rows of 64 tokens at a time
// (16-byte loads, 16 lanes per 256-byte row, staged in LDS), computes the
// logits of the group's heads with one lane per token (bf16 pairs through
// v_dot2_f32_bf16, fp32 accumulate), keeps an online softmax per head, and
// accumulates P.V with one lane per head dimension.  The next tile's rows are
// loaded into registers, and the pool addresses of the tile after it resolved
// (list entry -> page table -> row), while the current tile is processed.  A second kernel
// merges the per-chunk (max, sum, output) partials in chunk order.
//
// Bound: HBM bandwidth of the gathered rows (512 B per listed token for
// d = 128 bf16).  No matrix cores: the per-token work is a G x d by d x 1
// product, too thin to fill an MFMA tile.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kTile = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Work decomposition.  Every row's list is cut into chunks of C = 64 * tpc
// listed tokens; tpc is the same for all rows and follows from the total
// number of listed tiles and the (persistent) grid size, so that the chunks
// spread evenly over the blocks.  Items (row, chunk) are numbered row by row
// and block b takes items b, b + grid, ...
constexpr int kMaxRowsLds = 4096;  // rows whose chunk prefix fits in LDS

__device__ __forceinline__ int32_t row_count(const int32_t* count, int row, int32_t cap) {
  int32_t n = count[row];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// Tiles per chunk from the total listed tiles (same result in every block).
__device__ __forceinline__ int32_t plan_tpc(int64_t total_tiles, int32_t grid) {
  int64_t t = (total_tiles + 2 * (int64_t)grid - 1) / (2 * (int64_t)grid);
  return t < 1 ? 1 : (t > 16 ? 16 : (int32_t)t);
}

template <typename T, int D, int G>
struct DecodeCfg {
  static constexpr int NW = G < 4 ? G : 4;        // waves per block
  static constexpr int HPW = G / NW;              // heads per wave
  static constexpr int NT = NW * kWave;           // threads per block
  static constexpr int ROWB = D * (int)sizeof(T); // bytes per K/V row
  static constexpr int CPR = ROWB / 16;           // 16-byte pieces per row
  static constexpr int PITCH = ROWB + 16;         // LDS row pitch (bank spread)
  static constexpr int LPT = kTile * CPR / NT;    // pieces per thread per tensor
  static constexpr int DPL = D / kWave;           // head dims per lane in P.V
};

template <typename T, int D, int G>
__global__ void __launch_bounds__((G < 4 ? G : 4) * 64)
k_decode_split(const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
               const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
               const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int32_t cap,
               Shape s, float s_att, int32_t nchunk_max,
               float* __restrict__ part_ml, float* __restrict__ part_o) {
  using C = DecodeCfg<T, D, G>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = s.B * s.Hkv;

  __shared__ __align__(16) char Ks[kTile * C::PITCH];
  __shared__ __align__(16) char Vs[kTile * C::PITCH];
  __shared__ __align__(16) T Qs[G][D];
  __shared__ __align__(16) float Ps[G][kTile];
  __shared__ int32_t prefix[kMaxRowsLds + 1];
  __shared__ int64_t s_tiles;
  __shared__ int32_t s_red[4];

  // ---- plan: tiles per chunk and the item prefix over rows ----
  if (tid == 0) s_tiles = 0;
  __syncthreads();
  int64_t my_tiles = 0;
  for (int r = tid; r < rows; r += C::NT) my_tiles += (row_count(count, r, cap) + kTile - 1) / kTile;
  atomicAdd((unsigned long long*)&s_tiles, (unsigned long long)my_tiles);
  __syncthreads();
  const int32_t tpc = plan_tpc(s_tiles, gridDim.x);
  const int32_t csize = kTile * tpc;
  // prefix[r] = items before row r (sequential scan by wave 0, rows <= kMaxRowsLds)
  if (wave == 0) {
    int32_t carry = 0;
    for (int r0 = 0; r0 < rows; r0 += 64) {
      const int r = r0 + lane;
      const int32_t c = r < rows ? (row_count(count, r, cap) + csize - 1) / csize : 0;
      const int32_t inc = (int32_t)wave_incl_scan((uint32_t)c);
      if (r < rows) prefix[r] = carry + inc - c;
      carry += (int32_t)lane_u32((uint32_t)inc, 63);
    }
    if (lane == 0) prefix[rows] = carry;
  }
  __syncthreads();
  const int32_t n_items = prefix[rows];
  const int64_t head_stride = (int64_t)kPage * D;
  const int64_t page_stride = (int64_t)s.Hkv * head_stride;

  for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    // row of the item: last r with prefix[r] <= item
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int row = lo;
    const int32_t c = item - prefix[row];
    const int b = row / s.Hkv, g = row % s.Hkv;
    const int32_t n = row_count(count, row, cap);
    const int32_t t0 = c * csize;
    const int32_t t1 = min(n, t0 + csize);
    const int32_t L = clamp_len(seq_lens[b], s.max_len);
    const int32_t* pt = page_table + (int64_t)b * s.max_pages;
    const int32_t* list = idx + (int64_t)row * cap;

    __syncthreads();  // previous item done with Qs
    for (int i = tid; i < G * D; i += C::NT)
      Qs[i / D][i % D] = q[((int64_t)b * s.Hq + g * G) * D + i];

    float m_run[C::HPW], l_run[C::HPW], acc[C::HPW][C::DPL];
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < C::DPL; ++e) acc[hh][e] = 0.f;
    }
    // pool element offsets of the rows this thread moves in a tile
    int64_t ridn[C::LPT];
    auto load_rows = [&](int32_t ts, int64_t (&rid)[C::LPT]) {
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        const int r = (i * C::NT + tid) / C::CPR;
        rid[i] = -1;
        if (ts + r < t1) {
          int32_t j = list[ts + r];
          j = j < 0 ? 0 : (j >= L ? (L > 0 ? L - 1 : 0) : j);
          const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
          rid[i] = page * page_stride + g * head_stride + (int64_t)(j & 63) * D;
        }
      }
    };
    uint4 kr[C::LPT], vr[C::LPT];
    auto load_kv = [&](const int64_t (&rid)[C::LPT]) {
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        const int col = (i * C::NT + tid) % C::CPR;
        if (rid[i] >= 0) {
          kr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(k_pool + rid[i]) + col * 16);
          vr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(v_pool + rid[i]) + col * 16);
        } else {
          kr[i] = make_uint4(0, 0, 0, 0);
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    load_rows(t0, ridn);
    load_kv(ridn);
    if (t0 + kTile < t1) load_rows(t0 + kTile, ridn);
    for (int32_t ts = t0; ts < t1; ts += kTile) {
      const int32_t nt = min(kTile, t1 - ts);
      __syncthreads();  // previous tile fully consumed (and Qs written)
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        const int pc = i * C::NT + tid;
        const int r = pc / C::CPR, col = pc % C::CPR;
        *reinterpret_cast<uint4*>(Ks + r * C::PITCH + col * 16) = kr[i];
        *reinterpret_cast<uint4*>(Vs + r * C::PITCH + col * 16) = vr[i];
      }
      __syncthreads();
      if (ts + kTile < t1) {  // next tile's rows in flight, and the addresses after it
        load_kv(ridn);
        if (ts + 2 * kTile < t1) load_rows(ts + 2 * kTile, ridn);
      }

      // logits: lane = token of the tile
      float sc[C::HPW];
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) sc[hh] = 0.f;
      const char* krow = Ks + lane * C::PITCH;
#pragma unroll 4
      for (int pc = 0; pc < C::CPR; ++pc) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + pc * 16);
#pragma unroll
        for (int hh = 0; hh < C::HPW; ++hh) {
          const int h = wave * C::HPW + hh;
          if constexpr (sizeof(T) == 2) {
            const uint4 qv = *reinterpret_cast<const uint4*>(&Qs[h][pc * 8]);
            float a = sc[hh];
            a = dot2_bf16(kv.x, qv.x, a);
            a = dot2_bf16(kv.y, qv.y, a);
            a = dot2_bf16(kv.z, qv.z, a);
            a = dot2_bf16(kv.w, qv.w, a);
            sc[hh] = a;
          } else {
            const float4 qv = *reinterpret_cast<const float4*>(&Qs[h][pc * 4]);
            float a = sc[hh];
            a = fmaf(__uint_as_float(kv.x), qv.x, a);
            a = fmaf(__uint_as_float(kv.y), qv.y, a);
            a = fmaf(__uint_as_float(kv.z), qv.z, a);
            a = fmaf(__uint_as_float(kv.w), qv.w, a);
            sc[hh] = a;
          }
        }
      }
      float alpha[C::HPW];
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) {
        const float sv = lane < nt ? sc[hh] * s_att : -INFINITY;
        const float mt = wave_max(sv);
        const float m_new = fmaxf(m_run[hh], mt);
        const float p = lane < nt ? __expf(sv - m_new) : 0.f;
        const float lt = wave_sum(p);
        alpha[hh] = __expf(m_run[hh] - m_new);
        l_run[hh] = l_run[hh] * alpha[hh] + lt;
        m_run[hh] = m_new;
        Ps[wave * C::HPW + hh][lane] = p;
      }
      __syncthreads();
      // P.V: lane owns DPL consecutive dims of the wave's heads
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh)
#pragma unroll
        for (int e = 0; e < C::DPL; ++e) acc[hh][e] *= alpha[hh];
      for (int t = 0; t < kTile; t += 4) {
        float4 pv[C::HPW];
#pragma unroll
        for (int hh = 0; hh < C::HPW; ++hh)
          pv[hh] = *reinterpret_cast<const float4*>(&Ps[wave * C::HPW + hh][t]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float vv[C::DPL];
          const char* vrow = Vs + (t + u) * C::PITCH;
          if constexpr (sizeof(T) == 2) {
            if constexpr (C::DPL == 2) {
              const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + lane * 4);
              vv[0] = __uint_as_float(w << 16);
              vv[1] = __uint_as_float(w & 0xffff0000u);
            } else {
              const uint16_t w = *reinterpret_cast<const uint16_t*>(vrow + lane * 2);
              vv[0] = __uint_as_float((uint32_t)w << 16);
            }
          } else {
#pragma unroll
            for (int e = 0; e < C::DPL; ++e)
              vv[e] = *reinterpret_cast<const float*>(vrow + (lane * C::DPL + e) * 4);
          }
#pragma unroll
          for (int hh = 0; hh < C::HPW; ++hh) {
            const float p = u == 0 ? pv[hh].x : (u == 1 ? pv[hh].y : (u == 2 ? pv[hh].z : pv[hh].w));
#pragma unroll
            for (int e = 0; e < C::DPL; ++e) acc[hh][e] = fmaf(p, vv[e], acc[hh][e]);
          }
        }
      }
    }
    // partials of this chunk
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) {
      const int h = g * G + wave * C::HPW + hh;
      const int64_t pi = ((int64_t)b * s.Hq + h) * nchunk_max + c;
      if (lane == 0) {
        part_ml[pi * 2] = m_run[hh];
        part_ml[pi * 2 + 1] = l_run[hh];
      }
#pragma unroll
      for (int e = 0; e < C::DPL; ++e) part_o[pi * D + lane * C::DPL + e] = acc[hh][e];
    }
  }
}

// Merge the chunk partials of one (b, h): maximum and normaliser by a block
// reduction, then every output dimension summed over the chunks by
// 256 / D thread groups with independent (unrolled) loads; all orders fixed.
constexpr int kCombThreads = 256;
constexpr int kMaxChunkW = 4096;  // chunk weights kept in LDS

template <typename TO>
__global__ void __launch_bounds__(kCombThreads)
k_decode_combine(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                 const int32_t* __restrict__ count, int32_t cap, Shape s, int32_t split_grid,
                 int32_t nchunk_max, TO* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = s.Hq / s.Hkv;
  const int row = b * s.Hkv + h / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = s.B * s.Hkv;
  __shared__ int64_t s_tiles;
  if (tid == 0) s_tiles = 0;
  __syncthreads();
  int64_t my_tiles = 0;
  for (int r = tid; r < rows; r += kCombThreads) my_tiles += (row_count(count, r, cap) + kTile - 1) / kTile;
  atomicAdd((unsigned long long*)&s_tiles, (unsigned long long)my_tiles);
  __syncthreads();
  const int32_t csize = kTile * plan_tpc(s_tiles, split_grid);
  const int32_t n = row_count(count, row, cap);
  const int32_t nch = (n + csize - 1) / csize;
  const int64_t base = ((int64_t)b * s.Hq + h) * nchunk_max;
  __shared__ float wred[4];
  __shared__ float wts[kMaxChunkW];
  __shared__ float ored[kCombThreads];
  float m = -INFINITY;
  for (int c = tid; c < nch; c += kCombThreads) m = fmaxf(m, part_ml[(base + c) * 2]);
  m = wave_max(m);
  if (lane == 0) wred[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  __syncthreads();
  float l = 0.f;
  for (int c = tid; c < nch; c += kCombThreads) {
    const float wc = __expf(part_ml[(base + c) * 2] - M);
    if (c < kMaxChunkW) wts[c] = wc;
    l += part_ml[(base + c) * 2 + 1] * wc;
  }
  l = wave_sum(l);
  if (lane == 0) wred[wave] = l;
  __syncthreads();
  const float lsum = (wred[0] + wred[1]) + (wred[2] + wred[3]);
  const int D = s.D;
  const int NG = kCombThreads / D;
  const int d = tid % D, gi = tid / D;
  float o = 0.f;
  if (nch <= kMaxChunkW) {
#pragma unroll 8
    for (int c = gi; c < nch; c += NG) o = fmaf(wts[c], part_o[(base + c) * D + d], o);
  } else {
    for (int c = gi; c < nch; c += NG)
      o = fmaf(__expf(part_ml[(base + c) * 2] - M), part_o[(base + c) * D + d], o);
  }
  ored[tid] = o;
  __syncthreads();
  if (gi == 0) {
    float t = 0.f;
    for (int k = 0; k < NG; ++k) t += ored[k * D + d];
    out[((int64_t)b * s.Hq + h) * D + d] = from_f32<TO>(nch ? t / lsum : 0.f);
  }
  if (lse && tid == 0) lse[(int64_t)b * s.Hq + h] = nch ? M + logf(lsum) : -INFINITY;
}

// Persistent grid of the split kernel: blocks resident on the chip.
int split_grid(int nchunk_max, int rows) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const long long most = (long long)nchunk_max * rows;
  const long long g = 3LL * cus;
  return (int)(most < g ? (most < 1 ? 1 : most) : g);
}

template <typename T, int D>
hipError_t launch_t(const Shape& s, const sa_pages& pg, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* idx, const int32_t* count, int32_t cap,
                    float s_att, void* out, sa_dtype out_dt, float* lse, void* ws,
                    hipStream_t st) {
  const int32_t nchunk_max = (cap + kTile - 1) / kTile;
  float* part_ml = (float*)ws;
  float* part_o = part_ml + align_up((size_t)s.B * s.Hq * nchunk_max * 2, 64);
  const int gx = split_grid(nchunk_max, s.B * s.Hkv);
  dim3 grid(gx);
  const int G = s.Hq / s.Hkv;
#define SA_DS(GG)                                                                        \
  k_decode_split<T, D, GG><<<grid, DecodeCfg<T, D, GG>::NT, 0, st>>>(                     \
      (const T*)q, (const T*)k_pool, (const T*)v_pool, pg.page_table, pg.seq_lens, idx,   \
      count, cap, s, s_att, nchunk_max, part_ml, part_o)
  switch (G) {
    case 1: SA_DS(1); break;
    case 2: SA_DS(2); break;
    case 4: SA_DS(4); break;
    case 8: SA_DS(8); break;
    default: SA_DS(16); break;
  }
#undef SA_DS
  dim3 g2(s.Hq, s.B);
  if (out_dt == SA_BF16)
    k_decode_combine<bf16_raw><<<g2, kCombThreads, 0, st>>>(part_ml, part_o, count, cap, s,
                                                            gx, nchunk_max, (bf16_raw*)out, lse);
  else
    k_decode_combine<float><<<g2, kCombThreads, 0, st>>>(part_ml, part_o, count, cap, s, gx,
                                                         nchunk_max, (float*)out, lse);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(const Shape& s, int32_t cap) {
  const size_t nchunk_max = (size_t)(cap + kTile - 1) / kTile;
  const size_t n_ml = align_up((size_t)s.B * s.Hq * nchunk_max * 2, 64);
  return (n_ml + (size_t)s.B * s.Hq * nchunk_max * s.D) * sizeof(float);
}

hipError_t launch_sparse_decode(const Shape& s, const sa_pages& pg, const void* q,
                                const void* k_pool, const void* v_pool, sa_dtype dt,
                                const int32_t* idx, const int32_t* count, int32_t cap,
                                float s_att, void* out, sa_dtype out_dt, float* lse,
                                void* ws, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  if (dt == SA_BF16) {
    if (s.D == 128)
      return launch_t<bf16_raw, 128>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, st);
    return launch_t<bf16_raw, 64>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, st);
  }
  if (s.D == 128)
    return launch_t<float, 128>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, st);
  return launch_t<float, 64>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, st);
}

}  // namespace sa
