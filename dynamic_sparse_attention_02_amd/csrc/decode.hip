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
// accumulates P.V with one lane per head dimension; for bf16 and groups of 4
// to 16 heads the tile runs on the matrix cores instead (each wave takes 16
// of its tokens for all the group's heads, padded to 16: S^T = K Q^T and
// O^T += V^T P^T, P split into a bf16 high part and the rounding of the
// rest, the four waves' softmax states merged per chunk), which leaves the
// VALU most of the issue slots the gathers need.  The next tile's rows are
// loaded into registers, and the pool addresses of the tile after it resolved
// (list entry -> page table -> row), while the current tile is processed.  A second kernel
// merges the per-chunk (max, sum, output) partials in chunk order.
//
// Bound: HBM bandwidth of the gathered rows (512 B per listed token for
// d = 128 bf16).
#include <map>
#include <mutex>
#include <utility>

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
constexpr int kMaxRowsLds = 4096;    // rows whose chunk prefix fits in LDS
constexpr int kSmallRowsLds = 256;   // a smaller prefix leaves LDS for a fourth workgroup per CU

__device__ __forceinline__ int32_t row_count(const int32_t* count, int row, int32_t cap) {
  int32_t n = count[row];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// Tiles per chunk from the total listed tiles (same result in every block).
// At most 16 tiles per chunk (4 with the residual linear attention, whose
// larger LDS footprint leaves no room for a longer row list); a chunk starts
// with one dependent round trip for its rows, but longer chunks than this
// balance the blocks worse.
template <bool RLA>
constexpr int max_tpc() { return RLA ? 4 : 16; }
template <bool RLA>
__device__ __forceinline__ int32_t plan_tpc(int64_t total_tiles, int32_t grid) {
  int64_t t = (total_tiles + 2 * (int64_t)grid - 1) / (2 * (int64_t)grid);
  return t < 1 ? 1 : (t > max_tpc<RLA>() ? max_tpc<RLA>() : (int32_t)t);
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

// RLA: also the residual linear attention terms of the listed tokens
// ("SPLA", section 2.2): with phi = exp elementwise, per head
//   w_j = phi(q) . phi(k_j),  num += w_j v_j,  den += w_j
// from the K/V rows already staged for the exact attention.
constexpr int kPhiPitch = 4;  // extra floats per phi(K) row in LDS (bank spread)

template <typename T, int D, int G, bool RLA, int RMAX>
__global__ void __launch_bounds__((G < 4 ? G : 4) * 64)
k_decode_split(const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
               const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
               const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int32_t cap,
               Shape s, float s_att, int32_t nchunk_max,
               float* __restrict__ part_ml, float* __restrict__ part_o,
               float* __restrict__ part_rnum, float* __restrict__ part_rden) {
  using C = DecodeCfg<T, D, G>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = s.B * s.Hkv;

  __shared__ __align__(16) char Ks[kTile * C::PITCH];
  __shared__ __align__(16) char Vs[kTile * C::PITCH];
  __shared__ __align__(16) T Qs[G][D];
  __shared__ __align__(16) float Ps[G][kTile];
  __shared__ __align__(16) float PhiK[RLA ? kTile : 1][RLA ? D + kPhiPitch : 1];
  __shared__ __align__(16) float PhiQ[RLA ? G : 1][RLA ? D : 1];
  __shared__ __align__(16) float Ws[RLA ? G : 1][RLA ? kTile : 1];
  __shared__ int32_t prefix[RMAX + 1];
  __shared__ uint32_t s_rid[max_tpc<RLA>() * kTile];  // pool rows of the item's listed tokens
  __shared__ int64_t s_tiles;
  __shared__ int32_t s_red[4];

  // ---- plan: tiles per chunk and the item prefix over rows ----
  if (tid == 0) s_tiles = 0;
  __syncthreads();
  int64_t my_tiles = 0;
  for (int r = tid; r < rows; r += C::NT) my_tiles += (row_count(count, r, cap) + kTile - 1) / kTile;
  atomicAdd((unsigned long long*)&s_tiles, (unsigned long long)my_tiles);
  __syncthreads();
  const int32_t tpc = plan_tpc<RLA>(s_tiles, gridDim.x);
  const int32_t csize = kTile * tpc;
  // prefix[r] = items before row r (sequential scan by wave 0, rows <= RMAX)
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

    __syncthreads();  // previous item done with Qs and the row list
    // pool row of every listed token of the chunk (page << 6 | slot)
    for (int32_t e = tid; e < t1 - t0; e += C::NT) {
      int32_t j = list[t0 + e];
      j = j < 0 ? 0 : (j >= L ? (L > 0 ? L - 1 : 0) : j);
      s_rid[e] = ((uint32_t)clamp_page(pt[j >> 6], s.n_pool_pages) << 6) | (uint32_t)(j & 63);
    }
    for (int i = tid; i < G * D; i += C::NT) {
      const T qv = q[((int64_t)b * s.Hq + g * G) * D + i];
      Qs[i / D][i % D] = qv;
      if (RLA) PhiQ[i / D][i % D] = __expf(to_f32<T>(qv));
    }
    __syncthreads();  // the row list is read by every thread's gathers below
    float racc[RLA ? C::HPW : 1][RLA ? C::DPL : 1], rden[RLA ? C::HPW : 1];
    if (RLA) {
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) {
        rden[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < C::DPL; ++e) racc[hh][e] = 0.f;
      }
    }

    float m_run[C::HPW], l_run[C::HPW], acc[C::HPW][C::DPL];
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < C::DPL; ++e) acc[hh][e] = 0.f;
    }
    // Tiles of K/V rows go through registers (one vector value per buffer,
    // so they stay in registers) into LDS.  The gathers are branch-free:
    // rows past the chunk re-read its last token, whose logits are masked.
    // With two buffers (up to 8 pieces per thread) the next tile's rows and
    // the one after are in flight while a tile is computed; the addresses
    // come from the LDS row list, so no dependent load sits between a
    // prefetch and the staging that needs it.
    typedef uint32_t kvv_t __attribute__((ext_vector_type(4 * C::LPT)));
    auto gather = [&](int32_t ts, kvv_t& kr, kvv_t& vr) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        const int pc = i * C::NT + tid;
        const int r = pc / C::CPR, col = pc % C::CPR;
        const uint32_t v = s_rid[min(ts + r, t1 - 1) - t0];
        const int64_t off = (((int64_t)(v >> 6) * s.Hkv + g) * kPage + (v & 63)) * D;
        const uint4 k4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(k_pool + off) + col * 16);
        const uint4 v4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(v_pool + off) + col * 16);
        kr[4 * i] = k4.x; kr[4 * i + 1] = k4.y; kr[4 * i + 2] = k4.z; kr[4 * i + 3] = k4.w;
        vr[4 * i] = v4.x; vr[4 * i + 1] = v4.y; vr[4 * i + 2] = v4.z; vr[4 * i + 3] = v4.w;
      }
    };
    auto stage = [&](const kvv_t& kr, const kvv_t& vr) __attribute__((always_inline)) {
      __syncthreads();  // previous tile fully consumed
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        const int pc = i * C::NT + tid;
        const int r = pc / C::CPR, col = pc % C::CPR;
        const uint4 k4 = make_uint4(kr[4 * i], kr[4 * i + 1], kr[4 * i + 2], kr[4 * i + 3]);
        *reinterpret_cast<uint4*>(Ks + r * C::PITCH + col * 16) = k4;
        *reinterpret_cast<uint4*>(Vs + r * C::PITCH + col * 16) =
            make_uint4(vr[4 * i], vr[4 * i + 1], vr[4 * i + 2], vr[4 * i + 3]);
        if (RLA) {
          constexpr int EPP = 16 / (int)sizeof(T);  // elements per 16-byte piece
          const uint32_t w[4] = {k4.x, k4.y, k4.z, k4.w};
          float* dst = &PhiK[r][col * EPP];
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dst[2 * e] = __expf(__uint_as_float(w[e] << 16));
              dst[2 * e + 1] = __expf(__uint_as_float(w[e] & 0xffff0000u));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = __expf(__uint_as_float(w[e]));
          }
        }
      }
      __syncthreads();
    };
    // matrix-core tile (bf16, G in [4, 16], no residual terms): wave w takes
    // tokens [16 w, 16 w + 16); lane (hq, lg) holds tokens 16 w + 4 lg + v of
    // head hq (heads past G carry zero queries)
    constexpr bool MF = sizeof(T) == 2 && !RLA && G >= 4 && G <= 16 && C::NW == 4;
    typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
    typedef __attribute__((ext_vector_type(4))) short s16x4_t;
    typedef __attribute__((ext_vector_type(4))) float f32x4_t;
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
    constexpr int KS = D / 32, MB = D / 16;
    const int hq = lane & 15, lg = lane >> 4;
    bf16x8_t qB[MF ? KS : 1];
    f32x4_t oacc[MF ? MB : 1];
    float m_mf = -INFINITY, l_mf = 0.f;
    if constexpr (MF) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (hq < G) w = *reinterpret_cast<const uint4*>(&Qs[hq < G ? hq : 0][32 * ks + 8 * lg]);
        qB[ks] = __builtin_bit_cast(bf16x8_t, w);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    auto compute_mf = [&](int32_t ts) __attribute__((always_inline)) {
      const int32_t nt = min(kTile, t1 - ts);
      f32x4_t S = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const char* krow = Ks + (16 * wave + hq) * C::PITCH + 16 * lg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + 64 * ks);
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qB[ks], S, 0, 0, 0);
      }
      float sv[4], mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[v] = 16 * wave + 4 * lg + v < nt ? S[v] * s_att : -INFINITY;
        mt = fmaxf(mt, sv[v]);
      }
      mt = row4_max(mt);
      const float m_new = fmaxf(m_mf, mt);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __expf(m_mf - mu);  // 0 before the first valid token
      float pv[4], ls = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[v] = __expf(sv[v] - mu);
        ls += pv[v];
      }
      l_mf = l_mf * alpha + ls;
      m_mf = m_new;
      const f32x4_t pvv = f32x4_t{pv[0], pv[1], pv[2], pv[3]};
      const bf16x4_t phb = __builtin_convertvector(pvv, bf16x4_t);
      const bf16x4_t plb = __builtin_convertvector(pvv - __builtin_convertvector(phb, f32x4_t), bf16x4_t);
      const s16x4_t ph = __builtin_bit_cast(s16x4_t, phb);
      const s16x4_t pl = __builtin_bit_cast(s16x4_t, plb);
      const bool rescale = __any(alpha != 1.f);
      if (rescale) {  // (wave-uniform: a branch, not a select per accumulator)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const char* vcol = Vs + (16 * wave + 4 * lg) * C::PITCH + (16 * mb + hq) * 2;
        const uint32_t v0 = *reinterpret_cast<const uint16_t*>(vcol);
        const uint32_t v1 = *reinterpret_cast<const uint16_t*>(vcol + C::PITCH);
        const uint32_t v2 = *reinterpret_cast<const uint16_t*>(vcol + 2 * C::PITCH);
        const uint32_t v3 = *reinterpret_cast<const uint16_t*>(vcol + 3 * C::PITCH);
        const s16x4_t av = __builtin_bit_cast(s16x4_t, make_uint2(v0 | (v1 << 16), v2 | (v3 << 16)));
        oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, ph, oacc[mb], 0, 0, 0);
        oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pl, oacc[mb], 0, 0, 0);
      }
    };
    auto compute = [&](int32_t ts) __attribute__((always_inline)) {
      if constexpr (MF) {
        compute_mf(ts);
        return;
      }
      const int32_t nt = min(kTile, t1 - ts);
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
        if (RLA) {  // w = phi(q_h) . phi(k_lane)
          float wv[C::HPW];
  #pragma unroll
          for (int hh = 0; hh < C::HPW; ++hh) wv[hh] = 0.f;
          const float* prow = &PhiK[lane][0];
  #pragma unroll 4
          for (int i = 0; i < D; i += 4) {
            const float4 pk = *reinterpret_cast<const float4*>(prow + i);
  #pragma unroll
            for (int hh = 0; hh < C::HPW; ++hh) {
              const float4 pq = *reinterpret_cast<const float4*>(&PhiQ[wave * C::HPW + hh][i]);
              float a = wv[hh];
              a = fmaf(pq.x, pk.x, a);
              a = fmaf(pq.y, pk.y, a);
              a = fmaf(pq.z, pk.z, a);
              a = fmaf(pq.w, pk.w, a);
              wv[hh] = a;
            }
          }
  #pragma unroll
          for (int hh = 0; hh < C::HPW; ++hh) {
            const float w = lane < nt ? wv[hh] : 0.f;
            rden[hh] += wave_sum(w);
            Ws[wave * C::HPW + hh][lane] = w;
          }
        }
        __syncthreads();
        // P.V: lane owns DPL consecutive dims of the wave's heads
  #pragma unroll
        for (int hh = 0; hh < C::HPW; ++hh)
  #pragma unroll
          for (int e = 0; e < C::DPL; ++e) acc[hh][e] *= alpha[hh];
        for (int t = 0; t < kTile; t += 4) {
          float4 pv[C::HPW], wv4[RLA ? C::HPW : 1];
  #pragma unroll
          for (int hh = 0; hh < C::HPW; ++hh) {
            pv[hh] = *reinterpret_cast<const float4*>(&Ps[wave * C::HPW + hh][t]);
            if (RLA) wv4[hh] = *reinterpret_cast<const float4*>(&Ws[wave * C::HPW + hh][t]);
          }
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
              if (RLA) {
                const float w = u == 0 ? wv4[hh].x : (u == 1 ? wv4[hh].y : (u == 2 ? wv4[hh].z : wv4[hh].w));
  #pragma unroll
                for (int e = 0; e < C::DPL; ++e) racc[hh][e] = fmaf(w, vv[e], racc[hh][e]);
              }
            }
          }
        }
    };
    if constexpr (C::LPT <= 8) {
      kvv_t kA, vA, kB, vB;
      int32_t ts = t0;
      gather(t0, kA, vA);
      gather(t0 + kTile, kB, vB);
      for (; ts + kTile < t1; ts += 2 * kTile) {  // both tiles of the pair hold tokens
        stage(kA, vA);
        gather(ts + 2 * kTile, kA, vA);
        compute(ts);
        stage(kB, vB);
        gather(ts + 3 * kTile, kB, vB);
        compute(ts + kTile);
      }
      if (ts < t1) {  // an odd last tile
        stage(kA, vA);
        compute(ts);
      }
    } else {
      kvv_t kA, vA;
      gather(t0, kA, vA);
      for (int32_t ts = t0; ts < t1; ts += kTile) {
        stage(kA, vA);
        if (ts + kTile < t1) gather(ts + kTile, kA, vA);
        compute(ts);
      }
    }
    if constexpr (MF) {
      // merge the waves (lane (hq, lg) holds O^T[16 mb + 4 lg + v][hq]) and
      // store the chunk's partials
      static_assert(2 * D * 16 * 4 <= kTile * C::PITCH, "two waves' outputs fit one tile buffer");
      __shared__ float s_wm[4][16], s_wl[4][16];
      float lw = l_mf;
      lw += __shfl_xor(lw, 16, 64);
      lw += __shfl_xor(lw, 32, 64);
      __syncthreads();  // the tile buffers are free
      float* ob = reinterpret_cast<float*>(wave < 2 ? Ks : Vs) + (wave & 1) * D * 16;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) ob[(16 * mb + 4 * lg + v) * 16 + hq] = oacc[mb][v];
      if (lane < 16) {
        s_wm[wave][lane] = m_mf;
        s_wl[wave][lane] = lw;
      }
      __syncthreads();
      for (int e = tid; e < G * D; e += C::NT) {
        const int hl = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_wm[w][hl]);
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float wt = s_wm[w][hl] == -INFINITY ? 0.f : __expf(s_wm[w][hl] - M);
          const float* obw = reinterpret_cast<const float*>(w < 2 ? Ks : Vs) + (w & 1) * D * 16;
          lsum += s_wl[w][hl] * wt;
          osum += obw[d * 16 + hl] * wt;
        }
        const int64_t pi = ((int64_t)b * s.Hq + g * G + hl) * nchunk_max + c;
        part_o[pi * D + d] = osum;
        if (d == 0) {
          part_ml[pi * 2] = M;
          part_ml[pi * 2 + 1] = lsum;
        }
      }
      continue;
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
      if (RLA) {
        if (lane == 0) part_rden[pi] = rden[hh];
#pragma unroll
        for (int e = 0; e < C::DPL; ++e) part_rnum[pi * D + lane * C::DPL + e] = racc[hh][e];
      }
    }
  }
}

// Merge the chunk partials of one (b, h): maximum and normaliser by a block
// reduction, then every output dimension summed over the chunks by
// 256 / D thread groups with independent (unrolled) loads; all orders fixed.
constexpr int kCombThreads = 256;
constexpr int kMaxChunkW = 4096;  // chunk weights kept in LDS

// With RLA, also the residual linear attention over the unselected tokens by
// subtraction: num = phi(q)^T S_all - sum_chunks num_sel, den = phi(q) . z_all
// - sum_chunks den_sel (state [B][Hkv][D + 1][D]: rows 0 .. D-1 = S, row D = z).
template <typename TO, typename TQ, bool RLA>
__global__ void __launch_bounds__(kCombThreads)
k_decode_combine(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                 const int32_t* __restrict__ count, int32_t cap, Shape s, int32_t split_grid,
                 int32_t nchunk_max, TO* __restrict__ out, float* __restrict__ lse,
                 const TQ* __restrict__ q, const float* __restrict__ rla_state,
                 const float* __restrict__ part_rnum, const float* __restrict__ part_rden,
                 float* __restrict__ rla_num, float* __restrict__ rla_den) {
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
  const int32_t csize = kTile * plan_tpc<RLA>(s_tiles, split_grid);
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
  // output dims in float4 columns: thread (dq, gi) takes chunks gi, gi + NG, ...
  const int D = s.D;
  const int DQ = D / 4;
  const int NG = kCombThreads / DQ;
  const int dq = tid % DQ, gi = tid / DQ;
  __shared__ float4 ored4[kCombThreads];
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int c = gi; c < nch; c += NG) {
    const float wc = nch <= kMaxChunkW ? wts[c] : __expf(part_ml[(base + c) * 2] - M);
    const float4 p = *reinterpret_cast<const float4*>(&part_o[(base + c) * D + 4 * dq]);
    o.x = fmaf(wc, p.x, o.x);
    o.y = fmaf(wc, p.y, o.y);
    o.z = fmaf(wc, p.z, o.z);
    o.w = fmaf(wc, p.w, o.w);
  }
  ored4[tid] = o;
  __syncthreads();
  if (gi == 0) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < NG; ++k) {
      const float4 v = ored4[k * DQ + dq];
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
    }
    const float inv = nch ? 1.f / lsum : 0.f;
    TO* op = out + ((int64_t)b * s.Hq + h) * D + 4 * dq;
    op[0] = from_f32<TO>(nch ? t.x * inv : 0.f);
    op[1] = from_f32<TO>(nch ? t.y * inv : 0.f);
    op[2] = from_f32<TO>(nch ? t.z * inv : 0.f);
    op[3] = from_f32<TO>(nch ? t.w * inv : 0.f);
  }
  if (lse && tid == 0) lse[(int64_t)b * s.Hq + h] = nch ? M + logf(lsum) : -INFINITY;
  if (RLA) {
    __shared__ float phq[128];
    const TQ* qh = q + ((int64_t)b * s.Hq + h) * D;
    for (int i = tid; i < D; i += kCombThreads) phq[i] = __expf(to_f32<TQ>(qh[i]));
    __syncthreads();  // (also: every thread is past its ored4 read)
    const float* st = rla_state + ((int64_t)b * s.Hkv + h / G) * (D + 1) * D;
    // phi(q)^T S over rows i = gi, gi + NG, ..., minus the chunks' selected terms
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int i = gi; i < D; i += NG) {
      const float4 r = *reinterpret_cast<const float4*>(&st[(int64_t)i * D + 4 * dq]);
      a.x = fmaf(phq[i], r.x, a.x);
      a.y = fmaf(phq[i], r.y, a.y);
      a.z = fmaf(phq[i], r.z, a.z);
      a.w = fmaf(phq[i], r.w, a.w);
    }
#pragma unroll 4
    for (int c = gi; c < nch; c += NG) {
      const float4 r = *reinterpret_cast<const float4*>(&part_rnum[(base + c) * D + 4 * dq]);
      a.x -= r.x;
      a.y -= r.y;
      a.z -= r.z;
      a.w -= r.w;
    }
    ored4[tid] = a;
    // denominator: phi(q) . z (row D of the state) minus the chunks' sums
    float dz = 0.f;
    for (int i = tid; i < D; i += kCombThreads) dz = fmaf(phq[i], st[(int64_t)D * D + i], dz);
    for (int c = tid; c < nch; c += kCombThreads) dz -= part_rden[base + c];
    dz = wave_sum(dz);
    if (lane == 0) wred[wave] = dz;
    __syncthreads();
    if (gi == 0) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < NG; ++k) {
        const float4 v = ored4[k * DQ + dq];
        t.x += v.x;
        t.y += v.y;
        t.z += v.z;
        t.w += v.w;
      }
      *reinterpret_cast<float4*>(&rla_num[((int64_t)b * s.Hq + h) * D + 4 * dq]) = t;
    }
    if (tid == 0) rla_den[(int64_t)b * s.Hq + h] = (wred[0] + wred[1]) + (wred[2] + wred[3]);
  }
}

// Residual linear attention state ("SPLA", section 2.2): for each (sequence,
// group), S[i][c] += sum_j exp(k_j[i]) v_j[c] (rows 0 .. D-1) and
// z[i] += sum_j exp(k_j[i]) (row D) over tokens j in [first, seq_lens[b]).  Workgroup = 16 rows of S (a
// stripe); thread (r, cg) owns row r's columns cg, cg + 16, ... and, for
// cg = 0, z[r].  Tokens go through LDS 32 at a time; fixed summation order.
constexpr int kRlaTok = 32;

template <typename T, int D>
__global__ void __launch_bounds__(256)
k_rla_state(const T* __restrict__ k_pool, const T* __restrict__ v_pool,
            const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
            Shape s, int32_t first, float* __restrict__ state) {
  constexpr int NC = D / 16;  // columns per thread
  const int stripe = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, r = t / 16, cg = t % 16;
  const int i = stripe * 16 + r;
  const int32_t L = clamp_len(seq_lens[b], s.max_len);
  const int32_t* pt = page_table + (int64_t)b * s.max_pages;
  __shared__ float phk[kRlaTok][16];
  __shared__ float vs[kRlaTok][D];
  // compensated (Kahan) sums: the error of a state element stays a few fp32
  // rounding units of its magnitude however many tokens the cache holds
  float acc[NC], cmp[NC], zacc = 0.f, zcmp = 0.f;
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    acc[m] = 0.f;
    cmp[m] = 0.f;
  }
  for (int32_t j0 = first < 0 ? 0 : first; j0 < L; j0 += kRlaTok) {
    __syncthreads();
    // K: 32 tokens x this stripe's 16 dims; V: 32 tokens x D dims
    for (int e = t; e < kRlaTok * 16; e += 256) {
      const int tk = e / 16, dd = e % 16;
      const int32_t j = j0 + tk;
      float v = 0.f;
      if (j < L) {
        const int64_t row = (clamp_page(pt[j >> 6], s.n_pool_pages) * s.Hkv + g) * kPage + (j & 63);
        v = __expf(to_f32<T>(k_pool[row * D + stripe * 16 + dd]));
      }
      phk[tk][dd] = v;
    }
    for (int e = t; e < kRlaTok * D; e += 256) {
      const int tk = e / D, dd = e % D;
      const int32_t j = j0 + tk;
      float v = 0.f;
      if (j < L) {
        const int64_t row = (clamp_page(pt[j >> 6], s.n_pool_pages) * s.Hkv + g) * kPage + (j & 63);
        v = to_f32<T>(v_pool[row * D + dd]);
      }
      vs[tk][dd] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int tk = 0; tk < kRlaTok; ++tk) {
      const float p = phk[tk][r];
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        const float y = fmaf(p, vs[tk][cg + 16 * m], -cmp[m]);
        const float t2 = acc[m] + y;
        cmp[m] = (t2 - acc[m]) - y;
        acc[m] = t2;
      }
      const float yz = p - zcmp;
      const float tz = zacc + yz;
      zcmp = (tz - zacc) - yz;
      zacc = tz;
    }
  }
  float* st = state + ((int64_t)b * s.Hkv + g) * (D + 1) * D;
#pragma unroll
  for (int m = 0; m < NC; ++m) st[(int64_t)i * D + cg + 16 * m] += acc[m];
  if (cg == 0) st[(int64_t)D * D + i] += zacc;
}

// Workgroups of a kernel instance resident per compute unit (registers and
// LDS), from the runtime; cached per instance and device.
int resident_per_cu(const void* fn, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(fn, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess || n < 1) n = 1;
  cache[key] = n;
  return n;
}

// Persistent grid of the split kernel: blocks resident on the chip.
int split_grid(int nchunk_max, int rows, int per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const long long most = (long long)nchunk_max * rows;
  const long long g = (long long)per_cu * cus;
  return (int)(most < g ? (most < 1 ? 1 : most) : g);
}

struct RlaArgs {
  const float* state;  // [B][Hkv][D + 1][D]
  float* num;          // [B][Hq][D]
  float* den;          // [B][Hq]
  void* part;          // per-chunk sums, or NULL: after the other partials
};

template <typename T, int D, bool RLA>
hipError_t launch_t(const Shape& s, const sa_pages& pg, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* idx, const int32_t* count, int32_t cap,
                    float s_att, void* out, sa_dtype out_dt, float* lse, void* ws,
                    const RlaArgs& rla, hipStream_t st) {
  const int32_t nchunk_max = (cap + kTile - 1) / kTile;
  const size_t n_part = (size_t)s.B * s.Hq * nchunk_max;
  float* part_ml = (float*)ws;
  float* part_o = part_ml + align_up(n_part * 2, 64);
  float* part_rnum = rla.part ? (float*)rla.part : part_o + align_up(n_part * D, 64);
  float* part_rden = part_rnum + align_up(n_part * D, 64);
  const int G = s.Hq / s.Hkv;
  // few rows: the small row prefix leaves more LDS per workgroup free; the
  // persistent grid is as many workgroups as stay resident together
  const bool small = s.B * s.Hkv <= kSmallRowsLds;
  int gx = 1;
#define SA_DS(GG)                                                                              \
  {                                                                                            \
    const void* fn = small ? (const void*)k_decode_split<T, D, GG, RLA, kSmallRowsLds>         \
                           : (const void*)k_decode_split<T, D, GG, RLA, kMaxRowsLds>;          \
    constexpr int NT = DecodeCfg<T, D, GG>::NT;                                                \
    gx = split_grid(nchunk_max, s.B * s.Hkv, resident_per_cu(fn, NT));                         \
    dim3 grid(gx);                                                                             \
    if (small)                                                                                 \
      k_decode_split<T, D, GG, RLA, kSmallRowsLds><<<grid, NT, 0, st>>>(                        \
          (const T*)q, (const T*)k_pool, (const T*)v_pool, pg.page_table, pg.seq_lens, idx,    \
          count, cap, s, s_att, nchunk_max, part_ml, part_o, part_rnum, part_rden);            \
    else                                                                                       \
      k_decode_split<T, D, GG, RLA, kMaxRowsLds><<<grid, NT, 0, st>>>(                          \
          (const T*)q, (const T*)k_pool, (const T*)v_pool, pg.page_table, pg.seq_lens, idx,    \
          count, cap, s, s_att, nchunk_max, part_ml, part_o, part_rnum, part_rden);            \
  }
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
    k_decode_combine<bf16_raw, T, RLA><<<g2, kCombThreads, 0, st>>>(
        part_ml, part_o, count, cap, s, gx, nchunk_max, (bf16_raw*)out, lse, (const T*)q,
        rla.state, part_rnum, part_rden, rla.num, rla.den);
  else
    k_decode_combine<float, T, RLA><<<g2, kCombThreads, 0, st>>>(
        part_ml, part_o, count, cap, s, gx, nchunk_max, (float*)out, lse, (const T*)q,
        rla.state, part_rnum, part_rden, rla.num, rla.den);
  return hipGetLastError();
}

template <bool RLA>
hipError_t launch_decode(const Shape& s, const sa_pages& pg, const void* q, const void* k_pool,
                         const void* v_pool, sa_dtype dt, const int32_t* idx, const int32_t* count,
                         int32_t cap, float s_att, void* out, sa_dtype out_dt, float* lse, void* ws,
                         const RlaArgs& rla, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  // the kernels keep a listed token's pool row as page << 6 | slot in 32 bits
  if (s.n_pool_pages >= ((int64_t)1 << 26)) return hipErrorNotSupported;
  if (dt == SA_BF16) {
    if (s.D == 128)
      return launch_t<bf16_raw, 128, RLA>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, rla, st);
    return launch_t<bf16_raw, 64, RLA>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, rla, st);
  }
  if (s.D == 128)
    return launch_t<float, 128, RLA>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, rla, st);
  return launch_t<float, 64, RLA>(s, pg, q, k_pool, v_pool, idx, count, cap, s_att, out, out_dt, lse, ws, rla, st);
}

}  // namespace

size_t decode_rla_part_bytes(const Shape& s, int32_t cap) {
  const size_t n_part = (size_t)s.B * s.Hq * (size_t)((cap + kTile - 1) / kTile);
  return (align_up(n_part * s.D, 64) + align_up(n_part, 64)) * sizeof(float);
}

size_t decode_workspace_bytes(const Shape& s, int32_t cap, bool rla) {
  const size_t n_part = (size_t)s.B * s.Hq * (size_t)((cap + kTile - 1) / kTile);
  const size_t n = align_up(n_part * 2, 64) + align_up(n_part * s.D, 64);
  return n * sizeof(float) + (rla ? decode_rla_part_bytes(s, cap) : 0);
}

hipError_t launch_sparse_decode(const Shape& s, const sa_pages& pg, const void* q,
                                const void* k_pool, const void* v_pool, sa_dtype dt,
                                const int32_t* idx, const int32_t* count, int32_t cap,
                                float s_att, void* out, sa_dtype out_dt, float* lse,
                                void* ws, hipStream_t st) {
  return launch_decode<false>(s, pg, q, k_pool, v_pool, dt, idx, count, cap, s_att, out, out_dt,
                              lse, ws, RlaArgs{nullptr, nullptr, nullptr, nullptr}, st);
}

hipError_t launch_sparse_decode_rla(const Shape& s, const sa_pages& pg, const void* q,
                                    const void* k_pool, const void* v_pool, sa_dtype dt,
                                    const int32_t* idx, const int32_t* count, int32_t cap,
                                    float s_att, void* out, sa_dtype out_dt, float* lse,
                                    const float* rla_state, float* rla_num, float* rla_den,
                                    void* ws, void* rla_part, hipStream_t st) {
  return launch_decode<true>(s, pg, q, k_pool, v_pool, dt, idx, count, cap, s_att, out, out_dt,
                             lse, ws, RlaArgs{rla_state, rla_num, rla_den, rla_part}, st);
}

hipError_t launch_rla_state(const Shape& s, const sa_pages& pg, const void* k_pool,
                            const void* v_pool, sa_dtype dt, int32_t first, float* state,
                            hipStream_t st) {
  if (s.B == 0 || s.Hkv == 0) return hipSuccess;
  dim3 grid(s.D / 16, s.Hkv, s.B);
  if (dt == SA_BF16) {
    if (s.D == 128)
      k_rla_state<bf16_raw, 128><<<grid, 256, 0, st>>>((const bf16_raw*)k_pool, (const bf16_raw*)v_pool,
                                                       pg.page_table, pg.seq_lens, s, first, state);
    else
      k_rla_state<bf16_raw, 64><<<grid, 256, 0, st>>>((const bf16_raw*)k_pool, (const bf16_raw*)v_pool,
                                                      pg.page_table, pg.seq_lens, s, first, state);
  } else {
    if (s.D == 128)
      k_rla_state<float, 128><<<grid, 256, 0, st>>>((const float*)k_pool, (const float*)v_pool,
                                                    pg.page_table, pg.seq_lens, s, first, state);
    else
      k_rla_state<float, 64><<<grid, 256, 0, st>>>((const float*)k_pool, (const float*)v_pool,
                                                   pg.page_table, pg.seq_lens, s, first, state);
  }
  return hipGetLastError();
}

}  // namespace sa
