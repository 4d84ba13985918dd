// Whole decode step in one persistent launch, for problems with few
// (sequence, group) rows where a chain of separate launches would be latency
// bound.  Same arithmetic as the separate calls: head-collapsed low-rank
// indexer scores ("Full Attention Strikes Back", method section 2), top-p by
// attention mass or top-k found by a radix histogram threshold (method
// sections 3 and 5) with the sink/window tokens added (method section 1), and
// exact softmax attention over the support ("Oracle-Guided Sparse Prefill",
// section 2.1).
//
// Each row is served by NB co-resident workgroups, each owning a contiguous
// range of the row's tokens.  They meet at per-row barriers (one arrival flag
// per workgroup in the workspace, bounded spins that raise an error flag
// instead of waiting forever):
//   1. collapse the query, score the own tokens (kept in registers); top-p
//      rows exchange their maxima in the first barrier's flag words;
//                                                               -- barrier
//   2. per radix level: LDS histogram of the own tokens, flush non-empty bins
//      to the row's global histogram;                           -- barrier
//      every workgroup resolves the level from the same global histogram;
//   3. own selected tokens (minus sink/window) plus an even share of the
//      sink/window tokens are attended (split-KV partial per workgroup; bf16
//      on the matrix cores), the own selected count is published; -- barrier
//   4. each workgroup merges a slice of the row's outputs, and writes its
//      part of the index list at the prefix of lower workgroups' counts.
// Histograms and barrier flags are returned to zero before the launch ends.
//
// Page mode runs the same phases over a sequence's 64-token pages: Taylor
// page scores from the mean and diagonal variance of each page's keys
// ("SPLA", section 2.1) in phase 1, a top-k of pages in phase 2, and in
// phase 3 every workgroup attends the tokens of its own selected pages (a
// row's selected pages are few; exchanging them to split the tokens evenly
// cost a barrier more than the imbalance costs).  In both modes the first
// tiles of a workgroup's surely selected candidates (above the level-1
// crossing bin) are attended while the level-2 barrier completes.
// Selection-only mode takes the scores from memory in phase 1 and stops
// after the index list.
#include <map>
#include <mutex>
#include <utility>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kNT = 256;                  // threads per workgroup
constexpr int kBinsF = 4096;              // 12-bit digits
constexpr int kCoarseF = kBinsF / 64;
constexpr int kTileF = 64;                // attention tile (tokens)
constexpr uint32_t kSpinLimit = 1u << 20; // about a second of polling, then give up
constexpr int kMaxNB = 256;
constexpr int kFusedMaxPages = 32;        // page mode: largest top-k (pages)

enum : uint32_t { kSearch = 0, kGE = 1, kTies = 2 };

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2f_t;
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2f_t, a),
                                          __builtin_bit_cast(bf16x2f_t, b), c, false);
}

struct RowWs {            // per-row control block (zero between launches)
  uint32_t exit;          // workgroups done
  uint32_t err;           // set if a barrier of the row gave up waiting
  uint32_t pad[14];
};

struct FusedArgs {
  const void* q;          // [B][Hq][D]
  const void* stats;      // page mode: page statistics pool [P][Hkv][2][D]
  const void* w_q;        // [Hq][D][16]
  const void* kidx;       // pool [P][Hkv][64][16]
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  Shape s;
  float s_idx, s_att, p;
  int32_t top_k, n_sink, n_window;
  float* x;
  int64_t ldx;
  int32_t* idx;
  int32_t* count;
  int32_t cap;
  void* out;
  int32_t out_bf16;
  float* lse;
  int32_t nb;             // workgroups per row
  int32_t tpb;            // tokens per workgroup (multiple of kNT)
  // workspace
  RowWs* ctl;             // [rows]
  uint32_t* hcnt;         // [3][rows][kBinsF]
  uint64_t* hmass;        // [3][rows][kBinsF]
  uint32_t* ccnt;         // [3][rows][kCoarseF]
  uint64_t* cmass;        // [3][rows][kCoarseF]
  uint32_t* blk_sel;      // [rows][nb] selected tokens of each workgroup
  uint32_t* blk_eq;       // [rows][nb] threshold ties of each workgroup
  float* part_ml;         // [rows][nb][G][2]
  float* part_o;          // [rows][nb][G][D]
  // residual linear attention over the tokens left out (token mode, bf16):
  // state [B][Hkv][D + 1][D] (S rows, then z), outputs [B][Hq][D] and [B][Hq],
  // per-workgroup sums over the own listed tokens
  const float* rla_state;
  float* rla_num;
  float* rla_den;
  float* part_rnum;       // [rows][nb][G][D]
  float* part_rden;       // [rows][nb][G]
  uint64_t* trace;        // [rows * nb][kTraceSlots] phase timestamps (diagnostics)
  uint64_t* mflag;        // [rows][kMaxNB] marker bit 32 | own maximum score key
  uint32_t* flags;        // [rows][kMaxNB] barrier arrival flags (barriers passed)
};

constexpr int kTraceSlots = 16;

// Phase timestamp of this workgroup (100 MHz constant clock), thread 0 only.
__device__ __forceinline__ void stamp(const FusedArgs& a, int slot) {
  if (threadIdx.x == 0) a.trace[(int64_t)blockIdx.x * kTraceSlots + slot] = __builtin_amdgcn_s_memrealtime();
}

// Per-row barrier.  Everything one workgroup hands to another (histogram
// bins, counts, the row maximum, attention partials) is written with
// device-scope atomics or device-scope stores, which complete at the
// device's coherence point, and read with device-scope loads, which the L2
// does not serve stale.  So the barrier needs no L2 write-back or
// invalidate: each wave waits until its own memory operations have
// completed, then the workgroup raises its own arrival flag to the barrier's
// number.  One wave per workgroup polls the row's flags (one per workgroup,
// adjacent, so a poll is one vector load) until all reached that number.
// Separate flags keep the arrivals from queueing on one counter.  The spin
// is bounded: a barrier that waits too long raises the error flag and lets
// the launch finish instead of hanging.
__device__ __forceinline__ void row_barrier(uint32_t* flags, int nb, int bi, uint32_t epoch, uint32_t* err) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads, stores and atomics completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x < kWave) {
    if (threadIdx.x == 0) __hip_atomic_store(&flags[bi], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    for (;;) {
      bool ok = true;
      for (int k = (int)threadIdx.x; k < nb; k += kWave)
        ok = ok && __hip_atomic_load(&flags[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= epoch;
      if (__all(ok)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        if (threadIdx.x == 0) atomicOr(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// row_barrier in two halves: arrive (this workgroup's memory operations
// completed, its flag raised), later wait for the row's flags; between them
// the workgroup works on what it already holds.
__device__ __forceinline__ void row_arrive(uint32_t* flags, int bi, uint32_t epoch) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(&flags[bi], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void row_wait(uint32_t* flags, int nb, uint32_t epoch, uint32_t* err) {
  if (threadIdx.x < kWave) {
    uint32_t spins = 0;
    for (;;) {
      bool ok = true;
      for (int k = (int)threadIdx.x; k < nb; k += kWave)
        ok = ok && __hip_atomic_load(&flags[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= epoch;
      if (__all(ok)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        if (threadIdx.x == 0) atomicOr(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// The first barrier of a top-p row also yields the row's maximum score key:
// each workgroup stores its own maximum under a marker bit in one 64-bit
// word (written once per launch, so a word never changes while another
// workgroup polls it), and the polling wave reduces the words once every
// one is marked.  Bounded like row_barrier.
__device__ __forceinline__ uint32_t row_barrier_max(uint64_t* mflag, int nb, int bi, uint32_t mine,
                                                    uint32_t* err) {
  __shared__ uint32_t s_rowmax;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x < kWave) {
    if (threadIdx.x == 0)
      __hip_atomic_store(&mflag[bi], (1ull << 32) | mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    for (;;) {
      bool ok = true;
      uint32_t m = 0;
      for (int k = (int)threadIdx.x; k < nb; k += kWave) {
        const uint64_t f = __hip_atomic_load(&mflag[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = ok && (f >> 32) != 0;
        m = (uint32_t)f > m ? (uint32_t)f : m;
      }
      const bool done = __all(ok);
      if (done || ++spins > kSpinLimit) {
        m = wave_max_u32(m);
        if (threadIdx.x == 0) {
          s_rowmax = m;
          if (!done) atomicOr(err, 1u);
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return s_rowmax;
}

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename U>
__device__ __forceinline__ U blk_scan(U v, U* lds, U& total) {  // exclusive, kNT threads
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  static_assert(sizeof(U) == 4, "32-bit scan");
  const U inc = wave_incl_scan(v);
  if (lane == 63) lds[w] = inc;
  __syncthreads();
  U off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) {
    U s = lds[i];
    if (i < w) off += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// PAGES: the candidates are the sequence's pages, scored by the Taylor page
// score; the top-k pages' tokens are attended and listed.  SEL: selection
// only, over scores given in x (no attention, no outputs).
template <typename T, int D, int G, int TPT, bool PAGES, bool SEL, bool RLA = false>
__global__ void __launch_bounds__(kNT) k_decode_fused(FusedArgs a) {
  constexpr int HPW = G / 4 > 0 ? G / 4 : 1;   // heads per wave (G >= 4)
  constexpr int DPL = D / 64;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;
  constexpr int PITCH = ROWB + 16;
  constexpr int TM = kTileF;  // attention tile (tokens)
  constexpr int LPT = TM * CPR / kNT;
  const Shape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = a.nb;
  const int row = blockIdx.x / NB, bi = blockIdx.x % NB;
  const int rows = s.B * s.Hkv;
  const int b = row / s.Hkv, g = row % s.Hkv;
  const int32_t L = clamp_len(a.seq_lens[b], s.max_len);
  const int32_t n = PAGES ? (L + kPage - 1) / kPage : L;  // candidates of the row
  const int32_t j0 = bi * a.tpb;
  RowWs* ctl = a.ctl + row;
  uint32_t* err = &ctl->err;
  uint32_t epoch = 0;                       // barriers passed
  uint32_t* flags = a.flags + (int64_t)row * kMaxNB;

  // ---- LDS ----
  __shared__ float s_qc[kRank];
  __shared__ float red_f[4][kRank];
  __shared__ uint32_t red_u[4];
  __shared__ uint64_t red_u64[4];
  // the level histograms (selection) and the K/V tiles (attention, after
  // the last level) share one LDS region, so that two workgroups fit a
  // compute unit
  constexpr int kHistBytes = kBinsF * (4 + 8);
  constexpr int kTileBytes = 2 * TM * PITCH;
  __shared__ __align__(16) char lds_big[kHistBytes > kTileBytes ? kHistBytes : kTileBytes];
  uint32_t(&hcnt_l)[kBinsF] = *reinterpret_cast<uint32_t(*)[kBinsF]>(lds_big);
  uint64_t(&hmass_l)[kBinsF] = *reinterpret_cast<uint64_t(*)[kBinsF]>(lds_big + kBinsF * 4);
  char* const Ks = lds_big;
  char* const Vs = lds_big + TM * PITCH;
  __shared__ __align__(16) T Qs[G][D];
  __shared__ __align__(16) float Ps[G][kTileF];
  // pool token rows ((page * Hkv + g) * 64 + slot) of the tokens to attend
  __shared__ uint32_t my_list[PAGES ? kFusedMaxPages * kPage : TPT * kNT + 64];
  // pool pages of the own token range
  __shared__ int32_t s_pt[TPT * kNT / kPage];
  __shared__ uint32_t s_mode, s_prefix, s_thr, s_neq, s_need, s_cnt;
  __shared__ uint32_t s_base, s_total;
  __shared__ uint64_t s_rem;
  __shared__ uint32_t s_slice[TPT * 4];
  // page mode: the own selected pages in index order (sequence page, pool page)
  __shared__ int32_t s_spj[kFusedMaxPages], s_spp[kFusedMaxPages];
  __shared__ uint32_t s_np;
  // page mode: which own pages were attended early; the pool pages left
  __shared__ uint32_t s_spe[kFusedMaxPages];
  __shared__ int32_t s_spa[kFusedMaxPages];

  stamp(a, 0);
  const int32_t* pt = a.page_table + (int64_t)b * s.max_pages;
  float xk[TPT];
  uint32_t key[TPT];
  uint32_t M = 0;         // row maximum score key (top-p)
  uint32_t own_max = 0;   // this workgroup's maximum (thread 0)
  if constexpr (PAGES) {
    // ---- 1. Taylor scores of the own pages: D / 8 lanes per page as in the
    // page-score kernel (same operations, same scores).  The page table
    // entries and the query are fetched together, then up to 16 rounds of
    // page statistics are in flight at once; the scores are gathered in LDS
    // in candidate order (the slot of a page first holds its pool page) ----
    constexpr int LPP = D / 8, PPW = kWave / LPP, PPI = 4 * PPW;  // pages per workgroup round
    constexpr int PBM = G >= 16 ? 8 : 16;
    constexpr int NR = TPT * kNT / PPI, PB = NR < PBM ? NR : PBM;   // rounds, rounds in flight
    static_assert(sizeof(T) == 2, "page mode: bf16 statistics");
    __shared__ __align__(16) float s_qs[D];
    __shared__ __align__(16) float s_qq[G][D];
    __shared__ float s_ps[TPT * kNT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      s_ps[u * kNT + tid] = __int_as_float(j < n ? (int32_t)clamp_page(pt[j], s.n_pool_pages) : 0);
    }
    stage_page_query<T, D, G>((const T*)a.q + ((int64_t)b * s.Hq + g * G) * D, a.s_att, s_qs, s_qq, kNT);
    // the group's query rows for the attention phase
    for (int i = tid; i < G * D; i += kNT) Qs[i / D][i % D] = ((const T*)a.q)[((int64_t)b * s.Hq + g * G) * D + i];
    __syncthreads();
    const int sub = lane % LPP, slot = lane / LPP;
    const T* stats = (const T*)a.stats;
    typedef uint32_t w4_t __attribute__((ext_vector_type(4)));
    for (int r0 = 0; r0 < NR; r0 += PB) {
      w4_t mraw[PB], vraw[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int32_t jl = (r0 + u) * PPI + wave * PPW + slot;
        // (branch-free: a slot past the row holds pool page 0, whose
        // statistics are read and whose score is not kept)
        const int64_t page = __float_as_int(s_ps[jl]);
        const T* rowp = stats + (page * s.Hkv + g) * 2 * (int64_t)D + sub * 8;
        mraw[u] = *reinterpret_cast<const w4_t*>(rowp);
        vraw[u] = *reinterpret_cast<const w4_t*>(rowp + D);
      }
      float qs[8], qq[G][8];
      page_query_lane<D, G>(s_qs, s_qq, sub, qs, qq);
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int32_t jl = (r0 + u) * PPI + wave * PPW + slot;
        float mu[8], va[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mu[2 * i] = __uint_as_float(mraw[u][i] << 16);
          mu[2 * i + 1] = __uint_as_float(mraw[u][i] & 0xffff0000u);
          va[2 * i] = __uint_as_float(vraw[u][i] << 16);
          va[2 * i + 1] = __uint_as_float(vraw[u][i] & 0xffff0000u);
        }
        const float sum = page_score_sum<LPP, G>(mu, va, qs, qq, sub);
        if (sub == 0 && j0 + jl < n) s_ps[jl] = page_score_final<G>(sum, L, j0 + jl);
      }
    }
    __syncthreads();
    float* xr = a.x + (int64_t)row * a.ldx;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      xk[u] = j < n ? s_ps[u * kNT + tid] : 0.f;
      key[u] = j < n ? score_key(xk[u]) : 0u;
      if (j < n) xr[j] = xk[u];
    }
    stamp(a, 1);
  } else if constexpr (SEL) {
    // ---- 1. the own candidates' given scores ----
    const float* xr = a.x + (int64_t)row * a.ldx;
    uint32_t mk = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      xk[u] = j < n ? xr[j] : 0.f;
      key[u] = j < n ? score_key(xk[u]) : 0u;
      mk = key[u] > mk ? key[u] : mk;
    }
    mk = wave_max_u32(mk);
    if (lane == 0) red_u[wave] = mk;
    __syncthreads();
    if (tid == 0) {
      for (int i = 0; i < 4; ++i) mk = red_u[i] > mk ? red_u[i] : mk;
      own_max = mk;
    }
    stamp(a, 1);
    if (a.top_k <= 0) M = row_barrier_max(a.mflag + (int64_t)row * kMaxNB, NB, bi, own_max, err);
  } else {
    // ---- 1. scores of the own tokens ----
  const T* kidx = (const T*)a.kidx;
  const T* q = (const T*)a.q;
  const T* w_q = (const T*)a.w_q;
  {
    // Issued together: the pool pages of the own tokens (per lane straight
    // from the page table; a wave's lanes share each page, so a round is one
    // broadcast load), and the collapse's projector rows and query values.
    // The indexer keys follow as soon as the pages arrive, and the collapse
    // is computed while they are in flight.
    // (branch-free: a token past the row reads the row's last valid entry,
    // or entry 0 of an empty row, and its key is zeroed after the load, so
    // the compiler need not wait for each load where it is issued)
    const int32_t jlast = n > 0 ? n - 1 : 0;
    int64_t pgu[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = min(j0 + u * kNT + tid, jlast);
      pgu[u] = clamp_page(pt[j >> 6], s.n_pool_pages);
    }
    for (int i = tid; i < TPT * kNT / kPage; i += kNT)  // (for the lists; the barriers below publish it)
      s_pt[i] = j0 + i * kPage < n ? (int32_t)clamp_page(pt[(j0 >> 6) + i], s.n_pool_pages) : 0;
    constexpr int NPI = G * D / kNT;  // collapse products per thread
    static_assert(G * D % kNT == 0, "whole collapse rounds");
    float w[NPI][kRank], qv[NPI];
#pragma unroll
    for (int ip = 0; ip < NPI; ++ip) {
      const int pi = tid + ip * kNT;
      const int h = g * G + pi / D, i = pi % D;
      const T* wr = w_q + ((int64_t)h * D + i) * kRank;
      if constexpr (sizeof(T) == 2) {
        const uint4* v = reinterpret_cast<const uint4*>(wr);
        const uint4 x0 = v[0], x1 = v[1];
        const uint32_t w8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          w[ip][2 * k] = __uint_as_float(w8[k] << 16);
          w[ip][2 * k + 1] = __uint_as_float(w8[k] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kRank; ++k) w[ip][k] = to_f32<T>(wr[k]);
      }
      qv[ip] = to_f32<T>(q[((int64_t)b * s.Hq + h) * D + i]);
    }
    float kv[TPT][kRank];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t jt = j0 + u * kNT + tid;
      const bool valid = jt < n;
      const int32_t j = min(jt, jlast);
      const T* rowp = kidx + ((pgu[u] * s.Hkv + g) * kPage + (j & 63)) * kRank;
      if constexpr (sizeof(T) == 2) {
        const uint4* v = reinterpret_cast<const uint4*>(rowp);
        const uint4 x0 = v[0], x1 = v[1];
        const uint32_t w8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          kv[u][2 * i] = valid ? __uint_as_float(w8[i] << 16) : 0.f;
          kv[u][2 * i + 1] = valid ? __uint_as_float(w8[i] & 0xffff0000u) : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRank; ++i) kv[u][i] = valid ? to_f32<T>(rowp[i]) : 0.f;
      }
    }
    // head-collapsed query (same order of operations as k_collapse)
    float acc[kRank];
#pragma unroll
    for (int c = 0; c < kRank; ++c) acc[c] = 0.f;
#pragma unroll
    for (int ip = 0; ip < NPI; ++ip)
#pragma unroll
      for (int c = 0; c < kRank; ++c) acc[c] = fmaf(w[ip][c], qv[ip], acc[c]);
#pragma unroll
    for (int c = 0; c < kRank; ++c) {
      const float v = wave_sum(acc[c]);
      if (lane == 0) red_f[wave][c] = v;
    }
    // the group's query rows for the attention phase (just read by the collapse)
    for (int i = tid; i < G * D; i += kNT) Qs[i / D][i % D] = q[((int64_t)b * s.Hq + g * G) * D + i];
    __syncthreads();
    if (tid < kRank)
      s_qc[tid] = ((red_f[0][tid] + red_f[1][tid]) + (red_f[2][tid] + red_f[3][tid])) * (a.s_idx / (float)G);
    __syncthreads();
    float qc[kRank];
#pragma unroll
    for (int c = 0; c < kRank; ++c) qc[c] = s_qc[c];
    uint32_t mk = 0;
    float* xr = a.x + (int64_t)row * a.ldx;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      float acc1 = 0.f;
#pragma unroll
      for (int c = 0; c < kRank; ++c) acc1 = fmaf(qc[c], kv[u][c], acc1);
      xk[u] = acc1;
      key[u] = j < n ? score_key(acc1) : 0u;
      if (j < n) {
        xr[j] = acc1;
        mk = key[u] > mk ? key[u] : mk;
      }
    }
    mk = wave_max_u32(mk);
    if (lane == 0) red_u[wave] = mk;
    __syncthreads();
    if (tid == 0) {
      for (int i = 0; i < 4; ++i) mk = red_u[i] > mk ? red_u[i] : mk;
      own_max = mk;
    }
  }
    stamp(a, 1);
    // the row maximum is the top-p mass reference
    if (a.top_k <= 0) M = row_barrier_max(a.mflag + (int64_t)row * kMaxNB, NB, bi, own_max, err);
  }
  stamp(a, 2);

  // ---- attention machinery (the matrix-core tiles of phase 3; in token
  // mode it also runs during the level-2 barrier) ----
  const T* k_pool = (const T*)a.k_pool;
  const T* v_pool = (const T*)a.v_pool;
  int32_t n_cur = 0;  // tokens of the current attention job in my_list
  // Matrix-core attention: in each 64-token tile wave w takes tokens
  // [16w, 16w + 16).  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 leaves a lane
  // with 4 tokens of one head (head = lane % 16, the group's heads padded
  // to 16 with zero queries), which is the lane layout of the P^T operand
  // of O^T += V^T P^T on v_mfma_f32_16x16x16_bf16, so each wave runs its own
  // online softmax without exchanging scores.  P enters the product as a
  // bf16 high part plus the bf16 rounding of the remainder (16 significant
  // bits); K and V are staged row-major.  The four waves' softmax states
  // are merged once at the end.
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
  typedef __attribute__((ext_vector_type(4))) short s16x4_t;
  typedef __attribute__((ext_vector_type(4))) float f32x4_t;
  constexpr int KS = D / 32, MB = D / 16;
  static_assert(2 * D * 16 * 4 <= TM * PITCH, "two waves' outputs fit one tile buffer");
  __shared__ float s_wm[4][16], s_wl[4][16];
  const int hq = lane & 15, lg = lane >> 4;
  bf16x8_t qB[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (hq < G) w = *reinterpret_cast<const uint4*>(&Qs[hq < G ? hq : 0][32 * ks + 8 * lg]);
    qB[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x4_t oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // Residual linear attention over the tokens left out ("SPLA", section
  // 2.2, subtraction form), with RLA: this workgroup's sums over its own
  // listed tokens, num_h = sum_j w_hj v_j and den_h = sum_j w_hj, where
  // w_hj = phi(q_h) . phi(k_j) and phi = exp elementwise, on the matrix
  // cores beside the attention: W^T = phi(K) phi(Q)^T takes the A operand's
  // key registers of S^T (exponentiated) and phi(Q) in place of Q, each
  // fp32 factor split into a bf16 high part and the bf16 rounding of the
  // remainder (three products: hi.hi, hi.lo, lo.hi; the dropped lo.lo term
  // and the roundings stay below 2^-16 of each product); W^T has the lane
  // layout of P^T, so num^T += V^T W^T reuses the V^T operand, again with
  // W split into high and low parts.
  typedef __attribute__((ext_vector_type(8))) float f32x8_t;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  typedef __attribute__((ext_vector_type(4))) float f32x4v_t;
  bf16x8_t qH[RLA ? KS : 1], qL[RLA ? KS : 1];
  f32x4_t racc[RLA ? MB : 1];
  float rden = 0.f;  // lane (head hq): its tokens' weights
  if constexpr (RLA) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x8_t f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = hq < G ? __expf(to_f32<T>(Qs[hq < G ? hq : 0][32 * ks + 8 * lg + e])) : 0.f;
      qH[ks] = __builtin_convertvector(f, bf16x8_t);
      qL[ks] = __builtin_convertvector(f - __builtin_convertvector(qH[ks], f32x8_t), bf16x8_t);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) racc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // K and V rows: 16 lanes per row (contiguous loads), staged row-major;
  // the V^T operand is gathered from four rows by 2-byte LDS reads.  Tiles
  // go in pairs through two register buffers: while a tile is computed the
  // next tile's rows and the following pair's are in flight.  The gathers
  // are branch-free (rows past the list re-read its last token, whose
  // scores are masked), so the compiler waits for one buffer's loads at a
  // staging, not for every load in flight.
  // (each buffer is one vector value, so it stays in registers)
  typedef uint32_t kvv_t __attribute__((ext_vector_type(4 * LPT)));
  kvv_t kA, vA, kB, vB;
  // the pool rows of a tile's gather, read from the list one staging
  // ahead, so a gather waits for no LDS read
  typedef uint32_t ids_t __attribute__((ext_vector_type(LPT)));
  auto read_ids = [&](int32_t ts) __attribute__((always_inline)) {
    ids_t r;
#pragma unroll
    for (int i = 0; i < LPT; ++i) r[i] = my_list[min(ts + (i * kNT + tid) / CPR, n_cur - 1)];
    return r;
  };
  auto gather = [&](const ids_t& ids, kvv_t& kr, kvv_t& vr) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int pc = i * kNT + tid;
      const int ck = pc % CPR;
      const int64_t off = (int64_t)ids[i] * D + ck * 8;
      const uint4 k4 = *reinterpret_cast<const uint4*>(k_pool + off);
      const uint4 v4 = *reinterpret_cast<const uint4*>(v_pool + off);
      kr[4 * i] = k4.x; kr[4 * i + 1] = k4.y; kr[4 * i + 2] = k4.z; kr[4 * i + 3] = k4.w;
      vr[4 * i] = v4.x; vr[4 * i + 1] = v4.y; vr[4 * i + 2] = v4.z; vr[4 * i + 3] = v4.w;
    }
  };
  auto stage = [&](const kvv_t& kr, const kvv_t& vr) __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int pc = i * kNT + tid;
      const int rk = pc / CPR, ck = pc % CPR;
      *reinterpret_cast<uint4*>(Ks + rk * PITCH + ck * 16) =
          make_uint4(kr[4 * i], kr[4 * i + 1], kr[4 * i + 2], kr[4 * i + 3]);
      *reinterpret_cast<uint4*>(Vs + rk * PITCH + ck * 16) =
          make_uint4(vr[4 * i], vr[4 * i + 1], vr[4 * i + 2], vr[4 * i + 3]);
    }
    __syncthreads();
  };
  auto compute = [&](int32_t ts) __attribute__((always_inline)) {
    const int32_t nt = min(TM, n_cur - ts);
    f32x4_t S = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t W = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* krow = Ks + (16 * wave + hq) * PITCH + 16 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 kv = *reinterpret_cast<const uint4*>(krow + 64 * ks);
      const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kv);
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qB[ks], S, 0, 0, 0);
      if constexpr (RLA) {
        f32x8_t f = __builtin_convertvector(kb, f32x8_t);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = __expf(f[e]);
        const bf16x8_t kh = __builtin_convertvector(f, bf16x8_t);
        const bf16x8_t kl = __builtin_convertvector(f - __builtin_convertvector(kh, f32x8_t), bf16x8_t);
        W = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qH[ks], W, 0, 0, 0);
        W = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qL[ks], W, 0, 0, 0);
        W = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qH[ks], W, 0, 0, 0);
      }
    }
    float sv[4], mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = 16 * wave + 4 * lg + v < nt ? S[v] * a.s_att : -INFINITY;
      mt = fmaxf(mt, sv[v]);
    }
    mt = row4_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __expf(m_run - mu);  // 0 before the first valid token
    float pv[4], ls = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pv[v] = __expf(sv[v] - mu);
      ls += pv[v];
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // high part: round to nearest even (v_cvt_pk_bf16_f32); low part: the
    // remainder, exact in fp32, rounded the same way
    const f32x4v_t pvv = f32x4v_t{pv[0], pv[1], pv[2], pv[3]};
    const bf16x4_t phb = __builtin_convertvector(pvv, bf16x4_t);
    const bf16x4_t plb = __builtin_convertvector(pvv - __builtin_convertvector(phb, f32x4v_t), bf16x4_t);
    const s16x4_t ph = __builtin_bit_cast(s16x4_t, phb);
    const s16x4_t pl = __builtin_bit_cast(s16x4_t, plb);
    // the running maximum moved for no lane: the accumulators keep their scale
    const bool rescale = __any(alpha != 1.f);
    s16x4_t wh = s16x4_t{0, 0, 0, 0}, wl = s16x4_t{0, 0, 0, 0};
    if constexpr (RLA) {  // tokens past the list weigh nothing
      f32x4v_t wv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        wv[v] = 16 * wave + 4 * lg + v < nt ? W[v] : 0.f;
        rden += wv[v];
      }
      const bf16x4_t bh = __builtin_convertvector(wv, bf16x4_t);
      const bf16x4_t bl = __builtin_convertvector(wv - __builtin_convertvector(bh, f32x4v_t), bf16x4_t);
      wh = __builtin_bit_cast(s16x4_t, bh);
      wl = __builtin_bit_cast(s16x4_t, bl);
    }
    if (rescale) {  // (wave-uniform: a branch, not a select per accumulator)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const char* vcol = Vs + (16 * wave + 4 * lg) * PITCH + (16 * mb + hq) * 2;
      const uint32_t v0 = *reinterpret_cast<const uint16_t*>(vcol);
      const uint32_t v1 = *reinterpret_cast<const uint16_t*>(vcol + PITCH);
      const uint32_t v2 = *reinterpret_cast<const uint16_t*>(vcol + 2 * PITCH);
      const uint32_t v3 = *reinterpret_cast<const uint16_t*>(vcol + 3 * PITCH);
      const s16x4_t av = __builtin_bit_cast(s16x4_t, make_uint2(v0 | (v1 << 16), v2 | (v3 << 16)));
      oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, ph, oacc[mb], 0, 0, 0);
      oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pl, oacc[mb], 0, 0, 0);
      if constexpr (RLA) {
        racc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, wh, racc[mb], 0, 0, 0);
        racc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, wl, racc[mb], 0, 0, 0);
      }
    }
  };
  // the tiles of my_list[0, n_cur), continuing the running softmax state
  auto run_tiles = [&]() __attribute__((always_inline)) {
    int32_t ts = 0;
    if (n_cur > 0) {
      gather(read_ids(0), kA, vA);
      gather(read_ids(TM), kB, vB);
      ids_t nx = read_ids(2 * TM);
      for (; ts + TM < n_cur; ts += 2 * TM) {  // both tiles of the pair hold tokens
        stage(kA, vA);
        gather(nx, kA, vA);
        nx = read_ids(ts + 3 * TM);
        compute(ts);
        stage(kB, vB);
        gather(nx, kB, vB);
        nx = read_ids(ts + 4 * TM);
        compute(ts + TM);
      }
      if (ts < n_cur) {  // an odd last tile
        stage(kA, vA);
        compute(ts);
      }
    }
  };
  // Token mode on the matrix cores: the tokens above the level-1 crossing
  // bin are in the support whatever the later levels decide, so a
  // workgroup attends the first kEarlyTiles tiles of its own (sink/window
  // tokens aside) between arriving at the level-2 barrier and waiting on it
  // (about the barrier's latency; more would delay the row's resolve);
  // phase 3 then attends the rest.  Which tokens go early depends on the
  // scores only, so the result stays deterministic.
  // Page mode likewise, a candidate being a page: the first kEarlyTiles
  // surely selected pages go early.
  constexpr bool kEarly = sizeof(T) == 2 && !SEL;
  constexpr int kEarlyTiles = 3;
  uint32_t early_bits = 0;  // bit u: candidate u of this thread was attended early
  __shared__ int32_t s_epp[kEarlyTiles], s_epl[kEarlyTiles];  // page mode: early pages (pool page, tokens)
  auto early_attend = [&](uint32_t pre1) __attribute__((always_inline)) {
    uint32_t cnt = 0, sure = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      const bool b = j < n && (PAGES || !(j < a.n_sink || j >= n - a.n_window)) && (key[u] >> 20) > pre1;
      sure |= b ? (1u << u) : 0u;
      cnt += b ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t o = blk_scan<uint32_t>(cnt, red_u, tot);
    if constexpr (PAGES) {
      // pages in index order; only the sequence's last page (the last of
      // them) may be partial, so page k's tokens start at 64 k
#pragma unroll
      for (int u = 0; u < TPT; ++u)
        if (((sure >> u) & 1u) && o < (uint32_t)kEarlyTiles) {
          const int32_t j = j0 + u * kNT + tid;
          s_epp[o] = (int32_t)clamp_page(pt[j], s.n_pool_pages);
          s_epl[o] = min(kPage, L - j * kPage);
          ++o;
          early_bits |= 1u << u;
        }
      __syncthreads();
      const uint32_t ne = min(tot, (uint32_t)kEarlyTiles);
      const int32_t ntok = ne == 0 ? 0 : (int32_t)(ne - 1) * kPage + s_epl[ne - 1];
      for (int32_t e = tid; e < ntok; e += kNT)
        my_list[e] = (uint32_t)(((int64_t)s_epp[e / kPage] * s.Hkv + g) * kPage + (e % kPage));
      __syncthreads();
      n_cur = ntok;
    } else {
      const uint32_t cap = (uint32_t)(kEarlyTiles * TM);
#pragma unroll
      for (int u = 0; u < TPT; ++u)
        if (((sure >> u) & 1u) && o < cap) {
          const int32_t jl = u * kNT + tid;  // j - j0
          my_list[o++] = (uint32_t)(((int64_t)s_pt[jl >> 6] * s.Hkv + g) * kPage + (jl & 63));
          early_bits |= 1u << u;
        }
      __syncthreads();
      n_cur = (int32_t)min(tot, cap);
    }
    run_tiles();
  };

  // ---- 2. threshold by radix levels ----
  const bool topk = a.top_k > 0;
  const float mx = key_score(M);
  if (tid == 0) {
    s_mode = kSearch;
    s_prefix = 0;
    s_thr = 0;
    s_neq = 0;
    s_need = (uint32_t)a.top_k;
    s_rem = 0;
    if (n == 0 || (topk ? (a.top_k >= n) : (a.p >= 1.0f))) s_mode = kGE;
  }
  __syncthreads();
  for (int level = 1; level <= 3; ++level) {
    if (s_mode != kSearch) break;  // same decision in every workgroup of the row
    const int NBIN = level == 3 ? 256 : kBinsF;
    const int NC = NBIN / 64;
    const uint32_t pre = s_prefix;
    const int li = level - 1;
    uint32_t* gc = a.hcnt + ((int64_t)li * rows + row) * kBinsF;
    uint64_t* gm = a.hmass + ((int64_t)li * rows + row) * kBinsF;
    uint32_t* gcc = a.ccnt + ((int64_t)li * rows + row) * kCoarseF;
    uint64_t* gcm = a.cmass + ((int64_t)li * rows + row) * kCoarseF;
    if (level == 1) {
      // every candidate lands in this level: aggregate in LDS, flush the
      // non-empty bins of the coarse groups the own candidates occupy (a
      // 64-bit mask of them; scores of both signs leave wide gaps)
      uint64_t occ = 0;
#pragma unroll
      for (int u = 0; u < TPT; ++u)
        if (j0 + u * kNT + tid < n) occ |= 1ull << (key[u] >> 26);
      const uint32_t occ_lo = wave_allreduce_bits((uint32_t)occ, [](uint32_t x, uint32_t y) { return x | y; });
      const uint32_t occ_hi = wave_allreduce_bits((uint32_t)(occ >> 32), [](uint32_t x, uint32_t y) { return x | y; });
      if (lane == 0) red_u64[wave] = ((uint64_t)occ_hi << 32) | occ_lo;
      __syncthreads();
      const uint64_t occ_all = red_u64[0] | red_u64[1] | red_u64[2] | red_u64[3];
      {
        uint64_t m = occ_all;
        for (int k = 0; m; ++k) {  // the k-th occupied group goes to wave k mod 4
          const int cgz = __ffsll((long long)m) - 1;
          m &= m - 1;
          if ((k & 3) == wave) {
            hcnt_l[cgz * 64 + lane] = 0;
            hmass_l[cgz * 64 + lane] = 0;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int32_t j = j0 + u * kNT + tid;
        if (j >= n) continue;
        const uint32_t digit = key[u] >> 20;
        atomicAdd(&hcnt_l[digit], 1u);
        if (!topk) {
          const float e = __expf(xk[u] - mx);
          atomicAdd((unsigned long long*)&hmass_l[digit], (unsigned long long)(e * 1099511627776.0f));
        }
      }
      __syncthreads();
      stamp(a, 15);
      uint64_t mrem = occ_all;
      for (int k = 0; mrem; ++k) {
        const int cg = __ffsll((long long)mrem) - 1;
        mrem &= mrem - 1;
        if ((k & 3) != wave) continue;
        const int bin = cg * 64 + lane;
        const uint32_t cn = hcnt_l[bin];
        const uint64_t ms = hmass_l[bin];
        // top-p resolves level 1 by mass alone: its counts would only
        // serve the single-candidate shortcut, so they are not sent
        if (cn) {
          if (topk) atomicAdd(&gc[bin], cn);
          else atomicAdd((unsigned long long*)&gm[bin], (unsigned long long)ms);
        }
        const uint32_t csum = wave_sum_u32(cn);
        const uint64_t msum = topk ? 0ull : wave_sum_u64(ms);
        if (lane == 0 && csum) {
          if (topk) atomicAdd(&gcc[cg], csum);
          else atomicAdd((unsigned long long*)&gcm[cg], (unsigned long long)msum);
        }
      }
    } else {
      // only the tokens of the previous level's crossing bin: few, spread
      // over the digits, so they go straight to the row's fine bins; the
      // coarse groups (which all of them share) are summed in LDS first
      if (tid < NC) {
        hcnt_l[tid] = 0;
        hmass_l[tid] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int32_t j = j0 + u * kNT + tid;
        if (j >= n) continue;
        const uint32_t k = key[u];
        const bool match = level == 2 ? (k >> 20) == pre : (k >> 8) == pre;
        if (!match) continue;
        const uint32_t digit = level == 2 ? ((k >> 8) & 0xfffu) : (k & 0xffu);
        atomicAdd(&gc[digit], 1u);
        atomicAdd(&hcnt_l[digit >> 6], 1u);
        if (!topk) {
          const uint64_t e = (uint64_t)(__expf(xk[u] - mx) * 1099511627776.0f);
          atomicAdd((unsigned long long*)&gm[digit], (unsigned long long)e);
          atomicAdd((unsigned long long*)&hmass_l[digit >> 6], (unsigned long long)e);
        }
      }
      __syncthreads();
      if (tid < NC && hcnt_l[tid]) {
        atomicAdd(&gcc[tid], hcnt_l[tid]);
        if (!topk) atomicAdd((unsigned long long*)&gcm[tid], (unsigned long long)hmass_l[tid]);
      }
    }
    stamp(a, 3 * level);
    if (kEarly && level == 2) {
      row_arrive(flags, bi, ++epoch);
      early_attend(pre);
      row_wait(flags, NB, epoch, err);
    } else {
      row_barrier(flags, NB, bi, ++epoch, err);
    }
    stamp(a, 3 * level + 1);
    // resolve (wave 0): coarse groups, then the 64 bins of the crossing group
    if (wave == 0) {
      const int cgi = NC - 1 - lane;
      const uint32_t cc = lane < NC ? __hip_atomic_load(&gcc[cgi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      const uint64_t cm = (!topk && lane < NC) ? __hip_atomic_load(&gcm[cgi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      const uint32_t cinc = wave_incl_scan(cc);
      const uint64_t minc = wave_incl_scan_u64(cm);
      const uint64_t mtot = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(minc >> 32), 63) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)minc, 63);
      uint64_t target = s_rem;
      if (!topk && level == 1) {
        uint64_t tc = (uint64_t)ceil((double)a.p * (double)mtot);
        if (tc < 1) tc = 1;
        if (tc > mtot) tc = mtot;
        target = tc;
      }
      const uint32_t need = s_need;
      const uint32_t cbef = cinc - cc;
      const uint64_t mbef = minc - cm;
      const bool hit = lane < NC && (!topk ? (mbef < target && minc >= target) : (cbef < need && cinc >= need));
      const unsigned long long hb = __ballot(hit);
      int found = -1;
      uint32_t g_cb = 0;
      uint64_t g_mb = 0;
      if (hb) {
        const int src = __ffsll(hb) - 1;
        found = (int)lane_u32((uint32_t)cgi, src);
        g_cb = lane_u32(cbef, src);
        g_mb = lane_u64(mbef, src);
      }
      uint32_t bc = 0;
      uint64_t bm = 0;
      int bin = -1;
      if (found >= 0) {
        bin = found * 64 + 63 - lane;
        bc = __hip_atomic_load(&gc[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bm = !topk ? __hip_atomic_load(&gm[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      }
      const uint32_t binc = wave_incl_scan(bc);
      const uint64_t bminc = wave_incl_scan_u64(bm);
      const uint32_t bcb = g_cb + binc - bc;
      const uint64_t bmb = g_mb + bminc - bm;
      const bool hit2 = found >= 0 && (!topk ? (bmb < target && bmb + bm >= target)
                                             : (bcb < need && bcb + bc >= need));
      const unsigned long long hb2 = __ballot(hit2);
      if (!hb2) {
        if (lane == 0) {
          s_mode = kGE;  // inconsistent histogram (cannot happen): take everything
          s_thr = 0;
        }
      } else if (lane == __ffsll(hb2) - 1) {
        const uint32_t np = level == 1 ? (uint32_t)bin
                                       : (level == 2 ? ((pre << 12) | (uint32_t)bin) : ((pre << 8) | (uint32_t)bin));
        const int shift = level == 1 ? 20 : (level == 2 ? 8 : 0);
        const uint32_t bin_lo = np << shift;
        if (!topk) {
          const uint64_t rem = target - bmb;
          if (level < 3) {
            if (bc == 1 || rem == bm) {
              s_mode = kGE;
              s_thr = bin_lo;
            } else {
              s_prefix = np;
              s_rem = rem;
            }
          } else {
            const uint64_t m1 = bm / bc;
            const uint64_t take = (rem + m1 - 1) / m1;
            s_thr = bin_lo;
            if (take >= bc) {
              s_mode = kGE;
            } else {
              s_mode = kTies;
              s_neq = (uint32_t)take;
            }
          }
        } else {
          const uint32_t nd = need - bcb;
          if (nd == bc) {
            s_mode = kGE;
            s_thr = bin_lo;
          } else if (level < 3) {
            s_prefix = np;
            s_need = nd;
          } else {
            s_mode = kTies;
            s_thr = bin_lo;
            s_neq = nd;
          }
        }
      }
    }
    __syncthreads();
  }

  stamp(a, 11);
  // ---- 3. own selection, attention over it (plus a share of sink/window) ----
  const uint32_t mode = s_mode, thr = s_thr, neq = s_neq;
  uint32_t eq_before = 0;
  if (mode == kTies) {  // ties left out: rank the threshold ties across workgroups
    uint32_t e = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) e += (j0 + u * kNT + tid < n && key[u] == thr) ? 1u : 0u;
    uint32_t tot;
    blk_scan<uint32_t>(e, red_u, tot);
    if (tid == 0) __hip_atomic_store(&a.blk_eq[(int64_t)row * NB + bi], tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    row_barrier(flags, NB, bi, ++epoch, err);
    {
      uint32_t vb = 0;
      for (int k = tid; k < bi; k += kNT)
        vb += __hip_atomic_load(&a.blk_eq[(int64_t)row * NB + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t tb;
      blk_scan<uint32_t>(vb, red_u, tb);
      if (tid == 0) s_cnt = tb;
      __syncthreads();
    }
    eq_before = s_cnt;
  }
  // selection flags in index order (round u, wave, lane) and the own list
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t selmask[TPT];  // bit 0: selected, bit 1: forced
  {
    uint32_t eq_run = eq_before;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      const bool valid = j < n;
      bool top = valid && (mode == kTies ? key[u] > thr : key[u] >= thr);
      if (mode == kTies) {
        const bool eq = valid && key[u] == thr;
        const uint64_t m = __ballot(eq);
        if (lane == 0) s_slice[u * 4 + wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t before = eq_run;
        for (int w = 0; w < wave; ++w) before += s_slice[u * 4 + w];
        uint32_t round_tot = 0;
        for (int w = 0; w < 4; ++w) round_tot += s_slice[u * 4 + w];
        if (eq) top = (before + (uint32_t)__popcll(m & lt_mask)) < neq;
        eq_run += round_tot;
        __syncthreads();
      }
      const bool forced = valid && (j < a.n_sink || j >= n - a.n_window);
      selmask[u] = (top || forced ? 1u : 0u) | (forced ? 2u : 0u);
    }
  }
  if constexpr (PAGES) {
    // own selected pages in index order; each expands to its tokens (all 64
    // but the sequence's last page, which is also the last in this order).
    // A workgroup attends its own pages (those not attended early) and
    // publishes its token count for the ordered list.
    uint32_t run = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int32_t j = j0 + u * kNT + tid;
      const bool sel = selmask[u] & 1u;
      const uint64_t m = __ballot(sel);
      if (lane == 0) s_slice[u * 4 + wave] = (uint32_t)__popcll(m);
      __syncthreads();
      uint32_t before = run;
      for (int w = 0; w < wave; ++w) before += s_slice[u * 4 + w];
      uint32_t round_tot = 0;
      for (int w = 0; w < 4; ++w) round_tot += s_slice[u * 4 + w];
      if (sel) {
        const uint32_t k = before + (uint32_t)__popcll(m & lt_mask);
        if (k < (uint32_t)kFusedMaxPages) {  // at most top_k <= kFusedMaxPages pages per row
          s_spj[k] = j;
          s_spp[k] = (int32_t)clamp_page(pt[j], s.n_pool_pages);
          s_spe[k] = (early_bits >> u) & 1u;
        }
      }
      run += round_tot;
      __syncthreads();
    }
    const uint32_t np = run < (uint32_t)kFusedMaxPages ? run : (uint32_t)kFusedMaxPages;
    if (tid == 0) {
      // tokens of the own pages (output) and of those left to attend
      uint32_t na = 0;
      for (uint32_t k = 0; k < np; ++k)
        if (!s_spe[k]) s_spa[na++] = s_spp[k];
      const uint32_t last = np == 0 ? 0u : (uint32_t)min(kPage, L - s_spj[np - 1] * kPage);
      const uint32_t tok_out = np == 0 ? 0u : (np - 1) * kPage + last;
      s_np = np;
      s_cnt = na == 0 ? 0u : (na - 1) * kPage + (s_spe[np - 1] ? (uint32_t)kPage : last);
      __hip_atomic_store(&a.blk_sel[(int64_t)row * NB + bi], tok_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    for (uint32_t e = tid; e < s_cnt; e += kNT)
      my_list[e] = (uint32_t)(((int64_t)s_spa[e / kPage] * s.Hkv + g) * kPage + (e % kPage));
    __syncthreads();
  } else if constexpr (SEL) {
    // the own selected count, for the ordered list
    uint32_t my_sel = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) my_sel += selmask[u] & 1u;
    uint32_t tot_sel;
    blk_scan<uint32_t>(my_sel, red_u, tot_sel);
    if (tid == 0) __hip_atomic_store(&a.blk_sel[(int64_t)row * NB + bi], tot_sel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
  // own non-forced selected tokens -> LDS list (order irrelevant for attention)
  uint32_t my_sel = 0;
  {
    uint32_t cnt_nf = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      my_sel += selmask[u] & 1u;
      cnt_nf += (selmask[u] == 1u && !((early_bits >> u) & 1u)) ? 1u : 0u;  // (not attended early)
    }
    uint32_t tot_nf;
    const uint32_t off = blk_scan<uint32_t>(cnt_nf, red_u, tot_nf);
    uint32_t o = off;
#pragma unroll
    for (int u = 0; u < TPT; ++u)
      if (selmask[u] == 1u && !((early_bits >> u) & 1u)) {
        const int32_t jl = u * kNT + tid;  // j - j0
        my_list[o++] = (uint32_t)(((int64_t)s_pt[jl >> 6] * s.Hkv + g) * kPage + (jl & 63));
      }
    uint32_t tot_sel;
    blk_scan<uint32_t>(my_sel, red_u, tot_sel);
    // share of the forced tokens: the union of [0, n_sink) and
    // [n - n_window, n), enumerated in index order and split evenly
    const int32_t s_end = min(a.n_sink, n);
    const int32_t w_beg = max(s_end, n - a.n_window);
    const int32_t nf = s_end + (n - w_beg);
    const int32_t f0 = (int32_t)(((int64_t)nf * bi) / NB), f1 = (int32_t)(((int64_t)nf * (bi + 1)) / NB);
    for (int32_t f = f0 + tid; f < f1; f += kNT) {
      const int32_t j = f < s_end ? f : w_beg + (f - s_end);
      const int64_t page = clamp_page(pt[j >> 6], s.n_pool_pages);
      my_list[tot_nf + (f - f0)] = (uint32_t)((page * s.Hkv + g) * kPage + (j & 63));
    }
    if (tid == 0) {
      s_cnt = tot_nf + (uint32_t)(f1 - f0);
      __hip_atomic_store(&a.blk_sel[(int64_t)row * NB + bi], tot_sel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
  }
  stamp(a, 5);
  if constexpr (!SEL) {
  const int32_t n_att = (int32_t)s_cnt;
    if constexpr (sizeof(T) == 2) {
    n_cur = n_att;
    run_tiles();
    stamp(a, 8);
    // merge the waves: lane (lg, hq) holds O^T[16 mb + 4 lg + v][hq]
    float lw = l_run;
    lw += __shfl_xor(lw, 16, 64);
    lw += __shfl_xor(lw, 32, 64);
    __syncthreads();  // the tile buffers are free
    float* ob = reinterpret_cast<float*>(wave < 2 ? Ks : Vs) + (wave & 1) * D * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v) ob[(16 * mb + 4 * lg + v) * 16 + hq] = oacc[mb][v];
    if (lane < 16) {
      s_wm[wave][lane] = m_run;
      s_wl[wave][lane] = lw;
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += kNT) {
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
      const int64_t pi = ((int64_t)row * NB + bi) * G + hl;
      st_dev(&a.part_o[pi * D + d], osum);
      if (d == 0) {
        st_dev(&a.part_ml[pi * 2], M);
        st_dev(&a.part_ml[pi * 2 + 1], lsum);
      }
    }
    if constexpr (RLA) {
      // the residual sums of the four waves, once the outputs are merged:
      // numerators through the same LDS, denominators summed over the lane rows
      __shared__ float s_rd[4][16];
      static_assert(4 * D * 16 * 4 <= (int)sizeof(lds_big), "four waves' residual sums fit");
      float* rbuf = reinterpret_cast<float*>(lds_big);
      float rd = rden;
      rd += __shfl_xor(rd, 16, 64);
      rd += __shfl_xor(rd, 32, 64);
      __syncthreads();  // the outputs' merge is done with the buffer
      float* rb = rbuf + wave * D * 16;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) rb[(16 * mb + 4 * lg + v) * 16 + hq] = racc[mb][v];
      if (lane < 16) s_rd[wave][lane] = rd;
      __syncthreads();
      for (int e = tid; e < G * D; e += kNT) {
        const int hl = e / D, d = e % D;
        const int64_t pi = ((int64_t)row * NB + bi) * G + hl;
        float rn = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) rn += rbuf[w * D * 16 + d * 16 + hl];
        st_dev(&a.part_rnum[pi * D + d], rn);
        if (d == 0) st_dev(&a.part_rden[pi], (s_rd[0][hl] + s_rd[1][hl]) + (s_rd[2][hl] + s_rd[3][hl]));
      }
    }
    } else {
    float m_run[HPW], l_run[HPW], acc[HPW][DPL];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.f;
    }
    // K/V rows of two tiles in flight: the tile being staged and the next
    uint4 kA[LPT], vA[LPT], kB[LPT], vB[LPT];
    auto gather = [&](int32_t ts, uint4 (&kr)[LPT], uint4 (&vr)[LPT]) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int pc = i * kNT + tid;
        const int r = pc / CPR, col = pc % CPR;
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
        if (ts + r < n_att) {
          const int64_t off = (int64_t)my_list[ts + r] * D;
          kr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(k_pool + off) + col * 16);
          vr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(v_pool + off) + col * 16);
        }
      }
    };
    auto tile = [&](int32_t ts, uint4 (&kr)[LPT], uint4 (&vr)[LPT]) {
      const int32_t nt = min(kTileF, n_att - ts);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int pc = i * kNT + tid;
        const int r = pc / CPR, col = pc % CPR;
        *reinterpret_cast<uint4*>(Ks + r * PITCH + col * 16) = kr[i];
        *reinterpret_cast<uint4*>(Vs + r * PITCH + col * 16) = vr[i];
      }
      __syncthreads();
      if (ts + 2 * kTileF < n_att) gather(ts + 2 * kTileF, kr, vr);
      float sc[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) sc[hh] = 0.f;
      const char* krow = Ks + lane * PITCH;
#pragma unroll 4
      for (int pc = 0; pc < CPR; ++pc) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + pc * 16);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const int h = wave * HPW + hh;
          if constexpr (sizeof(T) == 2) {
            const uint4 qv = *reinterpret_cast<const uint4*>(&Qs[h][pc * 8]);
            float t = sc[hh];
            t = dot2(kv.x, qv.x, t);
            t = dot2(kv.y, qv.y, t);
            t = dot2(kv.z, qv.z, t);
            t = dot2(kv.w, qv.w, t);
            sc[hh] = t;
          } else {
            const float4 qv = *reinterpret_cast<const float4*>(&Qs[h][pc * 4]);
            float t = sc[hh];
            t = fmaf(__uint_as_float(kv.x), qv.x, t);
            t = fmaf(__uint_as_float(kv.y), qv.y, t);
            t = fmaf(__uint_as_float(kv.z), qv.z, t);
            t = fmaf(__uint_as_float(kv.w), qv.w, t);
            sc[hh] = t;
          }
        }
      }
      float alpha[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const float sv = lane < nt ? sc[hh] * a.s_att : -INFINITY;
        const float mt = wave_max(sv);
        const float m_new = fmaxf(m_run[hh], mt);
        const float pv = lane < nt ? __expf(sv - m_new) : 0.f;
        const float lt = wave_sum(pv);
        alpha[hh] = __expf(m_run[hh] - m_new);
        l_run[hh] = l_run[hh] * alpha[hh] + lt;
        m_run[hh] = m_new;
        Ps[wave * HPW + hh][lane] = pv;
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[hh][e] *= alpha[hh];
      for (int t = 0; t < kTileF; t += 4) {
        float4 pv4[HPW];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) pv4[hh] = *reinterpret_cast<const float4*>(&Ps[wave * HPW + hh][t]);
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          float vv[DPL];
          const char* vrow = Vs + (t + uu) * PITCH;
          if constexpr (sizeof(T) == 2) {
            if constexpr (DPL == 2) {
              const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + lane * 4);
              vv[0] = __uint_as_float(w << 16);
              vv[1] = __uint_as_float(w & 0xffff0000u);
            } else {
              const uint16_t w = *reinterpret_cast<const uint16_t*>(vrow + lane * 2);
              vv[0] = __uint_as_float((uint32_t)w << 16);
            }
          } else {
#pragma unroll
            for (int e = 0; e < DPL; ++e) vv[e] = *reinterpret_cast<const float*>(vrow + (lane * DPL + e) * 4);
          }
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh) {
            const float pp = uu == 0 ? pv4[hh].x : (uu == 1 ? pv4[hh].y : (uu == 2 ? pv4[hh].z : pv4[hh].w));
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[hh][e] = fmaf(pp, vv[e], acc[hh][e]);
          }
        }
      }
    };
    if (n_att > 0) gather(0, kA, vA);
    if (n_att > kTileF) gather(kTileF, kB, vB);
    for (int32_t ts = 0; ts < n_att; ts += 2 * kTileF) {
      tile(ts, kA, vA);
      if (ts + kTileF < n_att) tile(ts + kTileF, kB, vB);
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int hl = wave * HPW + hh;
      const int64_t pi = ((int64_t)row * NB + bi) * G + hl;
      if (lane == 0) {
        st_dev(&a.part_ml[pi * 2], m_run[hh]);
        st_dev(&a.part_ml[pi * 2 + 1], l_run[hh]);
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) st_dev(&a.part_o[pi * D + lane * DPL + e], acc[hh][e]);
    }
    }
  }
  stamp(a, 12);
  row_barrier(flags, NB, bi, ++epoch, err);
  stamp(a, 13);
  // no workgroup reads the row's histograms after the last barrier: return
  // this workgroup's slice of them to zero for the next launch
  {
    const int per = (kBinsF + NB - 1) / NB;
    for (int li = 0; li < 3; ++li) {
      uint32_t* gc = a.hcnt + ((int64_t)li * rows + row) * kBinsF;
      uint64_t* gm = a.hmass + ((int64_t)li * rows + row) * kBinsF;
      for (int i = bi * per + tid; i < min(kBinsF, (bi + 1) * per); i += kNT) {
        gc[i] = 0;
        gm[i] = 0;
      }
      if (bi == 0 && tid < kCoarseF) {
        a.ccnt[((int64_t)li * rows + row) * kCoarseF + tid] = 0;
        a.cmass[((int64_t)li * rows + row) * kCoarseF + tid] = 0;
      }
    }
  }

  // ---- 4. merge of this workgroup's output slice and the ordered index list ----
  {
    // the workgroups' selected counts, loaded now and used after the merge
    // (so their round trip overlaps the partials')
    uint32_t bsel = 0;
    if (tid < NB) bsel = __hip_atomic_load(&a.blk_sel[(int64_t)row * NB + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (!SEL) {
    // outputs [bi * opb, (bi + 1) * opb) of the row's G * D values
    const int n_out = G * D;
    const int opb = (n_out + NB - 1) / NB;
    const int o0 = bi * opb;
    const int lim = min(n_out, o0 + opb);
    for (int ob = o0; ob < lim; ob += kNT / 16) {
      // 16 threads per output, each taking every 16th partial
      const int oo = ob + tid / 16;
      const int sub = tid % 16;
      if (oo >= lim) continue;  // whole 16-lane groups skip together
      const int hl = oo / D, d = oo % D;
      // every partial this lane merges, loaded in one round trip
      constexpr int KP = kMaxNB / 16;
      float pm[KP], pl[KP], po[KP];
#pragma unroll
      for (int t = 0; t < KP; ++t) {
        const int k = sub + 16 * t;
        pm[t] = -INFINITY;
        pl[t] = 0.f;
        po[t] = 0.f;
        if (k < NB) {
          const int64_t pi = ((int64_t)row * NB + k) * G + hl;
          pm[t] = ld_dev(&a.part_ml[pi * 2]);
          pl[t] = ld_dev(&a.part_ml[pi * 2 + 1]);
          po[t] = ld_dev(&a.part_o[pi * D + d]);
        }
      }
      // residual linear attention (subtraction form): phi(q_h) . S[:, d]
      // over the state rows sub, sub + 16, ... minus the workgroups' sums
      constexpr int KR = D / 16;
      float pr[KP], sv[KR];
      if constexpr (RLA) {
        const float* st = a.rla_state + (int64_t)row * (D + 1) * D;
#pragma unroll
        for (int t = 0; t < KP; ++t) {
          const int k = sub + 16 * t;
          pr[t] = k < NB ? ld_dev(&a.part_rnum[(((int64_t)row * NB + k) * G + hl) * D + d]) : 0.f;
        }
#pragma unroll
        for (int t = 0; t < KR; ++t) sv[t] = st[(int64_t)(sub + 16 * t) * D + d];
      }
      float M2 = -INFINITY;
#pragma unroll
      for (int t = 0; t < KP; ++t) M2 = fmaxf(M2, pm[t]);
      M2 = row16_max(M2);
      float lsum = 0.f, osum = 0.f;
#pragma unroll
      for (int t = 0; t < KP; ++t) {
        if (sub + 16 * t >= NB) break;
        const float wgt = pm[t] == -INFINITY ? 0.f : __expf(pm[t] - M2);
        lsum += pl[t] * wgt;
        osum += po[t] * wgt;
      }
      lsum = row16_sum(lsum);
      osum = row16_sum(osum);
      if (sub == 0) {
        const int h = g * G + hl;
        const float v = lsum > 0.f ? osum / lsum : 0.f;
        if (a.out_bf16) ((bf16_raw*)a.out)[((int64_t)b * s.Hq + h) * D + d] = f32_to_bf16(v);
        else ((float*)a.out)[((int64_t)b * s.Hq + h) * D + d] = v;
        if (d == 0 && a.lse) a.lse[(int64_t)b * s.Hq + h] = lsum > 0.f ? M2 + logf(lsum) : -INFINITY;
      }
      if constexpr (RLA) {
        const int h = g * G + hl;
        float lin = 0.f, sel = 0.f;
#pragma unroll
        for (int t = 0; t < KR; ++t) lin = fmaf(__expf(to_f32<T>(Qs[hl][sub + 16 * t])), sv[t], lin);
#pragma unroll
        for (int t = 0; t < KP; ++t) sel += pr[t];
        lin = row16_sum(lin);
        sel = row16_sum(sel);
        if (sub == 0) a.rla_num[((int64_t)b * s.Hq + h) * D + d] = lin - sel;
        if (d == 0) {  // the denominator: phi(q_h) . z (state row D) minus the sums
          const float* z = a.rla_state + ((int64_t)row * (D + 1) + D) * D;
          float lz = 0.f, sz = 0.f;
#pragma unroll
          for (int t = 0; t < KR; ++t) lz = fmaf(__expf(to_f32<T>(Qs[hl][sub + 16 * t])), z[sub + 16 * t], lz);
#pragma unroll
          for (int t = 0; t < KP; ++t) {
            const int k = sub + 16 * t;
            if (k < NB) sz += ld_dev(&a.part_rden[((int64_t)row * NB + k) * G + hl]);
          }
          lz = row16_sum(lz);
          sz = row16_sum(sz);
          if (sub == 0) a.rla_den[(int64_t)b * s.Hq + h] = lz - sz;
        }
      }
    }
    }
    {
      const uint32_t vt = bsel, vb = tid < bi ? bsel : 0u;
      uint32_t tb, tt;
      blk_scan<uint32_t>(vb, red_u, tb);
      blk_scan<uint32_t>(vt, red_u, tt);
      if (tid == 0) {
        s_base = tb;
        s_total = tt;
      }
      __syncthreads();
    }
    int32_t* outl = a.idx + (int64_t)row * a.cap;
    if constexpr (PAGES) {
      // the own pages' tokens, in index order, after the lower workgroups'
      const uint32_t np = s_np;
      const uint32_t tok_out = np == 0 ? 0u
          : (np - 1) * kPage + (uint32_t)min(kPage, L - s_spj[np - 1] * kPage);
      for (uint32_t e = tid; e < tok_out; e += kNT) {
        const uint32_t pos = s_base + e;
        if (pos < (uint32_t)a.cap) outl[pos] = s_spj[e / kPage] * kPage + (int32_t)(e % kPage);
      }
    } else {
    // every round's per-wave counts first, so one barrier serves all rounds
    uint64_t msk[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      msk[u] = __ballot(selmask[u] & 1u);
      if (lane == 0) s_slice[u * 4 + wave] = (uint32_t)__popcll(msk[u]);
    }
    __syncthreads();
    uint32_t run = s_base;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      uint32_t before = run;
      for (int w = 0; w < wave; ++w) before += s_slice[u * 4 + w];
      uint32_t round_tot = 0;
      for (int w = 0; w < 4; ++w) round_tot += s_slice[u * 4 + w];
      if (selmask[u] & 1u) {
        const uint32_t pos = before + (uint32_t)__popcll(msk[u] & lt_mask);
        if (pos < (uint32_t)a.cap) outl[pos] = j0 + u * kNT + tid;
      }
      run += round_tot;
    }
    }
    const uint32_t total = s_total < (uint32_t)a.cap ? s_total : (uint32_t)a.cap;
    const int64_t pad = (int64_t)a.cap - total;
    const int64_t p0 = total + (pad * bi) / NB, p1 = total + (pad * (bi + 1)) / NB;
    for (int64_t o = p0 + tid; o < p1; o += kNT) outl[o] = -1;
  }

  stamp(a, 14);
  // ---- exit: the last workgroup of the row to leave writes the row's count
  // (-1 if any barrier of the row gave up, so a caller sees the failure) and
  // returns the barrier flags, the error word and the exit counter to zero
  // for the next launch (the histograms were zeroed after the last barrier) ----
  {
    __syncthreads();
    if (tid == 0) {
      // this workgroup's error report completes before its exit is counted
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const uint32_t old = atomicAdd(&ctl->exit, 1u);
      if (old == (uint32_t)NB - 1) {  // every workgroup of the row has left its barriers
        const uint32_t failed = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.count[row] = failed ? -1 : (int32_t)(s_total < (uint32_t)a.cap ? s_total : (uint32_t)a.cap);
        for (int k = 0; k < NB; ++k) {
          flags[k] = 0;
          a.mflag[(int64_t)row * kMaxNB + k] = 0;
        }
        *err = 0;
        ctl->exit = 0;
      }
    }
  }
}

}  // namespace

// Workspace of the fused step, in two parts.  The zero part holds what must
// be zero when a launch starts and is zero again when it ends (row control
// words, level histograms, barrier flags); it is laid out for rows_cap rows
// and a launch uses the first rows of it, so its offsets do not depend on
// the launch's shape.  The data part (counts, partial outputs,
// phase stamps) is written before it is read.
size_t fused_zero_bytes(int32_t rows_cap) {
  size_t b = 0;
  b += align_up(sizeof(RowWs) * rows_cap, 256);
  b += align_up(sizeof(uint32_t) * 3 * rows_cap * kBinsF, 256);
  b += align_up(sizeof(uint64_t) * 3 * rows_cap * kBinsF, 256);
  b += align_up(sizeof(uint32_t) * 3 * rows_cap * kCoarseF, 256);
  b += align_up(sizeof(uint64_t) * 3 * rows_cap * kCoarseF, 256);
  b += align_up(sizeof(uint32_t) * rows_cap * kMaxNB, 256);
  b += align_up(sizeof(uint64_t) * rows_cap * kMaxNB, 256);
  return b;
}

namespace {

size_t fused_data_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D) {
  size_t b = 0;
  b += 2 * align_up(sizeof(uint32_t) * rows * nb, 256);
  b += align_up(sizeof(float) * rows * nb * G * 2, 256);
  b += align_up(sizeof(float) * rows * nb * G * D, 256);
  b += align_up(sizeof(uint64_t) * rows * nb * kTraceSlots, 256);
  return b;
}

}  // namespace

// Workspace of the fused step; rows * nb workgroups, G heads, D dims: the
// zero part for these rows, then the data part.
size_t fused_workspace_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D) {
  return fused_zero_bytes(rows) + fused_data_bytes(rows, nb, G, D);
}

size_t fused_rla_bytes(int32_t rows, int32_t nb, int32_t G, int32_t D) {
  return align_up(sizeof(float) * rows * nb * G * D, 256) + align_up(sizeof(float) * rows * nb * G, 256);
}

namespace {

// The kernel instance a plan launches (mode 0: token step, 1: page step,
// 2: selection only, 3: token step with the residual linear attention).
template <typename T, int D, int G, bool PAGES, bool SEL, bool RLA = false>
const void* fused_instance(int tpt) {
  switch (tpt) {
    case 1: return (const void*)k_decode_fused<T, D, G, 1, PAGES, SEL, RLA>;
    case 2: return (const void*)k_decode_fused<T, D, G, 2, PAGES, SEL, RLA>;
    case 4: return (const void*)k_decode_fused<T, D, G, 4, PAGES, SEL, RLA>;
    case 8: return (const void*)k_decode_fused<T, D, G, 8, PAGES, SEL, RLA>;
    default: return (const void*)k_decode_fused<T, D, G, 16, PAGES, SEL, RLA>;
  }
}

template <typename T, int D, bool PAGES, bool RLA = false>
const void* fused_instance_g(int G, int tpt) {
  switch (G) {
    case 4: return fused_instance<T, D, 4, PAGES, false, RLA>(tpt);
    case 8: return fused_instance<T, D, 8, PAGES, false, RLA>(tpt);
    default: return fused_instance<T, D, 16, PAGES, false, RLA>(tpt);
  }
}

const void* fused_kernel_for(sa_dtype dt, int D, int G, int tpt, int mode) {
  if (mode == 2) return fused_instance<float, 64, 4, false, true>(tpt);
  if (mode == 3) return D == 128 ? fused_instance_g<bf16_raw, 128, false, true>(G, tpt)
                                 : fused_instance_g<bf16_raw, 64, false, true>(G, tpt);
  if (mode == 1) return D == 128 ? fused_instance_g<bf16_raw, 128, true>(G, tpt)
                                 : fused_instance_g<bf16_raw, 64, true>(G, tpt);
  if (dt == SA_BF16) return D == 128 ? fused_instance_g<bf16_raw, 128, false>(G, tpt)
                                     : fused_instance_g<bf16_raw, 64, false>(G, tpt);
  return D == 128 ? fused_instance_g<float, 128, false>(G, tpt) : fused_instance_g<float, 64, false>(G, tpt);
}

// How many workgroups of the kernel fit a compute unit at once (registers
// and LDS): every workgroup of a persistent launch must be resident at the
// same time.  Cached per kernel instance and device.
int fused_resident(const void* fn, int dev) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(fn, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nblk = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, fn, kNT, 0) != hipSuccess) nblk = 0;
  cache[key] = nblk;
  return nblk;
}

}  // namespace

// Plan: workgroups per row and tokens per workgroup, or false if the fused
// step does not apply (too many rows, rows too long, group size < 4, or a
// workgroup of the instance would not fit a compute unit).
bool fused_plan(const Shape& s, int32_t n_sink, int32_t n_window, sa_dtype dt, int mode,
                int32_t* nb, int32_t* tpb) {
  const int rows = s.B * s.Hkv;
  const int G = s.Hq / s.Hkv;
  if (G < 4 || rows > kFusedMaxRows || s.max_len < 1) return false;
  // attention lists hold pool token rows as 32-bit values
  if ((double)s.n_pool_pages * s.Hkv * kPage >= 4294967296.0) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  // one workgroup per compute unit (two per unit hide the gathers' latency
  // better but make every barrier of the row slower by more than the
  // attention gains); every workgroup of the launch must be resident at once
  int n_b = cus / rows;
  if (n_b > kMaxNB) n_b = kMaxNB;
  if (n_b < 1) return false;
  // tokens per workgroup: a power-of-two number of kNT rounds, at most 16
  const int32_t per = (s.max_len + n_b - 1) / n_b;
  int32_t rounds = 1;
  while (rounds * kNT < per) rounds *= 2;
  if (rounds > 16) return false;
  // each workgroup's share of the sink/window tokens must fit its list
  const int64_t forced = (int64_t)n_sink + n_window;
  if ((forced + n_b - 1) / n_b > 64) return false;
  if (fused_resident(fused_kernel_for(dt, s.D, G, rounds, mode), dev) < 1) return false;
  *nb = n_b;
  *tpb = rounds * kNT;
  return true;
}

// Plan of the page-level step: the candidates are the ceil(max_len / 64)
// pages, at most kFusedMaxPages of them selected.
bool fused_plan_pages(const Shape& s, int32_t top_k, int32_t* nb, int32_t* tpb) {
  if (top_k < 1 || top_k > kFusedMaxPages) return false;
  Shape sp = s;
  sp.max_len = (s.max_len + kPage - 1) / kPage;
  return fused_plan(sp, 0, 0, SA_BF16, 1, nb, tpb);
}

namespace {

// Carves the workspace laid out by fused_workspace_bytes.  zero: the zero
// part to use instead of the one at the front of ws (laid out for
// kFusedMaxRows rows), or NULL.
void fused_ws(FusedArgs& a, void* ws, void* zero, int rows, int nb, int G, int D) {
  const int rows_cap = zero ? kFusedMaxRows : rows;
  char* z = zero ? (char*)zero : (char*)ws;
  a.ctl = (RowWs*)z;            z += align_up(sizeof(RowWs) * rows_cap, 256);
  a.hcnt = (uint32_t*)z;        z += align_up(sizeof(uint32_t) * 3 * rows_cap * kBinsF, 256);
  a.hmass = (uint64_t*)z;       z += align_up(sizeof(uint64_t) * 3 * rows_cap * kBinsF, 256);
  a.ccnt = (uint32_t*)z;        z += align_up(sizeof(uint32_t) * 3 * rows_cap * kCoarseF, 256);
  a.cmass = (uint64_t*)z;       z += align_up(sizeof(uint64_t) * 3 * rows_cap * kCoarseF, 256);
  a.flags = (uint32_t*)z;       z += align_up(sizeof(uint32_t) * rows_cap * kMaxNB, 256);
  a.mflag = (uint64_t*)z;
  char* w = (char*)ws + fused_zero_bytes(rows);
  a.blk_sel = (uint32_t*)w;     w += align_up(sizeof(uint32_t) * rows * nb, 256);
  a.blk_eq = (uint32_t*)w;      w += align_up(sizeof(uint32_t) * rows * nb, 256);
  a.part_ml = (float*)w;        w += align_up(sizeof(float) * rows * nb * G * 2, 256);
  a.part_o = (float*)w;         w += align_up(sizeof(float) * rows * nb * G * D, 256);
  a.trace = (uint64_t*)w;
}

}  // namespace

hipError_t launch_decode_fused_pages(const Shape& s, const sa_pages& pg, const void* q,
                                     const void* stats_pool, const void* k_pool, const void* v_pool,
                                     float s_att, int32_t top_k, float* x, int64_t ldx,
                                     int32_t* idx, int32_t* count, int32_t cap, void* out,
                                     sa_dtype out_dt, float* lse, void* ws, void* zero, int32_t nb,
                                     int32_t tpb, hipStream_t st) {
  const int rows = s.B * s.Hkv;
  const int G = s.Hq / s.Hkv;
  FusedArgs a{};
  a.q = q; a.stats = stats_pool; a.k_pool = k_pool; a.v_pool = v_pool;
  a.page_table = pg.page_table; a.seq_lens = pg.seq_lens; a.s = s;
  a.s_att = s_att; a.p = 0.f; a.top_k = top_k; a.n_sink = 0; a.n_window = 0;
  a.x = x; a.ldx = ldx; a.idx = idx; a.count = count; a.cap = cap;
  a.out = out; a.out_bf16 = out_dt == SA_BF16; a.lse = lse; a.nb = nb; a.tpb = tpb;
  fused_ws(a, ws, zero, rows, nb, G, s.D);
  const int tpt = tpb / kNT;
  dim3 grid(rows * nb);
#define SA_FP(DD, GG, PP) k_decode_fused<bf16_raw, DD, GG, PP, true, false><<<grid, kNT, 0, st>>>(a)
#define SA_FP_T(DD, GG)                  \
  switch (tpt) {                         \
    case 1: SA_FP(DD, GG, 1); break;     \
    case 2: SA_FP(DD, GG, 2); break;     \
    case 4: SA_FP(DD, GG, 4); break;     \
    case 8: SA_FP(DD, GG, 8); break;     \
    default: SA_FP(DD, GG, 16); break;   \
  }
#define SA_FP_G(DD)                      \
  switch (G) {                           \
    case 4: SA_FP_T(DD, 4); break;       \
    case 8: SA_FP_T(DD, 8); break;       \
    default: SA_FP_T(DD, 16); break;     \
  }
  if (s.D == 128) { SA_FP_G(128); } else { SA_FP_G(64); }
#undef SA_FP_G
#undef SA_FP_T
#undef SA_FP
  return hipGetLastError();
}

// Selection only over given scores (unit 1, few long rows) in one persistent
// launch: the same levels, ties and ordered list as the fused step.
bool select_fused_plan(const SelectArgs& sa, int32_t* nb, int32_t* tpb) {
  if (sa.unit != 1 || sa.key16 || sa.prefill_bsel != 0 || sa.Hkv < 1 || sa.rows % sa.Hkv != 0) return false;
  Shape s{};
  s.B = sa.rows / sa.Hkv;
  s.Hkv = sa.Hkv;
  s.Hq = 4 * sa.Hkv;  // (the group size plays no part in selection)
  s.D = 64;
  s.max_len = sa.max_len;
  s.n_pool_pages = 1;
  return fused_plan(s, sa.n_sink, sa.n_window, SA_F32, 2, nb, tpb);
}

hipError_t launch_select_fused(const SelectArgs& sa, void* ws, int32_t nb, int32_t tpb,
                               hipStream_t st) {
  FusedArgs a{};
  a.s.B = sa.rows / sa.Hkv;
  a.s.Hkv = sa.Hkv;
  a.s.Hq = 4 * sa.Hkv;
  a.s.max_len = sa.max_len;
  a.seq_lens = sa.seq_lens;
  a.p = sa.p;
  a.top_k = sa.is_topk ? sa.k : 0;
  a.n_sink = sa.n_sink;
  a.n_window = sa.n_window;
  a.x = const_cast<float*>(sa.x);
  a.ldx = sa.ldx;
  a.idx = sa.idx;
  a.count = sa.count;
  a.cap = sa.cap;
  a.nb = nb;
  a.tpb = tpb;
  fused_ws(a, ws, sa.fused_zero, sa.rows, nb, 1, 0);
  dim3 grid(sa.rows * nb);
#define SA_FS(PP) k_decode_fused<float, 64, 4, PP, false, true><<<grid, kNT, 0, st>>>(a)
  switch (tpb / kNT) {
    case 1: SA_FS(1); break;
    case 2: SA_FS(2); break;
    case 4: SA_FS(4); break;
    case 8: SA_FS(8); break;
    default: SA_FS(16); break;
  }
#undef SA_FS
  return hipGetLastError();
}

hipError_t launch_decode_fused(const Shape& s, const sa_pages& pg, const void* q, const void* w_q,
                               const void* kidx_pool, const void* k_pool, const void* v_pool,
                               sa_dtype dt, float s_idx, float s_att, float p, int32_t top_k,
                               int32_t n_sink, int32_t n_window, float* x, int64_t ldx,
                               int32_t* idx, int32_t* count, int32_t cap, void* out,
                               sa_dtype out_dt, float* lse, void* ws, void* zero, int32_t nb,
                               int32_t tpb, const FusedRla* rla, hipStream_t st) {
  const int rows = s.B * s.Hkv;
  const int G = s.Hq / s.Hkv;
  // the residual linear attention rides on the matrix-core attention (bf16)
  if (rla && dt != SA_BF16) return hipErrorNotSupported;
  FusedArgs a{};
  a.q = q; a.w_q = w_q; a.kidx = kidx_pool; a.k_pool = k_pool; a.v_pool = v_pool;
  a.page_table = pg.page_table; a.seq_lens = pg.seq_lens; a.s = s;
  a.s_idx = s_idx; a.s_att = s_att; a.p = p; a.top_k = top_k; a.n_sink = n_sink;
  a.n_window = n_window; a.x = x; a.ldx = ldx; a.idx = idx; a.count = count; a.cap = cap;
  a.out = out; a.out_bf16 = out_dt == SA_BF16; a.lse = lse; a.nb = nb; a.tpb = tpb;
  fused_ws(a, ws, zero, rows, nb, G, s.D);
  if (rla) {
    a.rla_state = rla->state;
    a.rla_num = rla->num;
    a.rla_den = rla->den;
    a.part_rnum = (float*)rla->part;
    a.part_rden = (float*)((char*)rla->part + align_up(sizeof(float) * rows * nb * G * s.D, 256));
  }
  const int tpt = tpb / kNT;  // 1, 2, 4, 8 or 16 (fused_plan)
  dim3 grid(rows * nb);
#define SA_FZ(TT, DD, GG, PP)                                                         \
  do {                                                                                \
    if (rla) k_decode_fused<bf16_raw, DD, GG, PP, false, false, true><<<grid, kNT, 0, st>>>(a); \
    else k_decode_fused<TT, DD, GG, PP, false, false><<<grid, kNT, 0, st>>>(a);      \
  } while (0)
#define SA_FZ_T(TT, DD, GG)              \
  switch (tpt) {                         \
    case 1: SA_FZ(TT, DD, GG, 1); break;  \
    case 2: SA_FZ(TT, DD, GG, 2); break;  \
    case 4: SA_FZ(TT, DD, GG, 4); break;  \
    case 8: SA_FZ(TT, DD, GG, 8); break;  \
    default: SA_FZ(TT, DD, GG, 16); break; \
  }
#define SA_FZ_G(TT, DD)                       \
  switch (G) {                                \
    case 4: SA_FZ_T(TT, DD, 4); break;        \
    case 8: SA_FZ_T(TT, DD, 8); break;        \
    default: SA_FZ_T(TT, DD, 16); break;      \
  }
  if (dt == SA_BF16) {
    if (s.D == 128) { SA_FZ_G(bf16_raw, 128); } else { SA_FZ_G(bf16_raw, 64); }
  } else {  // (no residual terms: checked above)
    if (s.D == 128) { SA_FZ_G(float, 128); } else { SA_FZ_G(float, 64); }
  }
#undef SA_FZ_G
#undef SA_FZ_T
#undef SA_FZ
  return hipGetLastError();
}

}  // namespace sa
