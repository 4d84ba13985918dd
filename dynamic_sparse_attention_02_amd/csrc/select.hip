// Sort-free support selection by a radix histogram over order-preserving keys
// of the fp32 scores ("Full Attention Strikes Back", method section 5: a
// histogram threshold instead of a sort; section 3: dynamic top-p by attention
// mass, or static top-k).
//
// Rows (one per (sequence, key/value group)) are split into chunks of kChunk
// candidates, one block per chunk.  A key is the score's bit pattern mapped so
// that unsigned order equals float order; it is resolved 12 + 12 + 8 bits at a
// time.  Each level builds a per-block LDS histogram of the current digit
// (count, and for top-p the mass exp(x - max) in 2^-40 fixed point, so sums are
// exact integers whatever the order of the atomics), flushes its non-empty
// bins to a global per-row histogram, and the last block of the row to arrive
// finds the digit where the running count (top-k) or mass (top-p) crosses the
// target.  Ties on the final key are taken lowest index first.  Compaction
// then writes the ascending index list, unioned with the always-kept sink and
// window tokens (method section 1), or expands selected pages to tokens.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8192;                  // candidates per block
constexpr int kPer = kChunk / kThreads;       // candidates per thread
constexpr int kBins = 4096;                   // 12-bit digits
constexpr int kCoarse = kBins / 64;           // 64-bin groups (two-step resolve)
constexpr double kFix = 1099511627776.0;      // 2^40 fixed-point unit of mass

enum : uint32_t { kSearching = 0, kTakeGE = 1, kTakeTies = 2 };

struct RowState {
  uint32_t mode;     // kSearching / kTakeGE (key >= thr) / kTakeTies
  uint32_t prefix;   // resolved high bits of the threshold key
  uint32_t thr;      // threshold key
  uint32_t n_eq;     // kTakeTies: keys == thr to take (lowest index first)
  uint32_t need;     // top-k: candidates still needed inside the prefix bin
  uint32_t maxkey;   // top-p: key of the row maximum
  uint32_t arrive;   // arrival counter of the current level (reset by resolver)
  uint32_t n_cand;
  uint64_t rem;      // top-p: mass still needed inside the prefix bin
  uint64_t total;    // top-p: total mass of the row
};
static_assert(sizeof(RowState) == 48, "layout");

struct WsLayout {
  RowState* state;
  uint32_t* chunkmax;  // [rows][nchunk]
  uint32_t* cnt_eq;    // [rows][nchunk]
  uint32_t* cnt_out;   // [rows][nchunk]
  uint32_t* hcnt;      // [2][rows][kBins]
  uint64_t* hmass;     // [2][rows][kBins]
  uint32_t* ccnt;      // [2][rows][kCoarse] sums of 64 consecutive bins
  uint64_t* cmass;     // [2][rows][kCoarse]
};

__host__ __device__ inline int nchunk_of(int32_t max_cand) {
  return (max_cand + kChunk - 1) / kChunk;
}

WsLayout carve(void* ws, int32_t rows, int32_t max_cand) {
  const int nch = nchunk_of(max_cand);
  char* p = (char*)ws;
  WsLayout w;
  w.state = (RowState*)p;            p += align_up(sizeof(RowState) * rows, 256);
  w.chunkmax = (uint32_t*)p;         p += align_up(sizeof(uint32_t) * rows * nch, 256);
  w.cnt_eq = (uint32_t*)p;           p += align_up(sizeof(uint32_t) * rows * nch, 256);
  w.cnt_out = (uint32_t*)p;          p += align_up(sizeof(uint32_t) * rows * nch, 256);
  w.hcnt = (uint32_t*)p;             p += align_up(sizeof(uint32_t) * 2 * rows * kBins, 256);
  w.hmass = (uint64_t*)p;            p += align_up(sizeof(uint64_t) * 2 * rows * kBins, 256);
  w.ccnt = (uint32_t*)p;             p += align_up(sizeof(uint32_t) * 2 * rows * kCoarse, 256);
  w.cmass = (uint64_t*)p;
  return w;
}

__device__ __forceinline__ int32_t n_cand_of(const SelectArgs& a, int row) {
  if (a.prefill_bsel > 0) return a.prefill_bsel * (a.prefill_blk0 + row / a.Hkv) + a.prefill_self;
  const int b = row / a.Hkv;
  const int32_t L = clamp_len(a.seq_lens[b], a.max_len);
  return a.unit == 1 ? L : (L + a.unit - 1) / a.unit;
}

// Exclusive block scan (NW waves) of an unsigned value.
template <typename U, int NW = kWaves>
__device__ __forceinline__ U block_excl_scan(U v, U* lds4, U& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  U inc = v;
  if constexpr (sizeof(U) == 4) inc = wave_incl_scan(v);
  else inc = wave_incl_scan_u64(v);
  if (lane == 63) lds4[w] = inc;
  __syncthreads();
  U off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    U s = lds4[i];
    if (i < w) off += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

__device__ __forceinline__ uint64_t mass_fixed(float x, float mx) {
  const float e = __expf(x - mx);  // in (0, 1]
  return (uint64_t)(e * 1099511627776.0f);
}

// ---------------------------------------------------------------------------
// Init: per-chunk maximum key, zero level-1 histogram, row state.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_sel_init(SelectArgs a, WsLayout w, int nch) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int32_t n = n_cand_of(a, row);
  const float* xr = a.x + (int64_t)row * a.ldx;
  uint32_t mk = 0;
  for (int i = 0; i < kPer; ++i) {
    const int32_t j = c * kChunk + i * kThreads + threadIdx.x;
    if (j < n) {
      uint32_t k = score_key(xr[j]);
      mk = k > mk ? k : mk;
    }
  }
  mk = wave_max_u32(mk);
  __shared__ uint32_t red[kWaves];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mk;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < kWaves; ++i) m = red[i] > m ? red[i] : m;
    w.chunkmax[(int64_t)row * nch + c] = m;
  }
  // zero histogram buffer 0 of the row (bins spread over the row's chunks)
  uint32_t* hc = w.hcnt + (int64_t)row * kBins;
  uint64_t* hm = w.hmass + (int64_t)row * kBins;
  for (int i = c * kThreads + threadIdx.x; i < kBins; i += nch * kThreads) {
    hc[i] = 0;
    hm[i] = 0;
  }
  if (c == 0 && threadIdx.x < kCoarse) {
    w.ccnt[(int64_t)row * kCoarse + threadIdx.x] = 0;
    w.cmass[(int64_t)row * kCoarse + threadIdx.x] = 0;
  }
  if (c == 0 && threadIdx.x == 0) {
    RowState s;
    s.mode = kSearching;
    s.prefix = 0;
    s.thr = 0;
    s.n_eq = 0;
    s.need = (uint32_t)a.k;
    s.maxkey = 0;
    s.arrive = 0;
    s.n_cand = (uint32_t)n;
    s.rem = 0;
    s.total = 0;
    const bool all = (n == 0) || (a.is_topk ? (a.k >= n) : (a.p >= 1.0f));
    if (all) {
      s.mode = kTakeGE;  // every key >= 0
      s.thr = 0;
    }
    w.state[row] = s;
  }
}

// ---------------------------------------------------------------------------
// One radix level.  LEVEL 1: digit = key[31:20]; 2: key[19:8] under a 12-bit
// prefix; 3: key[7:0] under a 24-bit prefix.  Global histograms keep, beside
// the NB digit bins, NB/64 coarse sums of 64 consecutive bins, so the
// resolving block finds the crossing in two dependent reads of one wave.
// ---------------------------------------------------------------------------
template <int LEVEL, bool TOPP>
__global__ void __launch_bounds__(kThreads) k_sel_level(SelectArgs a, WsLayout w, int nch) {
  constexpr int NB = LEVEL == 3 ? 256 : kBins;
  constexpr int NC = NB / 64;
  const int c = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & 63;
  RowState* sp = &w.state[row];
  const uint32_t mode = __hip_atomic_load(&sp->mode, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (mode != kSearching) return;
  const RowState st = *sp;
  const int32_t n = (int32_t)st.n_cand;

  __shared__ uint32_t hcnt[NB];
  __shared__ uint64_t hmass[TOPP ? NB : 1];
  __shared__ uint32_t s_max;
  __shared__ int s_last;
  for (int i = threadIdx.x; i < NB; i += kThreads) {
    hcnt[i] = 0;
    if (TOPP) hmass[i] = 0;
  }
  if (TOPP && threadIdx.x == 0) {
    uint32_t m = st.maxkey;
    if (LEVEL == 1) {
      m = 0;
      for (int i = 0; i < nch; ++i) {
        uint32_t v = w.chunkmax[(int64_t)row * nch + i];
        m = v > m ? v : m;
      }
    }
    s_max = m;
  }
  __syncthreads();
  const float mx = TOPP ? key_score(s_max) : 0.f;
  const float* xr = a.x + (int64_t)row * a.ldx;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int32_t j = c * kChunk + i * kThreads + threadIdx.x;
    if (j >= n) continue;
    const float xv = xr[j];
    const uint32_t key = score_key(xv);
    uint32_t digit;
    if (LEVEL == 1) {
      digit = key >> 20;
    } else if (LEVEL == 2) {
      if ((key >> 20) != st.prefix) continue;
      digit = (key >> 8) & 0xfffu;
    } else {
      if ((key >> 8) != st.prefix) continue;
      digit = key & 0xffu;
    }
    atomicAdd(&hcnt[digit], 1u);
    if (TOPP) atomicAdd((unsigned long long*)&hmass[digit], (unsigned long long)mass_fixed(xv, mx));
  }
  __syncthreads();
  const int buf = (LEVEL == 2) ? 1 : 0;
  uint32_t* gc = w.hcnt + ((int64_t)buf * a.rows + row) * kBins;
  uint64_t* gm = w.hmass + ((int64_t)buf * a.rows + row) * kBins;
  uint32_t* gcc = w.ccnt + ((int64_t)buf * a.rows + row) * kCoarse;
  uint64_t* gcm = w.cmass + ((int64_t)buf * a.rows + row) * kCoarse;
  // flush: one wave per coarse group of 64 bins
  for (int cg = threadIdx.x >> 6; cg < NC; cg += kWaves) {
    const int bin = cg * 64 + lane;
    const uint32_t cn = hcnt[bin];
    const uint64_t ms = TOPP ? hmass[bin] : 0;
    if (cn) {
      atomicAdd(&gc[bin], cn);
      if (TOPP) atomicAdd((unsigned long long*)&gm[bin], (unsigned long long)ms);
    }
    const uint32_t csum = wave_sum_u32(cn);
    const uint64_t msum = TOPP ? wave_sum_u64(ms) : 0ull;
    if (lane == 0 && csum) {
      atomicAdd(&gcc[cg], csum);
      if (TOPP) atomicAdd((unsigned long long*)&gcm[cg], (unsigned long long)msum);
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&sp->arrive, 1u);
    s_last = (old == (uint32_t)gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- resolve (last block of the row, wave 0) ----
  __shared__ uint32_t r_bin, r_cnt, r_cbefore;
  __shared__ uint64_t r_mass, r_mbefore, r_target, r_total;
  if (threadIdx.x < 64) {
    // step 1: coarse groups in descending order, lane i <-> group NC-1-i
    const int cgi = NC - 1 - lane;
    const uint32_t cc = lane < NC ? __hip_atomic_load(&gcc[cgi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint64_t cm = (TOPP && lane < NC) ? __hip_atomic_load(&gcm[cgi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
    const uint32_t cinc = wave_incl_scan(cc);
    const uint64_t minc = wave_incl_scan_u64(cm);
    const uint64_t mtot = lane_u64(minc, 63);
    uint64_t target = st.rem;
    if (TOPP && LEVEL == 1) {
      const double t = (double)a.p * (double)mtot;
      uint64_t tc = (uint64_t)ceil(t);
      if (tc < 1) tc = 1;
      if (tc > mtot) tc = mtot;
      target = tc;
    }
    const uint32_t need = st.need;
    const uint32_t cbef = cinc - cc;
    const uint64_t mbef = minc - cm;
    const bool hit = lane < NC && (TOPP ? (mbef < target && minc >= target)
                                        : (cbef < need && cinc >= need));
    const unsigned long long hb = __ballot(hit);
    int found = -1;
    uint32_t g_cbef = 0;
    uint64_t g_mbef = 0;
    if (hb) {
      const int src = __ffsll(hb) - 1;
      found = (int)lane_u32((uint32_t)cgi, src);
      g_cbef = lane_u32(cbef, src);
      g_mbef = lane_u64(mbef, src);
    }
    // step 2: the 64 bins of the crossing group, descending
    uint32_t bc = 0;
    uint64_t bm = 0;
    int bin = -1;
    if (found >= 0) {
      bin = found * 64 + 63 - lane;
      bc = __hip_atomic_load(&gc[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bm = TOPP ? __hip_atomic_load(&gm[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
    }
    const uint32_t binc = wave_incl_scan(bc);
    const uint64_t bminc = wave_incl_scan_u64(bm);
    const uint32_t bcb = g_cbef + binc - bc;
    const uint64_t bmb = g_mbef + bminc - bm;
    const bool hit2 = found >= 0 && (TOPP ? (bmb < target && bmb + bm >= target)
                                          : (bcb < need && bcb + bc >= need));
    const unsigned long long hb2 = __ballot(hit2);
    if (lane == 0) {
      r_bin = 0xffffffffu;
      r_target = target;
      r_total = mtot;
    }
    if (hb2 && lane == __ffsll(hb2) - 1) {
      r_bin = (uint32_t)bin;
      r_cnt = bc;
      r_cbefore = bcb;
      r_mass = bm;
      r_mbefore = bmb;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState s = st;
    s.arrive = 0;
    const uint64_t target = r_target;
    if (TOPP && LEVEL == 1) {
      s.maxkey = s_max;
      s.total = r_total;
    }
    const uint32_t bin = r_bin;
    if (bin == 0xffffffffu) {
      // cannot happen for consistent inputs; fall back to taking everything
      s.mode = kTakeGE;
      s.thr = 0;
    } else {
      const uint32_t cnt_b = r_cnt;
      const uint32_t new_prefix =
          LEVEL == 1 ? bin : (LEVEL == 2 ? ((st.prefix << 12) | bin) : ((st.prefix << 8) | bin));
      const int shift = LEVEL == 1 ? 20 : (LEVEL == 2 ? 8 : 0);
      const uint32_t bin_lo = new_prefix << shift;
      if (TOPP) {
        const uint64_t rem = target - r_mbefore;  // 0 < rem <= mass of bin
        if (LEVEL < 3) {
          if (cnt_b == 1 || rem == r_mass) {
            s.mode = kTakeGE;
            s.thr = bin_lo;
          } else {
            s.prefix = new_prefix;
            s.rem = rem;
          }
        } else {
          const uint64_t m1 = r_mass / cnt_b;  // every tie has the same mass
          const uint64_t take = (rem + m1 - 1) / m1;
          if (take >= cnt_b) {
            s.mode = kTakeGE;
            s.thr = bin_lo;
          } else {
            s.mode = kTakeTies;
            s.thr = bin_lo;
            s.n_eq = (uint32_t)take;
          }
        }
      } else {
        const uint32_t nd = st.need - r_cbefore;  // 0 < nd <= cnt_b
        if (nd == cnt_b) {
          s.mode = kTakeGE;
          s.thr = bin_lo;
        } else if (LEVEL < 3) {
          s.prefix = new_prefix;
          s.need = nd;
        } else {
          s.mode = kTakeTies;
          s.thr = bin_lo;
          s.n_eq = nd;
        }
      }
    }
    *sp = s;
  }
  // zero the other histogram buffer for the next level
  if (LEVEL < 3) {
    const int nb = 1 - buf;
    uint32_t* zc = w.hcnt + ((int64_t)nb * a.rows + row) * kBins;
    uint64_t* zm = w.hmass + ((int64_t)nb * a.rows + row) * kBins;
    const int nz = LEVEL == 1 ? kBins : 256;
    for (int i = threadIdx.x; i < nz; i += kThreads) {
      zc[i] = 0;
      zm[i] = 0;
    }
    if (threadIdx.x < kCoarse) {
      w.ccnt[((int64_t)nb * a.rows + row) * kCoarse + threadIdx.x] = 0;
      w.cmass[((int64_t)nb * a.rows + row) * kCoarse + threadIdx.x] = 0;
    }
  }
  __threadfence();
}

// ---------------------------------------------------------------------------
// Compaction.  Per chunk: ties count (only when some ties are left out), then
// emitted-token count, then the writes.  Candidates are visited in index order
// in rounds of kThreads, so tie ranks and output positions follow the index.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_sel_ties(SelectArgs a, WsLayout w, int nch) {
  const int c = blockIdx.x, row = blockIdx.y;
  const RowState st = w.state[row];
  if (st.mode != kTakeTies) return;
  const int32_t n = (int32_t)st.n_cand;
  const float* xr = a.x + (int64_t)row * a.ldx;
  uint32_t cnt = 0;
  for (int i = 0; i < kPer; ++i) {
    const int32_t j = c * kChunk + i * kThreads + threadIdx.x;
    if (j < n && score_key(xr[j]) == st.thr) ++cnt;
  }
  __shared__ uint32_t l4[kWaves];
  uint32_t tot;
  block_excl_scan<uint32_t>(cnt, l4, tot);
  if (threadIdx.x == 0) w.cnt_eq[(int64_t)row * nch + c] = tot;
}

template <bool EMIT>
__global__ void __launch_bounds__(kThreads) k_sel_out(SelectArgs a, WsLayout w, int nch) {
  const int c = blockIdx.x, row = blockIdx.y;
  const RowState st = w.state[row];
  const int32_t n = (int32_t)st.n_cand;
  const int b = row / a.Hkv;
  const int32_t L = a.seq_lens ? clamp_len(a.seq_lens[b], a.max_len) : n;
  const float* xr = a.x + (int64_t)row * a.ldx;
  __shared__ uint32_t l4[kWaves];
  uint32_t eq_base = 0;
  if (st.mode == kTakeTies)
    for (int i = 0; i < c; ++i) eq_base += w.cnt_eq[(int64_t)row * nch + i];
  uint32_t out_base = 0, total_out = 0;
  if (EMIT) {
    for (int i = 0; i < nch; ++i) {
      const uint32_t v = w.cnt_out[(int64_t)row * nch + i];
      if (i < c) out_base += v;
      total_out += v;
    }
  }
  int32_t* out = a.idx + (int64_t)row * a.cap;
  uint32_t produced = 0;
  for (int i = 0; i < kPer; ++i) {
    const int32_t j = c * kChunk + i * kThreads + threadIdx.x;
    const bool valid = j < n;
    uint32_t key = valid ? score_key(xr[j]) : 0u;
    bool top = false;
    if (valid) {
      if (st.mode == kTakeGE) top = key >= st.thr;
      else top = key > st.thr;
    }
    if (st.mode == kTakeTies) {  // uniform branch
      const bool eq = valid && key == st.thr;
      uint32_t tot;
      const uint32_t rank = eq_base + block_excl_scan<uint32_t>(eq ? 1u : 0u, l4, tot);
      if (eq && rank < st.n_eq) top = true;
      eq_base += tot;
    }
    bool forced = false;
    if (valid && a.unit == 1) forced = (j < a.n_sink) || (j >= n - a.n_window);
    const bool sel = valid && (top || forced);
    uint32_t wgt = 0;
    if (sel) wgt = a.unit == 1 ? 1u : (uint32_t)min(a.unit, L - j * a.unit);
    uint32_t tot;
    const uint32_t pos = block_excl_scan<uint32_t>(wgt, l4, tot);
    if (EMIT && sel) {
      const uint32_t o = out_base + produced + pos;
      if (a.unit == 1) {
        if (o < (uint32_t)a.cap) out[o] = j;
      } else {
        for (uint32_t e = 0; e < wgt; ++e)
          if (o + e < (uint32_t)a.cap) out[o + e] = j * a.unit + (int32_t)e;
      }
    }
    produced += tot;
  }
  if (!EMIT) {
    if (threadIdx.x == 0) w.cnt_out[(int64_t)row * nch + c] = produced;
    return;
  }
  // pad the tail with -1 and publish the count
  const uint32_t T = total_out < (uint32_t)a.cap ? total_out : (uint32_t)a.cap;
  for (int64_t o = (int64_t)T + (int64_t)c * kThreads + threadIdx.x; o < a.cap;
       o += (int64_t)nch * kThreads)
    out[o] = -1;
  if (c == 0 && threadIdx.x == 0) a.count[row] = (int32_t)T;
}

// ---------------------------------------------------------------------------
// Row-resident selection: one block per row for rows of up to kRowMax
// candidates.  Keys of the first kRowRegs * kThreads candidates stay in
// registers, the next kCacheRounds * kThreads in LDS, the rest are re-read
// from the score row.  Only two passes touch every candidate: the one that
// loads the keys (and, for top-k, builds the level-1 histogram on the way),
// and a filter pass that marks every candidate above the level-1 threshold
// bin in an LDS bitmap (one ballot word per wave and round) and gathers the
// candidates inside that bin into an LDS buffer.  Levels 2 and 3 and the
// final marking run over that buffer alone (over every candidate again only
// when the bin overflows it).  Keys equal to the final threshold are ranked in
// index order by a block scan over a second bitmap; the ascending index list
// is a block scan over the bitmap's word popcounts.  Selected pages are
// staged in LDS and expanded to tokens by the whole block.
// ---------------------------------------------------------------------------
constexpr int kRowRegsTopp = 32;
constexpr int kRowRegsTopk = 48;
// rounds after the register-resident ones kept in LDS (top-k has no mass
// histogram, so more LDS is free for keys)
constexpr int kCacheRoundsTopk = 22;
constexpr int kCacheRoundsTopp = 14;
constexpr int kCacheRoundsHalf = 7;  // 512-thread top-k blocks: two per CU share its LDS
constexpr int kRowMax = kSelectRowMax;
constexpr int kMapWords = kRowMax / 64;   // 64-bit bitmap words: one per (round, wave)
constexpr int kBufCap = 4096;             // candidates of the level-1 bin held in LDS
static_assert(kMapWords * 2 == kBins, "the tie bitmap reuses the count histogram");

// Raw buffer view of a score row: full rounds load with the round's byte
// offset in a scalar register and the lane's in a vector one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* p, int32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, n * 4, 0x00020000);
}

struct RowRes {
  uint32_t mode, prefix, thr, n_eq, need, all;
  uint64_t rem;
};

// RR: register-resident rounds; NT: threads per block (1024: one block per
// CU; 512: two, for top-k, whose blocks fit twice into the LDS).
template <bool TOPP, int RR, int NT>
__global__ void __launch_bounds__(NT) k_select_row(SelectArgs a) {
  constexpr int NW = NT / 64;
  constexpr int WPT = (kRowMax / 32) / NT;    // 32-bit bitmap words per thread
  constexpr int kBufPerW = kBufCap / NW;      // each wave fills its own buffer segment
  constexpr int kRowRegs = RR;
  constexpr int kCacheRounds =
      NT == 512 ? kCacheRoundsHalf : (TOPP ? kCacheRoundsTopp : kCacheRoundsTopk);
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t n = n_cand_of(a, row);
  const int b = row / a.Hkv;
  const int32_t Lt = a.seq_lens ? clamp_len(a.seq_lens[b], a.max_len) : n;
  const float* xr = a.x + (int64_t)row * a.ldx;
  const int rounds = (n + NT - 1) / NT;
  const int full = n / NT;  // rounds with every lane inside the row
  const int32_t last = n > 0 ? n - 1 : 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(xr, n);
  // score of round i (every lane inside the row) as raw bits
  auto load_full = [&](int i) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, t * 4, i * NT * 4, 0);
  };

  __shared__ __align__(16) uint32_t hcnt[kBins];  // digit counts; after the last level, the tie bitmap
  __shared__ uint64_t hmass[TOPP ? kBins : 1];
  __shared__ uint64_t selmap[kMapWords];  // bit e: candidate e is selected
  __shared__ uint32_t kcache[kCacheRounds * NT];
  // level-1 bin candidates: keys in [0, kBufCap), indices in [kBufCap, 2 kBufCap);
  // after the marking, the index half stages the page list
  __shared__ uint32_t bufm[2 * kBufCap];
  uint32_t* const bkey = bufm;
  int32_t* const bidx = reinterpret_cast<int32_t*>(bufm + kBufCap);
  __shared__ uint32_t red32[NW];
  __shared__ uint64_t red64[NW];
  __shared__ RowRes res;
  __shared__ uint32_t s_hit_bin, s_hit_cnt, s_hit_cbef, s_last;
  __shared__ uint32_t s_wcnt[NW];
  __shared__ uint64_t s_hit_mass, s_hit_mbef;
  uint32_t* const sel32 = reinterpret_cast<uint32_t*>(selmap);
  uint32_t* const tie32 = hcnt;
  const int cached_end = kRowRegs + kCacheRounds;  // rounds [kRowRegs, cached_end) live in LDS

  // Full rounds [ib, ie) from the score row, two batches of 8 in turn: one
  // batch's loads are in flight while the other is consumed (round indices
  // past ie are clamped to ie - 1, so every load is issued unconditionally).
  // fn(i, raw score bits).
  auto stream_full = [&](int ib, int ie, auto&& fn) {
    if (ib >= ie) return;
    uint32_t va[8], vb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) va[u] = load_full(min(ib + u, ie - 1));
    for (int i0 = ib; i0 < ie; i0 += 16) {
#pragma unroll
      for (int u = 0; u < 8; ++u) vb[u] = load_full(min(i0 + 8 + u, ie - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < ie) fn(i0 + u, va[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) va[u] = load_full(min(i0 + 16 + u, ie - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 8 + u < ie) fn(i0 + 8 + u, vb[u]);
    }
  };
  // The row's partial last round (round `full`), lanes past the row read its
  // last score and get key 0.
  auto partial_key = [&]() -> uint32_t {
    const int32_t e = full * NT + t;
    const float v = xr[e < n ? e : last];
    return e < n ? score_key(v) : 0u;
  };
  // Visit rounds [kRowRegs, rounds): LDS-cached rounds, then the score row.
  auto for_rounds = [&](auto&& fn) {
    const int c_end = rounds < cached_end ? rounds : cached_end;
    for (int i = kRowRegs; i < c_end; ++i) fn(i, kcache[(i - kRowRegs) * NT + t]);
    stream_full(c_end, full, [&](int i, uint32_t raw) { fn(i, score_key(__uint_as_float(raw))); });
    if (rounds > full && full >= c_end) fn(full, partial_key());
  };
  uint32_t keys[kRowRegs];
  // every round (wave-uniform calls; fn checks the candidate's validity)
  auto for_all = [&](auto&& fn) {
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i)
      if (i < rounds) fn(i, keys[i]);
    for_rounds(fn);
  };
  // digit of `key` at `level` into the histogram when its resolved high bits
  // equal `pre`
  auto hist_add = [&](uint32_t key, int level, uint32_t pre, float mx) {
    const int shift = level == 1 ? 20 : (level == 2 ? 8 : 0);
    const int hshift = level == 2 ? 20 : 8;
    const uint32_t dmask = level == 3 ? 0xffu : 0xfffu;
    if (level == 1 || (key >> hshift) == pre) {
      const uint32_t digit = (key >> shift) & dmask;
      atomicAdd(&hcnt[digit], 1u);
      if (TOPP)
        atomicAdd((unsigned long long*)&hmass[digit],
                  (unsigned long long)mass_fixed(key_score(key), mx));
    }
  };

  if (t == 0) {
    res.mode = kSearching;
    res.prefix = 0;
    res.thr = 0;
    res.n_eq = 0;
    res.need = (uint32_t)a.k;
    res.all = 0;
    res.rem = 0;
    if (n == 0 || (a.is_topk ? (a.k >= n) : (a.p >= 1.0f))) res.mode = kTakeGE;
    s_last = 0;
  }
  for (int i = t; i < kBins; i += NT) {
    hcnt[i] = 0;
    if (TOPP) hmass[i] = 0;
  }
  for (int i = t; i < rounds * NW; i += NT) selmap[i] = 0;
  __syncthreads();

  // ---- load: keys to registers and LDS; top-k builds the level-1 histogram,
  // top-p takes the row maximum (the mass reference) first ----
  uint32_t mk = 0;
  // top-k: padding lanes (key 0) are counted into bin 0 and taken out below
  auto take = [&](uint32_t key) {
    if (TOPP) mk = key > mk ? key : mk;
    else hist_add(key, 1, 0, 0.f);
  };
  // every register round's load is issued before the first is used (raw
  // score bits; in the row's last round, lanes past it read its last score)
#pragma unroll
  for (int i0 = 0; i0 < kRowRegs; i0 += 8) {
    if (i0 + 8 <= full) {
#pragma unroll
      for (int u = 0; u < 8; ++u) keys[i0 + u] = load_full(i0 + u);
    } else if (i0 < rounds) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int32_t e = (i0 + u) * NT + t;
        keys[i0 + u] = __float_as_uint(xr[e < n ? e : last]);
      }
    }
  }
#pragma unroll
  for (int i0 = 0; i0 < kRowRegs; i0 += 8) {
    if (i0 + 8 <= full) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        keys[i0 + u] = score_key(__uint_as_float(keys[i0 + u]));
        take(keys[i0 + u]);
      }
    } else if (i0 < rounds) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int32_t e = (i0 + u) * NT + t;
        keys[i0 + u] = e < n ? score_key(__uint_as_float(keys[i0 + u])) : 0u;
        if (i0 + u < rounds) take(keys[i0 + u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) keys[i0 + u] = 0u;
    }
  }
  // later rounds: LDS cache, then keys only for the histogram / maximum
  auto keep = [&](int i, uint32_t k) {
    if (i < cached_end) kcache[(i - kRowRegs) * NT + t] = k;
    take(k);
  };
  stream_full(kRowRegs, full, [&](int i, uint32_t raw) { keep(i, score_key(__uint_as_float(raw))); });
  if (rounds > full && full >= kRowRegs) keep(full, partial_key());
  if (!TOPP && t == 0) atomicSub(&hcnt[0], (uint32_t)(rounds * NT - n));
  float mx = 0.f;
  if (TOPP) {
    mk = wave_max_u32(mk);
    if (lane == 0) red32[wave] = mk;
  }
  __syncthreads();
  if (TOPP) {
    uint32_t M = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = red32[i] > M ? red32[i] : M;
    mx = key_score(M);
    for_all([&](int i, uint32_t k) {
      if (i * NT + t < n) hist_add(k, 1, 0, mx);
    });
    __syncthreads();
  }

  // Resolve a level from its histogram: the bin (in descending order) where
  // the running count reaches the candidates still needed (top-k), or the
  // running mass the target (top-p).  Ends with a barrier.
  auto resolve = [&](int level) {
    const int NB = level == 3 ? 256 : kBins;
    const int shift = level == 1 ? 20 : (level == 2 ? 8 : 0);
    const uint32_t pre = res.prefix;
    // block scan over bins in descending order: thread t owns positions
    // [t*per, (t+1)*per), position q <-> bin NB-1-q
    const int per = NB / NT > 0 ? NB / NT : 1;
    const bool owns = t * per < NB;
    uint32_t cl = 0;
    uint64_t ml = 0;
    if (owns)
      for (int e = 0; e < per; ++e) {
        const int bin = NB - 1 - (t * per + e);
        cl += hcnt[bin];
        if (TOPP) ml += hmass[bin];
      }
    uint32_t ctot;
    uint64_t mtot = 0;
    const uint32_t cb0 = block_excl_scan<uint32_t, NW>(cl, red32, ctot);
    const uint64_t mb0 = TOPP ? block_excl_scan<uint64_t, NW>(ml, red64, mtot) : 0ull;
    uint64_t target = res.rem;
    if (TOPP && level == 1) {
      uint64_t tc = (uint64_t)ceil((double)a.p * (double)mtot);
      if (tc < 1) tc = 1;
      if (tc > mtot) tc = mtot;
      target = tc;
    }
    const uint32_t need = res.need;
    if (t == 0) s_hit_bin = 0xffffffffu;
    __syncthreads();
    if (owns) {
      uint32_t cb = cb0;
      uint64_t mb = mb0;
      for (int e = 0; e < per; ++e) {
        const int bin = NB - 1 - (t * per + e);
        const uint32_t c = hcnt[bin];
        const uint64_t m = TOPP ? hmass[bin] : 0ull;
        const bool hit = TOPP ? (mb < target && mb + m >= target) : (cb < need && cb + c >= need);
        if (hit) {
          s_hit_bin = bin;
          s_hit_cnt = c;
          s_hit_cbef = cb;
          s_hit_mass = m;
          s_hit_mbef = mb;
        }
        cb += c;
        mb += m;
      }
    }
    __syncthreads();
    if (t == 0) {
      const uint32_t bin = s_hit_bin;
      if (bin == 0xffffffffu) {
        res.mode = kTakeGE;  // inconsistent input: take everything
        res.thr = 0;
        res.all = 1;
      } else {
        const uint32_t cnt_b = s_hit_cnt;
        const uint32_t np = level == 1 ? bin : (level == 2 ? ((pre << 12) | bin) : ((pre << 8) | bin));
        const uint32_t bin_lo = np << shift;
        if (TOPP) {
          const uint64_t rem = target - s_hit_mbef;
          if (level < 3) {
            if (cnt_b == 1 || rem == s_hit_mass) {
              res.mode = kTakeGE;
              res.thr = bin_lo;
            } else {
              res.prefix = np;
              res.rem = rem;
            }
          } else {
            const uint64_t m1 = s_hit_mass / cnt_b;
            const uint64_t take_n = (rem + m1 - 1) / m1;
            res.thr = bin_lo;
            if (take_n >= cnt_b) {
              res.mode = kTakeGE;
            } else {
              res.mode = kTakeTies;
              res.n_eq = (uint32_t)take_n;
            }
          }
        } else {
          const uint32_t nd = need - s_hit_cbef;
          if (nd == cnt_b) {
            res.mode = kTakeGE;
            res.thr = bin_lo;
          } else if (level < 3) {
            res.prefix = np;
            res.need = nd;
          } else {
            res.mode = kTakeTies;
            res.thr = bin_lo;
            res.n_eq = nd;
          }
        }
      }
    }
    __syncthreads();
  };

  // ---- level 1, then the filter pass ----
  if (res.mode == kSearching) resolve(1);
  const uint32_t mode1 = res.mode, thr1 = res.thr, B1 = res.prefix;
  if (mode1 == kSearching) {
    // bins above B1 are in; bin B1 goes to this wave's buffer segment.  The
    // bitmap starts cleared, so a round with no key in or above bin B1 costs
    // one compare.
    uint32_t wcnt = 0;  // wave-uniform fill of the segment
    const uint32_t lo1 = B1 << 20, top1 = lo1 | 0xfffffu;  // bin B1 = [lo1, top1]
    uint64_t* const smap = selmap + wave;
    auto filter = [&](int i, uint32_t k, bool hi) {  // hi: valid and key >= lo1
      const uint64_t mh = __builtin_amdgcn_ballot_w64(hi);
      if (mh == 0) return;
      const uint64_t m = __builtin_amdgcn_ballot_w64(k > top1) & mh;
      if (m && lane == 0) smap[i * NW] = m;
      const uint64_t mb = mh & ~m;
      if (mb) {
        const uint32_t p = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, wcnt));
        if (hi && k <= top1 && p < (uint32_t)kBufPerW) {
          bkey[wave * kBufPerW + p] = k;
          bidx[wave * kBufPerW + p] = i * NT + t;
        }
        wcnt += (uint32_t)__popcll(mb);
      }
    };
    if (lo1 > 0)  // padding lanes (key 0) lie below the bin
      for_all([&](int i, uint32_t k) { filter(i, k, k >= lo1); });
    else
      for_all([&](int i, uint32_t k) { filter(i, k, i * NT + t < n); });
    if (lane == 0) s_wcnt[wave] = wcnt;
  } else {
    // key >= thr1 decides every candidate
    for_all([&](int i, uint32_t k) {
      const uint64_t m = __ballot(i * NT + t < n && k >= thr1);
      if (lane == 0 && m) selmap[i * NW + wave] = m;
    });
  }
  __syncthreads();
  bool use_buf = true;
  if (mode1 == kSearching) {
#pragma unroll
    for (int w = 0; w < NW; ++w) use_buf = use_buf && s_wcnt[w] <= (uint32_t)kBufPerW;
  }
  // buffer slot j holds a candidate when it lies inside its wave's fill
  auto in_buf = [&](int j) { return (uint32_t)(j % kBufPerW) < s_wcnt[j / kBufPerW]; };

  // ---- levels 2 and 3 over the bin's candidates ----
  for (int level = 2; level <= 3; ++level) {
    if (res.mode != kSearching) break;  // block-uniform (read after a barrier)
    const int NB = level == 3 ? 256 : kBins;
    const uint32_t pre = res.prefix;
    for (int i = t; i < NB; i += NT) {
      hcnt[i] = 0;
      if (TOPP) hmass[i] = 0;
    }
    __syncthreads();
    if (use_buf) {
      for (int j = t; j < kBufCap; j += NT)
        if (in_buf(j)) hist_add(bkey[j], level, pre, mx);
    } else {
      for_all([&](int i, uint32_t k) {
        if (i * NT + t < n) hist_add(k, level, pre, mx);
      });
    }
    __syncthreads();
    resolve(level);
  }

  // ---- final marking of the bin's candidates ----
  const uint32_t mode = res.mode, thr = res.thr, n_eq = res.n_eq;
  const bool take_all = res.all != 0;
  const bool ties = mode1 == kSearching && mode == kTakeTies;
  const int nw = (n + 31) >> 5;  // 32-bit bitmap words of the row
  if (ties) {
    for (int i = t; i < nw; i += NT) tie32[i] = 0;
    __syncthreads();
  }
  if (mode1 == kSearching) {
    if (use_buf) {
      for (int j = t; j < kBufCap; j += NT) {
        if (!in_buf(j)) continue;
        const uint32_t k = bkey[j];
        const int32_t e = bidx[j];
        if (k > thr || (mode == kTakeGE && k == thr)) atomicOr(&sel32[e >> 5], 1u << (e & 31));
        else if (ties && k == thr) atomicOr(&tie32[e >> 5], 1u << (e & 31));
      }
    } else {
      for_all([&](int i, uint32_t k) {
        const int32_t e = i * NT + t;
        const bool in = e < n && (k >> 20) == B1;
        const uint64_t ms = __ballot(in && (k > thr || (mode == kTakeGE && k == thr)));
        const uint64_t me = __ballot(in && ties && k == thr);
        if (lane == 0) {
          selmap[i * NW + wave] |= ms;
          if (ties) reinterpret_cast<uint64_t*>(tie32)[i * NW + wave] = me;
        }
      });
    }
    __syncthreads();
  }

  // ---- ordered compaction: thread t owns bitmap words [WPT t, WPT (t + 1)) ----
  uint32_t sw[WPT];
#pragma unroll
  for (int w = 0; w < WPT; ++w) sw[w] = WPT * t + w < nw ? sel32[WPT * t + w] : 0u;
  if (ties) {  // the n_eq lowest-index keys equal to the threshold
    uint32_t tw[WPT], c = 0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      tw[w] = WPT * t + w < nw ? tie32[WPT * t + w] : 0u;
      c += (uint32_t)__popc(tw[w]);
    }
    uint32_t tot;
    const uint32_t before = block_excl_scan<uint32_t, NW>(c, red32, tot);
    uint32_t left = before < n_eq ? n_eq - before : 0u;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = tw[w], keep = 0;
      while (bits && left) {
        keep |= bits & (0u - bits);
        bits &= bits - 1u;
        --left;
      }
      sw[w] |= keep;
    }
  }
  const int32_t unit = a.unit;
  const int ushift = __ffs(unit) - 1;          // unit is 1 or the page size (powers of two)
  const int32_t last_w = Lt - (n - 1) * unit;  // tokens of the last candidate (unit > 1)
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    const int widx = WPT * t + w;
    if (widx < nw) {
      const int32_t lo = widx * 32;
      const uint32_t vm = n - lo >= 32 ? ~0u : ((1u << (n - lo)) - 1u);
      uint32_t fm = 0;
      if (unit == 1) {  // always-kept sink and window candidates
        if (a.n_sink > lo) fm |= a.n_sink - lo >= 32 ? ~0u : ((1u << (a.n_sink - lo)) - 1u);
        const int32_t ws = n - a.n_window;
        if (ws < lo + 32) fm |= ws <= lo ? ~0u : (~0u << (ws - lo));
      }
      sw[w] = ((take_all ? ~0u : sw[w]) | fm) & vm;
      if (unit > 1 && widx == ((n - 1) >> 5)) s_last = (sw[w] >> ((n - 1) & 31)) & 1u;
    }
    c += (uint32_t)__popc(sw[w]);
  }
  uint32_t total;
  uint32_t rank = block_excl_scan<uint32_t, NW>(c, red32, total);  // barriers publish s_last
  int32_t* out = a.idx + (int64_t)row * a.cap;
  uint32_t T;
  if (unit == 1) {
    T = total < (uint32_t)a.cap ? total : (uint32_t)a.cap;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = sw[w];
      while (bits) {
        const int j = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (rank < (uint32_t)a.cap) out[rank] = (WPT * t + w) * 32 + j;
        ++rank;
      }
    }
  } else {
    const uint32_t tokens = (total << ushift) - (s_last ? (uint32_t)(unit - last_w) : 0u);
    T = tokens < (uint32_t)a.cap ? tokens : (uint32_t)a.cap;
    const bool staged = total < (uint32_t)kBufCap;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = sw[w];
      while (bits) {
        const int32_t e = (WPT * t + w) * 32 + __ffs(bits) - 1;
        bits &= bits - 1u;
        if (staged) {
          bidx[rank] = e;
        } else {
          const uint32_t pos = rank << ushift;
          const int32_t wd = e == n - 1 ? last_w : unit;
          for (int32_t q = 0; q < wd; ++q)
            if (pos + q < (uint32_t)a.cap) out[pos + q] = e * unit + q;
        }
        ++rank;
      }
    }
    if (staged) {  // block-uniform
      __syncthreads();
      for (uint32_t o = t; o < T; o += NT)
        out[o] = (bidx[o >> ushift] << ushift) + (int32_t)(o & (uint32_t)(unit - 1));
    }
  }
  for (int64_t o = (int64_t)T + t; o < a.cap; o += NT) out[o] = -1;
  if (t == 0) a.count[row] = (int32_t)T;
}
// ---------------------------------------------------------------------------
// Row selection over 16-bit keys (prefill top-k).  The score rows hold the
// top 16 bits of each candidate's order-preserving key, two per 32-bit word:
// in every 128-candidate block, candidate c sits in word (c / 128) * 64 +
// c % 64, low half for c % 128 < 64, high half otherwise, so the 64 lanes of
// a wave reading 64 consecutive words hold the block's first 64 candidates in
// their low halves and the next 64 in their high halves: each half gives one
// whole bitmap word per ballot.  The 16 bits hold the level-1 digit (12 bits)
// exactly, so the load and filter passes are those of k_select_row; the
// candidates of the threshold bin get their exact fp32 score recomputed from
// the block's mean query and the indexer keys (same products in the same
// order as the score kernel, so the same float), and levels 2-3, the ties
// and the marking run on exact keys.
// ---------------------------------------------------------------------------
template <int RR, int NT>
__global__ void __launch_bounds__(NT) k_select_row16(SelectArgs a) {
  constexpr int NW = NT / 64;
  constexpr int WPT = (kRowMax / 32) / NT;    // 32-bit bitmap words per thread
  constexpr int kBufPerW = kBufCap / NW;      // each wave fills its own buffer segment
  constexpr int kRowRegs = RR;
  constexpr int kCacheRounds = kCacheRoundsHalf;
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t n = n_cand_of(a, row);
  const uint32_t* xr = reinterpret_cast<const uint32_t*>(a.x) + (int64_t)row * a.ldx;  // ldx: words
  const int nwords = ((n + 127) / 128) * 64;
  const int rounds = (nwords + NT - 1) / NT;
  const int full = n / (2 * NT);  // rounds whose 2 * NT candidates all lie inside the row
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(reinterpret_cast<const float*>(xr), nwords);
  auto load_full = [&](int i) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, t * 4, i * NT * 4, 0);
  };
  // candidate of the low half of round i in this lane (the high half is +64)
  auto cand_lo = [&](int i) -> int32_t { return 2 * (i * NT + wave * 64) + lane; };

  __shared__ __align__(16) uint32_t hcnt[kBins];  // digit counts; after the last level, the tie bitmap
  __shared__ uint64_t selmap[kMapWords];          // bit c: candidate c is selected
  __shared__ uint32_t kcache[kCacheRounds * NT];
  __shared__ uint32_t bufm[2 * kBufCap];
  uint32_t* const bkey = bufm;
  int32_t* const bidx = reinterpret_cast<int32_t*>(bufm + kBufCap);
  __shared__ uint32_t red32[NW];
  __shared__ RowRes res;
  __shared__ uint32_t s_hit_bin, s_hit_cnt, s_hit_cbef;
  __shared__ uint32_t s_wcnt[NW];
  __shared__ float s_q[kRank];
  uint32_t* const sel32 = reinterpret_cast<uint32_t*>(selmap);
  uint32_t* const tie32 = hcnt;
  const int cached_end = kRowRegs + kCacheRounds;

  // the row's partial round (round `full`, if any): halves past the row read 0
  auto partial_word = [&]() -> uint32_t {
    const int32_t w = full * NT + t;
    const uint32_t v = w < nwords ? xr[w] : 0u;
    const int32_t c = cand_lo(full);
    return (c < n ? (v & 0xffffu) : 0u) | (c + 64 < n ? (v & 0xffff0000u) : 0u);
  };
  auto stream_full = [&](int ib, int ie, auto&& fn) {
    if (ib >= ie) return;
    uint32_t va[8], vb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) va[u] = load_full(min(ib + u, ie - 1));
    for (int i0 = ib; i0 < ie; i0 += 16) {
#pragma unroll
      for (int u = 0; u < 8; ++u) vb[u] = load_full(min(i0 + 8 + u, ie - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < ie) fn(i0 + u, va[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) va[u] = load_full(min(i0 + 16 + u, ie - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 8 + u < ie) fn(i0 + 8 + u, vb[u]);
    }
  };
  auto for_rounds = [&](auto&& fn) {
    const int c_end = rounds < cached_end ? rounds : cached_end;
    for (int i = kRowRegs; i < c_end; ++i) fn(i, kcache[(i - kRowRegs) * NT + t]);
    stream_full(c_end, full, fn);
    if (rounds > full && full >= c_end) fn(full, partial_word());
  };
  uint32_t words[kRowRegs];
  auto for_all = [&](auto&& fn) {  // fn(round, packed word); halves past the row are 0
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i)
      if (i < rounds) fn(i, words[i]);
    for_rounds(fn);
  };
  // exact key of candidate c: the score kernel's product of the block's mean
  // query with the candidate's indexer key
  const int g = row % a.Hkv;
  auto exact_key = [&](int32_t c) -> uint32_t {
    const int64_t page = clamp_page(a.pt[c >> 6], a.n_pool_pages);
    const int64_t off = ((page * a.Hkv + g) * kPage + (c & 63)) * kRank;
    float s = 0.f;
    if (a.kidx_bf16) {
      typedef uint32_t w4_t __attribute__((ext_vector_type(4)));
      const w4_t* v = reinterpret_cast<const w4_t*>(reinterpret_cast<const bf16_raw*>(a.kidx) + off);
      const w4_t x0 = v[0], x1 = v[1];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = i < 4 ? x0[i & 3] : x1[i & 3];
        s = fmaf(s_q[2 * i], __uint_as_float(u << 16), s);
        s = fmaf(s_q[2 * i + 1], __uint_as_float(u & 0xffff0000u), s);
      }
    } else {
      const float* kv = reinterpret_cast<const float*>(a.kidx) + off;
#pragma unroll
      for (int i = 0; i < kRank; ++i) s = fmaf(s_q[i], kv[i], s);
    }
    return score_key(s);
  };
  auto hist_add = [&](uint32_t key, int level, uint32_t pre) {
    const int shift = level == 2 ? 8 : 0;
    const int hshift = level == 2 ? 20 : 8;
    const uint32_t dmask = level == 3 ? 0xffu : 0xfffu;
    if ((key >> hshift) == pre) atomicAdd(&hcnt[(key >> shift) & dmask], 1u);
  };

  if (t == 0) {
    res.mode = kSearching;
    res.prefix = 0;
    res.thr = 0;
    res.n_eq = 0;
    res.need = (uint32_t)a.k;
    res.all = 0;
    res.rem = 0;
    if (n == 0 || a.k >= n) res.mode = kTakeGE;
  }
  if (t < kRank) {
    const int blk = a.prefill_blk0 + row / a.Hkv;
    s_q[t] = a.qcb[((int64_t)blk * a.Hkv + g) * kRank + t];
  }
  for (int i = t; i < kBins; i += NT) hcnt[i] = 0;
  for (int i = t; i < 2 * rounds * NW; i += NT) selmap[i] = 0;
  __syncthreads();

  // ---- load: packed keys to registers and LDS, level-1 histogram of both
  // halves (halves past the row hold 0, counted into bin 0 and taken out) ----
  auto take = [&](uint32_t w) {
    atomicAdd(&hcnt[(w & 0xffffu) >> 4], 1u);
    atomicAdd(&hcnt[w >> 20], 1u);
  };
#pragma unroll
  for (int i0 = 0; i0 < kRowRegs; i0 += 8) {
    if (i0 + 8 <= full) {
#pragma unroll
      for (int u = 0; u < 8; ++u) words[i0 + u] = load_full(i0 + u);
    } else if (i0 < rounds) {
#pragma unroll
      for (int u = 0; u < 8; ++u) words[i0 + u] = i0 + u < full ? load_full(i0 + u) : (i0 + u == full ? partial_word() : 0u);
    }
  }
#pragma unroll
  for (int i0 = 0; i0 < kRowRegs; i0 += 8) {
    if (i0 < rounds) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < rounds) take(words[i0 + u]);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) words[i0 + u] = 0u;
    }
  }
  auto keep = [&](int i, uint32_t w) {
    if (i < cached_end) kcache[(i - kRowRegs) * NT + t] = w;
    take(w);
  };
  stream_full(kRowRegs, full, keep);
  if (rounds > full && full >= kRowRegs) keep(full, partial_word());
  if (t == 0) atomicSub(&hcnt[0], (uint32_t)(2 * rounds * NT - n));
  __syncthreads();

  // Resolve a level from its histogram (counts only): the bin, in descending
  // order, where the running count reaches the candidates still needed.
  auto resolve = [&](int level) {
    const int NB = level == 3 ? 256 : kBins;
    const int shift = level == 1 ? 20 : (level == 2 ? 8 : 0);
    const uint32_t pre = res.prefix;
    const int per = NB / NT > 0 ? NB / NT : 1;
    const bool owns = t * per < NB;
    uint32_t cl = 0;
    if (owns)
      for (int e = 0; e < per; ++e) cl += hcnt[NB - 1 - (t * per + e)];
    uint32_t ctot;
    const uint32_t cb0 = block_excl_scan<uint32_t, NW>(cl, red32, ctot);
    const uint32_t need = res.need;
    if (t == 0) s_hit_bin = 0xffffffffu;
    __syncthreads();
    if (owns) {
      uint32_t cb = cb0;
      for (int e = 0; e < per; ++e) {
        const int bin = NB - 1 - (t * per + e);
        const uint32_t c = hcnt[bin];
        if (cb < need && cb + c >= need) {
          s_hit_bin = bin;
          s_hit_cnt = c;
          s_hit_cbef = cb;
        }
        cb += c;
      }
    }
    __syncthreads();
    if (t == 0) {
      const uint32_t bin = s_hit_bin;
      if (bin == 0xffffffffu) {
        res.mode = kTakeGE;  // inconsistent input: take everything
        res.thr = 0;
        res.all = 1;
      } else {
        const uint32_t cnt_b = s_hit_cnt;
        const uint32_t np = level == 1 ? bin : (level == 2 ? ((pre << 12) | bin) : ((pre << 8) | bin));
        const uint32_t bin_lo = np << shift;
        const uint32_t nd = need - s_hit_cbef;
        if (nd == cnt_b) {
          res.mode = kTakeGE;
          res.thr = bin_lo;
        } else if (level < 3) {
          res.prefix = np;
          res.need = nd;
        } else {
          res.mode = kTakeTies;
          res.thr = bin_lo;
          res.n_eq = nd;
        }
      }
    }
    __syncthreads();
  };

  // ---- level 1, then the filter pass ----
  if (res.mode == kSearching) resolve(1);
  const uint32_t mode1 = res.mode, thr1 = res.thr, B1 = res.prefix;
  if (mode1 == kSearching) {
    uint32_t wcnt = 0;  // wave-uniform fill of the buffer segment
    const uint32_t lo1 = B1 << 4, top1 = lo1 | 0xfu;  // bin B1 in 16-bit keys: [lo1, top1]
    uint64_t* const smap = selmap + 2 * wave;
    // one half of a round: k16 its keys, hi: valid and k16 >= lo1
    auto half = [&](int i, int h, uint32_t k16, bool hi) {
      const uint64_t mh = __builtin_amdgcn_ballot_w64(hi);
      if (mh == 0) return;
      const uint64_t m = __builtin_amdgcn_ballot_w64(k16 > top1) & mh;
      if (m && lane == 0) smap[2 * i * NW + h] = m;
      const uint64_t mb = mh & ~m;
      if (mb) {
        const uint32_t p = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, wcnt));
        if (hi && k16 <= top1 && p < (uint32_t)kBufPerW) bidx[wave * kBufPerW + p] = cand_lo(i) + 64 * h;
        wcnt += (uint32_t)__popcll(mb);
      }
    };
    auto filter = [&](int i, uint32_t w) {
      const uint32_t kl = w & 0xffffu, kh = w >> 16;
      if (lo1 > 0) {  // halves past the row (key 0) lie below the bin
        half(i, 0, kl, kl >= lo1);
        half(i, 1, kh, kh >= lo1);
      } else {
        half(i, 0, kl, cand_lo(i) < n);
        half(i, 1, kh, cand_lo(i) + 64 < n);
      }
    };
    for_all(filter);
    if (lane == 0) s_wcnt[wave] = wcnt;
  } else {
    const uint32_t t16 = thr1 >> 16;  // level-1 thresholds are bin floors: exact in 16 bits
    for_all([&](int i, uint32_t w) {
      const int32_t c = cand_lo(i);
      const uint64_t ml = __builtin_amdgcn_ballot_w64(c < n && (w & 0xffffu) >= t16);
      const uint64_t mh = __builtin_amdgcn_ballot_w64(c + 64 < n && (w >> 16) >= t16);
      if (lane == 0) {
        if (ml) selmap[2 * (i * NW + wave)] = ml;
        if (mh) selmap[2 * (i * NW + wave) + 1] = mh;
      }
    });
  }
  __syncthreads();
  bool use_buf = true;
  if (mode1 == kSearching) {
#pragma unroll
    for (int w = 0; w < NW; ++w) use_buf = use_buf && s_wcnt[w] <= (uint32_t)kBufPerW;
  }
  auto in_buf = [&](int j) { return (uint32_t)(j % kBufPerW) < s_wcnt[j / kBufPerW]; };
  // exact keys of the buffered candidates
  if (mode1 == kSearching && use_buf) {
    for (int j = t; j < kBufCap; j += NT)
      if (in_buf(j)) bkey[j] = exact_key(bidx[j]);
    __syncthreads();
  }
  // fallback (bin overflowed its buffer): every candidate of bin B1, exact;
  // rare, so it re-reads the packed keys from the score row one round at a
  // time instead of walking the register copies
  auto for_bin = [&](auto&& fn) {  // fn(candidate, exact key)
#pragma unroll 1
    for (int i = 0; i < rounds; ++i) {
      const uint32_t w = i < full ? load_full(i) : partial_word();
      const int32_t c = cand_lo(i);
      if (c < n && ((w & 0xffffu) >> 4) == B1) fn(c, exact_key(c));
      if (c + 64 < n && (w >> 20) == B1) fn(c + 64, exact_key(c + 64));
    }
  };

  // ---- levels 2 and 3 over the bin's candidates ----
  for (int level = 2; level <= 3; ++level) {
    if (res.mode != kSearching) break;  // block-uniform (read after a barrier)
    const int NB = level == 3 ? 256 : kBins;
    const uint32_t pre = res.prefix;
    for (int i = t; i < NB; i += NT) hcnt[i] = 0;
    __syncthreads();
    if (use_buf) {
      for (int j = t; j < kBufCap; j += NT)
        if (in_buf(j)) hist_add(bkey[j], level, pre);
    } else {
      for_bin([&](int32_t c, uint32_t k) { hist_add(k, level, pre); });
    }
    __syncthreads();
    resolve(level);
  }

  // ---- final marking of the bin's candidates ----
  const uint32_t mode = res.mode, thr = res.thr, n_eq = res.n_eq;
  const bool take_all = res.all != 0;
  const bool ties = mode1 == kSearching && mode == kTakeTies;
  const int nw = (n + 31) >> 5;  // 32-bit bitmap words of the row
  if (ties) {
    for (int i = t; i < nw; i += NT) tie32[i] = 0;
    __syncthreads();
  }
  if (mode1 == kSearching) {
    auto mark = [&](int32_t c, uint32_t k) {
      if (k > thr || (mode == kTakeGE && k == thr)) atomicOr(&sel32[c >> 5], 1u << (c & 31));
      else if (ties && k == thr) atomicOr(&tie32[c >> 5], 1u << (c & 31));
    };
    if (use_buf) {
      for (int j = t; j < kBufCap; j += NT)
        if (in_buf(j)) mark(bidx[j], bkey[j]);
    } else {
      for_bin(mark);
    }
    __syncthreads();
  }

  // ---- ordered compaction: thread t owns bitmap words [WPT t, WPT (t + 1)) ----
  uint32_t sw[WPT];
#pragma unroll
  for (int w = 0; w < WPT; ++w) sw[w] = WPT * t + w < nw ? sel32[WPT * t + w] : 0u;
  if (ties) {  // the n_eq lowest-index keys equal to the threshold
    uint32_t tw[WPT], c = 0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      tw[w] = WPT * t + w < nw ? tie32[WPT * t + w] : 0u;
      c += (uint32_t)__popc(tw[w]);
    }
    uint32_t tot;
    const uint32_t before = block_excl_scan<uint32_t, NW>(c, red32, tot);
    uint32_t left = before < n_eq ? n_eq - before : 0u;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = tw[w], keepb = 0;
      while (bits && left) {
        keepb |= bits & (0u - bits);
        bits &= bits - 1u;
        --left;
      }
      sw[w] |= keepb;
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    const int widx = WPT * t + w;
    if (widx < nw) {
      const int32_t lo = widx * 32;
      const uint32_t vm = n - lo >= 32 ? ~0u : ((1u << (n - lo)) - 1u);
      uint32_t fm = 0;  // always-kept sink and window candidates
      if (a.n_sink > lo) fm |= a.n_sink - lo >= 32 ? ~0u : ((1u << (a.n_sink - lo)) - 1u);
      const int32_t ws = n - a.n_window;
      if (ws < lo + 32) fm |= ws <= lo ? ~0u : (~0u << (ws - lo));
      sw[w] = ((take_all ? ~0u : sw[w]) | fm) & vm;
    }
    c += (uint32_t)__popc(sw[w]);
  }
  uint32_t total;
  uint32_t rank = block_excl_scan<uint32_t, NW>(c, red32, total);
  int32_t* out = a.idx + (int64_t)row * a.cap;
  const uint32_t T = total < (uint32_t)a.cap ? total : (uint32_t)a.cap;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    uint32_t bits = sw[w];
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1u;
      if (rank < (uint32_t)a.cap) out[rank] = (WPT * t + w) * 32 + j;
      ++rank;
    }
  }
  for (int64_t o = (int64_t)T + t; o < a.cap; o += NT) out[o] = -1;
  if (t == 0) a.count[row] = (int32_t)T;
}

}  // namespace

namespace {

// Multi-launch path: row state, per-chunk counters and the level histograms.
size_t select_multi_bytes(int32_t rows, int32_t max_cand) {
  const size_t nch = (size_t)nchunk_of(max_cand < 1 ? 1 : max_cand);
  size_t b = 0;
  b += align_up(sizeof(RowState) * rows, 256);
  b += 3 * align_up(sizeof(uint32_t) * rows * nch, 256);
  b += align_up(sizeof(uint32_t) * 2 * rows * kBins, 256);
  b += align_up(sizeof(uint64_t) * 2 * rows * kBins, 256);
  b += align_up(sizeof(uint32_t) * 2 * rows * kCoarse, 256);
  b += align_up(sizeof(uint64_t) * 2 * rows * kCoarse, 256);
  return b;
}

}  // namespace

// Few long rows may run as one persistent launch instead of the multi-launch
// path (which one depends on n_sink / n_window too): its state sits in a
// region of its own after the multi-launch region, so calls of either path
// can share a workspace.
size_t select_workspace_bytes(int32_t rows, int32_t max_cand) {
  size_t b = select_multi_bytes(rows, max_cand);
  if (rows <= 16) b += align_up(fused_workspace_bytes(rows, 256, 1, 0), 256);
  return b;
}

hipError_t launch_select(const SelectArgs& a, void* ws, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  if (a.key16) {  // prefill top-k over 16-bit keys (rows of at most kRowMax candidates)
    if (!a.is_topk || a.unit != 1 || a.max_cand > kRowMax) return hipErrorInvalidValue;
    k_select_row16<kRowRegsTopk, 512><<<a.rows, 512, 0, st>>>(a);
    return hipGetLastError();
  }
  // One block per row when a row's keys fit in one block's registers, or
  // when there are enough rows to fill the chip; few long rows are split
  // over many blocks instead.
  if (a.max_cand <= kRowRegsTopp * kThreads || (a.max_cand <= kRowMax && a.rows >= 32)) {
    if (!a.is_topk) k_select_row<true, kRowRegsTopp, kThreads><<<a.rows, kThreads, 0, st>>>(a);
    // top-k: two 512-thread blocks per CU when the rows fill the chip, else
    // 1024 threads per row (half the rounds per thread)
    else if (a.rows >= 256) k_select_row<false, kRowRegsTopk, 512><<<a.rows, 512, 0, st>>>(a);
    else k_select_row<false, kRowRegsTopk, kThreads><<<a.rows, kThreads, 0, st>>>(a);
    return hipGetLastError();
  }
  // few long rows: one persistent launch whose workgroups split each row and
  // meet at in-memory barriers, if the rows fit its plan
  int32_t fnb = 0, ftpb = 0;
  if (a.rows <= 16 && select_fused_plan(a, &fnb, &ftpb))
    return launch_select_fused(a, (char*)ws + select_multi_bytes(a.rows, a.max_cand), fnb, ftpb, st);
  const int nch = nchunk_of(a.max_cand < 1 ? 1 : a.max_cand);
  WsLayout w = carve(ws, a.rows, a.max_cand < 1 ? 1 : a.max_cand);
  dim3 grid(nch, a.rows);
  k_sel_init<<<grid, kThreads, 0, st>>>(a, w, nch);
  if (a.is_topk) {
    k_sel_level<1, false><<<grid, kThreads, 0, st>>>(a, w, nch);
    k_sel_level<2, false><<<grid, kThreads, 0, st>>>(a, w, nch);
    k_sel_level<3, false><<<grid, kThreads, 0, st>>>(a, w, nch);
  } else {
    k_sel_level<1, true><<<grid, kThreads, 0, st>>>(a, w, nch);
    k_sel_level<2, true><<<grid, kThreads, 0, st>>>(a, w, nch);
    k_sel_level<3, true><<<grid, kThreads, 0, st>>>(a, w, nch);
  }
  k_sel_ties<<<grid, kThreads, 0, st>>>(a, w, nch);
  k_sel_out<false><<<grid, kThreads, 0, st>>>(a, w, nch);
  k_sel_out<true><<<grid, kThreads, 0, st>>>(a, w, nch);
  return hipGetLastError();
}

}  // namespace sa
