// Attention-mass oracle support ("Oracle-Guided Sparse Prefill", section 2.1):
// the dense attention distribution of every query head over all cached keys,
// averaged over the heads of the key/value group, is the token importance the
// oracle support is taken from (its top k, or the shortest prefix by mass that
// reaches p), and the yardstick for how much of that mass another support
// covers.
//
// k_mass_logits: one workgroup per (256-token chunk, row).  The chunk's 64-token
// pages of K are staged in LDS with coalesced 16-byte loads (the next two
// pages' loads in flight while the current one is scored); one lane per token forms
// the logits of the group's heads (bf16 pairs through v_dot2_f32_bf16, fp32
// accumulate) in base 2 and writes them to the workspace, and each wave keeps
// a running (max, sum) per head for the chunk.
// k_mass_norm: per row, the chunks' pairs merged into each head's log2
// normaliser (a launch of its own: no cross-workgroup fences in the hot
// kernel).
// k_mass_finish: per token, the natural log of the head mean of
// 2^(logit - normaliser).
// k_coverage: per row, the summed mass of a support and its overlap with a
// reference support.
//
// Bound: HBM bandwidth of the K rows (256 B per token per group for d = 128
// bf16); the base-2 logits make a 4 B per head round trip through the
// workspace.  Deterministic: fixed partition and reduction orders.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kMassChunk = 256;          // tokens per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2m_t;
typedef uint32_t u32x4m_t __attribute__((ext_vector_type(4)));  // register-friendly 16-byte piece

__device__ __forceinline__ float dot2m(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2m_t, a),
                                          __builtin_bit_cast(bf16x2m_t, b), c, false);
}

template <typename T, int D, int G>
struct MassCfg {
  static constexpr int NW = G < 4 ? G : 4;        // waves per workgroup
  static constexpr int HPW = G / NW;              // heads per wave
  static constexpr int NT = NW * kWave;
  static constexpr int ROWB = D * (int)sizeof(T); // bytes per K row
  static constexpr int CPR = ROWB / 16;           // 16-byte pieces per row
  static constexpr int PITCH = ROWB + 16;         // LDS row pitch (bank spread)
  static constexpr int LPT = kPage * CPR / NT;    // pieces per thread per page
  static_assert(kPage * CPR % NT == 0, "page pieces must split evenly");
};

struct MassWs {
  float* lg;        // [rows][G][ldl] base-2 logits
  float2* part;     // [rows][nchunk][G] (max, sum) per chunk and head
  float* norm;      // [rows][G] log2 of each head's softmax normaliser
  int64_t ldl;
  int32_t nchunk;
  int32_t rows_fast;  // grid x = rows (rows sharing a key cache read a chunk together)
};

template <typename T, int D, int G>
__global__ void __launch_bounds__((G < 4 ? G : 4) * 64)
k_mass_logits(const T* __restrict__ q, const T* __restrict__ k_pool,
              const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
              Shape s, float c2, MassWs w) {
  using C = MassCfg<T, D, G>;
  constexpr int QP = G * D * (int)sizeof(T) / 16;        // 16-byte pieces of the group's queries
  constexpr int QPT = (QP + C::NT - 1) / C::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = w.rows_fast ? blockIdx.x : blockIdx.y, ch = w.rows_fast ? blockIdx.y : blockIdx.x;
  const int b = row / s.Hkv, g = row % s.Hkv;
  const int32_t L = clamp_len(seq_lens[b], s.max_len);
  const int32_t t0 = ch * kMassChunk;
  if (t0 >= L) return;  // this chunk is past the sequence: takes no part
  const int32_t t1 = min(L, t0 + kMassChunk);

  __shared__ __align__(16) char Ks[kPage * C::PITCH];
  __shared__ __align__(16) T Qs[G][D];

  // queries first, then the first two pages: waiting for the queries then
  // leaves the page loads in flight
  const char* qsrc = reinterpret_cast<const char*>(q + ((int64_t)b * s.Hq + g * G) * D);
  u32x4m_t qr[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int pc = i * C::NT + tid;
    if (pc < QP) qr[i] = *reinterpret_cast<const u32x4m_t*>(qsrc + pc * 16);
  }
  const int64_t head_stride = (int64_t)kPage * D;
  const int64_t page_stride = (int64_t)s.Hkv * head_stride;
  const int32_t* pt = page_table + (int64_t)b * s.max_pages;
  const char* kbase = reinterpret_cast<const char*>(k_pool + g * head_stride) + tid * 16;
  const int64_t npool = s.n_pool_pages;
  // ts is a multiple of 64 below L, so pt[ts / 64] is a listed page; rows of
  // the last page past L are read (the page exists) and masked below.
#define SA_MASS_LOAD(buf, ts)                                                               \
  do {                                                                                      \
    const char* src_ = kbase + clamp_page(pt[(ts) >> 6], npool) * page_stride * (int64_t)sizeof(T); \
    _Pragma("unroll") for (int i_ = 0; i_ < C::LPT; ++i_)                                   \
      buf[i_] = *reinterpret_cast<const u32x4m_t*>(src_ + i_ * C::NT * 16);                 \
  } while (0)
  u32x4m_t kA[C::LPT], kB[C::LPT];
  SA_MASS_LOAD(kA, t0);
  if (t0 + kPage < t1) SA_MASS_LOAD(kB, t0 + kPage);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int pc = i * C::NT + tid;
    if (pc < QP) *reinterpret_cast<u32x4m_t*>(reinterpret_cast<char*>(&Qs[0][0]) + pc * 16) = qr[i];
  }

  float m_run[C::HPW], l_run[C::HPW];
#pragma unroll
  for (int hh = 0; hh < C::HPW; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
  }
  float* lg_row = w.lg + (int64_t)row * G * w.ldl;

  // one page: stage it in LDS, refill its registers with the page two ahead,
  // score the staged page
#define SA_MASS_PAGE(buf, ts)                                                               \
  do {                                                                                      \
    const int32_t nt_ = min(kPage, t1 - (ts));                                              \
    __syncthreads();                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < C::LPT; ++i_) {                                 \
      const int pc_ = i_ * C::NT + tid;                                                     \
      *reinterpret_cast<u32x4m_t*>(Ks + (pc_ / C::CPR) * C::PITCH + (pc_ % C::CPR) * 16) = buf[i_]; \
    }                                                                                       \
    __syncthreads();                                                                        \
    if ((ts) + 2 * kPage < t1) SA_MASS_LOAD(buf, (ts) + 2 * kPage);                         \
    score_page(ts, nt_);                                                                    \
  } while (0)

  auto score_page = [&](int32_t ts, int32_t nt) {
    float sc[C::HPW];
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) sc[hh] = 0.f;
    const char* krow = Ks + lane * C::PITCH;
#pragma unroll 4
    for (int pc = 0; pc < C::CPR; ++pc) {
      const u32x4m_t kv = *reinterpret_cast<const u32x4m_t*>(krow + pc * 16);
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) {
        const int h = wave * C::HPW + hh;
        float a = sc[hh];
        if constexpr (sizeof(T) == 2) {
          const u32x4m_t qv = *reinterpret_cast<const u32x4m_t*>(&Qs[h][pc * 8]);
          a = dot2m(kv.x, qv.x, a);
          a = dot2m(kv.y, qv.y, a);
          a = dot2m(kv.z, qv.z, a);
          a = dot2m(kv.w, qv.w, a);
        } else {
          const float4 qv = *reinterpret_cast<const float4*>(&Qs[h][pc * 4]);
          a = fmaf(__uint_as_float(kv.x), qv.x, a);
          a = fmaf(__uint_as_float(kv.y), qv.y, a);
          a = fmaf(__uint_as_float(kv.z), qv.z, a);
          a = fmaf(__uint_as_float(kv.w), qv.w, a);
        }
        sc[hh] = a;
      }
    }
    const bool ok = lane < nt;
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) {
      const int h = wave * C::HPW + hh;
      const float a = sc[hh] * c2;
      if (ok) lg_row[(int64_t)h * w.ldl + ts + lane] = a;
      const float m_new = fmaxf(m_run[hh], wave_max(ok ? a : -INFINITY));
      const float e = ok ? exp2f(a - m_new) : 0.f;
      l_run[hh] = l_run[hh] * exp2f(m_run[hh] - m_new) + wave_sum(e);
      m_run[hh] = m_new;
    }
  };

  for (int32_t ts = t0; ts < t1; ts += 2 * kPage) {
    SA_MASS_PAGE(kA, ts);
    if (ts + kPage < t1) SA_MASS_PAGE(kB, ts + kPage);
  }
#undef SA_MASS_PAGE
#undef SA_MASS_LOAD

  // ---- the chunk's (max, sum) per head ----
  float2* part = w.part + ((int64_t)row * w.nchunk + ch) * G;
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < C::HPW; ++hh) part[wave * C::HPW + hh] = make_float2(m_run[hh], l_run[hh]);
  }
}

// Per row and head: merge the chunks' (max, sum) pairs in chunk order into
// log2 of the softmax normaliser.  One wave per head.
template <int G>
__global__ void __launch_bounds__(256)
k_mass_norm(const int32_t* __restrict__ seq_lens, Shape s, MassWs w) {
  const int row = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t L = clamp_len(seq_lens[row / s.Hkv], s.max_len);
  if (L == 0) return;
  const int32_t nch = (L + kMassChunk - 1) / kMassChunk;
  const float2* prow = w.part + (int64_t)row * w.nchunk * G;
  constexpr int kBatch = 8;  // pairs per lane loaded before merging
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY, l = 0.f;
    for (int c0 = 0; c0 < nch; c0 += kBatch * kWave) {  // lane's chunks in chunk order
      float2 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int c = c0 + k * kWave + lane;
        v[k] = c < nch ? prow[(int64_t)c * G + h] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float mn = fmaxf(m, v[k].x);
        l = (mn == -INFINITY) ? 0.f : l * exp2f(m - mn) + v[k].y * exp2f(v[k].x - mn);
        m = mn;
      }
    }
    const float M = wave_max(m);
    const float Ls = wave_sum(m == -INFINITY ? 0.f : l * exp2f(m - M));
    if (lane == 0) w.norm[(int64_t)row * G + h] = M + log2f(Ls);
  }
}

template <int G>
__global__ void __launch_bounds__(256)
k_mass_finish(const int32_t* __restrict__ seq_lens, Shape s, MassWs w, float* __restrict__ x,
              int64_t ldx) {
  const int row = w.rows_fast ? blockIdx.x : blockIdx.y, ch = w.rows_fast ? blockIdx.y : blockIdx.x;
  const int b = row / s.Hkv;
  const int32_t L = clamp_len(seq_lens[b], s.max_len);
  const int32_t t0 = ch * kMassChunk;
  if (t0 >= L) return;
  const int32_t t1 = min(L, t0 + kMassChunk);
  __shared__ float nrm[G];
  if (threadIdx.x < G) nrm[threadIdx.x] = w.norm[(int64_t)row * G + threadIdx.x];
  __syncthreads();
  const float* lg_row = w.lg + (int64_t)row * G * w.ldl;
  const float lnG = logf((float)G);
  for (int32_t j = t0 + threadIdx.x; j < t1; j += 256) {
    float u[G];
    float M = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u[h] = lg_row[(int64_t)h * w.ldl + j] - nrm[h];  // log2 of head h's probability
      M = fmaxf(M, u[h]);
    }
    float sum = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) sum += exp2f(u[h] - M);
    x[(int64_t)row * ldx + j] = kLn2 * (M + log2f(sum)) - lnG;
  }
}

__global__ void __launch_bounds__(256)
k_coverage(const float* __restrict__ x, int64_t ldx, const int32_t* __restrict__ seq_lens,
           int32_t Hkv, int32_t max_len, const int32_t* __restrict__ idx,
           const int32_t* __restrict__ count, int32_t cap, const int32_t* __restrict__ ridx,
           const int32_t* __restrict__ rcount, int32_t rcap, float* __restrict__ mass,
           int32_t* __restrict__ overlap) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t L = clamp_len(seq_lens[row / Hkv], max_len);
  int32_t n = count[row];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int32_t* list = idx + (int64_t)row * cap;
  int32_t nr = 0;
  const int32_t* rl = nullptr;
  if (ridx) {
    nr = rcount[row];
    nr = nr < 0 ? 0 : (nr > rcap ? rcap : nr);
    rl = ridx + (int64_t)row * rcap;
  }
  const float* xr = x + (int64_t)row * ldx;
  float m = 0.f;
  uint32_t hit = 0;
  for (int32_t i = tid; i < n; i += 256) {
    const int32_t j = list[i];
    if (j < 0 || j >= L) continue;
    m += expf(xr[j]);
    if (rl) {  // first reference entry >= j (reference ascending)
      int32_t lo = 0, hi = nr;
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (rl[mid] < j) lo = mid + 1; else hi = mid;
      }
      hit += (lo < nr && rl[lo] == j) ? 1u : 0u;
    }
  }
  __shared__ float sm[4];
  __shared__ uint32_t sh[4];
  const float ms = wave_sum(m);
  const uint32_t hs = wave_sum_u32(hit);
  if (lane == 0) {
    sm[wave] = ms;
    sh[wave] = hs;
  }
  __syncthreads();
  if (tid == 0) {
    mass[row] = ((sm[0] + sm[1]) + sm[2]) + sm[3];
    if (overlap) overlap[row] = (int32_t)(sh[0] + sh[1] + sh[2] + sh[3]);
  }
}

// Block form of the prefill oracle: xb[(b, g)][j] = ln of the mean over the
// block's rows r of exp(x[(r, g)][j]) (each row's head-averaged causal
// distribution) for the candidates j < 64 * (blk0 + b) of earlier blocks.
__global__ void __launch_bounds__(256)
k_block_mass(const float* __restrict__ x, int64_t ldx, int32_t nq, int32_t Hkv, int32_t blk0,
             float* __restrict__ xb) {
  const int b = blockIdx.y, g = blockIdx.z;
  const int32_t j = blockIdx.x * 256 + threadIdx.x;
  const int32_t n_cand = kPage * (blk0 + b);
  if (j >= n_cand) return;
  const int r0 = b * kPage, nr = min(kPage, nq - r0);
  float acc = 0.f;
  for (int r = 0; r < nr; ++r) acc += expf(x[((int64_t)(r0 + r) * Hkv + g) * ldx + j]);
  xb[((int64_t)b * Hkv + g) * ldx + j] = logf(acc / (float)nr);
}

__global__ void k_slab_lens(int32_t* __restrict__ lens, int32_t n, int32_t first) {
  const int32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) lens[i] = first + i + 1;
}

struct MassLayout {
  int64_t ldl;
  int32_t nchunk;
  size_t off_part, off_norm, total;
};

MassLayout mass_layout(const Shape& s) {
  MassLayout m;
  const int64_t rows = (int64_t)s.B * s.Hkv;
  const int G = s.Hq / s.Hkv;
  m.nchunk = (int32_t)((s.max_len + kMassChunk - 1) / kMassChunk);
  if (m.nchunk < 1) m.nchunk = 1;
  m.ldl = (int64_t)m.nchunk * kMassChunk;
  size_t off = align_up((size_t)rows * G * m.ldl * sizeof(float), 256);
  m.off_part = off;
  off += align_up((size_t)rows * m.nchunk * G * sizeof(float2), 256);
  m.off_norm = off;
  off += align_up((size_t)rows * G * sizeof(float), 256);
  m.total = off;
  return m;
}

template <typename T, int D>
hipError_t launch_mass_t(const Shape& s, const sa_pages& pg, const void* q, const void* k_pool,
                         float s_att, float* x, int64_t ldx, const MassWs& w, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  const dim3 grid = w.rows_fast ? dim3(s.B * s.Hkv, w.nchunk) : dim3(w.nchunk, s.B * s.Hkv);
  const float c2 = s_att * kLog2e;
#define SA_MASS_G(GG)                                                                          \
  case GG:                                                                                     \
    k_mass_logits<T, D, GG><<<grid, MassCfg<T, D, GG>::NT, 0, st>>>(                           \
        (const T*)q, (const T*)k_pool, pg.page_table, pg.seq_lens, s, c2, w);                  \
    k_mass_norm<GG><<<s.B * s.Hkv, 256, 0, st>>>(pg.seq_lens, s, w);                           \
    k_mass_finish<GG><<<grid, 256, 0, st>>>(pg.seq_lens, s, w, x, ldx);                        \
    break;
  switch (G) {
    SA_MASS_G(1)
    SA_MASS_G(2)
    SA_MASS_G(4)
    SA_MASS_G(8)
    SA_MASS_G(16)
    default: return hipErrorNotSupported;
  }
#undef SA_MASS_G
  return hipGetLastError();
}

// Prefill oracle plan: query slabs of up to 256 queries (a multiple of 64,
// at most 4096 (query, group) rows per launch).
struct OracleLayout {
  int32_t qs;
  size_t off_lens, off_x, off_xb, off_mass, off_sel, total;
};

OracleLayout oracle_layout(const Shape& s, int32_t n_tokens) {
  OracleLayout L;
  int32_t q = (4096 / s.Hkv) / kPage * kPage;
  L.qs = q < kPage ? kPage : (q > 256 ? 256 : q);
  Shape s2 = s;
  s2.B = L.qs;
  s2.max_len = n_tokens;
  size_t off = 0;
  L.off_lens = off;
  off += align_up((size_t)L.qs * sizeof(int32_t), 256);
  L.off_x = off;
  off += align_up((size_t)L.qs * s.Hkv * (size_t)n_tokens * sizeof(float), 256);
  L.off_xb = off;
  off += align_up((size_t)(L.qs / kPage) * s.Hkv * (size_t)n_tokens * sizeof(float), 256);
  L.off_mass = off;
  off += align_up(mass_layout(s2).total, 256);
  L.off_sel = off;
  off += align_up(select_workspace_bytes(L.qs * s.Hkv, n_tokens), 256);
  L.total = off;
  return L;
}

}  // namespace

size_t mass_workspace_bytes(const Shape& s) { return mass_layout(s).total; }

size_t prefill_oracle_workspace_bytes(const Shape& s, int32_t n_tokens) {
  return oracle_layout(s, n_tokens).total;
}

hipError_t launch_prefill_oracle_select(const Shape& s, const sa_pages& pg, int32_t n_tokens,
                                        const void* q, const void* k_pool, sa_dtype dt,
                                        float s_att, int32_t b_sel, int32_t k, int32_t* idx,
                                        int32_t* count, int32_t cap, void* ws, hipStream_t st) {
  const OracleLayout L = oracle_layout(s, n_tokens);
  char* base = (char*)ws;
  int32_t* lens = (int32_t*)(base + L.off_lens);
  float* xq = (float*)(base + L.off_x);
  float* xb = (float*)(base + L.off_xb);
  const size_t qe = dt == SA_BF16 ? 2 : 4;
  for (int32_t q0 = 0; q0 < n_tokens; q0 += L.qs) {
    const int32_t nq = n_tokens - q0 < L.qs ? n_tokens - q0 : L.qs;
    k_slab_lens<<<(nq + 255) / 256, 256, 0, st>>>(lens, nq, q0);
    Shape s2 = s;
    s2.B = nq;
    s2.max_len = n_tokens;
    s2.max_pages = 0;  // every query row reads page-table row 0
    sa_pages p2;
    p2.page_table = pg.page_table;
    p2.seq_lens = lens;
    hipError_t e = launch_attention_mass(s2, p2, (const char*)q + (size_t)q0 * s.Hq * s.D * qe,
                                         k_pool, dt, s_att, xq, n_tokens, base + L.off_mass, st,
                                         /*rows_fast=*/true);
    if (e != hipSuccess) return e;
    SelectArgs a{};
    a.ldx = n_tokens;
    a.seq_lens = nullptr;
    a.Hkv = s.Hkv;
    a.max_len = n_tokens;
    a.unit = 1;
    a.is_topk = 1;
    a.p = 0.f;
    a.k = k;
    a.n_sink = 0;
    a.cap = cap;
    if (b_sel == 1) {  // per query: candidates j <= i, the own token always kept
      a.x = xq;
      a.rows = nq * s.Hkv;
      a.max_cand = q0 + nq;
      a.n_window = 1;
      a.idx = idx + (int64_t)q0 * s.Hkv * cap;
      a.count = count + (int64_t)q0 * s.Hkv;
      a.prefill_bsel = 1;
      a.prefill_blk0 = q0;
      a.prefill_self = 1;
    } else {  // per 64-query block: candidates of earlier blocks
      const int32_t blk0 = q0 / kPage, nb = (nq + kPage - 1) / kPage;
      const int32_t cand_hi = kPage * (blk0 + nb - 1);
      if (cand_hi > 0) {
        dim3 grid((cand_hi + 255) / 256, nb, s.Hkv);
        k_block_mass<<<grid, 256, 0, st>>>(xq, n_tokens, nq, s.Hkv, blk0, xb);
      }
      a.x = xb;
      a.rows = nb * s.Hkv;
      a.max_cand = cand_hi > 0 ? cand_hi : 1;
      a.n_window = 0;
      a.idx = idx + (int64_t)blk0 * s.Hkv * cap;
      a.count = count + (int64_t)blk0 * s.Hkv;
      a.prefill_bsel = kPage;
      a.prefill_blk0 = blk0;
      a.prefill_self = 0;
    }
    e = launch_select(a, base + L.off_sel, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_attention_mass(const Shape& s, const sa_pages& pg, const void* q, const void* k_pool,
                                 sa_dtype dt, float s_att, float* x, int64_t ldx, void* ws,
                                 hipStream_t st, bool rows_fast) {
  const MassLayout m = mass_layout(s);
  char* base = (char*)ws;
  MassWs w;
  w.lg = (float*)base;
  w.part = (float2*)(base + m.off_part);
  w.norm = (float*)(base + m.off_norm);
  w.ldl = m.ldl;
  w.nchunk = m.nchunk;
  w.rows_fast = rows_fast && m.nchunk <= 65535 ? 1 : 0;
  if (dt == SA_BF16)
    return s.D == 128 ? launch_mass_t<bf16_raw, 128>(s, pg, q, k_pool, s_att, x, ldx, w, st)
                      : launch_mass_t<bf16_raw, 64>(s, pg, q, k_pool, s_att, x, ldx, w, st);
  return s.D == 128 ? launch_mass_t<float, 128>(s, pg, q, k_pool, s_att, x, ldx, w, st)
                    : launch_mass_t<float, 64>(s, pg, q, k_pool, s_att, x, ldx, w, st);
}

hipError_t launch_coverage(const Shape& s, const sa_pages& pg, const float* x, int64_t ldx,
                           const int32_t* idx, const int32_t* count, int32_t cap,
                           const int32_t* ridx, const int32_t* rcount, int32_t rcap, float* mass,
                           int32_t* overlap, hipStream_t st) {
  k_coverage<<<s.B * s.Hkv, 256, 0, st>>>(x, ldx, pg.seq_lens, s.Hkv, s.max_len, idx, count, cap,
                                          ridx, rcount, rcap, mass, overlap);
  return hipGetLastError();
}

}  // namespace sa
