"""Seeded generators for the five workloads of the sparse-attention path.

Bulk normal draws use a torch generator on the device the data will live on
(so the large workloads are drawn directly in GPU memory); every structural
draw (needle and heavy-hitter positions, sequence lengths, page permutations,
heavy-hitter fractions) uses a CPU generator, so the structure of a workload is
identical whichever device draws the values.  Values are drawn in fp32, the
planted signal is added in fp32, and the result is rounded once to the
storage dtype (torch's round-to-nearest-even for bf16).

The caller hands the same tensors (or exact host copies of them) to the HIP
path and to the oracle.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "PAGE",
    "RANK",
    "ALPHA_DECODE64K",
    "ALPHA_BATCHED",
    "DecodeInputs",
    "PrefillInputs",
    "make_tiny_decode",
    "make_decode64k",
    "make_decode1m",
    "make_batched_decode",
    "make_prefill128k",
    "make_prefill_query32k",
    "make_decode_custom",
    "make_prefill_custom",
    "seed_of",
]

PAGE = 64
RANK = 16

# Heavy-hitter strength of the top-p decode workloads.  Frozen from a
# bisection (oracle/calibrate_alpha.py) that brings the top-p(0.9) budget of
# group 0 to 10% of the context on the CPU-drawn 64K workload (8 query heads
# per group) and to 10% on a 64K, 4-heads-per-group, 1%-heavy-hitter row.
ALPHA_DECODE64K = 20.261
ALPHA_BATCHED = 11.577

# Streams of the seed tuple.
_S_Q, _S_K, _S_V, _S_W, _S_POS, _S_LEN, _S_PERM = range(7)


def seed_of(base: int, cfg: int, stream: int, chunk: int = 0) -> int:
    """Mix a (base, config, stream, chunk) tuple into a 63-bit torch seed
    (splitmix64 finaliser applied to a running combination)."""
    mask = (1 << 64) - 1
    z = 0x9E3779B97F4A7C15
    for v in (base, cfg, stream, chunk):
        z = (z ^ (v & mask)) & mask
        z = (z + 0x9E3779B97F4A7C15) & mask
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        z = z ^ (z >> 31)
    return z & ((1 << 63) - 1)


def _gen(device, base, cfg, stream, chunk=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(base, cfg, stream, chunk))
    return g


def _randn(shape, device, base, cfg, stream, chunk=0, std=1.0) -> torch.Tensor:
    g = _gen(device, base, cfg, stream, chunk)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _cpu_perm(n, base, cfg, stream, chunk=0) -> torch.Tensor:
    return torch.randperm(n, generator=_gen("cpu", base, cfg, stream, chunk))


def _unit(v: torch.Tensor) -> torch.Tensor:
    return v / v.norm()


@dataclass
class DecodeInputs:
    """One decode step over a paged key/value cache.

    Layouts (row-major):
      q         [B][H_q][d]
      w_q       [H_q][d][r]       pre-RoPE indexer projector per query head
      w_k       [H_kv][d][r]      pre-RoPE indexer projector per key/value head
      k_pool    [n_pages][H_kv][page][d]
      v_pool    [n_pages][H_kv][page][d]
      page_table[B][max_pages]    int32 pool page of each logical page, -1 pad
      seq_lens  [B]               int32 tokens per sequence
    """

    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    r: int
    dtype: torch.dtype
    seq_lens: list
    page_table: torch.Tensor
    q: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    s_idx: float
    s_att: float
    select: dict = field(default_factory=dict)
    planted: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_pages(self) -> int:
        return self.k_pool.shape[0]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    @property
    def device(self):
        return self.q.device

    def seq_lens_tensor(self) -> torch.Tensor:
        return torch.tensor(self.seq_lens, dtype=torch.int32, device=self.device)

    def _seq_rows(self, pool, b, g) -> torch.Tensor:
        L = self.seq_lens[b]
        npg = (L + PAGE - 1) // PAGE
        pages = self.page_table[b, :npg].long()
        rows = pool[pages, g]  # [npg, page, width]
        return rows.reshape(npg * PAGE, pool.shape[-1])[:L]

    def seq_keys(self, b, g) -> torch.Tensor:
        """Keys of sequence b, group g in token order: [L_b, d]."""
        return self._seq_rows(self.k_pool, b, g)

    def seq_values(self, b, g) -> torch.Tensor:
        return self._seq_rows(self.v_pool, b, g)

    def seq_rows(self, pool, b, g) -> torch.Tensor:
        """Rows of any pool with the same paging (e.g. indexer keys)."""
        return self._seq_rows(pool, b, g)

    def heads(self, g) -> list:
        return list(range(g * self.G, (g + 1) * self.G))

    def to(self, device) -> "DecodeInputs":
        """Copy with every tensor moved to device (bits unchanged)."""
        kw = {f: getattr(self, f) for f in self.__dataclass_fields__}
        for f in ("page_table", "q", "w_q", "w_k", "k_pool", "v_pool"):
            kw[f] = kw[f].to(device)
        return DecodeInputs(**kw)


@dataclass
class PrefillInputs:
    """Causal prefill of one sequence of N tokens.

      q        [N][H_q][d]
      k_pool, v_pool [n_pages][H_kv][page][d]   identity page table
      w_q [H_q][d][r], w_k [H_kv][d][r]
    """

    name: str
    N: int
    H_q: int
    H_kv: int
    d: int
    r: int
    dtype: torch.dtype
    q: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    page_table: torch.Tensor
    s_idx: float
    s_att: float
    b_sel: int = 64
    top_k: int = 2048
    planted: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_blocks(self) -> int:
        return (self.N + self.b_sel - 1) // self.b_sel

    @property
    def device(self):
        return self.q.device

    def keys(self, g) -> torch.Tensor:
        return self.k_pool[:, g].reshape(-1, self.d)[: self.N]

    def values(self, g) -> torch.Tensor:
        return self.v_pool[:, g].reshape(-1, self.d)[: self.N]

    def rows(self, pool, g) -> torch.Tensor:
        return pool[:, g].reshape(self.k_pool.shape[0] * PAGE, pool.shape[-1])[: self.N]

    def heads(self, g) -> list:
        return list(range(g * self.G, (g + 1) * self.G))


def _paged_layout(seq_lens, base, cfg, shuffle: bool):
    npg = [(L + PAGE - 1) // PAGE for L in seq_lens]
    total = sum(npg)
    maxp = max(npg) if npg else 0
    if shuffle:
        ids = _cpu_perm(total, base, cfg, _S_PERM).to(torch.int32)
    else:
        ids = torch.arange(total, dtype=torch.int32)
    table = torch.full((len(seq_lens), max(maxp, 1)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npg):
        table[b, :n] = ids[off : off + n]
        off += n
    return table, total


def _scatter_seq(pool, table_row, L, g, rows):
    """Write token rows [L, d] of one group into their pages of the pool."""
    npg = (L + PAGE - 1) // PAGE
    padded = torch.zeros((npg * PAGE, rows.shape[1]), dtype=pool.dtype, device=pool.device)
    padded[:L] = rows.to(pool.dtype)
    pool[table_row[:npg].long().to(pool.device), g] = padded.view(npg, PAGE, -1)


def _projectors(H_q, H_kv, d, r, device, base, cfg, tied: bool, dtype):
    """W ~ N(0, 1/d).  Tied: W_q[h] = W_k[h // G] (the indexer then sees the
    same low-rank subspace for queries and keys of a group)."""
    G = H_q // H_kv
    w_k = _randn((H_kv, d, r), device, base, cfg, _S_W, 0, std=1.0 / math.sqrt(d))
    if tied:
        w_q = w_k.repeat_interleave(G, dim=0)
    else:
        w_q = _randn((H_q, d, r), device, base, cfg, _S_W, 1, std=1.0 / math.sqrt(d))
    return w_q.to(dtype), w_k.to(dtype)


def make_decode_custom(*, name="custom", B=1, H_q=8, H_kv=2, d=64, seq_lens=(300,),
                       dtype=torch.float32, device="cpu", seed=0, cfg=99,
                       hh_frac=0.0, alpha=0.0, tied=True, shuffle=False,
                       select=None, s_idx=None) -> DecodeInputs:
    """General decode workload: N(0,1) q/K/V, optional heavy hitters (a
    fraction hh_frac of each sequence's tokens per group gets alpha times the
    unit mean query direction of the group added to its key)."""
    r = RANK
    seq_lens = list(seq_lens)
    assert len(seq_lens) == B
    G = H_q // H_kv
    table, total = _paged_layout(seq_lens, seed, cfg, shuffle)
    q32 = _randn((B, H_q, d), device, seed, cfg, _S_Q)
    q = q32.to(dtype)
    w_q, w_k = _projectors(H_q, H_kv, d, r, device, seed, cfg, tied, dtype)
    k_pool = torch.zeros((max(total, 1), H_kv, PAGE, d), dtype=dtype, device=device)
    v_pool = torch.zeros_like(k_pool)
    planted = {}
    qf = q.float()
    for b, L in enumerate(seq_lens):
        if L == 0:
            continue
        for g in range(H_kv):
            chunk = b * H_kv + g
            kk = _randn((L, d), device, seed, cfg, _S_K, chunk)
            vv = _randn((L, d), device, seed, cfg, _S_V, chunk)
            n_hh = int(round(hh_frac * L))
            if n_hh > 0 and alpha != 0.0:
                pos = _cpu_perm(L, seed, cfg, _S_POS, chunk)[:n_hh].sort().values
                u = _unit(qf[b, g * G:(g + 1) * G].mean(dim=0))
                kk[pos.to(device)] += alpha * u
                planted[(b, g)] = pos
            _scatter_seq(k_pool, table[b], L, g, kk)
            _scatter_seq(v_pool, table[b], L, g, vv)
    return DecodeInputs(
        name=name, B=B, H_q=H_q, H_kv=H_kv, d=d, r=r, dtype=dtype,
        seq_lens=seq_lens, page_table=table.to(device), q=q, w_q=w_q, w_k=w_k,
        k_pool=k_pool, v_pool=v_pool,
        s_idx=(math.sqrt(d) / r) if s_idx is None else s_idx,
        s_att=1.0 / math.sqrt(d), select=dict(select or {}), planted=planted)


def make_tiny_decode(device="cpu", seed=0) -> DecodeInputs:
    """Tiny decode: 1 key/value head, 4 query heads, d=64, L=1024, fp32.
    q, K, V iid N(0,1); 8 needle keys set to 3 x the mean query vector of the
    group; independent W_q (one [64 x 16] matrix shared by the 4 heads) and
    W_k, both N(0, 1/d)."""
    cfg = 1
    B, H_q, H_kv, d, r, L = 1, 4, 1, 64, RANK, 1024
    table, total = _paged_layout([L], seed, cfg, False)
    q = _randn((B, H_q, d), device, seed, cfg, _S_Q)
    w_q1 = _randn((d, r), device, seed, cfg, _S_W, 1, std=1.0 / math.sqrt(d))
    w_k = _randn((H_kv, d, r), device, seed, cfg, _S_W, 0, std=1.0 / math.sqrt(d))
    w_q = w_q1.unsqueeze(0).repeat(H_q, 1, 1)
    kk = _randn((L, d), device, seed, cfg, _S_K)
    vv = _randn((L, d), device, seed, cfg, _S_V)
    needles = _cpu_perm(L, seed, cfg, _S_POS)[:8].sort().values
    kk[needles.to(device)] = 3.0 * q[0].mean(dim=0)
    k_pool = torch.zeros((total, H_kv, PAGE, d), dtype=torch.float32, device=device)
    v_pool = torch.zeros_like(k_pool)
    _scatter_seq(k_pool, table[0], L, 0, kk)
    _scatter_seq(v_pool, table[0], L, 0, vv)
    return DecodeInputs(
        name="tiny_decode", B=B, H_q=H_q, H_kv=H_kv, d=d, r=r, dtype=torch.float32,
        seq_lens=[L], page_table=table.to(device), q=q, w_q=w_q, w_k=w_k,
        k_pool=k_pool, v_pool=v_pool, s_idx=math.sqrt(d) / r, s_att=1.0 / math.sqrt(d),
        select={"p": 0.9, "k": 64, "n_sink": 0, "n_window": 0},
        planted={(0, 0): needles})


def make_decode64k(device="cpu", seed=0, L=65536, alpha=ALPHA_DECODE64K) -> DecodeInputs:
    """Decode at 64K: B=1, 32 query / 4 key-value heads, d=128, bf16.  1% of
    the tokens of every group are heavy hitters (alpha times the unit mean
    query direction added); tied projectors; top-p 0.9 with 4 sink and 512
    window tokens always kept."""
    return make_decode_custom(
        name="decode64k", B=1, H_q=32, H_kv=4, d=128, seq_lens=[L], dtype=torch.bfloat16,
        device=device, seed=seed, cfg=2, hh_frac=0.01, alpha=alpha, tied=True,
        shuffle=False, select={"p": 0.9, "n_sink": 4, "n_window": 512})


def make_decode1m(device="cpu", seed=0, L=1 << 20, beta=2.0) -> DecodeInputs:
    """Decode at 1M: B=1, 32/4 heads, d=128, bf16 keys in 64-token pages over
    an N(0,1) background.  Per group, 16 planted pages in 4 runs of 4
    consecutive pages: the 1st and 3rd page of a run get beta times the unit
    mean query direction added to all 64 tokens, the 2nd and 4th get 8*beta
    added to 8 of their tokens (same mean shift, larger variance).  Selection:
    top-32 pages by the Taylor page score."""
    cfg = 3
    B, H_q, H_kv, d, r = 1, 32, 4, 128, RANK
    G = H_q // H_kv
    table, total = _paged_layout([L], seed, cfg, False)
    q = _randn((B, H_q, d), device, seed, cfg, _S_Q).to(torch.bfloat16)
    w_q, w_k = _projectors(H_q, H_kv, d, r, device, seed, cfg, True, torch.bfloat16)
    k_pool = torch.empty((total, H_kv, PAGE, d), dtype=torch.bfloat16, device=device)
    v_pool = torch.empty_like(k_pool)
    n_pages = L // PAGE
    planted = {}
    qf = q.float()
    chunk_pages = 4096
    for g in range(H_kv):
        u = _unit(qf[0, g * G:(g + 1) * G].mean(dim=0))
        # 4 runs of 4 pages at distinct, non-overlapping seeded offsets
        starts = (_cpu_perm(n_pages // 4, seed, cfg, _S_POS, g)[:4] * 4).sort().values
        plan = []
        for s in starts.tolist():
            for o in range(4):
                pg = s + o
                if o % 2 == 0:
                    plan.append((pg, None))
                else:
                    toks = _cpu_perm(PAGE, seed, cfg, _S_POS, 1000 + g * n_pages + pg)[:8]
                    plan.append((pg, toks))
        planted[(0, g)] = torch.tensor([p for p, _ in plan])
        for c0 in range(0, n_pages, chunk_pages):
            c1 = min(n_pages, c0 + chunk_pages)
            chunk = g * 4096 + c0 // chunk_pages
            kk = _randn(((c1 - c0) * PAGE, d), device, seed, cfg, _S_K, chunk)
            vv = _randn(((c1 - c0) * PAGE, d), device, seed, cfg, _S_V, chunk)
            for pg, toks in plan:
                if c0 <= pg < c1:
                    base = (pg - c0) * PAGE
                    if toks is None:
                        kk[base:base + PAGE] += beta * u
                    else:
                        kk[(base + toks).to(device)] += 8.0 * beta * u
            k_pool[c0:c1, g] = kk.view(c1 - c0, PAGE, d).to(torch.bfloat16)
            v_pool[c0:c1, g] = vv.view(c1 - c0, PAGE, d).to(torch.bfloat16)
    return DecodeInputs(
        name="decode1m", B=B, H_q=H_q, H_kv=H_kv, d=d, r=r, dtype=torch.bfloat16,
        seq_lens=[L], page_table=table.to(device), q=q, w_q=w_q, w_k=w_k,
        k_pool=k_pool, v_pool=v_pool, s_idx=math.sqrt(d) / r, s_att=1.0 / math.sqrt(d),
        select={"k_pages": 32}, planted=planted)


def make_batched_decode(device="cpu", seed=0, B=32, L_min=16384, L_max=131072,
                        alpha=ALPHA_BATCHED, f_min=0.005, f_max=0.05) -> DecodeInputs:
    """Batched decode: B sequences with lengths uniform in [L_min, L_max],
    32/8 heads, d=128, bf16, shuffled 64-token pages.  Each (sequence, group)
    draws its heavy-hitter fraction uniformly in [f_min, f_max].  Top-p 0.9
    with 4 sink and 512 window tokens."""
    cfg = 5
    H_q, H_kv, d, r = 32, 8, 128, RANK
    G = H_q // H_kv
    gl = _gen("cpu", seed, cfg, _S_LEN, 0)
    seq_lens = torch.randint(L_min, L_max + 1, (B,), generator=gl).tolist()
    fr = torch.rand((B, H_kv), generator=_gen("cpu", seed, cfg, _S_LEN, 1), dtype=torch.float64)
    fracs = (f_min + (f_max - f_min) * fr).tolist()
    table, total = _paged_layout(seq_lens, seed, cfg, True)
    q = _randn((B, H_q, d), device, seed, cfg, _S_Q).to(torch.bfloat16)
    w_q, w_k = _projectors(H_q, H_kv, d, r, device, seed, cfg, True, torch.bfloat16)
    k_pool = torch.empty((total, H_kv, PAGE, d), dtype=torch.bfloat16, device=device)
    v_pool = torch.empty_like(k_pool)
    qf = q.float()
    planted = {}
    for b, L in enumerate(seq_lens):
        for g in range(H_kv):
            chunk = b * H_kv + g
            kk = _randn((L, d), device, seed, cfg, _S_K, chunk)
            vv = _randn((L, d), device, seed, cfg, _S_V, chunk)
            n_hh = max(1, int(round(fracs[b][g] * L)))
            pos = _cpu_perm(L, seed, cfg, _S_POS, chunk)[:n_hh].sort().values
            u = _unit(qf[b, g * G:(g + 1) * G].mean(dim=0))
            kk[pos.to(device)] += alpha * u
            planted[(b, g)] = pos
            _scatter_seq(k_pool, table[b], L, g, kk)
            _scatter_seq(v_pool, table[b], L, g, vv)
            del kk, vv
    return DecodeInputs(
        name="batched_decode", B=B, H_q=H_q, H_kv=H_kv, d=d, r=r, dtype=torch.bfloat16,
        seq_lens=seq_lens, page_table=table.to(device), q=q, w_q=w_q, w_k=w_k,
        k_pool=k_pool, v_pool=v_pool, s_idx=math.sqrt(d) / r, s_att=1.0 / math.sqrt(d),
        select={"p": 0.9, "n_sink": 4, "n_window": 512},
        planted={"fracs": fracs, **planted})


def make_prefill_custom(*, name="prefill_custom", N=512, H_q=8, H_kv=2, d=64,
                        dtype=torch.bfloat16, device="cpu", seed=0, cfg=98,
                        n_hh=0, q_shift=2.0, k_shift=8.0, b_sel=64, top_k=2048,
                        tied=True) -> PrefillInputs:
    """Causal prefill of N tokens: Q, K, V iid N(0,1); n_hh column heavy
    hitters per group (K += k_shift * u_g at those keys, every query of the
    group's heads += q_shift * u_g, u_g a seeded unit vector)."""
    r = RANK
    G = H_q // H_kv
    table, total = _paged_layout([N], seed, cfg, False)
    q = _randn((N, H_q, d), device, seed, cfg, _S_Q)
    w_q, w_k = _projectors(H_q, H_kv, d, r, device, seed, cfg, tied, dtype)
    k_pool = torch.zeros((total, H_kv, PAGE, d), dtype=dtype, device=device)
    v_pool = torch.zeros_like(k_pool)
    planted = {}
    for g in range(H_kv):
        kk = _randn((N, d), device, seed, cfg, _S_K, g)
        vv = _randn((N, d), device, seed, cfg, _S_V, g)
        if n_hh > 0:
            u = _unit(torch.randn(d, generator=_gen("cpu", seed, cfg, _S_POS, 10 + g),
                                  dtype=torch.float32)).to(device)
            pos = _cpu_perm(N, seed, cfg, _S_POS, g)[:n_hh].sort().values
            kk[pos.to(device)] += k_shift * u
            q[:, g * G:(g + 1) * G] += q_shift * u
            planted[g] = pos
        _scatter_seq(k_pool, table[0], N, g, kk)
        _scatter_seq(v_pool, table[0], N, g, vv)
        del kk, vv
    return PrefillInputs(
        name=name, N=N, H_q=H_q, H_kv=H_kv, d=d, r=r, dtype=dtype, q=q.to(dtype),
        w_q=w_q, w_k=w_k, k_pool=k_pool, v_pool=v_pool, page_table=table.to(device),
        s_idx=math.sqrt(d) / r, s_att=1.0 / math.sqrt(d), b_sel=b_sel, top_k=top_k,
        planted=planted)


def make_prefill_query32k(device="cpu", seed=0, N=32768) -> PrefillInputs:
    """Per-query (b_sel = 1) causal sparse prefill at 32K: the 128K recipe
    (32 query / 8 key-value heads, d=128, bf16, 0.5% column heavy hitters per
    group) with one top-2048 support per query."""
    return make_prefill_custom(
        name="prefill32k_query", N=N, H_q=32, H_kv=8, d=128, dtype=torch.bfloat16, device=device,
        seed=seed, cfg=6, n_hh=int(round(0.005 * N)), q_shift=2.0, k_shift=8.0,
        b_sel=1, top_k=2048, tied=True)


def make_prefill128k(device="cpu", seed=0, N=131072) -> PrefillInputs:
    """Causal sparse prefill at 128K: 32 query / 8 key-value heads, d=128,
    bf16; 0.5% column heavy hitters per group; b_sel=64, top-k 2048."""
    return make_prefill_custom(
        name="prefill128k", N=N, H_q=32, H_kv=8, d=128, dtype=torch.bfloat16, device=device,
        seed=seed, cfg=4, n_hh=int(round(0.005 * N)), q_shift=2.0, k_shift=8.0,
        b_sel=64, top_k=2048, tied=True)
