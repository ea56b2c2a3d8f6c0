"""Seeded synthetic inputs for drafter block attention.

This module only draws and lays out inputs: it holds none of the method's
arithmetic (no normalisation, rotation, scores or softmax).  Both the fp64
oracle (``oracle/``) and the HIP path (``speculative_decoding_drafter_amd``)
consume what it produces; neither side imports the other.

Problem shape (TensorRT-LLM PR #20532 "Share Kimi K3 FP4 modeling and add
NVFP4 support on SM103", Conversation, the commit that adds
k3_drafter_attn / k3_drafter_attn_qknorm): up to 8 requests, each with a
draft block of up to 8 tokens; GQA with 6 query heads per KV head; head_dim
64; HND pages of 64 tokens; head layouts 6/1 and 24/4; context lengths 0 to
2041; dense or strided page-table rows with padded page strides; int32 or
int64 positions.

Layouts produced here (the readings the library documents in its header):

* ``qkv``: bf16 ``[R*T, row_stride]``; columns ``[q heads | k heads | v heads]``,
  each head 64 wide, request-major rows (``row = r*T + t``).
* pool: bf16 ``[P, 2, Hkv, 64, 64]`` (page, K/V, head, token slot, dim), so
  ``k_pool = pool[:, 0]`` and ``v_pool = pool[:, 1]`` share one page stride
  of ``2*Hkv*64*64`` elements.  ``separate_pools=True`` gives two
  ``[P, Hkv, 64, 64]`` tensors instead.
* page table: int32 ``[R, stride]``; logical page ``j`` of request ``r`` lives
  at physical page ``page_table[r, j]``.  Physical pages are handed out from a
  seeded permutation of the pool, in logical order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

HEAD_DIM = 64
PAGE = 64
GQA = 6
POISON_PAGE_ID = 0x7FFFFFFF


@dataclasses.dataclass
class DrafterCase:
    """One seeded problem instance, all tensors on the CPU."""

    R: int
    T: int
    Hq: int
    Hkv: int
    qkv: torch.Tensor             # bf16 [R*T, qkv_row_stride]
    k_pool: torch.Tensor          # bf16 [P, Hkv, 64, 64] (possibly a strided view)
    v_pool: torch.Tensor          # bf16 [P, Hkv, 64, 64] (possibly a strided view)
    pool: Optional[torch.Tensor]  # bf16 [P, 2, Hkv, 64, 64] backing store, or None
    page_table: torch.Tensor      # int32 [R, stride]
    context_lens: torch.Tensor    # int32 [R]
    block_lens: Optional[torch.Tensor]  # int32 [R] or None (= all T)
    positions: Optional[torch.Tensor]   # int32 / int64 [R*T] or None
    q_norm_weight: Optional[torch.Tensor]  # bf16 [64] or None
    k_norm_weight: Optional[torch.Tensor]  # bf16 [64] or None
    scale: float
    eps: float = 1e-5
    rope_base: float = 10000.0
    qknorm: bool = False
    name: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def stride(self) -> int:
        return int(self.page_table.shape[1])

    def kv_bytes(self) -> int:
        """Bytes of context K and V the definition reads (each bf16 element once)."""
        L = self.context_lens.to(torch.int64)
        return int(L.sum()) * self.Hkv * HEAD_DIM * 2 * 2

    # ---- float64 numpy views for the oracle (values are exact bf16 values) ----
    def np_args(self, pools=None) -> dict:
        """Oracle arguments; ``pools=(k, v)`` passes already converted float64 pools."""
        f = lambda t: None if t is None else t.to(torch.float64).numpy()
        i = lambda t: None if t is None else t.to(torch.int64).numpy()
        kp, vp = pools if pools is not None else (f(self.k_pool), f(self.v_pool))
        return dict(
            qkv=f(self.qkv), k_pool=kp, v_pool=vp,
            page_table=i(self.page_table), context_lens=i(self.context_lens),
            block_lens=i(self.block_lens), positions=i(self.positions),
            q_norm_weight=f(self.q_norm_weight), k_norm_weight=f(self.k_norm_weight),
            num_q_heads=self.Hq, num_kv_heads=self.Hkv, tokens_per_block=self.T,
            scale=self.scale, eps=self.eps, rope_base=self.rope_base,
        )


def _bf16(a: np.ndarray) -> torch.Tensor:
    """Round fp32 draws to bf16 (round to nearest even, torch's conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def draw_lengths(rng: np.random.Generator, R: int, lo: int = 0, hi: int = 2041,
                 force_extremes: bool = True) -> List[int]:
    """Context lengths ~ U{lo..hi}; with R >= 2, two random requests get lo and hi."""
    lens = rng.integers(lo, hi + 1, size=R).tolist()
    if force_extremes and R >= 2:
        a, b = rng.choice(R, size=2, replace=False)
        lens[int(a)] = lo
        lens[int(b)] = hi
    elif force_extremes and R == 1:
        lens[0] = int(rng.choice([lo, hi]))
    return [int(x) for x in lens]


def make_case(R: int, T: int, Hq: int, Hkv: int, lens: Sequence[int], *,
              seed: int, stride: Optional[int] = None, pool_pages: Optional[int] = None,
              qknorm: bool = False, pos_dtype: torch.dtype = torch.int32,
              block_lens: Optional[Sequence[int]] = None, poison: bool = False,
              separate_pools: bool = False, qkv_row_pad: int = 0,
              scale: Optional[float] = None, v_mean: float = 0.0,
              pos_offset: Optional[Sequence[int]] = None, name: str = "",
              pool_override: Optional[torch.Tensor] = None) -> DrafterCase:
    """Draw one case.

    q/k/v and pool values ~ N(0,1) (V ~ N(v_mean, 1)), rounded to bf16.
    Positions are ``context_len + t`` (plus ``pos_offset[r]`` when given).
    ``poison=True`` fills every pool element the definition never reads
    (unreferenced pages, slots past the context length in the last page),
    the qkv row padding and rows past a block length with NaN, and the unused
    page-table entries with 0x7FFFFFFF.  ``pool_override`` reuses an existing
    ``[P, 2, Hkv, 64, 64]`` bf16 pool instead of drawing one (no poison then).
    """
    assert len(lens) == R
    rng = np.random.default_rng(seed)
    D = HEAD_DIM
    npg = [math.ceil(L / PAGE) for L in lens]
    if stride is None:
        stride = max(npg) if npg else 0
    assert stride >= max(npg, default=0)
    need = sum(npg)
    if pool_pages is None:
        pool_pages = max(need, 1)
    assert pool_pages >= need

    width = (Hq + 2 * Hkv) * D
    qkv = rng.standard_normal((R * T, width + qkv_row_pad), dtype=np.float32)
    vcol = slice((Hq + Hkv) * D, width)
    qkv[:, vcol] += v_mean
    if pool_override is not None:
        assert not poison and tuple(pool_override.shape) == (pool_pages, 2, Hkv, PAGE, D)
        pool = None
    else:
        pool = rng.standard_normal((pool_pages, 2, Hkv, PAGE, D), dtype=np.float32)
        pool[:, 1] += v_mean

    perm = rng.permutation(pool_pages)
    wq = rng.uniform(0.5, 1.5, size=D)
    wk = rng.uniform(0.5, 1.5, size=D)
    # unused table entries come from a child stream so that the poisoned and the
    # clean draw of one seed agree on every value the definition reads
    fill_rng = np.random.default_rng([seed, 1])
    table = np.zeros((R, stride), dtype=np.int64)
    cursor = 0
    for r in range(R):
        for j in range(npg[r]):
            table[r, j] = perm[cursor]
            cursor += 1
        if poison:
            table[r, npg[r]:] = POISON_PAGE_ID
        else:
            # unused entries still hold in-range ids, drawn at random
            table[r, npg[r]:] = fill_rng.integers(0, pool_pages, size=stride - npg[r])

    bl = None
    if block_lens is not None:
        bl = [int(b) for b in block_lens]
        assert all(1 <= b <= T for b in bl)

    if poison:
        used = np.zeros(pool_pages, dtype=bool)
        for r in range(R):
            used[table[r, :npg[r]]] = True
            rem = lens[r] - (npg[r] - 1) * PAGE if npg[r] else PAGE
            if npg[r] and rem < PAGE:
                pool[table[r, npg[r] - 1], :, :, rem:, :] = np.nan
        pool[~used] = np.nan
        if qkv_row_pad:
            qkv[:, width:] = np.nan
        if bl is not None:
            for r in range(R):
                qkv[r * T + bl[r]:(r + 1) * T, :] = np.nan

    qkv_t = _bf16(qkv)
    pool_t = pool_override if pool_override is not None else _bf16(pool)
    if separate_pools:
        k_pool = pool_t[:, 0].contiguous()
        v_pool = pool_t[:, 1].contiguous()
        pool_keep = None
    else:
        k_pool = pool_t[:, 0]
        v_pool = pool_t[:, 1]
        pool_keep = pool_t

    positions = qn = kn = None
    if qknorm:
        off = [0] * R if pos_offset is None else list(pos_offset)
        pos = np.array([lens[r] + off[r] + t for r in range(R) for t in range(T)], dtype=np.int64)
        positions = torch.from_numpy(pos).to(pos_dtype)
        qn = _bf16(wq)
        kn = _bf16(wk)

    return DrafterCase(
        R=R, T=T, Hq=Hq, Hkv=Hkv, qkv=qkv_t, k_pool=k_pool, v_pool=v_pool, pool=pool_keep,
        page_table=torch.from_numpy(table).to(torch.int32),
        context_lens=torch.tensor(list(lens), dtype=torch.int32),
        block_lens=None if bl is None else torch.tensor(bl, dtype=torch.int32),
        positions=positions, q_norm_weight=qn, k_norm_weight=kn,
        scale=1.0 / math.sqrt(D) if scale is None else scale, qknorm=qknorm, name=name)


def device_normal_pool(pages: int, Hkv: int, *, seed: int, device, chunk_pages: int = 2048) -> torch.Tensor:
    """A ``[pages, 2, Hkv, 64, 64]`` bf16 pool ~ N(0,1) drawn on ``device`` with torch's seeded
    counter-based generator, a chunk of pages at a time -- for pools too large to draw on the
    host in reasonable time (pass it to ``make_case(pool_override=...)``)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    pool = torch.empty((pages, 2, Hkv, PAGE, HEAD_DIM), dtype=torch.bfloat16, device=device)
    for p0 in range(0, pages, chunk_pages):
        p1 = min(pages, p0 + chunk_pages)
        pool[p0:p1] = torch.randn((p1 - p0, 2, Hkv, PAGE, HEAD_DIM), generator=gen, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    return pool


# --------------------------------------------------------------------------------------
# The five benchmark-style workloads
# --------------------------------------------------------------------------------------

def config1(k: int = 0, poison: bool = False) -> DrafterCase:
    """1 request x 8 tokens, 6/1 heads, L=64 (one page) in a 4-page pool, plain path."""
    rng = np.random.default_rng(1000 * 1 + k)
    seed = int(rng.integers(1 << 31))
    return make_case(1, 8, 6, 1, [64], seed=seed, stride=1, pool_pages=4, qknorm=False,
                     poison=poison, name="cfg1")


def config2(k: int = 0, poison: bool = False) -> DrafterCase:
    """8x8, 6/1 heads, qknorm, L ~ U{0..2041} (0 and 2041 forced), 512-page pool,
    dense int32 rows (stride 32), int32 positions."""
    rng = np.random.default_rng(1000 * 2 + k)
    lens = draw_lengths(rng, 8)
    seed = int(rng.integers(1 << 31))
    return make_case(8, 8, 6, 1, lens, seed=seed, stride=32, pool_pages=512, qknorm=True,
                     pos_dtype=torch.int32, poison=poison, name="cfg2")


def config3(k: int = 0, poison: bool = False) -> DrafterCase:
    """8x8, 24/4 heads, qknorm, mixed L, strided rows with stride 40, int64 positions."""
    rng = np.random.default_rng(1000 * 3 + k)
    lens = draw_lengths(rng, 8)
    seed = int(rng.integers(1 << 31))
    return make_case(8, 8, 24, 4, lens, seed=seed, stride=40, pool_pages=512, qknorm=True,
                     pos_dtype=torch.int64, poison=poison, name="cfg3")


def config4_pool(hkv: int) -> torch.Tensor:
    """The 512-page pool shared by every cell of one head layout in the split sweep."""
    rng = np.random.default_rng(1000 * 4 + hkv)
    return _bf16(rng.standard_normal((512, 2, hkv, PAGE, HEAD_DIM), dtype=np.float32))


def config4_cell(r: int, t: int, hkv: int, k: int = 0, poison: bool = False,
                 pool: Optional[torch.Tensor] = None) -> DrafterCase:
    """One cell of the split sweep: r requests x t tokens, 6/1 (hkv=1) or 24/4 (hkv=4),
    qknorm, L ~ U{0..2041}, dense rows of stride 32 in a 512-page pool; int32
    positions for 6/1, int64 for 24/4.  ``k`` indexes the redraw (replay)."""
    rng = np.random.default_rng(1000 * 4 + 97 * (r * 8 + t) + 13 * hkv + 100003 * k)
    lens = draw_lengths(rng, r, force_extremes=(k == 0))
    seed = int(rng.integers(1 << 31))
    return make_case(r, t, 6 * hkv, hkv, lens, seed=seed, stride=32, pool_pages=512,
                     qknorm=True, pos_dtype=torch.int32 if hkv == 1 else torch.int64,
                     poison=poison, name=f"cfg4_r{r}t{t}h{hkv}_{k}", pool_override=pool)


def config5(k: int = 0, poison: bool = False) -> DrafterCase:
    """8x8, 24/4 heads, qknorm, L = 32768 per request (512 pages each), 4096 pages
    shuffled across a 5000-page pool, dense rows (stride 512), int32 positions."""
    rng = np.random.default_rng(1000 * 5 + k)
    seed = int(rng.integers(1 << 31))
    return make_case(8, 8, 24, 4, [32768] * 8, seed=seed, stride=512, pool_pages=5000,
                     qknorm=True, pos_dtype=torch.int32, poison=poison, name="cfg5")


CONFIGS = {1: config1, 2: config2, 3: config3, 5: config5}


def make_config(n: int, k: int = 0, poison: bool = False) -> DrafterCase:
    return CONFIGS[n](k, poison=poison)


def with_append_room(case: DrafterCase, seed: int) -> DrafterCase:
    """The same case with room to append every block to its request's paged row.

    Each request gets fresh pool pages for the logical pages its ``L + T``
    tokens need beyond its context (pages added at the end of the pool, values
    ~ N(0,1)), and the page table gets the columns to name them; no two
    requests share a page.  Needs a case drawn with one pool tensor.
    """
    assert case.pool is not None, "needs a case with a single [P, 2, Hkv, 64, 64] pool"
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in case.context_lens.tolist()]
    have = [math.ceil(L / PAGE) for L in lens]
    need = [math.ceil((L + case.T) / PAGE) for L in lens]
    extra = sum(n - h for n, h in zip(need, have))
    stride = max([case.stride] + need)
    P = case.num_pages
    add = _bf16(rng.standard_normal((extra, 2, case.Hkv, PAGE, HEAD_DIM), dtype=np.float32))
    pool = torch.cat([case.pool, add], dim=0)
    table = torch.from_numpy(rng.integers(0, P + extra, size=(case.R, stride))).to(torch.int32)
    table[:, :case.stride] = case.page_table
    nxt = P
    for r in range(case.R):
        for j in range(have[r], need[r]):
            table[r, j] = nxt
            nxt += 1
    return dataclasses.replace(case, pool=pool, k_pool=pool[:, 0], v_pool=pool[:, 1], page_table=table)


def splice_request(base: DrafterCase, donor: DrafterCase, k: int) -> DrafterCase:
    """``base`` with request ``k``'s inputs taken from ``donor``: its qkv rows, page-table row,
    context length, positions and block length.  Both cases must have the same sizes and
    share one pool (e.g. split-sweep cells drawn over ``config4_pool``)."""
    assert (base.R, base.T, base.Hq, base.Hkv, base.stride) == (donor.R, donor.T, donor.Hq, donor.Hkv, donor.stride)
    T = base.T
    rows = slice(k * T, (k + 1) * T)
    out = dataclasses.replace(base)
    out.qkv = base.qkv.clone()
    out.qkv[rows] = donor.qkv[rows]
    out.page_table = base.page_table.clone()
    out.page_table[k] = donor.page_table[k]
    out.context_lens = base.context_lens.clone()
    out.context_lens[k] = donor.context_lens[k]
    if base.positions is not None:
        out.positions = base.positions.clone()
        out.positions[rows] = donor.positions[rows]
    if base.block_lens is not None:
        out.block_lens = base.block_lens.clone()
        out.block_lens[k] = donor.block_lens[k]
    out.name = f"{base.name}+r{k}from{donor.name}"
    return out


@dataclasses.dataclass
class NormRopeRows:
    """Inputs of the standalone q/k norm + rotation op: packed rows, one position each."""
    qkv: torch.Tensor            # bf16 [N, (Hq + 2 Hkv) * 64 + pad]
    positions: torch.Tensor      # int32 / int64 [N]
    q_norm_weight: torch.Tensor  # bf16 [64]
    k_norm_weight: torch.Tensor  # bf16 [64]
    Hq: int
    Hkv: int


def make_norm_rope_rows(N: int, Hkv: int, *, seed: int, row_pad: int = 0, pos_dtype=torch.int32,
                        pos_max: int = 40000, poison_pad: bool = False) -> NormRopeRows:
    """Seeded rows: values ~ N(0,1), weights ~ U(0.5, 1.5), positions ~ U{0..pos_max};
    padding columns are N(0,1) or, with poison_pad, NaN."""
    rng = np.random.default_rng(seed)
    Hq = 6 * Hkv
    width = (Hq + 2 * Hkv) * 64
    vals = rng.standard_normal((N, width + row_pad)).astype(np.float32)
    if poison_pad and row_pad:
        vals[:, width:] = np.nan
    wq = rng.uniform(0.5, 1.5, 64)
    wk = rng.uniform(0.5, 1.5, 64)
    pos = rng.integers(0, pos_max + 1, N)
    return NormRopeRows(qkv=_bf16(vals), positions=torch.from_numpy(pos).to(pos_dtype),
                        q_norm_weight=_bf16(wq), k_norm_weight=_bf16(wk), Hq=Hq, Hkv=Hkv)


def to_device(case: DrafterCase, device) -> DrafterCase:
    """Copy every tensor of a case to ``device`` (keeping the pool views' strides)."""
    d = dataclasses.replace(case)
    mv = lambda t: None if t is None else t.to(device)
    if case.pool is not None:
        d.pool = case.pool.to(device)
        d.k_pool = d.pool[:, 0]
        d.v_pool = d.pool[:, 1]
    else:
        d.k_pool = mv(case.k_pool)
        d.v_pool = mv(case.v_pool)
    for f in ("qkv", "page_table", "context_lens", "block_lens", "positions",
              "q_norm_weight", "k_norm_weight"):
        setattr(d, f, mv(getattr(case, f)))
    return d
