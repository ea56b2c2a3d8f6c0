"""fp64 CPU oracle for the DFlash drafter's block attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.

What is computed (TensorRT-LLM PR #20532 "Share Kimi K3 FP4 modeling and add
NVFP4 support on SM103", Conversation, the commit that adds k3_drafter_attn
and k3_drafter_attn_qknorm, and the next commit that adds their contracts):

* batch: R <= 8 requests, T <= 8 block tokens per request.
* keys of request r: its context tokens (HND pages of 64 through its
  page-table row), then its block tokens' k/v columns of the packed qkv rows;
  no mask; the pool is only read.
* heads: GQA, 6 query heads per KV head, head_dim 64.
* k3_drafter_attn takes q/k already normalised and rotated;
  k3_drafter_attn_qknorm applies the per-head q/k RMSNorm (eps 1e-5) and the
  NeoX rotary embedding (base 10000) itself.

The method is an exact reformulation of softmax attention, so this oracle is
that definition written out in float64 on the exact bf16 input values, with
nothing rounded.  Readings of points the pages leave open (the same ones the
library's header documents):

* qkv row ``r*T + t`` holds ``[q heads | k heads | v heads]``, 64 columns each.
* Query head ``h`` uses KV head ``h // 6`` (contiguous GQA groups).
* Page ``p`` of a pool holds ``[Hkv][64 slots][64 dims]``; context token ``c``
  of request ``r`` is slot ``c % 64`` of page ``page_table[r, c // 64]``.
  Only the first ``ceil(L/64)`` entries of a page-table row are meaningful;
  slots past ``L`` in the last page are not part of the input.
* A request may bring fewer than T tokens (``block_lens``); its rows past that
  length are neither keys nor outputs and their outputs are zero.
* RMSNorm is ``x * w / sqrt(mean(x^2) + eps)`` over one head's 64 values with
  one weight vector for all q heads and one for all k heads.
* NeoX rotation pairs dimension ``i`` with ``i + 32`` at angle
  ``pos * base**(-2i/64)``; only the block's q and k are rotated, never v and
  never the context (the pool holds keys that are already processed).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

HEAD_DIM = 64
PAGE = 64
GQA = 6


class OracleContractError(ValueError):
    """An input outside the operation's contract (the library clamps and flags these)."""


# --------------------------------------------------------------------------------------
# q/k preprocessing (the qknorm variant)
# --------------------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the last axis (64 values of one head).

    PR #20532, commit adding fused_qk_norm_rope's drafter cell: eps 1e-5,
    head_dim 64; the attention commit names a per-head q/k RMSNorm.
    ``x * w / sqrt(mean(x**2) + eps)``.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(w, dtype=np.float64) / np.sqrt(ms + eps)


def rope_inv_freq(base: float, dim: int = HEAD_DIM) -> np.ndarray:
    """Rotary frequencies ``base**(-2i/dim)`` for ``i < dim/2`` (base 10000 in the cell)."""
    i = np.arange(dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / dim)


YARN_RAMPS = ("turns", "index", "index_unrounded")


def yarn_pair_at_turns(base: float, original_max_position: float, turns: float, dim: int = HEAD_DIM) -> float:
    """The (fractional) rotary pair index at which a pair turns exactly ``turns`` times over
    the original context ``L``: solving ``L * base**(-2i/dim) / (2 pi) = turns`` for ``i``
    gives ``i = (dim/2) * ln(L / (2 pi turns)) / ln(base)`` (``+inf`` for ``turns = 0``).
    Pairs below it turn more often, pairs above it less."""
    if turns <= 0.0:
        return math.inf
    return (dim / 2.0) * math.log(float(original_max_position) / (2.0 * math.pi * turns)) / math.log(float(base))


def yarn_inv_freq(base: float, factor: float, original_max_position: int, alpha: float = 1.0,
                  beta: float = 32.0, dim: int = HEAD_DIM, ramp: str = "turns") -> np.ndarray:
    """YaRN's frequencies ("NTK-by-parts"), for the drafter checkpoint's "YaRN 4.0".

    The drafter line of "K3 DFlash Sequence-Compaction GB300 Validation" (Scope and
    results) names YaRN with factor 4.0 and no other parameter; the method is the
    published one (Peng, Quesnelle, Fan, Shippole, "YaRN: Efficient Context Window
    Extension of Large Language Models", 2023, Section 3): for rotary pair ``i`` with
    base frequency ``theta``, the number of turns it makes over the original context
    is ``r = L * theta / (2 pi)``; the weight ``gamma`` of the unscaled frequency is 1
    for pairs that turn at least ``beta`` times, 0 for pairs that turn at most
    ``alpha`` times, and ramps between them; the new frequency is
    ``(1 - gamma) * theta / s + gamma * theta``: pairs that turn many times keep their
    frequency, pairs that turn less than ``alpha`` times are interpolated by ``s``.

    ``ramp`` says what the ramp is linear in:

    * ``"turns"`` (the paper's ``gamma(r)``): ``gamma = clamp((r - alpha) / (beta - alpha))``.
    * ``"index"``: linear in the pair index between ``lo = floor(i(beta))`` and
      ``hi = ceil(i(alpha))``, where ``i(rho)`` is the fractional index at which a pair
      turns ``rho`` times (``yarn_pair_at_turns``), both clamped to ``[0, dim/2 - 1]``:
      ``gamma = 1 - clamp((i - lo) / (hi - lo))``.  The same end points as ``"turns"``
      (up to the rounding of the bounds to whole pairs), a different shape in between:
      the parametrisation checkpoint configurations commonly use.
    * ``"index_unrounded"``: the same with ``lo = i(beta)``, ``hi = i(alpha)`` not rounded.

    Where the clamped bounds meet or cross (``hi <= lo``: an original context so short
    or so long that the ramp leaves the pair range), pairs up to ``lo`` keep their
    frequency and the others are interpolated.
    """
    if ramp not in YARN_RAMPS:
        raise OracleContractError(f"unknown YaRN ramp {ramp!r}")
    if ramp != "turns" and not float(base) > 1.0:
        raise OracleContractError("YaRN ramps in the pair index need base > 1")
    theta = rope_inv_freq(base, dim)
    if ramp == "turns":
        turns = float(original_max_position) * theta / (2.0 * math.pi)
        gamma = np.clip((turns - alpha) / (beta - alpha), 0.0, 1.0)
    else:
        top = dim // 2 - 1
        lo = min(max(yarn_pair_at_turns(base, original_max_position, beta, dim), 0.0), float(top))
        hi = min(max(yarn_pair_at_turns(base, original_max_position, alpha, dim), 0.0), float(top))
        if ramp == "index":
            lo, hi = float(math.floor(lo)), float(math.ceil(hi))
        i = np.arange(dim // 2, dtype=np.float64)
        if hi > lo:
            gamma = 1.0 - np.clip((i - lo) / (hi - lo), 0.0, 1.0)
        else:
            gamma = (i <= lo).astype(np.float64)
    return (1.0 - gamma) * theta / float(factor) + gamma * theta


def yarn_mscale(factor: float) -> float:
    """YaRN's attention temperature as a factor on q and on k: ``sqrt(1/t) = 0.1 ln(s) + 1``
    (the same paper, Section 3.4), so the logits are divided by ``t``."""
    return 0.1 * math.log(float(factor)) + 1.0


def rope_neox(x: np.ndarray, pos, base: float, yarn: Optional[dict] = None) -> np.ndarray:
    """NeoX ("rotate half") rotary embedding over the last axis.

    PR #20532, fused_qk_norm_rope drafter cell: NeoX style, base 10000.
    Dimension ``i`` pairs with ``i + dim/2``; the pair is turned by the angle
    ``pos * inv_freq[i]``.  ``pos`` broadcasts against ``x[..., 0]``.  With
    ``yarn`` (``factor``, ``original_max_position``, optional ``alpha`` = 1,
    ``beta`` = 32, ``ramp`` = ``"turns"`` and ``mscale``) the frequencies are
    YaRN's and the rotated vector is scaled by ``mscale`` when it is given and
    positive (a checkpoint that folds the temperature into the softmax scale
    instead gives 1), else by ``yarn_mscale(factor)``.
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    if yarn is None:
        inv_freq, m = rope_inv_freq(base, x.shape[-1]), 1.0
    else:
        inv_freq = yarn_inv_freq(base, yarn["factor"], yarn["original_max_position"], yarn.get("alpha", 1.0),
                                 yarn.get("beta", 32.0), x.shape[-1], yarn.get("ramp", "turns"))
        m = float(yarn["mscale"]) if yarn.get("mscale", 0.0) > 0.0 else yarn_mscale(yarn["factor"])
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return m * np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------------------
# paged context
# --------------------------------------------------------------------------------------

def gather_context(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray,
                   L: int, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """Context K and V of one request and KV head, in logical token order.

    Walks the page-table row page by page: logical page ``j`` is physical page
    ``table_row[j]``, holding tokens ``64*j .. 64*j+63`` (HND: head, slot, dim).
    Only the first ``L - 64*j`` slots of the last page are taken.
    """
    P = k_pool.shape[0]
    npg = -(-L // PAGE)
    ks, vs = [], []
    for j in range(npg):
        phys = int(table_row[j])
        if not 0 <= phys < P:
            raise OracleContractError(f"page id {phys} out of range [0, {P})")
        n = min(PAGE, L - PAGE * j)
        ks.append(k_pool[phys, g, :n, :])
        vs.append(v_pool[phys, g, :n, :])
    if not ks:
        z = np.zeros((0, k_pool.shape[-1]))
        return z, z.copy()
    return np.concatenate(ks, axis=0).astype(np.float64), np.concatenate(vs, axis=0).astype(np.float64)


# --------------------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------------------

def kv_head_of(h: int) -> int:
    """GQA: query head ``h`` reads KV head ``h // 6`` (6 query heads per KV head)."""
    return h // GQA


def q_cols(h: int, Hq: int, Hkv: int) -> slice:
    """qkv columns of query head ``h``."""
    return slice(h * HEAD_DIM, (h + 1) * HEAD_DIM)


def k_cols(g: int, Hq: int, Hkv: int) -> slice:
    """qkv columns of the block's key head ``g`` (after the Hq query heads)."""
    return slice((Hq + g) * HEAD_DIM, (Hq + g + 1) * HEAD_DIM)


def v_cols(g: int, Hq: int, Hkv: int) -> slice:
    """qkv columns of the block's value head ``g`` (after the q and k heads)."""
    return slice((Hq + Hkv + g) * HEAD_DIM, (Hq + Hkv + g + 1) * HEAD_DIM)


def _softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Dense softmax attention of query rows over all keys (no mask).

    Stable form: subtract each row's maximum score before exponentiating.
    Returns the outputs and the softmax weights.
    """
    s = scale * (q @ keys.T)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return p @ vals, p


def _check_shapes(qkv, k_pool, v_pool, page_table, context_lens, block_lens,
                  Hq: int, Hkv: int, T: int):
    if Hkv < 1 or Hq != GQA * Hkv:
        raise OracleContractError(f"need Hq == 6*Hkv, got {Hq}/{Hkv}")
    R = len(context_lens)
    if not (1 <= R <= 8 and 1 <= T <= 8):
        raise OracleContractError(f"R={R}, T={T} outside 1..8")
    if qkv.shape[0] != R * T or qkv.shape[1] < (Hq + 2 * Hkv) * HEAD_DIM:
        raise OracleContractError("qkv shape")
    if k_pool.shape[1:] != (Hkv, PAGE, HEAD_DIM) or v_pool.shape != k_pool.shape:
        raise OracleContractError("pool shape")
    stride = page_table.shape[1] if page_table is not None and page_table.ndim == 2 else 0
    for r in range(R):
        L = int(context_lens[r])
        if not 0 <= L <= stride * PAGE:
            raise OracleContractError(f"context length {L} outside [0, {stride * PAGE}]")
    if block_lens is not None:
        for r in range(R):
            if not 1 <= int(block_lens[r]) <= T:
                raise OracleContractError("block length outside [1, T]")
    return R


def _run(qkv, k_pool, v_pool, page_table, context_lens, block_lens, Hq, Hkv, T, scale,
         prep_q, prep_k, return_probs: bool):
    R = _check_shapes(qkv, k_pool, v_pool, page_table, context_lens, block_lens, Hq, Hkv, T)
    D = HEAD_DIM
    qkv = np.asarray(qkv, dtype=np.float64)
    out = np.zeros((R * T, Hq * D), dtype=np.float64)
    probs: Dict[Tuple[int, int, int], np.ndarray] = {}
    for r in range(R):
        L = int(context_lens[r])
        b = T if block_lens is None else int(block_lens[r])
        rows = slice(r * T, r * T + b)
        kv = {}
        for g in range(Hkv):
            kc, vc = gather_context(k_pool, v_pool, page_table[r] if L else None, L, g)
            kb = prep_k(qkv[rows, k_cols(g, Hq, Hkv)], r, b)
            vb = qkv[rows, v_cols(g, Hq, Hkv)]
            kv[g] = (np.concatenate([kc, kb], axis=0), np.concatenate([vc, vb], axis=0))
        for h in range(Hq):
            keys, vals = kv[kv_head_of(h)]
            q = prep_q(qkv[rows, q_cols(h, Hq, Hkv)], r, b)
            o, p = _softmax_attend(q, keys, vals, scale)
            out[rows, h * D:(h + 1) * D] = o
            if return_probs:
                for t in range(b):
                    probs[(r, h, t)] = p[t]
    return (out, probs) if return_probs else out


def drafter_attn(qkv, k_pool, v_pool, page_table, context_lens, block_lens=None, *,
                 num_q_heads: int, num_kv_heads: int, tokens_per_block: int,
                 scale: Optional[float] = None, return_probs: bool = False, **_unused):
    """k3_drafter_attn: block attention over paged context + own block, q/k used as given.

    Returns ``out`` float64 ``[R*T, Hq*64]`` (and the softmax weights per
    (request, head, token) when ``return_probs``).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    ident = lambda x, r, b: np.asarray(x, dtype=np.float64)
    return _run(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads,
                num_kv_heads, tokens_per_block, scale, ident, ident, return_probs)


def drafter_attn_qknorm(qkv, k_pool, v_pool, page_table, context_lens, block_lens=None, *,
                        positions, q_norm_weight, k_norm_weight, num_q_heads: int,
                        num_kv_heads: int, tokens_per_block: int, scale: Optional[float] = None,
                        eps: float = 1e-5, rope_base: float = 10000.0, yarn: Optional[dict] = None,
                        return_probs: bool = False, **_unused):
    """k3_drafter_attn_qknorm: RMSNorm then NeoX RoPE on the block's q and k, then attention.

    The block's v and the whole paged context are used as stored.  Positions
    are read per token (``positions[r*T + t]``).  ``yarn``: see ``rope_neox``.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    T = tokens_per_block
    pos = np.asarray(positions, dtype=np.int64)

    def prep(w):
        def f(x, r, b):
            return rope_neox(rms_norm(x, w, eps), pos[r * T:r * T + b], rope_base, yarn)
        return f

    return _run(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads,
                num_kv_heads, T, scale, prep(q_norm_weight), prep(k_norm_weight), return_probs)


def qk_norm_rope(qkv, positions, q_norm_weight, k_norm_weight, *, num_q_heads: int,
                 num_kv_heads: int, eps: float = 1e-5, rope_base: float = 10000.0,
                 yarn: Optional[dict] = None) -> np.ndarray:
    """fused_qk_norm_rope, the drafter's cell, on packed qkv rows.

    PR #20532, commit adding fused_qk_norm_rope's drafter cell (head_dim 64,
    6 query heads per KV head, 1 to 64 tokens, eps 1e-5, base 10000, NeoX); the
    attention commit says the qknorm variant uses that op's arithmetic.  Every
    query head of a row is RMS-normalised with ``q_norm_weight`` and every key
    head with ``k_norm_weight``, then NeoX-rotated at the row's position.  The
    value heads and any columns past the heads are returned unchanged.  The
    result is a float64 copy; the op itself works in place on bf16 rows.
    """
    x = np.array(qkv, dtype=np.float64, copy=True)
    pos = np.asarray(positions, dtype=np.int64)
    Hq, Hkv = int(num_q_heads), int(num_kv_heads)
    if x.ndim != 2 or pos.shape != (x.shape[0],):
        raise OracleContractError("qkv must be [N, width] with one position per row")
    if x.shape[1] < (Hq + 2 * Hkv) * HEAD_DIM or Hkv < 1 or Hq != GQA * Hkv:
        raise OracleContractError("qkv narrower than its heads, or not 6 query heads per KV head")
    for h in range(Hq):
        c = q_cols(h, Hq, Hkv)
        x[:, c] = rope_neox(rms_norm(x[:, c], q_norm_weight, eps), pos, rope_base, yarn)
    for g in range(Hkv):
        c = k_cols(g, Hq, Hkv)
        x[:, c] = rope_neox(rms_norm(x[:, c], k_norm_weight, eps), pos, rope_base, yarn)
    return x


# --------------------------------------------------------------------------------------
# the path the fused kernel replaces (built as an A/B baseline): append, then attend
# --------------------------------------------------------------------------------------

def kv_append(k_pool, v_pool, qkv, page_table, context_lens, block_lens=None, *, num_q_heads: int,
              num_kv_heads: int, tokens_per_block: int):
    """append_paged_kv_cache as the replaced DFlash path uses it.

    PR #20532, Conversation, the attention commit: the fused kernel reads the
    block's K/V from qkv instead of appending them to the cache first and then
    running a non-causal context kernel.  Token ``t < b_r`` of request ``r`` is
    logical token ``L_r + t`` of the request, i.e. slot ``(L_r + t) % 64`` of
    page ``page_table[r, (L_r + t) // 64]``; for every KV head ``g`` its K comes
    from the block's k columns and its V from the v columns.  Returns new
    ``(k_pool, v_pool)`` float64 copies; no other slot changes.
    """
    Hq, Hkv, T = int(num_q_heads), int(num_kv_heads), int(tokens_per_block)
    k = np.array(k_pool, dtype=np.float64, copy=True)
    v = np.array(v_pool, dtype=np.float64, copy=True)
    qkv = np.asarray(qkv, dtype=np.float64)
    R = len(context_lens)
    stride = page_table.shape[1]
    for r in range(R):
        L = int(context_lens[r])
        b = T if block_lens is None else int(block_lens[r])
        if L < 0 or L + b > stride * PAGE:
            raise OracleContractError(f"request {r}: {L} + {b} tokens do not fit {stride} pages")
        for t in range(b):
            phys = int(page_table[r, (L + t) // PAGE])
            if not 0 <= phys < k.shape[0]:
                raise OracleContractError(f"page id {phys} out of range")
            slot = (L + t) % PAGE
            for g in range(Hkv):
                k[phys, g, slot] = qkv[r * T + t, k_cols(g, Hq, Hkv)]
                v[phys, g, slot] = qkv[r * T + t, v_cols(g, Hq, Hkv)]
    return k, v


def paged_attn(qkv, k_pool, v_pool, page_table, kv_lens, block_lens=None, *, num_q_heads: int,
               num_kv_heads: int, tokens_per_block: int, scale: Optional[float] = None) -> np.ndarray:
    """The replaced path's non-causal context attention: the block's query rows of
    request ``r`` attend to the first ``kv_lens[r]`` tokens of its paged row (the
    context and, after ``kv_append``, the block itself); qkv supplies only the
    queries.  Rows past the block length, and every row of a request with no
    keys, are zero.
    """
    Hq, Hkv, T = int(num_q_heads), int(num_kv_heads), int(tokens_per_block)
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    qkv = np.asarray(qkv, dtype=np.float64)
    R = len(kv_lens)
    out = np.zeros((R * T, Hq * HEAD_DIM), dtype=np.float64)
    for r in range(R):
        n = int(kv_lens[r])
        b = T if block_lens is None else int(block_lens[r])
        if n == 0:
            continue
        rows = slice(r * T, r * T + b)
        kv = {g: gather_context(k_pool, v_pool, page_table[r], n, g) for g in range(Hkv)}
        for h in range(Hq):
            keys, vals = kv[kv_head_of(h)]
            o, _ = _softmax_attend(qkv[rows, q_cols(h, Hq, Hkv)], keys, vals, scale)
            out[rows, h * HEAD_DIM:(h + 1) * HEAD_DIM] = o
    return out


def drafter_attn_split_merge(qkv, k_pool, v_pool, page_table, context_lens, block_lens=None, *,
                             num_splits: int, num_q_heads: int, num_kv_heads: int,
                             tokens_per_block: int, scale: Optional[float] = None,
                             positions=None, q_norm_weight=None, k_norm_weight=None,
                             eps: float = 1e-5, rope_base: float = 10000.0,
                             qknorm: bool = False, group: Optional[int] = None, **_unused):
    """The same attention computed split-KV (flash-decoding) style.

    The context pages of a request are cut into ``num_splits`` consecutive page
    ranges; the own block is one more range.  Each range yields its running
    maximum ``m``, weight sum ``l`` and unnormalised output ``O``; the ranges
    are merged by rescaling with ``exp(m_s - M)``, ``M = max_s m_s``.  This is
    the algebra of the split-combine pass, checked here against the plain
    definition independently of any GPU code.  With ``group`` the context
    ranges are first merged in consecutive groups of that many, each group
    giving one (m, l, O) of the same form, and the groups are merged after
    (a two-level combine: the merge is associative).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    Hq, Hkv, T, D = num_q_heads, num_kv_heads, tokens_per_block, HEAD_DIM
    R = _check_shapes(qkv, k_pool, v_pool, page_table, context_lens, block_lens, Hq, Hkv, T)
    qkv = np.asarray(qkv, dtype=np.float64)
    if qknorm:
        pos = np.asarray(positions, dtype=np.int64)
        pq = lambda x, r, b: rope_neox(rms_norm(x, q_norm_weight, eps), pos[r * T:r * T + b], rope_base)
        pk = lambda x, r, b: rope_neox(rms_norm(x, k_norm_weight, eps), pos[r * T:r * T + b], rope_base)
    else:
        pq = pk = lambda x, r, b: x
    stride = page_table.shape[1] if page_table is not None and page_table.ndim == 2 else 0
    per = max(1, -(-stride // num_splits))
    out = np.zeros((R * T, Hq * D))
    for r in range(R):
        L = int(context_lens[r])
        b = T if block_lens is None else int(block_lens[r])
        rows = slice(r * T, r * T + b)
        rng_of = {}
        for g in range(Hkv):
            kc, vc = gather_context(k_pool, v_pool, page_table[r] if L else None, L, g)
            kb = pk(qkv[rows, k_cols(g, Hq, Hkv)], r, b)
            vb = qkv[rows, v_cols(g, Hq, Hkv)]
            rng_of[g] = [(kc[s * per * PAGE:(s + 1) * per * PAGE], vc[s * per * PAGE:(s + 1) * per * PAGE])
                         for s in range(num_splits)] + [(kb, vb)]
        for h in range(Hq):
            ranges = rng_of[kv_head_of(h)]
            q = pq(qkv[rows, q_cols(h, Hq, Hkv)], r, b)
            parts = []
            for kk, vv in ranges:
                if kk.shape[0] == 0:
                    parts.append((np.full(b, -np.inf), np.zeros(b), np.zeros((b, D))))
                    continue
                s = scale * (q @ kk.T)
                m = s.max(axis=-1)
                e = np.exp(s - m[:, None])
                parts.append((m, e.sum(axis=-1), e @ vv))
            if group:
                ctx = parts[:num_splits]  # the context ranges; the own block stays a range of its own
                parts = [_merge_parts(ctx[i:i + group], b, D) for i in range(0, num_splits, group)] + parts[num_splits:]
            m_all, den, num = _merge_parts(parts, b, D)
            out[rows, h * D:(h + 1) * D] = num / den[:, None]
    return out


def _merge_parts(parts, b: int, D: int):
    """Merge (m, l, O) range results into one of the same form: ``M = max m``,
    ``l = sum l exp(m - M)``, ``O = sum O exp(m - M)`` (a range without keys has
    ``m = -inf`` and weight 0)."""
    M = np.max([p[0] for p in parts], axis=0)
    num = np.zeros((b, D))
    den = np.zeros(b)
    for m, l, o in parts:
        w = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(M), M, 0.0)), 0.0)
        num += w[:, None] * o
        den += w * l
    return M, den, num
