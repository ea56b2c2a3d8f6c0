"""torch binding of the drafter block-attention C ABI (argument marshalling only).

Every step of the computation runs in the HIP library; torch provides device
memory and the current stream.  Shape, dtype and device problems raise
``DrafterAttnError`` (a ``ValueError``) before anything is launched, as do the
library's own host-side checks.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

HEAD_DIM = 64
PAGE = 64
GQA = 6
POS_DTYPES = {torch.int32: 0, torch.int64: 1}


class DrafterAttnError(ValueError):
    """An argument outside the operation's contract."""


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def workspace_bytes(num_requests: int, tokens_per_block: int, num_q_heads: int, num_kv_heads: int,
                    page_table_stride: int, head_dim: int = HEAD_DIM) -> int:
    n = _lib.load().drafter_attn_workspace_bytes(num_requests, tokens_per_block, num_q_heads,
                                                 num_kv_heads, head_dim, page_table_stride)
    if n == 0:
        raise DrafterAttnError("sizes outside the contract")
    return int(n)


def plan(num_requests: int, num_kv_heads: int, page_table_stride: int) -> Tuple[int, int]:
    """(num_splits, pages_per_split) the library uses for these sizes."""
    s, p = ctypes.c_int32(), ctypes.c_int32()
    rc = _lib.load().drafter_attn_plan(num_requests, num_kv_heads, page_table_stride,
                                       ctypes.byref(s), ctypes.byref(p))
    if rc != 0:
        raise DrafterAttnError(_lib.last_error())
    return s.value, p.value


def make_workspace(num_requests: int, tokens_per_block: int, num_q_heads: int, num_kv_heads: int,
                   page_table_stride: int, device) -> torch.Tensor:
    """A zeroed workspace (its counters must start at zero; every call leaves them zero)."""
    n = workspace_bytes(num_requests, tokens_per_block, num_q_heads, num_kv_heads, page_table_stride)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _yarn(yarn: Optional[dict]):
    """A YaRN parameter dict (``factor``, ``original_max_position``, optional ``alpha`` = 1,
    ``beta`` = 32, ``ramp`` = ``"turns"`` (or ``"index"``, ``"index_unrounded"``) and
    ``mscale`` = 0, the default temperature) as the header's host struct, or None."""
    if yarn is None:
        return None
    _check(isinstance(yarn, dict) and "factor" in yarn and "original_max_position" in yarn,
           "yarn must be a dict with factor and original_max_position (alpha, beta, ramp, mscale optional)")
    _check(set(yarn) <= {"factor", "original_max_position", "alpha", "beta", "ramp", "mscale"},
           "unknown yarn parameter")
    ramp = yarn.get("ramp", "turns")
    _check(ramp in _lib.YARN_RAMPS, f"yarn ramp must be one of {sorted(_lib.YARN_RAMPS)}")
    return ctypes.pointer(_lib.DaYarn(float(yarn["factor"]), int(yarn["original_max_position"]),
                                      float(yarn.get("alpha", 1.0)), float(yarn.get("beta", 32.0)),
                                      _lib.YARN_RAMPS[ramp], float(yarn.get("mscale", 0.0))))


def _check(cond: bool, msg: str):
    if not cond:
        raise DrafterAttnError(msg)


def _common(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads, num_kv_heads,
            tokens_per_block, out, workspace, *, takes_workspace: bool = True):
    dev = qkv.device
    _check(dev.type == "cuda", "qkv must be a GPU tensor (there is no CPU path)")
    R = int(context_lens.shape[0]) if context_lens.dim() == 1 else -1
    T = int(tokens_per_block)
    Hq, Hkv = int(num_q_heads), int(num_kv_heads)
    _check(context_lens.dim() == 1 and context_lens.dtype == torch.int32, "context_lens must be int32 [R]")
    _check(qkv.dtype == torch.bfloat16 and qkv.dim() == 2 and qkv.stride(1) == 1,
           "qkv must be bf16 [R*T, row_stride] with unit column stride")
    _check(qkv.shape[0] == R * T, f"qkv has {qkv.shape[0]} rows, expected R*T = {R * T}")
    _check(qkv.shape[1] >= (Hq + 2 * Hkv) * HEAD_DIM, "qkv is narrower than (Hq + 2*Hkv) * 64")
    _check(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.shape[0] == R,
           "page_table must be int32 [R, stride]")
    stride = int(page_table.shape[1])
    _check(stride == 0 or (page_table.stride(1) == 1 and page_table.stride(0) == stride),
           "page_table must be contiguous")
    for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
        _check(pool.dtype == torch.bfloat16 and pool.dim() == 4, f"{name} must be bf16 [P, Hkv, 64, 64]")
        _check(tuple(pool.shape[1:]) == (Hkv, PAGE, HEAD_DIM), f"{name} must be [P, {Hkv}, 64, 64]")
        _check(pool.stride()[1:] == (PAGE * HEAD_DIM, HEAD_DIM, 1), f"{name} pages must be contiguous HND")
        _check(pool.device == dev, f"{name} must be on {dev}")
    _check(k_pool.shape[0] == v_pool.shape[0] and k_pool.stride(0) == v_pool.stride(0),
           "k_pool and v_pool must have the same page count and page stride")
    for name, t in (("page_table", page_table), ("context_lens", context_lens), ("block_lens", block_lens),
                    ("out", out), ("workspace", workspace)):
        if t is not None:
            _check(t.device == dev, f"{name} must be on {dev}")
    if block_lens is not None:
        _check(block_lens.dtype == torch.int32 and tuple(block_lens.shape) == (R,), "block_lens must be int32 [R]")
        _check(block_lens.is_contiguous(), "block_lens must be contiguous")
    _check(context_lens.is_contiguous(), "context_lens must be contiguous")
    if out is None:
        out = torch.empty(R * T, Hq * HEAD_DIM, dtype=torch.bfloat16, device=dev)
    _check(out.dtype == torch.bfloat16 and out.dim() == 2 and out.stride(1) == 1 and
           out.shape[0] == R * T and out.shape[1] >= Hq * HEAD_DIM, "out must be bf16 [R*T, >= Hq*64]")
    if takes_workspace:
        if workspace is None:
            workspace = make_workspace(R, T, Hq, Hkv, stride, dev)
        _check(workspace.is_contiguous(), "workspace must be contiguous")
    return dict(R=R, T=T, Hq=Hq, Hkv=Hkv, stride=stride, out=out, workspace=workspace, dev=dev)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _raise(rc: int):
    if rc != 0:
        raise DrafterAttnError(f"drafter_attn error {rc}: {_lib.last_error()}")


def drafter_attn(qkv: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                 context_lens: torch.Tensor, *, num_q_heads: int, num_kv_heads: int, tokens_per_block: int,
                 block_lens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """k3_drafter_attn (q/k already normalised and rotated).  Returns ``out`` [R*T, Hq*64] bf16."""
    lib = _lib.load()
    a = _common(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads, num_kv_heads,
                tokens_per_block, out, workspace)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    if status is not None:
        _check(status.dtype == torch.int32 and status.numel() >= 1 and status.device == a["dev"],
               "status must be an int32 GPU tensor")
    rc = lib.drafter_attn(
        qkv.data_ptr(), qkv.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0), k_pool.shape[0],
        _ptr(page_table) if a["stride"] else None, a["stride"], context_lens.data_ptr(), _ptr(block_lens),
        a["R"], a["T"], a["Hq"], a["Hkv"], HEAD_DIM, PAGE, scale,
        a["workspace"].data_ptr(), a["workspace"].numel(), a["out"].data_ptr(), a["out"].stride(0),
        _ptr(status), _stream(a["dev"]))
    _raise(rc)
    return a["out"]


def drafter_attn_qknorm(qkv: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                        context_lens: torch.Tensor, positions: torch.Tensor, q_norm_weight: torch.Tensor,
                        k_norm_weight: torch.Tensor, *, num_q_heads: int, num_kv_heads: int,
                        tokens_per_block: int, block_lens: Optional[torch.Tensor] = None,
                        scale: Optional[float] = None, eps: float = 1e-5, rope_base: float = 10000.0,
                        yarn: Optional[dict] = None, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """k3_drafter_attn_qknorm (per-head q/k RMSNorm + NeoX RoPE in the kernel).  ``yarn``
    (``factor``, ``original_max_position``, optional ``alpha``, ``beta``) selects YaRN-scaled
    rotation (drafter_attn_qknorm_yarn)."""
    lib = _lib.load()
    y = _yarn(yarn)
    a = _common(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads, num_kv_heads,
                tokens_per_block, out, workspace)
    _check(positions.dtype in POS_DTYPES and positions.dim() == 1 and positions.numel() == a["R"] * a["T"]
           and positions.is_contiguous() and positions.device == a["dev"], "positions must be int32/int64 [R*T]")
    for name, wt in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _check(wt.dtype == torch.bfloat16 and tuple(wt.shape) == (HEAD_DIM,) and wt.is_contiguous()
               and wt.device == a["dev"], f"{name} must be bf16 [64]")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    if status is not None:
        _check(status.dtype == torch.int32 and status.numel() >= 1 and status.device == a["dev"],
               "status must be an int32 GPU tensor")
    head = (qkv.data_ptr(), qkv.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0), k_pool.shape[0],
            _ptr(page_table) if a["stride"] else None, a["stride"], context_lens.data_ptr(), _ptr(block_lens),
            a["R"], a["T"], a["Hq"], a["Hkv"], HEAD_DIM, PAGE, scale,
            positions.data_ptr(), POS_DTYPES[positions.dtype], q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
            float(eps), float(rope_base))
    tail = (a["workspace"].data_ptr(), a["workspace"].numel(), a["out"].data_ptr(), a["out"].stride(0),
            _ptr(status), _stream(a["dev"]))
    if y is None:
        rc = lib.drafter_attn_qknorm(*head, *tail)
    else:
        rc = lib.drafter_attn_qknorm_yarn(*head, y, *tail)
    _raise(rc)
    return a["out"]


def drafter_attn_qknorm_noalloc(qkv: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                page_table: torch.Tensor, context_lens: torch.Tensor, positions: torch.Tensor,
                                q_norm_weight: torch.Tensor, k_norm_weight: torch.Tensor, out: torch.Tensor, *,
                                num_q_heads: int, num_kv_heads: int, tokens_per_block: int,
                                block_lens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                                eps: float = 1e-5, rope_base: float = 10000.0,
                                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """drafter_attn_qknorm for callers that cannot allocate: no workspace argument (the library's
    own per-GPU scratch holds the split partials), and ``out`` must be given.  Calls whose kernels
    overlap on one GPU race.  Returns ``out``."""
    lib = _lib.load()
    _check(out is not None, "out must be given (this entry point allocates nothing)")
    a = _common(qkv, k_pool, v_pool, page_table, context_lens, block_lens, num_q_heads, num_kv_heads,
                tokens_per_block, out, None, takes_workspace=False)
    _check(positions.dtype in POS_DTYPES and positions.dim() == 1 and positions.numel() == a["R"] * a["T"]
           and positions.is_contiguous() and positions.device == a["dev"], "positions must be int32/int64 [R*T]")
    for name, wt in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _check(wt.dtype == torch.bfloat16 and tuple(wt.shape) == (HEAD_DIM,) and wt.is_contiguous()
               and wt.device == a["dev"], f"{name} must be bf16 [64]")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    if status is not None:
        _check(status.dtype == torch.int32 and status.numel() >= 1 and status.device == a["dev"],
               "status must be an int32 GPU tensor")
    rc = lib.drafter_attn_qknorm_noalloc(
        qkv.data_ptr(), qkv.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0), k_pool.shape[0],
        _ptr(page_table) if a["stride"] else None, a["stride"], context_lens.data_ptr(), _ptr(block_lens),
        a["R"], a["T"], a["Hq"], a["Hkv"], HEAD_DIM, PAGE, scale,
        positions.data_ptr(), POS_DTYPES[positions.dtype], q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
        float(eps), float(rope_base), out.data_ptr(), out.stride(0), _ptr(status), _stream(a["dev"]))
    _raise(rc)
    return out


def qk_norm_rope(qkv: torch.Tensor, positions: torch.Tensor, q_norm_weight: torch.Tensor,
                 k_norm_weight: torch.Tensor, *, num_q_heads: int, num_kv_heads: int, eps: float = 1e-5,
                 rope_base: float = 10000.0, yarn: Optional[dict] = None) -> torch.Tensor:
    """fused_qk_norm_rope (the drafter's cell), in place on ``qkv`` [N, >= (Hq+2Hkv)*64] bf16.

    Every q and k head of each row is RMS-normalised and NeoX-rotated at the row's
    position; v heads and padding are left as they are.  Returns ``qkv``.  ``yarn``
    as for ``drafter_attn_qknorm``.
    """
    lib = _lib.load()
    y = _yarn(yarn)
    _check(qkv.device.type == "cuda", "qkv must be a GPU tensor (there is no CPU path)")
    _check(qkv.dtype == torch.bfloat16 and qkv.dim() == 2 and qkv.stride(1) == 1,
           "qkv must be bf16 [N, row_stride] with unit column stride")
    N = int(qkv.shape[0])
    Hq, Hkv = int(num_q_heads), int(num_kv_heads)
    _check(qkv.shape[1] >= (Hq + 2 * Hkv) * HEAD_DIM, "qkv is narrower than (Hq + 2*Hkv) * 64")
    _check(positions.dtype in POS_DTYPES and positions.dim() == 1 and positions.numel() == N
           and positions.is_contiguous() and positions.device == qkv.device, "positions must be int32/int64 [N]")
    for name, wt in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _check(wt.dtype == torch.bfloat16 and tuple(wt.shape) == (HEAD_DIM,) and wt.is_contiguous()
               and wt.device == qkv.device, f"{name} must be bf16 [64]")
    args = (qkv.data_ptr(), qkv.stride(0), N, Hq, Hkv, HEAD_DIM, positions.data_ptr(), POS_DTYPES[positions.dtype],
            q_norm_weight.data_ptr(), k_norm_weight.data_ptr(), float(eps), float(rope_base))
    if y is None:
        rc = lib.drafter_qk_norm_rope(*args, _stream(qkv.device))
    else:
        rc = lib.drafter_qk_norm_rope_yarn(*args, y, _stream(qkv.device))
    _raise(rc)
    return qkv


def kv_append(qkv: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
              context_lens: torch.Tensor, *, num_q_heads: int, num_kv_heads: int, tokens_per_block: int,
              block_lens: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> None:
    """append_paged_kv_cache of the replaced path: the block's K/V rows go to slots L..L+b-1 of
    each request's paged row (in place on the pools)."""
    lib = _lib.load()
    dev = qkv.device
    _check(dev.type == "cuda", "qkv must be a GPU tensor (there is no CPU path)")
    R, T = int(context_lens.shape[0]), int(tokens_per_block)
    _check(page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.shape[0] == R
           and page_table.is_contiguous(), "page_table must be contiguous int32 [R, stride]")
    _check(context_lens.dtype == torch.int32 and context_lens.is_contiguous(), "context_lens must be int32 [R]")
    _check(qkv.dtype == torch.bfloat16 and qkv.dim() == 2 and qkv.stride(1) == 1 and qkv.shape[0] == R * T,
           "qkv must be bf16 [R*T, row_stride]")
    for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
        _check(pool.dtype == torch.bfloat16 and pool.dim() == 4 and tuple(pool.shape[1:]) == (num_kv_heads, PAGE, HEAD_DIM)
               and pool.stride()[1:] == (PAGE * HEAD_DIM, HEAD_DIM, 1) and pool.device == dev,
               f"{name} must be bf16 [P, Hkv, 64, 64] with contiguous pages on {dev}")
    if block_lens is not None:
        _check(block_lens.dtype == torch.int32 and tuple(block_lens.shape) == (R,) and block_lens.is_contiguous(),
               "block_lens must be int32 [R]")
    rc = lib.drafter_kv_append(qkv.data_ptr(), qkv.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0),
                               k_pool.shape[0], page_table.data_ptr(), page_table.shape[1], context_lens.data_ptr(),
                               _ptr(block_lens), R, T, int(num_q_heads), int(num_kv_heads), HEAD_DIM, PAGE,
                               _ptr(status), _stream(dev))
    _raise(rc)


def paged_attn(qkv: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
               kv_lens: torch.Tensor, *, num_q_heads: int, num_kv_heads: int, tokens_per_block: int,
               block_lens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The replaced path's non-causal context attention: the block's queries over the first
    kv_lens[r] pooled tokens only.  Returns ``out`` [R*T, Hq*64] bf16."""
    lib = _lib.load()
    a = _common(qkv, k_pool, v_pool, page_table, kv_lens, block_lens, num_q_heads, num_kv_heads,
                tokens_per_block, out, workspace)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    rc = lib.drafter_paged_attn(
        qkv.data_ptr(), qkv.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0), k_pool.shape[0],
        _ptr(page_table) if a["stride"] else None, a["stride"], kv_lens.data_ptr(), _ptr(block_lens),
        a["R"], a["T"], a["Hq"], a["Hkv"], HEAD_DIM, PAGE, scale,
        a["workspace"].data_ptr(), a["workspace"].numel(), a["out"].data_ptr(), a["out"].stride(0),
        _ptr(status), _stream(a["dev"]))
    _raise(rc)
    return a["out"]
