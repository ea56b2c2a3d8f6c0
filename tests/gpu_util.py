"""Shared helpers of the GPU tests (they call the HIP library through its binding)."""
import numpy as np
import torch

import drafter_synth as ds
import oracle

ATOL = 2e-2
RTOL = 2e-2
MEAN_TOL = 2e-3


def say(msg: str):
    print(msg, flush=True)


def run(case: ds.DrafterCase, dev_case: ds.DrafterCase = None, **kw) -> torch.Tensor:
    """One library call on a device copy of ``case``."""
    from speculative_decoding_drafter_amd import drafter_attn, drafter_attn_qknorm

    g = dev_case if dev_case is not None else ds.to_device(case, "cuda")
    common = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T,
                  block_lens=g.block_lens, scale=case.scale)
    if case.qknorm:
        common.update(eps=case.eps, rope_base=case.rope_base)
    common.update(kw)
    if case.qknorm:
        return drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                   g.q_norm_weight, g.k_norm_weight, **common)
    return drafter_attn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, **common)


def reference(case: ds.DrafterCase, pools=None) -> np.ndarray:
    a = case.np_args(pools)
    return oracle.drafter_attn_qknorm(**a) if case.qknorm else oracle.drafter_attn(**a)


def to_np(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, name: str = ""):
    """The acceptance bar: |err| <= 2e-2 + 2e-2|ref| everywhere, mean |err| <= 2e-3, no NaN."""
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    rel2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"{name}: max|err|={err.max():.3e} mean|err|={err.mean():.3e} rel_l2={rel2:.3e}")
    assert np.all(err <= bound), f"{name}: |err| {err[worst]:.3e} > bound at {worst}"
    assert err.mean() <= MEAN_TOL, f"{name}: mean|err| {err.mean():.3e}"
    return rel2
