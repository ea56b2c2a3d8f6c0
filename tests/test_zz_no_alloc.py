"""The no-allocation entry point (drafter_attn_qknorm_noalloc) against drafter_attn_qknorm.

Both run the same kernels; the first keeps its split partials and counters in the
library's own per-GPU scratch instead of a caller's workspace.  Two calls in a row, the
second on a smaller problem (the scratch keeps the first call's partials, and the
counters must be back at zero), each equal bit for bit to drafter_attn_qknorm on the
same inputs and within the acceptance bar of the fp64 oracle; then the call captured in
a HIP graph, replayed after its inputs are rewritten.
"""
import numpy as np
import pytest
import torch

import drafter_synth as ds
from tests.gpu_util import check, reference, say, to_np

pytestmark = pytest.mark.gpu


def _both(case: ds.DrafterCase, g: ds.DrafterCase):
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, drafter_attn_qknorm_noalloc

    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, block_lens=g.block_lens,
              scale=case.scale)
    args = (g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight, g.k_norm_weight)
    out_na = torch.full((case.R * case.T, case.Hq * 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    drafter_attn_qknorm_noalloc(*args, out_na, **kw)
    out_ws = drafter_attn_qknorm(*args, **kw)
    torch.cuda.synchronize()
    return out_na, out_ws


def test_noalloc_matches_workspace_entry_point_twice():
    big = ds.make_config(5)            # 8 x 8, 24/4, 32k-token contexts: 256 partial slots
    small = ds.make_case(3, 4, 12, 2, [0, 700, 1300], seed=401, qknorm=True, pos_dtype=torch.int64,
                         block_lens=[4, 1, 3], name="small")
    pools = None
    for case in (big, small):
        say(f"noalloc: {case.name or 'cfg5'} R={case.R} T={case.T} Hq={case.Hq} Hkv={case.Hkv} "
            f"L={case.context_lens.tolist()}")
        g = ds.to_device(case, "cuda")
        out_na, out_ws = _both(case, g)
        assert torch.equal(out_na, out_ws), f"{case.name}: no-allocation output differs from the workspace call"
        check(to_np(out_na), reference(case, pools), f"noalloc-{case.name or 'cfg5'}")


def test_noalloc_one_long_request_two_level_combine():
    # one 32k-token request: a plan of 64 splits, merged in two levels (counter words 1..8
    # of the scratch's counter lines as well as word 0), twice in a row
    case = ds.make_case(1, 8, 24, 4, [32768 - 5], seed=402, qknorm=True, name="one-long")
    g = ds.to_device(case, "cuda")
    for k in range(2):
        say(f"noalloc: one long request, call {k}")
        out_na, out_ws = _both(case, g)
        assert torch.equal(out_na, out_ws), f"call {k}: no-allocation output differs from the workspace call"
    check(to_np(out_na), reference(case), "noalloc-one-long")


def test_noalloc_graph_replay_with_rewritten_inputs():
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, drafter_attn_qknorm_noalloc

    pool = ds.config4_pool(4)
    case = ds.config4_cell(8, 8, 4, 0, pool=pool)
    g = ds.to_device(case, "cuda")
    pool_dev = pool.cuda()
    g.pool, g.k_pool, g.v_pool = pool_dev, pool_dev[:, 0], pool_dev[:, 1]
    out = torch.empty(64, 24 * 64, dtype=torch.bfloat16, device="cuda")
    kw = dict(num_q_heads=24, num_kv_heads=4, tokens_per_block=8, scale=case.scale)
    args = lambda: (g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight,
                    g.k_norm_weight)
    say("noalloc: capture")
    drafter_attn_qknorm_noalloc(*args(), out, **kw)   # outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        drafter_attn_qknorm_noalloc(*args(), out, **kw)
    torch.cuda.synchronize()
    pools_np = (pool[:, 0].double().numpy(), pool[:, 1].double().numpy())
    for k in range(1, 4):
        new = ds.config4_cell(8, 8, 4, k, pool=pool)
        for name in ("qkv", "page_table", "context_lens", "positions", "q_norm_weight", "k_norm_weight"):
            getattr(g, name).copy_(getattr(new, name))
        say(f"noalloc: replay {k} L={new.context_lens.tolist()}")
        graph.replay()
        eager = drafter_attn_qknorm(*args(), **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k}: differs from drafter_attn_qknorm"
        check(to_np(out), reference(new, pools_np), f"noalloc-replay-{k}")
    assert np.isfinite(to_np(out)).all()
