"""The split combine with more than 8 splits per request (GPU).

Such a request's partials are merged in chunks of 8 in split order, against a running
maximum that rescales the sums when a chunk raises it.  The cases put requests on both
sides of each chunk boundary (8, 9, 16, 17, 24, 33 splits), end on partial chunks, reach
the 64-split maximum, and make the maximum move from chunk to chunk (keys that grow or
shrink along the context, a near one-hot softmax); each against the fp64 oracle and rerun
bit-identical.
"""
import pytest
import torch

import drafter_synth as ds
from speculative_decoding_drafter_amd import plan
from tests.gpu_util import check, reference, run, say, to_np

pytestmark = pytest.mark.gpu

R, HQ, HKV, STRIDE = 4, 6, 1, 512


def _lens(splits, extras, ps):
    """Context lengths that need exactly `splits[i]` splits of `ps` pages (the last one
    holding 1 + extras[i] pages, its last page partial)."""
    out = []
    for n, e in zip(splits, extras):
        assert 0 <= e < ps
        pages = (n - 1) * ps + 1 + e
        out.append(pages * 64 - 13)
    return out


def _ramp(case, grow: bool):
    # scale every key page by a factor that rises (or falls) along each request's context
    ramp = torch.ones(case.k_pool.shape[0], 1, 1, 1)
    for r, L in enumerate(case.context_lens.tolist()):
        n = -(-L // 64)
        for j in range(n):
            f = j / max(1, n - 1)
            ramp[int(case.page_table[r, j])] = 1.0 + 15.0 * (f if grow else 1.0 - f)
    case.k_pool.copy_((case.k_pool.float() * ramp).to(torch.bfloat16))  # a view into the fused pool


def _plan():
    S, ps = plan(R, HKV, STRIDE)
    if S < 64:
        pytest.skip(f"plan ({S} splits of {ps} pages) leaves no room for 64 splits per request")
    return S, ps


CASES = {
    # splits per request, extra pages in the last split, scale, key ramp, qknorm
    "boundaries": ([9, 16, 17, 63], [0, 7, 0, 3], None, None, False),
    "to_the_maximum": ([8, 24, 33, 64], [7, 2, 5, 7], None, None, True),
    "rising_keys": ([9, 17, 40, 64], [3, 0, 6, 7], 0.5, True, False),
    "falling_keys": ([12, 23, 41, 57], [1, 4, 0, 2], 0.5, False, False),
    "near_one_hot": ([10, 31, 48, 64], [5, 7, 1, 7], 4.0, None, False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_many_split_combine(name):
    _, ps = _plan()
    splits, extras, scale, grow, qk = CASES[name]
    lens = _lens(splits, extras, ps)
    case = ds.make_case(R, 8, HQ, HKV, lens, seed=400 + len(name), stride=STRIDE, qknorm=qk, scale=scale,
                        pos_dtype=torch.int64 if qk else torch.int32)
    if grow is not None:
        _ramp(case, grow)
    say(f"many-split combine {name}: splits {splits}, lengths {lens}")
    from speculative_decoding_drafter_amd import make_workspace

    g = ds.to_device(case, "cuda")
    ws = make_workspace(R, 8, HQ, HKV, STRIDE, "cuda")
    a = run(case, g, workspace=ws)
    b = run(case, g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b), f"{name}: rerun not bit-identical"
    # every counter word of every (request, head) line is back at zero
    assert int(ws[:R * HKV * 256].view(torch.int32).count_nonzero()) == 0
    check(to_np(a), reference(case), name)


def test_many_split_graph_replays_with_rewritten_lengths():
    # one captured call of a 64-split plan, replayed with lengths that move the request
    # between one split, the chunked merge and the two-level merge; every replay equals an
    # eager call bit for bit (the group counters reset themselves between replays)
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace

    _, ps = _plan()
    lens_seq = [_lens([64], [7], ps)[0], 100, _lens([12], [3], ps)[0], _lens([17], [0], ps)[0],
                _lens([40], [5], ps)[0], 64 * 8]
    case = ds.make_case(R, 8, HQ, HKV, [lens_seq[0]] * R, seed=410, stride=STRIDE, qknorm=True)
    g = ds.to_device(case, "cuda")
    ws = make_workspace(R, 8, HQ, HKV, STRIDE, "cuda")
    out = torch.empty(R * 8, HQ * 64, dtype=torch.bfloat16, device="cuda")
    kw = dict(num_q_heads=HQ, num_kv_heads=HKV, tokens_per_block=8, scale=case.scale, workspace=ws)
    args = (g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight, g.k_norm_weight)
    drafter_attn_qknorm(*args, out=out, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        drafter_attn_qknorm(*args, out=out, **kw)
    torch.cuda.synchronize()
    for i, L in enumerate(lens_seq):
        lens = torch.tensor([L, L // 3, max(0, L - 4000), 7], dtype=torch.int32)
        g.context_lens.copy_(lens)
        g.positions.copy_((lens.view(-1, 1) + torch.arange(8)).view(-1).to(g.positions.dtype))
        say(f"replay {i}: lengths {lens.tolist()}")
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = drafter_attn_qknorm(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {i} differs from an eager call"
        assert int(ws[:R * HKV * 256].view(torch.int32).count_nonzero()) == 0
        if i in (0, 4):
            ref_case = ds.make_case(R, 8, HQ, HKV, lens.tolist(), seed=410, stride=STRIDE, qknorm=True)
            # the same pool, page table, qkv and weights as the captured case; only lengths/positions differ
            ref_case.qkv, ref_case.pool, ref_case.page_table = case.qkv, case.pool, case.page_table
            ref_case.k_pool, ref_case.v_pool = case.k_pool, case.v_pool
            ref_case.q_norm_weight, ref_case.k_norm_weight = case.q_norm_weight, case.k_norm_weight
            ref_case.positions = g.positions.cpu()
            check(to_np(got), reference(ref_case), f"replay-{i}")
