"""The length-aware split schedule on the GPU.

When the host plan leaves room (more than one split, at least 32 pages per split), the
kernel decides on the device, from the context lengths, between the static plan (split x
of request z has pages [x*Ps, (x+1)*Ps)) and the balanced plan (the requests' N pages cut
into splits of Pb pages; request i takes max(1, ceil(npg_i / Pb)) consecutive entries).
These tests check, against the fp64 oracle, workloads on which the balanced plan is taken
(mixed long contexts, one long request among short ones, short contexts under a padded
page-table stride), observe which partial slots the kernel writes (the schedule the header
documents), and check reruns, poison, graph replays that switch plans between replays,
the counters left at zero, and what request isolation keeps under the balanced plan.
"""
import math

import numpy as np
import pytest
import torch

import drafter_synth as ds
from tests.gpu_util import check, reference, run, say, to_np

pytestmark = pytest.mark.gpu

ROW = 48 * 64 * 4  # bytes of one partial's fp32 output block


def _plan(R, hkv, stride):
    from speculative_decoding_drafter_amd import plan

    return plan(R, hkv, stride)


def _expected_schedule(case):
    """The documented schedule for these lengths: (balanced, ps, {(r, g): (slot0, splits)})."""
    S, Ps = _plan(case.R, case.Hkv, case.stride)
    maxL = case.stride * 64
    npg = [math.ceil(min(max(int(L), 0), maxL) / 64) for L in case.context_lens.tolist()]
    N, nmax = sum(npg), max(npg)
    balanced, ps = False, Ps
    if S > 1 and Ps >= 32 and N > 0:
        X = case.R * (S - 1)
        pb = max(math.ceil(N / X), math.ceil(nmax / 32))
        pb = max(8, math.ceil(pb / 8) * 8)
        if pb <= (3 * Ps // 4) // 8 * 8:
            balanced, ps = True, pb
    slots = {}
    base = 0
    for r in range(case.R):
        k = max(1, math.ceil(npg[r] / ps))
        for g in range(case.Hkv):
            slots[(r, g)] = (g * case.R * S + base if balanced else (r * case.Hkv + g) * S, k)
        base += k
    return balanced, ps, slots


def _mk(R, hq, hkv, lens, stride, seed, **kw):
    npg = sum(-(-L // 64) for L in lens)
    return ds.make_case(R, 8, hq, hkv, lens, seed=seed, stride=stride, pool_pages=npg + 7, qknorm=True, **kw)


CASES = {
    # 8 x 8 tokens, 24/4 heads, stride 256 (Ps 32): mixed lengths up to 16k tokens
    "mixed16k": lambda: _mk(8, 24, 4, [16384, 9000, 313, 0, 12000, 64, 4097, 777], 256, 501),
    # one 64k-token request among short ones: 32 splits of 32 pages for it
    "onelong": lambda: _mk(8, 24, 4, [65536, 100, 0, 2000, 0, 1, 0, 64], 1024, 502),
    # short contexts under a padded stride of 1024 pages: splits of 8 pages
    "padded": lambda: _mk(8, 24, 4, [1850, 1247, 719, 781, 198, 1225, 927, 1967], 1024, 503),
    # 6/1 heads, 3 requests, int64 positions, ragged blocks
    "ragged61": lambda: _mk(3, 6, 1, [40000, 1000, 33], 3000, 504, pos_dtype=torch.int64, block_lens=[8, 3, 1]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_balanced_plan_matches_oracle_and_writes_the_documented_slots(name):
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace

    case = CASES[name]()
    balanced, ps, slots = _expected_schedule(case)
    assert balanced, f"{name}: the case was meant to take the balanced plan"
    S, _ = _plan(case.R, case.Hkv, case.stride)
    g = ds.to_device(case, "cuda")
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
    # counters first (zero), then the fp32 partial outputs: poison those with NaN bytes
    part_o = (case.R * case.Hkv * 256 + 255) // 256 * 256
    ws[part_o:part_o + case.R * case.Hkv * S * ROW] = 0xFF
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"{name}: balanced plan, splits of {ps} pages, L={case.context_lens.tolist()}")
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, block_lens=g.block_lens,
              scale=case.scale, workspace=ws, status=status)
    args = (g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight, g.k_norm_weight)
    out = drafter_attn_qknorm(*args, **kw).clone()
    torch.cuda.synchronize()
    check(to_np(out), reference(case), name)
    assert int(status.item()) == 0
    # which partial slots were written: exactly those of the requests with more than one split
    written = torch.isfinite(ws[part_o:part_o + case.R * case.Hkv * S * ROW].view(torch.float32)
                             .view(-1, 48 * 64)[:, 0]).cpu().numpy()
    want = np.zeros_like(written)
    for (r, gg), (slot0, k) in slots.items():
        if k > 1:
            want[slot0:slot0 + k] = True
    assert (written == want).all(), f"{name}: written slots {np.nonzero(written)[0].tolist()}"
    assert int(ws[:case.R * case.Hkv * 256].view(torch.int32).count_nonzero()) == 0  # counters back at zero
    # reruns bit-identical
    again = drafter_attn_qknorm(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def test_static_plan_is_kept_for_equal_long_contexts():
    # equal 16k-token contexts at stride 256: Pb would be 40 > 24 = 3/4 of Ps 32: static plan
    case = _mk(8, 24, 4, [16384] * 8, 256, 505)
    balanced, _, slots = _expected_schedule(case)
    assert not balanced
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace

    S, _ = _plan(case.R, case.Hkv, case.stride)
    g = ds.to_device(case, "cuda")
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
    part_o = (case.R * case.Hkv * 256 + 255) // 256 * 256
    ws[part_o:part_o + case.R * case.Hkv * S * ROW] = 0xFF
    say("equal 16k contexts: static plan")
    out = drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight,
                              g.k_norm_weight, num_q_heads=24, num_kv_heads=4, tokens_per_block=8, workspace=ws)
    torch.cuda.synchronize()
    check(to_np(out), reference(case), "equal16k")
    written = torch.isfinite(ws[part_o:part_o + case.R * case.Hkv * S * ROW].view(torch.float32)
                             .view(-1, 48 * 64)[:, 0]).cpu().numpy()
    assert written.all()  # every request uses every split of the static plan


def test_balanced_plan_poison_changes_nothing():
    clean = _mk(8, 24, 4, [16384, 9000, 313, 0, 12000, 64, 4097, 777], 256, 506)
    poisoned = _mk(8, 24, 4, [16384, 9000, 313, 0, 12000, 64, 4097, 777], 256, 506, poison=True)
    assert _expected_schedule(clean)[0]
    say("balanced plan over poisoned pool and table")
    a, b = run(clean), run(poisoned)
    torch.cuda.synchronize()
    assert torch.isfinite(b.float()).all()
    assert torch.equal(a, b)


def test_paged_attention_under_the_balanced_plan():
    # the replaced path's attention (no own-block keys) uses the same schedule
    import oracle
    from speculative_decoding_drafter_amd import paged_attn

    case = _mk(8, 24, 4, [65536, 100, 0, 2000, 0, 1, 0, 64], 1024, 507)
    g = ds.to_device(case, "cuda")
    say("paged attention, balanced plan")
    out = paged_attn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, num_q_heads=24, num_kv_heads=4,
                     tokens_per_block=8, scale=case.scale)
    torch.cuda.synchronize()
    a = case.np_args()
    ref = oracle.paged_attn(a["qkv"], a["k_pool"], a["v_pool"], a["page_table"], a["context_lens"],
                            num_q_heads=24, num_kv_heads=4, tokens_per_block=8, scale=case.scale)
    got = to_np(out)
    empty = [r for r, L in enumerate(case.context_lens.tolist()) if L == 0]
    for r in empty:  # no key at all: zero rows
        assert not got[8 * r:8 * (r + 1)].any()
    keep = np.ones(64, dtype=bool)
    for r in empty:
        keep[8 * r:8 * (r + 1)] = False
    check(got[keep], ref[keep], "paged-balanced")


def test_graph_replays_switch_between_plans():
    # one captured call; lengths rewritten between replays so that the device takes the static
    # plan, then the balanced one, then the static one again: every replay equals an eager call
    # bit for bit, meets the bar, and leaves the counters at zero
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace

    pool_pages = 8 * 256 + 8
    pool = ds.device_normal_pool(pool_pages, 4, seed=508, device="cuda")
    draws = {
        "static": [16384] * 8,
        "balanced": [16384, 9000, 313, 0, 12000, 64, 4097, 777],
        "balanced2": [100, 16000, 2, 16384, 0, 5000, 0, 3],
    }
    cases = {k: ds.make_case(8, 8, 24, 4, v, seed=509 + i, stride=256, pool_pages=pool_pages, qknorm=True,
                             pool_override=pool) for i, (k, v) in enumerate(draws.items())}
    assert [_expected_schedule(c)[0] for c in cases.values()] == [False, True, True]
    g = ds.to_device(cases["static"], "cuda")
    out = torch.empty(64, 24 * 64, dtype=torch.bfloat16, device="cuda")
    ws = make_workspace(8, 8, 24, 4, 256, "cuda")
    ws_eager = make_workspace(8, 8, 24, 4, 256, "cuda")
    kw = dict(num_q_heads=24, num_kv_heads=4, tokens_per_block=8, scale=cases["static"].scale)

    def call(o, w):
        return drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                   g.q_norm_weight, g.k_norm_weight, out=o, workspace=w, **kw)

    call(out, ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, ws)
    torch.cuda.synchronize()
    pools_np = (pool[:, 0].double().cpu().numpy(), pool[:, 1].double().cpu().numpy())
    for name in ("static", "balanced", "static", "balanced2", "balanced"):
        new = cases[name]
        for f in ("qkv", "page_table", "context_lens", "positions", "q_norm_weight", "k_norm_weight"):
            getattr(g, f).copy_(getattr(new, f))
        say(f"replay with the {name} lengths")
        graph.replay()
        eager = call(torch.empty_like(out), ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{name}: replay != eager"
        assert int(ws[:8 * 4 * 256].view(torch.int32).count_nonzero()) == 0
        check(to_np(out), reference(new, pools_np), f"replay-{name}")


def test_request_isolation_under_the_balanced_plan():
    # The balanced plan depends on the lengths only.  Rewriting one request's qkv rows, pages
    # and positions leaves every other request's output bits unchanged, and so does a new
    # length for it that keeps the split size Pb; a length that moves Pb moves the other
    # requests' split boundaries, so their outputs stay within the bar but may change bits.
    base = _mk(8, 24, 4, [16384, 9000, 313, 0, 12000, 64, 4097, 777], 256, 510)
    g = ds.to_device(base, "cuda")
    say("isolation, balanced plan")
    before = run(base, g).clone()
    pb0 = _expected_schedule(base)[1]
    k = 2
    rows = slice(8 * k, 8 * (k + 1))
    other = torch.ones(64, dtype=torch.bool, device="cuda")
    other[rows] = False

    donor = _mk(8, 24, 4, [16384, 9000, 313, 0, 12000, 64, 4097, 777], 256, 511)
    # same length for request k: new rows, pages (its own page ids from another draw of the
    # same pool size) and positions
    mixed = ds.splice_request(base, donor, k)
    assert _expected_schedule(mixed)[1] == pb0
    g2 = ds.to_device(mixed, "cuda")
    g2.pool, g2.k_pool, g2.v_pool = g.pool, g.k_pool, g.v_pool
    got = run(mixed, g2)
    torch.cuda.synchronize()
    assert torch.equal(got[other], before[other])
    assert not torch.equal(got[rows], before[rows])

    # a new length for request k that keeps Pb
    same_pb = ds.splice_request(base, donor, k)
    same_pb.context_lens[k] = 600
    same_pb.positions[8 * k:8 * (k + 1)] = 600 + torch.arange(8, dtype=same_pb.positions.dtype)
    assert _expected_schedule(same_pb)[1] == pb0
    g3 = ds.to_device(same_pb, "cuda")
    g3.pool, g3.k_pool, g3.v_pool = g.pool, g.k_pool, g.v_pool
    got = run(same_pb, g3)
    torch.cuda.synchronize()
    assert torch.equal(got[other], before[other])
    check(to_np(got), reference(same_pb), "isolation-same-pb")

    # a length that moves Pb: the bar still holds for every request
    moved = ds.splice_request(base, donor, k)
    moved.context_lens[k] = 16384
    moved.positions[8 * k:8 * (k + 1)] = 16384 + torch.arange(8, dtype=moved.positions.dtype)
    assert _expected_schedule(moved)[1] != pb0
    moved = ds.make_case(8, 8, 24, 4, moved.context_lens.tolist(), seed=510, stride=256,
                         pool_pages=base.num_pages + 256, qknorm=True)
    check(to_np(run(moved)), reference(moved), "isolation-moved-pb")
