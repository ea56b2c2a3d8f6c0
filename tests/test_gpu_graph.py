"""HIP-graph capture and replay with rewritten device inputs (the split sweep).

For every (requests, tokens) pair in 1..8 x 1..8 and both head layouts (6/1 with
int32 positions, 24/4 with int64), one qknorm call is captured into a graph
after an eager warm-up.  Three times, the context lengths, page table, qkv,
positions and norm weights are redrawn and rewritten in place; the replay must
match the fp64 oracle within tolerance and an eager call on the same buffers
bit for bit.  Then, with two or more requests, only one request's qkv rows,
page-table row, length and positions are rewritten: the next replay must leave
every other request's output rows bit-identical (requests isolated), change that
request's rows, and match the oracle.  Lengths, page tables and qkv are read on
the device, which is what makes the replays valid.
"""
import numpy as np
import pytest
import torch

import drafter_synth as ds
from tests.gpu_util import check, reference, say

pytestmark = pytest.mark.gpu


class Captured:
    """Device buffers of one cell, a workspace and a graph holding one call."""

    def __init__(self, case: ds.DrafterCase, pool_dev: torch.Tensor):
        from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace

        self.case = case
        g = ds.to_device(case, "cuda")
        g.pool, g.k_pool, g.v_pool = pool_dev, pool_dev[:, 0], pool_dev[:, 1]
        self.g = g
        self.out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device="cuda")
        self.out_eager = torch.empty_like(self.out)
        self.ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
        self.ws_eager = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
        self.fn = drafter_attn_qknorm

        self.call(self.out, self.ws)            # warm-up outside capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.call(self.out, self.ws)
        torch.cuda.synchronize()

    def call(self, out, ws):
        g, c = self.g, self.case
        return self.fn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions, g.q_norm_weight,
                       g.k_norm_weight, num_q_heads=c.Hq, num_kv_heads=c.Hkv, tokens_per_block=c.T,
                       scale=c.scale, out=out, workspace=ws)

    def rewrite(self, new: ds.DrafterCase):
        g = self.g
        for name in ("qkv", "page_table", "context_lens", "positions", "q_norm_weight", "k_norm_weight"):
            getattr(g, name).copy_(getattr(new, name))
        self.case = new


@pytest.fixture(scope="module")
def pools():
    out = {}
    for hkv in (1, 4):
        p = ds.config4_pool(hkv)
        out[hkv] = (p, p.cuda(), (p[:, 0].double().numpy(), p[:, 1].double().numpy()))
    return out


@pytest.mark.parametrize("hkv", [1, 4])
def test_split_sweep_graph_replay(hkv, pools):
    pool, pool_dev, pools_np = pools[hkv]
    worst = 0.0
    for r in range(1, 9):
        for t in range(1, 9):
            say(f"sweep Hkv={hkv} r={r} t={t}")
            cap = Captured(ds.config4_cell(r, t, hkv, 0, pool=pool), pool_dev)
            for k in range(3):
                new = ds.config4_cell(r, t, hkv, k, pool=pool)
                cap.rewrite(new)
                cap.graph.replay()
                eager = cap.call(cap.out_eager, cap.ws_eager)
                torch.cuda.synchronize()
                assert torch.equal(cap.out, eager), f"replay != eager at r={r} t={t} k={k}"
                got = cap.out.float().cpu().numpy().astype(np.float64)
                ref = reference(new, pools_np)
                err = np.abs(got - ref)
                assert np.isfinite(got).all()
                assert np.all(err <= 2e-2 + 2e-2 * np.abs(ref)), f"r={r} t={t} k={k}: max err {err.max():.3e}"
                assert err.mean() <= 2e-3
                worst = max(worst, float(err.max()))
            if r >= 2:
                worst = max(worst, _isolated_replay(cap, r, t, hkv, pool, pools_np))
    say(f"sweep Hkv={hkv}: worst max|err| {worst:.3e}")


def _isolated_replay(cap: Captured, r: int, t: int, hkv: int, pool, pools_np) -> float:
    """Rewrite one request in place between two replays; the others' rows keep their bits."""
    k = (3 * r + t) % r
    donor = ds.config4_cell(r, t, hkv, 5, pool=pool)
    if int(donor.context_lens[k]) == int(cap.case.context_lens[k]):
        donor.context_lens[k] = int(donor.context_lens[k]) // 3   # the length must change too
        donor.positions[k * t:(k + 1) * t] = donor.context_lens[k] + torch.arange(t, dtype=donor.positions.dtype)
    mixed = ds.splice_request(cap.case, donor, k)
    before = cap.out.clone()
    g, rows = cap.g, slice(k * t, (k + 1) * t)
    g.qkv[rows].copy_(donor.qkv[rows])
    g.page_table[k].copy_(donor.page_table[k])
    g.context_lens[k:k + 1].copy_(donor.context_lens[k:k + 1])
    g.positions[rows].copy_(donor.positions[rows])
    cap.case = mixed
    cap.graph.replay()
    eager = cap.call(cap.out_eager, cap.ws_eager)
    torch.cuda.synchronize()
    mine = torch.zeros(r * t, dtype=torch.bool, device="cuda")
    mine[rows] = True
    assert torch.equal(cap.out[~mine], before[~mine]), f"r={r} t={t}: rewriting request {k} moved other requests"
    assert not torch.equal(cap.out[mine], before[mine]), f"r={r} t={t}: request {k} did not change"
    assert torch.equal(cap.out, eager), f"r={r} t={t}: isolated replay != eager"
    got = cap.out.float().cpu().numpy().astype(np.float64)
    ref = reference(mixed, pools_np)
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert np.all(err <= 2e-2 + 2e-2 * np.abs(ref)), f"isolation r={r} t={t}: max err {err.max():.3e}"
    assert err.mean() <= 2e-3
    return float(err.max())


def test_replay_bit_stable_2000(pools):
    # 2,000 replays of one captured call with fixed inputs: every output identical
    pool, pool_dev, pools_np = pools[4]
    cap = Captured(ds.config4_cell(8, 8, 4, 0, pool=pool), pool_dev)
    say("2000 replays")
    cap.graph.replay()
    torch.cuda.synchronize()
    first = cap.out.clone()
    check(first.float().cpu().numpy().astype(np.float64), reference(cap.case, pools_np), "replay-first")
    mismatches = 0
    for i in range(2000):
        cap.graph.replay()
        if i % 100 == 99:
            cap.call(cap.out_eager, cap.ws_eager)  # eager work between replays
        mismatches += int(not torch.equal(cap.out, first))
    assert mismatches == 0


def test_capture_with_poisoned_memory():
    # capture at R = 8 over a poisoned pool and table, then replay after rewriting
    case = ds.config4_cell(8, 8, 4, 0, poison=True)
    pool_dev = case.pool.cuda()
    say("poisoned capture")
    cap = Captured(case, pool_dev)
    cap.graph.replay()
    torch.cuda.synchronize()
    got = cap.out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    clean = ds.config4_cell(8, 8, 4, 0)
    check(got, reference(clean), "poison-capture")
