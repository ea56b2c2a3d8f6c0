"""Workspace counters and concurrent streams (GPU).

* Every call leaves the workspace's arrival counters at zero, also when a request
  uses fewer splits than the plan has (length-aware split use) -- the next call,
  or a graph replay, needs them zeroed.
* Calls on two streams at once, each with its own workspace, give the same bits
  as the same calls one after the other.
"""
import pytest
import torch

import drafter_synth as ds
from tests.gpu_util import run, say

pytestmark = pytest.mark.gpu


def _counters(ws: torch.Tensor, R: int, Hkv: int) -> torch.Tensor:
    # the workspace starts with one 32-bit arrival counter per (request, KV head), 256 bytes apart
    # (the words between them are never touched: the whole region must read zero)
    return ws[:256 * R * Hkv].view(torch.int32)


@pytest.mark.parametrize("name", ["cfg2", "cfg3", "short_and_long", "single_split"])
def test_counters_left_zero(name):
    from speculative_decoding_drafter_amd import make_workspace, plan

    case = {
        "cfg2": lambda: ds.make_config(2),
        "cfg3": lambda: ds.make_config(3),
        # one request reaches every split, the others only the first one or two
        "short_and_long": lambda: ds.make_case(4, 8, 24, 4, [20000, 0, 700, 64], seed=81, qknorm=True),
        "single_split": lambda: ds.make_case(2, 3, 6, 1, [5, 130], seed=82),
    }[name]()
    g = ds.to_device(case, "cuda")
    S, _ = plan(case.R, case.Hkv, case.stride)
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
    say(f"counters {name}: S={S}")
    for _ in range(3):
        run(case, g, workspace=ws)
        torch.cuda.synchronize()
        assert int(_counters(ws, case.R, case.Hkv).abs().sum()) == 0


def test_two_streams_concurrently():
    from speculative_decoding_drafter_amd import make_workspace

    cases = [ds.make_config(3), ds.make_config(2), ds.make_case(8, 8, 24, 4, [4096] * 8, seed=83, qknorm=True)]
    devs = [ds.to_device(c, "cuda") for c in cases]
    wss = [make_workspace(c.R, c.T, c.Hq, c.Hkv, c.stride, "cuda") for c in cases]
    ref = [run(c, d, workspace=w).clone() for c, d, w in zip(cases, devs, wss)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[] for _ in cases]
    say("three streams, 20 calls each, interleaved")
    for _ in range(20):
        for k, (c, d, w, st) in enumerate(zip(cases, devs, wss, streams)):
            with torch.cuda.stream(st):
                outs[k].append(run(c, d, workspace=w))
    torch.cuda.synchronize()
    for k in range(len(cases)):
        for o in outs[k]:
            assert torch.equal(o.view(torch.int16), ref[k].view(torch.int16)), f"stream {k}"
