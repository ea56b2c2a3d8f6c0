"""YaRN-scaled rotation in the qknorm attention and in the standalone norm/rotation (GPU).

The drafter checkpoint is named with "YaRN 4.0"; the other parameters are the
caller's (here a 4096-token original context and the published ramp 1..32).
* the attention against the fp64 oracle at the acceptance bar (configs 2, 3, 5 and
  positions far past the original context);
* factor 1 gives the plain rotation's bits;
* the standalone op against the oracle within one bf16 ulp plus fp32 rounding, and
  plain attention on its rows == the fused attention, bit for bit;
* graph replay with rewritten positions equals eager calls, bit for bit;
* the ramps linear in the pair index (rounded and unrounded bounds) and an explicit
  factor on q and k, against the oracle, in the attention and the standalone op.
"""
import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
from tests.gpu_util import ATOL, MEAN_TOL, RTOL, check, say, to_np

pytestmark = pytest.mark.gpu

YARN = dict(factor=4.0, original_max_position=4096, alpha=1.0, beta=32.0)


def _fused(case, g, yarn, **kw):
    from speculative_decoding_drafter_amd import drafter_attn_qknorm

    return drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                               g.q_norm_weight, g.k_norm_weight, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                               tokens_per_block=case.T, block_lens=g.block_lens, scale=case.scale, eps=case.eps,
                               rope_base=case.rope_base, yarn=yarn, **kw)


def _ref(case, yarn):
    return oracle.drafter_attn_qknorm(**case.np_args(), yarn=yarn)


@pytest.mark.parametrize("name", ["cfg2", "cfg3", "cfg5", "far_positions"])
def test_qknorm_yarn_matches_oracle(name):
    case = {
        "cfg2": lambda: ds.make_config(2),
        "cfg3": lambda: ds.make_config(3),
        "cfg5": lambda: ds.make_config(5),
        "far_positions": lambda: ds.make_case(3, 8, 24, 4, [300, 0, 1500], seed=41, qknorm=True,
                                              pos_dtype=torch.int64, pos_offset=[100000, 7, 3_000_000]),
    }[name]()
    g = ds.to_device(case, "cuda")
    say(f"yarn {name}")
    got = to_np(_fused(case, g, YARN))
    ref = _ref(case, YARN)
    check(got, ref, f"yarn-{name}")
    # the scaling really changes the answer: the plain rotation's result would fail the bar
    plain = _ref(case, None)
    err = np.abs(plain - ref)
    assert err.mean() > MEAN_TOL or np.any(err > ATOL + RTOL * np.abs(ref))


def test_yarn_factor_one_is_the_plain_rotation_bitwise():
    case = ds.make_config(3)
    g = ds.to_device(case, "cuda")
    say("yarn factor 1")
    plain = _fused(case, g, None)
    one = _fused(case, g, dict(factor=1.0, original_max_position=64, alpha=0.5, beta=2.0))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), one.view(torch.int16))


def _bf16_ulp(x):
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


@pytest.mark.parametrize("hkv,pdt", [(1, torch.int32), (4, torch.int64)])
def test_norm_rope_yarn_matches_oracle(hkv, pdt):
    from speculative_decoding_drafter_amd import qk_norm_rope

    rows = ds.make_norm_rope_rows(257, hkv, seed=600 + hkv, row_pad=16, pos_dtype=pdt, pos_max=1 << 20,
                                  poison_pad=True)
    say(f"norm_rope yarn Hkv={hkv}")
    got = qk_norm_rope(rows.qkv.cuda(), rows.positions.cuda(), rows.q_norm_weight.cuda(), rows.k_norm_weight.cuda(),
                       num_q_heads=rows.Hq, num_kv_heads=rows.Hkv, yarn=YARN).cpu()
    ref = oracle.qk_norm_rope(rows.qkv.double().numpy(), rows.positions.numpy(), rows.q_norm_weight.double().numpy(),
                              rows.k_norm_weight.double().numpy(), num_q_heads=rows.Hq, num_kv_heads=rows.Hkv,
                              yarn=YARN)
    qk = slice(0, (rows.Hq + rows.Hkv) * 64)
    rest = slice((rows.Hq + rows.Hkv) * 64, None)
    assert torch.equal(got[:, rest].view(torch.int16), rows.qkv[:, rest].view(torch.int16))
    gq, rq = got[:, qk].double().numpy(), ref[:, qk]
    head_max = np.abs(rq).reshape(rq.shape[0], -1, 64).max(axis=2, keepdims=True)
    fp32 = np.ldexp(np.broadcast_to(head_max, (rq.shape[0], rq.shape[1] // 64, 64)).reshape(rq.shape), -18)
    bound = np.maximum(_bf16_ulp(rq), _bf16_ulp(gq)) + fp32
    err = np.abs(gq - rq)
    say(f"max |err|/bound = {np.max(err / bound):.3f}")
    assert np.isfinite(gq).all() and np.all(err <= bound)


@pytest.mark.parametrize("n", [2, 3])
def test_processed_rows_compose_with_plain_attention_bitwise(n):
    from speculative_decoding_drafter_amd import drafter_attn, qk_norm_rope

    case = ds.make_config(n)
    g = ds.to_device(case, "cuda")
    say(f"yarn composition config {n}")
    fused = _fused(case, g, YARN)
    rows = g.qkv.clone()
    qk_norm_rope(rows, g.positions, g.q_norm_weight, g.k_norm_weight, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                 eps=case.eps, rope_base=case.rope_base, yarn=YARN)
    plain = drafter_attn(rows, g.k_pool, g.v_pool, g.page_table, g.context_lens, num_q_heads=case.Hq,
                         num_kv_heads=case.Hkv, tokens_per_block=case.T, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), fused.view(torch.int16))


def test_graph_replay_with_rewritten_positions():
    from speculative_decoding_drafter_amd import make_workspace

    case = ds.make_config(3)
    g = ds.to_device(case, "cuda")
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, "cuda")
    out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device="cuda")
    _fused(case, g, YARN, out=out, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _fused(case, g, YARN, out=out, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    for k in range(3):
        g.positions.copy_(torch.from_numpy(rng.integers(0, 200000, case.R * case.T)).to(g.positions.dtype))
        say(f"yarn replay {k}")
        graph.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        eager = _fused(case, g, YARN)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), eager.view(torch.int16))
        case.positions = g.positions.cpu()
        check(to_np(replayed), _ref(case, YARN), f"yarn-replay{k}")


VARIANTS = {
    "index": dict(YARN, ramp="index"),
    "index_unrounded": dict(YARN, ramp="index_unrounded", mscale=1.0),
    "index_mscale": dict(YARN, ramp="index", mscale=1.25),
    "turns_mscale_one": dict(YARN, mscale=1.0),
    "factor_one_mscale": dict(factor=1.0, original_max_position=4096, ramp="index", mscale=1.3),
}


@pytest.mark.parametrize("name", ["cfg3", "far_positions"])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_qknorm_yarn_variants_match_oracle(name, variant):
    case = {
        "cfg3": lambda: ds.make_config(3),
        "far_positions": lambda: ds.make_case(3, 8, 24, 4, [300, 0, 1500], seed=41, qknorm=True,
                                              pos_dtype=torch.int64, pos_offset=[100000, 7, 3_000_000]),
    }[name]()
    yarn = VARIANTS[variant]
    g = ds.to_device(case, "cuda")
    say(f"yarn {variant} {name}")
    got = to_np(_fused(case, g, yarn))
    ref = _ref(case, yarn)
    check(got, ref, f"yarn-{variant}-{name}")
    # the variant really changes the answer: the default YaRN rotation's result would fail the bar
    other = _ref(case, YARN if variant != "factor_one_mscale" else None)
    err = np.abs(other - ref)
    assert err.mean() > MEAN_TOL or np.any(err > ATOL + RTOL * np.abs(ref))


def test_index_ramp_factor_one_is_the_plain_rotation_bitwise():
    case = ds.make_config(2)
    g = ds.to_device(case, "cuda")
    say("yarn index ramp, factor 1")
    plain = _fused(case, g, None)
    for ramp in ("index", "index_unrounded"):
        one = _fused(case, g, dict(factor=1.0, original_max_position=4096, ramp=ramp))
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16), one.view(torch.int16)), ramp


@pytest.mark.parametrize("variant", ["index", "index_unrounded", "factor_one_mscale"])
def test_norm_rope_yarn_variants_match_oracle(variant):
    from speculative_decoding_drafter_amd import qk_norm_rope

    yarn = VARIANTS[variant]
    rows = ds.make_norm_rope_rows(131, 4, seed=640, row_pad=8, pos_dtype=torch.int64, pos_max=1 << 22)
    say(f"norm_rope yarn {variant}")
    got = qk_norm_rope(rows.qkv.cuda(), rows.positions.cuda(), rows.q_norm_weight.cuda(), rows.k_norm_weight.cuda(),
                       num_q_heads=rows.Hq, num_kv_heads=rows.Hkv, yarn=yarn).cpu()
    ref = oracle.qk_norm_rope(rows.qkv.double().numpy(), rows.positions.numpy(), rows.q_norm_weight.double().numpy(),
                              rows.k_norm_weight.double().numpy(), num_q_heads=rows.Hq, num_kv_heads=rows.Hkv,
                              yarn=yarn)
    qk = slice(0, (rows.Hq + rows.Hkv) * 64)
    gq, rq = got[:, qk].double().numpy(), ref[:, qk]
    head_max = np.abs(rq).reshape(rq.shape[0], -1, 64).max(axis=2, keepdims=True)
    fp32 = np.ldexp(np.broadcast_to(head_max, (rq.shape[0], rq.shape[1] // 64, 64)).reshape(rq.shape), -18)
    bound = np.maximum(_bf16_ulp(rq), _bf16_ulp(gq)) + fp32
    err = np.abs(gq - rq)
    say(f"max |err|/bound = {np.max(err / bound):.3f}")
    assert np.isfinite(gq).all() and np.all(err <= bound)
