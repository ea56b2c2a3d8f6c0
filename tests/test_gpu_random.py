"""Seeded random cases across the whole contract, against the fp64 oracle (GPU).

Each case draws R, T in 1..8, Hkv in {1, 2, 4, 8, 16}, context lengths biased
toward page edges (0, 64k-1, 64k, 64k+1) up to 4 pages past a few hundred,
a page-table stride at or above the need, ragged block lengths, qknorm or
plain, int32 or int64 positions with offsets, poison, qkv row padding and
separate pools; about a third of the qknorm cases use YaRN with drawn
parameters (factor, original context, ramp bounds and shape, factor on q and k).  Each must meet the acceptance bar; a rerun must be bit-identical.
Also: the binding refuses wrong dtypes and shapes.
"""
import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
from tests.gpu_util import check, reference, run, say, to_np

pytestmark = pytest.mark.gpu


def _draw(i: int) -> ds.DrafterCase:
    rng = np.random.default_rng(9000 + i)
    R = int(rng.integers(1, 9))
    T = int(rng.integers(1, 9))
    hkv = int(rng.choice([1, 2, 4, 8, 16]))
    lens = []
    for _ in range(R):
        k = int(rng.integers(0, 12))
        edge = [0, 64 * k - 1, 64 * k, 64 * k + 1][int(rng.integers(0, 4))]
        lens.append(max(0, edge) if rng.random() < 0.6 else int(rng.integers(0, 800)))
    need = max(-(-L // 64) for L in lens)
    stride = need + int(rng.integers(0, 4))
    qknorm = bool(rng.random() < 0.6)
    block_lens = [int(rng.integers(1, T + 1)) for _ in range(R)] if rng.random() < 0.4 else None
    return ds.make_case(
        R, T, 6 * hkv, hkv, lens, seed=9100 + i, stride=stride, pool_pages=max(1, sum(-(-L // 64) for L in lens)) + 3,
        qknorm=qknorm, pos_dtype=torch.int64 if rng.random() < 0.5 else torch.int32, block_lens=block_lens,
        poison=bool(rng.random() < 0.4), separate_pools=bool(rng.random() < 0.3),
        qkv_row_pad=int(rng.choice([0, 8, 64])),
        pos_offset=[int(x) for x in rng.integers(0, 100000, R)] if qknorm and rng.random() < 0.5 else None)


def _yarn_draw(i: int, case: ds.DrafterCase):
    # about a third of the qknorm cases use YaRN with drawn parameters
    rng = np.random.default_rng(9500 + i)
    if not case.qknorm or rng.random() >= 0.35:
        return None
    a = float(rng.uniform(0.0, 4.0))
    y = dict(factor=float(rng.choice([1.0, 2.0, 4.0, 8.0])), original_max_position=int(rng.choice([256, 4096, 32768])),
             alpha=a, beta=a + float(rng.uniform(1.0, 64.0)))
    # the ramp's shape and the factor on q and k (drawn after the rest, which stays as it was)
    y["ramp"] = str(rng.choice(["turns", "index", "index_unrounded"]))
    if rng.random() < 0.3:
        y["mscale"] = float(rng.uniform(0.5, 2.0))
    return y


@pytest.mark.parametrize("i", range(40))
def test_random_case(i):
    case = _draw(i)
    yarn = _yarn_draw(i, case)
    say(f"random {i}: R={case.R} T={case.T} Hkv={case.Hkv} lens={case.context_lens.tolist()} "
        f"stride={case.stride} qknorm={case.qknorm} blens={None if case.block_lens is None else case.block_lens.tolist()} "
        f"yarn={yarn}")
    g = ds.to_device(case, "cuda")
    kw = {} if yarn is None else dict(yarn=yarn)
    out = run(case, g, **kw)
    again = run(case, g, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "rerun not bit-identical"
    ref = reference(case) if yarn is None else oracle.drafter_attn_qknorm(**case.np_args(), yarn=yarn)
    check(to_np(out), ref, f"random{i}")


def test_binding_refuses_wrong_dtypes_and_shapes():
    from speculative_decoding_drafter_amd import DrafterAttnError, qk_norm_rope

    case = ds.make_config(2)
    g = ds.to_device(case, "cuda")
    say("dtype and shape errors")
    bad = [
        dict(qkv=g.qkv.half()),
        dict(page_table=g.page_table.long()),
        dict(context_lens=g.context_lens.long()),
        dict(positions=g.positions.float()),
        dict(q_norm_weight=g.q_norm_weight.float()),
        dict(k_norm_weight=g.k_norm_weight[:32]),
        dict(block_lens=torch.ones(3, dtype=torch.int32, device="cuda")),
        dict(out=torch.empty(case.R * case.T, 100, dtype=torch.bfloat16, device="cuda")),
    ]
    for over in bad:
        h = ds.to_device(case, "cuda")
        for k, v in over.items():
            setattr(h, k, v)
        with pytest.raises(DrafterAttnError):
            run(case, h, **({"out": over["out"]} if "out" in over else {}))
    with pytest.raises(DrafterAttnError):       # tokens_per_block above 8
        run(case, g, tokens_per_block=9)
    with pytest.raises(DrafterAttnError):       # qkv rows != R*T
        run(case, g, tokens_per_block=4)
    with pytest.raises(DrafterAttnError):       # CPU tensors: there is no CPU path
        run(case, case)
    with pytest.raises(DrafterAttnError):
        qk_norm_rope(g.qkv, g.positions[:5], g.q_norm_weight, g.k_norm_weight, num_q_heads=6, num_kv_heads=1)
