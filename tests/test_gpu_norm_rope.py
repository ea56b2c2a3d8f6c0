"""The standalone q/k RMSNorm + NeoX rotation (fused_qk_norm_rope's drafter cell) on the GPU.

* against the fp64 oracle: every q/k value within one bf16 ulp of the exact result plus
  fp32 rounding on the scale of its head (fp32 arithmetic, one rounding to bf16 at the
  end; a rotated value can cancel to near zero), v heads and row padding
  bit-untouched, for 1..64 tokens (the cell) and a long row list, both layouts,
  int32 and int64 positions;
* composition: plain attention on rows processed by this op is bit-identical to
  the qknorm attention on the original rows (the two share the arithmetic);
* graph capture with rewritten rows and positions; reruns bit-identical.
"""
import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _apply(rows: ds.NormRopeRows, qkv=None, positions=None):
    from speculative_decoding_drafter_amd import qk_norm_rope

    return qk_norm_rope(rows.qkv.cuda() if qkv is None else qkv,
                        rows.positions.cuda() if positions is None else positions,
                        rows.q_norm_weight.cuda(), rows.k_norm_weight.cuda(),
                        num_q_heads=rows.Hq, num_kv_heads=rows.Hkv)


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    # bf16 keeps 8 significant bits: ulp(x) = 2^(e - 8) with x = m 2^e, 0.5 <= |m| < 1
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


def _check_rows(rows: ds.NormRopeRows, got: torch.Tensor, name: str):
    ref = oracle.qk_norm_rope(rows.qkv.double().numpy(), rows.positions.numpy(),
                              rows.q_norm_weight.double().numpy(), rows.k_norm_weight.double().numpy(),
                              num_q_heads=rows.Hq, num_kv_heads=rows.Hkv)
    g = got.cpu()
    qk = slice(0, (rows.Hq + rows.Hkv) * 64)
    rest = slice((rows.Hq + rows.Hkv) * 64, None)
    # v heads and padding: the same bits as the input (NaN padding included)
    assert torch.equal(g[:, rest].view(torch.int16), rows.qkv[:, rest].view(torch.int16)), f"{name}: v/padding changed"
    gq = g[:, qk].double().numpy()
    rq = ref[:, qk]
    err = np.abs(gq - rq)
    # One bf16 ulp of the result (the final rounding, which fp32 noise can tip at a
    # midpoint), plus the fp32 rounding of the rotation a*cos - b*sin, which scales with
    # the head's values rather than with a result that cancels to near zero: bounded by
    # 2^-18 of the head's largest value (about 64x the fp32 unit roundoff).
    head_max = np.abs(rq).reshape(rq.shape[0], -1, 64).max(axis=2, keepdims=True)
    fp32 = np.ldexp(np.broadcast_to(head_max, (rq.shape[0], rq.shape[1] // 64, 64)).reshape(rq.shape), -18)
    bound = np.maximum(_bf16_ulp(rq), _bf16_ulp(gq)) + fp32
    say(f"{name}: max |err|/bound = {np.max(err / bound):.3f}, max|err| = {err.max():.3e}")
    assert np.isfinite(gq).all()
    assert np.all(err <= bound), f"{name}: beyond one bf16 ulp + fp32 rounding of the fp64 result"


@pytest.mark.parametrize("N", [1, 7, 8, 9, 33, 64])
@pytest.mark.parametrize("hkv,pdt", [(1, torch.int32), (4, torch.int64)])
def test_matches_oracle(N, hkv, pdt):
    rows = ds.make_norm_rope_rows(N, hkv, seed=500 + N + 10 * hkv, row_pad=16, pos_dtype=pdt, poison_pad=True)
    say(f"norm_rope N={N} Hkv={hkv} {pdt}")
    _check_rows(rows, _apply(rows), f"N{N}H{hkv}")


def test_long_row_list_and_large_positions():
    rows = ds.make_norm_rope_rows(4099, 4, seed=77, pos_dtype=torch.int64, pos_max=1 << 20)
    say("norm_rope N=4099 Hkv=4 pos<=2^20")
    _check_rows(rows, _apply(rows), "N4099")


def test_int64_positions_beyond_int32():
    # positions up to 2^33 (past the int32 range, and past fp32's 24-bit exact integers by
    # 2^9): the angle is formed and reduced in fp64
    rows = ds.make_norm_rope_rows(256, 4, seed=78, pos_dtype=torch.int64, pos_max=1 << 33)
    assert int(rows.positions.max()) > 1 << 31
    say("norm_rope int64 positions up to 2^33")
    _check_rows(rows, _apply(rows), "pos2^33")


def test_reruns_bit_identical():
    rows = ds.make_norm_rope_rows(64, 4, seed=9)
    a, b = _apply(rows), _apply(rows)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n,blens", [(2, None), (3, None), (5, None), (3, [8, 1, 5, 8, 3, 8, 2, 7])])
def test_plain_attention_of_processed_rows_equals_qknorm_attention(n, blens):
    # the pool holds already-processed keys; only the block's q and k differ between the two paths
    from speculative_decoding_drafter_amd import drafter_attn, drafter_attn_qknorm, qk_norm_rope

    case = ds.make_config(n)
    g = ds.to_device(case, "cuda")
    bl = None if blens is None else torch.tensor(blens, dtype=torch.int32, device="cuda")
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, scale=case.scale, block_lens=bl)
    say(f"composition config {n} block_lens={blens}")
    fused = drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                g.q_norm_weight, g.k_norm_weight, eps=case.eps, rope_base=case.rope_base, **kw)
    rows = g.qkv.clone()
    qk_norm_rope(rows, g.positions, g.q_norm_weight, g.k_norm_weight, num_q_heads=case.Hq,
                 num_kv_heads=case.Hkv, eps=case.eps, rope_base=case.rope_base)
    plain = drafter_attn(rows, g.k_pool, g.v_pool, g.page_table, g.context_lens, **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), fused.view(torch.int16))


def test_graph_replay_with_rewritten_rows():
    from speculative_decoding_drafter_amd import qk_norm_rope

    first = ds.make_norm_rope_rows(40, 1, seed=31)
    qkv = first.qkv.cuda()
    pos = first.positions.cuda()
    wq, wk = first.q_norm_weight.cuda(), first.k_norm_weight.cuda()
    qk_norm_rope(qkv, pos, wq, wk, num_q_heads=6, num_kv_heads=1)   # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qk_norm_rope(qkv, pos, wq, wk, num_q_heads=6, num_kv_heads=1)
    torch.cuda.synchronize()
    for k in range(3):
        new = ds.make_norm_rope_rows(40, 1, seed=32 + k)
        qkv.copy_(new.qkv)
        pos.copy_(new.positions)
        say(f"replay {k}")
        graph.replay()
        eager = qk_norm_rope(new.qkv.cuda(), new.positions.cuda(), wq, wk, num_q_heads=6, num_kv_heads=1)
        torch.cuda.synchronize()
        assert torch.equal(qkv.view(torch.int16), eager.view(torch.int16))
        # the graph used the first draw's weights, which are the same tensors as above
        new.q_norm_weight, new.k_norm_weight = first.q_norm_weight, first.k_norm_weight
        _check_rows(new, qkv, f"replay{k}")
