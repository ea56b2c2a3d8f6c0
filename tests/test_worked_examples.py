"""Hand-derived worked examples for the oracle, plus the pages' problem constants.

Each example is small enough to solve on paper; the expected values are those
derivations evaluated with Python's ``math`` (nothing is taken from the oracle
or from the GPU path).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLDEN, "contract_facts.json")) as f:
        return json.load(f)


def test_two_key_softmax_example():
    """One context key e_0 (value e_1) and one block key 0 (value e_2); q = 8 e_0, scale 1/8.

    Scores are (1, 0), so the output is sigmoid(1) e_1 + (1 - sigmoid(1)) e_2 for every head.
    """
    case = ds.make_case(1, 1, 6, 1, [1], seed=1, pool_pages=2)
    case.qkv.zero_()
    for h in range(6):
        case.qkv[0, h * 64] = 8.0
    case.qkv[0, 7 * 64 + 2] = 1.0                      # block value e_2 (block key stays 0)
    p = int(case.page_table[0, 0])
    case.k_pool[p, 0, 0].zero_()
    case.k_pool[p, 0, 0, 0] = 1.0
    case.v_pool[p, 0, 0].zero_()
    case.v_pool[p, 0, 0, 1] = 1.0
    out = oracle.drafter_attn(**case.np_args())
    w = 1.0 / (1.0 + math.exp(-1.0))
    for h in range(6):
        exp = np.zeros(64)
        exp[1], exp[2] = w, 1.0 - w
        np.testing.assert_allclose(out[0, h * 64:(h + 1) * 64], exp, rtol=0, atol=1e-15)


def test_norm_and_rotation_example():
    """No context, two block tokens at positions 5 and 6, unit weights.

    q = k = e_0 for both tokens; RMSNorm scales e_0 by n = 1/sqrt(1/64 + 1e-5);
    rotation by p puts it at n (cos p e_0 + sin p e_32), so the score of token t
    against key j is (n^2 / 8) cos(p_t - p_j).  Values are e_3 and e_4.
    """
    case = ds.make_case(1, 2, 6, 1, [0], seed=2, stride=0, qknorm=True)
    case.qkv.zero_()
    for t in range(2):
        for h in range(6):
            case.qkv[t, h * 64] = 1.0
        case.qkv[t, 6 * 64] = 1.0
        case.qkv[t, 7 * 64 + 3 + t] = 1.0
    case.q_norm_weight.fill_(1.0)
    case.k_norm_weight.fill_(1.0)
    case.positions = torch.tensor([5, 6], dtype=torch.int32)
    out = oracle.drafter_attn_qknorm(**case.np_args())
    n2 = 1.0 / (1.0 / 64 + 1e-5)
    s_same, s_diff = n2 / 8, n2 / 8 * math.cos(1.0)
    w_same = 1.0 / (1.0 + math.exp(s_diff - s_same))
    for t in range(2):
        exp = np.zeros(64)
        exp[3 + t] = w_same
        exp[3 + (1 - t)] = 1.0 - w_same
        for h in range(6):
            np.testing.assert_allclose(out[t, h * 64:(h + 1) * 64], exp, rtol=0, atol=1e-14)


def test_oracle_respects_contract_facts():
    f = _facts()
    assert oracle.drafter_attn_oracle.GQA == f["q_heads_per_kv_head"]
    assert oracle.drafter_attn_oracle.HEAD_DIM == f["head_dim"]
    assert oracle.drafter_attn_oracle.PAGE == f["page_size"]
    lo, hi = f["context_length_range"]
    for hq, hkv in f["head_layouts"]:
        case = ds.make_case(f["max_requests"], f["max_tokens_per_block"], hq, hkv,
                            [lo, hi] + [7] * (f["max_requests"] - 2), seed=3, qknorm=True)
        out = oracle.drafter_attn_qknorm(**case.np_args(), )
        assert np.isfinite(out).all()
    big = ds.make_case(1, 1, 6, 1, [1], seed=4)
    a = big.np_args()
    a["qkv"] = np.zeros((9, 512))
    a["context_lens"] = np.ones(9, dtype=np.int64)
    a["page_table"] = np.zeros((9, 1), dtype=np.int64)
    with pytest.raises(oracle.OracleContractError):
        oracle.drafter_attn(**a)
