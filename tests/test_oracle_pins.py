"""Pins of the fp64 oracle against things other than itself (CPU only).

The pages print no worked example for this kernel, so the oracle is pinned by:
an independently built brute force (one masked softmax over the whole batch),
torch's float64 scaled_dot_product_attention on gathered tensors, closed forms
(L=0/T=1, q=0, constant V, needle keys, RMSNorm of a constant vector, rotary
values at exactly representable frequencies), and invariants (softmax weights
sum to one, physical page placement, request isolation, poison, composition of
the qknorm variant, split-merge algebra).
"""
import math

import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
from tests.bruteforce import bruteforce

TOL = 1e-12


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1.0, float(np.max(np.abs(b)))))


def _tiny_cases():
    out = []
    seed = 11
    for R in (1, 2, 3):
        for T in (1, 2, 3):
            for Hkv in (1, 2):
                lens = [[0, 1, 63, 64, 65, 130][(R * 7 + T * 3 + i + Hkv) % 6] for i in range(R)]
                for qk in (False, True):
                    seed += 1
                    out.append(ds.make_case(R, T, 6 * Hkv, Hkv, lens, seed=seed,
                                            stride=max(3, max(-(-L // 64) for L in lens)),
                                            pool_pages=12, qknorm=qk,
                                            pos_dtype=torch.int64 if qk else torch.int32))
    return out


def _oracle(case, **kw):
    a = case.np_args()
    a.update(kw)
    if case.qknorm:
        return oracle.drafter_attn_qknorm(**a)
    return oracle.drafter_attn(**a)


# ---------------------------------------------------------------------------------------
# P1: independent brute force
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: f"R{c.R}T{c.T}H{c.Hkv}{'n' if c.qknorm else 'p'}")
def test_bruteforce_tiny(case):
    ref = bruteforce(**case.np_args(), qknorm=case.qknorm)
    assert _rel(_oracle(case), ref) <= TOL


@pytest.mark.parametrize("n", [1, 2, 3])
def test_bruteforce_configs(n):
    case = ds.make_config(n)
    ref = bruteforce(**case.np_args(), qknorm=case.qknorm)
    assert _rel(_oracle(case), ref) <= TOL


def test_bruteforce_block_lens():
    case = ds.make_case(3, 5, 12, 2, [70, 0, 129], seed=5, block_lens=[2, 5, 1], qknorm=True,
                        pool_pages=8)
    out = _oracle(case)
    assert _rel(out, bruteforce(**case.np_args(), qknorm=True)) <= TOL
    # rows past a block length are zero
    assert np.all(out[2:5] == 0) and np.all(out[11:15] == 0)


# ---------------------------------------------------------------------------------------
# P2: library routine (torch float64 SDPA on gathered dense tensors, GQA expanded)
# ---------------------------------------------------------------------------------------

def _sdpa_reference(case):
    a = case.np_args()
    Hq, Hkv, T, D = case.Hq, case.Hkv, case.T, 64
    qkv = torch.from_numpy(a["qkv"])
    kp, vp = torch.from_numpy(a["k_pool"]), torch.from_numpy(a["v_pool"])
    out = torch.zeros(case.R * T, Hq * D, dtype=torch.float64)
    for r in range(case.R):
        L = int(a["context_lens"][r])
        idx = torch.arange(L)
        pages = torch.from_numpy(a["page_table"][r])[idx // 64] if L else idx
        rows = qkv[r * T:(r + 1) * T]
        q = rows[:, :Hq * D].reshape(T, Hq, D).transpose(0, 1)             # [Hq, T, D]
        kb = rows[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D).transpose(0, 1)
        vb = rows[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(T, Hkv, D).transpose(0, 1)
        kc = kp[pages, :, idx % 64, :].transpose(0, 1)                      # [Hkv, L, D]
        vc = vp[pages, :, idx % 64, :].transpose(0, 1)
        k = torch.cat([kc, kb], 1).repeat_interleave(6, 0)
        v = torch.cat([vc, vb], 1).repeat_interleave(6, 0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), scale=case.scale)[0]
        out[r * T:(r + 1) * T] = o.transpose(0, 1).reshape(T, Hq * D)
    return out.numpy()


@pytest.mark.parametrize("n", [1, 2, 3])
def test_sdpa_plain(n):
    case = ds.make_config(n)
    case.qknorm = False  # plain path on the same tensors
    assert _rel(oracle.drafter_attn(**case.np_args()), _sdpa_reference(case)) <= TOL


def test_sdpa_decode_special_case():
    # T=1, Hkv=1: ordinary single-query paged decode attention
    case = ds.make_case(4, 1, 6, 1, [1, 64, 700, 2041], seed=3, pool_pages=60)
    assert _rel(oracle.drafter_attn(**case.np_args()), _sdpa_reference(case)) <= TOL


# ---------------------------------------------------------------------------------------
# P3: split-merge algebra; P4 / I1: weights sum to one
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 2, 3, 7, 32])
def test_split_merge_equals_definition(S):
    case = ds.make_config(2)
    ref = _oracle(case)
    got = oracle.drafter_attn_split_merge(**case.np_args(), num_splits=S, qknorm=True)
    assert _rel(got, ref) <= 1e-13


@pytest.mark.parametrize("S,G", [(17, 8), (33, 8), (64, 8), (9, 4)])
def test_two_level_split_merge_equals_definition(S, G):
    # ranges merged in groups of G first, then the groups (the GPU's two-level combine);
    # with 64 splits of a 33-page row most groups hold no key at all
    case = ds.make_config(2)
    ref = _oracle(case)
    got = oracle.drafter_attn_split_merge(**case.np_args(), num_splits=S, group=G, qknorm=True)
    assert _rel(got, ref) <= 1e-13


def test_softmax_weights_sum_to_one():
    case = ds.make_config(3)
    _, probs = _oracle(case, return_probs=True)
    L = case.context_lens.tolist()
    for (r, h, t), p in probs.items():
        assert abs(p.sum() - 1.0) <= 1e-13
        assert p.shape[0] == L[r] + case.T
        assert np.all(p >= 0)


# ---------------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("qk", [False, True])
def test_empty_context_single_token_returns_v(qk):
    # P5: one key, weight one -> the output is the block's own v (never normalised)
    case = ds.make_case(3, 1, 24, 4, [0, 0, 0], seed=9, stride=0, qknorm=qk)
    out = _oracle(case)
    qkv = case.np_args()["qkv"]
    for h in range(24):
        g = h // 6
        np.testing.assert_array_equal(out[:, h * 64:(h + 1) * 64], qkv[:, (24 + 4 + g) * 64:(24 + 4 + g + 1) * 64])


@pytest.mark.parametrize("qk", [False, True])
def test_zero_query_gives_uniform_mean(qk):
    # P6: q = 0 -> all scores 0 -> plain mean of the L + T values (rms(0)=0, rope(0)=0)
    case = ds.make_case(2, 3, 6, 1, [100, 5], seed=21, qknorm=qk)
    case.qkv[:, :6 * 64] = 0
    a = case.np_args()
    out = _oracle(case)
    for r in range(2):
        L = int(a["context_lens"][r])
        kc, vc = oracle.gather_context(a["k_pool"], a["v_pool"], a["page_table"][r], L, 0)
        vals = np.concatenate([vc, a["qkv"][r * 3:(r + 1) * 3, 7 * 64:8 * 64]])
        mean = vals.sum(0) / (L + 3)
        for t in range(3):
            for h in range(6):
                np.testing.assert_allclose(out[r * 3 + t, h * 64:(h + 1) * 64], mean, rtol=0, atol=1e-14)


def test_gathered_context_matches_direct_indexing():
    case = ds.make_config(2)
    a = case.np_args()
    for r in range(8):
        L = int(a["context_lens"][r])
        kc, vc = oracle.gather_context(a["k_pool"], a["v_pool"], a["page_table"][r], L, 0)
        for c in [0, L // 2, L - 1] if L else []:
            p = a["page_table"][r][c // 64]
            np.testing.assert_array_equal(kc[c], a["k_pool"][p, 0, c % 64])
            np.testing.assert_array_equal(vc[c], a["v_pool"][p, 0, c % 64])


@pytest.mark.parametrize("qk", [False, True])
def test_constant_v_gives_constant(qk):
    # P7: every value row equal to c -> output c whatever the keys are
    case = ds.make_case(2, 4, 12, 2, [130, 64], seed=4, qknorm=qk, pool_pages=4)
    c = torch.linspace(-2, 2, 64).to(torch.bfloat16)
    case.qkv[:, (12 + 2) * 64:] = c.repeat(2)
    case.pool[:, 1] = c
    out = _oracle(case)
    for h in range(12):
        np.testing.assert_allclose(out[:, h * 64:(h + 1) * 64], np.tile(c.double().numpy(), (8, 1)),
                                   rtol=0, atol=1e-13)


@pytest.mark.parametrize("where", ["first", "last_page", "tail_slot", "block"])
def test_needle(where):
    # P8: one key aligned with q and scaled up, its value e_m -> the output is e_m
    R, T = 2, 2
    case = ds.make_case(R, T, 6, 1, [200, 130], seed=31, pool_pages=8)
    a = case.np_args()
    r, t, h, m = 1, 1, 3, 17
    L = 130
    j = {"first": 0, "last_page": 64 + 5, "tail_slot": L - 1, "block": L + 1}[where]
    q = np.zeros(64)
    q[5] = 1.0
    case.qkv[r * T + t, h * 64:(h + 1) * 64] = torch.from_numpy(q).to(torch.bfloat16)
    e = torch.zeros(64)
    e[m] = 1.0
    if j < L:
        p = int(a["page_table"][r][j // 64])
        case.k_pool[p, 0, j % 64] = torch.from_numpy(2000.0 * q).to(torch.bfloat16)
        case.v_pool[p, 0, j % 64] = e.to(torch.bfloat16)
    else:
        row = r * T + (j - L)
        case.qkv[row, 6 * 64:7 * 64] = torch.from_numpy(2000.0 * q).to(torch.bfloat16)
        case.qkv[row, 7 * 64:8 * 64] = e.to(torch.bfloat16)
    out = _oracle(case)
    np.testing.assert_allclose(out[r * T + t, h * 64:(h + 1) * 64], e.double().numpy(), atol=1e-12)


def test_rmsnorm_closed_forms():
    w = np.linspace(0.5, 1.5, 64)
    for c in (1e-3, 0.5, 3.0, -7.0):
        x = np.full(64, c)
        np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-5), w * c / math.sqrt(c * c + 1e-5), rtol=1e-15)
    # scale invariance for |alpha x| >> sqrt(eps)
    x = np.random.default_rng(0).standard_normal(64)
    np.testing.assert_allclose(oracle.rms_norm(1e3 * x, w, 1e-5), oracle.rms_norm(x, w, 1e-5), rtol=1e-5)
    # unit weight and unit-mean-square input -> unchanged up to eps
    y = np.sign(x)
    np.testing.assert_allclose(oracle.rms_norm(y, np.ones(64), 0.0), y, rtol=1e-15)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    # pos 0 is the identity
    np.testing.assert_array_equal(oracle.rope_neox(x, np.zeros(5), 10000.0), x)
    # e_i at position p lands on (cos, sin) of p * f_i in dims (i, i+32); exact decimal
    # frequencies at i = 0, 8, 16, 24: 10000**(-2i/64) = 1, 0.1, 0.01, 0.001
    for i, f in [(0, 1.0), (8, 0.1), (16, 0.01), (24, 0.001)]:
        for p in (1, 7, 2041, 32775):
            e = np.zeros(64)
            e[i] = 1.0
            y = oracle.rope_neox(e, np.array(p), 10000.0)
            assert abs(y[i] - math.cos(p * f)) < 1e-12 and abs(y[i + 32] - math.sin(p * f)) < 1e-12
            assert np.count_nonzero(np.abs(y) > 1e-15) <= 2
            e2 = np.zeros(64)
            e2[i + 32] = 1.0
            y2 = oracle.rope_neox(e2, np.array(p), 10000.0)
            assert abs(y2[i] + math.sin(p * f)) < 1e-12 and abs(y2[i + 32] - math.cos(p * f)) < 1e-12
    # each (i, i+32) pair keeps its length
    y = oracle.rope_neox(x, np.arange(5) * 977, 10000.0)
    np.testing.assert_allclose(np.hypot(y[:, :32], y[:, 32:]), np.hypot(x[:, :32], x[:, 32:]), rtol=1e-13)


# ---- YaRN ("YaRN 4.0" of the drafter checkpoint; the method as published).  The pins use
# special cases with closed forms: factor 1 is plain RoPE; an original context so short that no
# pair turns once is position interpolation (every frequency / s); one so long that every pair
# turns more than beta times keeps every frequency; factors e and e^10 give the temperature
# factors 1.1 and 2.0 exactly; and a chosen context puts one pair at the middle of the ramp.

def _xp():
    rng = np.random.default_rng(21)
    return rng.standard_normal((6, 64)), np.array([0, 4, 8, 401, 2044, 40000])


def test_yarn_factor_one_is_plain_rope():
    x, pos = _xp()
    for L in (1, 64, 4096, 10 ** 9):
        a = oracle.rope_neox(x, pos, 1e4, dict(factor=1.0, original_max_position=L))
        # (1 - g) * f + g * f rounds within an ulp of f: angles near 4e4 agree to ~1e-11
        np.testing.assert_allclose(a, oracle.rope_neox(x, pos, 1e4), rtol=0, atol=1e-10)


def test_yarn_short_original_context_is_position_interpolation():
    x, pos = _xp()
    a = oracle.rope_neox(x, pos, 1e4, dict(factor=math.e, original_max_position=1))
    np.testing.assert_allclose(a, 1.1 * oracle.rope_neox(x, pos / math.e, 1e4), rtol=0, atol=1e-9)


def test_yarn_long_original_context_only_scales():
    x, pos = _xp()
    a = oracle.rope_neox(x, pos, 1e4, dict(factor=math.e ** 10, original_max_position=10 ** 12))
    np.testing.assert_allclose(a, 2.0 * oracle.rope_neox(x, pos, 1e4), rtol=0, atol=1e-9)


def test_yarn_ramp_midpoint_and_shape():
    i = np.arange(32)
    theta = 10.0 ** (-i / 8.0)                      # 10000**(-2i/64)
    # pair 8 (frequency 0.1) turns 16.5 times over L = 16.5 * 2 pi / 0.1: half way from 1 to 32
    f = oracle.yarn_inv_freq(1e4, 4.0, 16.5 * 2 * math.pi / 0.1, 1.0, 32.0)
    ratio = f / theta
    assert abs(ratio[8] - (0.5 / 4 + 0.5)) < 1e-12
    assert ratio[0] == 1.0 and abs(ratio[31] - 0.25) < 1e-15
    assert np.all(np.diff(ratio) <= 1e-15) and np.all((ratio >= 0.25 - 1e-15) & (ratio <= 1.0))
    # at the drafter's factor over a 4096-token original context all three regimes occur
    r4 = oracle.yarn_inv_freq(1e4, 4.0, 4096) / theta
    assert (r4 == 1.0).any() and (np.abs(r4 - 0.25) < 1e-15).any() and ((r4 > 0.26) & (r4 < 0.99)).any()


# ---- YaRN's ramp linear in the pair index (checkpoint configurations).  The bounds are pinned
# by the turn counts themselves, evaluated directly: the ramp starts at the last pair that turns
# at least beta times and ends at the first pair that turns at most alpha times; the unrounded
# bounds are the fractional pairs whose turn count is exactly beta and alpha.

YARN_INDEX_CASES = [(1e4, 4096, 1.0, 32.0), (1e4, 32768, 1.0, 32.0), (5e5, 8192, 2.0, 16.0), (1e4, 300, 0.5, 4.0)]


def _turn_counts(base, L):
    theta = float(base) ** (-np.arange(32) / 32.0)       # base**(-2i/64)
    return theta, L * theta / (2 * math.pi)


@pytest.mark.parametrize("base,L,a,b", YARN_INDEX_CASES)
def test_yarn_index_ramp_bounds_from_turn_counts(base, L, a, b):
    s = 4.0
    i = np.arange(32)
    theta, r = _turn_counts(base, L)
    assert np.min(np.abs(r - b)) > 1e-6 and np.min(np.abs(r - a)) > 1e-6   # no pair sits on a bound
    lo = int(np.nonzero(r >= b)[0].max())
    hi = int(np.nonzero(r <= a)[0].min())
    assert 0 < lo < hi < 31
    ratio = oracle.yarn_inv_freq(base, s, L, a, b, ramp="index") / theta
    np.testing.assert_allclose(ratio[:lo + 1], 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ratio[hi:], 1.0 / s, rtol=0, atol=1e-15)
    # in between: the straight line from (lo, 1) to (hi, 1/s), one step per pair
    step = (1.0 - 1.0 / s) / (hi - lo)
    np.testing.assert_allclose(ratio[lo:hi + 1], 1.0 - step * (i[lo:hi + 1] - lo), rtol=0, atol=1e-14)


@pytest.mark.parametrize("base,L,a,b", YARN_INDEX_CASES)
def test_yarn_unrounded_index_ramp(base, L, a, b):
    s = 8.0
    theta, r = _turn_counts(base, L)
    lo, hi = oracle.yarn_pair_at_turns(base, L, b), oracle.yarn_pair_at_turns(base, L, a)
    # the fractional pairs turn exactly beta and alpha times
    for x, want in ((lo, b), (hi, a)):
        assert abs(L * float(base) ** (-2.0 * x / 64) / (2 * math.pi) - want) < 1e-10 * want
    ratio = oracle.yarn_inv_freq(base, s, L, a, b, ramp="index_unrounded") / theta
    inside = np.nonzero((np.arange(32) > lo) & (np.arange(32) < hi))[0]
    assert len(inside) >= 3
    np.testing.assert_allclose(ratio[np.arange(32) <= lo], 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ratio[np.arange(32) >= hi], 1.0 / s, rtol=0, atol=1e-15)
    # straight inside, and its extension reaches 1 at lo and 1/s at hi
    d = np.diff(ratio[inside])
    np.testing.assert_allclose(d, d[0], rtol=0, atol=1e-14)
    assert abs(ratio[inside[0]] + d[0] * (lo - inside[0]) - 1.0) < 1e-12
    assert abs(ratio[inside[0]] + d[0] * (hi - inside[0]) - 1.0 / s) < 1e-12


def test_yarn_ramps_agree_outside_the_ramp():
    s, (base, L, a, b) = 4.0, YARN_INDEX_CASES[0]
    theta, r = _turn_counts(base, L)
    f = {k: oracle.yarn_inv_freq(base, s, L, a, b, ramp=k) / theta for k in oracle.YARN_RAMPS}
    keep, interp = r >= b, r <= a
    for k in oracle.YARN_RAMPS:
        np.testing.assert_allclose(f[k][keep], 1.0, rtol=0, atol=1e-15)
        np.testing.assert_allclose(f[k][interp], 1.0 / s, rtol=0, atol=1e-15)
    mid = ~(keep | interp)
    assert np.abs(f["turns"][mid] - f["index"][mid]).max() > 0.05      # different shapes in between


def test_yarn_index_ramp_degenerate_bounds():
    s = 4.0
    theta = 1e4 ** (-np.arange(32) / 32.0)
    for ramp in ("index", "index_unrounded"):
        # every pair turns more than beta times: nothing is scaled (as with the ramp in turns)
        f = oracle.yarn_inv_freq(1e4, s, 10 ** 7, 1.0, 32.0, ramp=ramp)
        np.testing.assert_allclose(f / theta, 1.0, rtol=0, atol=1e-15)
        # no pair turns even alpha times: both bounds clamp to pair 0, which keeps its frequency
        f = oracle.yarn_inv_freq(1e4, s, 1, 1.0, 32.0, ramp=ramp)
        assert f[0] == theta[0]
        np.testing.assert_allclose(f[1:] / theta[1:], 1.0 / s, rtol=0, atol=1e-15)
    with pytest.raises(oracle.OracleContractError):
        oracle.yarn_inv_freq(1e4, s, 4096, ramp="dims")
    # with base <= 1 the frequencies do not fall along the pairs: no index ramp
    for base in (1.0, 0.5):
        with pytest.raises(oracle.OracleContractError):
            oracle.yarn_inv_freq(base, s, 4096, ramp="index")


def test_yarn_index_ramp_factor_one_and_explicit_mscale():
    x, pos = _xp()
    plain = oracle.rope_neox(x, pos, 1e4)
    for ramp in oracle.YARN_RAMPS:
        a = oracle.rope_neox(x, pos, 1e4, dict(factor=1.0, original_max_position=4096, ramp=ramp))
        np.testing.assert_allclose(a, plain, rtol=0, atol=1e-10)
        # an explicit factor on q and k replaces the temperature 0.1 ln s + 1 (here e: 1.1)
        y = dict(factor=math.e, original_max_position=4096, ramp=ramp)
        d = oracle.rope_neox(x, pos, 1e4, y)
        m = oracle.rope_neox(x, pos, 1e4, dict(y, mscale=0.75))
        np.testing.assert_allclose(m, d * (0.75 / 1.1), rtol=1e-13, atol=1e-15)
        # the rotation keeps each pair's length: only the factor changes it
        np.testing.assert_allclose(np.hypot(m[:, :32], m[:, 32:]), 0.75 * np.hypot(x[:, :32], x[:, 32:]),
                                   rtol=1e-12)


def test_yarn_attention_equals_explicit_steps():
    # the qknorm attention with YaRN == plain attention on q/k normalised and YaRN-rotated first
    yarn = dict(factor=4.0, original_max_position=256)
    case = ds.make_case(3, 5, 12, 2, [100, 0, 700], seed=22, qknorm=True, pos_dtype=torch.int64,
                        pos_offset=[5000, 0, 30000])
    a = case.np_args()
    fused = oracle.drafter_attn_qknorm(**a, yarn=yarn)
    q = a["qkv"].copy()
    for h in range(case.Hq):
        c = slice(h * 64, (h + 1) * 64)
        q[:, c] = oracle.rope_neox(oracle.rms_norm(q[:, c], a["q_norm_weight"], 1e-5), a["positions"], 1e4, yarn)
    for g in range(case.Hkv):
        c = slice((case.Hq + g) * 64, (case.Hq + g + 1) * 64)
        q[:, c] = oracle.rope_neox(oracle.rms_norm(q[:, c], a["k_norm_weight"], 1e-5), a["positions"], 1e4, yarn)
    b = dict(a)
    b["qkv"] = q
    np.testing.assert_allclose(oracle.drafter_attn(**b), fused, rtol=0, atol=1e-12)
    # and the temperature is really applied: without YaRN the result differs
    assert np.abs(oracle.drafter_attn_qknorm(**a) - fused).max() > 1e-3


def test_rope_relative_position_property():
    # with no context, scores depend only on position differences: shift all positions
    case = ds.make_case(2, 6, 12, 2, [0, 0], seed=8, stride=0, qknorm=True)
    a = case.np_args()
    base = oracle.drafter_attn_qknorm(**a)
    a["positions"] = a["positions"] + 12345
    np.testing.assert_allclose(oracle.drafter_attn_qknorm(**a), base, atol=1e-12)


# ---------------------------------------------------------------------------------------
# fused_qk_norm_rope (the drafter's cell) on packed rows
# ---------------------------------------------------------------------------------------

_EXACT_FREQ = [(0, 1.0), (8, 0.1), (16, 0.01), (24, 0.001)]  # 10000**(-2i/64), exact decimals


def test_qk_norm_rope_closed_forms():
    # Hkv = 2 (12 q heads, 2 k heads, 2 v heads) + 16 padding columns.  Every q/k head of a
    # row is a one-hot a*e_j: RMSNorm gives a*w_j/sqrt(a^2/64 + eps) at j, then the rotation
    # puts cos/sin of p*f (exact angles) at (j, j+32) -- or (-sin, cos) for j >= 32.  q and k
    # use different weight vectors; v heads and padding must come back unchanged.
    Hq, Hkv, eps = 12, 2, 1e-5
    wq = np.linspace(0.5, 1.5, 64)
    wk = np.linspace(1.7, 0.3, 64)
    rng = np.random.default_rng(21)
    pos = np.array([0, 1, 7, 2041, 32775])
    N = len(pos)
    qkv = rng.standard_normal((N, (Hq + 2 * Hkv) * 64 + 16))
    expect = qkv.copy()
    heads = [(h, h * 64, wq) for h in range(Hq)] + [(Hq + g, (Hq + g) * 64, wk) for g in range(Hkv)]
    for r in range(N):
        for k, (h, c0, w) in enumerate(heads):
            i, f = _EXACT_FREQ[(h + r) % 4]
            j = i + 32 * ((h + 2 * r) % 2)          # the one-hot sits in the first or second half
            a = (0.25 + 0.5 * k) * (-1.0) ** (h + r)
            qkv[r, c0:c0 + 64] = 0.0
            qkv[r, c0 + j] = a
            n = a * w[j] / math.sqrt(a * a / 64 + eps)
            expect[r, c0:c0 + 64] = 0.0
            ang = pos[r] * f
            if j < 32:
                expect[r, c0 + j], expect[r, c0 + j + 32] = n * math.cos(ang), n * math.sin(ang)
            else:
                expect[r, c0 + j - 32], expect[r, c0 + j] = -n * math.sin(ang), n * math.cos(ang)
    got = oracle.qk_norm_rope(qkv, pos, wq, wk, num_q_heads=Hq, num_kv_heads=Hkv, eps=eps)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-12)
    vcols = slice((Hq + Hkv) * 64, None)
    np.testing.assert_array_equal(got[:, vcols], qkv[:, vcols])


def test_qk_norm_rope_constant_heads_at_position_zero():
    # position 0 rotates nothing: a constant head c becomes w * c / sqrt(c^2 + eps)
    Hq, Hkv, eps = 6, 1, 1e-5
    wq, wk = np.linspace(0.5, 1.5, 64), np.linspace(1.5, 0.5, 64)
    qkv = np.zeros((3, 8 * 64))
    cs = [0.3, -2.0, 5.0, 0.01, 1.0, -0.7, 3.3]
    for r in range(3):
        for h in range(Hq + Hkv):
            qkv[r, h * 64:(h + 1) * 64] = cs[h] * (r + 1)
    qkv[:, 7 * 64:] = np.arange(64)
    got = oracle.qk_norm_rope(qkv, np.zeros(3, dtype=np.int64), wq, wk, num_q_heads=Hq, num_kv_heads=Hkv, eps=eps)
    for r in range(3):
        for h in range(Hq + Hkv):
            c = cs[h] * (r + 1)
            w = wq if h < Hq else wk
            np.testing.assert_allclose(got[r, h * 64:(h + 1) * 64], w * c / math.sqrt(c * c + eps), rtol=1e-13)
    np.testing.assert_array_equal(got[:, 7 * 64:], qkv[:, 7 * 64:])


def test_qk_norm_rope_heads_and_rows_independent():
    Hq, Hkv = 24, 4
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((6, 32 * 64))
    pos = rng.integers(0, 40000, 6)
    w1, w2 = rng.uniform(0.5, 1.5, 64), rng.uniform(0.5, 1.5, 64)
    base = oracle.qk_norm_rope(qkv, pos, w1, w2, num_q_heads=Hq, num_kv_heads=Hkv)
    for h in (0, 5, 23, 24, 27):
        x = qkv.copy()
        x[2, h * 64:(h + 1) * 64] *= -3.0
        got = oracle.qk_norm_rope(x, pos, w1, w2, num_q_heads=Hq, num_kv_heads=Hkv)
        changed = np.zeros_like(got, dtype=bool)
        changed[2, h * 64:(h + 1) * 64] = True
        np.testing.assert_array_equal(got[~changed], base[~changed])
        # RMSNorm is odd and scale-free (up to eps): the head flips sign
        np.testing.assert_allclose(got[2, h * 64:(h + 1) * 64], -base[2, h * 64:(h + 1) * 64], rtol=1e-5, atol=1e-9)


def test_attention_of_norm_roped_rows_equals_qknorm_attention():
    case = ds.make_config(2)
    a = case.np_args()
    ref = oracle.drafter_attn_qknorm(**a)
    b = dict(a)
    b["qkv"] = oracle.qk_norm_rope(a["qkv"], a["positions"], a["q_norm_weight"], a["k_norm_weight"],
                                   num_q_heads=case.Hq, num_kv_heads=case.Hkv)
    np.testing.assert_array_equal(oracle.drafter_attn(**b), ref)


def test_qk_norm_rope_rejects_out_of_contract():
    with pytest.raises(oracle.OracleContractError):
        oracle.qk_norm_rope(np.zeros((2, 512)), np.zeros(3), np.ones(64), np.ones(64), num_q_heads=6, num_kv_heads=1)
    with pytest.raises(oracle.OracleContractError):
        oracle.qk_norm_rope(np.zeros((2, 500)), np.zeros(2), np.ones(64), np.ones(64), num_q_heads=6, num_kv_heads=1)
    with pytest.raises(oracle.OracleContractError):
        oracle.qk_norm_rope(np.zeros((2, 1024)), np.zeros(2), np.ones(64), np.ones(64), num_q_heads=12, num_kv_heads=1)


# ---------------------------------------------------------------------------------------
# the replaced path: append the block to the pool, then attend to the pool only
# ---------------------------------------------------------------------------------------

def _replaced(case: ds.DrafterCase):
    """norm/rope (qknorm cases), kv_append, paged_attn over L + b keys -- all fp64."""
    a = case.np_args()
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv)
    rows = a["qkv"]
    if case.qknorm:
        rows = oracle.qk_norm_rope(rows, a["positions"], a["q_norm_weight"], a["k_norm_weight"], **kw)
    k, v = oracle.kv_append(a["k_pool"], a["v_pool"], rows, a["page_table"], a["context_lens"], a["block_lens"],
                            tokens_per_block=case.T, **kw)
    b = np.full(case.R, case.T) if a["block_lens"] is None else a["block_lens"]
    return oracle.paged_attn(rows, k, v, a["page_table"], a["context_lens"] + b, a["block_lens"],
                             tokens_per_block=case.T, scale=case.scale, **kw), (k, v)


def _append_cases():
    return [
        ds.make_case(2, 3, 12, 2, [64, 130], seed=41, qknorm=True, pool_pages=6),
        ds.make_case(3, 5, 6, 1, [0, 61, 127], seed=42, qknorm=False, pool_pages=5, stride=3),
        ds.make_case(2, 8, 24, 4, [1, 2041], seed=43, qknorm=True, pool_pages=40, block_lens=[3, 8],
                     pos_dtype=torch.int64),
    ]


@pytest.mark.parametrize("i", range(3))
def test_replaced_path_equals_fused_definition(i):
    # the fused op attends to the same keys in the same order as append + non-causal paged attention
    case = ds.with_append_room(_append_cases()[i], seed=100 + i)
    got, _ = _replaced(case)
    np.testing.assert_array_equal(got, _oracle(case))


def test_kv_append_writes_exactly_the_block_slots():
    case = ds.with_append_room(ds.make_case(3, 5, 12, 2, [0, 61, 127], seed=44, pool_pages=5, stride=3,
                                            block_lens=[5, 2, 4]), seed=7)
    a = case.np_args()
    k, v = oracle.kv_append(a["k_pool"], a["v_pool"], a["qkv"], a["page_table"], a["context_lens"],
                            a["block_lens"], num_q_heads=12, num_kv_heads=2, tokens_per_block=5)
    touched = np.zeros(k.shape[:3], dtype=bool)
    for r, (L, b) in enumerate(zip([0, 61, 127], [5, 2, 4])):
        for t in range(b):
            page = a["page_table"][r, (L + t) // 64]
            touched[page, :, (L + t) % 64] = True
            for g in range(2):
                np.testing.assert_array_equal(k[page, g, (L + t) % 64], a["qkv"][r * 5 + t, (12 + g) * 64:(13 + g) * 64])
                np.testing.assert_array_equal(v[page, g, (L + t) % 64], a["qkv"][r * 5 + t, (14 + g) * 64:(15 + g) * 64])
    np.testing.assert_array_equal(k[~touched], a["k_pool"][~touched])
    np.testing.assert_array_equal(v[~touched], a["v_pool"][~touched])
    assert touched.sum() == 2 * (5 + 2 + 4)


def test_paged_attn_closed_forms():
    case = ds.make_case(2, 4, 6, 1, [64, 5], seed=45, pool_pages=3)
    a = case.np_args()
    kw = dict(num_q_heads=6, num_kv_heads=1, tokens_per_block=4)
    # no keys: zero rows; one key: every row returns that key's value
    out0 = oracle.paged_attn(a["qkv"], a["k_pool"], a["v_pool"], a["page_table"], np.array([0, 0]), **kw)
    np.testing.assert_array_equal(out0, 0.0)
    out1 = oracle.paged_attn(a["qkv"], a["k_pool"], a["v_pool"], a["page_table"], np.array([1, 1]), **kw)
    for r in range(2):
        val = a["v_pool"][a["page_table"][r, 0], 0, 0]
        for h in range(6):
            np.testing.assert_allclose(out1[r * 4:(r + 1) * 4, h * 64:(h + 1) * 64], np.tile(val, (4, 1)), rtol=1e-15)


def test_kv_append_rejects_overflow():
    case = ds.make_case(1, 8, 6, 1, [60], seed=46, pool_pages=1)      # 60 + 8 > 64 slots
    a = case.np_args()
    with pytest.raises(oracle.OracleContractError):
        oracle.kv_append(a["k_pool"], a["v_pool"], a["qkv"], a["page_table"], a["context_lens"], None,
                         num_q_heads=6, num_kv_heads=1, tokens_per_block=8)


# ---------------------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------------------

def test_qknorm_equals_explicit_norm_rope_then_attention():
    # I7: the qknorm variant == plain attention on explicitly normalised+rotated q and k
    case = ds.make_config(3)
    a = case.np_args()
    ref = oracle.drafter_attn_qknorm(**a)
    qkv = a["qkv"].copy()
    T, Hq, Hkv = case.T, case.Hq, case.Hkv
    pos = a["positions"]
    for h in range(Hq):
        qkv[:, h * 64:(h + 1) * 64] = oracle.rope_neox(oracle.rms_norm(qkv[:, h * 64:(h + 1) * 64], a["q_norm_weight"], 1e-5), pos, 1e4)
    for g in range(Hkv):
        c = slice((Hq + g) * 64, (Hq + g + 1) * 64)
        qkv[:, c] = oracle.rope_neox(oracle.rms_norm(qkv[:, c], a["k_norm_weight"], 1e-5), pos, 1e4)
    a["qkv"] = qkv
    np.testing.assert_array_equal(oracle.drafter_attn(**a), ref)


def test_page_permutation_invariance():
    # I2: moving pages to other physical slots (and the table with them) changes nothing
    case = ds.make_config(2)
    a = case.np_args()
    ref = oracle.drafter_attn_qknorm(**a)
    P = a["k_pool"].shape[0]
    perm = np.random.default_rng(5).permutation(P)
    inv = np.argsort(perm)
    a2 = dict(a)
    a2["k_pool"] = a["k_pool"][perm]
    a2["v_pool"] = a["v_pool"][perm]
    a2["page_table"] = inv[a["page_table"]]
    np.testing.assert_array_equal(oracle.drafter_attn_qknorm(**a2), ref)


def test_request_isolation():
    # I4: another request's rows, pages and length do not move this request's output
    case = ds.make_config(3)
    a = case.np_args()
    ref = oracle.drafter_attn_qknorm(**a)
    a2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    k = 2
    a2["qkv"][k * 8:(k + 1) * 8] += 1.0
    L = int(a2["context_lens"][k])
    for p in a2["page_table"][k][: -(-L // 64)]:
        a2["k_pool"][p] *= -1
    a2["context_lens"][k] = max(0, L - 37)
    got = oracle.drafter_attn_qknorm(**a2)
    keep = np.ones(64, bool)
    keep[k * 8:(k + 1) * 8] = False
    np.testing.assert_array_equal(got[keep], ref[keep])
    assert not np.array_equal(got[~keep], ref[~keep])


def test_empty_context_attends_to_own_block_only():
    # I3: L = 0 -> softmax over the block's own keys only
    case = ds.make_case(2, 5, 6, 1, [0, 0], seed=12, stride=2, pool_pages=3)
    a = case.np_args()
    out = oracle.drafter_attn(**a)
    qkv = a["qkv"]
    for r in range(2):
        rows = qkv[r * 5:(r + 1) * 5]
        q = torch.from_numpy(rows[:, :6 * 64].reshape(5, 6, 64).transpose(1, 0, 2).copy())
        k = torch.from_numpy(rows[:, 6 * 64:7 * 64].copy()).expand(6, 5, 64)
        v = torch.from_numpy(rows[:, 7 * 64:8 * 64].copy()).expand(6, 5, 64)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.125)
        np.testing.assert_allclose(out[r * 5:(r + 1) * 5], o.transpose(0, 1).reshape(5, 384).numpy(), atol=1e-13)


def test_poison_does_not_change_result():
    # I6: NaN in unreferenced pages / tail slots / row padding and garbage table entries
    clean = ds.make_config(2)
    dirty = ds.make_config(2, poison=True)
    np.testing.assert_array_equal(_oracle(dirty), _oracle(clean))
    assert not np.isnan(_oracle(dirty)).any()


def test_oracle_rejects_out_of_contract():
    case = ds.make_config(2)
    a = case.np_args()
    bad = dict(a)
    bad["context_lens"] = a["context_lens"].copy()
    bad["context_lens"][0] = 32 * 64 + 1
    with pytest.raises(oracle.OracleContractError):
        oracle.drafter_attn_qknorm(**bad)
    bad = dict(a)
    bad["page_table"] = a["page_table"].copy()
    r = int(np.argmax(a["context_lens"]))
    bad["page_table"][r, 0] = 10_000
    with pytest.raises(oracle.OracleContractError):
        oracle.drafter_attn_qknorm(**bad)
    with pytest.raises(oracle.OracleContractError):
        oracle.drafter_attn(**dict(a, num_q_heads=12))
