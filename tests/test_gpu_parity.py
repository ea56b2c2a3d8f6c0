"""GPU parity of the HIP path against the fp64 oracle, and its bitwise invariants.

Every call goes through the C ABI (ctypes binding).  Tolerance (per element):
|gpu - oracle| <= 2e-2 + 2e-2*|oracle|, mean |err| <= 2e-3, no NaN.  The
invariants the method fixes exactly (page placement, request isolation,
reruns, poison, untouched inputs, the single-key case) are checked bit for bit.
"""
import hashlib

import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
from tests.gpu_util import check, reference, run, say, to_np

pytestmark = pytest.mark.gpu


def _digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_config_parity(n):
    case = ds.make_config(n)
    say(f"config {n}: R={case.R} T={case.T} Hq/Hkv={case.Hq}/{case.Hkv} stride={case.stride}")
    got = to_np(run(case))
    torch.cuda.synchronize()
    check(got, reference(case), f"cfg{n}")


@pytest.mark.parametrize("n", [1, 2, 3])
def test_config_parity_poisoned(n):
    # NaN in every pool element / row padding the definition never reads, garbage table entries
    case = ds.make_config(n, poison=True)
    clean = ds.make_config(n)
    say(f"config {n} poisoned")
    got = run(case)
    ref_bits = run(clean)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_bits), "poison changed the output bits"
    check(to_np(got), reference(clean), f"cfg{n}-poison")


def test_value_mean_one_diagnostic():
    # V ~ N(1, 1): outputs are about 1, so relative errors are visible
    case = ds.make_case(8, 8, 24, 4, [2041, 0, 1, 64, 65, 1000, 1500, 33], seed=55, qknorm=True,
                        v_mean=1.0, pos_dtype=torch.int64, stride=40, pool_pages=300)
    say("v-mean-1 diagnostic")
    rel2 = check(to_np(run(case)), reference(case), "vmean1")
    assert rel2 < 5e-3


def test_long_context_vmean1():
    case = ds.make_case(2, 8, 24, 4, [32768, 20000], seed=56, qknorm=True, v_mean=1.0, pool_pages=900)
    say("long context v-mean-1")
    rel2 = check(to_np(run(case)), reference(case), "long-vmean1")
    assert rel2 < 5e-3


def test_reruns_bit_identical():
    case = ds.make_config(3)
    g = ds.to_device(case, "cuda")
    say("reruns")
    first = run(case, g).clone()
    for _ in range(20):
        assert torch.equal(run(case, g), first)


def test_page_permutation_bitwise():
    # I2: the same logical context at other physical pages gives the same bits
    case = ds.make_config(3)
    say("page permutation")
    base = run(case).clone()
    P = case.num_pages
    perm = torch.from_numpy(np.random.default_rng(3).permutation(P))
    inv = torch.argsort(perm)
    moved = ds.make_config(3)
    moved.pool = case.pool[perm].contiguous()
    moved.k_pool, moved.v_pool = moved.pool[:, 0], moved.pool[:, 1]
    moved.page_table = inv[case.page_table.long()].to(torch.int32)
    assert torch.equal(run(moved), base)


def test_request_isolation_bitwise():
    # I4: rewriting one request's rows, pages and length leaves the others' bits alone
    case = ds.make_config(2)
    say("request isolation")
    base = run(case).clone()
    k = int(np.argmax(case.context_lens.numpy()))
    other = ds.make_config(2)
    other.qkv[k * 8:(k + 1) * 8] = torch.randn(8, other.qkv.shape[1]).to(torch.bfloat16)
    L = int(other.context_lens[k])
    for pg in other.page_table[k, : -(-L // 64)].tolist():
        other.pool[pg] = -other.pool[pg]
    other.context_lens[k] = L // 3
    other.positions[k * 8:(k + 1) * 8] += 1000
    got = run(other)
    keep = torch.ones(64, dtype=torch.bool)
    keep[k * 8:(k + 1) * 8] = False
    assert torch.equal(got[keep.cuda()], base[keep.cuda()])
    assert not torch.equal(got[~keep.cuda()], base[~keep.cuda()])


def test_inputs_untouched():
    # I5: pool, qkv and page table are bit-identical after the call
    case = ds.make_config(3)
    g = ds.to_device(case, "cuda")
    before = [_digest(g.pool), _digest(g.qkv), _digest(g.page_table), _digest(g.context_lens), _digest(g.positions)]
    say("inputs untouched")
    run(case, g)
    torch.cuda.synchronize()
    after = [_digest(g.pool), _digest(g.qkv), _digest(g.page_table), _digest(g.context_lens), _digest(g.positions)]
    assert before == after


@pytest.mark.parametrize("qk", [False, True])
def test_single_key_returns_v_exactly(qk):
    # P5: L = 0, T = 1 -> one key with weight 1 -> out == v bit for bit (v is never normalised)
    case = ds.make_case(8, 1, 24, 4, [0] * 8, seed=19, stride=0, qknorm=qk)
    say(f"single key qk={qk}")
    out = run(case).cpu()
    for h in range(24):
        g = h // 6
        assert torch.equal(out[:, h * 64:(h + 1) * 64], case.qkv[:, (28 + g) * 64:(29 + g) * 64])


def test_qknorm_equals_cpu_norm_rope_then_plain():
    # I7 on the GPU: the fused prologue vs the plain kernel on q/k normalised+rotated on the CPU
    case = ds.make_config(3)
    a = case.np_args()
    qkv = a["qkv"].copy()
    pos = a["positions"]
    for h in range(case.Hq):
        c = slice(h * 64, (h + 1) * 64)
        qkv[:, c] = oracle.rope_neox(oracle.rms_norm(qkv[:, c], a["q_norm_weight"], 1e-5), pos, 1e4)
    for g in range(case.Hkv):
        c = slice((case.Hq + g) * 64, (case.Hq + g + 1) * 64)
        qkv[:, c] = oracle.rope_neox(oracle.rms_norm(qkv[:, c], a["k_norm_weight"], 1e-5), pos, 1e4)
    plain = ds.make_config(3)
    plain.qkv = torch.from_numpy(qkv).to(torch.bfloat16)
    plain.qknorm = False
    say("qknorm vs cpu-prepared plain")
    fused = to_np(run(case))
    unfused = to_np(run(plain))
    err = np.abs(fused - unfused)
    assert err.max() <= 2e-2 and err.mean() <= 1e-3


def test_qknorm_int64_positions_beyond_int32():
    # positions past the int32 range (up to 2^33 + L): the kernel forms and reduces the angle in fp64
    case = ds.make_case(3, 8, 24, 4, [100, 700, 64], seed=96, qknorm=True, pos_dtype=torch.int64,
                        pos_offset=[3_000_000_000, 1 << 33, 2 ** 31 + 5])
    say("qknorm, int64 positions beyond 2^31")
    check(to_np(run(case)), reference(case), "pos>2^31")


def test_block_lens_and_layout_variants():
    # ragged blocks, separate pools, padded qkv rows (NaN padding), out with a wider row stride
    case = ds.make_case(5, 7, 24, 4, [0, 1, 64, 1999, 130], seed=23, block_lens=[7, 1, 3, 5, 2], qknorm=True,
                        separate_pools=True, qkv_row_pad=40, stride=37, pool_pages=64, pos_dtype=torch.int64,
                        poison=True)
    say("block lens / layout variants")
    out = torch.full((35, 24 * 64 + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    run(case, out=out[:, :24 * 64 + 64])
    got = out.float().cpu().numpy().astype(np.float64)
    ref = reference(case)
    check(got[:, :24 * 64], ref, "variants")
    assert np.all(got[:, 24 * 64:] == 7.0), "wrote past the output row"
    bl = [7, 1, 3, 5, 2]
    for r in range(5):
        assert np.all(got[r * 7 + bl[r]:(r + 1) * 7, :24 * 64] == 0.0)


@pytest.mark.parametrize("R,T,hkv,lens", [
    (1, 1, 1, [0]), (1, 8, 1, [1]), (2, 3, 4, [63, 64]), (3, 5, 1, [65, 127, 128]),
    (8, 8, 4, [2041] * 8), (8, 2, 1, [0] * 8), (4, 8, 2, [4096, 0, 3000, 17]),
])
def test_edge_shapes(R, T, hkv, lens):
    case = ds.make_case(R, T, 6 * hkv, hkv, lens, seed=sum(lens) + R * 31 + T, qknorm=True, pool_pages=None)
    say(f"edge R={R} T={T} Hkv={hkv} L={lens}")
    check(to_np(run(case)), reference(case), f"edge-{R}-{T}-{hkv}")


def test_max_context_many_splits():
    # a page-table stride long enough to hit the split cap, mixed with an empty request
    case = ds.make_case(2, 4, 6, 1, [131072, 0], seed=77, qknorm=True, pool_pages=2100)
    say("max context / split cap")
    check(to_np(run(case)), reference(case), "maxctx")


def test_large_stride_caps_pages_per_split():
    # 8 x 4 heads with a 4096-page row stride: the plan caps a split at 512 pages
    # (64 per wave); one request uses the whole row, the others are short
    lens = [4096 * 64, 3, 0, 700, 64, 65, 1, 2041]
    case = ds.make_case(8, 8, 24, 4, lens, seed=91, stride=4096, qknorm=True, pos_dtype=torch.int64)
    say("large stride")
    check(to_np(run(case)), reference(case), "stride4096")


def test_contract_maximum_context():
    # the longest row the contract allows: 16384 pages = 1,048,576 tokens (64 splits of 256
    # pages, 32 per wave), next to an empty request
    case = ds.make_case(2, 8, 6, 1, [16384 * 64, 0], seed=93, stride=16384, qknorm=True,
                        pos_dtype=torch.int64)
    say("contract maximum context (1M tokens)")
    check(to_np(run(case)), reference(case), "ctx1M")


def test_widest_head_layout_long_contexts():
    # 8 requests x 8 tokens with 96 query / 16 KV heads and 16k-token contexts
    case = ds.make_case(8, 8, 96, 16, [16384] * 7 + [16383], seed=94, qknorm=True)
    say("96/16 heads, 16k contexts")
    check(to_np(run(case)), reference(case), "h96x16")


def test_widest_layout_at_the_longest_row():
    # 96/16 heads with a 1,048,576-token context: the largest pages per split (512, 64 per
    # wave), 32 splits x 16 KV heads = 512 workgroups (two per CU in turn) and 512 partial
    # slots.  The 4.3 GB pool is drawn on the device; KV groups 0, 7 and 15 (their 6 query
    # heads each) are checked against fp64 one by one.
    pages = 16384
    pool = ds.device_normal_pool(pages + 3, 16, seed=99, device="cuda")
    case = ds.make_case(1, 8, 96, 16, [pages * 64], seed=99, stride=pages, pool_pages=pages + 3, qknorm=True,
                        pos_dtype=torch.int64, pool_override=pool)
    g = ds.to_device(case, "cuda")
    say("96/16 heads, 1M-token context")
    out = to_np(run(case, g))
    pt = case.page_table.numpy().astype(np.int64)
    cl = case.context_lens.numpy().astype(np.int64)
    for grp in (0, 7, 15):
        cols = (list(range(6 * grp * 64, 6 * (grp + 1) * 64)) + list(range((96 + grp) * 64, (97 + grp) * 64)) +
                list(range((112 + grp) * 64, (113 + grp) * 64)))
        ref = oracle.drafter_attn_qknorm(
            case.qkv[:, cols].double().numpy(), g.k_pool[:, grp:grp + 1].double().cpu().numpy(),
            g.v_pool[:, grp:grp + 1].double().cpu().numpy(), pt, cl, positions=case.positions.numpy(),
            q_norm_weight=case.q_norm_weight.double().numpy(), k_norm_weight=case.k_norm_weight.double().numpy(),
            num_q_heads=6, num_kv_heads=1, tokens_per_block=8, scale=case.scale)
        check(out[:, 6 * grp * 64:6 * (grp + 1) * 64], ref, f"h96x16-1M-group{grp}")


def test_every_dimension_at_its_maximum():
    # 8 requests x 8 tokens x 96/16 heads, every context 1,048,576 tokens: 4096 workgroups (16 per
    # CU in turn), a 34 GB pool drawn on the device.  Sampled (request, KV group) pairs are checked
    # against fp64 one by one, each on its own request's pages gathered into a small pool.
    pages = 16384
    pool = ds.device_normal_pool(8 * pages, 16, seed=100, device="cuda")
    case = ds.make_case(8, 8, 96, 16, [pages * 64] * 8, seed=100, stride=pages, pool_pages=8 * pages, qknorm=True,
                        pos_dtype=torch.int64, pool_override=pool)
    g = ds.to_device(case, "cuda")
    say("8 x 8 x 96/16, 1M-token contexts")
    out = to_np(run(case, g))
    for r, grp in ((0, 0), (3, 9), (7, 15)):
        rows = slice(8 * r, 8 * (r + 1))
        cols = (list(range(6 * grp * 64, 6 * (grp + 1) * 64)) + list(range((96 + grp) * 64, (97 + grp) * 64)) +
                list(range((112 + grp) * 64, (113 + grp) * 64)))
        ids = g.page_table[r].long()
        kp = g.k_pool[ids, grp:grp + 1].double().cpu().numpy()
        vp = g.v_pool[ids, grp:grp + 1].double().cpu().numpy()
        ref = oracle.drafter_attn_qknorm(
            case.qkv[rows][:, cols].double().numpy(), kp, vp, np.arange(pages, dtype=np.int64)[None, :],
            np.array([pages * 64]), positions=case.positions[rows].numpy(),
            q_norm_weight=case.q_norm_weight.double().numpy(), k_norm_weight=case.k_norm_weight.double().numpy(),
            num_q_heads=6, num_kv_heads=1, tokens_per_block=8, scale=case.scale)
        check(out[rows, 6 * grp * 64:6 * (grp + 1) * 64], ref, f"max-all-r{r}-group{grp}")


def test_pages_beyond_2_31_elements_of_pool():
    # with 96/16 heads a page is 128 KiB per pool: ids near 40,000 put a page 5.2 GB (2.6e9
    # elements) into each pool, past any 32-bit element or byte offset; every other page is NaN
    case = ds.make_case(2, 8, 96, 16, [300, 129], seed=95, qknorm=True, pool_pages=8)
    g = ds.to_device(case, "cuda")
    P = 40000
    big_k = torch.full((P, 16, 64, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    big_v = torch.full_like(big_k, float("nan"))
    pt = g.page_table.clone()
    k = 0
    for r, L in enumerate(case.context_lens.tolist()):
        for j in range(-(-L // 64)):
            old, new = int(case.page_table[r, j]), P - 1 - 3 * k
            big_k[new].copy_(g.k_pool[old])
            big_v[new].copy_(g.v_pool[old])
            pt[r, j] = new
            k += 1
    g.k_pool, g.v_pool, g.page_table = big_k, big_v, pt
    say(f"pages up to id {P - 1} ({(P - 1) * 16 * 4096 * 2 / 1e9:.1f} GB into each pool)")
    out = run(case, g)
    del big_k, big_v
    check(to_np(out), reference(case), "pool-beyond-2^31")


@pytest.mark.parametrize("scale", [2.0, 4.0, 1e-4])
def test_sharp_and_flat_softmax(scale):
    # scale 2-4 (16-32x the usual): the softmax is close to one-hot and the running maximum
    # jumps by more than the lazy-rescale headroom page after page; 1e-4: nearly uniform.
    # Plain path only: q and k are exact bf16 inputs there.  (With qknorm the bf16 rounding of
    # the normalised q/k that the contractions need moves a near one-hot softmax by more than
    # the bar at such scales -- 773 elements out at scale 4, 28 at scale 1, in fp64 alone.)
    case = ds.make_case(3, 8, 24, 4, [2041, 700, 5000], seed=97, scale=scale)
    say(f"softmax scale {scale}")
    check(to_np(run(case)), reference(case), f"scale{scale}")


def test_rising_scores_force_rescales():
    # keys grow along the context (x1 .. x16), so page after page holds a larger maximum: every
    # wave's reference maximum moves many times (the rescale path), against fp64
    case = ds.make_case(2, 8, 12, 2, [4096, 1500], seed=98, scale=0.5)
    ramp = torch.ones(case.k_pool.shape[0], 1, 1, 1)
    for r, L in enumerate(case.context_lens.tolist()):
        for j in range(-(-L // 64)):
            ramp[int(case.page_table[r, j])] = 1.0 + 15.0 * j / max(1, -(-L // 64) - 1)
    case.k_pool.copy_((case.k_pool.float() * ramp).to(torch.bfloat16))   # a view into the fused pool
    say("rising scores")
    check(to_np(run(case)), reference(case), "rising")


def test_status_flags_and_clamping():
    # device-value contract breaks are clamped (no out-of-range reads) and reported
    case = ds.make_case(2, 2, 6, 1, [100, 50], seed=5, stride=2, pool_pages=4)
    g = ds.to_device(case, "cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("status flags")
    run(case, g, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    g.context_lens[0] = 10_000          # > stride * 64
    g.page_table[1, 0] = 1_000_000      # page id out of range
    run(case, g, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1 and int(status.item()) & 2
    bl = torch.tensor([0, 9], dtype=torch.int32, device="cuda")
    status.zero_()
    run(case, g, status=status, block_lens=bl)
    torch.cuda.synchronize()
    assert int(status.item()) & 4


def test_out_of_contract_raises():
    from speculative_decoding_drafter_amd import DrafterAttnError

    case = ds.make_config(2)
    g = ds.to_device(case, "cuda")
    say("out of contract")
    with pytest.raises(DrafterAttnError):
        run(case, g, num_q_heads=12)
    with pytest.raises(DrafterAttnError):
        run(case, g, scale=-1.0)
    with pytest.raises(DrafterAttnError):
        run(case, g, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(DrafterAttnError):   # out aliasing qkv
        run(case, g, out=g.qkv[:, :384])
    with pytest.raises(DrafterAttnError):
        run(case, g, eps=float("nan"))


@pytest.mark.parametrize("low_word", [0x80000000, 0xFFFF0000])
def test_pool_at_high_addresses(low_word):
    # Regression: page base addresses are moved to SGPRs 32 bits at a time; a signed
    # widening of the low half once smeared bit 31 into the high half.  Place the
    # pool where the low word has bit 31 set (and where pages straddle a 4 GiB line).
    case = ds.make_config(2)
    pool = case.pool
    nbytes = pool.numel() * pool.element_size()
    buf = torch.empty(nbytes + (1 << 33), dtype=torch.uint8, device="cuda")
    base = buf.data_ptr()
    off = (low_word - (base & 0xFFFFFFFF)) % (1 << 32)
    off -= off % 4096
    assert off + nbytes <= buf.numel()
    view = buf[off:off + nbytes].view(torch.bfloat16).view(pool.shape)
    view.copy_(pool.to("cuda"))
    say(f"pool at 0x{view.data_ptr():x}")
    assert (view.data_ptr() & 0x80000000) != 0
    g = ds.to_device(case, "cuda")
    g.pool = view
    g.k_pool, g.v_pool = view[:, 0], view[:, 1]
    check(to_np(run(case, g)), reference(case), f"highaddr-{low_word:x}")
