"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side checks reject out-of-contract calls before touching a device.

No call here reaches a kernel launch: every call is either a pure host query
(workspace size, split plan) or fails validation first.
"""
import ctypes
import json
import os
import re

import pytest

from speculative_decoding_drafter_amd import _lib
from speculative_decoding_drafter_amd.build import INCLUDE

HEADER = os.path.join(INCLUDE, "drafter_attn.h")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "contract_facts.json")

DA_OK, DA_EINVAL, DA_EUNSUPPORTED, DA_EWORKSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(drafter_\w*)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    assert _declared() == sorted(["drafter_attn", "drafter_attn_qknorm", "drafter_attn_workspace_bytes",
                                  "drafter_attn_plan", "drafter_attn_last_error", "drafter_qk_norm_rope",
                                  "drafter_kv_append", "drafter_paged_attn", "drafter_attn_qknorm_yarn",
                                  "drafter_qk_norm_rope_yarn", "drafter_attn_qknorm_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES)


def test_header_constants_match_the_pages():
    facts = json.load(open(GOLDEN))
    text = open(HEADER).read()
    val = lambda n: int(re.search(rf"#define {n} (\d+)", text).group(1))
    assert val("DA_MAX_REQUESTS") == facts["max_requests"]
    assert val("DA_MAX_TOKENS") == facts["max_tokens_per_block"]
    assert val("DA_HEAD_DIM") == facts["head_dim"]
    assert val("DA_PAGE_SIZE") == facts["page_size"]
    assert val("DA_GQA") == facts["q_heads_per_kv_head"]


def test_workspace_bytes(lib):
    f = lib.drafter_attn_workspace_bytes
    for R, T, hkv, stride in [(1, 8, 1, 1), (8, 8, 1, 32), (8, 8, 4, 40), (8, 8, 4, 512), (3, 2, 4, 0)]:
        n = f(R, T, 6 * hkv, hkv, 64, stride)
        s, p = ctypes.c_int32(), ctypes.c_int32()
        assert lib.drafter_attn_plan(R, hkv, stride, ctypes.byref(s), ctypes.byref(p)) == DA_OK
        assert n >= R * hkv * s.value * 48 * 66 * 4
        assert n % 256 == 0
    assert f(9, 8, 6, 1, 64, 4) == 0      # too many requests
    assert f(1, 9, 6, 1, 64, 4) == 0      # too many tokens
    assert f(1, 8, 12, 1, 64, 4) == 0     # GQA ratio
    assert f(1, 8, 6, 1, 128, 4) == 0     # head_dim
    assert f(1, 8, 6, 1, 64, -1) == 0


def test_plan_covers_the_row_and_is_data_independent(lib):
    for R in range(1, 9):
        for hkv in (1, 4):
            for stride in (0, 1, 3, 32, 40, 512, 2048, 4096):
                s, p = ctypes.c_int32(), ctypes.c_int32()
                assert lib.drafter_attn_plan(R, hkv, stride, ctypes.byref(s), ctypes.byref(p)) == DA_OK
                assert 1 <= s.value <= 64 and p.value >= 1
                assert s.value * p.value >= stride
                assert (s.value - 1) * p.value < max(stride, 1)   # no split is entirely past the row
    assert lib.drafter_attn_plan(0, 1, 4, None, None) == DA_EINVAL
    assert lib.drafter_attn_plan(1, 1, 16385, None, None) == DA_EINVAL


def test_plan_keeps_a_waves_page_ids_in_one_register(lib):
    # a wave owns every 8th page of its split: at most 64 of them (one id per lane)
    for R in (1, 2, 8):
        for hkv in (1, 2, 4, 8, 16):
            for stride in (1, 7, 64, 511, 512, 2048, 4096, 8191, 16384):
                s, p = ctypes.c_int32(), ctypes.c_int32()
                assert lib.drafter_attn_plan(R, hkv, stride, ctypes.byref(s), ctypes.byref(p)) == DA_OK
                assert -(-p.value // 8) <= 64, (R, hkv, stride, s.value, p.value)
                assert s.value <= 64 and s.value * p.value >= stride


def _call(lib, **over):
    """A drafter_attn call with fake (never dereferenced) pointers; every case must fail validation."""
    a = dict(qkv=0x10000, qkv_row_stride=512, k_pool=0x200000, v_pool=0x200000 + 8192, pool_page_stride=16384,
             num_pages=4, page_table=0x900000, page_table_stride=1, context_lens=0x900100, block_lens=None,
             R=1, T=8, Hq=6, Hkv=1, head_dim=64, page_size=64, scale=0.125, workspace=0xA00000,
             workspace_bytes=1 << 20, out=0xB00000, out_row_stride=384, status=None, stream=None)
    a.update(over)
    return lib.drafter_attn(a["qkv"], a["qkv_row_stride"], a["k_pool"], a["v_pool"], a["pool_page_stride"],
                            a["num_pages"], a["page_table"], a["page_table_stride"], a["context_lens"],
                            a["block_lens"], a["R"], a["T"], a["Hq"], a["Hkv"], a["head_dim"], a["page_size"],
                            a["scale"], a["workspace"], a["workspace_bytes"], a["out"], a["out_row_stride"],
                            a["status"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=128), DA_EUNSUPPORTED),
    (dict(page_size=32), DA_EUNSUPPORTED),
    (dict(Hq=12), DA_EUNSUPPORTED),
    (dict(R=9), DA_EINVAL),
    (dict(R=0), DA_EINVAL),
    (dict(T=9), DA_EINVAL),
    (dict(T=0), DA_EINVAL),
    (dict(Hkv=0, Hq=0), DA_EINVAL),
    (dict(Hkv=17, Hq=102), DA_EINVAL),
    (dict(page_table_stride=-1), DA_EINVAL),
    (dict(qkv=None), DA_EINVAL),
    (dict(out=None), DA_EINVAL),
    (dict(context_lens=None), DA_EINVAL),
    (dict(page_table=None), DA_EINVAL),
    (dict(k_pool=None), DA_EINVAL),
    (dict(num_pages=0), DA_EINVAL),
    (dict(pool_page_stride=4095), DA_EINVAL),
    (dict(pool_page_stride=4100), DA_EINVAL),
    (dict(qkv_row_stride=500), DA_EINVAL),
    (dict(qkv_row_stride=516), DA_EINVAL),
    (dict(out_row_stride=380), DA_EINVAL),
    (dict(qkv=0x10008), DA_EINVAL),        # misaligned
    (dict(out=0xB00004), DA_EINVAL),
    (dict(scale=0.0), DA_EINVAL),
    (dict(scale=float("inf")), DA_EINVAL),
    (dict(scale=float("nan")), DA_EINVAL),
    (dict(workspace=None), DA_EWORKSPACE),
    (dict(workspace_bytes=64), DA_EWORKSPACE),
    (dict(workspace=0xA00000 + 16), DA_EWORKSPACE),  # not 256-byte aligned
    (dict(out=0x10000 + 256), DA_EINVAL),  # out overlaps qkv
    (dict(out=0x200000), DA_EINVAL),       # out overlaps the pool
    (dict(workspace=0x200000), DA_EINVAL), # workspace overlaps the pool
    (dict(out=0xA00000 + 4096), DA_EINVAL),  # out overlaps workspace
])
def test_invalid_arguments_rejected_before_launch(lib, over, code):
    assert _call(lib, **over) == code
    assert _lib.last_error() != ""


def test_qknorm_specific_checks(lib):
    base = dict(qkv=0x10000, stride=512, kp=0x200000, vp=0x202000)

    def q(**o):
        a = dict(positions=0x900200, pdt=0, wq=0x900300, wk=0x900400, eps=1e-5, base=10000.0, R=1)
        a.update(o)
        return lib.drafter_attn_qknorm(0x10000, 512, 0x200000, 0x202000, 16384, 4, 0x900000, 1, 0x900100,
                                       None, a["R"], 8, 6, 1, 64, 64, 0.125, a["positions"], a["pdt"],
                                       a["wq"], a["wk"], a["eps"], a["base"], 0xA00000, 1 << 20, 0xB00000,
                                       384, None, None)
    assert q(positions=None) == DA_EINVAL
    assert q(pdt=2) == DA_EINVAL
    assert q(wq=None) == DA_EINVAL
    assert q(wk=0x900402) == DA_EINVAL      # misaligned
    assert q(eps=-1.0) == DA_EINVAL
    assert q(eps=float("nan")) == DA_EINVAL
    assert q(base=0.0) == DA_EINVAL
    assert q(positions=0xB00000) == DA_EINVAL   # out overlaps positions
    assert q(positions=0x900202) == DA_EINVAL and "aligned" in _lib.last_error()
    assert q(positions=0x900204, pdt=1) == DA_EINVAL and "aligned" in _lib.last_error()
    assert q(R=9) == DA_EINVAL


def _nr(lib, **over):
    """A drafter_qk_norm_rope call with fake (never dereferenced) pointers."""
    a = dict(qkv=0x10000, stride=512, N=8, Hq=6, Hkv=1, hd=64, pos=0x900000, pdt=0, wq=0x900100, wk=0x900200,
             eps=1e-5, base=10000.0)
    a.update(over)
    return lib.drafter_qk_norm_rope(a["qkv"], a["stride"], a["N"], a["Hq"], a["Hkv"], a["hd"], a["pos"], a["pdt"],
                                    a["wq"], a["wk"], a["eps"], a["base"], None)


@pytest.mark.parametrize("over,code", [
    (dict(hd=128), DA_EUNSUPPORTED),
    (dict(Hq=12), DA_EUNSUPPORTED),
    (dict(Hkv=0, Hq=0), DA_EINVAL),
    (dict(Hkv=17, Hq=102), DA_EINVAL),
    (dict(N=0), DA_EINVAL),
    (dict(N=65537), DA_EINVAL),
    (dict(qkv=None), DA_EINVAL),
    (dict(pos=None), DA_EINVAL),
    (dict(wk=None), DA_EINVAL),
    (dict(stride=500), DA_EINVAL),
    (dict(stride=516), DA_EINVAL),
    (dict(qkv=0x10008), DA_EINVAL),
    (dict(wq=0x900108), DA_EINVAL),
    (dict(pdt=2), DA_EINVAL),
    (dict(eps=-1.0), DA_EINVAL),
    (dict(eps=float("inf")), DA_EINVAL),
    (dict(base=0.0), DA_EINVAL),
    (dict(base=float("nan")), DA_EINVAL),
    (dict(pos=0x10000 + 1024), DA_EINVAL),   # positions inside qkv (written in place)
    (dict(wq=0x10000 + 4096), DA_EINVAL),
])
def test_norm_rope_invalid_arguments_rejected_before_launch(lib, over, code):
    assert _nr(lib, **over) == code
    assert _lib.last_error() != ""


def _ap(lib, **over):
    """A drafter_kv_append call with fake (never dereferenced) pointers."""
    a = dict(qkv=0x10000, qs=512, kp=0x200000, vp=0x200000 + 8192, ps=16384, np_=4, pt=0x900000, pts=2,
             cl=0x900100, bl=None, R=1, T=8, Hq=6, Hkv=1, hd=64, pg=64, st=None)
    a.update(over)
    return lib.drafter_kv_append(a["qkv"], a["qs"], a["kp"], a["vp"], a["ps"], a["np_"], a["pt"], a["pts"], a["cl"],
                                 a["bl"], a["R"], a["T"], a["Hq"], a["Hkv"], a["hd"], a["pg"], a["st"], None)


@pytest.mark.parametrize("over,code", [
    (dict(hd=128), DA_EUNSUPPORTED),
    (dict(Hq=12), DA_EUNSUPPORTED),
    (dict(R=9), DA_EINVAL),
    (dict(T=0), DA_EINVAL),
    (dict(pts=0), DA_EINVAL),
    (dict(pt=None), DA_EINVAL),
    (dict(kp=None), DA_EINVAL),
    (dict(cl=None), DA_EINVAL),
    (dict(np_=0), DA_EINVAL),
    (dict(ps=4095), DA_EINVAL),
    (dict(qs=500), DA_EINVAL),
    (dict(kp=0x200008), DA_EINVAL),
    (dict(qkv=0x200000 + 100 * 1024), DA_EINVAL),   # qkv inside the pool (written)
    (dict(pt=0x200000 + 1024), DA_EINVAL),          # page table inside the pool
    (dict(st=0x200000 + 64), DA_EINVAL),            # status word inside the pool
])
def test_kv_append_invalid_arguments_rejected_before_launch(lib, over, code):
    assert _ap(lib, **over) == code
    assert _lib.last_error() != ""


def test_paged_attn_shares_the_attention_checks(lib):
    # same argument list and host checks as drafter_attn (kv_lens in place of context_lens)
    def call(**o):
        a = dict(qkv=0x10000, out=0xB00000, ws=0xA00000, wsb=1 << 20, hd=64, T=8)
        a.update(o)
        return lib.drafter_paged_attn(a["qkv"], 512, 0x200000, 0x202000, 16384, 4, 0x900000, 1, 0x900100, None,
                                      1, a["T"], 6, 1, a["hd"], 64, 0.125, a["ws"], a["wsb"], a["out"], 384,
                                      None, None)
    assert call(hd=128) == DA_EUNSUPPORTED
    assert call(T=9) == DA_EINVAL
    assert call(ws=None) == DA_EWORKSPACE
    assert call(ws=0xA00010) == DA_EWORKSPACE
    assert call(out=0x10000 + 256) == DA_EINVAL
    assert call(qkv=0x10008) == DA_EINVAL


def test_small_arrays_must_be_aligned_to_their_elements(lib):
    # an int32 array or the status word (updated atomically) at an address that is not a
    # multiple of 4, or int64 positions not on 8, is refused before any launch
    for over in (dict(page_table=0x900002), dict(context_lens=0x900102), dict(block_lens=0x900202),
                 dict(status=0x900302)):
        assert _call(lib, **over) == DA_EINVAL, over
        assert "aligned" in _lib.last_error()
    for over in (dict(pt=0x900001), dict(cl=0x900103), dict(bl=0x900202), dict(st=0x900302)):
        assert _ap(lib, **over) == DA_EINVAL, over
        assert "aligned" in _lib.last_error()
    assert _nr(lib, pos=0x900002) == DA_EINVAL and "aligned" in _lib.last_error()
    assert _nr(lib, pos=0x900004, pdt=1) == DA_EINVAL and "aligned" in _lib.last_error()


@pytest.mark.parametrize("yarn", [
    (0.5, 4096, 1.0, 32.0),              # factor below 1
    (float("nan"), 4096, 1.0, 32.0),
    (float("inf"), 4096, 1.0, 32.0),
    (4.0, 0, 1.0, 32.0),                 # no original context
    (4.0, 4096, 32.0, 32.0),             # empty ramp
    (4.0, 4096, 5.0, 2.0),               # reversed ramp
    (4.0, 4096, -1.0, 32.0),
    (4.0, 4096, 1.0, float("nan")),
    (4.0, 4096, 1.0, 32.0, 3, 0.0),      # ramp outside DA_YARN_RAMP_*
    (4.0, 4096, 1.0, 32.0, -1, 0.0),
    (4.0, 4096, 1.0, 32.0, 0, -1.0),     # negative factor on q and k
    (4.0, 4096, 1.0, 32.0, 1, float("nan")),
    (4.0, 4096, 1.0, 32.0, 2, float("inf")),
    (4.0, 4096, 1.0, 32.0, 1, 0.0, 1.0),   # a ramp in the pair index with base 1 (no falling frequencies)
    (4.0, 4096, 1.0, 32.0, 2, 1.0, 0.5),
])
def test_yarn_parameters_rejected_before_launch(lib, yarn):
    base = yarn[6] if len(yarn) > 6 else 1e4
    y = ctypes.pointer(_lib.DaYarn(*yarn[:6]))
    rc = lib.drafter_qk_norm_rope_yarn(0x10000, 512, 8, 6, 1, 64, 0x900000, 0, 0x900100, 0x900200, 1e-5, base, y, None)
    assert rc == DA_EINVAL and "yarn" in _lib.last_error()
    rc = lib.drafter_attn_qknorm_yarn(0x10000, 512, 0x200000, 0x202000, 16384, 4, 0x900000, 1, 0x900100, None,
                                      1, 8, 6, 1, 64, 64, 0.125, 0x900200, 0, 0x900300, 0x900400, 1e-5, base, y,
                                      0xA00000, 1 << 20, 0xB00000, 384, None, None)
    assert rc == DA_EINVAL and "yarn" in _lib.last_error()


@pytest.mark.parametrize("ramp,mscale", [(0, 0.0), (1, 1.0), (2, 0.5)])
def test_acceptable_yarn_passes_the_yarn_checks(lib, ramp, mscale):
    # an acceptable YaRN struct gets past the YaRN checks: the call then fails on the next
    # host check (positions inside the qkv rows it would rewrite), before any launch
    y = ctypes.pointer(_lib.DaYarn(4.0, 4096, 1.0, 32.0, ramp, mscale))
    rc = lib.drafter_qk_norm_rope_yarn(0x10000, 512, 8, 6, 1, 64, 0x10100, 0, 0x900100, 0x900200, 1e-5, 1e4, y, None)
    assert rc == DA_EINVAL and "overlaps" in _lib.last_error()


def test_binding_rejects_malformed_yarn():
    from speculative_decoding_drafter_amd import DrafterAttnError
    from speculative_decoding_drafter_amd.ops import _yarn

    assert _yarn(None) is None
    assert _yarn(dict(factor=4.0, original_max_position=4096)).contents.beta == 32.0
    y = _yarn(dict(factor=4.0, original_max_position=4096, ramp="index_unrounded", mscale=1.0)).contents
    assert (y.ramp, y.mscale) == (2, 1.0)
    for bad in (dict(factor=4.0), dict(original_max_position=4096), (4.0, 4096),
                dict(factor=4.0, original_max_position=4096, ramp="dims"),
                dict(factor=4.0, original_max_position=4096, rope_type="yarn")):
        with pytest.raises(DrafterAttnError):
            _yarn(bad)


def _na(lib, **over):
    """A drafter_attn_qknorm_noalloc call with fake (never dereferenced) pointers: every case here is
    refused by a host check before the device is touched (no GPU in this environment)."""
    a = dict(qkv=0x10000, qs=512, kp=0x200000, vp=0x202000, ps=16384, np_=4, pt=0x900000, pts=1, cl=0x900100,
             bl=None, R=1, T=8, Hq=6, Hkv=1, hd=64, pg=64, scale=0.125, pos=0x900200, pdt=0, wq=0x900300,
             wk=0x900400, eps=1e-5, base=10000.0, out=0xB00000, os=384, st=None)
    a.update(over)
    return lib.drafter_attn_qknorm_noalloc(
        a["qkv"], a["qs"], a["kp"], a["vp"], a["ps"], a["np_"], a["pt"], a["pts"], a["cl"], a["bl"], a["R"], a["T"],
        a["Hq"], a["Hkv"], a["hd"], a["pg"], a["scale"], a["pos"], a["pdt"], a["wq"], a["wk"], a["eps"], a["base"],
        a["out"], a["os"], a["st"], None)


@pytest.mark.parametrize("over,code", [
    (dict(hd=128), DA_EUNSUPPORTED),
    (dict(Hq=12), DA_EUNSUPPORTED),
    (dict(R=9), DA_EINVAL),
    (dict(T=0), DA_EINVAL),
    (dict(qkv=None), DA_EINVAL),
    (dict(out=None), DA_EINVAL),
    (dict(qs=500), DA_EINVAL),
    (dict(out=0x10000 + 256), DA_EINVAL),     # out overlaps qkv
    (dict(scale=float("nan")), DA_EINVAL),
    (dict(pos=None), DA_EINVAL),
    (dict(pdt=2), DA_EINVAL),
    (dict(wk=0x900402), DA_EINVAL),
    (dict(eps=-1.0), DA_EINVAL),
    (dict(pos=0xB00000), DA_EINVAL),          # out overlaps positions
    # 8 requests x 16 KV heads with 1M-token rows: 8 * 16 * 32 partial slots, above the scratch
    (dict(R=8, Hq=96, Hkv=16, pts=16384, qkv=0x1000000, qs=128 * 64, ps=16 * 4096 * 2, out=0x2000000,
          os=96 * 64, pt=0x3000000, cl=0x3100000, pos=0x3200000, wq=0x3300000, wk=0x3300100), DA_EWORKSPACE),
])
def test_noalloc_refused_before_touching_the_device(lib, over, code):
    assert _na(lib, **over) == code
    assert _lib.last_error() != ""


def test_noalloc_scratch_limit_in_partial_slots(lib):
    # the header's limit: 32768 bytes of counters plus R*Hkv*S slots of 12,672 bytes (two regions
    # rounded to 256) within DA_NOALLOC_SCRATCH_BYTES -- 1,321 slots.  Sizes whose plan needs more
    # are refused with DA_EWORKSPACE.  Only refused sizes are called here: a size that fits would
    # pass every host check and reach the device with these fake pointers.
    text = open(HEADER).read()
    cap = eval(re.search(r"#define DA_NOALLOC_SCRATCH_BYTES \((\d+u << \d+)\)", text).group(1).replace("u", ""))
    a256 = lambda x: (x + 255) // 256 * 256
    fits = lambda n: 32768 + a256(n * 48 * 64 * 4) + a256(n * 48 * 2 * 4) <= cap
    assert fits(1321) and not fits(1322)
    refused = 0
    for R, hkv, stride in [(8, 16, 16384), (8, 16, 4096), (8, 4, 16384), (8, 4, 512), (2, 16, 16384), (8, 8, 8192),
                           (8, 16, 256), (1, 1, 16384), (8, 16, 8192), (8, 12, 16384), (6, 16, 8192)]:
        s, p = ctypes.c_int32(), ctypes.c_int32()
        assert lib.drafter_attn_plan(R, hkv, stride, ctypes.byref(s), ctypes.byref(p)) == DA_OK
        n = R * hkv * s.value
        if (R, hkv, stride) in ((8, 4, 512), (8, 4, 16384), (8, 16, 256)):
            assert fits(n), (R, hkv, stride, n)   # the 32k workload, 1M tokens at 24/4, 16k at 96/16
        if fits(n):
            continue
        rc = _na(lib, R=R, Hq=6 * hkv, Hkv=hkv, pts=stride, qkv=0x1000000, qs=(8 * hkv) * 64,
                 ps=hkv * 4096 * 2, out=0x2000000, os=6 * hkv * 64, pt=0x3000000, cl=0x3100000, pos=0x3200000,
                 wq=0x3300000, wk=0x3300100)
        assert rc == DA_EWORKSPACE and "scratch" in _lib.last_error(), (R, hkv, stride, n)
        refused += 1
    assert refused >= 3


# ---- the page-stream probe (measurement library of bench.py --ceiling): loads, exports its
# entry point and refuses arguments that do not fit before any device call

@pytest.fixture(scope="module")
def probe_lib():
    from speculative_decoding_drafter_amd import build
    if not os.path.exists(build.LIB_PROBE):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(build.LIB_PROBE)
    fn = lib.page_stream_probe
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return fn


PROBE_OK = dict(mode=0, k=0x1000, v=0x2000, num_pages=5000, page_bytes=65536, Hkv=4, pt=0x3000, stride=512,
                lens=0x4000, R=8, S=8, Ps=64, stream=268435456, out=0x5000, out_words=2048, hip_stream=None)


@pytest.mark.parametrize("over", [
    dict(mode=4), dict(mode=-1), dict(k=None), dict(v=None), dict(pt=None), dict(lens=None), dict(out=None),
    dict(R=0), dict(Hkv=0), dict(S=0), dict(Ps=0), dict(Ps=513), dict(stride=0),
    dict(S=7),                      # 7 splits of 64 pages do not cover a 512-page row
    dict(num_pages=0), dict(out_words=2047),
    dict(page_bytes=32768 - 16), dict(page_bytes=65536 + 8), dict(page_bytes=(1 << 32) + 16),
    dict(mode=3, stream=8), dict(mode=3, stream=268435456 + 4), dict(mode=3, stream=4999 * 65536 + 32768 + 16),
])
def test_probe_refuses_arguments_that_do_not_fit(probe_lib, over):
    a = dict(PROBE_OK, **over)
    assert probe_lib(a["mode"], a["k"], a["v"], a["num_pages"], a["page_bytes"], a["Hkv"], a["pt"], a["stride"],
                     a["lens"], a["R"], a["S"], a["Ps"], a["stream"], a["out"], a["out_words"], a["hip_stream"]) == -1
