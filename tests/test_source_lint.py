"""Source lint of the kernels' LDS hand-offs (CPU): every LDS buffer that one wave writes and
another reads has a workgroup barrier between the write and the read, and every page slot is
refilled by DMA only after the wave's own reads of it have returned.

The checks are on the source text (comments stripped), in program order; each is also run on
a copy with the barrier taken out, to show that the lint would catch that.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "speculative_decoding_drafter_amd", "csrc", "drafter_attn.hip")


def _code(text: str) -> str:
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return re.sub(r"//[^\n]*", " ", text)


def _barrier_between(code: str, write: str, read: str, nth: int = 0) -> bool:
    """The nth occurrence of `write`, then the first `read` after it: a __syncthreads() between."""
    pos = -1
    for _ in range(nth + 1):
        pos = code.index(write, pos + 1)
    end = code.index(read, pos + len(write))
    return "__syncthreads()" in code[pos:end]


# (what, written by, read by, occurrence): buffers one thread writes and others read
HANDOFFS = [
    ("rotation table (attention)", "cs[tid] = rope_cos_sin", "cs + t * 32", 0),
    ("query tile and own-block rows", "smem + kOffQ + qoff(sub, u)", "const unsigned char* qt = smem + kOffQ;", 0),
    ("per-wave row statistics", "mW[(16 * nt + lane) * kWaves + w] =", "mW + row * kWaves", 0),
    ("per-wave output in the page slot", "ob + (16 * nt + (lane & 15)) * kObufStride", "row * kObufStride + 4 * oc", 0),
    ("last-workgroup flag", "*last = is_last;", "if (!*last", 0),
    ("rotation table (norm/rotation)", "cs[tid] = rope_cos_sin", "cs + t * 32", 1),
]


@pytest.mark.parametrize("what,write,read,nth", HANDOFFS, ids=[h[0] for h in HANDOFFS])
def test_barrier_between_write_and_read(what, write, read, nth):
    code = _code(open(SRC).read())
    assert _barrier_between(code, write, read, nth), what


@pytest.mark.parametrize("what,write,read,nth", HANDOFFS, ids=[h[0] for h in HANDOFFS])
def test_lint_catches_a_missing_barrier(what, write, read, nth):
    code = _code(open(SRC).read())
    pos = -1
    for _ in range(nth + 1):
        pos = code.index(write, pos + 1)
    end = code.index(read, pos + len(write))
    planted = code[:pos] + code[pos:end].replace("__syncthreads()", "(void)0") + code[end:]
    assert not _barrier_between(planted, write, read, nth)


def _page_loop(code: str) -> str:
    start = code.index("for (int i = 0; i < cnt; ++i)")
    return code[start:code.index("attend_page<NT>(kslot", start)]


def test_slot_refilled_only_after_its_reads_returned():
    loop = _page_loop(_code(open(SRC).read()))
    calls = [m.start() for m in re.finditer(r"stage_tile<", loop)]
    assert len(calls) == 2  # the next page's K, then its V
    for c in calls:
        before = loop[:c].rstrip()
        assert before.endswith("wait_lds_reads();"), loop[max(0, c - 80):c]


def test_last_page_waits_for_every_dma_before_the_slot_is_reused():
    # after the loop each wave writes its output into its own page slot: the last page's wait
    # must drain every DMA (vmcnt 0), not just this page's K
    loop = _page_loop(_code(open(SRC).read()))
    assert re.search(r"if \(more\) wait_vmcnt<8>\(\); else wait_vmcnt<0>\(\);", loop)


# ---- m0: the DMA helper writes it from inline asm without declaring it (clang rejects m0 as a
# clobber), so the compiler must never use m0 itself in this device code.  The check compiles
# the device code to gfx950 assembly and requires every m0 reference to sit inside one of the
# helper's asm blocks, as its `s_mov_b32 m0, s<N>` followed by the LDS DMA.

def _m0_outside_asm(asm: str):
    inside, outside, blocks = 0, [], []
    cur = None
    for ln in asm.splitlines():
        if ";;#ASMSTART" in ln:
            cur = []
            continue
        if ";;#ASMEND" in ln:
            blocks.append(cur)
            cur = None
            continue
        code = ln.split(";")[0].strip()
        if cur is not None and code:
            cur.append(code)
        if re.search(r"\bm0\b", code):
            if cur is None:
                outside.append(code)
            else:
                inside += 1
    bad_blocks = [b for b in blocks if any(re.search(r"\bm0\b", c) for c in b)
                  and not (re.fullmatch(r"s_mov_b32 m0, s\d+", b[0]) and
                           all(c.startswith(("s_nop", "global_load_lds_dwordx4")) for c in b[1:]))]
    return inside, outside, bad_blocks


PROBE_SRC = os.path.join(os.path.dirname(SRC), "page_stream_probe.hip")


@pytest.fixture(scope="module", params=[SRC, PROBE_SRC], ids=["attention", "page_stream_probe"])
def device_asm(request, tmp_path_factory):
    import shutil
    import subprocess

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    inc = os.path.join(os.path.dirname(os.path.dirname(SRC)), "..", "include")
    out = tmp_path_factory.mktemp("asm") / "device.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.abspath(inc), "-o", str(out),
           request.param]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    return out.read_text()


def test_m0_is_written_only_by_the_dma_helper(device_asm):
    inside, outside, bad = _m0_outside_asm(device_asm)
    assert inside > 0, "no DMA helper found in the assembly"
    assert outside == [], f"compiler-managed m0 uses: {outside[:5]}"
    assert bad == [], f"asm blocks touching m0 that are not the DMA helper: {bad[:2]}"


def test_m0_lint_catches_a_compiler_use(device_asm):
    planted = device_asm.replace(";;#ASMSTART", "\ts_mov_b32 m0, -1\n;;#ASMSTART", 1)
    assert _m0_outside_asm(planted)[1] != []
    # an asm block that reads m0 (whatever else it holds) is not the DMA helper's
    planted = device_asm.replace(";;#ASMEND", "\ts_mov_b32 s0, m0\n;;#ASMEND", 1)
    assert _m0_outside_asm(planted)[2] != []
