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
