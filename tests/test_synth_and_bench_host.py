"""Host-side pieces (CPU only): the seeded input generators are deterministic, and the
bench's counter-file pipeline turns rocprofv3 CSVs into the traffic record correctly."""
import csv
import json
import os
import sys

import numpy as np
import torch

import drafter_synth as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bits(t):
    return None if t is None else t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype == torch.bfloat16 \
        else t.numpy().tobytes()


def test_generators_are_deterministic():
    for n in (1, 2, 3):
        a, b = ds.make_config(n), ds.make_config(n)
        for name in ("qkv", "pool", "page_table", "context_lens", "positions", "q_norm_weight"):
            assert _bits(getattr(a, name)) == _bits(getattr(b, name)), (n, name)
    # another draw index gives other values; the poisoned draw agrees on everything read
    a, c = ds.make_config(2, k=0), ds.make_config(2, k=1)
    assert _bits(a.qkv) != _bits(c.qkv)
    p = ds.make_config(2, poison=True)
    assert torch.equal(p.context_lens, a.context_lens)
    for r in range(a.R):
        L = int(a.context_lens[r])
        npg = -(-L // 64)
        assert torch.equal(p.page_table[r, :npg], a.page_table[r, :npg])
    rows = ds.make_norm_rope_rows(17, 2, seed=3, row_pad=8)
    again = ds.make_norm_rope_rows(17, 2, seed=3, row_pad=8)
    assert _bits(rows.qkv) == _bits(again.qkv) and torch.equal(rows.positions, again.positions)


def test_append_room_gives_fresh_distinct_pages():
    case = ds.make_config(3)
    room = ds.with_append_room(case, seed=5)
    P = case.num_pages
    used = set()
    for r in range(case.R):
        L = int(case.context_lens[r])
        have, need = -(-L // 64), -(-(L + case.T) // 64)
        assert torch.equal(room.page_table[r, :have], case.page_table[r, :have])
        for j in range(have, need):
            pg = int(room.page_table[r, j])
            assert pg >= P and pg not in used
            used.add(pg)
    assert room.num_pages == P + len(used)
    assert torch.equal(room.pool[:P].view(torch.int16), case.pool.view(torch.int16))


def _write_csv(path, rows):
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_traffic_record_from_counter_csvs(tmp_path):
    sys.path.insert(0, ROOT)
    import bench

    kern = "void (anonymous namespace)::drafter_attn_kernel<3, true, false>((anonymous namespace)::Params)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(1, 1024, copy, "FETCH_SIZE", 12.5),           # a small copy: ignored
             (2, 131072, copy, "FETCH_SIZE", 262144.0),     # the 512 MiB copy reads 524288 KiB
             (3, 131072, copy, "FETCH_SIZE", 262144.0),
             (4, 256, kern, "FETCH_SIZE", 100.0), (5, 256, kern, "FETCH_SIZE", 300.0)]
    write = [(2, 131072, copy, "WRITE_SIZE", 524288.0), (4, 256, kern, "WRITE_SIZE", 10.0),
             (5, 256, kern, "WRITE_SIZE", 30.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "traffic.json"
    _write_csv(fp, fetch)
    _write_csv(wp, write)
    rec = bench.write_traffic(str(fp), str(wp), 5, dest=str(out))
    assert rec["kernel"] == kern and rec["dispatches"] == 2
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    # (mean fetch 200 KiB x 2 + mean write 20 KiB x 1) per launch
    assert rec["traffic_bytes_per_launch"] == 1024 * (200.0 * 2 + 20.0)
    assert json.load(open(out)) == rec
    assert rec["kernel_code_sha256"] == bench.kernel_code_hash()


def test_cpu_baseline_reports_pool_and_one_thread():
    import bench

    case = ds.make_config(1)
    rec = bench.cpu_baseline(case, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] >= 1
    assert rec["one_thread"]["cores"] == 1 and rec["one_thread"]["value"] > 0


def test_traffic_record_key_follows_device_code_and_plan(tmp_path, monkeypatch):
    # the record stays valid across host-side validation edits, not across device or plan edits
    import bench

    src = open(bench.KERNEL_SRC).read()
    base = bench.kernel_code_hash()

    def hash_of(text):
        f = tmp_path / "k.hip"
        f.write_text(text)
        monkeypatch.setattr(bench, "KERNEL_SRC", str(f))
        return bench.kernel_code_hash()

    assert hash_of(src) == base
    host_edit = src.replace('"qkv and out must be 16-byte aligned"', '"qkv and out: 16-byte alignment"')
    assert host_edit != src and hash_of(host_edit) == base
    device_edit = src.replace("kRescaleLog2 = 8", "kRescaleLog2 = 7")
    assert device_edit != src and hash_of(device_edit) != base
    plan_edit = src.replace("kTargetWorkgroups = 256", "kTargetWorkgroups = 512")
    assert plan_edit != src and hash_of(plan_edit) != base


def test_balanced_plan_of_the_mixed_workloads():
    # the plan bench.py --mixed reports for each of its workloads, by the documented rule
    # (Pb = smallest multiple of 8 >= ceil(N / (R (S-1))) and >= ceil(max npg / 32), taken
    # only when Pb <= 3/4 of the static split rounded down to a multiple of 8)
    sys.path.insert(0, ROOT)
    import bench

    want = [(True, 32), (True, 64), (True, 32), (True, 8), (False, 64), (False, 64)]
    got = []
    for _, R, Hq, Hkv, stride, lens in bench.MIXED:
        if isinstance(lens, tuple):
            lens = [int(x) for x in np.random.default_rng(lens[0]).integers(0, lens[1] + 1, R)]
        got.append(bench.balanced_plan(R, Hkv, stride, lens))
    assert got == want
    # equal lengths never balance; one long request among empty ones always does when there is room
    assert bench.balanced_plan(8, 4, 512, [32768] * 8) == (False, 64)
    assert bench.balanced_plan(8, 4, 1024, [65536] + [0] * 7)[0]
