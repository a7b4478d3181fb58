"""Host logic of the rocprofv3 summaries: counter calibration against a copy
of known size, per-dispatch averaging, and the kernel-trace table."""

import csv
import json
import os
import sqlite3

import pytest

from paged_kv_decode_attention_amd import counters, inputs as I

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": val})


DEC = "void pa::(anonymous namespace)::decode_mfma_balanced<pa::BF16, 16>(pa::DecodeArgs)"
MRG = "void pa::(anonymous namespace)::merge_balanced<pa::BF16>(pa::DecodeArgs)"
CPY = "pa::(anonymous namespace)::copy_kernel(unsigned int __vector(4)*, unsigned long)"


def test_traffic_scaled_by_copy_readings(tmp_path):
    n = 1 << 30
    # the copy reads n bytes: FETCH_SIZE reports half of them in KiB; WRITE_SIZE all
    write_csv(tmp_path / "cf", "FETCH_SIZE", [(CPY, n / 2048)] * 3)
    write_csv(tmp_path / "cw", "WRITE_SIZE", [(CPY, n / 1024)] * 3)
    # two dispatches each of the decode and merge kernels, plus an unrelated kernel
    write_csv(tmp_path / "f", "FETCH_SIZE", [(DEC, 1000.0), (DEC, 1002.0), (MRG, 10.0),
                                             (MRG, 10.0), ("other", 5e6)])
    write_csv(tmp_path / "w", "WRITE_SIZE", [(DEC, 4.0), (DEC, 4.0), (MRG, 2.0), (MRG, 2.0)])
    out = tmp_path / "t.json"
    rc = counters.main(["traffic", "--fetch", str(tmp_path / "f"), "--write",
                        str(tmp_path / "w"), "--copy-fetch", str(tmp_path / "cf"),
                        "--copy-write", str(tmp_path / "cw"), "--copy-bytes", str(n),
                        "--config", "tiny_fp32", "--out", str(out), "--command", "c1"])
    assert rc == 0
    rec = json.loads(out.read_text())
    assert rec["fetch_factor_bytes_per_kib"] == pytest.approx(2048.0)
    assert rec["write_factor_bytes_per_kib"] == pytest.approx(1024.0)
    expect = 1001.0 * 2048 + 4.0 * 1024 + 10.0 * 2048 + 2.0 * 1024
    assert rec["hbm_bytes_per_launch"] == pytest.approx(expect)
    assert set(rec["kernels"]) == {"decode_mfma_balanced<pa::BF16, 16>",
                                   "merge_balanced<pa::BF16>"}
    cfg = I.CONFIGS["tiny_fp32"]
    assert rec["alg_bytes_per_launch"] == I.kv_bytes_read(cfg, I.draw_context_lens(cfg))
    assert rec["commands"] == ["c1"]


def test_draw_context_lens_matches_generate():
    small = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=4, num_blocks=1024,
                             num_kv_heads=1, num_heads=1)
    for cfg in (I.CONFIGS["tiny_fp32"], small):
        assert (I.draw_context_lens(cfg) == I.generate(cfg).context_lens.numpy()).all()


def test_trace_table(tmp_path):
    db = tmp_path / "k.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, end integer)")
    rows = [(DEC, 0, 50_000), (DEC, 100_000, 160_000), (MRG, 60_000, 65_000)]
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    table = counters.trace_table(str(db))
    assert [r[0] for r in table] == ["decode_mfma_balanced<pa::BF16, 16>",
                                     "merge_balanced<pa::BF16>"]
    k, calls, avg, lo, hi, share = table[0]
    assert (calls, avg, lo, hi) == (2, 55.0, 50.0, 60.0)
    assert share == pytest.approx(100.0 * 110 / 115)
    # the JSON record bench.py reads: per-kernel durations and the source hash
    out, js = tmp_path / "t.md", tmp_path / "t.json"
    counters.main(["trace", "--db", str(db), "--out", str(out), "--title", "t",
                   "--command", "c", "--json", str(js), "--sha", "abc"])
    rec = json.load(open(js))
    assert rec["kernel_src_sha"] == "abc"
    dec = rec["kernels"]["decode_mfma_balanced<pa::BF16, 16>"]
    assert (dec["calls"], dec["avg_us"], dec["median_us"], dec["min_us"], dec["max_us"]) == \
        (2, 55.0, 55.0, 50.0, 60.0)
    assert rec["kernels"]["merge_balanced<pa::BF16>"]["median_us"] == 5.0
    assert counters.median([1.0, 2.0, 7.0]) == 2.0


def test_compute_counter_summary(tmp_path):
    """Per-dispatch means of the instruction counters and the per-wavefront
    figures derived from them, for the decode kernels only."""
    d = tmp_path / "c"
    os.makedirs(d)
    vals = {"SQ_WAVES": (1024, 576), "SQ_INSTS_VALU": (2048000, 57600),
            "SQ_INSTS_MFMA": (409600, 0), "SQ_INSTS_SALU": (102400, 5760),
            "SQ_INSTS_LDS": (20480, 576), "SQ_INSTS_VMEM_RD": (163840, 2304),
            "SQ_LDS_BANK_CONFLICT": (100, 0), "MfmaUtil": (12.5, 0.0)}
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        i = 0
        for c, (vd, vm) in vals.items():
            for name, v in ((DEC, vd), (DEC, vd), (MRG, vm), ("other", 7.0)):
                w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                            "Counter_Name": c, "Counter_Value": v})
                i += 1
    out = tmp_path / "c.md"
    counters.main(["compute", "--run", str(d), "--out", str(out), "--title", "t",
                   "--command", "cmd"])
    text = out.read_text()
    assert "other" not in text
    dec_rows = [l for l in text.splitlines() if l.startswith("| decode_mfma_balanced")]
    assert dec_rows[0].split("|")[2].strip() == "2"             # dispatches
    assert dec_rows[0].split("|")[-2].strip() == "12.50"        # MFMA busy %
    # per wavefront: 2048000 / 1024 VALU, 409600 / 1024 MFMA, 160 VMEM reads
    assert [c.strip() for c in dec_rows[1].split("|")[2:7]] == ["2000", "400", "100", "20", "160"]
