"""Host-side pieces of bench.py, on the CPU: the oracle baseline leg (fed
the oracle's own streams in place of the GPU's, so every comparison must
hold) and the per-call timing summary."""
import numpy as np

import bench
import workloads as W
from oracle import codebook as cb
from oracle import coder


def test_cpu_baseline_leg_on_oracle_streams():
    w = W.WORKLOADS["normal_1m"]
    x = W.make("normal_1m", 0)
    counts = np.bincount(W.make("normal_1m", 1), minlength=256)
    book = cb.codebook([int(c) for c in counts], "huffman", None)
    s = coder.encode(x, book["lengths"], book["codes"], w.chunk, threads=4)
    streams = {
        "payload": lambda m: s["payload"][:m],
        "chunk_bits": s["chunk_bits"].astype(np.uint32),
        "chunk_word_offset": s["chunk_word_offset"],
        "sub_off": s["sub_off"].astype(np.uint32),
    }
    res, parity = bench.cpu_baseline_leg(x, counts, "huffman", None, w.chunk, streams, 0.2, 4)
    assert all(v for k, v in parity.items() if k != "chunks"), parity
    assert parity["chunks"] >= 1
    assert res["kind"] == "oracle" and res["cores"] == 4 and res["value"] > 0
    assert res["single_thread"]["value"] > 0 and res["single_thread"]["bytes"] % w.chunk == 0


def test_ms_stats():
    st = bench.ms_stats([1.0, 2.0, 3.0, 4.0, 5.0])
    assert st["mean"] == 3.0 and st["median"] == 3.0 and st["min"] == 1.0 and st["max"] == 5.0
    assert st["p10"] == 1.4 and st["p90"] == 4.6


def test_oracle_parity_leg_on_oracle_streams():
    """The per-configuration oracle comparison of the cpu_baseline leg, fed the
    oracle's own stream (every array must compare equal), and one that has a
    flipped payload bit (the payload must compare unequal)."""
    x = W.make("normal_1m", 0)[: 5 * 4096 + 77]
    counts = np.bincount(W.make("normal_1m", 1), minlength=256)
    book = cb.codebook([int(c) for c in counts], "huffman", None)
    s = coder.encode(x, book["lengths"], book["codes"], 4096, threads=2)
    host = {k: s[k].copy() for k in ("payload", "chunk_bits", "chunk_word_offset", "sub_off")}
    got = bench.oracle_parity((x, counts, "huffman", None, 4096, host), 2)
    assert all(got.values()), got
    host["payload"][3] ^= 1
    got = bench.oracle_parity((x, counts, "huffman", None, 4096, host), 2)
    assert not got["payload"] and got["chunk_bits"] and got["oracle_round_trip"]


def test_pmc_summary_scales_by_the_probe_copy(tmp_path):
    """Counter summary on hand-made rocprofv3 CSVs: both calibration copies
    move copy_bytes each way; the probe's scale converts the coder kernels'
    counts, the runtime copy's is printed beside it."""
    import csv

    cb_ = 1 << 20
    rows = {  # KiB per dispatch
        "FETCH_SIZE": [("__amd_rocclr_copyBuffer", 512.0), ("pc::probe_copy_kernel(...)", 512.0),
                       ("pc::encode_unit_kernel<8>(...)", 600.0), ("pc::decode_kernel<0, true>(...)", 400.0),
                       ("pc::decode_kernel<0, true>(...)", 420.0), ("pc::decode_kernel<0, true>(...)", 410.0)],
        "WRITE_SIZE": [("__amd_rocclr_copyBuffer", 1024.0), ("pc::probe_copy_kernel(...)", 1000.0),
                       ("pc::encode_unit_kernel<8>(...)", 800.0), ("pc::decode_kernel<0, true>(...)", 1024.0)],
    }
    dirs = {}
    for counter, rs in rows.items():
        d = tmp_path / counter
        d.mkdir()
        with open(d / "bench_counter_collection.csv", "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for k, v in rs:
                wr.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})
        dirs[counter] = str(d)
    out = tmp_path / "traffic.txt"
    bench.pmc_summary(dirs["FETCH_SIZE"], dirs["WRITE_SIZE"], cb_, out=str(out))
    text = out.read_text()
    assert "fetch_scale 2.000000 (copyBuffer 2.000000)" in text
    assert "write_scale 1.024000 (copyBuffer 1.000000)" in text
    kern = {l.split()[1]: l.split() for l in text.splitlines() if l.startswith("kernel ")}
    # (printed to whole bytes)
    assert abs(float(kern["encode"][5]) - 600.0 * 1024 * 2) < 1
    assert abs(float(kern["encode"][7]) - 800.0 * 1024 * 1.024) < 1
    assert abs(float(kern["decode"][5]) - 410.0 * 1024 * 2) < 1  # the median dispatch


def test_l2_summary_medians_and_hit_share(tmp_path):
    """L2 counter table on a hand-made rocprofv3 CSV: per kernel the median
    over dispatches of each counter, and hits / (hits + misses)."""
    import csv

    d = tmp_path / "l2"
    d.mkdir()
    rows = [("pc::encode_unit_kernel<64>(...)", "TCC_HIT_sum", v) for v in (90.0, 80.0, 70.0)]
    rows += [("pc::encode_unit_kernel<64>(...)", "TCC_MISS_sum", v) for v in (10.0, 20.0, 30.0)]
    rows += [("pc::decode_kernel<0, true>(...)", "TCC_HIT_sum", 50.0), ("pc::decode_kernel<0, true>(...)", "TCC_MISS_sum", 150.0)]
    rows += [("__amd_rocclr_copyBuffer", "TCC_HIT_sum", 1.0)]
    with open(d / "bench_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    out = tmp_path / "l2.txt"
    bench.l2_summary([str(d)], str(out), ["rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum -- python3 bench.py"])
    lines = {l.split()[0]: l.split() for l in out.read_text().splitlines() if not l.startswith("#")}
    assert lines["counter"][1:] == ["encode", "decode"]
    assert lines["TCC_HIT_sum"][1:] == ["80", "50"] and lines["TCC_MISS_sum"][1:] == ["20", "150"]
    share = [l for l in out.read_text().splitlines() if l.startswith("L2 hit share")][0].split()
    assert share[-2:] == ["0.8000", "0.2500"]
