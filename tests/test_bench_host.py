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
