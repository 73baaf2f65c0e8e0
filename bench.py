#!/usr/bin/env python3
"""Throughput of fixed-codebook encode + decode on one MI355X.

One step = the whole hot path over one batch: pc_encode (codeword lookup,
bit-length scan, cross-chunk scan, bit packing, stores) followed by pc_decode
(side-index sub-streams through the 12-bit peek table) of the same stream.
Inputs are resident in HBM before timing starts; the codebook is built
offline from previous batches and is not timed.  Before the W warmup steps,
untimed steps run until their time stops falling (the GPU's first ~25
encode/decode pairs after start-up are up to 15-20% slower; the line reports
the steady state and the number of such steps as `settle_steps`).

Prints one JSON line.  `value` = uncompressed bytes per second of the round
trip (n / step time), in GB/s.  Also reported: encode-only and decode-only
GB/s from HIP events on the launch stream, bits/symbol against the entropy,
the HBM roofline of the slower kernel, and the CPU oracle timed on a bounded
sample of the same stream (with its outputs compared to the GPU's).

    python bench.py [--steps K] [--warmup W] [--workload stream_1g]
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR   # write profiles/traffic.txt
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import shlex
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "coder_kernels_stream_1g_hbm_traffic.txt")
KERNEL_SOURCES = {
    "encode": os.path.join(ROOT, "static_codebook_lossless_amd", "csrc", "encode.hip"),
    "decode": os.path.join(ROOT, "static_codebook_lossless_amd", "csrc", "decode.hip"),
}
KERNEL_NAMES = {"encode": "encode_unit_kernel", "decode": "decode_kernel<0, true>"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kind: str) -> str:
    with open(KERNEL_SOURCES[kind], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters (FETCH_SIZE / WRITE_SIZE, KiB per
# dispatch), scaled by what the same counters read for a plain copy of
# known size that runs in the same program.
# ---------------------------------------------------------------------------

def _read_counter_csv(d, counter):
    import csv

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under " + d)
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def pmc_summary(fetch_dir, write_dir, copy_bytes, out=TRAFFIC_FILE):
    """Per-dispatch HBM bytes of the coder kernels.  bench.py copies
    copy_bytes bytes twice: with the runtime's copy kernel, and with
    pc_traffic_probe, which uses the coder kernels' own 16-byte non-temporal
    loads and stores.  Each reads copy_bytes and writes copy_bytes, so
    scale = copy_bytes / counter(copy).  The probe's scale converts the coder
    kernels' counts; the runtime copy's is printed beside it as a check."""
    res = {}
    copy_bytes16 = copy_bytes // 16 * 16
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for name, val in _read_counter_csv(d, counter):
            per.setdefault(name, []).append(val * 1024.0)  # KiB -> bytes
        blit = [max(vs) for k, vs in per.items() if "copyBuffer" in k]
        probe = [sorted(vs)[len(vs) // 2] for k, vs in per.items() if "probe_copy_kernel" in k]
        if not blit or not probe:
            raise RuntimeError("no calibration copy found for the %s scale" % counter)
        res[counter] = {"scale_blit": copy_bytes / max(blit), "scale": copy_bytes16 / probe[0],
                        "kernels": {k: sorted(v)[len(v) // 2] for k, v in per.items()}}
    labels = ["copyBuffer", "probe_copy_kernel"] + list(KERNEL_NAMES.values())
    lines = ["# HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of bench.py.",
             "# Made by (from the repository root, after cd /tmp && export TMPDIR=/tmp):",
             "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o bench -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs --no-secondary" % fetch_dir,
             "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o bench -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-configs --no-secondary" % write_dir,
             "#   python3 bench.py --pmc-summary %s %s" % (fetch_dir, write_dir),
             "# Each counter is scaled by copy_bytes / counter(copy of copy_bytes bytes made with the coder",
             "# kernels' 16-byte non-temporal loads and stores, pc_traffic_probe); the scale from the runtime's",
             "# copy kernel (copyBuffer) is given beside it.",
             "# Raw medians (KiB per dispatch): " + "; ".join(
                 "%s %s %.1f" % (c, lab, v / 1024.0)
                 for c in ("FETCH_SIZE", "WRITE_SIZE")
                 for k, v in res[c]["kernels"].items()
                 for lab in [next((kn for kn in labels if kn in k), None)]
                 if lab),
             "copy_bytes %d" % copy_bytes,
             "fetch_scale %.6f (copyBuffer %.6f)" % (res["FETCH_SIZE"]["scale"], res["FETCH_SIZE"]["scale_blit"]),
             "write_scale %.6f (copyBuffer %.6f)" % (res["WRITE_SIZE"]["scale"], res["WRITE_SIZE"]["scale_blit"])]
    for kind, kname in KERNEL_NAMES.items():
        f = [v for k, v in res["FETCH_SIZE"]["kernels"].items() if kname in k]
        w = [v for k, v in res["WRITE_SIZE"]["kernels"].items() if kname in k]
        if f and w:
            fb = f[0] * res["FETCH_SIZE"]["scale"]
            wb = w[0] * res["WRITE_SIZE"]["scale"]
            lines.append("kernel %s sha %s fetch_bytes %.0f write_bytes %.0f" % (kind, source_sha(kind), fb, wb))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _short_kernel(name):
    n = name.replace("pc::(anonymous namespace)::", "").replace("pc::", "")
    i = n.find("(")
    return n[:i] if i > 0 else n


def trace_summary(trace_dir, out, command, title=None, last=0):
    """Per-kernel lines (calls, average/min/max ns, share) from a
    rocprofv3 --kernel-trace --stats --output-format csv run; with ``last``,
    also the coder kernels' mean over their last ``last`` dispatches (the
    timed steps, after the settle and warmup steps)."""
    import csv

    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no kernel_stats.csv under " + trace_dir)
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
                         float(r["Percentage"]), _short_kernel(r["Name"])))
    rows.sort(key=lambda t: -t[4])
    lines = ["# " + (title or "rocprofv3 kernel trace of bench.py on the 1 GiB e4m3 stream (64 KiB chunks, Huffman-12)"),
             "# Command (from the repository root, after cd /tmp && export TMPDIR=/tmp):",
             "#   " + command,
             "#   python3 bench.py " + " ".join(shlex.quote(a) for a in sys.argv[1:]),
             "# Columns: calls, average ns, min ns, max ns, share of GPU time, kernel"]
    for c, avg, mn, mx, pct, name in rows[:12]:
        lines.append("%6d %10.0f %10.0f %10.0f %7.2f%%  %s" % (c, avg, mn, mx, pct, name[:90]))
    if last:
        tfiles = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
        durs = {}
        with open(tfiles[0]) as f:
            for r in csv.DictReader(f):
                for kind, kname in KERNEL_NAMES.items():
                    if kname in r["Kernel_Name"]:
                        durs.setdefault(kind, []).append(
                            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines.append("# Timed steps only (the last %d dispatches of each coder kernel): mean, min, max ns" % last)
        for kind, d in sorted(durs.items()):
            t = [v for _, v in sorted(d)[-last:]]
            lines.append("%6d %10.0f %10.0f %10.0f           %s" % (len(t), sum(t) / len(t), min(t), max(t),
                                                                 KERNEL_NAMES[kind]))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# SQ counters summed over the device per dispatch; *_CYCLES and LEVEL
# counters count in the SQ's own units (the ratios below only divide
# counters of the same kind).
SQ_RATIOS = [
    ("VALU instructions per wave", "SQ_INSTS_VALU", "SQ_WAVES"),
    ("LDS instructions per wave", "SQ_INSTS_LDS", "SQ_WAVES"),
    ("VMEM instructions per wave", "SQ_INSTS_VMEM", "SQ_WAVES"),
    ("SALU instructions per wave", "SQ_INSTS_SALU", "SQ_WAVES"),
    ("VALU-active share of wave cycles", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
    ("LDS-active share of wave cycles", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
    ("waiting-on-LDS share of wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
    ("waiting-on-anything share of wave cycles", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("LDS bank-conflict cycles per LDS-active cycle", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
]


def counter_summary(dirs, out, commands, title, self_cmd, ratios, shares=()):
    """Median per-dispatch counters of the coder kernels, from one or more
    rocprofv3 --pmc runs; `ratios` divides two counters, `shares` gives
    a / (a + b)."""
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError("no counter_collection.csv under " + d)
        import csv

        with open(files[0]) as f:
            for r in csv.DictReader(f):
                for kind, kname in KERNEL_NAMES.items():
                    if kname in r["Kernel_Name"]:
                        vals.setdefault(kind, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: {c: sorted(v)[len(v) // 2] for c, v in cs.items()} for k, cs in vals.items()}
    lines = list(title) + ["# Commands (from the repository root, after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["#   " + c for c in commands]
    lines.append("#   python3 bench.py " + self_cmd + " " + " ".join(dirs))
    kinds = [k for k in KERNEL_NAMES if k in med]
    counters = sorted({c for k in kinds for c in med[k]})
    lines.append("%-44s " % "counter" + " ".join("%18s" % k for k in kinds))
    for c in counters:
        lines.append("%-44s " % c + " ".join("%18.0f" % med[k].get(c, float("nan")) for k in kinds))
    for label, a, b in ratios:
        if all(a in med[k] and b in med[k] and med[k][b] for k in kinds):
            lines.append("%-44s " % label + " ".join("%18.4f" % (med[k][a] / med[k][b]) for k in kinds))
    for label, a, b in shares:
        if all(a in med[k] and b in med[k] and med[k][a] + med[k][b] for k in kinds):
            lines.append("%-44s " % label + " ".join("%18.4f" % (med[k][a] / (med[k][a] + med[k][b])) for k in kinds))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sq_summary(dirs, out, commands):
    """Median per-dispatch SQ counters of the coder kernels, and the ratios
    in SQ_RATIOS."""
    counter_summary(dirs, out, commands,
                    ["# SQ counters of the coder kernels on the 1 GiB e4m3 stream (64 KiB chunks, Huffman-12),",
                     "# median over dispatches, summed over the device."], "--sq-summary", SQ_RATIOS)


def l2_summary(dirs, out, commands):
    """Median per-dispatch L2 (TCC) hits and misses of the coder kernels."""
    counter_summary(dirs, out, commands,
                    ["# L2 (TCC) requests of the coder kernels on the 1 GiB e4m3 stream (64 KiB chunks, Huffman-12),",
                     "# median over dispatches, summed over the device's TCC channels."], "--l2-summary", [],
                    [("L2 hit share of requests", "TCC_HIT_sum", "TCC_MISS_sum")])


def load_traffic(kind):
    """Scaled HBM bytes per dispatch of `kind`, or None when absent/stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        p = line.split()
        if len(p) >= 8 and p[0] == "kernel" and p[1] == kind:
            if p[3] != source_sha(kind):
                return None
            return float(p[5]) + float(p[7])
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same stream.
# ---------------------------------------------------------------------------

def cpu_baseline_leg(x_np, counts_prev, kind, qlc_bits, chunk, gpu_streams, target_seconds, threads):
    """Time the oracle's bit-serial encoder and decoder on the first chunks
    of the stream and compare their outputs with the GPU's for those chunks."""
    import numpy as np

    from oracle import codebook as ocb
    from oracle import coder

    book = ocb.codebook([int(c) for c in counts_prev], kind, qlc_bits)
    nchunks_total = (x_np.size + chunk - 1) // chunk

    def run(nch):
        part = x_np[: min(nch * chunk, x_np.size)]
        t0 = time.perf_counter()
        s = coder.encode(part, book["lengths"], book["codes"], chunk, threads=threads)
        t1 = time.perf_counter()
        y, rc = coder.decode(s, part.size, chunk, book, threads=threads)
        t2 = time.perf_counter()
        return part, s, y, rc, t1 - t0, t2 - t1

    pilot = min(nchunks_total, max(threads, 8))
    part, s, y, rc, te, td = run(pilot)
    rate = part.size / max(te + td, 1e-6)
    want = int(min(nchunks_total, max(pilot, (target_seconds * rate) // chunk)))
    if want > pilot:
        part, s, y, rc, te, td = run(want)
    nch = (part.size + chunk - 1) // chunk
    cwo = gpu_streams["chunk_word_offset"][: nch + 1]
    words = int(cwo[nch])
    spc = chunk // 256
    nsub = s["sub_off"].size
    parity = {
        "chunks": int(nch),
        "payload_words_equal": bool(np.array_equal(gpu_streams["payload"](words), s["payload"])),
        "chunk_bits_equal": bool(np.array_equal(gpu_streams["chunk_bits"][:nch], s["chunk_bits"])),
        "chunk_word_offset_equal": bool(np.array_equal(cwo, s["chunk_word_offset"])),
        "sub_off_equal": bool(np.array_equal(gpu_streams["sub_off"][:nsub], s["sub_off"])),
        "oracle_round_trip": bool(rc == 0 and np.array_equal(y, part)),
    }
    del spc
    # one thread, on a smaller sample (about a second of work)
    n1 = int(min(x_np.size, max(chunk, (rate / max(threads, 1)) * 1.0 // chunk * chunk)))
    p1 = x_np[:n1]
    t0 = time.perf_counter()
    s1 = coder.encode(p1, book["lengths"], book["codes"], chunk, threads=1)
    t1 = time.perf_counter()
    coder.decode(s1, p1.size, chunk, book, threads=1)
    t2 = time.perf_counter()
    single = {"value": round(p1.size / (t2 - t0) / 1e9, 4), "bytes": int(p1.size),
              "encode_GBps": round(p1.size / (t1 - t0) / 1e9, 4), "decode_GBps": round(p1.size / (t2 - t1) / 1e9, 4)}
    return {
        "value": round(part.size / (te + td) / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "first %d of %d chunks (%d bytes) of the same stream; bit-serial C encode %.2f s + "
                  "decode %.2f s" % (nch, nchunks_total, part.size, te, td),
        "encode_GBps": round(part.size / te / 1e9, 4),
        "decode_GBps": round(part.size / td / 1e9, 4),
        "single_thread": single,
        "cpu_model": _cpu_model(),
    }, parity


def ms_stats(v):
    """mean, median, p10, p90, min and max of per-call times (ms)."""
    import numpy as np

    a = np.asarray(v, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4), "p90": round(float(np.percentile(a, 90)), 4),
            "min": round(float(a.min()), 4), "max": round(float(a.max()), 4)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------


def settle(fn, block=5, max_calls=80, tol=0.015):
    """Untimed calls of fn (the work about to be timed), in blocks of
    ``block``, until a block's mean time is no more than ``tol`` below the
    previous block's (or ``max_calls`` calls); returns the number of calls.
    On these GPUs the first ~25 encode/decode pairs after start-up, or after
    an idle gap, run up to 15-20% slower than the ones after them, whatever
    ran before (device copies and fp32 GEMMs as a first load do not remove
    it); the timed calls are meant to see the steady state."""
    import torch

    prev, calls = None, 0
    while calls < max_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(block):
            fn()
        e1.record()
        torch.cuda.synchronize()
        calls += block
        cur = e0.elapsed_time(e1) / block
        if prev is not None and cur >= prev * (1.0 - tol):
            break
        prev = cur
    return calls


def time_calls(fn, reps):
    """Mean milliseconds of fn() (device work, timed with events on the
    current stream) over reps calls after two warmup calls."""
    import torch

    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def qlc_leg(pc, W, dev):
    """The QLC codebook on the GELU tensor (64 MiB, 16 KiB chunks): encode,
    the generic 12-bit-peek decoder and the QLC decoder, with the QLC and
    Huffman-12 bits per symbol of the same tensor."""
    import numpy as np
    import torch

    w = W.WORKLOADS["gelu_act"]
    counts = torch.zeros(256, dtype=torch.int64, device=dev)
    for s in w.prev_seeds:
        pc.pc_histogram(torch.from_numpy(W.make(w.name, s)).to(dev), counts)
    counts_np = counts.cpu().numpy().astype(np.uint64)
    x = torch.from_numpy(W.make(w.name, 0)).to(dev)
    n = w.n
    book_q = pc.pc_codebook_build(counts_np, "qlc", w.qlc_bits)
    book_h = pc.pc_codebook_build(counts_np, "huffman")
    dq = book_q.to(dev)
    outs = pc.alloc_encode_outputs(n, w.chunk, dev)
    out = torch.empty(n, dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    settle(lambda: pc.pc_encode(dq, x, w.chunk, outs))
    enc_ms = time_calls(lambda: pc.pc_encode(dq, x, w.chunk, outs), 10)
    enc = pc.pc_encode(dq, x, w.chunk, outs)
    torch.cuda.synchronize()
    enc_ok = int(enc.status.item()) == 0
    settle(lambda: pc.pc_decode(dq, enc, out=out, status=st))
    dec_ms = time_calls(lambda: pc.pc_decode(dq, enc, out=out, status=st), 10)
    ok_lut = int(st.item()) == 0 and bool(torch.equal(out, x))
    st.zero_()
    settle(lambda: pc.pc_decode_qlc(dq, enc, out=out, status=st))
    qdec_ms = time_calls(lambda: pc.pc_decode_qlc(dq, enc, out=out, status=st), 10)
    ok_qlc = int(st.item()) == 0 and bool(torch.equal(out, x))
    xc = pc.pc_histogram(x).cpu().numpy().astype(np.float64)
    lq = pc.codebook_fields(book_q)["length"].astype(np.float64)
    lh = pc.codebook_fields(book_h)["length"].astype(np.float64)
    ls = pc.pc_shard_code_lengths(xc.astype(np.uint64)).astype(np.float64)
    p = xc[xc > 0] / n
    H = float(-(p * np.log2(p)).sum())
    bq, bh, bs = (float((xc * l).sum()) / n for l in (lq, lh, ls))
    return {"n_bytes": n, "chunk": w.chunk, "qlc_bits": list(w.qlc_bits),
            "encode_GBps": round(n / (enc_ms * 1e-3) / 1e9, 1),
            "decode_lut12_GBps": round(n / (dec_ms * 1e-3) / 1e9, 1),
            "decode_qlc_GBps": round(n / (qdec_ms * 1e-3) / 1e9, 1),
            "round_trip_ok": bool(enc_ok and ok_lut and ok_qlc),
            "bits_per_symbol": {"qlc": round(bq, 5), "huffman12_same_counts": round(bh, 5),
                                "huffman12_own_counts": round(bs, 5), "entropy": round(H, 5),
                                "qlc_compressibility": round(1 - bq / 8, 5),
                                "huffman12_compressibility": round(1 - bh / 8, 5)}}


def stream_stats(pc, x, enc, n, chunk):
    """Bits/symbol of an encoded stream: payload, with the side index and
    chunk tables, order-0 entropy, and the per-shard Huffman-12 comparator
    (absent byte values excluded)."""
    import numpy as np

    nc = pc.pc_num_chunks(n, chunk)
    nsub = pc.pc_num_substreams(n, chunk)
    cbits = enc.chunk_bits.cpu().numpy().view(np.uint32).astype(np.int64)
    words = int(enc.chunk_word_offset[nc].item())
    xc = pc.pc_histogram(x).cpu().numpy().astype(np.float64)
    p = xc[xc > 0] / n
    H = float(-(p * np.log2(p)).sum())
    shard_len = pc.pc_shard_code_lengths(xc.astype(np.uint64)).astype(np.float64)
    shard = float((xc * shard_len).sum()) / n
    b = float(cbits.sum()) / n
    return {"payload": round(b, 5), "with_side_index": round((words * 32 + 32 * nsub + 96 * nc) / n, 5),
            "entropy": round(H, 5), "per_shard_huffman12": round(shard, 5),
            "gap_vs_entropy_rel": round(b / H - 1, 5), "gap_vs_per_shard_rel": round(b / shard - 1, 5),
            "compressibility": round(1 - b / 8, 5)}, words


def config_leg(pc, W, name, dev, reps, decoders):
    """One benchmark configuration: encode and decode times (HIP events on the
    launch stream, per call), GB/s of uncompressed bytes, HBM roofline
    fraction on algorithmic bytes, bits/symbol.  Returns the report and the
    device outputs (for the oracle comparison of the cpu_baseline leg)."""
    import numpy as np
    import torch

    w = W.WORKLOADS[name]
    counts = torch.zeros(256, dtype=torch.int64, device=dev)
    for s in w.prev_seeds:
        pc.pc_histogram(torch.from_numpy(W.make(name, s)).to(dev), counts)
    counts_np = counts.cpu().numpy().astype(np.uint64)
    x_np = W.make(name, 0)
    x = torch.from_numpy(x_np).to(dev)
    n, chunk = w.n, w.chunk
    dcb = pc.pc_codebook_build(counts_np, w.kind, w.qlc_bits).to(dev)
    outs = pc.alloc_encode_outputs(n, chunk, dev)
    out = torch.empty(n, dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn):
        settle(fn)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    enc_ms = timed(lambda: pc.pc_encode(dcb, x, chunk, outs))
    enc = pc.pc_encode(dcb, x, chunk, outs)
    torch.cuda.synchronize()
    enc_ok = int(enc.status.item()) == 0
    bits, words = stream_stats(pc, x, enc, n, chunk)
    alg = n + words * 4 + 4 * pc.pc_num_substreams(n, chunk) + 12 * pc.pc_num_chunks(n, chunk) + 8
    rep = {"n_bytes": n, "chunk": chunk, "codebook": w.kind, "qlc_bits": list(w.qlc_bits) if w.qlc_bits else None,
           "algorithmic_bytes": alg, "encode": None, "decode": {}, "bits_per_symbol": bits}

    def line(ms):
        med = float(np.median(ms))
        return {"ms": ms_stats(ms), "GBps": round(n / (med * 1e-3) / 1e9, 1),
                "roofline_frac": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    rep["encode"] = line(enc_ms)
    rep["encode"]["status_ok"] = enc_ok
    for dname in decoders:
        fn = pc.pc_decode_qlc if dname == "qlc" else pc.pc_decode
        st.zero_()
        dec_ms = timed(lambda: fn(dcb, enc, out=out, status=st))
        torch.cuda.synchronize()
        rep["decode"][dname] = line(dec_ms)
        rep["decode"][dname]["round_trip_ok"] = bool(int(st.item()) == 0 and torch.equal(out, x))
    host = {"payload": enc.payload[:words].cpu().numpy().view(np.uint32).copy(),
            "chunk_bits": enc.chunk_bits.cpu().numpy().view(np.uint32).copy(),
            "chunk_word_offset": enc.chunk_word_offset.cpu().numpy().view(np.uint64).copy(),
            "sub_off": enc.sub_off.cpu().numpy().view(np.uint32).copy()}
    return rep, (x_np, counts_np, w.kind, w.qlc_bits, chunk, host)


def oracle_parity(case, threads):
    """Part of the cpu_baseline leg: the oracle's bit-serial coder on a whole
    configuration, every array compared with the GPU's."""
    import numpy as np

    from oracle import codebook as ocb
    from oracle import coder

    x_np, counts, kind, qlc_bits, chunk, host = case
    book = ocb.codebook([int(c) for c in counts], kind, qlc_bits)
    s = coder.encode(x_np, book["lengths"], book["codes"], chunk, threads=threads)
    y, rc = coder.decode(s, x_np.size, chunk, book, threads=threads)
    return {k: bool(np.array_equal(host[k], s[k])) for k in ("payload", "chunk_bits", "chunk_word_offset", "sub_off")} | \
        {"oracle_round_trip": bool(rc == 0 and np.array_equal(y, x_np))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stream_1g")
    ap.add_argument("--decoder", default="lut12", choices=["lut12", "qlc"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--trace-summary", metavar="TRACE_DIR")
    ap.add_argument("--trace-command", default="")
    ap.add_argument("--trace-out", default="coder_kernels_stream_1g_kernel_trace.txt")
    ap.add_argument("--trace-title", default=None)
    ap.add_argument("--trace-last", type=int, default=0,
                    help="with --trace-summary: also the mean of each coder kernel's last N dispatches")
    ap.add_argument("--sq-summary", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--l2-summary", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--sq-commands", nargs="*", default=[],
                    help="with --sq-summary or --l2-summary: the profiler commands, recorded in the file")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the QLC (GELU tensor) and histogram measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration lines (configurations 1-4)")
    ap.add_argument("--config-reps", type=int, default=20)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.trace_summary:
        trace_summary(args.trace_summary, os.path.join(ROOT, "profiles", os.path.basename(args.trace_out)),
                      args.trace_command, args.trace_title, args.trace_last)
        return 0
    if args.sq_summary:
        sq_summary(args.sq_summary, os.path.join(ROOT, "profiles", "coder_kernels_stream_1g_sq_counters.txt"),
                   args.sq_commands)
        return 0
    if args.l2_summary:
        l2_summary(args.l2_summary, os.path.join(ROOT, "profiles", "coder_kernels_stream_1g_l2_hits.txt"),
                   args.sq_commands)
        return 0
    if args.pmc_summary:
        import workloads as W

        cb = args.copy_bytes or W.WORKLOADS[args.workload].n
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], cb)
        return 0
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this coder needs no second device and no figure at "
              "several GPUs is measured (asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import static_codebook_lossless_amd as pc
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    n, chunk = w.n, w.chunk

    # ---- inputs (host synthesis, then resident in HBM) -----------------
    log("generating %s (%d bytes) and %d previous batch(es)" % (w.name, n, len(w.prev_seeds)))
    t0 = time.perf_counter()
    counts_dev = torch.zeros(256, dtype=torch.int64, device=dev)
    for s in w.prev_seeds:
        prev = torch.from_numpy(W.make(w.name, s)).to(dev)
        pc.pc_histogram(prev, counts_dev)  # pooled counts of previous batches
        del prev
    counts_prev = counts_dev.cpu().numpy().astype(np.uint64)
    x_np = W.make(w.name, 0)
    x = torch.from_numpy(x_np).to(dev)
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))

    blob = pc.pc_codebook_build(counts_prev, w.kind, w.qlc_bits)
    dcb = blob.to(dev)
    fields = pc.codebook_fields(blob)
    outs = pc.alloc_encode_outputs(n, chunk, dev)
    dec_out = torch.empty(n, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    decode = pc.pc_decode_qlc if args.decoder == "qlc" else pc.pc_decode

    def step(evs=None):
        if evs:
            evs[0].record()
        enc = pc.pc_encode(dcb, x, chunk, outs)
        if evs:
            evs[1].record()
        decode(dcb, enc, out=dec_out, status=status)
        if evs:
            evs[2].record()
        return enc

    settle_steps = settle(step)
    log("settled after %d untimed steps" % settle_steps)
    # plain device copy of the input: context for the roofline
    cpy = torch.empty_like(x)
    for _ in range(3):
        cpy.copy_(x)
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    for _ in range(5):
        cpy.copy_(x)
    ce1.record()
    torch.cuda.synchronize()
    copy_GBps = 2 * n * 5 / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    # the same copy through the coder kernels' own 16-byte non-temporal loads
    # and stores (calibrates the hardware traffic counters, see pmc_summary)
    n16 = n // 16 * 16
    for _ in range(2):
        pc.pc_traffic_probe(x[:n16], cpy[:n16])
    ce0.record()
    for _ in range(5):
        pc.pc_traffic_probe(x[:n16], cpy[:n16])
    ce1.record()
    torch.cuda.synchronize()
    probe_GBps = 2 * n16 * 5 / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del cpy

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        enc = step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        enc = step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps

    # ---- checks and stream statistics ---------------------------------
    st = int(status.item())
    est = int(enc.status.item())
    same = bool(torch.equal(dec_out, x))
    if st != 0 or est != 0 or not same:
        log("ROUND TRIP FAILED: encode status %d, decode status %d, equal %s" % (est, st, same))
    nc = pc.pc_num_chunks(n, chunk)
    nsub = pc.pc_num_substreams(n, chunk)
    cbits = enc.chunk_bits.cpu().numpy().view(np.uint32).astype(np.int64)
    cwo = enc.chunk_word_offset.cpu().numpy().view(np.uint64)
    words = int(cwo[nc])
    payload_bits = int(cbits.sum())
    xcounts = pc.pc_histogram(x).cpu().numpy().astype(np.float64)
    p = xcounts[xcounts > 0] / n
    H = float(-(p * np.log2(p)).sum())
    # per-shard comparator: a 12-bit Huffman code on the stream's own counts,
    # absent byte values excluded
    shard_len = pc.pc_shard_code_lengths(xcounts.astype(np.uint64)).astype(np.float64)
    shard_bits = float((xcounts * shard_len).sum()) / n
    b_payload = payload_bits / n
    b_total = (words * 32 + 32 * nsub + 96 * nc) / n

    # ---- roofline of the slower kernel --------------------------------
    payload_bytes = words * 4
    side_bytes = 4 * nsub + 12 * nc + 8
    alg = {"encode": n + payload_bytes + side_bytes, "decode": payload_bytes + side_bytes + n}
    avg = {"encode": sum(enc_ms) / len(enc_ms), "decode": sum(dec_ms) / len(dec_ms)}
    dom = max(avg, key=avg.get)
    achieved = alg[dom] / (avg[dom] * 1e-3) / 1e9
    traffic = load_traffic(dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": alg[dom], "avg_ms": round(avg[dom], 4),
                # against what a plain device copy reaches on the same GPU
                "frac_of_device_copy": round(achieved / copy_GBps, 4)}
    other = "decode" if dom == "encode" else "encode"
    other_ach = alg[other] / (avg[other] * 1e-3) / 1e9

    # ---- CPU baseline (oracle), rank 0 at N=1 -------------------------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(os.cpu_count() or 1, 16)
        host_streams = {
            "payload": lambda m: enc.payload[:m].cpu().numpy().view(np.uint32),
            "chunk_bits": cbits.astype(np.uint32),
            "chunk_word_offset": cwo,
            "sub_off": enc.sub_off.cpu().numpy().view(np.uint32),
        }
        log("cpu baseline: oracle on a bounded sample (%d threads)" % threads)
        cpu, parity = cpu_baseline_leg(x_np, counts_prev, w.kind, w.qlc_bits, chunk, host_streams,
                                       args.cpu_seconds, threads)

    per_config = None
    if not args.no_configs:
        per_config = {}
        cases = {}
        for name in W.CONFIG_ORDER:
            if name == w.name:
                continue
            log("config %s" % name)
            decs = ["lut12", "qlc"] if W.WORKLOADS[name].kind == "qlc" else ["lut12"]
            per_config[name], cases[name] = config_leg(pc, W, name, dev, args.config_reps, decs)
        if not args.no_cpu_baseline:
            threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(os.cpu_count() or 1, 16)
            for name, case in cases.items():
                log("oracle parity %s" % name)
                per_config[name]["oracle_parity"] = oracle_parity(case, threads)
        del cases
        per_config[w.name] = {"n_bytes": n, "chunk": chunk, "headline": True,
                              "encode": {"ms": ms_stats(enc_ms), "GBps": round(n / (avg["encode"] * 1e-3) / 1e9, 1),
                                         "roofline_frac": round(alg["encode"] / (avg["encode"] * 1e-3) / 1e9 /
                                                                HBM_PEAK_GBPS, 4)},
                              "decode": {args.decoder: {"ms": ms_stats(dec_ms),
                                                        "GBps": round(n / (avg["decode"] * 1e-3) / 1e9, 1),
                                                        "roofline_frac": round(alg["decode"] / (avg["decode"] * 1e-3)
                                                                               / 1e9 / HBM_PEAK_GBPS, 4)}},
                              "oracle_parity": parity}

    secondary = None
    if not args.no_secondary:
        settle(lambda: pc.pc_histogram(x))
        hist_ms = time_calls(lambda: pc.pc_histogram(x), 10)
        secondary = {"histogram_GBps": round(n / (hist_ms * 1e-3) / 1e9, 1)}
        secondary["qlc_gelu_act"] = qlc_leg(pc, W, dev)

    res = {
        "metric": "encode+decode GB/s (uncompressed bytes per round trip), 1 MI355X",
        "value": round(n / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": w.name, "n_bytes": n, "chunk": chunk, "codebook": w.kind,
                   "qlc_bits": list(w.qlc_bits) if w.qlc_bits else None, "decoder": args.decoder,
                   "description": w.description},
        "encode_GBps": round(n / (avg["encode"] * 1e-3) / 1e9, 1),
        "decode_GBps": round(n / (avg["decode"] * 1e-3) / 1e9, 1),
        "encode_ms": ms_stats(enc_ms),
        "decode_ms": ms_stats(dec_ms),
        "roofline": roofline,
        "roofline_other": {"kernel": other, "achieved": round(other_ach, 1),
                           "frac": round(other_ach / HBM_PEAK_GBPS, 4),
                           "frac_of_device_copy": round(other_ach / copy_GBps, 4)},
        "device_copy_GBps": round(copy_GBps, 1),
        "probe_copy_GBps": round(probe_GBps, 1),
        "bits_per_symbol": {"payload": round(b_payload, 5), "with_side_index": round(b_total, 5),
                            "entropy": round(H, 5), "per_shard_huffman12": round(shard_bits, 5),
                            "gap_vs_entropy_rel": round(b_payload / H - 1, 5),
                            "gap_vs_per_shard_rel": round(b_payload / shard_bits - 1, 5),
                            "compressibility": round(1 - b_payload / 8, 5),
                            "entropy_compressibility": round(1 - H / 8, 5)},
        "codebook_id": "%08x" % fields["codebook_id"],
        "round_trip_ok": bool(st == 0 and est == 0 and same),
        "cpu_baseline": cpu,
        "oracle_parity_sample": parity,
        "per_config": per_config,
        "secondary": secondary,
    }
    print(json.dumps(res), flush=True)
    ok = st == 0 and est == 0 and same and (parity is None or all(v for k, v in parity.items() if k != "chunks"))
    for name, c in (per_config or {}).items():
        if c.get("headline"):
            continue
        ok = ok and c["encode"]["status_ok"] and all(d["round_trip_ok"] for d in c["decode"].values())
        ok = ok and all(c.get("oracle_parity", {}).values())
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
