"""Bit-exact parity of the HIP path with the oracle (needs an MI355X).

Every comparison is element by element: payload words, chunk bit counts,
chunk word offsets, side index and decoded bytes.  The oracle's codebook (not
the library's) drives the oracle's encoder, so a codebook mismatch also
fails here.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import codebook as cb
from oracle import coder

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import static_codebook_lossless_amd as pc

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make_book(counts, kind="huffman", bits=None):
    counts = [int(c) for c in counts]
    blob = pc.pc_codebook_build(np.array(counts, dtype=np.uint64), kind, bits)
    oracle_book = cb.codebook(counts, kind, bits)
    return blob.to(DEV), oracle_book


def gpu_encode(dcb, x_np, chunk):
    x = torch.from_numpy(x_np).to(DEV)
    enc = pc.pc_encode(dcb, x, chunk)
    torch.cuda.synchronize()
    assert int(enc.status.item()) == pc.PC_OK
    return x, enc


def host(enc):
    nc = pc.pc_num_chunks(enc.n, enc.chunk)
    cwo = enc.chunk_word_offset.cpu().numpy().view(np.uint64)
    total = int(cwo[nc]) if enc.n else 0
    return {
        "payload": enc.payload[:total].cpu().numpy().view(np.uint32),
        "chunk_bits": enc.chunk_bits.cpu().numpy().view(np.uint32),
        "chunk_word_offset": cwo,
        "sub_off": enc.sub_off.cpu().numpy().view(np.uint32),
    }


def assert_same_stream(got, want):
    for k in ("chunk_bits", "chunk_word_offset", "sub_off", "payload"):
        a, b = np.asarray(got[k]), np.asarray(want[k]).astype(np.asarray(got[k]).dtype)
        assert a.shape == b.shape, (k, a.shape, b.shape)
        if not np.array_equal(a, b):
            i = int(np.flatnonzero(a != b)[0])
            raise AssertionError("%s differs first at %d: %d vs %d" % (k, i, int(a[i]), int(b[i])))


def roundtrip(dcb, obook, x_np, chunk, qlc_decoder=False):
    x, enc = gpu_encode(dcb, x_np, chunk)
    got = host(enc)
    want = coder.encode(x_np, obook["lengths"], obook["codes"], chunk, threads=8)
    assert_same_stream(got, want)
    out, status = pc.pc_decode(dcb, enc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, x)
    if qlc_decoder:
        out2, status2 = pc.pc_decode_qlc(dcb, enc)
        torch.cuda.synchronize()
        assert int(status2.item()) == 0
        assert torch.equal(out2, x)
    return enc


@pytest.mark.parametrize("name", ["normal_1m", "ffn1_act", "gelu_act", "int8_weight"])
def test_workload_parity(name):
    w = W.WORKLOADS[name]
    say("workload parity:", name)
    x_np = W.make(name, 0)
    counts = np.zeros(256, dtype=np.int64)
    for s in w.prev_seeds:
        counts += np.bincount(W.make(name, s), minlength=256)
    dcb, obook = make_book(counts, w.kind, w.qlc_bits)
    roundtrip(dcb, obook, x_np, w.chunk, qlc_decoder=(w.kind == "qlc"))


def test_stream_1g_full_size():
    """The 1 GiB stream in the benchmark's launch configuration, compared in
    full: every chunk's payload words, bit count, word offset and side index
    against the oracle (its bit-serial coder on 16 host threads), and the
    decoded bytes against the input."""
    name = "stream_1g"
    w = W.WORKLOADS[name]
    say("stream_1g: generating")
    prev = W.make(name, 1)
    counts = np.bincount(prev, minlength=256)
    del prev
    dcb, obook = make_book(counts)
    x_np = W.make(name, 0)
    say("stream_1g: encode")
    x, enc = gpu_encode(dcb, x_np, w.chunk)
    say("stream_1g: decode")
    out, status = pc.pc_decode(dcb, enc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, x)
    del out
    say("stream_1g: oracle encode of all", pc.pc_num_chunks(x_np.size, w.chunk), "chunks")
    want = coder.encode(x_np, obook["lengths"], obook["codes"], w.chunk, threads=16)
    say("stream_1g: compare")
    assert_same_stream(host(enc), want)
    xc = np.bincount(x_np, minlength=256)
    assert int(host(enc)["chunk_bits"].astype(np.int64).sum()) == cb.coded_bits(xc, obook["lengths"])


def test_large_qlc_stream_both_decoders():
    """A 300 MB stream under a QLC code (an incomplete code: both decoders
    test every codeword for validity) at the size where the decoders stream
    their second-half loads and output stores: the whole stream against the
    oracle, and both decoders back to the input."""
    bits = (1, 3, 3, 3, 3, 5, 6, 7)
    n = 300_000_000 + 123
    say("large QLC stream: generating", n)
    x_np = skewed(n, 71)
    dcb, obook = make_book(np.bincount(x_np[: 1 << 24], minlength=256), "qlc", bits)
    assert pc.codebook_fields(dcb)["complete"] == 0  # Kraft sum 511/512
    x, enc = gpu_encode(dcb, x_np, 65536)
    say("large QLC stream: oracle encode")
    want = coder.encode(x_np, obook["lengths"], obook["codes"], 65536, threads=16)
    assert_same_stream(host(enc), want)
    del want
    for name, fn in (("pc_decode", pc.pc_decode), ("pc_decode_qlc", pc.pc_decode_qlc)):
        say("large QLC stream:", name)
        out, status = fn(dcb, enc)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(out, x)
        del out


@pytest.mark.parametrize("units_per_cu", [2, 3])
def test_unit_path_few_units(units_per_cu):
    """64 KiB chunks take the persistent unit encoder from one unit per
    workgroup on: exactly one unit each, then one or two, with units of long
    codes that go out in two halves and a short chunk left over; compared in
    full with the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = units_per_cu * cus * 65536 + 1000
    counts = random_counts(9)
    dcb, obook = make_book(counts)
    long_syms = np.flatnonzero(np.asarray(obook["lengths"]) >= 10).astype(np.uint8)
    say("unit path, few units: per CU", units_per_cu, "n", n)
    x_np = skewed(n, 300 + units_per_cu)
    rng = np.random.default_rng(units_per_cu)
    for u in (0, 5, units_per_cu * cus - 1):
        x_np[u * 65536:(u + 1) * 65536] = rng.choice(long_syms, 65536)
    roundtrip(dcb, obook, x_np, 65536)


@pytest.mark.parametrize("chunk", [65536, 32768, 16384, 8192, 4096, 2048, 1024])
def test_persistent_unit_path(chunk):
    """Inputs large enough for the persistent 64 KiB-unit encoder (four
    units per workgroup at two workgroups per CU), with whole chunks and a
    short chunk left over for the re-reading kernel, and units of symbols
    whose codes are 10 bits or longer (more than the buffer holds at once,
    so they go out in two halves), compared in full with the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = 8 * cus * 65536 + 3 * chunk + 100
    counts = random_counts(7)
    dcb, obook = make_book(counts)
    lengths = np.asarray(obook["lengths"])
    long_syms = np.flatnonzero(lengths >= 10).astype(np.uint8)
    assert long_syms.size > 0
    say("unit path: chunk", chunk, "n", n, "long symbols", long_syms.size)
    x_np = skewed(n, chunk)
    rng = np.random.default_rng(chunk)
    for u in (1, 37, 8 * cus - 1):  # whole 64 KiB units of long codes
        x_np[u * 65536:(u + 1) * 65536] = rng.choice(long_syms, 65536)
    x, enc = gpu_encode(dcb, x_np, chunk)
    got = host(enc)
    cwo = got["chunk_word_offset"].astype(np.int64)
    per = 65536 // chunk
    assert (cwo[38 * per] - cwo[37 * per]) > 16384  # that unit did not fit
    want = coder.encode(x_np, obook["lengths"], obook["codes"], chunk, threads=16)
    assert_same_stream(got, want)
    out, status = pc.pc_decode(dcb, enc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, x)


@pytest.mark.parametrize("chunk", [1 << 17, 1 << 20, 1 << 24])
def test_multi_unit_chunks(chunk):
    """Chunks of several 64 KiB units (count, scan and place launches, units
    joined mid-word with atomic ORs on the shared words), with a short last
    chunk for the re-reading kernel, and 64 KiB runs of long codes (units
    that go out in two halves) at a chunk's start, inside, and at its end;
    compared in full with the oracle, and decoded back."""
    n = (2 if chunk == 1 << 24 else 3) * chunk + 1000
    dcb, obook = make_book(random_counts(5))
    long_syms = np.flatnonzero(np.asarray(obook["lengths"]) >= 10).astype(np.uint8)
    x_np = skewed(n, chunk + 1)
    rng = np.random.default_rng(chunk)
    U = chunk // 65536
    for u in (0, U // 2 + 1, 2 * U - 1):  # whole units of long codes
        x_np[u * 65536:(u + 1) * 65536] = rng.choice(long_syms, 65536)
    say("multi-unit chunks: chunk", chunk, "n", n)
    x, enc = gpu_encode(dcb, x_np, chunk)
    want = coder.encode(x_np, obook["lengths"], obook["codes"], chunk, threads=16)
    assert_same_stream(host(enc), want)
    out, status = pc.pc_decode(dcb, enc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, x)


def skewed(n, seed):
    rng = np.random.default_rng(seed)
    return ((rng.zipf(1.4, n) * 37) % 256).astype(np.uint8)


def random_counts(seed):
    rng = np.random.default_rng(1000 + seed)
    return (rng.pareto(1.1, 256) * 1000).astype(np.int64)


@pytest.mark.parametrize("chunk", [256, 768, 4096, 8192, 16384, 32768, 65536, 131072])
def test_edge_sizes(chunk):
    """Sizes around one chunk, and runs of chunks that fill the multi-chunk
    workgroups (up to 8 chunks each) exactly, or leave whole chunks and a
    short chunk over for the re-reading kernel."""
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7))):
        dcb, obook = make_book(random_counts(chunk), kind, bits)
        sizes = sorted({0, 1, 255, 256, 257, chunk - 1, chunk, chunk + 1, 3 * chunk + 100, 8 * chunk,
                        11 * chunk + 100})
        for n in sizes:
            say("edge size:", kind, "chunk", chunk, "n", n)
            x_np = skewed(n, n + chunk)
            if n == 0:
                x = torch.empty(0, dtype=torch.uint8, device=DEV)
                enc = pc.pc_encode(dcb, x, chunk)
                torch.cuda.synchronize()
                assert int(enc.chunk_word_offset[0].item()) == 0
                assert int(enc.status.item()) == pc.PC_OK
                out, status = pc.pc_decode(dcb, enc)
                torch.cuda.synchronize()
                assert out.numel() == 0 and int(status.item()) == 0
                continue
            roundtrip(dcb, obook, x_np, chunk, qlc_decoder=(kind == "qlc"))


def test_group_boundaries():
    """Sizes around whole groups of 256 sub-streams (65536 symbols): full
    groups and a ragged last group take different decode kernels.  QLC
    layouts with shrinking and with empty areas move the codeword of rank
    256, which bounds the QLC decoder's valid windows."""
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7)), ("qlc", (5, 4, 3, 3, 3, 3, 3, 8)),
                       ("qlc", (0, 0, 1, 2, 4, 6, 7, 7))):
        dcb, obook = make_book(random_counts(21), kind, bits)
        for chunk in (4096, 65536):
            for n in (65535, 65536, 65537, 2 * 65536 - 256, 2 * 65536 + 255, 2 * 65536 + 256, 3 * 65536):
                say("group boundary:", kind, "chunk", chunk, "n", n)
                roundtrip(dcb, obook, skewed(n, n), chunk, qlc_decoder=(kind == "qlc"))


def test_full_groups_tight_payload():
    """Whole groups only, decoded with payload_words equal to the payload's
    exact length: the last sub-streams' LDS segments reach past the end of
    the payload, so their loads are clamped to its last four words and
    written at their true positions; nothing outside [0, n) is written."""
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7))):
        dcb, obook = make_book(random_counts(29), kind, bits)
        for chunk in (4096, 65536):
            for n in (65536, 3 * 65536):
                x_np = skewed(n, n + chunk)
                say("tight payload:", kind, "chunk", chunk, "n", n)
                x, enc = gpu_encode(dcb, x_np, chunk)
                total = int(enc.chunk_word_offset[-1].item())
                for qlc in ((False, True) if kind == "qlc" else (False,)):
                    out, st = decode_guarded(dcb, enc, total, qlc=qlc)
                    assert st == 0
                    assert torch.equal(out, x)


def light(n, seed):
    """e4m3 of N(0,1): about 6.5 bits per symbol under a code built for it
    (the density of the 1 GiB benchmark stream)."""
    rng = np.random.default_rng(seed)
    return W.e4m3_from_f32(rng.standard_normal(max(n, 1), dtype=np.float32))[:n]


def light_book(kind="huffman", bits=None):
    return make_book(np.bincount(light(1 << 20, 99), minlength=256), kind, bits)


def test_light_group_boundaries():
    """Streams of about 6.5 bits per symbol at sizes off the 65536-symbol
    group grid (steps of 81920 symbols, ragged ends): full groups decoded out
    of the LDS segments, the ragged last group from global memory."""
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7))):
        dcb, obook = light_book(kind, bits)
        for chunk in (4096, 65536):
            for n in (65536 + 100, 81919, 81920, 81921, 2 * 81920 - 256, 2 * 81920 + 255, 3 * 81920,
                      5 * 81920 + 77):
                x_np = light(n, n)
                say("light group boundary:", kind, "chunk", chunk, "n", n)
                enc = roundtrip(dcb, obook, x_np, chunk, qlc_decoder=(kind == "qlc"))
                if kind == "huffman" and n >= 81920:
                    assert int(host(enc)["chunk_bits"].astype(np.int64).sum()) < 6.9 * n


def test_dense_and_light_segments():
    """Segments of 81920 symbols, light data with every k-th segment uniform
    random bytes (about 11 bits per symbol under the light code, so their
    halves overflow the 40-word LDS segments and their groups are decoded
    again from global memory): one in 40 and one in 6 such segments, i.e. a
    stream below and one above 6.9 bits per symbol on average."""
    dcb, obook = light_book()
    rng = np.random.default_rng(5)
    for every, want_light in ((40, True), (6, False)):
        segs = [rng.integers(0, 256, 81920, dtype=np.uint8) if i % every == every - 1 else light(81920, 500 + i)
                for i in range(90)]
        x_np = np.concatenate(segs + [light(999, 3)])
        say("dense and light segments: dense segment every", every)
        enc = roundtrip(dcb, obook, x_np, 16384)
        bps = host(enc)["chunk_bits"].astype(np.int64).sum() / x_np.size
        say("dense and light segments: %.3f bits per symbol" % bps)
        assert (bps <= 6.9) == want_light


def test_many_chunks_lookback():
    """Tens of thousands of small chunks: stresses the cross-chunk scan."""
    dcb, obook = make_book(random_counts(3))
    x_np = skewed(40000 * 256 + 77, 5)
    say("lookback stress: 40001 chunks of 256")
    roundtrip(dcb, obook, x_np, 256)


@pytest.mark.parametrize("chunk", [4096, 8192])
def test_many_small_chunks(chunk):
    """8195 chunks and a short one: enough small chunks for the encoder's
    multi-chunk workgroups (32K symbols each) with whole chunks and a short
    chunk left over.  Every fifth 32K block is uniform bytes (~9.8 bits per
    symbol under this code), so those workgroups' output overflows the LDS
    buffer and takes the tile-by-tile path."""
    dcb, obook = make_book(np.bincount(skewed(1 << 20, 99), minlength=256))  # ~4.9 bits on skewed data
    n = 8195 * chunk + 100
    x_np = skewed(n, 12)
    blocks = x_np[: (n // 32768) * 32768].reshape(-1, 32768)
    rng = np.random.default_rng(13)
    blocks[::5] = rng.integers(0, 256, blocks[::5].shape, dtype=np.uint8)
    say("many small chunks:", chunk, "n", n)
    roundtrip(dcb, obook, x_np, chunk)


@pytest.mark.parametrize("chunk", [256, 512, 768, 1024, 2048, 3072, 12288, 20480, 32512])
def test_small_chunks_several_per_workgroup(chunk):
    """Chunks below 32 KiB that no specialised encoder takes (not a power of
    two, or a power of two below 4 KiB on a small input) go K to a workgroup
    (K * chunk <= 64 KiB, K <= 64): three and a half workgroups' worth of
    skewed data, then whole chunks and a short chunk for the re-reading
    kernel; then a run where every other chunk is uniform bytes (about 10
    bits per symbol under this code, so tiles span the most words), and one
    of 2 MB."""
    dcb, obook = make_book(np.bincount(skewed(1 << 20, 98), minlength=256))
    K = min(64, 65536 // chunk)
    rng = np.random.default_rng(chunk)
    n = 3 * K * chunk + (K // 2) * chunk + 5 * chunk + 100
    say("several chunks per workgroup:", chunk, "K", K, "n", n)
    roundtrip(dcb, obook, skewed(n, chunk + 1), chunk)
    x_np = skewed(n, chunk + 2)
    for c in range(0, n // chunk, 2):
        x_np[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    say("several chunks per workgroup, mixed:", chunk)
    roundtrip(dcb, obook, x_np, chunk)
    n2 = 2_000_000
    say("several chunks per workgroup, 2 MB:", chunk)
    roundtrip(dcb, obook, skewed(n2, chunk + 3), chunk)


@pytest.mark.parametrize("kind", ["huffman", "qlc"])
def test_degenerate_data(kind):
    bits = (1, 3, 3, 3, 3, 5, 6, 7) if kind == "qlc" else None
    counts = np.zeros(256, dtype=np.int64)
    counts[:40] = np.arange(40, 0, -1) * 1000  # most byte values never seen
    dcb, obook = make_book(counts, kind, bits)
    lengths = np.array(obook["lengths"])
    cases = {
        "one_frequent_symbol": np.full(100_000, 0, np.uint8),
        "one_rare_symbol": np.full(100_000, int(np.argmax(lengths)), np.uint8),
        "uniform": np.tile(np.arange(256, dtype=np.uint8), 400),
        "unseen_symbols_only": np.arange(40, 256, dtype=np.uint8).repeat(300),
        # whole groups of 65536 symbols: a compressible one (decoded out of
        # the LDS segments), two of 12-bit codewords (halves too long for a
        # segment: decoded from global memory), a ragged tail
        "segment_and_global_groups": np.concatenate([
            np.tile(np.arange(40, dtype=np.uint8), 1639)[:65536],
            np.tile(np.arange(40, 256, dtype=np.uint8), 607)[:131072],
            np.arange(40, dtype=np.uint8).repeat(25)]),
    }
    for cname, x_np in cases.items():
        say("degenerate:", kind, cname)
        roundtrip(dcb, obook, x_np, 4096, qlc_decoder=(kind == "qlc"))


@pytest.mark.parametrize("chunk", [4096, 8192, 16384, 32768, 65536])
def test_incompressible_data(chunk):
    """Uniform random bytes under the code of their own (flat) histogram: 8
    bits per symbol (a half of 128 symbols takes 32 of a segment's 40
    words), and with two byte values made rarer, 9-bit codes for some
    symbols."""
    rng = np.random.default_rng(77)
    n = 3 * 65536 + 1000
    x_np = rng.integers(0, 256, n, dtype=np.uint8)
    say("incompressible: flat code, chunk", chunk)
    dcb, obook = make_book(np.full(256, 1000, dtype=np.int64), "huffman", None)
    assert set(obook["lengths"]) == {8}
    roundtrip(dcb, obook, x_np, chunk)
    say("incompressible: skewed code, chunk", chunk)
    counts = np.full(256, 1000, dtype=np.int64)
    counts[:2] = 10  # two 9-bit codes (and shorter ones elsewhere)
    dcb, obook = make_book(counts, "huffman", None)
    assert max(obook["lengths"]) > 8
    roundtrip(dcb, obook, x_np, chunk)



def test_segment_and_global_groups_mixed():
    """Many groups, every third one too dense for the LDS segments: segments
    of 65536 bytes alternate between data the code fits and uniform random
    bytes it codes at more than 8 bits per symbol.  Workgroups then meet
    groups whose halves do not fit in the middle of their persistent loop
    and decode them again from global memory; the ragged last group comes
    after their full groups."""
    counts = np.bincount(skewed(1 << 20, 41), minlength=256).astype(np.int64)
    dcb, obook = make_book(counts, "huffman", None)
    rng = np.random.default_rng(43)
    segs = []
    for i in range(1100):
        segs.append(rng.integers(0, 256, 65536, dtype=np.uint8) if i % 3 == 2 else skewed(65536, 1000 + i))
    x_np = np.concatenate(segs + [skewed(777, 7)])
    say("segment and global groups: n", x_np.size)
    enc = roundtrip(dcb, obook, x_np, 65536)
    bits = host(enc)["chunk_bits"].astype(np.int64)
    assert (bits[2:1100:3] > 8 * 65536).all() and (bits[0:1100:3] < 8 * 65536).all()

# --------------------------------------------------------------------------
# corruption: the decoder's status must agree with the oracle decoder's and
# nothing outside [0, n) may be written
# --------------------------------------------------------------------------

def decode_guarded(dcb, enc, payload_words=None, qlc=False):
    n = enc.n
    guard = 4096
    buf = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
    out = buf[guard:guard + n]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    fn = pc.pc_decode_qlc if qlc else pc.pc_decode
    fn(dcb, enc, payload_words=payload_words, out=out, status=status)
    torch.cuda.synchronize()
    assert bool((buf[:guard] == 0xA5).all()) and bool((buf[guard + n:] == 0xA5).all()), "write outside [0, n)"
    return out.clone(), int(status.item())


def modified(enc, **kw):
    d = enc._asdict()
    d.update(kw)
    return pc.Encoded(**d)


def oracle_status(enc, obook, payload_words=None):
    h = host(enc)
    h["chunk_word_offset"] = enc.chunk_word_offset.cpu().numpy().view(np.uint64)
    pw = payload_words if payload_words is not None else enc.payload.numel()
    h["payload"] = enc.payload[:pw].cpu().numpy().view(np.uint32)
    return coder.decode(h, enc.n, enc.chunk, obook)[1]


@pytest.mark.parametrize("kind", ["huffman", "qlc"])
def test_corruptions_detected(kind):
    bits = (1, 3, 3, 3, 3, 5, 6, 7) if kind == "qlc" else None
    dcb, obook = make_book(random_counts(11), kind, bits)
    chunk = 4096
    x_np = skewed(20 * chunk + 1000, 2)
    x, enc = gpu_encode(dcb, x_np, chunk)
    total = int(enc.chunk_word_offset[-1].item())
    say("corruption:", kind)
    cases = []
    cb2 = enc.chunk_bits.clone()
    cb2[3] -= 1
    cases.append(("chunk_bits-1", modified(enc, chunk_bits=cb2), None))
    cb3 = enc.chunk_bits.clone()
    cb3[5] += 40
    cases.append(("chunk_bits+40", modified(enc, chunk_bits=cb3), None))
    so = enc.sub_off.clone()
    so[7] += 1
    cases.append(("sub_off+1", modified(enc, sub_off=so), None))
    so0 = enc.sub_off.clone()
    so0[16] = 3  # first sub-stream of chunk 1
    cases.append(("sub_off[first]!=0", modified(enc, sub_off=so0), None))
    cw = enc.chunk_word_offset.clone()
    cw[4] += 1
    cases.append(("cwo+1", modified(enc, chunk_word_offset=cw), None))
    cases.append(("short payload", enc, total - 1))
    cases.append(("payload under one quad", enc, 3))
    for cname, e2, pw in cases:
        say("  case", cname)
        _, st = decode_guarded(dcb, e2, pw)
        assert st == pc.PC_ERR_CORRUPT, cname
        assert oracle_status(e2, obook, pw) == coder.CORRUPT, cname
    # random bit flips: status agrees with the oracle; an accepted stream
    # decodes to what the oracle decodes
    rng = np.random.default_rng(1)
    for t in range(24):
        p2 = enc.payload.clone()
        i = int(rng.integers(0, total))
        p2[i] ^= int(np.int32(np.uint32(1 << int(rng.integers(0, 32))).view(np.int32)))
        e2 = modified(enc, payload=p2)
        out, st = decode_guarded(dcb, e2, total)
        ost = oracle_status(e2, obook, total)
        assert (st == pc.PC_ERR_CORRUPT) == (ost == coder.CORRUPT), (t, st, ost)
        if st == 0:
            h = host(e2)
            want, _ = coder.decode(h, enc.n, chunk, obook)
            assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("bits", [(1, 3, 3, 3, 3, 5, 6, 7), (5, 4, 3, 3, 3, 3, 3, 8)])
def test_unused_qlc_code_detected(bits):
    counts = np.arange(256, 0, -1) * 10
    dcb, obook = make_book(counts, "qlc", bits)
    data = np.arange(256, dtype=np.uint8).repeat(4)  # byte r has rank r
    lengths, codes = list(obook["lengths"]), list(obook["codes"])
    assert lengths[255] == 3 + bits[7]  # rank 255 lies in the last area
    codes_bad = codes[:]
    codes_bad[255] = (7 << bits[7]) | ((1 << bits[7]) - 1)  # unused slot of the last area
    from tests_helpers import string_encode
    s = string_encode(list(data), lengths, codes_bad, 1024)
    enc = pc.Encoded(
        torch.from_numpy(np.concatenate([s["payload"], np.zeros(4, np.uint32)]).view(np.int32)).to(DEV),
        torch.from_numpy(s["chunk_bits"].view(np.int32)).to(DEV),
        torch.from_numpy(s["chunk_word_offset"].view(np.int64)).to(DEV),
        torch.from_numpy(s["sub_off"].view(np.int32)).to(DEV), data.size, 1024)
    for q in (False, True):
        _, st = decode_guarded(dcb, enc, len(s["payload"]), qlc=q)
        assert st == pc.PC_ERR_CORRUPT
    assert coder.decode(s, data.size, 1024, obook)[1] == coder.CORRUPT


def test_qlc_decoder_rejects_huffman_codebook():
    dcb, obook = make_book(random_counts(4))
    x_np = skewed(10000, 1)
    x, enc = gpu_encode(dcb, x_np, 4096)
    _, st = decode_guarded(dcb, enc, qlc=True)
    assert st == pc.PC_ERR_CORRUPT


# --------------------------------------------------------------------------
# device histogram (statistics for the offline codebook build)
# --------------------------------------------------------------------------

def test_histogram_matches_bincount():
    rng = np.random.default_rng(3)
    base = torch.from_numpy(skewed(3_000_017, 9)).to(DEV)
    for off in (0, 1, 7, 15):
        for n in (0, 1, 15, 16, 17, 100_000, 3_000_000):
            say("histogram: offset", off, "n", n)
            x = base[off:off + n]
            counts = pc.pc_histogram(x)
            pc.pc_histogram(x, counts)  # accumulates
            torch.cuda.synchronize()
            want = 2 * np.bincount(x.cpu().numpy(), minlength=256)
            assert np.array_equal(counts.cpu().numpy(), want)
    # large enough that every workgroup loops: 4-load rounds, the single
    # loads after them, and a ragged tail
    big = torch.from_numpy(skewed(40_000_021, 11)).to(DEV)[3:]
    say("histogram: offset 3 n", big.numel())
    counts = pc.pc_histogram(big)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), np.bincount(big.cpu().numpy(), minlength=256))
    del rng


# --------------------------------------------------------------------------
# streams and buffer reuse
# --------------------------------------------------------------------------

def test_side_streams_and_reused_buffers():
    """Two encode + decode pipelines on two non-default streams at once,
    each with its own outputs and workspace, run twice with the buffers of
    the first run reused (stale contents, including the look-back
    workspace, must not matter)."""
    dcb, obook = make_book(random_counts(31))
    chunk = 65536
    inputs = [skewed(5 * chunk + 300, 41), skewed(7 * chunk, 42)]
    xs = [torch.from_numpy(a).to(DEV) for a in inputs]
    outs = [pc.alloc_encode_outputs(a.size, chunk, torch.device(DEV)) for a in inputs]
    dec_out = [torch.empty(a.size, dtype=torch.uint8, device=DEV) for a in inputs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    for rep in range(2):
        say("side streams: pass", rep)
        encs, stats = [None, None], [None, None]
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                encs[i] = pc.pc_encode(dcb, xs[i], chunk, outputs=outs[i])
                stats[i] = torch.zeros(1, dtype=torch.int32, device=DEV)
                pc.pc_decode(dcb, encs[i], out=dec_out[i], status=stats[i])
        torch.cuda.synchronize()
        for i in range(2):
            want = coder.encode(inputs[i], obook["lengths"], obook["codes"], chunk, threads=4)
            assert_same_stream(host(encs[i]), want)
            assert int(encs[i].status.item()) == pc.PC_OK
            assert int(stats[i].item()) == 0
            assert torch.equal(dec_out[i][:inputs[i].size], xs[i])
        for i in range(2):  # stale contents for the second pass
            outs[i][0].fill_(-1)
            outs[i][4].fill_(-1)
            dec_out[i].fill_(0)
        torch.cuda.synchronize()


def test_largest_chunk_size():
    """Chunks of 2^24 symbols (the largest the container allows): one full
    chunk and a short one, and a single partial chunk."""
    dcb, obook = make_book(random_counts(51))
    chunk = 1 << 24
    for n in (chunk + 12345, 3 * (1 << 20) + 7):
        say("largest chunk:", chunk, "n", n)
        roundtrip(dcb, obook, skewed(n, n % 1000), chunk)


def test_encode_wait_give_up_is_reported():
    """The cross-chunk scan's bounded wait, cut to one poll from the host, gives
    up while earlier workgroups are still running and reports PC_ERR_TIMEOUT
    through the status word (every kernel still ends normally: no wait is
    longer than one poll).  With the default limit the same call is correct
    again.  1024 workgroups of 4 chunks: the first 512 run at once, so many
    look-backs meet an unpublished predecessor on their first poll."""
    w = W.WORKLOADS["ffn1_act"]
    x_np = W.make("ffn1_act", 0)
    dcb, obook = make_book(np.bincount(W.make("ffn1_act", 1), minlength=256))
    x = torch.from_numpy(x_np).to(DEV)
    outs = pc.alloc_encode_outputs(x_np.size, w.chunk, torch.device(DEV))
    seen = []
    prev = pc.pc_encode_set_wait_limit(1)
    try:
        for rep in range(3):
            say("wait give-up: call", rep)
            enc = pc.pc_encode(dcb, x, w.chunk, outputs=outs)
            torch.cuda.synchronize()
            seen.append(int(enc.status.item()))
            if seen[-1] == pc.PC_ERR_TIMEOUT:
                break
    finally:
        pc.pc_encode_set_wait_limit(prev)
    say("wait give-up: statuses", seen)
    assert set(seen) <= {pc.PC_OK, pc.PC_ERR_TIMEOUT}
    assert pc.PC_ERR_TIMEOUT in seen
    enc = pc.pc_encode(dcb, x, w.chunk, outputs=outs)
    torch.cuda.synchronize()
    assert int(enc.status.item()) == pc.PC_OK
    want = coder.encode(x_np, obook["lengths"], obook["codes"], w.chunk, threads=8)
    assert_same_stream(host(enc), want)


def test_unit_encoder_wait_limit_one_poll():
    """The persistent unit encoder (an input of four units per workgroup)
    with its bounded wait cut to one poll: every call ends, the status is
    PC_OK or PC_ERR_TIMEOUT (a walk that met an unpublished predecessor gave
    up), and with the default limit the same call is bit-exact again."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = 8 * cus * 65536
    dcb, obook = make_book(random_counts(3))
    x_np = skewed(n, 3)
    x = torch.from_numpy(x_np).to(DEV)
    outs = pc.alloc_encode_outputs(n, 65536, torch.device(DEV))
    seen = []
    prev = pc.pc_encode_set_wait_limit(1)
    try:
        for rep in range(3):
            enc = pc.pc_encode(dcb, x, 65536, outputs=outs)
            torch.cuda.synchronize()
            seen.append(int(enc.status.item()))
    finally:
        pc.pc_encode_set_wait_limit(prev)
    say("unit encoder, one-poll limit: statuses", seen)
    assert set(seen) <= {pc.PC_OK, pc.PC_ERR_TIMEOUT}
    enc = pc.pc_encode(dcb, x, 65536, outputs=outs)
    torch.cuda.synchronize()
    assert int(enc.status.item()) == pc.PC_OK
    want = coder.encode(x_np, obook["lengths"], obook["codes"], 65536, threads=16)
    assert_same_stream(host(enc), want)


def test_traffic_probe_copies():
    """The counter-calibration copy moves the bytes unchanged (sizes around
    one grid pass and a ragged tail of 16-byte quads)."""
    rng = np.random.default_rng(5)
    for nbytes in (16, 4096 + 48, (1 << 22) + 16 * 7):
        src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to(DEV)
        dst = torch.zeros_like(src)
        pc.pc_traffic_probe(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)


def test_refresh_pools_on_the_device():
    """CodebookRefresh.observe_batch (histograms counted and pooled by
    pc_histogram on the device) makes the same rebuild decisions and the
    same codebooks as observe on host histograms of the same batches,
    including batches leaving the window, and its pool equals the sum of the
    window's bincounts."""
    rng = np.random.default_rng(17)
    batches = []
    for k in range(9):
        scale = 1.0 if k < 5 else 4.0  # drift from batch 5 on
        v = rng.standard_normal(1 << 16) * scale
        batches.append(((np.clip(v, -7.9, 7.9) * 16).astype(np.int64) % 256).astype(np.uint8))
    host = pc.CodebookRefresh(window=3, threshold=0.02)
    dev = pc.CodebookRefresh(window=3, threshold=0.02)
    for k, b in enumerate(batches):
        a = host.observe(np.bincount(b, minlength=256))
        d = dev.observe_batch(torch.from_numpy(b).to(DEV))
        assert a == d, k
        assert torch.equal(host.codebook, dev.codebook), k
        want = sum(np.bincount(x, minlength=256) for x in batches[max(0, k - 2):k + 1])
        assert np.array_equal(dev.pool_dev.cpu().numpy(), want), k
    assert host.rebuilds == dev.rebuilds >= 2
