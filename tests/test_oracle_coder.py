"""Pins of the oracle's bit-serial coder.

The C coder is checked against an independent restatement of the container
(codewords concatenated as a '0'/'1' string, cut into 32-character words,
zero-padded), against round-trip identity, against sum(count * length), and
against planted corruptions that the decoder must reject.
"""
import numpy as np
import pytest

from oracle import codebook as cb
from oracle import coder
from tests_helpers import string_encode

SUB = 256


def random_book(seed, kind="huffman"):
    rng = np.random.default_rng(seed)
    counts = [int(v) for v in (rng.pareto(1.2, 256) * 100).astype(np.int64)]
    if kind == "qlc":
        return cb.codebook(counts, "qlc", (1, 3, 3, 3, 3, 5, 6, 7))
    return cb.codebook(counts)


def same(a, b):
    for k in ("payload", "chunk_bits", "chunk_word_offset", "sub_off"):
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


@pytest.mark.parametrize("kind", ["huffman", "qlc"])
@pytest.mark.parametrize("n,chunk", [(0, 256), (1, 256), (255, 256), (256, 256), (257, 256),
                                     (1023, 512), (1025, 512), (3 * 768 + 100, 768), (5000, 4096)])
def test_c_encoder_equals_string_reference(kind, n, chunk):
    book = random_book(n + chunk, kind)
    rng = np.random.default_rng(n)
    data = rng.integers(0, 256, n, dtype=np.uint8)
    want = string_encode(list(data), book["lengths"], book["codes"], chunk)
    got = coder.encode(data, book["lengths"], book["codes"], chunk, threads=3)
    same(got, want)
    out, rc = coder.decode(got, n, chunk, book, threads=2)
    assert rc == coder.OK
    assert np.array_equal(out, data)


@pytest.mark.parametrize("kind", ["huffman", "qlc"])
def test_round_trip_and_bit_count(kind):
    book = random_book(5, kind)
    rng = np.random.default_rng(6)
    # skewed data drawn from the codebook's own ranking
    data = (rng.zipf(1.3, 200_000) % 256).astype(np.uint8)
    chunk = 4096
    s = coder.encode(data, book["lengths"], book["codes"], chunk, threads=4)
    counts = cb.histogram(data)
    assert int(s["chunk_bits"].sum()) == cb.coded_bits(counts, book["lengths"])
    # per-chunk count and side index are prefix sums of code lengths
    L = np.asarray(book["lengths"], dtype=np.int64)[data]
    for c in range(0, len(s["chunk_bits"]), 7):
        part = L[c * chunk:(c + 1) * chunk]
        assert int(s["chunk_bits"][c]) == int(part.sum())
        pref = np.concatenate([[0], np.cumsum(part)])
        subs = s["sub_off"][c * (chunk // SUB):(c + 1) * (chunk // SUB)]
        assert np.array_equal(subs, pref[0:len(part):SUB])
    # padding bits after each chunk are zero
    for c in range(len(s["chunk_bits"])):
        b = int(s["chunk_bits"][c])
        if b % 32:
            w = int(s["payload"][int(s["chunk_word_offset"][c]) + b // 32])
            assert w & ((1 << (32 - b % 32)) - 1) == 0
    out, rc = coder.decode(s, data.size, chunk, book, threads=4)
    assert rc == coder.OK and np.array_equal(out, data)


def test_single_symbol_and_uniform_data():
    book = random_book(9)
    for data in (np.full(70_000, 17, np.uint8), np.tile(np.arange(256, dtype=np.uint8), 300)):
        s = coder.encode(data, book["lengths"], book["codes"], 1024, threads=2)
        out, rc = coder.decode(s, data.size, 1024, book, threads=2)
        assert rc == coder.OK and np.array_equal(out, data)


def test_threads_do_not_change_the_stream():
    book = random_book(3)
    data = np.random.default_rng(1).integers(0, 256, 100_000, dtype=np.uint8)
    a = coder.encode(data, book["lengths"], book["codes"], 2048, threads=1)
    b = coder.encode(data, book["lengths"], book["codes"], 2048, threads=7)
    same(a, b)


# --------------------------------------------------------------------------
# corruption detection
# --------------------------------------------------------------------------

def _stream(kind="huffman", n=20_000, chunk=2048, seed=4):
    book = random_book(seed, kind)
    data = np.random.default_rng(seed).integers(0, 256, n, dtype=np.uint8)
    return book, data, coder.encode(data, book["lengths"], book["codes"], chunk, threads=2), chunk


def _copy(s):
    return {k: np.array(v, copy=True) for k, v in s.items()}


def test_truncated_chunk_bits_detected():
    book, data, s, chunk = _stream()
    t = _copy(s)
    t["chunk_bits"][2] -= 1
    assert coder.decode(t, data.size, chunk, book)[1] == coder.CORRUPT


def test_shifted_side_index_detected():
    book, data, s, chunk = _stream()
    t = _copy(s)
    t["sub_off"][3] += 1
    assert coder.decode(t, data.size, chunk, book)[1] == coder.CORRUPT
    t = _copy(s)
    t["sub_off"][0] = 1  # first sub-stream of a chunk must start at bit 0
    assert coder.decode(t, data.size, chunk, book)[1] == coder.CORRUPT


def test_bad_word_offsets_detected():
    book, data, s, chunk = _stream()
    t = _copy(s)
    t["chunk_word_offset"][3] += 1
    assert coder.decode(t, data.size, chunk, book)[1] == coder.CORRUPT
    t = _copy(s)
    t["payload"] = t["payload"][:-1]
    assert coder.decode(t, data.size, chunk, book)[1] == coder.CORRUPT


def test_unused_qlc_code_detected():
    bits = (1, 3, 3, 3, 3, 5, 6, 7)
    counts = list(range(256, 0, -1))
    book = cb.codebook(counts, "qlc", bits)
    data = np.arange(256, dtype=np.uint8)  # byte r has rank r
    lengths, codes = list(book["lengths"]), list(book["codes"])
    # swap the code of rank 255 (area 8, index 125) for the unused index 126
    codes_bad = codes[:]
    codes_bad[255] = (7 << 7) | 126
    s = string_encode(list(data), lengths, codes_bad, 256)
    assert coder.decode(s, 256, 256, book)[1] == coder.CORRUPT
    s = string_encode(list(data), lengths, codes, 256)
    out, rc = coder.decode(s, 256, 256, book)
    assert rc == coder.OK and np.array_equal(out, data)


def test_flipped_bit_changes_output_or_is_rejected():
    book, data, s, chunk = _stream(n=50_000)
    rng = np.random.default_rng(0)
    cwo = s["chunk_word_offset"].astype(np.int64)
    for _ in range(40):
        t = _copy(s)
        i = int(rng.integers(0, t["payload"].size))
        b = int(rng.integers(0, 32))
        t["payload"][i] ^= np.uint32(1 << b)
        c = int(np.searchsorted(cwo, i, side="right") - 1)
        pos = (i - int(cwo[c])) * 32 + (31 - b)
        out, rc = coder.decode(t, data.size, chunk, book)
        if pos >= int(s["chunk_bits"][c]):  # a padding bit carries nothing
            assert rc == coder.OK and np.array_equal(out, data)
        else:
            assert rc == coder.CORRUPT or not np.array_equal(out, data)
