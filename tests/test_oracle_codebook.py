"""Pins of the codebook oracle against facts fixed outside the oracle.

Each test checks the oracle against something other than itself: values
printed on the pages (QLC Tables 1 and 2), closed forms, brute force on tiny
alphabets, textbook inequalities and a published worked example of canonical
code assignment.
"""
import itertools
import math
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import codebook as cb


# --------------------------------------------------------------------------
# histogram / pooling
# --------------------------------------------------------------------------

def test_histogram_brute_force():
    rng = random.Random(1)
    data = [rng.randrange(256) for _ in range(3000)] + [7] * 50
    counts = cb.histogram(np.array(data, dtype=np.uint8))
    for s in range(256):
        assert counts[s] == sum(1 for v in data if v == s)
    assert sum(counts) == len(data)


def test_pooled_counts_is_sum_of_batches():
    rng = np.random.default_rng(3)
    batches = [rng.integers(0, 256, 1000, dtype=np.uint8) for _ in range(4)]
    pooled = cb.pooled_counts(batches)
    allbytes = np.concatenate(batches)
    assert pooled == cb.histogram(allbytes)


def test_floor_keeps_every_symbol_codable():
    counts = [0] * 256
    counts[3] = 1000
    counts[200] = 5
    w = cb.floor_weights(counts)
    assert min(w) == 1 and w[3] == 1000 and w[200] == 5
    lengths = cb.package_merge(w)
    assert all(1 <= l <= 12 for l in lengths)
    assert cb.kraft(lengths) == 1


# --------------------------------------------------------------------------
# package-merge: optimality and closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_package_merge_matches_brute_force(seed):
    rng = random.Random(seed)
    n = rng.randint(2, 8)
    # skewed weights so that short limits bind
    weights = [rng.choice([1, 1, 2, 3, 5, 8, 13, 40, 200, 1000]) for _ in range(n)]
    min_l = max(1, math.ceil(math.log2(n)))
    for L in range(min_l, n):
        if n == 8 and L > 4:
            break  # keep the exhaustive search small
        lengths = cb.package_merge(weights, L)
        assert max(lengths) <= L
        assert cb.kraft(lengths) <= 1
        assert cb.cost(weights, lengths) == cb.brute_force_cost(weights, L), (weights, L)


def test_brute_force_itself_on_hand_case():
    # weights 1,1,2,4: Huffman lengths 3,3,2,1 cost 1*3+1*3+2*2+4*1 = 14;
    # with L = 2 every length is 2: cost 16.
    assert cb.brute_force_cost([1, 1, 2, 4], 3) == 14
    assert cb.brute_force_cost([1, 1, 2, 4], 2) == 16


@pytest.mark.parametrize("seed", range(20))
def test_kraft_exactly_one_and_limit(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 257))
    w = [int(v) for v in rng.integers(1, 10**6, n)]
    if seed % 3 == 0:
        w = [int(2 ** (v % 40)) for v in range(n)]  # heavy skew: limit binds
    lengths = cb.package_merge(w, 12)
    assert max(lengths) <= 12
    assert cb.kraft(lengths) == Fraction(1)


@pytest.mark.parametrize("seed", range(10))
def test_equals_huffman_cost_when_huffman_fits(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 200))
    w = [int(v) for v in rng.integers(1, 1000, n)]
    h = cb.huffman_lengths(w)
    if max(h) <= 12:
        assert cb.cost(w, cb.package_merge(w, 12)) == cb.cost(w, h)
    # L = n - 1 never binds: package-merge is then plain Huffman
    if n <= 64:
        assert cb.cost(w, cb.package_merge(w, max(n - 1, 1))) == cb.cost(w, h)


@pytest.mark.parametrize("seed", range(10))
def test_huffman_within_entropy_plus_one(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(2, 257))
    w = [int(v) for v in rng.integers(1, 10**5, n)]
    h = cb.huffman_lengths(w)
    tot = sum(w)
    avg = cb.cost(w, h) / tot
    H = cb.entropy_bits(w)
    assert H - 1e-12 <= avg < H + 1
    # the length limit costs at most what it must: never below Huffman
    assert cb.cost(w, cb.package_merge(w, 12)) >= cb.cost(w, h)


def test_uniform_gives_all_eights():
    assert cb.package_merge([7] * 256, 12) == [8] * 256


def test_dyadic_gives_minus_log2_p():
    # p_s = 2^-k_s with a complete dyadic distribution, max k = 12
    ks = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 12]
    assert sum(Fraction(1, 2 ** k) for k in ks) == 1
    w = [2 ** (12 - k) for k in ks]
    lengths = cb.package_merge(w, 12)
    assert lengths == ks
    # average length equals the entropy exactly
    tot = sum(w)
    assert abs(cb.cost(w, lengths) / tot - cb.entropy_bits(w)) < 1e-12


def test_fibonacci_limit_binds():
    fib = [1, 1]
    while len(fib) < 20:
        fib.append(fib[-1] + fib[-2])
    h = cb.huffman_lengths(fib)
    assert max(h) == 19  # unconstrained depth n-1
    pm = cb.package_merge(fib, 12)
    assert max(pm) == 12
    assert cb.kraft(pm) == 1
    assert cb.cost(fib, pm) > cb.cost(fib, h)


def test_tie_rule_is_deterministic_and_weight_monotone():
    # Equal weights and a skewed tail: heavier symbols never get longer codes,
    # and among equal weights a lower byte value never gets a longer code
    # (leaves are ordered by (weight, byte value); the merge keeps leaves first).
    rng = np.random.default_rng(7)
    w = [int(v) for v in rng.integers(1, 6, 256)]
    lengths = cb.package_merge(w, 12)
    for a in range(256):
        for b in range(256):
            if w[a] > w[b]:
                assert lengths[a] <= lengths[b]
            if w[a] == w[b] and a < b:
                assert lengths[a] >= lengths[b]


# --------------------------------------------------------------------------
# canonical codes
# --------------------------------------------------------------------------

def test_canonical_matches_deflate_worked_example(golden):
    rows = golden("deflate_canonical_example.txt")
    lengths = [int(r[1]) for r in rows]
    codes = cb.canonical_codes(lengths)
    for (s, l, want), c in zip(rows, codes):
        assert cb.code_string(c, int(l)) == want


@pytest.mark.parametrize("seed", range(8))
def test_canonical_prefix_free_and_ordered(seed):
    rng = np.random.default_rng(300 + seed)
    counts = [int(v) for v in rng.integers(0, 10**4, 256)]
    lengths, codes = cb.huffman_codebook(counts)
    strs = [cb.code_string(c, l) for c, l in zip(codes, lengths)]
    assert len(set(strs)) == 256
    for i in range(256):
        for j in range(256):
            if i != j:
                assert not strs[j].startswith(strs[i])
    order = sorted(range(256), key=lambda s: (lengths[s], s))
    assert codes[order[0]] == 0
    assert codes[order[-1]] == (1 << lengths[order[-1]]) - 1  # Kraft = 1
    for a, b in zip(order, order[1:]):
        # read as binary fractions, codes strictly increase along the order
        assert Fraction(codes[a] + 1, 1 << lengths[a]) <= Fraction(codes[b], 1 << lengths[b])


# --------------------------------------------------------------------------
# Quad Length Codes: the printed tables
# --------------------------------------------------------------------------

@pytest.mark.parametrize("table", ["qlc_table1.txt", "qlc_table2.txt"])
def test_qlc_layout_reproduces_printed_table(golden, table):
    rows = golden(table)
    bits = [int(r[3]) for r in rows] + [7, 7]  # areas 7-8 unprinted: any value
    layout = cb.qlc_layout(bits)
    for r, (a, slots, b, length, start) in zip(rows, layout):
        area, code, nsym, sbits, clen, lo, hi = r
        assert int(area) == a + 1
        assert code == format(a, "03b")
        assert int(nsym) == slots == 2 ** int(sbits)
        assert int(clen) == length == 3 + int(sbits)
        assert (int(lo), int(hi)) == (start, start + slots - 1)


def test_qlc_table_lengths_are_the_printed_ones(golden):
    assert [int(r[4]) for r in golden("qlc_table1.txt")] == [6, 6, 6, 6, 6, 7]
    assert [int(r[4]) for r in golden("qlc_table2.txt")] == [4, 6, 6, 6, 6, 8]


def test_qlc_codes_follow_table2_ranks(golden):
    rows = golden("qlc_table2.txt")
    bits = (1, 3, 3, 3, 3, 5, 6, 7)
    rng = np.random.default_rng(11)
    counts = [int(v) for v in rng.integers(0, 10**6, 256)]
    lengths, codes, rank_of, order = cb.qlc_code(counts, bits)
    # rank r = position in descending-count order, ties by byte value
    for r in range(255):
        a, b = order[r], order[r + 1]
        assert counts[a] > counts[b] or (counts[a] == counts[b] and a < b)
    for area, code, nsym, sbits, clen, lo, hi in rows:
        for r in range(int(lo), int(hi) + 1):
            s = order[r]
            assert lengths[s] == int(clen)
            want = code + format(r - int(lo), "0%sb" % sbits)
            assert cb.code_string(codes[s], lengths[s]) == want


def test_qlc_gelu_layout_closed_forms():
    bits = (1, 3, 3, 3, 3, 5, 6, 7)
    counts = list(range(256, 0, -1))  # rank r is byte r
    lengths, codes, rank_of, order = cb.qlc_code(counts, bits)
    assert order == list(range(256))
    assert all(lengths[r] == 9 for r in range(66, 130))
    assert all(lengths[r] == 10 for r in range(130, 256))
    assert cb.kraft(lengths) == Fraction(511, 512)
    # exactly 8 of the 4096 12-bit prefixes start with no codeword
    strs = [cb.code_string(c, l) for c, l in zip(codes, lengths)]
    covered = sum(2 ** (12 - len(s)) for s in strs)
    assert 4096 - covered == 8
    # prefix-free
    for i in range(256):
        for j in range(256):
            if i != j:
                assert not strs[j].startswith(strs[i])


def test_qlc_equals_canonical_when_lengths_do_not_decrease():
    # Lengths grow across areas here, so the QLC codes are the canonical codes
    # of (length, rank) order: a cross-check of the two code-assignment rules.
    bits = (1, 3, 3, 3, 3, 5, 6, 7)
    rng = np.random.default_rng(5)
    counts = [int(v) for v in rng.integers(0, 1000, 256)]
    lengths, codes, rank_of, order = cb.qlc_code(counts, bits)
    by_rank_len = [lengths[order[r]] for r in range(256)]
    canon = cb.canonical_codes(by_rank_len)
    for r in range(256):
        assert codes[order[r]] == canon[r]


@pytest.mark.parametrize("bits", [(1, 3, 3, 3, 3, 5, 6, 7), (3, 3, 3, 3, 3, 4, 7, 7), (5, 4, 3, 3, 3, 3, 3, 8),
                                  (0, 0, 1, 2, 4, 6, 7, 7), (8, 0, 0, 0, 0, 0, 0, 0)])
def test_qlc_valid_windows_are_one_interval(bits):
    # The QLC decoder's invalid-codeword test rests on this: read as
    # left-aligned numbers, the windows that start with a codeword of the
    # QLC code (ranks 0..255) are exactly those below the left-aligned
    # codeword that rank 256 would get (none, when the areas hold exactly
    # 256 ranks).  Checked by brute force over every 12-bit window, for
    # layouts with growing, shrinking and empty areas.
    lengths, codes, _, _ = cb.qlc_code(list(range(256, 0, -1)), bits)
    valid = [False] * 4096
    for s in range(256):
        lo = codes[s] << (12 - lengths[s])
        for p in range(lo, lo + (1 << (12 - lengths[s]))):
            assert not valid[p]  # prefix-free
            valid[p] = True
    start, bound = 0, 4096
    for a, b in enumerate(bits):
        if start <= 256 < start + (1 << b):
            bound = ((a << b) | (256 - start)) << (12 - 3 - b)
            break
        start += 1 << b
    assert valid == [p < bound for p in range(4096)]


def test_qlc_rejects_short_cover():
    with pytest.raises(ValueError):
        cb.qlc_code([1] * 256, (1, 1, 1, 1, 1, 1, 1, 1))


# --------------------------------------------------------------------------
# measurement quantities
# --------------------------------------------------------------------------

def test_entropy_closed_forms():
    assert cb.entropy_bits([5] * 256) == pytest.approx(8.0, abs=1e-12)
    assert cb.entropy_bits([0] * 255 + [9]) == 0.0
    assert cb.entropy_bits([1, 1]) == pytest.approx(1.0)
    assert cb.entropy_bits([2, 1, 1]) == pytest.approx(1.5)


@pytest.mark.parametrize("seed", range(5))
def test_gibbs_fixed_code_costs_at_least_entropy(seed):
    rng = np.random.default_rng(400 + seed)
    prev = [int(v) for v in rng.integers(0, 10**4, 256)]
    cur = [int(v) for v in rng.integers(0, 10**4, 256)]
    lengths, _ = cb.huffman_codebook(prev)
    n = sum(cur)
    b = cb.coded_bits(cur, lengths) / n
    assert b >= cb.entropy_bits(cur) - 1e-12
    shard = cb.per_shard_lengths(cur)
    assert cb.coded_bits(cur, shard) <= cb.coded_bits(cur, lengths)


# --------------------------------------------------------------------------
# per-shard comparator ("Single-Stage Huffman Encoder for ML Compression",
# abstract: the fixed code is compared with Huffman codes built per shard)
# --------------------------------------------------------------------------

def test_per_shard_code_gives_absent_bytes_no_codeword():
    # four byte values that occur equally often: a code over just those four
    # is four 2-bit codewords, and the 252 absent values get none.  A build
    # that floors absent values to weight 1 codes all 256 values and gives
    # the four present ones lengths of 5-6 bits instead.
    counts = [0] * 256
    for s in (3, 77, 128, 255):
        counts[s] = 10
    lengths = cb.per_shard_lengths(counts)
    assert [lengths[s] for s in (3, 77, 128, 255)] == [2, 2, 2, 2]
    assert sum(lengths) == 8
    assert cb.coded_bits(counts, lengths) == 80


def test_per_shard_pins_reject_a_floored_build():
    # the mistake the pins above guard against: flooring absent values to
    # weight 1 (as the fixed codebook must) before building the shard's code
    counts = [0] * 256
    for s in (3, 77, 128, 255):
        counts[s] = 10
    floored = cb.package_merge(cb.floor_weights(counts))
    assert [floored[s] for s in (3, 77, 128, 255)] != [2, 2, 2, 2]
    assert cb.coded_bits(counts, floored) > 80


def test_per_shard_code_dyadic_present_bytes():
    # counts 8, 4, 2, 1, 1 (probabilities 1/2 .. 1/16) on five scattered byte
    # values: the optimal code has lengths -log2 p = 1, 2, 3, 4, 4 and costs
    # exactly the entropy, 16 * 1.875 = 30 bits
    counts = [0] * 256
    for s, c in ((200, 8), (5, 4), (17, 2), (0, 1), (99, 1)):
        counts[s] = c
    lengths = cb.per_shard_lengths(counts)
    assert [lengths[s] for s in (200, 5, 17, 0, 99)] == [1, 2, 3, 4, 4]
    assert sum(1 for v in lengths if v) == 5
    assert cb.coded_bits(counts, lengths) == 30
    assert cb.coded_bits(counts, lengths) == pytest.approx(16 * cb.entropy_bits(counts))


def test_per_shard_code_degenerate_histograms():
    one = [0] * 256
    one[42] = 1000
    lengths = cb.per_shard_lengths(one)
    assert lengths[42] == 1 and sum(lengths) == 1  # a lone byte value still takes one bit
    assert cb.per_shard_lengths([0] * 256) == [0] * 256


# --------------------------------------------------------------------------
# exhaustive QLC layout search (the best 8 area widths for a ranked PMF;
# "Quad Length Codes for Lossless Compression of e4m3", abstract: the scheme
# adapts to the distribution)
# --------------------------------------------------------------------------

def test_qlc_search_uniform_counts():
    # 256 equally likely bytes: every prefix code spends >= 8 bits a symbol,
    # with equality only when every length is 8, and a QLC length 3 + b is 8
    # only for b = 5, which 8 areas of 32 ranks give: the unique optimum
    assert cb.qlc_optimal_bits_bruteforce([7] * 256) == (5,) * 8


def test_qlc_search_dyadic_counts():
    # Widths (1,1,2,3,4,5,6,7) cover exactly 256 ranks and every area adds
    # 2^b * 2^-(3+b) = 1/8 to the Kraft sum: a complete code.  Give rank r the
    # count 2^(10 - length(r)) (64,64,64,64, 32 x4, 16 x8, ..., 1 x128: 1024
    # in all).  Then every length is -log2 p and the cost is the entropy, the
    # least any prefix code can spend; by Gibbs' inequality a layout of equal
    # cost has the same length at every rank, which fixes all 8 widths.
    widths = (1, 1, 2, 3, 4, 5, 6, 7)
    per_rank = [1 << (10 - (3 + b)) for b in widths for _ in range(1 << b)]
    assert len(per_rank) == 256 and sum(per_rank) == 1024
    rng = np.random.default_rng(5)
    perm = rng.permutation(256)  # scatter the ranks over the byte values
    counts = [0] * 256
    for r, s in enumerate(perm):
        counts[int(s)] = per_rank[r]
    assert cb.qlc_optimal_bits_bruteforce(counts) == widths
    assert cb.qlc_cost(counts, widths) == 6784  # = 1024 * entropy (6.625 bits)
    assert cb.qlc_cost(counts, widths) == pytest.approx(1024 * cb.entropy_bits(counts))


def test_qlc_search_ties_take_the_smallest_vector():
    # with no counts every covering layout costs 0; the lexicographically
    # smallest covering vector is seven 1-slot areas and a 256-slot last one
    assert cb.qlc_optimal_bits_bruteforce([0] * 256) == (0, 0, 0, 0, 0, 0, 0, 8)


def test_compressibility_reading():
    assert cb.compressibility(8.0) == 0.0
    assert cb.compressibility(6.728) == pytest.approx(0.159)
