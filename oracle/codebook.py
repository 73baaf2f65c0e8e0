"""Oracle for codebook construction -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct Python for every host-side step of a fixed
(single-stage) codebook.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product path
(the C-ABI library and its binding) never does, and this module imports
nothing from the product.

What the pages fix, and the readings taken where they are silent:

* "Single-Stage Huffman Encoder for ML Compression" (abstract): one codebook
  is fixed beforehand from the averaged byte statistics of earlier batches,
  so nothing is counted, built or sent alongside the data at run time.  Averaging is read as *pooled counts*
  (sum of per-batch counts; all batches have equal size, so this is
  proportional to the mean PMF).
* Every one of the 256 byte values must stay codable even if it never
  occurred in the previous batches: weights are floored at 1.
* Length limit 12 bits, built by package-merge (coin-collector form of
  Larmore and Hirschberg); ties in the merge put leaves before packages,
  leaves ordered by (weight, byte value), packages by creation order.
* Canonical codes: symbols ordered by (length, byte value), consecutive code
  values, left-shifted when the length grows (DEFLATE-style).
* "Quad Length Codes for Lossless Compression of e4m3" (abstract, Tables 1
  and 2): 3 prefix bits select one of 8 areas; area a holds 2**b_a symbols
  coded with a fixed b_a-bit index, so its code length is 3 + b_a.  The
  "Symbol Range" column counts ranks of the *sorted* PMF (Figures 1 and 4
  plot sorted PMFs): rank 0 is the most frequent symbol; equal counts are
  ranked by lower byte value first.  The in-area index is plain binary,
  most significant bit first.
* Shannon entropy (the bound "Single-Stage Huffman Encoder for ML
  Compression" compares the fixed code with) is the order-0 empirical
  entropy of the tensor's own byte histogram.

Parity pins for every function here live in ``tests/test_oracle_codebook.py``
(brute force, closed forms, the printed Tables 1 and 2, Kraft, entropy
bounds).  Table 1's areas 7 and 8 are not printed in "Quad Length Codes for
Lossless Compression of e4m3": nothing about
them is pinned ("parity unpinned" for those two rows only).
"""
from __future__ import annotations

import heapq
import itertools
import math
from fractions import Fraction

import numpy as np

ALPHABET = 256
MAX_LEN = 12
QLC_AREAS = 8
QLC_PREFIX_BITS = 3

# ----------------------------------------------------------------------------
# Statistics ("Single-Stage Huffman Encoder for ML Compression", abstract:
# the codebook comes from the averaged distribution of earlier batches).
# ----------------------------------------------------------------------------


def histogram(data) -> list:
    """counts[s] = number of bytes equal to s (a library counting primitive)."""
    a = np.asarray(data, dtype=np.uint8).reshape(-1)
    return [int(c) for c in np.bincount(a, minlength=ALPHABET)]


def pooled_counts(batches) -> list:
    """Pool the histograms of several previous batches by summing counts."""
    tot = [0] * ALPHABET
    for b in batches:
        for s, c in enumerate(histogram(b)):
            tot[s] += c
    return tot


def floor_weights(counts) -> list:
    """w_s = max(count_s, 1): a fixed codebook must code every byte value."""
    return [max(int(c), 1) for c in counts]


# ----------------------------------------------------------------------------
# Optimal prefix-code lengths.
# ----------------------------------------------------------------------------


class _Leaf:
    __slots__ = ("w", "sym")

    def __init__(self, w, sym):
        self.w = w
        self.sym = sym


class _Pkg:
    __slots__ = ("w", "a", "b")

    def __init__(self, a, b):
        self.w = a.w + b.w
        self.a = a
        self.b = b


def _count_leaves(node, lengths):
    if isinstance(node, _Leaf):
        lengths[node.sym] += 1
    else:
        _count_leaves(node.a, lengths)
        _count_leaves(node.b, lengths)


def package_merge(weights, max_len=MAX_LEN) -> list:
    """Optimal length-limited code lengths (coin-collector package-merge).

    Every symbol is a coin of face value 2**-l for each depth l = 1..max_len
    with numismatic value w_s.  The cheapest collection of total face value
    n-1 uses 2n-2 items of the depth-1 list; a symbol's code length is the
    number of times it occurs in that collection.
    """
    n = len(weights)
    if n == 0:
        return []
    if n == 1:
        return [1]
    if (1 << max_len) < n:
        raise ValueError("max_len too small for the alphabet")
    # Leaves ordered by (weight, byte value).
    leaves = [_Leaf(w, s) for (w, s) in sorted((int(w), s) for s, w in enumerate(weights))]
    cur = list(leaves)  # list of the deepest level
    for _ in range(max_len - 1):
        pkgs = [_Pkg(cur[2 * i], cur[2 * i + 1]) for i in range(len(cur) // 2)]
        merged = []
        i = j = 0
        while i < len(leaves) and j < len(pkgs):
            if leaves[i].w <= pkgs[j].w:  # equal weight: the leaf goes first
                merged.append(leaves[i])
                i += 1
            else:
                merged.append(pkgs[j])
                j += 1
        merged.extend(leaves[i:])
        merged.extend(pkgs[j:])
        cur = merged
    lengths = [0] * n
    for node in cur[: 2 * n - 2]:
        _count_leaves(node, lengths)
    return lengths


def huffman_lengths(weights) -> list:
    """Unconstrained Huffman code lengths (textbook two-smallest merging)."""
    n = len(weights)
    if n == 1:
        return [1]
    tie = itertools.count()
    heap = [(int(w), next(tie), (s,)) for s, w in enumerate(weights)]
    heapq.heapify(heap)
    lengths = [0] * n
    while len(heap) > 1:
        w1, _, s1 = heapq.heappop(heap)
        w2, _, s2 = heapq.heappop(heap)
        for s in s1 + s2:
            lengths[s] += 1
        heapq.heappush(heap, (w1 + w2, next(tie), s1 + s2))
    return lengths


def brute_force_cost(weights, max_len) -> int:
    """Minimum sum(w*l) over all l in [1,max_len]^n with Kraft sum <= 1."""
    n = len(weights)
    full = 1 << max_len
    best = [None]

    def rec(i, used, cost):
        if best[0] is not None and cost >= best[0]:
            return
        if i == n:
            best[0] = cost
            return
        for l in range(1, max_len + 1):
            u = used + (full >> l)
            if u <= full:
                rec(i + 1, u, cost + int(weights[i]) * l)

    rec(0, 0, 0)
    return best[0]


def cost(weights, lengths) -> int:
    return sum(int(w) * int(l) for w, l in zip(weights, lengths))


def kraft(lengths) -> Fraction:
    """Exact Kraft sum of a length vector."""
    return sum((Fraction(1, 1 << int(l)) for l in lengths), Fraction(0))


# ----------------------------------------------------------------------------
# Canonical codes.
# ----------------------------------------------------------------------------


def canonical_codes(lengths) -> list:
    """Right-aligned code values of the canonical code for ``lengths``.

    Symbols sorted by (length, byte value); the first gets 0; each next code
    is the previous plus one, shifted left by the growth in length.
    """
    order = sorted((l, s) for s, l in enumerate(lengths) if l > 0)
    codes = [0] * len(lengths)
    code = 0
    prev_len = order[0][0] if order else 0
    first = True
    for l, s in order:
        if first:
            code = 0
            first = False
        else:
            code = (code + 1) << (l - prev_len)
        codes[s] = code
        prev_len = l
    return codes


def code_string(code, length) -> str:
    """The code as a string of '0'/'1', most significant bit first."""
    return format(code, "0%db" % length) if length else ""


# ----------------------------------------------------------------------------
# Quad Length Codes.
# ----------------------------------------------------------------------------


def qlc_rank(counts) -> list:
    """Symbols in order of descending count, equal counts by lower byte value."""
    return sorted(range(len(counts)), key=lambda s: (-int(counts[s]), s))


def qlc_layout(bits):
    """Per area: (area code, number of slots, index bits, code length, first rank)."""
    if len(bits) != QLC_AREAS:
        raise ValueError("QLC needs 8 areas")
    rows = []
    start = 0
    for a, b in enumerate(bits):
        rows.append((a, 1 << b, b, QLC_PREFIX_BITS + b, start))
        start += 1 << b
    return rows


def qlc_code(counts, bits):
    """QLC codebook: (lengths, codes, rank_of, sym_of_rank) for 256 symbols."""
    layout = qlc_layout(bits)
    if sum(r[1] for r in layout) < ALPHABET:
        raise ValueError("QLC areas cover fewer than 256 ranks")
    if any(b > MAX_LEN - QLC_PREFIX_BITS for b in bits):
        raise ValueError("QLC area index too wide")
    order = qlc_rank(counts)
    lengths = [0] * ALPHABET
    codes = [0] * ALPHABET
    rank_of = [0] * ALPHABET
    for r, s in enumerate(order):
        rank_of[s] = r
        for a, slots, b, l, start in layout:
            if start <= r < start + slots:
                lengths[s] = l
                codes[s] = (a << b) | (r - start)
                break
    return lengths, codes, rank_of, order


# ----------------------------------------------------------------------------
# Whole codebooks and measurement quantities.
# ----------------------------------------------------------------------------


def huffman_codebook(counts, max_len=MAX_LEN):
    lengths = package_merge(floor_weights(counts), max_len)
    return lengths, canonical_codes(lengths)


def codebook(counts, kind="huffman", qlc_bits=None):
    """dict(kind, lengths, codes[, rank_of, sym_of_rank, qlc_bits])."""
    if kind == "huffman":
        lengths, codes = huffman_codebook(counts)
        return {"kind": kind, "lengths": lengths, "codes": codes}
    if kind == "qlc":
        lengths, codes, rank_of, order = qlc_code(counts, qlc_bits)
        return {"kind": kind, "lengths": lengths, "codes": codes, "rank_of": rank_of,
                "sym_of_rank": order, "qlc_bits": list(qlc_bits)}
    raise ValueError(kind)


def entropy_bits(counts) -> float:
    """Order-0 Shannon entropy (bits/symbol) of an empirical histogram."""
    tot = sum(int(c) for c in counts)
    if tot == 0:
        return 0.0
    h = 0.0
    for c in counts:
        if c:
            p = int(c) / tot
            h -= p * math.log2(p)
    return h


def coded_bits(counts, lengths) -> int:
    """Total payload bits of a stream with these counts: sum(count * length)."""
    return sum(int(c) * int(l) for c, l in zip(counts, lengths))


def per_shard_lengths(counts, max_len=MAX_LEN):
    """Three-stage comparator: a length-limited code built on the tensor's own
    counts, over the symbols that occur (absent symbols get no code)."""
    present = [s for s in range(len(counts)) if counts[s] > 0]
    sub = package_merge([counts[s] for s in present], max_len)
    lengths = [0] * len(counts)
    for s, l in zip(present, sub):
        lengths[s] = l
    return lengths


def compressibility(bits_per_symbol: float) -> float:
    """Saved fraction of the 8-bit representation: 1 - b/8."""
    return 1.0 - bits_per_symbol / 8.0


def qlc_cost(counts, bits) -> int:
    """Total bits of a histogram under QLC widths ``bits`` (ranked counts)."""
    lengths, _, _, _ = qlc_code(counts, bits)
    return coded_bits(counts, lengths)


def qlc_optimal_bits_bruteforce(counts):
    """The plain definition of the best QLC layout: among all 10**8 width
    vectors (each width 0..9, areas covering 256 ranks) the one of least total
    bits, ties to the lexicographically smallest vector.  Exhaustive, with
    numpy evaluating the last four areas of every vector at once."""
    ranked = [int(counts[s]) for s in qlc_rank(counts)]
    pre = np.zeros(ALPHABET + 1, dtype=np.int64)
    pre[1:] = np.cumsum(np.array(ranked, dtype=np.int64))
    widths = np.arange(10)
    tail = np.array(list(itertools.product(range(10), repeat=4)), dtype=np.int64)  # lexicographic
    best = None
    for head in itertools.product(range(10), repeat=4):
        start = 0
        cost_head = 0
        for b in head:
            end = min(start + (1 << b), ALPHABET)
            cost_head += (3 + b) * int(pre[end] - pre[start])
            start = end
        st = np.full(len(tail), start, dtype=np.int64)
        cost = np.full(len(tail), cost_head, dtype=np.int64)
        for k in range(4):
            b = tail[:, k]
            end = np.minimum(st + (1 << b), ALPHABET)
            cost += (3 + b) * (pre[end] - pre[st])
            st = end
        cost[st < ALPHABET] = np.iinfo(np.int64).max  # does not cover 256 ranks
        i = int(np.argmin(cost))  # first minimum = lexicographically smallest tail
        cand = (int(cost[i]), tuple(head) + tuple(int(v) for v in tail[i]))
        if best is None or cand[0] < best[0]:
            best = cand
    del widths
    return best[1]
