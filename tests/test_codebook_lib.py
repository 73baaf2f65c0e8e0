"""Host logic of libpc.so against the oracle (no GPU needed: codebook build,
validation and size queries are host functions)."""
import numpy as np
import pytest

import static_codebook_lossless_amd as pc
import workloads as W
from oracle import codebook as cb
from oracle import coder


def lib_book(counts, kind="huffman", bits=None):
    blob = pc.pc_codebook_build(np.asarray(counts, dtype=np.uint64), kind, bits)
    pc.pc_codebook_validate(blob)
    return pc.codebook_fields(blob)


def check_same(counts, kind="huffman", bits=None):
    f = lib_book(counts, kind, bits)
    o = cb.codebook([int(c) for c in counts], kind, bits)
    assert f["length"].tolist() == o["lengths"]
    assert f["code"].tolist() == o["codes"]
    if kind == "qlc":
        assert f["sym_of_rank"].tolist() == o["sym_of_rank"]
        assert f["rank_of"].tolist() == o["rank_of"]
    return f, o


@pytest.mark.parametrize("seed", range(40))
def test_huffman_matches_oracle_random_histograms(seed):
    rng = np.random.default_rng(seed)
    mode = seed % 4
    if mode == 0:
        counts = rng.integers(0, 10**6, 256)
    elif mode == 1:  # heavy ties
        counts = rng.integers(0, 4, 256) * 1000
    elif mode == 2:  # most symbols absent
        counts = np.zeros(256, dtype=np.int64)
        counts[rng.choice(256, 20, replace=False)] = rng.integers(1, 10**9, 20)
    else:  # geometric: the 12-bit limit binds
        counts = (2.0 ** (40 - rng.permutation(256) % 41)).astype(np.int64)
    check_same(counts)


@pytest.mark.parametrize("name", ["normal_1m", "ffn1_act", "gelu_act", "int8_weight"])
def test_huffman_matches_oracle_on_workloads(name):
    x = W.make(name, 1)
    counts = np.bincount(x, minlength=256)
    f, o = check_same(counts)
    assert f["complete"] == 1 and max(o["lengths"]) == 12


@pytest.mark.parametrize("bits", [(1, 3, 3, 3, 3, 5, 6, 7), (3, 3, 3, 3, 3, 4, 7, 7), (8, 0, 0, 0, 0, 0, 0, 0),
                                  (0, 1, 2, 3, 4, 5, 6, 8), (9, 9, 9, 9, 9, 9, 9, 9)])
@pytest.mark.parametrize("seed", range(3))
def test_qlc_matches_oracle(bits, seed):
    rng = np.random.default_rng(50 + seed)
    counts = rng.integers(0, 50, 256) * (seed + 1)  # many ties
    check_same(counts, "qlc", bits)


def test_decode_tables_follow_the_codes():
    rng = np.random.default_rng(9)
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7))):
        f = lib_book(rng.integers(0, 10**5, 256), kind, bits)
        strs = [cb.code_string(int(c), int(l)) for c, l in zip(f["code"], f["length"])]
        for peek in range(4096):
            p = format(peek, "012b")
            match = [s for s in range(256) if p.startswith(strs[s])]
            if match:
                assert f["dec_sym"][peek] == match[0] and f["dec_len"][peek] == len(strs[match[0]])
            else:
                assert f["dec_len"][peek] == 0
        assert f["complete"] == (1 if kind == "huffman" else 0)


def test_invalid_arguments_rejected():
    with pytest.raises(pc.PcError):
        pc.pc_codebook_build(np.ones(256, np.uint64), "qlc", (1, 1, 1, 1, 1, 1, 1, 1))  # covers 16 ranks
    with pytest.raises(pc.PcError):
        pc.pc_codebook_build(np.ones(256, np.uint64), "qlc", (10, 0, 0, 0, 0, 0, 0, 0))  # 13-bit codes
    with pytest.raises(pc.PcError):
        pc.pc_codebook_build(np.ones(256, np.uint64), 7)
    blob = pc.pc_codebook_build(np.ones(256, np.uint64))
    bad = blob.clone()
    bad[800] ^= 1  # decode table no longer matches the codes
    with pytest.raises(pc.PcError):
        pc.pc_codebook_validate(bad)
    assert pc.pc_num_chunks(100, 100) == 0  # chunk not a multiple of 256


@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 4095, 4097, 3 * 4096 + 100, 1 << 20])
@pytest.mark.parametrize("chunk", [256, 768, 4096, 65536])
def test_size_queries_match_oracle(n, chunk):
    assert pc.pc_num_chunks(n, chunk) == coder.num_chunks(n, chunk)
    assert pc.pc_num_substreams(n, chunk) == coder.num_substreams(n, chunk)
    assert pc.pc_max_payload_words(n, chunk) == coder.max_payload_words(n, chunk)
    assert pc.pc_encode_workspace_bytes(n, chunk) >= 8 * (1 + coder.num_chunks(n, chunk))


@pytest.mark.parametrize("seed", range(6))
def test_shard_code_lengths_match_oracle(seed):
    rng = np.random.default_rng(90 + seed)
    counts = rng.integers(0, 10**6, 256)
    counts[rng.random(256) < [0.0, 0.1, 0.5, 0.9, 0.98, 0.3][seed]] = 0  # absent byte values
    if seed == 5:
        counts = (rng.pareto(0.7, 256) * 10).astype(np.int64)  # skewed: the 12-bit limit binds
    got = pc.pc_shard_code_lengths(counts)
    want = cb.per_shard_lengths([int(c) for c in counts])
    assert got.tolist() == want


@pytest.mark.parametrize("name", ["normal_1m", "int8_weight"])
def test_shard_code_lengths_match_oracle_on_workloads(name):
    counts = np.bincount(W.make(name, 0), minlength=256)
    assert pc.pc_shard_code_lengths(counts).tolist() == cb.per_shard_lengths([int(c) for c in counts])


def test_shard_code_lengths_degenerate():
    assert pc.pc_shard_code_lengths(np.zeros(256, dtype=np.uint64)).tolist() == [0] * 256
    one = np.zeros(256, dtype=np.uint64)
    one[9] = 5
    got = pc.pc_shard_code_lengths(one)
    assert got[9] == 1 and int(got.sum()) == 1
    two = np.zeros(256, dtype=np.uint64)
    two[[0, 255]] = [3, 1000]
    assert pc.pc_shard_code_lengths(two)[[0, 255]].tolist() == [1, 1]


@pytest.mark.parametrize("seed", range(2))
def test_qlc_optimal_bits_matches_exhaustive_search(seed):
    rng = np.random.default_rng(70 + seed)
    counts = (rng.pareto(1.0, 256) * 1000).astype(np.int64)
    bits = pc.pc_qlc_optimal_bits(counts)
    assert bits == cb.qlc_optimal_bits_bruteforce([int(c) for c in counts])


def test_qlc_optimal_bits_on_gelu_beats_table2_layout():
    x = W.make("gelu_act", 1)
    counts = [int(c) for c in np.bincount(x, minlength=256)]
    bits = pc.pc_qlc_optimal_bits(np.array(counts))
    assert cb.qlc_cost(counts, bits) <= cb.qlc_cost(counts, (1, 3, 3, 3, 3, 5, 6, 7))


# ---- codebook fit and refresh (pc_codebook_fit, CodebookRefresh) ----------

@pytest.mark.parametrize("seed", range(12))
def test_codebook_fit_matches_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    build = rng.integers(0, 1 << 20, 256).astype(np.uint64)
    batch = (rng.integers(0, 1 << 16, 256) * (rng.random(256) < 0.7)).astype(np.uint64)
    for kind, bits in (("huffman", None), ("qlc", (1, 3, 3, 3, 3, 5, 6, 7))):
        blob = pc.pc_codebook_build(build, kind, bits)
        avg, ent = pc.pc_codebook_fit(blob, batch)
        lengths = cb.codebook([int(c) for c in build], kind, bits)["lengths"]
        n = int(batch.sum())
        assert avg == pytest.approx(cb.coded_bits([int(c) for c in batch], lengths) / n, rel=1e-12)
        assert ent == pytest.approx(cb.entropy_bits([int(c) for c in batch]), rel=1e-12)
        assert avg >= ent - 1e-12  # no prefix code beats the entropy


def test_codebook_fit_closed_forms():
    blob = pc.pc_codebook_build(np.ones(256, dtype=np.uint64))  # 8 bits for every byte
    uniform = np.full(256, 7, dtype=np.uint64)
    assert pc.pc_codebook_fit(blob, uniform) == pytest.approx((8.0, 8.0))
    two = np.zeros(256, dtype=np.uint64)
    two[[3, 200]] = 5
    assert pc.pc_codebook_fit(blob, two) == pytest.approx((8.0, 1.0))
    dyadic = np.zeros(256, dtype=np.uint64)
    dyadic[[0, 1, 2, 3]] = [4, 2, 1, 1]  # p = 1/2, 1/4, 1/8, 1/8
    assert pc.pc_codebook_fit(blob, dyadic)[1] == pytest.approx(1.75)
    # every byte dyadic (lengths 1, 2, 3, 250 x 11, 3 x 10: Kraft sum 1): the
    # optimal code has exactly these lengths, so its average is the entropy
    full = np.array([1024, 512, 256] + [1] * 250 + [2] * 3, dtype=np.uint64)
    h = (1024 * 1 + 512 * 2 + 256 * 3 + 250 * 11 + 6 * 10) / 2048
    avg, ent = pc.pc_codebook_fit(pc.pc_codebook_build(full), full)
    assert ent == pytest.approx(h, rel=1e-12)
    assert avg == pytest.approx(h, rel=1e-12)
    assert pc.pc_codebook_fit(blob, np.zeros(256, dtype=np.uint64)) == (0.0, 0.0)


def test_codebook_fit_rejects_bad_blob():
    blob = pc.pc_codebook_build(np.ones(256, dtype=np.uint64)).clone()
    blob[0] ^= 1  # magic
    with pytest.raises(pc.PcError):
        pc.pc_codebook_fit(blob, np.ones(256, dtype=np.uint64))


def _e4m3_batch(seed, draw):
    rng = np.random.default_rng(seed)
    return np.bincount(W.e4m3_from_f32(draw(rng, 1 << 16).astype(np.float32)), minlength=256).astype(np.uint64)


def test_refresh_rebuilds_only_on_drift():
    normal = lambda rng, n: rng.standard_normal(n)  # noqa: E731
    heavy = lambda rng, n: rng.standard_t(2, n)     # noqa: E731  (a heavy-tailed drift)
    r = pc.CodebookRefresh(window=4, threshold=0.02)
    assert r.observe(_e4m3_batch(1, normal))  # first batch: a codebook is built
    for s in range(2, 7):  # same distribution, new seeds: the fixed codebook keeps fitting
        assert not r.observe(_e4m3_batch(s, normal))
        avg, ent = r.last_fit
        assert (avg - ent) / ent < 0.02
    drifted = _e4m3_batch(7, heavy)
    before = pc.pc_codebook_fit(r.codebook, drifted)
    assert r.observe(drifted)  # the gap grew past the threshold: rebuilt
    assert r.rebuilds == 2
    # the rebuilt codebook pools the window (3 old batches + the drifted one)
    pooled = r.pooled()
    assert pc.codebook_fields(r.codebook)["length"].tolist() == cb.codebook([int(c) for c in pooled])["lengths"]
    after = pc.pc_codebook_fit(r.codebook, drifted)
    assert after[0] < before[0]


def test_refresh_qlc_widths_follow_the_pool():
    r = pc.CodebookRefresh(kind="qlc")
    c = _e4m3_batch(11, lambda rng, n: rng.standard_normal(n))
    assert r.observe(c)
    f = pc.codebook_fields(r.codebook)
    assert tuple(f["qlc_bits"].tolist()) == pc.pc_qlc_optimal_bits(c)
