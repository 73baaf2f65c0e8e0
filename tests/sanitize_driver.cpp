// Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
// library's codebook construction (codebook.cpp) and the oracle's
// bit-serial coder (oracle/coder.c), driven over edge cases, random inputs,
// invalid arguments and corrupted streams.  Built and run by
// test_sanitizers.py with -fsanitize=address,undefined and no recovery, so
// any report ends the run with a non-zero status; the checks below add
// round-trip and status expectations.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "pc.h"

extern "C" {
int oracle_encode(const uint8_t *in, uint64_t n, uint64_t chunk, const uint8_t len[256], const uint16_t code[256],
                  uint32_t *payload, uint64_t capacity_words, uint32_t *chunk_bits, uint64_t *chunk_word_offset,
                  uint32_t *sub_off, int threads);
int oracle_decode(const uint32_t *payload, uint64_t payload_words, const uint32_t *chunk_bits,
                  const uint64_t *chunk_word_offset, const uint32_t *sub_off, uint64_t n, uint64_t chunk,
                  const uint8_t len[256], int qlc, const uint8_t qlc_bits[8], const uint8_t sym_of_rank[256],
                  uint8_t *out, int threads);
}

static int g_fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++g_fails;                                                        \
        }                                                                     \
    } while (0)

static std::vector<std::vector<uint64_t>> count_cases(std::mt19937_64 &rng) {
    std::vector<std::vector<uint64_t>> cs;
    cs.push_back(std::vector<uint64_t>(256, 0));  // empty histogram
    std::vector<uint64_t> one(256, 0);
    one[77] = 1000;
    cs.push_back(one);  // a single symbol
    std::vector<uint64_t> two(256, 0);
    two[0] = 3;
    two[255] = 1;
    cs.push_back(two);
    cs.push_back(std::vector<uint64_t>(256, 5));  // uniform
    std::vector<uint64_t> geo(256);
    for (int s = 0; s < 256; ++s) geo[s] = s < 60 ? (1ull << (60 - s)) : 0;  // steeper than 12 bits allow
    cs.push_back(geo);
    std::vector<uint64_t> big(256);
    for (int s = 0; s < 256; ++s) big[s] = (1ull << 40) + (uint64_t)s * 977;
    cs.push_back(big);
    for (int k = 0; k < 12; ++k) {
        std::vector<uint64_t> r(256);
        std::uniform_real_distribution<double> u(0.0, 1.0);
        for (int s = 0; s < 256; ++s) {
            const double p = u(rng);
            r[s] = (k % 3 == 0 && p < 0.3) ? 0 : (uint64_t)(1000.0 / (p * p * p + 1e-6));
        }
        cs.push_back(r);
    }
    return cs;
}

static void codebook_calls(const std::vector<uint64_t> &c) {
    pc_codebook h, q;
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_HUFFMAN, nullptr, &h) == PC_OK);
    CHECK(pc_codebook_validate(&h) == PC_OK);
    uint8_t bits[8];
    CHECK(pc_qlc_optimal_bits(c.data(), bits) == PC_OK);
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_QLC, bits, &q) == PC_OK);
    CHECK(pc_codebook_validate(&q) == PC_OK);
    double avg = 0, ent = 0;
    CHECK(pc_codebook_fit(&h, c.data(), &avg, &ent) == PC_OK);
    CHECK(pc_codebook_fit(&q, c.data(), &avg, &ent) == PC_OK);
    uint8_t lens[256];
    CHECK(pc_shard_code_lengths(c.data(), lens) == PC_OK);
    // a damaged blob is rejected, not read past its tables
    pc_codebook bad = h;
    bad.length[3] = 0;
    CHECK(pc_codebook_validate(&bad) != PC_OK);
    bad = h;
    bad.magic ^= 1u;
    CHECK(pc_codebook_validate(&bad) != PC_OK);
}

static void invalid_calls() {
    std::vector<uint64_t> c(256, 1);
    pc_codebook cb;
    const uint8_t short_areas[8] = {1, 1, 1, 1, 1, 1, 1, 1};  // 16 slots < 256
    const uint8_t wide_areas[8] = {20, 0, 0, 0, 0, 0, 0, 0};
    CHECK(pc_codebook_build(nullptr, PC_CODEBOOK_HUFFMAN, nullptr, &cb) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_HUFFMAN, nullptr, nullptr) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_build(c.data(), 7, nullptr, &cb) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_QLC, nullptr, &cb) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_QLC, short_areas, &cb) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_build(c.data(), PC_CODEBOOK_QLC, wide_areas, &cb) == PC_ERR_INVALID_ARG);
    CHECK(pc_codebook_validate(nullptr) == PC_ERR_INVALID_ARG);
    CHECK(pc_qlc_optimal_bits(nullptr, nullptr) == PC_ERR_INVALID_ARG);
    CHECK(pc_shard_code_lengths(nullptr, nullptr) == PC_ERR_INVALID_ARG);
    for (int s = -2; s < 12; ++s) CHECK(pc_status_string(s) != nullptr);
}

struct Stream {
    std::vector<uint32_t> payload, chunk_bits, sub_off;
    std::vector<uint64_t> cwo;
};

static Stream encode(const std::vector<uint8_t> &x, uint64_t chunk, const pc_codebook &cb, int threads) {
    const uint64_t n = x.size(), nc = (n + chunk - 1) / chunk;
    Stream s;
    s.payload.assign(n * 12 / 32 + 2 * nc + 1, 0u);
    s.chunk_bits.assign(nc + 1, 0u);
    s.cwo.assign(nc + 1, 0u);
    s.sub_off.assign((n + 255) / 256 + 1, 0u);
    CHECK(oracle_encode(x.data(), n, chunk, cb.length, cb.code, s.payload.data(), s.payload.size(),
                        s.chunk_bits.data(), s.cwo.data(), s.sub_off.data(), threads) == 0);
    return s;
}

static int decode(const Stream &s, uint64_t words, uint64_t n, uint64_t chunk, const pc_codebook &cb, int qlc,
                  std::vector<uint8_t> &out, int threads) {
    out.assign(n + 1, 0xEE);
    return oracle_decode(s.payload.data(), words, s.chunk_bits.data(), s.cwo.data(), s.sub_off.data(), n, chunk,
                         cb.length, qlc, cb.qlc_bits, cb.sym_of_rank, out.data(), threads);
}

static void coder_calls(std::mt19937_64 &rng) {
    std::vector<uint64_t> counts(256);
    for (int s = 0; s < 256; ++s) counts[s] = 1 + (1000000ull >> (s % 20));
    pc_codebook h, q;
    CHECK(pc_codebook_build(counts.data(), PC_CODEBOOK_HUFFMAN, nullptr, &h) == PC_OK);
    const uint8_t layout[8] = {1, 3, 3, 3, 3, 5, 6, 7};
    CHECK(pc_codebook_build(counts.data(), PC_CODEBOOK_QLC, layout, &q) == PC_OK);
    for (uint64_t chunk : {(uint64_t)256, (uint64_t)4096, (uint64_t)65536}) {
        for (uint64_t n : {(uint64_t)0, (uint64_t)1, (uint64_t)255, (uint64_t)256, (uint64_t)257, chunk - 1, chunk,
                           chunk + 1, 3 * chunk + 100}) {
            std::vector<uint8_t> x(n);
            std::geometric_distribution<int> g(0.15);
            for (auto &b : x) b = (uint8_t)(g(rng) % 256);
            for (const pc_codebook *cb : {&h, &q}) {
                const int qlc = cb == &q;
                const int threads = n > 4 * chunk ? 3 : 1;
                Stream s = encode(x, chunk, *cb, threads);
                const uint64_t nc = (n + chunk - 1) / chunk;
                const uint64_t words = s.cwo[nc];
                std::vector<uint8_t> out;
                CHECK(decode(s, words, n, chunk, *cb, qlc, out, threads) == 0);
                CHECK((n == 0 || std::memcmp(out.data(), x.data(), n) == 0) && out[n] == 0xEE);
                if (n == 0) continue;
                // corruptions: flipped payload bits, a short payload, bad
                // side-index entries, bad chunk tables -- any status, but no
                // access outside the buffers and no write past n
                for (int t = 0; t < 6; ++t) {
                    Stream c = s;
                    if (words) c.payload[rng() % words] ^= 1u << (rng() % 32);
                    decode(c, words, n, chunk, *cb, qlc, out, 1);
                    CHECK(out[n] == 0xEE);
                }
                decode(s, words / 2, n, chunk, *cb, qlc, out, 1);
                CHECK(out[n] == 0xEE);
                for (uint32_t v : {0xFFFFFFFFu, 0x7FFFFFFFu, (uint32_t)(words * 32 + 5)}) {
                    Stream c = s;
                    c.sub_off[(rng() % ((n + 255) / 256))] = v;
                    decode(c, words, n, chunk, *cb, qlc, out, 1);
                    CHECK(out[n] == 0xEE);
                }
                {
                    Stream c = s;
                    c.chunk_bits[0] = 0xFFFFFFFFu;
                    CHECK(decode(c, words, n, chunk, *cb, qlc, out, 1) != 0);
                    c = s;
                    c.cwo[nc] = words + 1000;
                    CHECK(decode(c, words, n, chunk, *cb, qlc, out, 1) != 0);
                }
            }
        }
    }
    // invalid oracle arguments
    std::vector<uint8_t> x(1000, 1);
    Stream s;
    s.payload.assign(1000, 0u);
    s.chunk_bits.assign(8, 0u);
    s.cwo.assign(8, 0u);
    s.sub_off.assign(8, 0u);
    CHECK(oracle_encode(x.data(), x.size(), 300, h.length, h.code, s.payload.data(), 1000, s.chunk_bits.data(),
                        s.cwo.data(), s.sub_off.data(), 1) != 0);
    CHECK(oracle_encode(x.data(), x.size(), 256, h.length, h.code, s.payload.data(), 1, s.chunk_bits.data(),
                        s.cwo.data(), s.sub_off.data(), 1) != 0);
}

int main() {
    std::mt19937_64 rng(12345);
    for (const auto &c : count_cases(rng)) codebook_calls(c);
    invalid_calls();
    coder_calls(rng);
    if (g_fails) {
        std::fprintf(stderr, "%d checks failed\n", g_fails);
        return 1;
    }
    std::printf("sanitized host code: all checks passed\n");
    return 0;
}
