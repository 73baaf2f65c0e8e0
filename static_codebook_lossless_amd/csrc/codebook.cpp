// Host-side construction of the fixed codebook (libpc.so).
//
// "Single-Stage Huffman Encoder for ML Compression" (abstract): the codebook
// is derived offline from the average distribution of previous batches and
// never travels with the data.  "Quad Length Codes for Lossless Compression
// of e4m3" (abstract, Tables 1 and 2): 8 areas selected by a 3-bit prefix,
// each with its own fixed index width, over the probability-ranked symbols.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "pc.h"

static_assert(sizeof(pc_codebook) == 9536, "pc_codebook layout");
static_assert(offsetof(pc_codebook, length) == 32, "layout");
static_assert(offsetof(pc_codebook, code) == 288, "layout");
static_assert(offsetof(pc_codebook, dec_sym) == 800, "layout");
static_assert(offsetof(pc_codebook, dec_len) == 4896, "layout");
static_assert(offsetof(pc_codebook, qlc_bits) == 8992, "layout");
static_assert(offsetof(pc_codebook, qlc_start) == 9000, "layout");
static_assert(offsetof(pc_codebook, rank_of) == 9016, "layout");
static_assert(offsetof(pc_codebook, sym_of_rank) == 9272, "layout");

namespace {

constexpr int kN = PC_ALPHABET;
constexpr int kL = PC_MAX_LEN;

// Package-merge (coin collector) for n weights (2 <= n <= 256) and depth
// limit L.
//
// Level lists are built bottom-up: the deepest list is the sorted leaves;
// each shallower list merges the leaves with the pairs ("packages") of the
// list below, a leaf going first on equal weight.  The optimal collection is
// the first 2n-2 items of the top list.  Because packages are formed from
// consecutive pairs and lists are merged in order, the selected items of
// every level form a prefix of that level's list; a leaf's code length is
// the number of levels whose selected prefix contains it.
void package_merge_lengths(const uint64_t *w, int n, uint8_t *len_out) {
    int order[kN];
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order, order + n, [&](int a, int b) {
        return w[a] < w[b] || (w[a] == w[b] && a < b);
    });
    std::vector<uint64_t> leafw(n);
    for (int i = 0; i < n; ++i) leafw[i] = w[order[i]];

    // is_pkg[level][k]: whether item k of the level's list is a package.
    // Level 0 is the deepest list (leaves only), level L-1 the top.
    std::vector<std::vector<uint8_t>> is_pkg(kL);
    std::vector<uint64_t> cur(leafw);
    is_pkg[0].assign(n, 0);
    for (int lev = 1; lev < kL; ++lev) {
        const size_t npk = cur.size() / 2;
        std::vector<uint64_t> next;
        std::vector<uint8_t> flags;
        next.reserve(n + npk);
        flags.reserve(n + npk);
        size_t i = 0, j = 0;
        while (i < (size_t)n || j < npk) {
            uint64_t pw = j < npk ? cur[2 * j] + cur[2 * j + 1] : 0;
            bool take_leaf = j >= npk || (i < (size_t)n && leafw[i] <= pw);
            if (take_leaf) {
                next.push_back(leafw[i++]);
                flags.push_back(0);
            } else {
                next.push_back(pw);
                flags.push_back(1);
                ++j;
            }
        }
        cur.swap(next);
        is_pkg[lev].swap(flags);
    }
    // Walk down from the top list: prefix m selected at this level; the
    // leaves in the prefix each gain one bit; the packages in it select a
    // prefix of twice their number in the level below.
    int depth[kN] = {0};
    size_t m = 2 * (size_t)n - 2;
    for (int lev = kL - 1; lev >= 0; --lev) {
        size_t leaves = 0, pkgs = 0;
        const auto &f = is_pkg[lev];
        for (size_t k = 0; k < m && k < f.size(); ++k) (f[k] ? pkgs : leaves)++;
        for (size_t k = 0; k < leaves; ++k) depth[k]++;
        m = 2 * pkgs;
    }
    for (int i = 0; i < n; ++i) len_out[order[i]] = (uint8_t)depth[i];
}

// Canonical code values: symbols in (length, byte value) order, consecutive
// values within a length, shifted left where the length grows.
void canonical_codes(const uint8_t *len, uint16_t *code) {
    int count[kL + 2] = {0};
    for (int s = 0; s < kN; ++s) count[len[s]]++;
    uint32_t next[kL + 2] = {0};
    uint32_t c = 0;
    count[0] = 0;
    for (int l = 1; l <= kL; ++l) {
        c = (c + count[l - 1]) << 1;
        next[l] = c;
    }
    // next[l] is the first code of length l; the loop above starts at 0 for
    // the shortest length in use because lower lengths have count 0.
    for (int s = 0; s < kN; ++s) code[s] = (uint16_t)next[len[s]]++;
}

uint32_t fnv1a(uint32_t h, const void *p, size_t n) {
    const uint8_t *b = static_cast<const uint8_t *>(p);
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 16777619u;
    }
    return h;
}

void fill_tables(pc_codebook *cb) {
    std::memset(cb->dec_sym, 0, sizeof cb->dec_sym);
    std::memset(cb->dec_len, 0, sizeof cb->dec_len);
    uint32_t kraft4096 = 0;
    uint32_t maxl = 0;
    for (int s = 0; s < kN; ++s) {
        const uint32_t l = cb->length[s];
        const uint32_t span = 1u << (kL - l);
        const uint32_t first = (uint32_t)cb->code[s] << (kL - l);
        for (uint32_t p = first; p < first + span; ++p) {
            cb->dec_sym[p] = (uint8_t)s;
            cb->dec_len[p] = (uint8_t)l;
        }
        kraft4096 += span;
        maxl = std::max(maxl, l);
    }
    cb->max_len = maxl;
    cb->complete = kraft4096 == (1u << kL) ? 1u : 0u;
    uint32_t h = 2166136261u;
    uint32_t kind = cb->kind;
    h = fnv1a(h, &kind, 4);
    h = fnv1a(h, cb->length, kN);
    h = fnv1a(h, cb->qlc_bits, PC_QLC_AREAS);
    cb->codebook_id = h;
}

void rank_symbols(const uint64_t *counts, uint8_t *sym_of_rank, uint8_t *rank_of) {
    int order[kN];
    for (int i = 0; i < kN; ++i) order[i] = i;
    std::stable_sort(order, order + kN, [&](int a, int b) {
        return counts[a] > counts[b] || (counts[a] == counts[b] && a < b);
    });
    for (int r = 0; r < kN; ++r) {
        sym_of_rank[r] = (uint8_t)order[r];
        rank_of[order[r]] = (uint8_t)r;
    }
}

bool qlc_bits_ok(const uint8_t *bits) {
    uint32_t cover = 0;
    for (int a = 0; a < PC_QLC_AREAS; ++a) {
        if (bits[a] > kL - 3) return false;
        cover += 1u << bits[a];
    }
    return cover >= (uint32_t)kN;
}

}  // namespace

extern "C" {

const char *pc_status_string(int status) {
    switch (status) {
        case PC_OK: return "ok";
        case PC_ERR_INVALID_ARG: return "invalid argument";
        case PC_ERR_UNSUPPORTED: return "unsupported";
        case PC_ERR_CAPACITY: return "buffer too small";
        case PC_ERR_CORRUPT: return "corrupt stream";
        case PC_ERR_HIP: return "HIP runtime error";
        case PC_ERR_TIMEOUT: return "device wait gave up";
        default: return "unknown status";
    }
}

pc_status pc_codebook_build(const uint64_t counts[256], int kind, const uint8_t qlc_bits[8],
                            pc_codebook *out) {
    if (!counts || !out) return PC_ERR_INVALID_ARG;
    pc_codebook cb;
    std::memset(&cb, 0, sizeof cb);
    cb.magic = PC_CODEBOOK_MAGIC;
    cb.version = PC_CODEBOOK_VERSION;
    cb.kind = (uint32_t)kind;
    if (kind == PC_CODEBOOK_HUFFMAN) {
        if (qlc_bits) return PC_ERR_INVALID_ARG;
        uint64_t w[kN];
        for (int s = 0; s < kN; ++s) w[s] = counts[s] ? counts[s] : 1;  // every byte stays codable
        package_merge_lengths(w, kN, cb.length);
        canonical_codes(cb.length, cb.code);
    } else if (kind == PC_CODEBOOK_QLC) {
        if (!qlc_bits || !qlc_bits_ok(qlc_bits)) return PC_ERR_INVALID_ARG;
        std::memcpy(cb.qlc_bits, qlc_bits, PC_QLC_AREAS);
        rank_symbols(counts, cb.sym_of_rank, cb.rank_of);
        uint32_t start = 0;
        for (int a = 0; a < PC_QLC_AREAS; ++a) {
            cb.qlc_start[a] = (uint16_t)std::min<uint32_t>(start, 0xFFFFu);
            const uint32_t slots = 1u << qlc_bits[a];
            for (uint32_t r = start; r < start + slots && r < (uint32_t)kN; ++r) {
                const int s = cb.sym_of_rank[r];
                cb.length[s] = (uint8_t)(3 + qlc_bits[a]);
                cb.code[s] = (uint16_t)(((uint32_t)a << qlc_bits[a]) | (r - start));
            }
            start += slots;
        }
    } else {
        return PC_ERR_INVALID_ARG;
    }
    fill_tables(&cb);
    *out = cb;
    return PC_OK;
}

pc_status pc_codebook_validate(const pc_codebook *cb) {
    if (!cb) return PC_ERR_INVALID_ARG;
    if (cb->magic != PC_CODEBOOK_MAGIC || cb->version != PC_CODEBOOK_VERSION) return PC_ERR_INVALID_ARG;
    if (cb->kind != PC_CODEBOOK_HUFFMAN && cb->kind != PC_CODEBOOK_QLC) return PC_ERR_INVALID_ARG;
    uint32_t kraft4096 = 0;
    for (int s = 0; s < kN; ++s) {
        if (cb->length[s] < 1 || cb->length[s] > kL) return PC_ERR_INVALID_ARG;
        if (cb->code[s] >> cb->length[s]) return PC_ERR_INVALID_ARG;
        kraft4096 += 1u << (kL - cb->length[s]);
    }
    if (kraft4096 > (1u << kL)) return PC_ERR_INVALID_ARG;
    // the decode tables must agree with the codes
    for (int s = 0; s < kN; ++s) {
        const uint32_t l = cb->length[s];
        const uint32_t first = (uint32_t)cb->code[s] << (kL - l);
        for (uint32_t p = first; p < first + (1u << (kL - l)); ++p)
            if (cb->dec_sym[p] != s || cb->dec_len[p] != l) return PC_ERR_INVALID_ARG;
    }
    if (cb->kind == PC_CODEBOOK_QLC && !qlc_bits_ok(cb->qlc_bits)) return PC_ERR_INVALID_ARG;
    return PC_OK;
}

pc_status pc_codebook_fit(const pc_codebook *cb, const uint64_t counts[256], double *avg_bits, double *entropy) {
    if (!counts || !avg_bits || !entropy) return PC_ERR_INVALID_ARG;
    if (pc_codebook_validate(cb) != PC_OK) return PC_ERR_INVALID_ARG;
    long double total = 0, bits = 0;
    for (int s = 0; s < kN; ++s) {
        total += (long double)counts[s];
        bits += (long double)counts[s] * cb->length[s];
    }
    if (total == 0) {
        *avg_bits = 0;
        *entropy = 0;
        return PC_OK;
    }
    long double h = 0;
    for (int s = 0; s < kN; ++s) {
        if (!counts[s]) continue;
        const long double p = (long double)counts[s] / total;
        h -= p * std::log2(p);
    }
    *avg_bits = (double)(bits / total);
    *entropy = (double)h;
    return PC_OK;
}

// The comparator of a per-shard ("three-stage") code: package-merge on the
// shard's own counts over the byte values that occur, so an absent value
// gets no codeword; one present value gets a 1-bit code.
pc_status pc_shard_code_lengths(const uint64_t counts[256], uint8_t lengths_out[256]) {
    if (!counts || !lengths_out) return PC_ERR_INVALID_ARG;
    uint64_t w[kN];
    int sym[kN], n = 0;
    for (int s = 0; s < kN; ++s) {
        lengths_out[s] = 0;
        if (counts[s]) {
            w[n] = counts[s];
            sym[n++] = s;
        }
    }
    if (n == 1) lengths_out[sym[0]] = 1;
    if (n < 2) return PC_OK;
    uint8_t sub[kN];
    package_merge_lengths(w, n, sub);
    for (int i = 0; i < n; ++i) lengths_out[sym[i]] = sub[i];
    return PC_OK;
}

// Dynamic programme over contiguous rank ranges: best[a][r] = least cost of
// coding ranks r..255 with areas a..7.  Area a of width b covers
// [r, r + 2^b); every symbol in it costs 3 + b bits.
pc_status pc_qlc_optimal_bits(const uint64_t counts[256], uint8_t bits_out[8]) {
    if (!counts || !bits_out) return PC_ERR_INVALID_ARG;
    uint8_t sym_of_rank[kN], rank_of[kN];
    rank_symbols(counts, sym_of_rank, rank_of);
    // prefix sums of counts in rank order; 128-bit so that 256 counts of up
    // to 2^64 - 1, times 12 bits, cannot overflow
    std::vector<unsigned __int128> ipre(kN + 1, 0);
    for (int r = 0; r < kN; ++r) ipre[r + 1] = ipre[r] + counts[sym_of_rank[r]];
    constexpr int kA = PC_QLC_AREAS, kB = kL - 3;
    const unsigned __int128 INF = ~(unsigned __int128)0;
    std::vector<std::vector<unsigned __int128>> best(kA + 1, std::vector<unsigned __int128>(kN + 1));
    for (int r = 0; r <= kN; ++r) best[kA][r] = (r == kN) ? 0 : INF;
    for (int a = kA - 1; a >= 0; --a) {
        for (int r = 0; r <= kN; ++r) {
            unsigned __int128 m = INF;
            for (int b = 0; b <= kB; ++b) {
                const int e = std::min(kN, r + (1 << b));
                if (best[a + 1][e] == INF) continue;
                const unsigned __int128 c = (unsigned __int128)(3 + b) * (ipre[e] - ipre[r]) + best[a + 1][e];
                if (c < m) m = c;
            }
            best[a][r] = m;
        }
    }
    int r = 0;
    for (int a = 0; a < kA; ++a) {
        for (int b = 0; b <= kB; ++b) {
            const int e = std::min(kN, r + (1 << b));
            if (best[a + 1][e] == INF) continue;
            const unsigned __int128 c = (unsigned __int128)(3 + b) * (ipre[e] - ipre[r]) + best[a + 1][e];
            if (c == best[a][r]) {
                bits_out[a] = (uint8_t)b;
                r = e;
                break;
            }
        }
    }
    return PC_OK;
}

size_t pc_num_chunks(size_t n, size_t chunk) {
    if (chunk < PC_SUBSTREAM || chunk % PC_SUBSTREAM || chunk > ((size_t)1 << 24)) return 0;
    return (n + chunk - 1) / chunk;
}

size_t pc_num_substreams(size_t n, size_t chunk) {
    const size_t nc = pc_num_chunks(n, chunk);
    if (!nc) return 0;
    const size_t last = n - (nc - 1) * chunk;
    return (nc - 1) * (chunk / PC_SUBSTREAM) + (last + PC_SUBSTREAM - 1) / PC_SUBSTREAM;
}

size_t pc_max_payload_words(size_t n, size_t chunk) {
    const size_t nc = pc_num_chunks(n, chunk);
    if (!nc) return 0;
    const size_t last = n - (nc - 1) * chunk;
    return (nc - 1) * ((PC_MAX_LEN * chunk + 31) / 32) + (PC_MAX_LEN * last + 31) / 32;
}

}  // extern "C"
