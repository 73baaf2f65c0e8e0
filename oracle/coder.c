/*
 * Oracle bitstream coder -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, bit-serial C.  No lookup-table decoding, no SIMD, no word
 * tricks: every codeword bit is written and read one at a time.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load this
 * code; the product library shares nothing with it (no headers, no tables).
 *
 * Method: "Single-Stage Huffman Encoder for ML Compression" (abstract) -- the
 * encoder maps every symbol through one fixed codebook known to both sides
 * and concatenates the codewords; nothing about the codebook travels with
 * the data.  "Quad Length Codes for Lossless Compression of e4m3" (abstract)
 * -- a QLC codeword is a 3-bit area number followed by a fixed-width index
 * into the probability-ranked symbols; decode_qlc() reads it that way.
 *
 * Container (the pages define none; this is the reading used throughout):
 *  - the input is cut into chunks of `chunk` symbols (last one may be short);
 *    each chunk is an independent bitstream;
 *  - stream bit j of a chunk is bit (31 - j%32) of 32-bit word j/32, i.e.
 *    codewords are concatenated most-significant-bit first;
 *  - a chunk is zero-padded to a whole word; chunk c's words start at word
 *    chunk_word_offset[c] of the payload, chunks are back to back,
 *    chunk_word_offset[num_chunks] is the total;
 *  - chunk_bits[c] is the exact unpadded bit count of chunk c;
 *  - sub_off[] holds, per chunk and for j = 0 .. ceil(len_c/256)-1, the bit
 *    offset (relative to the chunk's first bit) of symbol 256*j of the chunk.
 *
 * Corruption rules (decode returns ORACLE_CORRUPT when any holds):
 *  - chunk_word_offset[c+1] < chunk_word_offset[c], or
 *    chunk_word_offset[c+1] - chunk_word_offset[c] != ceil(chunk_bits[c]/32),
 *    or chunk_word_offset[num_chunks] > payload_words;
 *  - the first sub-stream of a chunk does not start at bit 0;
 *  - a sub-stream reads a bit at or past chunk_bits[c], meets a bit pattern
 *    that is no codeword, or after its symbols does not end exactly where the
 *    next sub-stream starts (chunk_bits[c] for the chunk's last one).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_INVALID_ARG 1
#define ORACLE_CAPACITY 3
#define ORACLE_CORRUPT 4

#define SUB 256
#define LMAX 12

static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

/* ------------------------------------------------------------------------ */
/* bit I/O, one bit at a time                                                */
/* ------------------------------------------------------------------------ */

static void put_bit(uint32_t *words, uint64_t pos, unsigned bit) {
    if (bit) words[pos >> 5] |= (uint32_t)1u << (31u - (unsigned)(pos & 31u));
}

static unsigned get_bit(const uint32_t *words, uint64_t pos) {
    return (words[pos >> 5] >> (31u - (unsigned)(pos & 31u))) & 1u;
}

/* ------------------------------------------------------------------------ */
/* encoder                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint8_t *in;
    uint64_t n, chunk, c0, c1;
    const uint8_t *len;
    const uint16_t *code;
    uint32_t *payload;
    const uint32_t *chunk_bits;
    const uint64_t *cwo;
    uint32_t *sub_off;
} enc_job;

static void encode_chunk(const enc_job *J, uint64_t c) {
    uint64_t begin = c * J->chunk;
    uint64_t end = begin + J->chunk < J->n ? begin + J->chunk : J->n;
    uint32_t *w = J->payload + J->cwo[c];
    uint64_t nwords = J->cwo[c + 1] - J->cwo[c];
    uint64_t subs_per_chunk = J->chunk / SUB;
    uint32_t *so = J->sub_off + c * subs_per_chunk;
    memset(w, 0, nwords * sizeof(uint32_t));
    uint64_t pos = 0;
    for (uint64_t i = begin; i < end; ++i) {
        uint64_t k = i - begin;
        if (k % SUB == 0) so[k / SUB] = (uint32_t)pos;
        unsigned s = J->in[i];
        unsigned l = J->len[s];
        for (int b = (int)l - 1; b >= 0; --b) put_bit(w, pos++, (J->code[s] >> b) & 1u);
    }
}

static void *enc_worker(void *arg) {
    enc_job *J = (enc_job *)arg;
    for (uint64_t c = J->c0; c < J->c1; ++c) encode_chunk(J, c);
    return NULL;
}

/* Returns ORACLE_OK, ORACLE_INVALID_ARG or ORACLE_CAPACITY. */
int oracle_encode(const uint8_t *in, uint64_t n, uint64_t chunk,
                  const uint8_t len[256], const uint16_t code[256],
                  uint32_t *payload, uint64_t capacity_words,
                  uint32_t *chunk_bits, uint64_t *chunk_word_offset, uint32_t *sub_off,
                  int threads) {
    if (chunk == 0 || chunk % SUB) return ORACLE_INVALID_ARG;
    for (int s = 0; s < 256; ++s)
        if (len[s] < 1 || len[s] > LMAX) return ORACLE_INVALID_ARG;
    uint64_t nc = ceil_div(n, chunk);
    /* chunk_bits[c] = sum of the code lengths of the chunk's symbols */
    chunk_word_offset[0] = 0;
    for (uint64_t c = 0; c < nc; ++c) {
        uint64_t begin = c * chunk, end = begin + chunk < n ? begin + chunk : n;
        uint64_t bits = 0;
        for (uint64_t i = begin; i < end; ++i) bits += len[in[i]];
        chunk_bits[c] = (uint32_t)bits;
        chunk_word_offset[c + 1] = chunk_word_offset[c] + ceil_div(bits, 32);
    }
    if (chunk_word_offset[nc] > capacity_words) return ORACLE_CAPACITY;
    enc_job base = {in, n, chunk, 0, 0, len, code, payload, chunk_bits, chunk_word_offset, sub_off};
    if (threads < 1) threads = 1;
    if ((uint64_t)threads > nc) threads = nc ? (int)nc : 1;
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    enc_job *jobs = (enc_job *)calloc((size_t)threads, sizeof(enc_job));
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].c0 = nc * (uint64_t)t / (uint64_t)threads;
        jobs[t].c1 = nc * (uint64_t)(t + 1) / (uint64_t)threads;
        pthread_create(&tid[t], NULL, enc_worker, &jobs[t]);
    }
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* decoders                                                                  */
/* ------------------------------------------------------------------------ */

/* Canonical-Huffman tables: how many codes of each length, and the symbols
 * in (length, byte value) order.  Decoding reads one bit at a time and
 * compares against the first code of the current length. */
typedef struct {
    int count[LMAX + 1];
    uint8_t sorted[256];
    int nsorted;
} canon_t;

static void canon_build(canon_t *T, const uint8_t len[256]) {
    memset(T, 0, sizeof(*T));
    for (int l = 1; l <= LMAX; ++l)
        for (int s = 0; s < 256; ++s)
            if (len[s] == l) {
                T->count[l]++;
                T->sorted[T->nsorted++] = (uint8_t)s;
            }
}

typedef struct {
    const uint32_t *w;  /* chunk's first word */
    uint64_t limit;     /* chunk_bits */
    uint64_t pos;
    int bad;
} reader_t;

static unsigned rd(reader_t *R) {
    if (R->pos >= R->limit) {
        R->bad = 1;
        return 0;
    }
    return get_bit(R->w, R->pos++);
}

static int decode_canon(const canon_t *T, reader_t *R) {
    int code = 0, first = 0, index = 0;
    for (int l = 1; l <= LMAX; ++l) {
        code |= (int)rd(R);
        if (R->bad) return -1;
        int cnt = T->count[l];
        if (code - first < cnt) return T->sorted[index + code - first];
        index += cnt;
        first = (first + cnt) << 1;
        code <<= 1;
    }
    return -1; /* no codeword of length <= 12 matches */
}

static int decode_qlc(const uint8_t bits[8], const uint8_t sym_of_rank[256], reader_t *R) {
    unsigned area = 0;
    for (int i = 0; i < 3; ++i) area = (area << 1) | rd(R);
    if (R->bad) return -1;
    unsigned start = 0;
    for (unsigned a = 0; a < area; ++a) start += 1u << bits[a];
    unsigned idx = 0;
    for (unsigned i = 0; i < bits[area]; ++i) idx = (idx << 1) | rd(R);
    if (R->bad) return -1;
    unsigned r = start + idx;
    if (r >= 256) return -1; /* unused slot */
    return sym_of_rank[r];
}

typedef struct {
    const uint32_t *payload;
    const uint32_t *chunk_bits;
    const uint64_t *cwo;
    const uint32_t *sub_off;
    uint64_t n, chunk, c0, c1;
    const canon_t *canon;
    int qlc;
    const uint8_t *qbits, *sym_of_rank;
    uint8_t *out;
    int bad;
} dec_job;

static int decode_chunk(const dec_job *J, uint64_t c) {
    uint64_t begin = c * J->chunk;
    uint64_t end = begin + J->chunk < J->n ? begin + J->chunk : J->n;
    uint64_t nsub = ceil_div(end - begin, SUB);
    const uint32_t *so = J->sub_off + c * (J->chunk / SUB);
    reader_t R;
    R.w = J->payload + J->cwo[c];
    R.limit = J->chunk_bits[c];
    R.bad = 0;
    if (so[0] != 0) return 1;
    for (uint64_t j = 0; j < nsub; ++j) {
        R.pos = so[j];
        uint64_t stop = (j + 1 < nsub) ? so[j + 1] : J->chunk_bits[c];
        uint64_t a = begin + j * SUB;
        uint64_t b = a + SUB < end ? a + SUB : end;
        for (uint64_t i = a; i < b; ++i) {
            int s = J->qlc ? decode_qlc(J->qbits, J->sym_of_rank, &R) : decode_canon(J->canon, &R);
            if (s < 0 || R.bad) return 1;
            J->out[i] = (uint8_t)s;
        }
        if (R.pos != stop) return 1;
    }
    return 0;
}

static void *dec_worker(void *arg) {
    dec_job *J = (dec_job *)arg;
    for (uint64_t c = J->c0; c < J->c1; ++c)
        if (decode_chunk(J, c)) {
            J->bad = 1;
            break;
        }
    return NULL;
}

/* qlc = 0: canonical Huffman decoding from len[]; qlc = 1: area decoding
 * from qlc_bits[] and sym_of_rank[].  Returns ORACLE_OK or ORACLE_CORRUPT
 * (ORACLE_INVALID_ARG for a bad chunk size). */
int oracle_decode(const uint32_t *payload, uint64_t payload_words,
                  const uint32_t *chunk_bits, const uint64_t *chunk_word_offset,
                  const uint32_t *sub_off, uint64_t n, uint64_t chunk,
                  const uint8_t len[256], int qlc, const uint8_t qlc_bits[8],
                  const uint8_t sym_of_rank[256], uint8_t *out, int threads) {
    if (chunk == 0 || chunk % SUB) return ORACLE_INVALID_ARG;
    uint64_t nc = ceil_div(n, chunk);
    for (uint64_t c = 0; c < nc; ++c) {
        if (chunk_word_offset[c + 1] < chunk_word_offset[c]) return ORACLE_CORRUPT;
        if (chunk_word_offset[c + 1] - chunk_word_offset[c] != ceil_div(chunk_bits[c], 32))
            return ORACLE_CORRUPT;
    }
    if (nc && chunk_word_offset[nc] > payload_words) return ORACLE_CORRUPT;
    canon_t T;
    canon_build(&T, len);
    dec_job base = {payload, chunk_bits, chunk_word_offset, sub_off, n, chunk, 0, 0,
                    &T, qlc, qlc_bits, sym_of_rank, out, 0};
    if (threads < 1) threads = 1;
    if ((uint64_t)threads > nc) threads = nc ? (int)nc : 1;
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    dec_job *jobs = (dec_job *)calloc((size_t)threads, sizeof(dec_job));
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].c0 = nc * (uint64_t)t / (uint64_t)threads;
        jobs[t].c1 = nc * (uint64_t)(t + 1) / (uint64_t)threads;
        pthread_create(&tid[t], NULL, dec_worker, &jobs[t]);
    }
    int bad = 0;
    for (int t = 0; t < threads; ++t) {
        pthread_join(tid[t], NULL);
        bad |= jobs[t].bad;
    }
    free(tid);
    free(jobs);
    return bad ? ORACLE_CORRUPT : ORACLE_OK;
}
