/*
 * pc.h -- fixed-codebook ("single-stage") prefix coding of 8-bit tensors on
 * AMD Instinct MI355X (gfx950).  C ABI of libpc.so.
 *
 * Method
 *   "Single-Stage Huffman Encoder for ML Compression" (abstract): a Huffman
 *   code is normally built per message (frequency analysis, codebook
 *   generation, codebook sent with the data).  The single-stage encoder
 *   instead uses one fixed codebook derived from the average distribution of
 *   previous batches, so the run-time work is only the symbol-to-codeword
 *   mapping and nothing but the codewords is transmitted.
 *   "Quad Length Codes for Lossless Compression of e4m3" (abstract, Tables 1
 *   and 2): the second codebook kind -- a 3-bit prefix names one of 8 areas,
 *   and area a carries a fixed-width b_a-bit index into the symbols ranked by
 *   descending probability (code length 3 + b_a).
 *
 * Alphabet 256 (one byte per symbol: e4m3 or int8).  Code lengths are 1..12
 * bits.  All integers are little-endian.
 *
 * Container (the pages define none; this is the library's format)
 *   - The input of n symbols is cut into chunks of `chunk` symbols (a
 *     multiple of 256, at most 2^24; the last chunk may be short).  Each chunk
 *     is an independent bitstream: its codewords concatenated, most
 *     significant bit first; stream bit j is bit (31 - j%32) of 32-bit word
 *     j/32; the chunk is zero-padded to a whole word.
 *   - payload: the chunks' words back to back; chunk c starts at word
 *     chunk_word_offset[c]; chunk_word_offset[num_chunks] is the total.
 *   - chunk_bits[c]: exact unpadded bit count of chunk c.
 *   - sub_off: for every chunk c and j = 0 .. ceil(len_c/256)-1, the bit
 *     offset (relative to chunk c's first bit) of the chunk's symbol 256*j.
 *     Flattened in chunk order; entry j = 0 is always 0.  This side index
 *     lets the decoder run one independent 256-symbol sub-stream per lane.
 *   Nothing of the codebook travels with the data: encoder and decoder must
 *   use the same pc_codebook (compare codebook_id).
 *
 * Errors
 *   Every entry point returns a pc_status synchronously for argument, size
 *   and launch errors.  Device entry points are asynchronous on `stream` (a
 *   hipStream_t; NULL is the default stream).  Data-dependent decode errors
 *   are reported through a device status word (see pc_decode).
 *
 * Memory
 *   The library never allocates.  Every buffer belongs to the caller; device
 *   pointers must stay valid until the stream has executed the call.
 */
#ifndef PC_H
#define PC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PC_ALPHABET 256
#define PC_MAX_LEN 12
#define PC_SUBSTREAM 256
#define PC_QLC_AREAS 8
#define PC_CODEBOOK_MAGIC 0x31424350u /* "PCB1" */
#define PC_CODEBOOK_VERSION 1u

typedef enum pc_status {
    PC_OK = 0,
    PC_ERR_INVALID_ARG = 1, /* a pointer, size, alignment or enum is invalid */
    PC_ERR_UNSUPPORTED = 2, /* valid request the library cannot serve */
    PC_ERR_CAPACITY = 3,    /* an output or workspace buffer is too small */
    PC_ERR_CORRUPT = 4,     /* data do not form a valid container (decode) */
    PC_ERR_HIP = 5,         /* the HIP runtime reported an error */
    PC_ERR_TIMEOUT = 6      /* a bounded device wait gave up (encode); outputs invalid */
} pc_status;

typedef enum pc_codebook_kind {
    PC_CODEBOOK_HUFFMAN = 0, /* canonical, package-merge length-limited to 12 bits */
    PC_CODEBOOK_QLC = 1      /* Quad Length Code: 3-bit area + fixed-width index */
} pc_codebook_kind;

/*
 * The codebook: a flat, position-independent blob (9536 bytes).  Build it on
 * the host with pc_codebook_build, copy it to device memory once, and pass
 * the device copy to pc_encode / pc_decode.  Layout is fixed (offsets in
 * bytes): header 0, length 32, code 288, dec_sym 800, dec_len 4896,
 * qlc_bits 8992, qlc_start 9000, rank_of 9016, sym_of_rank 9272.
 */
typedef struct pc_codebook {
    uint32_t magic;          /* PC_CODEBOOK_MAGIC */
    uint32_t version;        /* PC_CODEBOOK_VERSION */
    uint32_t kind;           /* pc_codebook_kind */
    uint32_t max_len;        /* longest code length in use (<= 12) */
    uint32_t codebook_id;    /* FNV-1a 32 over kind (4 bytes), length[256], qlc_bits[8] */
    uint32_t complete;       /* 1 when the Kraft sum is exactly 1 */
    uint32_t reserved[2];
    uint8_t length[256];     /* code length of every byte value, 1..12 */
    uint16_t code[256];      /* code value, right-aligned (MSB first on the wire) */
    uint8_t dec_sym[4096];   /* 12-bit peek (next 12 stream bits) -> symbol */
    uint8_t dec_len[4096];   /* 12-bit peek -> code length; 0 = no codeword */
    uint8_t qlc_bits[8];     /* QLC: index width of each area (zeros for Huffman) */
    uint16_t qlc_start[8];   /* QLC: first rank of each area */
    uint8_t rank_of[256];    /* QLC: rank (descending count) of each byte value */
    uint8_t sym_of_rank[256];/* QLC: byte value of each rank */
    uint8_t pad[8];
} pc_codebook;

/* Human-readable name of a status code (static storage; library-defined). */
const char *pc_status_string(int status);

/*
 * Build a fixed codebook on the host.  Pure, deterministic, thread-safe.
 *
 * counts: the pooled histogram of previous batches ("Single-Stage Huffman
 *   Encoder for ML Compression", abstract: the average distribution of
 *   previous data batches; pooling equal-size batches by summing counts is
 *   proportional to averaging their PMFs).
 * kind = PC_CODEBOOK_HUFFMAN: weights max(count,1) (every byte stays
 *   codable), package-merge length-limited to 12 bits (on equal weight a leaf
 *   precedes a package; leaves ordered by (weight, byte value)), then
 *   canonical codes in (length, byte value) order.  qlc_bits must be NULL.
 * kind = PC_CODEBOOK_QLC: qlc_bits[a] (0..9) is the index width of area a
 *   ("Quad Length Codes for Lossless Compression of e4m3", Tables 1 and 2);
 *   the areas must cover 256 ranks (sum 2^b >= 256).  Ranks order bytes by descending count, equal counts
 *   by lower byte value; the byte of rank r in area a gets code
 *   (a << b_a) | (r - start_a) of length 3 + b_a.
 * Returns PC_ERR_INVALID_ARG for NULL pointers, an unknown kind, or bad
 * QLC widths; `out` is fully written on PC_OK.
 */
pc_status pc_codebook_build(const uint64_t counts[256], int kind, const uint8_t qlc_bits[8],
                            pc_codebook *out);

/*
 * Host check of a codebook blob (magic, version, lengths, tables).  The
 * pages define no codebook format ("Single-Stage Huffman Encoder for ML
 * Compression", abstract, only requires that encoder and decoder hold the
 * same precomputed codebook); this checks the library's own layout above.
 */
pc_status pc_codebook_validate(const pc_codebook *cb);

/*
 * Choose QLC area widths for a histogram: the 8 widths (each 0..9, areas
 * covering 256 ranks) that minimise sum(count * (3 + b_area(rank))) over the
 * ranked histogram, by dynamic programming over contiguous rank ranges --
 * "Quad Length Codes for Lossless Compression of e4m3" (abstract) notes
 * that the scheme adapts to the distribution.  Ties keep the
 * lexicographically smallest width vector.  Host only.
 */
pc_status pc_qlc_optimal_bits(const uint64_t counts[256], uint8_t bits_out[8]);

/*
 * How well a fixed codebook fits a batch (host, pure).  For the byte
 * histogram `counts` of the batch:
 *   *avg_bits = sum(count * length) / sum(count): the payload bits per
 *               symbol the codebook spends on that batch;
 *   *entropy  = the batch's Shannon entropy, -sum(p log2 p), in bits per
 *               symbol: the bound a code built for the batch itself
 *               approaches.
 * The single-stage codebook is built once from earlier batches ("Single-
 * Stage Huffman Encoder for ML Compression", abstract), so avg_bits -
 * entropy measures how far the batches have drifted from it; the Shannonic
 * page ("Shannonic: Efficient Entropy-Optimal Compression for ML
 * Workloads", key observation 1) expects static tables to be refreshed when
 * the distribution drifts.  A caller rebuilds (pc_codebook_build on the
 * pooled counts of recent batches) once the gap passes its threshold.
 * An all-zero histogram gives 0 and 0.  PC_ERR_INVALID_ARG for NULL
 * pointers or a blob that fails pc_codebook_validate.
 */
pc_status pc_codebook_fit(const pc_codebook *cb, const uint64_t counts[256], double *avg_bits, double *entropy);

/*
 * Code lengths of the per-shard comparator (host, pure).  "Single-Stage
 * Huffman Encoder for ML Compression" (abstract) measures the fixed codebook
 * against Huffman codes built for each shard from its own statistics (the
 * three-stage scheme: count, build, send the codebook).  This returns that
 * code for one shard's histogram: package-merge limited to 12 bits over the
 * byte values that occur (count > 0), with the same tie rules as
 * pc_codebook_build; an absent byte value gets length 0 (no codeword), a
 * histogram with one byte value gives it length 1, an all-zero histogram
 * gives all zeros.  Unlike pc_codebook_build, counts are not floored: a
 * shard's own code never has to code a byte it does not contain.
 *   lengths_out[256]   written in full on PC_OK.
 * PC_ERR_INVALID_ARG for NULL pointers.
 */
pc_status pc_shard_code_lengths(const uint64_t counts[256], uint8_t lengths_out[256]);

/*
 * Size queries (host, pure) of the container above, which is the library's
 * own (the pages define no container).  chunk must be a valid chunk size,
 * else 0.  The payload bound uses the 12-bit length limit (PC_MAX_LEN).
 */
size_t pc_num_chunks(size_t n, size_t chunk);          /* ceil(n / chunk) */
size_t pc_num_substreams(size_t n, size_t chunk);      /* sum over chunks of ceil(len_c / 256) */
size_t pc_max_payload_words(size_t n, size_t chunk);   /* sum over chunks of ceil(12 len_c / 32) */
size_t pc_encode_workspace_bytes(size_t n, size_t chunk);  /* 8 (1 + chunks), + 4 per 64 KiB of full
                                                          chunks for chunks of several 64 KiB (rounded up to 8) */

/*
 * Encode n symbols (device, asynchronous on `stream`): every byte becomes
 * its codeword from the fixed codebook and the codewords are concatenated
 * ("Single-Stage Huffman Encoder for ML Compression", abstract: symbol to
 * codeword mapping with one precomputed codebook; "Quad Length Codes for
 * Lossless Compression of e4m3", abstract, for the QLC codewords), chunk by
 * chunk into the container described above.
 *   d_cb       device copy of a pc_codebook.
 *   d_in       n input bytes, 16-byte aligned.
 *   chunk      symbols per chunk: multiple of 256, 256 <= chunk <= 2^24.
 *   d_payload  >= pc_max_payload_words(n, chunk) words (capacity is checked
 *              against that bound, so encoding can never overflow), 16-byte
 *              aligned.  Exactly chunk_word_offset[num_chunks] words are
 *              written.
 *   d_chunk_bits          [num_chunks] u32
 *   d_chunk_word_offset   [num_chunks + 1] u64 (exclusive prefix of words)
 *   d_sub_off             [pc_num_substreams(n, chunk)] u32
 *   d_ws, ws_bytes        scratch of at least pc_encode_workspace_bytes,
 *              8-byte aligned; its contents need no initialisation.
 *   d_status   one u32 in device memory (4-byte aligned).  The call first
 *              sets it to 0 on the stream, then to PC_ERR_TIMEOUT if the
 *              cross-chunk scan gave up waiting for an earlier workgroup's
 *              word count (see pc_encode_set_wait_limit); the outputs are
 *              then invalid.  Read it after the stream has executed the call.
 * n = 0 writes chunk_word_offset[0] = 0, *d_status = 0 and nothing else.
 * Calls that share a workspace must be ordered on one stream.  More than
 * 2^31 - 1 chunks: PC_ERR_UNSUPPORTED.
 */
pc_status pc_encode(const pc_codebook *d_cb, const uint8_t *d_in, size_t n, size_t chunk,
                    uint32_t *d_payload, size_t payload_capacity_words,
                    uint32_t *d_chunk_bits, uint64_t *d_chunk_word_offset, uint32_t *d_sub_off,
                    void *d_ws, size_t ws_bytes, uint32_t *d_status, void *stream);

/*
 * pc_encode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs, status word and errors as pc_encode, without the
 * workspace: the cross-chunk scan's ticket and descriptors live in a static
 * device array of the library (8 MiB + 8 bytes per GPU, held until the
 * process ends), so the call allocates nothing.  At most 2^20 chunks per
 * call, and pc_encode_workspace_bytes(n, chunk) at most that array's size
 * (PC_ERR_CAPACITY beyond; it binds for chunks of several 64 KiB, which
 * keep one u32 per 64 KiB in the array).  Every call on one GPU shares that GPU's
 * array and clears it first on its stream: calls that overlap on one GPU
 * (several streams, or host threads) race and must be serialised by the
 * caller, e.g. by issuing them on one stream.
 */
pc_status pc_encode_noalloc(const pc_codebook *d_cb, const uint8_t *d_in, size_t n, size_t chunk,
                            uint32_t *d_payload, size_t payload_capacity_words,
                            uint32_t *d_chunk_bits, uint64_t *d_chunk_word_offset, uint32_t *d_sub_off,
                            uint32_t *d_status, void *stream);

/*
 * Bound of the encoder's one device-side wait (host, process-wide; returns
 * the previous bound).  The pages describe no GPU encoder; this library's
 * chunks learn their output offsets from a single-pass scan in which a
 * workgroup waits until the workgroups of all earlier chunks have published
 * their word counts.  Every wave of that wait polls at most `polls` times,
 * then gives up and reports PC_ERR_TIMEOUT through pc_encode's d_status
 * instead of waiting on.  The default (polls = 0 restores it) is 2^20 polls,
 * about a second: far beyond a correct run's wait, short enough that a
 * workgroup held up by other work on a time-sliced GPU ends in an error
 * rather than a hang.  Small limits make give-ups frequent (the tests use 1
 * to exercise the report); each call reads the bound when it is made.
 */
uint32_t pc_encode_set_wait_limit(uint32_t polls);

/*
 * Decode n symbols (device, asynchronous on `stream`) with the generic
 * engine: one lane per 256-symbol sub-stream, one 12-bit peek per codeword
 * through the dec_sym/dec_len tables held in LDS.  Works for both codebook
 * kinds.  The decoder holds the same fixed codebook as the encoder, so no
 * table travels with the data ("Single-Stage Huffman Encoder for ML
 * Compression", abstract); one table lookup per codeword instead of a
 * bit-by-bit tree walk is the decoding-speed concern of "Quad Length Codes
 * for Lossless Compression of e4m3" (abstract).
 *   d_payload, payload_words   the payload (16-byte aligned) and its length;
 *              no word at or past payload_words is ever read.
 *   d_chunk_bits, d_chunk_word_offset, d_sub_off   as written by pc_encode.
 *   d_out      n output bytes, 16-byte aligned; nothing outside [0, n) is
 *              written.
 *   d_status   one u32 in device memory.  The caller zeroes it before the
 *              call; the decoder sets it to PC_ERR_CORRUPT when the
 *              container is inconsistent (chunk_word_offset steps that differ
 *              from ceil(chunk_bits/32) or run past payload_words, a chunk
 *              whose first sub-stream does not start at bit 0, a bit pattern
 *              that is no codeword, or a sub-stream that does not end exactly
 *              where the next one starts / at chunk_bits).  On such an error
 *              d_out holds unspecified bytes.
 * 2^32 - 256 or more sub-streams (n of about 2^40 and up, past one GPU's
 * memory): PC_ERR_UNSUPPORTED.
 */
pc_status pc_decode(const pc_codebook *d_cb, const uint32_t *d_payload, size_t payload_words,
                    const uint32_t *d_chunk_bits, const uint64_t *d_chunk_word_offset,
                    const uint32_t *d_sub_off, size_t n, size_t chunk, uint8_t *d_out,
                    uint32_t *d_status, void *stream);

/*
 * Decode a QLC-coded stream the way "Quad Length Codes for Lossless
 * Compression of e4m3" (abstract) describes its decoder: read the 3-bit
 * area number, read that area's fixed-width index, map the rank to the
 * symbol through the 256-entry table.  Same arguments, container
 * and error rules as pc_decode; d_cb must be a PC_CODEBOOK_QLC codebook
 * (PC_ERR_CORRUPT in *d_status otherwise).
 */
pc_status pc_decode_qlc(const pc_codebook *d_cb, const uint32_t *d_payload, size_t payload_words,
                        const uint32_t *d_chunk_bits, const uint64_t *d_chunk_word_offset,
                        const uint32_t *d_sub_off, size_t n, size_t chunk, uint8_t *d_out,
                        uint32_t *d_status, void *stream);

/*
 * Byte histogram on the device: d_counts[s] += number of bytes equal to s in
 * d_in[0, n).  Accumulates, so pooling previous batches is repeated calls on
 * the same d_counts (256 u64, 8-byte aligned).  d_in needs no alignment.
 * The pooled histogram of previous batches is what the fixed codebook is
 * built from ("Single-Stage Huffman Encoder for ML Compression", abstract:
 * the average distribution of previous data batches).
 */
pc_status pc_histogram(const uint8_t *d_in, size_t n, uint64_t *d_counts, void *stream);

/*
 * Measurement helper, not part of the coding method: copies `bytes` bytes
 * from d_src to d_dst with the 16-byte non-temporal loads and stores the
 * coder kernels use, so that the HBM bytes hardware counters report for this
 * known transfer (read `bytes`, write `bytes`) can calibrate the counts
 * taken on the coder kernels.  Both pointers 16-byte aligned device memory,
 * bytes a multiple of 16 (PC_ERR_INVALID_ARG otherwise); asynchronous on
 * `stream`; bytes == 0 does nothing.
 */
pc_status pc_traffic_probe(const void *d_src, void *d_dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PC_H */
