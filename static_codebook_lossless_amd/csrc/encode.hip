// Fixed-codebook encoder for gfx950 ("Single-Stage Huffman Encoder for ML
// Compression", abstract: every symbol goes through one fixed codebook; the
// codewords are concatenated and nothing else is sent).
//
// One workgroup (256 lanes, 4 waves) encodes one chunk.  Per 4096-symbol
// tile every lane owns 16 consecutive symbols (one 16-byte load, so a wave
// reads 1 KiB contiguous):
//   1. code/length lookup in LDS (the 256-entry codebook is copied to LDS);
//   2. per-lane bit count, wave64 DPP inclusive scan, LDS combine across the
//      4 waves -> every lane's bit offset inside the chunk, the tile totals
//      and the chunk's total bit count;
//   3. the chunk's word offset in the output comes from a single-pass device
//      exclusive scan over chunks (decoupled look-back on per-chunk
//      descriptors), so the chunk is written straight to its final place:
//      the scan and the compaction of chunk payloads are fused here;
//   4. each lane packs its codewords (4 symbols -> one <=48-bit group) and
//      ORs them into LDS-staged 32-bit words MSB first; complete words of
//      the tile are stored coalesced; the partial last word carries over.
// The side index (bit offset of every 256th symbol) falls out of step 2.
#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kSymPerLane = 16;
constexpr uint32_t kTile = kThreads * kSymPerLane;                // 4096

// Look-back descriptor per chunk: state in bits 62..63, word count below.
constexpr uint64_t kDescAggregate = 1ull << 62;
constexpr uint64_t kDescInclusive = 2ull << 62;
constexpr uint64_t kDescValue = (1ull << 62) - 1;

__device__ __forceinline__ uint64_t ld_desc(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_desc(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix (in words) of descriptor c over all earlier ones (a
// descriptor covers the chunks of one workgroup, in chunk order).  Called by
// one whole wave.  The workgroup got ticket c from an atomic counter, so
// every earlier descriptor's workgroup is already running and will publish.
// Each round reads 128 predecessors (2 per lane, nearest first) in one trip
// to memory and polls, without pausing, until all have published; it then
// sums counts up to the nearest inclusive prefix, or walks 128 chunks
// further back.  (Descriptors written on other dies are read through the
// fabric: more loads per poll made each trip slower, measured.)
// The wait on predecessors is bounded: it ends once they publish, but a
// predecessor that stays silent longer than max_polls polls (by default
// ~2^20, about a second: a workgroup preempted for that long, or a bug) makes
// the wave give up instead of spinning forever.  It then reports
// PC_ERR_TIMEOUT through *status and publishes an inclusive prefix that
// assumes nothing before it (the caller discards the output), so that its
// successors' walks end there instead of each waiting out its own limit.
constexpr int kLookWin = 2;  // descriptors per lane per round

// Publish descriptor c's own count: inclusive for c == 0, else aggregate.
__device__ __forceinline__ void publish_count(uint64_t *desc, uint32_t c, uint64_t words) {
    st_desc(&desc[c], (c == 0 ? kDescInclusive : kDescAggregate) | words);
}

// `published`: the caller already ran publish_count for c.
__device__ uint64_t lookback(uint64_t *desc, uint32_t c, uint64_t words, uint32_t lane, uint32_t max_polls,
                             uint32_t *status, bool published = false) {
    if (c == 0) {
        if (lane == 0 && !published) st_desc(&desc[0], kDescInclusive | words);
        return 0;
    }
    if (lane == 0 && !published) st_desc(&desc[c], kDescAggregate | words);
    uint64_t excl = 0;
    int64_t idx = (int64_t)c - 1;
    while (true) {
        // window w, lane l looks at chunk idx - (64 w + l)
        uint64_t d[kLookWin];
        bool wait[kLookWin];
#pragma unroll
        for (int w = 0; w < kLookWin; ++w) {
            d[w] = kDescInclusive;  // before chunk 0: an inclusive zero
            wait[w] = idx - (int64_t)(64 * w + lane) >= 0;
        }
        for (uint32_t polls = 0;; ++polls) {
            bool any = false;
#pragma unroll
            for (int w = 0; w < kLookWin; ++w) {
                if (wait[w]) {
                    d[w] = ld_desc(&desc[idx - (int64_t)(64 * w + lane)]);
                    wait[w] = (d[w] >> 62) == 0;
                }
                any |= wait[w];
            }
            if (!__any(any)) break;
            if (polls + 1 >= max_polls) {
                if (lane == 0) {
                    atomicCAS(status, 0u, (uint32_t)PC_ERR_TIMEOUT);
                    st_desc(&desc[c], kDescInclusive | words);
                }
                return 0;
            }
        }
        bool found = false;
#pragma unroll
        for (int w = 0; w < kLookWin; ++w) {
            if (!found) {
                const uint64_t inc = __ballot((d[w] >> 62) == 2);
                const uint32_t stop = inc ? (uint32_t)__ffsll((unsigned long long)inc) - 1 : 63;
                excl += wave_sum_u64(lane <= stop ? (d[w] & kDescValue) : 0);
                found = inc != 0;
            }
        }
        if (found) break;
        idx -= 64 * kLookWin;
    }
    if (lane == 0) st_desc(&desc[c], kDescInclusive | (excl + words));
    return excl;
}

template <uint32_t THREADS>
struct Shared {
    static constexpr uint32_t kTileSyms = THREADS * kSymPerLane;
    static constexpr uint32_t kStage = kTileSyms * PC_MAX_LEN / 32 + 8;
    uint16_t code[256];
    uint8_t len[256];
    uint32_t wave_tot[16][THREADS / 64];  // per tile, per wave: bits (then: bits before the wave)
    uint32_t tile_beg[17];                // per tile: first bit inside the chunk; [NT] = total
    uint32_t misc[4];
    uint32_t stage[kStage];
};

// Bits of the (at most 16) symbols of one lane; symbols at k >= valid count 0.
template <class SH>
__device__ __forceinline__ uint32_t lane_bits(const uint4 &x, uint32_t valid, const SH &sh) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t t = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        uint32_t l0 = sh.len[v & 0xFF], l1 = sh.len[(v >> 8) & 0xFF];
        uint32_t l2 = sh.len[(v >> 16) & 0xFF], l3 = sh.len[v >> 24];
        if (valid < 16) {
            l0 = 4 * q + 0 < (int)valid ? l0 : 0;
            l1 = 4 * q + 1 < (int)valid ? l1 : 0;
            l2 = 4 * q + 2 < (int)valid ? l2 : 0;
            l3 = 4 * q + 3 < (int)valid ? l3 : 0;
        }
        t += l0 + l1 + l2 + l3;
    }
    return t;
}

// OR the codewords of one lane's symbols into the staging words, starting at
// bit p (bit 0 = MSB of stage[0]).
template <class SH>
__device__ __forceinline__ void pack_lane(const uint4 &x, uint32_t valid, uint32_t p, SH &sh) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        const uint32_t s0 = v & 0xFF, s1 = (v >> 8) & 0xFF, s2 = (v >> 16) & 0xFF, s3 = v >> 24;
        uint32_t c0 = sh.code[s0], c1 = sh.code[s1], c2 = sh.code[s2], c3 = sh.code[s3];
        uint32_t l0 = sh.len[s0], l1 = sh.len[s1], l2 = sh.len[s2], l3 = sh.len[s3];
        if (valid < 16) {
            if (4 * q + 0 >= (int)valid) { c0 = 0; l0 = 0; }
            if (4 * q + 1 >= (int)valid) { c1 = 0; l1 = 0; }
            if (4 * q + 2 >= (int)valid) { c2 = 0; l2 = 0; }
            if (4 * q + 3 >= (int)valid) { c3 = 0; l3 = 0; }
        }
        // two pairs of <= 24 bits, then one group of <= 48 bits
        const uint32_t p01 = (c0 << l1) | c1, n01 = l0 + l1;
        const uint32_t p23 = (c2 << l3) | c3, n23 = l2 + l3;
        const uint64_t g = ((uint64_t)p01 << n23) | p23;
        const uint32_t ng = n01 + n23;
        // left-align the group in 64 bits, then spread it over 3 words at
        // bit offset o inside word wi; a lane with no bits (past the end)
        // ORs zeros, in bounds, so every OR is issued by every lane (see
        // place_group)
        const uint64_t a = ng ? g << (64 - ng) : 0ull;
        const uint32_t hi = (uint32_t)(a >> 32), lo = (uint32_t)a;
        const uint32_t o = p & 31, wi = p >> 5;
        atomicOr(&sh.stage[wi], hi >> o);
        atomicOr(&sh.stage[wi + 1], __builtin_amdgcn_alignbit(hi, lo, o));
        atomicOr(&sh.stage[wi + 2], __builtin_amdgcn_alignbit(lo, 0u, o));
        p += ng;
    }
}

__device__ __forceinline__ uint4 load_lane(const uint8_t *in, uint64_t base, uint32_t off, uint32_t lenc) {
    if (off + 16 <= lenc) return *reinterpret_cast<const uint4 *>(in + base + off);
    uint32_t b[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) b[k] = (off + k < lenc) ? in[base + off + k] : 0u;
    uint4 x;
    x.x = b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24;
    x.y = b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24;
    x.z = b[8] | b[9] << 8 | b[10] << 16 | b[11] << 24;
    x.w = b[12] | b[13] << 8 | b[14] << 16 | b[15] << 24;
    return x;
}

__device__ __forceinline__ uint32_t lane_valid(uint32_t off, uint32_t lenc) {
    return off >= lenc ? 0u : (lenc - off >= 16 ? 16u : lenc - off);
}

// Store the finished words of a tile and reset the staging buffer.
// Stage word 0 is chunk word `first_word`; bits [tile_begin, tile_end) of the
// chunk are in the buffer.
template <uint32_t THREADS, class SH>
__device__ __forceinline__ void flush_tile(SH &sh, uint32_t *dst, uint32_t tile_begin, uint32_t tile_end,
                                           bool last, uint32_t tid) {
    const uint32_t first_word = tile_begin >> 5;
    const uint32_t nfull = (tile_end >> 5) - first_word;
    const uint32_t nstore = last ? ((tile_end + 31) >> 5) - first_word : nfull;
    for (uint32_t i = tid; i < nstore; i += THREADS) dst[first_word + i] = sh.stage[i];
    const uint32_t carry = sh.stage[nfull];
    __syncthreads();
    for (uint32_t i = tid; i <= nfull; i += THREADS) sh.stage[i] = (i == 0 && !last) ? carry : 0u;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Whole-chunk kernel: a workgroup encodes NT tiles of THREADS x 16 symbols,
// NT / TPC consecutive chunks of exactly TPC tiles each.
//
// Every symbol is looked up once: the table entry is code << 16 | length.
// Per tile, each lane turns its 16 symbols into 4 groups (<= 48 bits each),
// the tile's bit offsets come from a wave scan plus a scan of the wave
// totals, and the groups are ORed straight into an LDS buffer that holds the
// workgroup's whole output, each chunk starting on a new word.  After the
// last tile the size is known; one cross-workgroup scan (look-back) gives
// the word offset of the first chunk and the buffer is stored in one
// coalesced pass.  Output that would not fit the buffer (more than BUFW
// words: only data that does not compress) is redone tile by tile with a
// store per tile.
// ---------------------------------------------------------------------------

template <uint32_t THREADS, int NT, uint32_t BUFW>
struct ChunkShared {
    uint32_t tab[256];                    // code << 16 | length
    uint32_t wave_tot[NT][THREADS / 64];  // per tile, per wave: bits
    uint32_t misc[4];
    uint32_t guard[4];                    // right before buf; its last two take zeros only (place_group_end)
    uint32_t buf[BUFW + 8];
};

// Four table entries -> one group of ng (<= 48) bits, right-aligned in g.
// An entry is code << 16 | length: the length sits in the bits a shift
// instruction reads as its count, and the code in the upper half, which the
// instructions can take as an operand directly, so no field is extracted on
// its own.
__device__ __forceinline__ void make_group(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3, uint64_t &g,
                                           uint32_t &ng) {
    const uint32_t p01 = ((e0 >> 16) << (e1 & 31)) | (e1 >> 16);
    const uint32_t p23 = ((e2 >> 16) << (e3 & 31)) | (e3 >> 16);
    const uint32_t n23 = (e2 & 0xFF) + (e3 & 0xFF);
    g = ((uint64_t)p01 << n23) | p23;
    ng = (e0 & 0xFF) + (e1 & 0xFF) + n23;
}

// OR one group (ng bits of g) into the buffer at bit p (bit 0 = MSB of
// buf[0]); it spans at most 3 words.  All three ORs are issued for every
// lane (an OR with zero changes nothing), which keeps the placement free of
// branches.
__device__ __forceinline__ void place_group(uint64_t g, uint32_t ng, uint32_t p, uint32_t *buf) {
    const uint64_t a = g << (64 - ng);
    const uint32_t hi = (uint32_t)(a >> 32), lo = (uint32_t)a;
    const uint32_t o = p & 31, wi = p >> 5;
    atomicOr(&buf[wi], hi >> o);
    atomicOr(&buf[wi + 1], __builtin_amdgcn_alignbit(hi, lo, o));
    atomicOr(&buf[wi + 2], __builtin_amdgcn_alignbit(lo, 0u, o));
}

// The same three ORs for a group given by its end e (the bit after its
// last, bit 0 = MSB of the buffer's first word): the right-aligned group
// (hi:lo) shifted left by 32 - e % 32 spans buffer words e / 32 - 2 ..
// e / 32, which are hi >> e, alignbit(hi, lo, e) and alignbit(lo, 0, e)
// (the shifts read e % 32; for e % 32 == 0 the last is zero).  base is the
// word two before the buffer's first (the guard words before it take the
// zeros of groups that end in its first two words).
__device__ __forceinline__ void place_group_end(uint32_t hi, uint32_t lo, uint32_t e, uint32_t *base) {
    uint32_t *w = base + (e >> 5);
    atomicOr(w, hi >> (e & 31));
    atomicOr(w + 1, __builtin_amdgcn_alignbit(hi, lo, e));
    atomicOr(w + 2, __builtin_amdgcn_alignbit(lo, 0u, e));
}

// make_group without masking the lengths out of the entries: ng comes back
// with the group's length in its low 16 bits and the sum of the four codes
// above them (entries hold zeros in bits 8-15, so no carry reaches bit 16),
// n23 likewise, and the 64-bit shift reads only the low 6 bits of its
// count.  Callers mask the sum of a tile's four ng, and keep_groups takes
// byte 0 of each.
__device__ __forceinline__ void make_group_raw(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3, uint64_t &g,
                                               uint32_t &ng) {
    const uint32_t p01 = ((e0 >> 16) << (e1 & 31)) | (e1 >> 16);
    const uint32_t p23 = ((e2 >> 16) << (e3 & 31)) | (e3 >> 16);
    const uint32_t n23 = e2 + e3;
    g = ((uint64_t)p01 << (n23 & 63)) | p23;
    ng = e0 + e1 + n23;
}

template <class SH>
__device__ __forceinline__ void lane_groups_raw(const uint4 &x, const SH &sh, uint64_t g[4], uint32_t ng[4]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        make_group_raw(sh.tab[v & 0xFF], sh.tab[(v >> 8) & 0xFF], sh.tab[(v >> 16) & 0xFF], sh.tab[v >> 24], g[q],
                       ng[q]);
    }
}

template <class SH>
__device__ __forceinline__ void lane_groups(const uint4 &x, const SH &sh, uint64_t g[4], uint32_t ng[4]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        make_group(sh.tab[v & 0xFF], sh.tab[(v >> 8) & 0xFF], sh.tab[(v >> 16) & 0xFF], sh.tab[v >> 24], g[q],
                   ng[q]);
    }
}

// Bits of tile r before this lane, and the tile's total (both from the
// per-wave totals the tile just published).
template <uint32_t NW>
__device__ __forceinline__ void tile_offsets(const uint32_t *wave_tot, uint32_t lane, uint32_t wave,
                                             uint32_t &before, uint32_t &total) {
    const uint32_t v = lane < NW ? wave_tot[lane] : 0u;
    const uint32_t vs = wave_incl_scan(v);
    before = wave ? (uint32_t)__builtin_amdgcn_readlane((int)vs, (int)wave - 1) : 0u;
    total = (uint32_t)__builtin_amdgcn_readlane((int)vs, (int)NW - 1);
}

template <uint32_t THREADS, int NT, uint32_t BUFW, int TPC>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(THREADS == 1024 ? 8 : 1))) void encode_chunk_kernel(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint64_t n, uint32_t chunk,
    uint32_t num_chunks, uint32_t *__restrict__ payload, uint32_t *__restrict__ chunk_bits,
    uint64_t *__restrict__ cwo, uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws,
    uint32_t *__restrict__ status, uint32_t max_polls) {
    using SH = ChunkShared<THREADS, NT, BUFW>;
    static_assert(offsetof(SH, buf) == offsetof(SH, guard) + 16 && offsetof(SH, buf) % 16 == 0,
                  "the guard words sit right before the buffer, which is cleared in 16-byte stores");
    constexpr uint32_t TILE = THREADS * kSymPerLane;
    constexpr uint32_t NW = THREADS / 64;
    constexpr int NC = NT / TPC;  // chunks per workgroup
    static_assert(NT % TPC == 0, "whole chunks per workgroup");
    __shared__ SH sh;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sh.misc[0] = atomicAdd(reinterpret_cast<uint32_t *>(ws), 1u);
    if (tid < 256) {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.tab[tid] = ((uint32_t)reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid] << 16) | cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < (BUFW + 8) / 4; i += THREADS) reinterpret_cast<uint4 *>(sh.buf)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    const uint32_t s = uniform(sh.misc[0]);  // the workgroup's look-back index
    const uint32_t c0 = s * NC;               // its first chunk
    const uint8_t *src = in + (uint64_t)c0 * chunk + tid * 16;
    uint32_t *so = sub_off + (uint64_t)c0 * (chunk / kSub);

    // ---- one pass: lookups, offsets, packing into the chunk buffer -------
    // (the next tile's 16 bytes are in flight while a tile is processed).
    // Chunk k of the workgroup starts at word cw[k] of the buffer; tbase
    // counts bits from the current chunk's start.  The last kHold tiles are
    // placed only after the workgroup's word count has been published
    // (their groups wait in registers, two groups of <= 48 bits in three
    // words), so successors' look-backs see the count earlier.
    constexpr int kHold = NC == 1 ? 1 : 0;  // (more held tiles, or several chunks, spill registers)
    uint32_t tbase = 0, cword = 0;
    uint32_t cw[NC], cbits[NC];
    uint32_t HG[kHold + 1][6], HN[kHold + 1], HP[kHold + 1];  // held tiles: groups, lengths, first bit
    bool fits = true;
    uint4 xn = load_stream16(src);
#pragma unroll
    for (int r = 0; r < NT; ++r) {
        if (r % TPC == 0) {
            if (r) {
                cbits[r / TPC - 1] = tbase;
                cword = uniform(cword + ((tbase + 31) >> 5));
                tbase = 0;
            }
            cw[r / TPC] = cword;
        }
        const uint4 xc = xn;
        if (r + 1 < NT) xn = load_stream16(src + (r + 1) * TILE);
        uint64_t g[4];
        uint32_t ng[4];
        lane_groups_raw(xc, sh, g, ng);
        const uint32_t bits = (ng[0] + ng[1] + ng[2] + ng[3]) & 0xFFFF;
        const uint32_t incl = wave_incl_scan(bits);
        if (lane == 63) sh.wave_tot[r][wave] = incl;
        __syncthreads();
        uint32_t before, ttot;
        tile_offsets<NW>(sh.wave_tot[r], lane, wave, before, ttot);
        const uint32_t my = tbase + before + incl - bits;
        if ((tid & 15) == 0) so[(r * TILE + tid * kSymPerLane) / kSub] = my;
        if (cword * 32 + tbase + ttot + 64 > BUFW * 32) {
            fits = false;
            break;
        }
        uint32_t p = cword * 32 + my;
        if (r < NT - kHold) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                p += ng[q] & 0xFF;
                place_group_end((uint32_t)(g[q] >> 32), (uint32_t)g[q], p, sh.guard + 2);
            }
        } else {
            const int hr = r - (NT - kHold);  // unrolled: a constant
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                HG[hr][3 * h] = (uint32_t)g[2 * h];
                HG[hr][3 * h + 1] = (uint32_t)g[2 * h + 1];
                HG[hr][3 * h + 2] = (uint32_t)(g[2 * h] >> 32) | (uint32_t)(g[2 * h + 1] >> 32) << 16;
            }
            // formed here, not kept as table entries
            asm volatile("" : "+v"(HG[hr][0]), "+v"(HG[hr][1]), "+v"(HG[hr][2]), "+v"(HG[hr][3]), "+v"(HG[hr][4]),
                         "+v"(HG[hr][5]));
            HN[hr] = __builtin_amdgcn_perm(ng[1], ng[0], 0x0C0C0400u) | __builtin_amdgcn_perm(ng[3], ng[2], 0x04000C0Cu);
            HP[hr] = p;
        }
        tbase = uniform(tbase + ttot);
    }

    if (fits) {
        cbits[NC - 1] = tbase;
        const uint64_t words = cword + ((tbase + 31) >> 5);
        if (kHold && tid == 0) publish_count(ws + 1, s, words);
#pragma unroll
        for (int hr = 0; hr < kHold; ++hr) {
            uint32_t p = HP[hr];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t h = q >> 1;
                const uint32_t hi = (q & 1) ? HG[hr][3 * h + 2] >> 16 : HG[hr][3 * h + 2] & 0xFFFF;
                p += (HN[hr] >> (8 * q)) & 0xFF;
                place_group_end(hi, HG[hr][3 * h + (q & 1)], p, sh.guard + 2);
            }
        }
        __syncthreads();
        if (wave == 0) {
            const uint64_t excl = lookback(ws + 1, s, words, lane, max_polls, status, kHold > 0);
            if (lane == 0) {
                sh.misc[1] = (uint32_t)excl;
                sh.misc[2] = (uint32_t)(excl >> 32);
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    chunk_bits[c0 + k] = cbits[k];
                    cwo[c0 + k] = excl + cw[k];
                }
                if (c0 + NC == num_chunks) cwo[num_chunks] = excl + words;
            }
        }
        __syncthreads();
        const uint64_t excl = ((uint64_t)sh.misc[2] << 32) | sh.misc[1];
        uint32_t *dst = payload + excl;
        // streaming stores (the payload is not read again here); after a
        // head up to a 128-byte boundary every wave writes whole lines
        const uint32_t head = (uint32_t)((32 - (excl & 31)) & 31) < words ? (uint32_t)((32 - (excl & 31)) & 31)
                                                                          : (uint32_t)words;
        if (tid < head) __builtin_nontemporal_store(sh.buf[tid], dst + tid);
        for (uint32_t i = head + tid; i < words; i += THREADS) __builtin_nontemporal_store(sh.buf[i], dst + i);
        return;
    }

    // ---- the chunks do not fit: offsets of all tiles, then tile by tile --
    // tb[r]: bit of the workgroup's output where tile r starts (each chunk
    // starts on a word)
    uint32_t tb[NT + 1], e[NT];
    tb[0] = 0;
#pragma unroll
    for (int r = 0; r < NT; ++r) {
        uint64_t g[4];
        uint32_t ng[4];
        lane_groups(*reinterpret_cast<const uint4 *>(src + r * TILE), sh, g, ng);
        const uint32_t bits = ng[0] + ng[1] + ng[2] + ng[3];
        const uint32_t incl = wave_incl_scan(bits);
        __syncthreads();  // earlier readers of wave_tot[r] are done
        if (lane == 63) sh.wave_tot[r][wave] = incl;
        __syncthreads();
        uint32_t before, ttot;
        tile_offsets<NW>(sh.wave_tot[r], lane, wave, before, ttot);
        e[r] = before + incl - bits;
        const uint32_t cstart = tb[r - r % TPC];  // the chunk's first bit (a word boundary)
        if ((tid & 15) == 0) so[(r * TILE + tid * kSymPerLane) / kSub] = tb[r] - cstart + e[r];
        const uint32_t end = uniform(tb[r] + ttot);
        if (r % TPC == TPC - 1) {
            cbits[r / TPC] = end - cstart;
            cw[r / TPC] = cstart >> 5;
            tb[r + 1] = (end + 31) & ~31u;
        } else {
            tb[r + 1] = end;
        }
    }
    const uint64_t words = tb[NT] >> 5;
    for (uint32_t i = tid; i < (BUFW + 8) / 4; i += THREADS) reinterpret_cast<uint4 *>(sh.buf)[i] = make_uint4(0, 0, 0, 0);
    if (wave == 0) {
        const uint64_t excl = lookback(ws + 1, s, words, lane, max_polls, status);
        if (lane == 0) {
            sh.misc[1] = (uint32_t)excl;
            sh.misc[2] = (uint32_t)(excl >> 32);
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                chunk_bits[c0 + k] = cbits[k];
                cwo[c0 + k] = excl + cw[k];
            }
            if (c0 + NC == num_chunks) cwo[num_chunks] = excl + words;
        }
    }
    __syncthreads();
    uint32_t *dst = payload + (((uint64_t)sh.misc[2] << 32) | sh.misc[1]);
#pragma unroll
    for (int r = 0; r < NT; ++r) {
        uint64_t g[4];
        uint32_t ng[4];
        lane_groups(*reinterpret_cast<const uint4 *>(src + r * TILE), sh, g, ng);
        uint32_t p = (tb[r] & 31) + e[r];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            place_group(g[q], ng[q], p, sh.buf);
            p += ng[q];
        }
        __syncthreads();
        // a chunk's last tile ends with its partial word (the next chunk
        // starts on a new word); other tiles carry it to the next
        const bool last = r % TPC == TPC - 1;
        const uint32_t tend = last ? (uint32_t)(cw[r / TPC] * 32 + cbits[r / TPC]) : tb[r + 1];
        const uint32_t first_word = tb[r] >> 5;
        const uint32_t nfull = (tend >> 5) - first_word;
        const uint32_t nstore = last ? ((tend + 31) >> 5) - first_word : nfull;
        for (uint32_t i = tid; i < nstore; i += THREADS) dst[first_word + i] = sh.buf[i];
        const uint32_t carry = sh.buf[nfull];
        __syncthreads();
        for (uint32_t i = tid; i <= nfull + 2; i += THREADS) sh.buf[i] = (i == 0 && !last) ? carry : 0u;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Units of 64 KiB (1 to 64 whole chunks of 64 .. 1 KiB), persistent 512-lane
// workgroups, two per CU (128 registers per lane), taking units by ticket.
// A unit is eight tiles of 8 KiB; lane l of tile r owns its 16 symbols at
// r * 8192 + 16 l; entry 8 r + w is wave w's part of tile r (1 KiB), and a
// chunk is E consecutive entries.  One round, with unit B's input in
// registers and unit A (the previous one) placed in the LDS buffer:
//   phase 1: per tile, 16 (code, length) lookups become four groups of
//     <= 48 bits, kept in registers, and a wave scan of the bit counts; the
//     next unit's ticket is taken.
//   offsets: one barrier, then a wave scan over the 64 entry totals and one
//     over the chunks' words give every lane's bit offset in every tile, the
//     chunks' bit counts and first words, and B's word count, which is
//     published at once.
//   A's look-back (wave 0; A's count was published a round ago, so its
//     predecessors have mostly published theirs), then A is stored,
//     coalesced, at its final offset, clearing the buffer.
//   phase 2: B's groups are ORed into the buffer with no barrier; each
//     tile's registers then take the next unit's input for that tile.
// A unit whose words would not fit the buffer (only data that does not
// compress) does its look-back at once and is placed and stored in two
// halves of four tiles from the same registers.
// ---------------------------------------------------------------------------
constexpr uint32_t kUT = 512;                  // lanes
constexpr uint32_t kUW = kUT / 64;             // waves
constexpr uint32_t kUTiles = 8;                // tiles per unit
constexpr uint32_t kUTile = kUT * kSymPerLane; // 8192 symbols
constexpr uint32_t kUBufW = 16392;             // a unit at 8 bits per symbol, chunk padding and the fit margin

struct UnitShared {
    uint32_t tab[256];                 // code << 16 | length
    uint32_t wtot[kUTiles * kUW];      // per (tile, wave): bits
    uint32_t misc[4];                  // [0] ticket of this unit, [1] of the next, [2..3] its word offset
    uint2 cmeta[2][kUTiles * kUW];     // per round (two in flight), chunk's first entry: (bits, first word)
    uint32_t guard[4];                 // right before buf; its last two take zeros only (place_tile)
    uint32_t buf[kUBufW + 8];
};
static_assert(offsetof(UnitShared, buf) == offsetof(UnitShared, guard) + 16 && offsetof(UnitShared, buf) % 16 == 0,
              "the guard words sit right before the buffer, which is cleared in 16-byte stores");

// One lane's groups of one tile: two groups of <= 48 bits in three words (the
// high 16 bits of both in the third), and the four group lengths in bytes.
struct TileGroups {
    uint32_t w[6];
    uint32_t n;
};

__device__ __forceinline__ void keep_groups(const uint64_t (&g)[4], const uint32_t (&ng)[4], TileGroups &tg) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        tg.w[3 * h] = (uint32_t)g[2 * h];
        tg.w[3 * h + 1] = (uint32_t)g[2 * h + 1];
        tg.w[3 * h + 2] = (uint32_t)(g[2 * h] >> 32) | (uint32_t)(g[2 * h + 1] >> 32) << 16;
    }
    // byte 0 of each ng (the length; make_group_raw)
    tg.n = __builtin_amdgcn_perm(ng[1], ng[0], 0x0C0C0400u) | __builtin_amdgcn_perm(ng[3], ng[2], 0x04000C0Cu);
    // the packed words are what stays live (the compiler would otherwise
    // keep the 64-bit groups and the unpacked counts instead)
#pragma unroll
    for (int i = 0; i < 6; ++i) asm volatile("" : "+v"(tg.w[i]));
    asm volatile("" : "+v"(tg.n));
}

// A tile's four groups from bit p on, each placed from its end
// (place_group_end); base is the word two before buf[0] (in
// UnitShared::guard).
__device__ __forceinline__ void place_tile(const TileGroups &tg, uint32_t p, uint32_t *base) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t h = q >> 1;
        const uint32_t hi = (q & 1) ? tg.w[3 * h + 2] >> 16 : tg.w[3 * h + 2] & 0xFFFF;
        const uint32_t lo = tg.w[3 * h + (q & 1)];
        p += (tg.n >> (8 * q)) & 0xFF;
        place_group_end(hi, lo, p, base);
    }
}

// The unit's look-back (one wave) and its chunks' metadata; the exclusive
// word offset goes to sh.misc[2..3].  The chunks' bit counts and first words
// in the unit sit in sh.cmeta[slot] at each chunk's first entry (i % E == 0).
template <uint32_t E>
__device__ __forceinline__ void unit_meta(UnitShared &sh, uint32_t slot, uint64_t *desc, uint32_t s, uint64_t words,
                                          uint32_t lane, uint32_t max_polls, uint32_t *status, uint32_t *chunk_bits,
                                          uint64_t *cwo, uint32_t num_chunks) {
    constexpr uint32_t NC = 64 / E;
    const uint64_t excl = lookback(desc, s, words, lane, max_polls, status, true);
    const uint32_t c0 = s * NC;
    if (lane % E == 0) {
        const uint2 m = sh.cmeta[slot][lane];
        chunk_bits[c0 + lane / E] = m.x;
        cwo[c0 + lane / E] = excl + m.y;
    }
    if (lane == 0) {
        sh.misc[2] = (uint32_t)excl;
        sh.misc[3] = (uint32_t)(excl >> 32);
        if (c0 + NC == num_chunks) cwo[num_chunks] = excl + words;
    }
}

__device__ __forceinline__ uint64_t unit_excl(const UnitShared &sh) {
    return ((uint64_t)sh.misc[3] << 32) | sh.misc[2];
}

// Stores words [0, nw) of the buffer at dst (unit word fb sits at dst) and
// clears them: after a head up to a 128-byte boundary every wave writes
// whole lines.
__device__ __forceinline__ void store_unit(uint32_t *buf, uint32_t *dst, uint64_t at, uint32_t nw, uint32_t tid) {
    const uint32_t hd = (uint32_t)((32 - (at & 31)) & 31);
    const uint32_t head = hd < nw ? hd : nw;
    if (tid < head) {
        __builtin_nontemporal_store(buf[tid], dst + tid);
        buf[tid] = 0;
    }
    for (uint32_t i = head + tid; i < nw; i += kUT) {
        __builtin_nontemporal_store(buf[i], dst + i);
        buf[i] = 0;
    }
}

template <uint32_t E>  // (tile, wave) entries per chunk: 64 .. 1 (chunks of 64 .. 1 KiB)
__global__ __launch_bounds__(kUT) __attribute__((amdgpu_waves_per_eu(4))) void encode_unit_kernel(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint32_t num_chunks, uint32_t num_units,
    uint32_t *__restrict__ payload, uint32_t *__restrict__ chunk_bits, uint64_t *__restrict__ cwo,
    uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws, uint32_t *__restrict__ status, uint32_t max_polls) {
    __shared__ UnitShared sh;
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = uniform(tid >> 6);
    uint32_t *ticket = reinterpret_cast<uint32_t *>(ws);
    uint64_t *desc = ws + 1;
    if (tid == 0) sh.misc[0] = atomicAdd(ticket, 1u);
    if (tid < 256) {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.tab[tid] = ((uint32_t)reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid] << 16) | cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < (kUBufW + 8) / 4; i += kUT) reinterpret_cast<uint4 *>(sh.buf)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    uint32_t s = uniform(sh.misc[0]);
    uint4 x[kUTiles];
    if (s < num_units) {
        const uint8_t *src = in + (uint64_t)s * (kUTiles * kUTile) + tid * 16;
#pragma unroll
        for (uint32_t r = 0; r < kUTiles; ++r) x[r] = load_stream16(src + r * kUTile);
    }
    // the unit placed in the buffer last round, still to be stored
    bool have_a = false;
    uint32_t sa = 0, words_a = 0, slot = 0;  // slot: this round's half of sh.cmeta
    while (true) {
        // the lane index passes an opaque step each round, so that values
        // derived from it are recomputed rather than held (and spilled)
        // across the loop
        uint32_t tl = tid;
        asm volatile("" : "+v"(tl));
        const uint32_t ln = tl & 63;
        const bool live = s < num_units;
        // ---- phase 1: lookups, groups, wave scans ----------------------
        TileGroups tg[kUTiles];
        uint32_t ex[kUTiles];  // bits before the lane within its wave, per tile
        if (live) {
#pragma unroll
            for (uint32_t r = 0; r < kUTiles; ++r) {
                uint64_t g[4];
                uint32_t ng[4];
                // one tile's lookups at a time: the input passes an opaque
                // step ordered after the previous tile's packed groups
                // (hoisting all lookups would keep 128 results live)
                asm volatile("" : "+v"(x[r].x), "+v"(x[r].y), "+v"(x[r].z), "+v"(x[r].w));
                lane_groups_raw(x[r], sh, g, ng);
                const uint32_t bits = (ng[0] + ng[1] + ng[2] + ng[3]) & 0xFFFF;
                const uint32_t incl = wave_incl_scan(bits);
                if (ln == 63) sh.wtot[r * kUW + wave] = incl;
                ex[r] = incl - bits;
                keep_groups(g, ng, tg[r]);
            }
            if (tl == 0) sh.misc[1] = atomicAdd(ticket, 1u);
        }
        __syncthreads();
        // ---- offsets: a scan over the 64 (tile, wave) totals -------------
        // lane i of every wave holds entry i = 8 r + w (tile r, wave w);
        // chunk k of the unit is entries k E .. k E + E - 1 and starts on a
        // new word (word cw of the unit's buffer)
        uint32_t s_next = 0, words = 0, half_base = 0;
        uint32_t pos[kUTiles];
        if (live) {
            s_next = uniform(sh.misc[1]);
            const uint32_t v = sh.wtot[ln];
            const uint32_t incl = wave_incl_scan(v);
            const uint32_t exs = incl - v;
            const uint32_t lead = ln & ~(E - 1);  // the chunk's first entry
            const uint32_t cstart = (uint32_t)__shfl((int)exs, (int)lead);
            const uint32_t cbits = (uint32_t)__shfl((int)incl, (int)(lead + E - 1)) - cstart;
            const uint32_t cwords = ln == lead ? (cbits + 31) >> 5 : 0u;
            const uint32_t wincl = wave_incl_scan(cwords);
            const uint32_t cw = (uint32_t)__shfl((int)(wincl - cwords), (int)lead);
            words = (uint32_t)__builtin_amdgcn_readlane((int)wincl, 63);
            if (wave == 0 && ln == lead) sh.cmeta[slot][ln] = make_uint2(cbits, cw);
            const uint32_t cwb = cw * 32;
            const uint32_t base = cwb + exs - cstart;  // entry's first bit in the unit's buffer
            half_base = (uint32_t)__builtin_amdgcn_readlane((int)base, (int)(kUTiles / 2 * kUW));
            // the lane's first bit of tile r in the unit's buffer
#pragma unroll
            for (uint32_t r = 0; r < kUTiles; ++r)
                pos[r] = (uint32_t)__builtin_amdgcn_readlane((int)base, (int)(r * kUW + wave)) + ex[r];
            // side index: every 256th symbol starts on a lane with
            // lane % 16 == 0 (a chunk has E * 4 sub-streams, so the unit's
            // run from s * 256); entries are relative to their chunk
            if ((ln & 15) == 0) {
                uint32_t *so = sub_off + (uint64_t)s * (kUTiles * kUTile / kSub) + (tl >> 4);
#pragma unroll
                for (uint32_t r = 0; r < kUTiles; ++r)
                    so[r * (kUTile / kSub)] = pos[r] - (uint32_t)__builtin_amdgcn_readlane((int)cwb, (int)(r * kUW + wave));
            }
            if (wave == 0 && ln == 0) publish_count(desc, s, words);
        }
        // ---- the previous unit: look-back, then its store ----------------
        // (its count was published a round ago, so its predecessors have
        // mostly published theirs)
        if (have_a) {
            if (wave == 0)
                unit_meta<E>(sh, slot ^ 1u, desc, sa, words_a, ln, max_polls, status, chunk_bits, cwo, num_chunks);
            __syncthreads();
            const uint64_t at = unit_excl(sh);
            store_unit(sh.buf, payload + at, at, words_a, tl);
        }
        // the buffer is clear and every wave has read the totals
        __syncthreads();
        if (!live) break;
        // the next unit's input is loaded while this one is placed; after
        // the last unit every lane reads the input's first 16 bytes (a
        // load on every path: a conditional one would keep the old values
        // live through both phases)
        const bool more = s_next < num_units;
        const uint8_t *nsrc = more ? in + (uint64_t)s_next * (kUTiles * kUTile) + tl * 16 : in;
        const uint32_t nstride = more ? kUTile : 0u;
        if (words <= kUBufW - 2) {
            // ---- phase 2: place every group, no barrier -----------------
#pragma unroll
            for (uint32_t r = 0; r < kUTiles; ++r) {
                place_tile(tg[r], pos[r], sh.guard + 2);
                x[r] = load_stream16(nsrc + r * nstride);
                asm volatile("" ::: "memory");
            }
            have_a = true;
            sa = s;
            words_a = words;
        } else {
            // ---- a unit that does not fit the buffer (only data that does
            // not compress): its look-back now, then two halves of four
            // tiles (each fits) -------------------------------------------
            if (wave == 0) unit_meta<E>(sh, slot, desc, s, words, ln, max_polls, status, chunk_bits, cwo, num_chunks);
            constexpr uint32_t kHalf = kUTiles / 2;
#pragma unroll
            for (uint32_t r = 0; r < kHalf; ++r) place_tile(tg[r], pos[r], sh.guard + 2);
            __syncthreads();
            const uint64_t excl = unit_excl(sh);
            // unit word fb holds the bits of both halves; whole words
            // before it go out, it moves to buf[0]
            const uint32_t fb = half_base >> 5;
            for (uint32_t i = tl; i < fb; i += kUT) payload[excl + i] = sh.buf[i];
            const uint32_t carry = sh.buf[fb];
            __syncthreads();
            for (uint32_t i = tl; i <= fb + 2; i += kUT) sh.buf[i] = i == 0 ? carry : 0u;
            __syncthreads();
#pragma unroll
            for (uint32_t r = kHalf; r < kUTiles; ++r) place_tile(tg[r], pos[r] - fb * 32, sh.guard + 2);
            __syncthreads();
            store_unit(sh.buf, payload + excl + fb, excl + fb, words - fb, tl);
#pragma unroll
            for (uint32_t r = 0; r < kUTiles; ++r) x[r] = load_stream16(nsrc + r * nstride);
            __syncthreads();
            have_a = false;
        }
        s = s_next;
        slot ^= 1u;
    }
}

// ---------------------------------------------------------------------------
// Chunks of a multiple of 64 KiB above 64 KiB.  A chunk is then several
// 64 KiB units whose bitstreams join mid-word, so a unit cannot start on a
// word boundary, and a look-back over units would have to round up to a
// word at every chunk end.  Three launches instead, with no device-side
// wait: count (every unit's bit count), scan (one workgroup: the chunks' bit
// counts and word offsets, each unit's bit offset in its chunk, and the
// payload words at unit edges cleared), place (every unit at its known
// offset: inner words stored, the first and last word OR-ed in with device
// atomics, since the neighbouring unit of the chunk may share them).  The
// input is read twice.
// ---------------------------------------------------------------------------
constexpr uint32_t kBigUnit = kUTiles * kUTile;  // 65536 symbols

__global__ __launch_bounds__(256) void encode_count_kernel(const pc_codebook *__restrict__ cb,
                                                           const uint8_t *__restrict__ in,
                                                           uint32_t *__restrict__ unit_bits) {
    __shared__ uint32_t len[256];
    __shared__ uint32_t wsum[4];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    len[tid] = reinterpret_cast<const uint8_t *>(cb)[kOffLength + tid];
    const uint8_t *src = in + (uint64_t)blockIdx.x * kBigUnit + tid * 16;
    uint4 x[16];
#pragma unroll
    for (uint32_t r = 0; r < 16; ++r) x[r] = load_stream16(src + r * 4096);
    __syncthreads();
    uint32_t bits = 0;
#pragma unroll
    for (uint32_t r = 0; r < 16; ++r) {
        const uint32_t w[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bits += len[w[q] & 0xFF] + len[(w[q] >> 8) & 0xFF] + len[(w[q] >> 16) & 0xFF] + len[w[q] >> 24];
    }
    const uint32_t incl = wave_incl_scan(bits);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) unit_bits[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// One workgroup.  In: unit_bits[u] for the nfull * U units.  Out:
// chunk_bits and chunk_word_offset of the full chunks (cwo[nfull] = their
// total words), unit_bits[u] replaced by the unit's bit offset in its chunk,
// the payload words at both edges of every unit cleared, and descriptor 0
// published inclusive with the total (a short last chunk looks back to it).
__global__ __launch_bounds__(1024) void encode_unit_scan_kernel(uint32_t *__restrict__ unit_bits, uint32_t U,
                                                                uint32_t nfull, uint32_t *__restrict__ chunk_bits,
                                                                uint64_t *__restrict__ cwo,
                                                                uint32_t *__restrict__ payload,
                                                                uint64_t *__restrict__ desc0) {
    __shared__ uint32_t wtot[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t carry = 0;  // words of the chunks before this block (uniform)
    for (uint32_t base = 0; base < nfull; base += 1024) {
        const uint32_t c = base + tid;
        uint32_t cbits = 0;
        if (c < nfull)
            for (uint32_t k = 0; k < U; ++k) cbits += unit_bits[(uint64_t)c * U + k];
        // a chunk has at most 2^24 * 12 bits, so 64 chunks' words fit 32 bits
        const uint32_t words = c < nfull ? (cbits + 31) >> 5 : 0u;
        const uint32_t incl = wave_incl_scan(words);
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        uint64_t before = carry, total = carry;
        for (uint32_t w = 0; w < 16; ++w) {
            const uint64_t t = wtot[w];
            before += w < wave ? t : 0;
            total += t;
        }
        if (c < nfull) {
            const uint64_t cw = before + incl - words;
            chunk_bits[c] = cbits;
            cwo[c] = cw;
            uint32_t off = 0;
            for (uint32_t k = 0; k < U; ++k) {
                const uint64_t u = (uint64_t)c * U + k;
                const uint32_t b = unit_bits[u];
                unit_bits[u] = off;
                const uint64_t p = cw * 32 + off;
                payload[p >> 5] = 0;
                payload[(p + b - 1) >> 5] = 0;
                off += b;
            }
        }
        carry = total;
        __syncthreads();  // wtot is read before the next block writes it
    }
    if (tid == 0) {
        cwo[nfull] = carry;
        st_desc(desc0, kDescInclusive | carry);
    }
}

// Stores buffer words [i0, i1) to dst[i0 ..] (plain, non-temporal), lanes
// spread over whole lines from the first 128-byte boundary on.
__device__ __forceinline__ void store_words(const uint32_t *buf, uint32_t *dst, uint64_t dst_word, uint32_t i0,
                                            uint32_t i1, uint32_t tid) {
    if (i1 <= i0) return;
    const uint32_t hd = (uint32_t)((32 - ((dst_word + i0) & 31)) & 31);
    const uint32_t head = i0 + (hd < i1 - i0 ? hd : i1 - i0);
    if (i0 + tid < head) __builtin_nontemporal_store(buf[i0 + tid], dst + i0 + tid);
    for (uint32_t i = head + tid; i < i1; i += kUT) __builtin_nontemporal_store(buf[i], dst + i);
}

__global__ __launch_bounds__(kUT) __attribute__((amdgpu_waves_per_eu(4))) void encode_placed_kernel(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint32_t U,
    const uint32_t *__restrict__ unit_off, const uint64_t *__restrict__ cwo, uint32_t *__restrict__ payload,
    uint32_t *__restrict__ sub_off) {
    __shared__ UnitShared sh;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = uniform(tid >> 6);
    const uint32_t u = blockIdx.x;
    const uint32_t c = u / U;
    if (tid < 256) {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.tab[tid] = ((uint32_t)reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid] << 16) | cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < (kUBufW + 8) / 4; i += kUT) reinterpret_cast<uint4 *>(sh.buf)[i] = make_uint4(0, 0, 0, 0);
    uint4 x[kUTiles];
    const uint8_t *src = in + (uint64_t)u * kBigUnit + tid * 16;
#pragma unroll
    for (uint32_t r = 0; r < kUTiles; ++r) x[r] = load_stream16(src + r * kUTile);
    // the unit's first bit in the payload
    const uint64_t P = cwo[c] * 32 + unit_off[u];
    __syncthreads();
    TileGroups tg[kUTiles];
    uint32_t ex[kUTiles];
#pragma unroll
    for (uint32_t r = 0; r < kUTiles; ++r) {
        uint64_t g[4];
        uint32_t ng[4];
        asm volatile("" : "+v"(x[r].x), "+v"(x[r].y), "+v"(x[r].z), "+v"(x[r].w));
        lane_groups_raw(x[r], sh, g, ng);
        const uint32_t bits = (ng[0] + ng[1] + ng[2] + ng[3]) & 0xFFFF;
        const uint32_t incl = wave_incl_scan(bits);
        if (lane == 63) sh.wtot[r * kUW + wave] = incl;
        ex[r] = incl - bits;
        keep_groups(g, ng, tg[r]);
    }
    __syncthreads();
    const uint32_t v = sh.wtot[lane];
    const uint32_t incl = wave_incl_scan(v);
    const uint32_t exs = incl - v;
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t p0 = (uint32_t)(uniform64(P) & 31);
    const uint64_t w0 = uniform64(P) >> 5;
    const uint32_t off = unit_off[u];
    uint32_t pos[kUTiles];
#pragma unroll
    for (uint32_t r = 0; r < kUTiles; ++r)
        pos[r] = (uint32_t)__builtin_amdgcn_readlane((int)exs, (int)(r * kUW + wave)) + ex[r];
    // side index: a chunk has U * 256 sub-streams, unit u's run from u * 256
    if ((lane & 15) == 0) {
        uint32_t *so = sub_off + (uint64_t)u * (kBigUnit / kSub) + (tid >> 4);
#pragma unroll
        for (uint32_t r = 0; r < kUTiles; ++r) so[r * (kUTile / kSub)] = off + pos[r];
    }
    const uint32_t nw = (p0 + total + 31) >> 5;
    uint32_t *dst = payload + w0;
    if (nw <= kUBufW - 2) {
#pragma unroll
        for (uint32_t r = 0; r < kUTiles; ++r) place_tile(tg[r], p0 + pos[r], sh.guard + 2);
        __syncthreads();
        // the unit's first and last word may hold a neighbour's bits
        if (tid == 0) atomicOr(dst, sh.buf[0]);
        if (tid == kUT - 1 && nw > 1) atomicOr(dst + nw - 1, sh.buf[nw - 1]);
        store_words(sh.buf, dst, w0, 1, nw - 1, tid);
    } else {
        // more words than the buffer holds (data that does not compress):
        // two halves of four tiles
        constexpr uint32_t kHalf = kUTiles / 2;
#pragma unroll
        for (uint32_t r = 0; r < kHalf; ++r) place_tile(tg[r], p0 + pos[r], sh.guard + 2);
        __syncthreads();
        const uint32_t fb = (p0 + (uint32_t)__builtin_amdgcn_readlane((int)exs, (int)(kHalf * kUW))) >> 5;
        if (tid == 0) atomicOr(dst, sh.buf[0]);
        store_words(sh.buf, dst, w0, 1, fb, tid);
        const uint32_t carry = sh.buf[fb];
        __syncthreads();
        for (uint32_t i = tid; i <= fb + 2; i += kUT) sh.buf[i] = i == 0 ? carry : 0u;
        __syncthreads();
#pragma unroll
        for (uint32_t r = kHalf; r < kUTiles; ++r) place_tile(tg[r], p0 + pos[r] - fb * 32, sh.guard + 2);
        __syncthreads();
        if (tid == kUT - 1) atomicOr(dst + nw - 1, sh.buf[nw - 1 - fb]);
        store_words(sh.buf, dst + fb, w0 + fb, 0, nw - 1 - fb, tid);
    }
}

// Any chunk size: the counting pass and the packing pass each read the
// chunk (the second read is served by the caches for moderate chunks).
// A workgroup takes ticket t from counter `counter` (0 or 1) of workspace
// word 0; its look-back index is t + dbase and it encodes chunk t + cbase
// (a launch of multi-chunk workgroups may go first).
__global__ __launch_bounds__(kThreads) void encode_kernel_any(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint64_t n, uint32_t chunk,
    uint32_t num_chunks, uint32_t *__restrict__ payload, uint32_t *__restrict__ chunk_bits,
    uint64_t *__restrict__ cwo, uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws, uint32_t counter,
    uint32_t dbase, uint32_t cbase, uint32_t *__restrict__ status, uint32_t max_polls) {
    using SH = Shared<kThreads>;
    __shared__ SH sh;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sh.misc[0] = atomicAdd(reinterpret_cast<uint32_t *>(ws) + counter, 1u) + dbase;
    {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.code[tid] = reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid];
        sh.len[tid] = cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < SH::kStage; i += kThreads) sh.stage[i] = 0;
    __syncthreads();
    const uint32_t t = uniform(sh.misc[0]);
    const uint32_t c = t - dbase + cbase;
    const uint64_t base = (uint64_t)c * chunk;
    const uint32_t lenc = (uint32_t)((n - base) < chunk ? (n - base) : chunk);
    const uint32_t ntiles = (lenc + kTile - 1) / kTile;

    uint32_t mine = 0;
    for (uint32_t r = 0; r < ntiles; ++r) {
        const uint32_t off = r * kTile + tid * kSymPerLane;
        mine += lane_bits(load_lane(in, base, off, lenc), lane_valid(off, lenc), sh);
    }
    const uint32_t wsum = wave_incl_scan(mine);
    if (lane == 63) sh.wave_tot[0][wave] = wsum;
    __syncthreads();
    const uint32_t total = uniform(sh.wave_tot[0][0] + sh.wave_tot[0][1] + sh.wave_tot[0][2] + sh.wave_tot[0][3]);
    const uint64_t words = (total + 31) >> 5;
    if (wave == 0) {
        const uint64_t excl = lookback(ws + 1, t, words, lane, max_polls, status);
        if (lane == 0) {
            sh.misc[1] = (uint32_t)excl;
            sh.misc[2] = (uint32_t)(excl >> 32);
        }
    }
    __syncthreads();
    const uint64_t excl = ((uint64_t)sh.misc[2] << 32) | sh.misc[1];
    if (tid == 0) {
        chunk_bits[c] = total;
        cwo[c] = excl;
        if (c == num_chunks - 1) cwo[num_chunks] = excl + words;
    }
    uint32_t *dst = payload + excl;
    uint32_t *so = sub_off + (uint64_t)c * (chunk / kSub);

    uint32_t tbeg = 0;
    for (uint32_t r = 0; r < ntiles; ++r) {
        const uint32_t off = r * kTile + tid * kSymPerLane;
        const uint32_t valid = lane_valid(off, lenc);
        const uint4 x = load_lane(in, base, off, lenc);
        const uint32_t bits = lane_bits(x, valid, sh);
        const uint32_t incl = wave_incl_scan(bits);
        // wave_tot[1] holds this tile's per-wave totals (wave_tot[0] is read
        // above only before the look-back barrier)
        if (lane == 63) sh.wave_tot[1][wave] = incl;
        __syncthreads();
        const uint32_t w0 = sh.wave_tot[1][0], w1 = sh.wave_tot[1][1];
        const uint32_t w2 = sh.wave_tot[1][2], w3 = sh.wave_tot[1][3];
        const uint32_t e = incl - bits + (wave > 0 ? w0 : 0) + (wave > 1 ? w1 : 0) + (wave > 2 ? w2 : 0);
        const uint32_t tend = uniform(tbeg + w0 + w1 + w2 + w3);
        if ((tid & 15) == 0 && valid) so[off / kSub] = tbeg + e;
        pack_lane(x, valid, (tbeg & 31) + e, sh);
        __syncthreads();
        flush_tile<kThreads>(sh, dst, tbeg, tend, r + 1 == ntiles, tid);
        tbeg = tend;
    }
}

// ---------------------------------------------------------------------------
// Small chunks of any size (a multiple of 256 bytes, at most 32 KiB): a
// workgroup takes K consecutive full chunks (K * chunk <= 64 KiB, K <= 64),
// so that the cross-chunk scan runs once per K chunks instead of once per
// chunk.  Two passes over the K chunks:
//   1. count: every lane's 16 code lengths, summed over its row of 16 lanes
//      (one 256-symbol sub-stream; rows and sub-streams coincide because a
//      tile starts on a sub-stream); then one scan over the <= 256
//      sub-streams gives each sub-stream's bit offset inside its chunk (the
//      side index), each chunk's bit count and, by a wave scan over the K
//      chunks' word counts, each chunk's first word relative to the first
//      chunk; the look-back turns the K chunks' word total into their
//      offset in the payload;
//   2. pack: per tile of 4096 symbols, every lane's codewords are ORed into
//      the staging words at its known bit position (chunk start word * 32 +
//      sub-stream offset + the lane's offset in its row) and the tile's
//      words are stored, the tile ending where the next one starts (so the
//      zero padding after a chunk that ends inside a tile is stored with it).
// ---------------------------------------------------------------------------
constexpr uint32_t kMultiMaxChunks = 64;
constexpr uint32_t kMultiBytes = 65536;

struct MultiShared {
    // a tile spans <= 4096 * 12 bits, the padding of <= 16 chunk ends and the
    // offset of its first bit in its first word; pack_lane may OR zeros two
    // words past the last
    static constexpr uint32_t kStage = kTile * PC_MAX_LEN / 32 + 16 + 8;
    uint16_t code[256];
    uint8_t len[256];
    uint32_t wave_tot[kThreads / 64];
    uint32_t sub_bits[kMultiBytes / kSub];  // per sub-stream of the K chunks
    uint32_t sub_excl[kMultiBytes / kSub];  // bits before it, counted from the first chunk's start (no padding)
    uint32_t rel[kMultiMaxChunks + 1];      // chunk j's first word relative to chunk 0's; [K] = the total
    uint32_t misc[4];
    uint32_t stage[kStage];
};

// Inclusive prefix sum over each row of 16 lanes.
__device__ __forceinline__ uint32_t row_incl_scan(uint32_t v) {
    v += dpp_u32<0x111>(v);  // row_shr:1
    v += dpp_u32<0x112>(v);  // row_shr:2
    v += dpp_u32<0x114>(v);  // row_shr:4
    v += dpp_u32<0x118>(v);  // row_shr:8
    return v;
}

// Bit position, relative to chunk 0's first word, of sub-stream s's first
// bit (s below the K chunks' sub-stream count).
__device__ __forceinline__ uint32_t multi_sub_pos(const MultiShared &sh, uint32_t s, uint32_t spc) {
    const uint32_t j = s / spc;
    return sh.rel[j] * 32 + (sh.sub_excl[s] - sh.sub_excl[j * spc]);
}

__global__ __launch_bounds__(kThreads) void encode_multi_kernel(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint32_t chunk, uint32_t K,
    uint32_t num_chunks, uint32_t *__restrict__ payload, uint32_t *__restrict__ chunk_bits,
    uint64_t *__restrict__ cwo, uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws,
    uint32_t *__restrict__ status, uint32_t max_polls) {
    __shared__ MultiShared sh;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sh.misc[0] = atomicAdd(reinterpret_cast<uint32_t *>(ws), 1u);
    {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.code[tid] = reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid];
        sh.len[tid] = cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < MultiShared::kStage; i += kThreads) sh.stage[i] = 0;
    __syncthreads();
    const uint32_t t = uniform(sh.misc[0]);  // look-back index; chunks t K .. t K + K - 1
    const uint32_t c0 = t * K;
    const uint64_t base = (uint64_t)c0 * chunk;
    const uint32_t L = K * chunk;  // bytes of the K chunks (all full)
    const uint32_t spc = chunk / kSub, nsub = L / kSub;
    const uint32_t ntiles = (L + kTile - 1) / kTile;

    // ---- 1. count: bits per sub-stream ------------------------------------
    for (uint32_t r = 0; r < ntiles; ++r) {
        const uint32_t off = r * kTile + tid * kSymPerLane;
        const uint32_t valid = lane_valid(off, L);
        const uint32_t row = row_incl_scan(lane_bits(load_lane(in, base, off, L), valid, sh));
        const uint32_t s = r * (kTile / kSub) + (tid >> 4);
        if ((tid & 15) == 15 && s < nsub) sh.sub_bits[s] = row;
    }
    __syncthreads();
    const uint32_t bs = tid < nsub ? sh.sub_bits[tid] : 0u;
    const uint32_t incl = wave_incl_scan(bs);
    if (lane == 63) sh.wave_tot[wave] = incl;
    __syncthreads();
    const uint32_t sx = incl - bs + (wave > 0 ? sh.wave_tot[0] : 0u) + (wave > 1 ? sh.wave_tot[1] : 0u) +
                        (wave > 2 ? sh.wave_tot[2] : 0u);
    sh.sub_excl[tid] = sx;
    __syncthreads();
    if (tid < nsub) {
        const uint32_t j = tid / spc, first = j * spc;
        const uint32_t in_chunk = sx - sh.sub_excl[first];
        sub_off[(uint64_t)c0 * spc + tid] = in_chunk;
        if (tid - first == spc - 1) {
            const uint32_t bits = in_chunk + bs;
            chunk_bits[c0 + j] = bits;
            sh.rel[j] = (bits + 31) >> 5;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t wj = lane < K ? sh.rel[lane] : 0u;
        const uint32_t wi = wave_incl_scan(wj);
        const uint32_t W = uniform((uint32_t)__shfl(wi, 63, 64));
        const uint64_t excl = lookback(ws + 1, t, W, lane, max_polls, status);
        if (lane < K) {
            cwo[c0 + lane] = excl + (wi - wj);
            sh.rel[lane] = wi - wj;
        }
        if (lane == 0) {
            sh.rel[K] = W;
            if (c0 + K == num_chunks) cwo[num_chunks] = excl + W;
            sh.misc[1] = (uint32_t)excl;
            sh.misc[2] = (uint32_t)(excl >> 32);
        }
    }
    __syncthreads();
    uint32_t *dst = payload + (((uint64_t)sh.misc[2] << 32) | sh.misc[1]);
    const uint32_t total_bits = sh.rel[K] * 32;

    // ---- 2. pack ------------------------------------------------------------
    for (uint32_t r = 0; r < ntiles; ++r) {
        const uint32_t off = r * kTile + tid * kSymPerLane;
        const uint32_t valid = lane_valid(off, L);
        const uint4 x = load_lane(in, base, off, L);
        const uint32_t b = lane_bits(x, valid, sh);
        const uint32_t rowx = row_incl_scan(b) - b;
        const uint32_t s0 = r * (kTile / kSub);
        const uint32_t tbeg = uniform(multi_sub_pos(sh, s0, spc));
        const uint32_t s1 = s0 + kTile / kSub;
        const uint32_t tend = uniform(s1 < nsub ? multi_sub_pos(sh, min(s1, nsub - 1), spc) : total_bits);
        const uint32_t s = min(s0 + (tid >> 4), nsub - 1);
        // a lane past the end ORs zeros at the stage's start
        const uint32_t p = valid ? multi_sub_pos(sh, s, spc) + rowx - (tbeg & ~31u) : 0u;
        pack_lane(x, valid, p, sh);
        __syncthreads();
        flush_tile<kThreads>(sh, dst, tbeg, tend, r + 1 == ntiles, tid);
    }
}

// Zero the ticket, the look-back descriptors and the status word; write the
// total-word entry for an empty input.
__global__ void encode_init_kernel(uint64_t *ws, uint64_t ws_words, uint64_t *cwo, int empty, uint32_t *status) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = i; k < ws_words; k += stride) ws[k] = 0;
    if (i == 0) {
        *status = 0;
        if (empty) cwo[0] = 0;
    }
}

}  // namespace

hipError_t launch_encode(const pc_codebook *cb, const uint8_t *in, uint64_t n, uint32_t chunk,
                         uint32_t *payload, uint32_t *chunk_bits, uint64_t *cwo, uint32_t *sub_off,
                         uint64_t *ws, uint32_t *status, uint32_t max_polls, hipStream_t stream) {
    const uint64_t nc = (n + chunk - 1) / chunk;
    const uint64_t ws_words = 1 + nc;
    const uint32_t init_blocks = (uint32_t)((ws_words + 255) / 256 < 1024 ? (ws_words + 255) / 256 : 1024);
    hipLaunchKernelGGL(encode_init_kernel, dim3(init_blocks ? init_blocks : 1), dim3(256), 0, stream, ws,
                       ws_words, cwo, n == 0 ? 1 : 0, status);
    if (n == 0) return hipGetLastError();
    const uint64_t nfull = n / chunk;  // chunks of exactly `chunk` symbols
    // Full chunks go to one of three launches, and the full chunks left
    // over and a short last chunk to the re-reading kernel, launched after
    // it, so that their look-backs find every predecessor finished:
    //   - power-of-two chunks of 1 .. 64 KiB on large inputs: the persistent
    //     unit kernel (64 KiB units of whole chunks);
    //   - multiples of 64 KiB above it: count, scan and place launches;
    //   - other chunks of at most 32 KiB: K consecutive chunks per
    //     workgroup (encode_multi_kernel), unless they are 4 .. 64 KiB
    //     powers of two:
    //   - otherwise 4 .. 64 KiB chunks: workgroups of NT tiles (TPC tiles per
    //     chunk, so NT / TPC consecutive chunks and one look-back per
    //     workgroup).  The 1024-lane kernels hold 64K symbols per
    //     workgroup; the LDS output buffer holds them at 8 bits per symbol
    //     plus the padding words between chunks and the 64-bit margin of the
    //     fit test (two such workgroups fit a CU).  4K and 8K symbol chunks
    //     take 256-lane workgroups of 32K symbols when there are many of
    //     them, else one chunk per workgroup, so that a small input still
    //     spreads over the CUs (the 1-chunk buffers hold 12 bits per symbol).
    // Other chunk sizes go to the re-reading kernel whole.
    constexpr uint64_t kManySmall = 8192;
    uint64_t done = 0, tickets = 0;  // chunks and look-back indices of the multi-chunk launch
    uint32_t counter = 0;            // the ticket counter of the re-reading kernel
#define PC_ENC(T, NT, BW, TPC)                                                                             \
    do {                                                                                                   \
        const uint64_t nsup = nfull / ((NT) / (TPC));                                                      \
        if (nsup) {                                                                                        \
            hipLaunchKernelGGL((encode_chunk_kernel<T, NT, BW, TPC>), dim3((uint32_t)nsup), dim3(T), 0,    \
                               stream, cb, in, n, chunk, (uint32_t)nc, payload, chunk_bits, cwo, sub_off,  \
                               ws, status, max_polls);                                                     \
            done = nsup * ((NT) / (TPC));                                                                  \
            tickets = nsup;                                                                                \
        }                                                                                               \
    } while (0)
#define PC_ENC_MULTI()                                                                                     \
    do {                                                                                                   \
        const uint32_t K = kMultiBytes / chunk < kMultiMaxChunks ? kMultiBytes / chunk : kMultiMaxChunks;  \
        const uint64_t nsup = nfull / K;                                                                   \
        if (nsup) {                                                                                        \
            hipLaunchKernelGGL(encode_multi_kernel, dim3((uint32_t)nsup), dim3(kThreads), 0, stream, cb, in, \
                               chunk, K, (uint32_t)nc, payload, chunk_bits, cwo, sub_off, ws, status,      \
                               max_polls);                                                                 \
            done = nsup * K;                                                                               \
            tickets = nsup;                                                                                \
        }                                                                                               \
    } while (0)
#define PC_ENC_UNIT(E)                                                                                     \
    do {                                                                                                   \
        const uint64_t nunits = nfull / (64 / (E));                                                        \
        uint64_t grid = 2 * (uint64_t)cus;                                                                 \
        if (grid > nunits) grid = nunits;                                                                  \
        hipLaunchKernelGGL((encode_unit_kernel<E>), dim3((uint32_t)grid), dim3(kUT), 0, stream, cb, in,    \
                           (uint32_t)nc, (uint32_t)nunits, payload, chunk_bits, cwo, sub_off, ws, status,  \
                           max_polls);                                                                     \
        done = nunits * (64 / (E));                                                                        \
        tickets = nunits;                                                                                  \
        counter = 1;                                                                                       \
    } while (0)
    // 64 .. 1 KiB chunks: the persistent unit kernel once every
    // workgroup gets at least four units (it keeps two in flight; below
    // that the chunk kernels, which start all their workgroups at once, are
    // as fast or faster, measured), or for 64 KiB chunks at least one (a
    // 43 MiB input: 0.045 against 0.0515 ms; 16 KiB chunks at 64 MiB stay
    // 7% faster on the chunk kernel)
    int cus = 0;
    if (chunk <= 65536 && chunk >= 1024 && (chunk & (chunk - 1)) == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const uint64_t unit_min = chunk == 65536 ? 2 : 8;  // units per CU (two workgroups each)
    const bool units = nfull * chunk >= (uint64_t)cus * unit_min * kUTiles * kUTile && cus > 0;
    uint64_t dbase = 0, cbase = 0;  // look-back index and chunk of the re-reading kernel's ticket 0
    bool dset = false;
    if (chunk > kBigUnit && chunk % kBigUnit == 0) {
        if (nfull) {
            // chunks of several 64 KiB units: count, scan, place (above)
            const uint32_t U = chunk / kBigUnit;
            const uint64_t nunits = nfull * U;
            uint32_t *unit_bits = reinterpret_cast<uint32_t *>(ws + 1 + nc);
            hipLaunchKernelGGL(encode_count_kernel, dim3((uint32_t)nunits), dim3(256), 0, stream, cb, in, unit_bits);
            hipLaunchKernelGGL(encode_unit_scan_kernel, dim3(1), dim3(1024), 0, stream, unit_bits, U, (uint32_t)nfull,
                               chunk_bits, cwo, payload, ws + 1);
            hipLaunchKernelGGL(encode_placed_kernel, dim3((uint32_t)nunits), dim3(kUT), 0, stream, cb, in, U,
                               unit_bits, cwo, payload, sub_off);
            done = nfull;
            // a short last chunk looks back to descriptor 0, which the scan
            // published inclusive
            dbase = 1;
            cbase = nfull;
            dset = true;
        }
    } else if (chunk == 65536 && units) PC_ENC_UNIT(64);
    else if (chunk == 32768 && units) PC_ENC_UNIT(32);
    else if (chunk == 16384 && units) PC_ENC_UNIT(16);
    else if (chunk == 8192 && units) PC_ENC_UNIT(8);
    else if (chunk == 4096 && units) PC_ENC_UNIT(4);
    else if (chunk == 2048 && units) PC_ENC_UNIT(2);
    else if (chunk == 1024 && units) PC_ENC_UNIT(1);
    else if (chunk == 65536) PC_ENC(1024, 4, 16392, 4);
    else if (chunk == 32768) PC_ENC(1024, 4, 16392, 2);
    else if (chunk == 16384) PC_ENC(1024, 4, 16392, 1);
    else if (chunk == 8192 && nfull >= kManySmall) PC_ENC(256, 8, 8200, 2);
    else if (chunk == 8192) PC_ENC(256, 2, 3072, 2);
    else if (chunk == 4096 && nfull >= kManySmall) PC_ENC(256, 8, 8200, 1);
    else if (chunk == 4096) PC_ENC(256, 1, 1536, 1);
    else if (2 * chunk <= kMultiBytes) PC_ENC_MULTI();
    const uint64_t rest = nc - done;
    // look-back indices continue from the multi-chunk launch's: after the
    // chunk kernels (which take exactly `tickets` tickets from counter 0)
    // ticket t encodes chunk t + done - tickets; after the persistent unit
    // kernel (which may take extra tickets of counter 0) the tickets of
    // counter 1 start at 0, look-back index tickets + t, chunk done + t;
    // after the three launches of multi-unit chunks, ticket 0 of counter 0
    // has look-back index 1 (descriptor 0 holds the full chunks' words)
    if (rest) {
        if (!dset) {
            dbase = counter ? tickets : 0u;
            cbase = counter ? done : done - tickets;
        }
        hipLaunchKernelGGL(encode_kernel_any, dim3((uint32_t)rest), dim3(kThreads), 0, stream, cb, in, n, chunk,
                           (uint32_t)nc, payload, chunk_bits, cwo, sub_off, ws, counter, (uint32_t)dbase,
                           (uint32_t)cbase, status, max_polls);
    }
#undef PC_ENC
#undef PC_ENC_MULTI
#undef PC_ENC_UNIT
    return hipGetLastError();
}

}  // namespace pc
