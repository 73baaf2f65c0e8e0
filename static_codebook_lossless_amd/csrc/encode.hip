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
// The wait on predecessors is bounded: it always ends once they publish,
// but should an ordering bug ever leave a predecessor silent, the wave gives
// up after ~2^20 polls (about a second) and sets bit 32 of workspace word 0
// instead of spinning forever.
constexpr uint32_t kMaxPolls = 1u << 20;
constexpr int kLookWin = 2;  // descriptors per lane per round

// Publish descriptor c's own count: inclusive for c == 0, else aggregate.
__device__ __forceinline__ void publish_count(uint64_t *desc, uint32_t c, uint64_t words) {
    st_desc(&desc[c], (c == 0 ? kDescInclusive : kDescAggregate) | words);
}

// `published`: the caller already ran publish_count for c.
__device__ uint64_t lookback(uint64_t *desc, uint32_t c, uint64_t words, uint32_t lane, bool published = false) {
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
            if (polls == kMaxPolls) {
                if (lane == 0) atomicOr(reinterpret_cast<unsigned long long *>(desc - 1), 1ull << 32);
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
// lane (an OR with zero changes nothing): with the second and third made
// conditional, exec-masked LDS atomics of this shape were seen to lose
// updates on gfx950 (one wave's words of a tile came out with bits missing,
// varying from run to run).
__device__ __forceinline__ void place_group(uint64_t g, uint32_t ng, uint32_t p, uint32_t *buf) {
    const uint64_t a = g << (64 - ng);
    const uint32_t hi = (uint32_t)(a >> 32), lo = (uint32_t)a;
    const uint32_t o = p & 31, wi = p >> 5;
    atomicOr(&buf[wi], hi >> o);
    atomicOr(&buf[wi + 1], __builtin_amdgcn_alignbit(hi, lo, o));
    atomicOr(&buf[wi + 2], __builtin_amdgcn_alignbit(lo, 0u, o));
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
    uint64_t *__restrict__ cwo, uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws) {
    using SH = ChunkShared<THREADS, NT, BUFW>;
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
        lane_groups(xc, sh, g, ng);
        const uint32_t bits = ng[0] + ng[1] + ng[2] + ng[3];
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
                place_group(g[q], ng[q], p, sh.buf);
                p += ng[q];
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
            HN[hr] = ng[0] | ng[1] << 8 | ng[2] << 16 | ng[3] << 24;
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
                const uint64_t g = ((uint64_t)hi << 32) | HG[hr][3 * h + (q & 1)];
                const uint32_t ng = (HN[hr] >> (8 * q)) & 0xFF;
                place_group(g, ng, p, sh.buf);
                p += ng;
            }
        }
        __syncthreads();
        if (wave == 0) {
            const uint64_t excl = lookback(ws + 1, s, words, lane, kHold > 0);
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
        const uint64_t excl = lookback(ws + 1, s, words, lane);
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

// Any chunk size: the counting pass and the packing pass each read the
// chunk (the second read is served by the caches for moderate chunks).
// A workgroup's ticket t is its look-back index; it encodes chunk t + coff
// (coff > 0 when a launch of multi-chunk workgroups went first).
__global__ __launch_bounds__(kThreads) void encode_kernel_any(
    const pc_codebook *__restrict__ cb, const uint8_t *__restrict__ in, uint64_t n, uint32_t chunk,
    uint32_t num_chunks, uint32_t *__restrict__ payload, uint32_t *__restrict__ chunk_bits,
    uint64_t *__restrict__ cwo, uint32_t *__restrict__ sub_off, uint64_t *__restrict__ ws, uint32_t coff) {
    using SH = Shared<kThreads>;
    __shared__ SH sh;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sh.misc[0] = atomicAdd(reinterpret_cast<uint32_t *>(ws), 1u);
    {
        const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
        sh.code[tid] = reinterpret_cast<const uint16_t *>(cbb + kOffCode)[tid];
        sh.len[tid] = cbb[kOffLength + tid];
    }
    for (uint32_t i = tid; i < SH::kStage; i += kThreads) sh.stage[i] = 0;
    __syncthreads();
    const uint32_t t = uniform(sh.misc[0]);
    const uint32_t c = t + coff;
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
        const uint64_t excl = lookback(ws + 1, t, words, lane);
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

// Zero the ticket and the look-back descriptors; write the total-word entry
// for an empty input.
__global__ void encode_init_kernel(uint64_t *ws, uint64_t ws_words, uint64_t *cwo, int empty) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = i; k < ws_words; k += stride) ws[k] = 0;
    if (empty && i == 0) cwo[0] = 0;
}

}  // namespace

hipError_t launch_encode(const pc_codebook *cb, const uint8_t *in, uint64_t n, uint32_t chunk,
                         uint32_t *payload, uint32_t *chunk_bits, uint64_t *cwo, uint32_t *sub_off,
                         uint64_t *ws, hipStream_t stream) {
    const uint64_t nc = (n + chunk - 1) / chunk;
    const uint64_t ws_words = 1 + nc;
    const uint32_t init_blocks = (uint32_t)((ws_words + 255) / 256 < 1024 ? (ws_words + 255) / 256 : 1024);
    hipLaunchKernelGGL(encode_init_kernel, dim3(init_blocks ? init_blocks : 1), dim3(256), 0, stream, ws,
                       ws_words, cwo, n == 0 ? 1 : 0);
    if (n == 0) return hipGetLastError();
    const uint64_t nfull = n / chunk;  // chunks of exactly `chunk` symbols
    // Full chunks go to workgroups of NT tiles (TPC tiles per chunk, so
    // NT / TPC consecutive chunks and one look-back per workgroup); the
    // full chunks left over and a short last chunk go to the re-reading
    // kernel, launched after them, so their look-backs find every
    // predecessor finished.  The 1024-lane kernels hold 64K symbols per
    // workgroup; the LDS output buffer holds them at 8 bits per symbol plus
    // the padding words between chunks and the 64-bit margin of the fit
    // test (two such workgroups fit a CU).  4K and 8K symbol chunks take
    // 256-lane workgroups of 32K symbols when there are many of them, else
    // one chunk per workgroup, so that a small input still spreads over the
    // CUs (the 1-chunk buffers hold 12 bits per symbol).
    constexpr uint64_t kManySmall = 8192;
    uint64_t done = 0, tickets = 0;  // chunks and workgroups of the multi-chunk launch
#define PC_ENC(T, NT, BW, TPC)                                                                             \
    do {                                                                                                   \
        const uint64_t nsup = nfull / ((NT) / (TPC));                                                      \
        if (nsup) {                                                                                        \
            hipLaunchKernelGGL((encode_chunk_kernel<T, NT, BW, TPC>), dim3((uint32_t)nsup), dim3(T), 0,    \
                               stream, cb, in, n, chunk, (uint32_t)nc, payload, chunk_bits, cwo, sub_off,  \
                               ws);                                                                        \
            done = nsup * ((NT) / (TPC));                                                                  \
            tickets = nsup;                                                                                \
        }                                                                                               \
    } while (0)
    if (chunk == 65536) PC_ENC(1024, 4, 16392, 4);
    else if (chunk == 32768) PC_ENC(1024, 4, 16392, 2);
    else if (chunk == 16384) PC_ENC(1024, 4, 16392, 1);
    else if (chunk == 8192 && nfull >= kManySmall) PC_ENC(256, 8, 8200, 2);
    else if (chunk == 8192) PC_ENC(256, 2, 3072, 2);
    else if (chunk == 4096 && nfull >= kManySmall) PC_ENC(256, 8, 8200, 1);
    else if (chunk == 4096) PC_ENC(256, 1, 1536, 1);
    const uint64_t rest = nc - done;
    // tickets continue from the multi-chunk launch's: ticket t encodes
    // chunk t + done - tickets
    if (rest)
        hipLaunchKernelGGL(encode_kernel_any, dim3((uint32_t)rest), dim3(kThreads), 0, stream, cb, in, n, chunk,
                           (uint32_t)nc, payload, chunk_bits, cwo, sub_off, ws, (uint32_t)(done - tickets));
#undef PC_ENC
    return hipGetLastError();
}

}  // namespace pc
