// Fixed-codebook decoder for gfx950.
//
// One lane decodes one 256-symbol sub-stream; the side index gives every
// sub-stream's first bit, so lanes are independent ("Quad Length Codes for
// Lossless Compression of e4m3", abstract, blames bit-sequential tree walks
// for slow Huffman decoding; here every codeword costs one table lookup).
//
// A "group" is 256 consecutive sub-streams (one per lane of a 256-lane
// workgroup); its payload is one contiguous span of words.  Workgroups are
// persistent and walk the groups with a stride of the grid size.  While a
// workgroup decodes group k out of LDS, the loads of group k+1 (its
// container entries, then its payload span into registers, two 16-byte
// loads per lane after each of the steps 0-8 of the first 128 symbols; the
// span's entries come one group earlier still) are in flight, so HBM
// latency is hidden behind decoding.  Per group:
//   1. the staged span sits in LDS in rows of 68 words: 64 payload words plus
//      copies of the next row's first four, so any 4-word window read stays
//      in one row, rows start 16-byte aligned, and lanes whose sub-streams
//      start ~50 words apart spread over the LDS banks instead of falling on
//      a few;
//   2. per lane and per 8 symbols: fetch 4 words at the current bit, funnel
//      them into a 96-bit window (>= 96 valid bits), then 8 times: read the
//      16-bit table entry ((19 - length) | symbol << 8) of the 12 bits at the
//      current position, take the next entry's offset from the unadvanced
//      window shifted by the entry, and advance the window with funnel
//      shifts (v_alignbit) by the entry + 13;
//   3. every 128 decoded bytes of a lane go out as eight adjacent 16-byte
//      stores (whole 128-byte lines);
//   4. the sub-stream must end exactly at the next sub-stream's first bit (or
//      at chunk_bits); any mismatch sets *status = PC_ERR_CORRUPT.
// A group whose span does not fit the LDS budget, and a last group that is
// not full, are leftovers: after its staged groups, each workgroup decodes
// its share of them straight from global memory (only data that barely
// compresses produces unstaged groups).  The QLC variant replaces the 12-bit
// table with the page's own decoder: a 3-bit area number, that area's
// fixed-width index, and the 256-entry rank -> symbol table.  Its per-area
// widths and first ranks sit in registers (looked up with v_perm), so the
// decoding chain holds no memory read; only the rank -> symbol read, beside
// the chain, goes to LDS.
#include <atomic>

#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kRow = 64;     // payload words per LDS row
constexpr uint32_t kRowPad = 68;  // row + copies of the next row's first 4 words
// Staged span: up to 16512 words of payload, enough for a group at 8 bits
// per symbol (16384 words) from a row-aligned start (17 x 16 B per lane in
// flight), with two workgroups in a CU's LDS.
constexpr uint32_t kPrefetch = 17;
constexpr uint32_t kMaxStageWords = kPrefetch * 4 * kThreads;  // 17408
constexpr uint32_t kStageRows = 258;
static_assert(kStageRows * kRow <= kMaxStageWords, "prefetch covers the staged span");
constexpr uint32_t kGroupsPerCU = 2;

__device__ __forceinline__ void flag_corrupt(uint32_t *status) {
    atomicCAS(status, 0u, (uint32_t)PC_ERR_CORRUPT);
}

__device__ __forceinline__ uint32_t row_index(uint32_t a) { return a + 4 * (a >> 6); }

// Payload word sources.  Indices are clamped so that corrupt positions never
// read outside the staged words or the payload.
struct LdsWords {
    const uint32_t *w;
    uint32_t last;  // last staged word (relative)
    __device__ __forceinline__ void fetch4(uint32_t a, uint32_t (&v)[4]) const {
        a = a < last ? a : last;
        const uint32_t i = row_index(a);
        v[0] = w[i];
        v[1] = w[i + 1];
        v[2] = w[i + 2];
        v[3] = w[i + 3];
    }
};

struct GlobalWords {
    const uint32_t *w;  // payload + wbase
    uint64_t last;      // last readable index relative to w
    __device__ __forceinline__ void fetch4(uint32_t a, uint32_t (&v)[4]) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = w[(uint64_t)a + k < last ? (uint64_t)a + k : last];
    }
};

struct Tables {
    const uint16_t *lut;  // LDS: 4096 x ((19 - length) | symbol << 8), 0 = no codeword
    const uint8_t *sym;   // LDS (QLC mode): symbol of rank r for r < 256, 0 up to 1023
    // QLC mode, one byte per area a (a = 0..3 in *_lo, 4..7 in *_hi), read
    // with v_perm, so that no table on the decoding chain sits in memory:
    uint32_t sh_lo, sh_hi;  // 29 - b_a = 32 - codeword length
    uint32_t bw_lo, bw_hi;  // b_a
    uint32_t st_lo, st_hi;  // first rank of the area (0 when past 255)
    // QLC codewords read as left-aligned 32-bit numbers (area number, then
    // index) grow with the rank, so a window starts with a codeword of a
    // rank below 256 exactly when it is below the left-aligned codeword of
    // rank 256 -- when the areas have a slot for rank 256 at all
    uint32_t qlc_lim;
    bool qlc_check;
};

// Whether a sub-stream met a bit pattern that is no codeword: LUT mode ORs
// the entries' invalid flags, QLC mode keeps the largest window seen.
template <int MODE>
__device__ __forceinline__ bool saw_invalid(uint32_t bad, const Tables &t) {
    return MODE == kDecodeLut12 ? bad != 0 : (t.qlc_check && bad >= t.qlc_lim);
}

// Decode 8 symbols from the 96-bit window (h, m, l); returns them packed
// little-endian in two words and adds the bits consumed to pos.  Symbols at
// index >= lim (masked variant only) consume nothing.
//
// Entries are (19 - length) | symbol << 8 in LUT mode; QLC mode keeps
// 32 - length and the symbol in two registers.  In LUT mode the
// byte offset of the next entry is taken from the window before it is
// advanced: the 12 bits after a codeword of length len start len bits into
// h, so (h >> (19 - len)) & 0x1FFE is twice their value, and v_lshrrev reads
// exactly the 5 low bits of the entry as its count.  The window advance
// (funnel shifts by 32 - len = entry + 13 in the low 5 bits) then runs
// beside the next table read instead of before it: per symbol the chain of
// dependent instructions is one LDS read, one shift and one mask.  (The
// window has >= 96 valid bits and 7 codewords take <= 84, so the 12 bits
// after any of the first 7 are valid.)
template <int MODE, bool MASKED, bool CHECK>
__device__ __forceinline__ void decode8(uint32_t h, uint32_t m, uint32_t l, uint32_t &pos, uint32_t &bad,
                                        const Tables &t, uint32_t k0, uint32_t lim, uint32_t &o0, uint32_t &o1) {
    uint32_t e[8], y[8];  // y: the symbols (QLC mode)
    uint32_t a = (h >> (31 - kPeek)) & 0x1FFE;  // byte offset of the first entry (LUT mode)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t ek, inv, sh;  // sh: 32 - length in the 5 bits v_alignbit reads
        const bool masked = MASKED && k0 + k >= lim;  // length 0: the window is kept
        if (MODE == kDecodeLut12) {
            ek = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(t.lut) + a);
            inv = (ek & 0xFF) == 0;
            if (masked) ek = (ek & 0xFF00) | 19;
            if (k < 7) a = (h >> (ek & 31)) & 0x1FFE;
            sh = ek + 13;
        } else {
            // the area number (3 bits) selects bytes of the area registers
            // (the other selector bytes, 0x0C, give zeros; one funnel shift
            // forms the selector: (0x01818180 << 3) | (h >> 29)); the chain
            // per symbol is funnel shift, v_perm, funnel shift, with the
            // rank and the symbol read beside it (a rank past 255 reads a
            // zero of the 1 KiB table)
            const uint32_t sel = __builtin_amdgcn_alignbit(0x01818180u, h, 29);
            sh = __builtin_amdgcn_perm(t.sh_hi, t.sh_lo, sel);
            const uint32_t bw = __builtin_amdgcn_perm(t.bw_hi, t.bw_lo, sel);
            const uint32_t r = __builtin_amdgcn_perm(t.st_hi, t.st_lo, sel) + __builtin_amdgcn_ubfe(h, sh, bw);
            if (CHECK && !masked) bad = bad > h ? bad : h;
            ek = masked ? 32u : sh;
            y[k] = t.sym[r];
            inv = 0;
        }
        if (MODE == kDecodeLut12) {
            if (masked) inv = 0;
            if (CHECK) bad |= inv;
        }
        const uint32_t h2 = __builtin_amdgcn_alignbit(h, m, sh);
        const uint32_t m2 = __builtin_amdgcn_alignbit(m, l, sh);
        const uint32_t l2 = __builtin_amdgcn_alignbit(l, 0u, sh);
        if (!masked) {  // (a funnel shift by 32 would read as 0)
            h = h2;
            m = m2;
            l = l2;
        }
        e[k] = ek;
    }
    if (MODE == kDecodeLut12) {
        // each low byte is 19 - length: 4 of them sum below 256
        const uint32_t s0 = (e[0] + e[1] + e[2] + e[3]) & 0xFF, s1 = (e[4] + e[5] + e[6] + e[7]) & 0xFF;
        pos += 8 * 19 - s0 - s1;
        o0 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0501u) | __builtin_amdgcn_perm(e[3], e[2], 0x05010C0Cu);
        o1 = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0501u) | __builtin_amdgcn_perm(e[7], e[6], 0x05010C0Cu);
    } else {
        // e[k] = 32 - length (<= 32 each)
        pos += 8 * 32 - (e[0] + e[1] + e[2] + e[3]) - (e[4] + e[5] + e[6] + e[7]);
        o0 = __builtin_amdgcn_perm(y[1], y[0], 0x0C0C0400u) | __builtin_amdgcn_perm(y[3], y[2], 0x04000C0Cu);
        o1 = __builtin_amdgcn_perm(y[5], y[4], 0x0C0C0400u) | __builtin_amdgcn_perm(y[7], y[6], 0x04000C0Cu);
    }
    // pack and check here: left to the scheduler, the packing sinks towards
    // the store and the checks towards the end of the stream, and both keep
    // all eight entries of every step alive until then
    asm volatile("" : "+v"(o0), "+v"(o1));
    if (CHECK) asm volatile("" : "+v"(bad));
}

// Masked decode (the leftover groups): symbols [s_begin, s_end) of one
// sub-stream in blocks of 16; a lane writes only its bytes below lim (lanes
// past the end of the stream own none).
template <int MODE, class Src>
__device__ __forceinline__ uint32_t decode_masked(const Src &src, uint32_t pos, uint32_t lim, const Tables &t,
                                                  uint8_t *dst, uint32_t &bad, uint32_t s_begin, uint32_t s_end) {
#pragma unroll 1
    for (uint32_t base = s_begin; base < s_end; base += 16) {
        uint32_t o[4];
#pragma unroll
        for (uint32_t q = 0; q < 2; ++q) {
            uint32_t w[4];
            src.fetch4(pos >> 5, w);
            const uint32_t sh = pos & 31;
            const uint32_t h = (uint32_t)(((((uint64_t)w[0] << 32) | w[1]) << sh) >> 32);
            const uint32_t m = (uint32_t)(((((uint64_t)w[1] << 32) | w[2]) << sh) >> 32);
            const uint32_t l = (uint32_t)(((((uint64_t)w[2] << 32) | w[3]) << sh) >> 32);
            decode8<MODE, true, true>(h, m, l, pos, bad, t, base + q * 8, lim, o[2 * q], o[2 * q + 1]);
        }
        if (base + 16 <= lim) {
            *reinterpret_cast<uint4 *>(dst + base) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q)
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k)
                    if (base + 4 * q + k < lim) dst[base + 4 * q + k] = (uint8_t)(o[q] >> (8 * k));
        }
    }
    return pos;
}

// Loaded values pass through pin() where they are first needed: the empty
// asm fixes that point, so the compiler cannot hoist arithmetic on a value
// still in flight (and with it a wait for every load issued before it) to
// right after the load.  The loads themselves are unconditional, with
// clamped indices, for the same reason: a conditional load merged with a
// default value needs its result at the merge.
__device__ __forceinline__ void pin(uint32_t &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint64_t &v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ uint32_t vgpr_copy(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Half a sub-stream (128 symbols) of a lane whose 256 symbols all lie in
// [0, n), decoded into registers and then stored as one 128-byte line per
// lane (eight adjacent 16-byte stores: the L2 receives whole lines, not
// 16-byte pieces that other stores complete much later).
constexpr uint32_t kHalf = kSub / 2;
constexpr uint32_t kHalfWords = kHalf / 4;

// side(q) runs after step q (8 symbols) of the 16: the memory instructions
// of a group are spread over its decode steps, where the wave mostly waits
// for LDS results, instead of being issued in bursts that stall the waves
// of a workgroup together behind the CU's memory pipeline.
template <int MODE, bool CHECK, class Side>
__device__ __forceinline__ uint32_t decode_half(const LdsWords &src, uint32_t pos, const Tables &t, uint32_t &bad,
                                                uint32_t (&o)[kHalfWords], Side &&side) {
#pragma unroll
    for (uint32_t q = 0; q < kHalf / 8; ++q) {
        uint32_t w[4];
        src.fetch4(pos >> 5, w);
        const uint32_t sh = pos & 31;
        const uint32_t h = (uint32_t)(((((uint64_t)w[0] << 32) | w[1]) << sh) >> 32);
        const uint32_t m = (uint32_t)(((((uint64_t)w[1] << 32) | w[2]) << sh) >> 32);
        const uint32_t l = (uint32_t)(((((uint64_t)w[2] << 32) | w[3]) << sh) >> 32);
        decode8<MODE, false, CHECK>(h, m, l, pos, bad, t, 0, kHalf, o[2 * q], o[2 * q + 1]);
        side(q);
        asm volatile("" ::: "memory");  // the side work stays at this step
    }
    return pos;
}

__device__ __forceinline__ void store_half(uint8_t *dst, const uint32_t (&o)[kHalfWords]) {
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (uint32_t k = 0; k < kHalfWords / 4; ++k)
        d[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
}

// Container entries a lane depends on (loaded one group ahead).
struct LaneMeta {
    uint64_t w0, w1;      // chunk_word_offset[c], [c + 1]
    uint32_t cbits;       // chunk_bits[c]
    uint32_t start;       // sub-stream start
    uint32_t next;        // next sub-stream's start (meaningful if has_end)
    uint32_t has_end;     // 0: the sub-stream ends at chunk_bits
    uint32_t lim;         // symbols owed by this lane (0 if inactive)
    uint32_t first;       // first sub-stream of its chunk
};

__device__ __forceinline__ LaneMeta load_meta(uint64_t g, uint64_t num_sub, uint64_t n, uint32_t chunk,
                                              const uint32_t *chunk_bits, const uint64_t *cwo,
                                              const uint32_t *sub_off) {
    const bool active = g < num_sub;
    const uint32_t gc = (uint32_t)(active ? g : num_sub - 1);  // num_sub < 2^32 - 256 (checked by the entry point)
    const uint32_t spc = chunk / kSub;
    const uint32_t c = gc / spc;
    const uint32_t j = gc - c * spc;
    const uint64_t cbase = (uint64_t)c * chunk;
    const uint32_t lenc = (uint32_t)((n - cbase) < chunk ? (n - cbase) : chunk);
    const uint32_t nsub_c = (lenc + kSub - 1) / kSub;
    const uint32_t left = lenc - j * kSub;
    LaneMeta m;
    m.lim = active ? (left < kSub ? left : kSub) : 0;
    m.first = j == 0;
    m.has_end = j + 1 < nsub_c;
    m.w0 = cwo[c];
    m.w1 = cwo[c + 1];
    m.cbits = chunk_bits[c];
    m.start = sub_off[gc];
    m.next = sub_off[vgpr_copy(m.has_end ? gc + 1 : gc)];
    return m;
}

// Words [lo, hi) of the payload a group needs: from the first sub-stream's
// start to the next group's first sub-stream (or the end of the payload).
// Every lane loads the same four entries with vector loads (scalar loads
// would share a wait counter with the LDS reads of the decode loop), and
// every lane later checks its own range against the span.
struct SpanEntries {
    uint64_t w_first, w_next;
    uint32_t off_first, off_next;  // off_next: meaningful if has_next
    uint32_t has_next;
};

__device__ __forceinline__ SpanEntries load_span(uint64_t grp, uint64_t num_sub, uint32_t chunk, uint64_t num_chunks,
                                                 const uint64_t *cwo, const uint32_t *sub_off) {
    const uint32_t spc = chunk / kSub;
    const uint32_t g0 = vgpr_copy((uint32_t)(grp * kThreads));
    const uint32_t g1 = g0 + kThreads;
    SpanEntries e;
    e.has_next = g1 < num_sub;
    e.w_first = cwo[g0 / spc];
    e.off_first = sub_off[g0];
    // opaque indices: a load the compiler could merge with the one above
    // would come back as a conditional load plus a copy that waits for it
    e.w_next = cwo[vgpr_copy(e.has_next ? g1 / spc : (uint32_t)num_chunks)];
    e.off_next = sub_off[vgpr_copy(e.has_next ? g1 : g0)];
    return e;
}

// Bit addresses of the span's ends (the first use of the loaded entries).
__device__ __forceinline__ void span_bits(SpanEntries e, uint64_t &a, uint64_t &b) {
    pin(e.w_first);
    pin(e.w_next);
    pin(e.off_first);
    pin(e.off_next);
    a = e.w_first * 32 + e.off_first;
    b = e.w_next * 32 + (e.has_next ? e.off_next : 0u);
}

// Per-lane form (each lane may hold a different group's entries).
__device__ __forceinline__ void span_words_lane(const SpanEntries &e, uint64_t payload_words, uint64_t &lo,
                                                uint64_t &hi) {
    uint64_t a, b;
    span_bits(e, a, b);
    lo = a >> 5;
    hi = (b + 31) >> 5;
    if (lo > payload_words) lo = payload_words;
    if (hi > payload_words) hi = payload_words;
    if (hi < lo) hi = lo;
}

__device__ __forceinline__ void span_words(const SpanEntries &e, uint64_t payload_words, uint64_t &lo, uint64_t &hi) {
    uint64_t a, b;
    span_bits(e, a, b);
    lo = uniform64(a >> 5);
    hi = uniform64((b + 31) >> 5);
    if (lo > payload_words) lo = payload_words;
    if (hi > payload_words) hi = payload_words;
    if (hi < lo) hi = lo;
}

// Prefetch of a staged span into registers: one 16-byte load per quad of
// words, unconditional and branch-free (control flow here would make the
// compiler's wait counting conservative for the whole loop).  Quad indices
// are clamped to the payload's last whole quad (the kernel runs only when
// there is one); quads past it, or of a span too large to stage, are never
// staged.  The up to 3 words after the last whole quad are read while
// staging, by the one lane that needs them.  Nothing is read at or past
// payload_words.
struct Prefetch {
    uint4 q[kPrefetch];
};

// The payload as the prefetch sees it: a global pointer passed through an
// empty asm, so that the compiler no longer knows that nothing writes the
// words and keeps each load at the decode step it is issued at (loads of
// memory known to be read-only are moved freely, and end up together).
typedef const __attribute__((address_space(1))) u32x4 gquad;

__device__ __forceinline__ gquad *opaque_quads(const uint32_t *payload) {
    gquad *p = (gquad *)payload;
    asm volatile("" : "+s"(p));
    return p;
}

// Quad k of lane tid of the span [lo, hi): quads past the span's last one
// (or the payload's last whole one) read that quad again, so lanes with no
// quad of their own add no traffic.
__device__ __forceinline__ uint64_t last_quad(uint64_t lo, uint64_t hi, uint64_t payload_words) {
    const uint64_t q0 = (lo & ~(uint64_t)(kRow - 1)) / 4;
    uint64_t qe = (hi + 3) / 4;  // one past the span's last quad
    if (qe <= q0) qe = q0 + 1;
    if (qe > payload_words / 4) qe = payload_words / 4;
    return qe - 1;
}

__device__ __forceinline__ void prefetch_quad(Prefetch &pf, uint32_t k, gquad *payload, uint64_t lo,
                                              uint64_t q_last, uint32_t tid) {
    const uint64_t q = (lo & ~(uint64_t)(kRow - 1)) / 4 + tid + k * kThreads;
    const u32x4 v = __builtin_nontemporal_load(payload + (q < q_last ? q : q_last));
    pf.q[k] = make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void issue_prefetch(Prefetch &pf, gquad *payload, uint64_t lo, uint64_t q_last,
                                               uint32_t tid) {
#pragma unroll
    for (uint32_t k = 0; k < kPrefetch; ++k) prefetch_quad(pf, k, payload, lo, q_last, tid);
}

// Tables into LDS (shared by both kernels).
template <int MODE>
__device__ __forceinline__ void load_tables(const uint8_t *cbb, uint4 *tab4, uint32_t tid) {
    if (MODE == kDecodeLut12) {
        // 16-bit entries (19 - length) | symbol << 8 (0: no codeword)
        const uint8_t *ds = cbb + kOffDecSym, *dl = cbb + kOffDecSym + 4096;
        uint16_t *lut = reinterpret_cast<uint16_t *>(tab4);
        for (uint32_t i = tid; i < 4096; i += kThreads) {
            const uint32_t len = dl[i];
            lut[i] = (uint16_t)(len ? ((19 - len) | ((uint32_t)ds[i] << 8)) : 0u);
        }
    } else {
        // symbol of rank r, then zeros up to rank 1023 (a rank is below
        // 255 + 2^9 for any layout; ranks past 255 are no codeword)
        for (uint32_t i = tid; i < 256; i += kThreads)
            reinterpret_cast<uint32_t *>(tab4)[i] =
                i < 64 ? reinterpret_cast<const uint32_t *>(cbb + kOffSymOfRank)[i] : 0u;
    }
}

// The QLC area registers (see Tables), from the blob's widths and starts.
__device__ __forceinline__ void qlc_area_regs(const uint8_t *cbb, Tables &t) {
    uint32_t sh[2] = {0, 0}, bw[2] = {0, 0}, st[2] = {0, 0};
    t.qlc_lim = 0;
    t.qlc_check = false;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        uint32_t b = cbb[kOffQlcBits + a];
        b = b > PC_MAX_LEN - 3 ? PC_MAX_LEN - 3 : b;  // a valid blob has b <= 9
        const uint32_t start = reinterpret_cast<const uint16_t *>(cbb + kOffQlcStart)[a];
        const uint32_t j = a >> 2, sft = 8 * (a & 3);
        sh[j] |= (29 - b) << sft;
        bw[j] |= b << sft;
        st[j] |= (start > 255 ? 0u : start) << sft;
        if (!t.qlc_check && start <= 256 && start + (1u << b) > 256) {  // the area of rank 256
            t.qlc_lim = ((uint32_t)a << 29) | ((256 - start) << (29 - b));
            t.qlc_check = true;
        }
    }
    t.sh_lo = sh[0];
    t.sh_hi = sh[1];
    t.bw_lo = bw[0];
    t.bw_hi = bw[1];
    t.st_lo = st[0];
    t.st_hi = st[1];
}

__device__ __forceinline__ bool span_staged(uint64_t lo, uint64_t hi, uint64_t payload_words, uint32_t stage_cap) {
    const uint64_t wb = lo & ~(uint64_t)(kRow - 1);
    return hi - wb <= stage_cap && payload_words > wb;
}

// Per-lane checks of a sub-stream against its group's span [wbase, hi).
struct LaneJob {
    bool ok;
    uint32_t lim, pos0, pos_want;
};

__device__ __forceinline__ LaneJob lane_job(LaneMeta m, bool kind_ok, uint64_t payload_words, uint64_t wbase,
                                            uint64_t hi, uint32_t *status) {
    pin(m.w0);
    pin(m.w1);
    pin(m.cbits);
    pin(m.start);
    pin(m.next);
    const uint32_t end = m.has_end ? m.next : m.cbits;
    const uint64_t abs_s = m.w0 * 32 + m.start, abs_e = m.w0 * 32 + end;
    const bool active = m.lim > 0;
    LaneJob j;
    j.ok = active && kind_ok && m.w1 >= m.w0 && (m.w1 - m.w0) == ((uint64_t)m.cbits + 31) / 32 &&
           m.w1 <= payload_words && (!m.first || m.start == 0) && m.start <= end && end <= m.cbits &&
           abs_s >= wbase * 32 && abs_e <= hi * 32 && hi - wbase < (1u << 26);
    if (active && !j.ok) flag_corrupt(status);
    j.lim = j.ok ? m.lim : 0;
    j.pos0 = j.ok ? (uint32_t)(abs_s - wbase * 32) : 0;
    j.pos_want = j.ok ? (uint32_t)(abs_e - wbase * 32) : 0;
    return j;
}

// The group loop of a workgroup (CHECK: test every table entry for "no
// codeword", needed only when the code is incomplete).  Every lane decodes
// on every pass; a group whose span is not staged decodes stale rows and
// stores nothing (it is decoded later as a leftover).
template <int MODE, bool CHECK>
__device__ __forceinline__ void decode_groups(uint64_t grp, uint32_t tid0, const Tables &t, bool kind_ok,
                                              uint32_t *stage, uint4 *stage4, const uint32_t *payload,
                                              uint64_t payload_words, const uint32_t *chunk_bits,
                                              const uint64_t *cwo, const uint32_t *sub_off, uint64_t n,
                                              uint32_t chunk, uint64_t num_sub, uint64_t num_full,
                                              uint64_t num_chunks, uint8_t *out, uint32_t *status,
                                              uint32_t stage_cap) {
    gquad *pq = opaque_quads(payload);
    // ---- prologue: loads of the first group --------------------------
    LaneMeta meta = load_meta(grp * kThreads + tid0, num_sub, n, chunk, chunk_bits, cwo, sub_off);
    uint64_t lo, hi;
    span_words(load_span(grp, num_sub, chunk, num_chunks, cwo, sub_off), payload_words, lo, hi);
    Prefetch pf;
    issue_prefetch(pf, pq, lo, last_quad(lo, hi, payload_words), tid0);
    // the next group's span entries, one group ahead
    SpanEntries nspan = load_span(grp + gridDim.x < num_full ? grp + gridDim.x : grp, num_sub, chunk, num_chunks,
                                  cwo, sub_off);
    uint32_t o1[kHalfWords], o2[kHalfWords];

    for (;;) {
        // the lane index as an opaque value: computations from it are not
        // hoisted out of the loop to hold dozens of registers across it
        const uint32_t tid = vgpr_copy(tid0);
        const uint64_t wbase = lo & ~(uint64_t)(kRow - 1);
        const uint64_t cnt = hi - wbase;
        const bool staged = span_staged(lo, hi, payload_words, stage_cap);
        // ---- stage the current group (its loads were issued earlier) --
        __syncthreads();  // every lane is done with the previous group's rows
        // wait for the whole prefetch here, on every path (waits left to the
        // compiler would sit in the branches below, and every later write
        // of these registers would wait again, for whatever is in flight)
#pragma unroll
        for (uint32_t k = 0; k < kPrefetch; ++k) {
            pin(pf.q[k].x);
            pin(pf.q[k].y);
            pin(pf.q[k].z);
            pin(pf.q[k].w);
        }
        if (staged) {
            const uint32_t nq = (uint32_t)((cnt + 3) / 4);
            const uint64_t full_q = (payload_words - wbase) / 4;
#pragma unroll
            for (uint32_t k = 0; k < kPrefetch; ++k) {
                const uint32_t q = tid + k * kThreads;
                if (q < nq && q < full_q) {
                    const uint32_t i = row_index(4 * q);  // a multiple of 4
                    stage4[i / 4] = pf.q[k];
                    if ((q & 15) == 0 && q) stage4[i / 4 - 1] = pf.q[k];  // copies ending the previous row
                }
            }
            if (nq > full_q && tid == (uint32_t)full_q % kThreads) {
                // the span reaches the payload's last quad, which may be
                // partial: its words are read one by one
                uint32_t v[4];
#pragma unroll
                for (uint32_t w = 0; w < 4; ++w) {
                    const uint64_t i = wbase + 4 * full_q + w;
                    v[w] = i < payload_words ? payload[i] : 0u;
                }
                const uint32_t i = row_index(4 * (uint32_t)full_q);
                const uint4 qv = make_uint4(v[0], v[1], v[2], v[3]);
                stage4[i / 4] = qv;
                if ((full_q & 15) == 0 && full_q) stage4[i / 4 - 1] = qv;
            }
        }
        __syncthreads();

        // ---- the next group's entries and payload ----------------------
        // Loads and prefetch are issued on every pass (for the last, of this
        // group's own entries and span again): control flow around them
        // makes the compiler's wait counting conservative, and it then waits
        // for the prefetch right after issuing it.
        const uint64_t nxt = grp + gridDim.x;
        const bool more = nxt < num_full;
        const uint64_t nxt_c = more ? nxt : grp;
        const LaneMeta nmeta = load_meta(nxt_c * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
        const uint64_t nn = nxt + gridDim.x;
        const SpanEntries nspan2 = load_span(nn < num_full ? nn : nxt_c, num_sub, chunk, num_chunks, cwo, sub_off);
        uint64_t nlo = 0, nhi = 0, nq_lo = 0, nq_last = 0;
        span_words(nspan, payload_words, nlo, nhi);
        nq_last = more ? last_quad(nlo, nhi, payload_words) : 0;
        nq_lo = more ? nlo : 0;
        const LaneJob job = lane_job(meta, kind_ok, payload_words, wbase, hi, status);
        uint8_t *dst = out + (grp * kThreads + tid) * kSub;
        const LdsWords src{stage, (uint32_t)((cnt < stage_cap ? cnt : stage_cap) - (cnt > 0 ? 1 : 0))};
        uint32_t bad = 0;
        // first half: the next group's payload loads, two per step from step
        // 0 (its span entries were loaded one group ahead)
        uint32_t pos = decode_half<MODE, CHECK>(src, job.pos0, t, bad, o1, [&](uint32_t q) {
            if (2 * q < kPrefetch) prefetch_quad(pf, 2 * q, pq, nq_lo, nq_last, tid);
            if (2 * q + 1 < kPrefetch) prefetch_quad(pf, 2 * q + 1, pq, nq_lo, nq_last, tid);
        });
        // second half: the first half's 128 bytes, 16 per step
        if (staged) store_half(dst, o1);
        pos = decode_half<MODE, CHECK>(src, pos, t, bad, o2, [&](uint32_t q) {});
        if (staged) {
            if (job.ok && (saw_invalid<MODE>(bad, t) || pos != job.pos_want)) flag_corrupt(status);
            store_half(dst + kHalf, o2);
        }

        if (!more) break;
        grp = nxt;
        meta = nmeta;
        lo = nlo;
        hi = nhi;
        nspan = nspan2;
    }
}

// The groups the main kernel leaves: those whose span exceeds the LDS
// budget (the same span test picks them) and the last group when it is not
// full.  Each lane reads its words straight from global memory and writes
// only bytes below its symbol count.  Workgroup b owns the groups b, b + G,
// b + 2G, ... (G workgroups); its first wave tests 64 of them at once (one
// per lane), then the workgroup decodes the ones that were not staged, so
// that a stream with no such group costs one round of entry loads, and a
// stream of such groups is spread over all workgroups.
constexpr uint32_t kTestBatch = 64;

struct Leftovers {
    uint32_t todo[kTestBatch];
    uint32_t ntodo;
};

// Test the batch of groups base + l G, l = 0 .. 63: the ones for the
// global-memory path go to lo.todo; returns their number (uniform).
__device__ __forceinline__ uint32_t test_batch(Leftovers &lo_, uint64_t base, uint64_t G, uint64_t num_groups,
                                               uint64_t num_full, uint64_t num_sub, uint32_t chunk,
                                               uint64_t num_chunks, const uint64_t *cwo, const uint32_t *sub_off,
                                               uint64_t payload_words, uint32_t stage_cap, uint32_t tid) {
    if (tid == 0) lo_.ntodo = 0;
    __syncthreads();
    if (tid < kTestBatch && base + tid * G < num_groups) {
        const uint64_t g = base + tid * G;
        uint64_t lo, hi;
        span_words_lane(load_span(g, num_sub, chunk, num_chunks, cwo, sub_off), payload_words, lo, hi);
        if (g >= num_full || !span_staged(lo, hi, payload_words, stage_cap)) lo_.todo[atomicAdd(&lo_.ntodo, 1u)] = tid;
    }
    __syncthreads();
    return uniform(lo_.ntodo);
}

// Decode the nt groups a test_batch of `base` listed (tables in LDS).
template <int MODE>
__device__ __forceinline__ void decode_batch(const Leftovers &lo_, uint32_t nt, uint64_t base, uint64_t G,
                                             const Tables &t, bool kind_ok, const uint32_t *payload,
                                             uint64_t payload_words, const uint32_t *chunk_bits,
                                             const uint64_t *cwo, const uint32_t *sub_off, uint64_t n,
                                             uint32_t chunk, uint64_t num_sub, uint64_t num_chunks, uint8_t *out,
                                             uint32_t *status, uint32_t tid) {
    for (uint32_t i = 0; i < nt; ++i) {
        const uint64_t grp = base + lo_.todo[i] * G;
        uint64_t lo, hi;
        span_words(load_span(grp, num_sub, chunk, num_chunks, cwo, sub_off), payload_words, lo, hi);
        const uint64_t wbase = lo & ~(uint64_t)(kRow - 1);
        const LaneMeta meta = load_meta(grp * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
        const LaneJob job = lane_job(meta, kind_ok, payload_words, wbase, hi, status);
        if (payload_words <= wbase) continue;  // nothing readable: every lane was flagged
        uint8_t *dst = out + (grp * kThreads + tid) * kSub;
        GlobalWords src{payload + wbase, payload_words - wbase - 1};
        uint32_t bad = 0;
        const uint32_t pos_end = decode_masked<MODE>(src, job.pos0, job.lim, t, dst, bad, 0, kSub);
        if (job.ok && (saw_invalid<MODE>(bad, t) || pos_end != job.pos_want)) flag_corrupt(status);
    }
}

// Main kernel: the full groups (all 256 sub-streams of 256 symbols inside
// [0, n)) whose span fits the staging rows, so no lane needs masking, then
// the workgroup's leftover groups.  Each
// half's 128 bytes per lane are stored as soon as they are decoded.  Lanes
// of a corrupt sub-stream decode from the start of the staged span (LDS
// reads are clamped) and write unspecified bytes into their own 256-byte
// range.
template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const pc_codebook *__restrict__ cb, const uint32_t *__restrict__ payload, uint64_t payload_words,
    const uint32_t *__restrict__ chunk_bits, const uint64_t *__restrict__ cwo,
    const uint32_t *__restrict__ sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub, uint64_t num_full,
    uint64_t num_chunks, uint64_t num_groups, uint8_t *__restrict__ out, uint32_t *__restrict__ status,
    uint32_t stage_cap) {
    // Tables at fixed LDS addresses (folded into the instructions' offset
    // fields); the payload staging rows are the dynamic part.
    __shared__ uint4 tab4[MODE == kDecodeLut12 ? 512 : 64];
    __shared__ Leftovers left;
    extern __shared__ uint4 stage4[];
    uint32_t *stage = reinterpret_cast<uint32_t *>(stage4);
    const uint32_t tid = threadIdx.x;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
    const pc_codebook *cbp = reinterpret_cast<const pc_codebook *>(cb);
    load_tables<MODE>(cbb, tab4, tid);
    const bool kind_ok = MODE == kDecodeLut12 || cbp->kind == PC_CODEBOOK_QLC;
    Tables t;
    t.lut = reinterpret_cast<const uint16_t *>(tab4);
    t.sym = reinterpret_cast<const uint8_t *>(tab4);
    if (MODE == kDecodeQlc) qlc_area_regs(cbb, t);

    // this workgroup's first batch of leftover groups (see below), tested
    // while the tables arrive; decoded after the staged groups
    const uint64_t G = gridDim.x;
    const uint32_t nt0 = test_batch(left, blockIdx.x, G, num_groups, num_full, num_sub, chunk, num_chunks, cwo,
                                    sub_off, payload_words, stage_cap, tid);
    const uint64_t grp = blockIdx.x;
    if (grp < num_full) {
        if (cbp->complete == 1)
            decode_groups<MODE, false>(grp, tid, t, kind_ok, stage, stage4, payload, payload_words, chunk_bits, cwo,
                                       sub_off, n, chunk, num_sub, num_full, num_chunks, out, status, stage_cap);
        else
            decode_groups<MODE, true>(grp, tid, t, kind_ok, stage, stage4, payload, payload_words, chunk_bits, cwo,
                                      sub_off, n, chunk, num_sub, num_full, num_chunks, out, status, stage_cap);
    }
    __syncthreads();  // the tables are in LDS
    decode_batch<MODE>(left, nt0, blockIdx.x, G, t, kind_ok, payload, payload_words, chunk_bits, cwo, sub_off, n,
                       chunk, num_sub, num_chunks, out, status, tid);
    for (uint64_t base = blockIdx.x + G * kTestBatch; base < num_groups; base += G * kTestBatch) {
        __syncthreads();  // the previous batch's list is read
        const uint32_t nt = test_batch(left, base, G, num_groups, num_full, num_sub, chunk, num_chunks, cwo, sub_off,
                                       payload_words, stage_cap, tid);
        decode_batch<MODE>(left, nt, base, G, t, kind_ok, payload, payload_words, chunk_bits, cwo, sub_off, n, chunk,
                           num_sub, num_chunks, out, status, tid);
    }
}

// Leftover groups alone, for inputs without a full group (no main kernel).
template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_global_kernel(
    const pc_codebook *__restrict__ cb, const uint32_t *__restrict__ payload, uint64_t payload_words,
    const uint32_t *__restrict__ chunk_bits, const uint64_t *__restrict__ cwo,
    const uint32_t *__restrict__ sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub, uint64_t num_groups,
    uint64_t num_full, uint64_t num_chunks, uint8_t *__restrict__ out, uint32_t *__restrict__ status,
    uint32_t stage_cap) {
    __shared__ uint4 tab4[MODE == kDecodeLut12 ? 512 : 64];
    __shared__ Leftovers left;
    const uint32_t tid = threadIdx.x;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
    const pc_codebook *cbp = reinterpret_cast<const pc_codebook *>(cb);
    bool loaded = false;
    const bool kind_ok = MODE == kDecodeLut12 || cbp->kind == PC_CODEBOOK_QLC;
    Tables t;
    t.lut = reinterpret_cast<const uint16_t *>(tab4);
    t.sym = reinterpret_cast<const uint8_t *>(tab4);
    if (MODE == kDecodeQlc) qlc_area_regs(cbb, t);
    const uint64_t G = gridDim.x;
    for (uint64_t base = blockIdx.x; base < num_groups; base += G * kTestBatch) {
        const uint32_t nt = test_batch(left, base, G, num_groups, num_full, num_sub, chunk, num_chunks, cwo, sub_off,
                                       payload_words, stage_cap, tid);
        if (nt && !loaded) {
            load_tables<MODE>(cbb, tab4, tid);
            __syncthreads();
            loaded = true;
        }
        decode_batch<MODE>(left, nt, base, G, t, kind_ok, payload, payload_words, chunk_bits, cwo, sub_off, n, chunk,
                           num_sub, num_chunks, out, status, tid);
        __syncthreads();  // the list is rewritten by the next batch
    }
}

}  // namespace

hipError_t launch_decode(int mode, const pc_codebook *cb, const uint32_t *payload, uint64_t payload_words,
                         const uint32_t *chunk_bits, const uint64_t *cwo, const uint32_t *sub_off,
                         uint64_t n, uint32_t chunk, uint8_t *out, uint32_t *status, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint64_t nc = (n + chunk - 1) / chunk;
    const uint64_t last = n - (nc - 1) * chunk;
    const uint64_t num_sub = (nc - 1) * (chunk / kSub) + (last + kSub - 1) / kSub;
    const uint64_t num_groups = (num_sub + kThreads - 1) / kThreads;
    // LDS budget for a staged span: two workgroups share a CU's 160 KiB:
    // 258 rows of 68 words beside the 8 KiB table, i.e. up to 16512 payload
    // words (8 bits per symbol from a row-aligned start).
    const uint64_t cap = kStageRows * kRow;
    const size_t shmem = kStageRows * kRowPad * 4;
    // Per device (the current one), set once: its CU count, and the
    // dynamic-LDS limit of the main kernels.  Concurrent first calls may
    // both query and set; they store the same values.
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus_of[kMaxDevices];
    static std::atomic<bool> attr_of[kMaxDevices][2];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int num_cus = cus_of[dev].load(std::memory_order_relaxed);
    if (!num_cus) {
        e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus_of[dev].store(num_cus, std::memory_order_relaxed);
    }
    const void *fn = mode == kDecodeLut12 ? (const void *)decode_kernel<kDecodeLut12>
                                          : (const void *)decode_kernel<kDecodeQlc>;
    if (!attr_of[dev][mode].load(std::memory_order_relaxed)) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kStageRows * kRowPad * 4);
        if (e != hipSuccess) return e;
        attr_of[dev][mode].store(true, std::memory_order_relaxed);
    }
    // groups whose 256 sub-streams all hold 256 symbols inside [0, n)
    // (the main kernel's prefetch needs one whole 16-byte quad of payload)
    const uint64_t num_full = payload_words >= 4 ? n / ((uint64_t)kThreads * kSub) : 0;
    uint64_t grid = (uint64_t)num_cus * kGroupsPerCU;
    if (grid > num_full) grid = num_full;
    uint64_t grid_g = (uint64_t)num_cus * kGroupsPerCU;
    if (grid_g > num_groups) grid_g = num_groups;
    if (num_sub >= kMaxDecodeSubstreams) return hipErrorInvalidValue;  // the entry point checks first
#define PC_DEC(K)                                                                                             \
    hipLaunchKernelGGL(K, dim3((uint32_t)grid), dim3(kThreads), shmem, stream, cb, payload, payload_words,     \
                       chunk_bits, cwo, sub_off, n, chunk, num_sub, num_full, nc, num_groups, out, status,    \
                       (uint32_t)cap)
#define PC_DEC_G(K)                                                                                           \
    hipLaunchKernelGGL(K, dim3((uint32_t)grid_g), dim3(kThreads), 0, stream, cb, payload, payload_words,       \
                       chunk_bits, cwo, sub_off, n, chunk, num_sub, num_groups, num_full, nc, out, status,    \
                       (uint32_t)cap)
    // with a full group the main kernel also takes the leftover groups;
    // without one, only the leftover kernel runs
    if (mode == kDecodeLut12) {
        if (grid) PC_DEC(decode_kernel<kDecodeLut12>);
        else PC_DEC_G(decode_global_kernel<kDecodeLut12>);
    } else {
        if (grid) PC_DEC(decode_kernel<kDecodeQlc>);
        else PC_DEC_G(decode_global_kernel<kDecodeQlc>);
    }
#undef PC_DEC
#undef PC_DEC_G
    return hipGetLastError();
}

}  // namespace pc
