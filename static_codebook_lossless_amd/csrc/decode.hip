// Fixed-codebook decoder for gfx950.
//
// One lane decodes one 256-symbol sub-stream; the side index gives every
// sub-stream's first bit, so lanes are independent ("Quad Length Codes for
// Lossless Compression of e4m3", abstract, blames bit-sequential tree walks
// for slow Huffman decoding; here every codeword costs one table lookup).
//
// A "group" is 256 consecutive sub-streams, one per lane of a 256-lane
// workgroup; three workgroups share a CU.  Workgroups are persistent and walk
// the groups with a stride of the grid size.  A group is decoded in two
// halves of 128 symbols per lane, each out of an LDS segment of 40 words per
// lane: the first half from the 40 words that start at the word holding the
// sub-stream's first bit, the second from the 40 words that end at the word
// holding its last bit.  Both start words are known from the side index
// before the group is decoded, so each half's segments are loaded (one
// 16-byte load per lane and decode step, consecutive lanes reading
// consecutive quads of a segment) while the previous half decodes, and HBM
// latency stays hidden.  A half fits its segment up to ~9.8 bits per
// symbol; a group where some half does not is decoded again from global
// memory (decode_group_global).  Per half and lane:
//   1. per 8 symbols: fetch 4 words around the current bit, funnel them into
//      a 96-bit window (>= 96 valid bits), then 8 times: read the 16-bit
//      table entry ((19 - length) | symbol << 8) of the 12 bits at the
//      current position, take the next entry's offset from the unadvanced
//      window shifted by the entry, and advance the window with funnel
//      shifts (v_alignbit) by the entry + 13 (lut16_step8, lut16_step8_fast);
//   2. once the group is decoded, its output goes out through the segment
//      area, half a sub-stream at a time, so that every store instruction
//      writes whole 128-byte lines (store_group);
//   3. the sub-stream must end exactly at the next sub-stream's first bit (or
//      at chunk_bits); any mismatch sets *status = PC_ERR_CORRUPT.
// A last group that is not full is a leftover: after its full groups, each
// workgroup decodes its share of them straight from global memory.  The QLC
// variant replaces the 12-bit table with the decoder of "Quad Length Codes
// for Lossless Compression of e4m3" (abstract): a 3-bit area number, that
// area's fixed-width index, and the 256-entry rank -> symbol table.  Its
// per-area widths and first ranks sit in registers (looked up with v_perm),
// so the decoding chain holds no memory read; only the rank -> symbol read,
// beside the chain, goes to LDS.
#include <atomic>

#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
// Each sub-stream is staged in two segments of kSlotData words, one for its
// first 128 symbols and one for its last 128.  Segment j of a group sits at
// word 41 j of the segment area, so lanes reading the same word of their own
// segments hit 32 different LDS banks.
constexpr uint32_t kSlotWords = 41;            // segment stride in LDS (odd: 32 banks)
constexpr uint32_t kSlotData = kSlotWords - 1;  // words staged per segment: whole 16-byte quads
constexpr uint32_t kSlotBits = kSlotData * 32;
constexpr uint32_t kSegQuads = kSlotData / 4;  // 16-byte loads per segment, by consecutive lanes
constexpr uint32_t kSetLoads = kSegQuads;
static_assert(kSlotData % 4 == 0 && kSlotWords % 2 == 1, "whole quads, odd stride");
constexpr uint32_t kLutBytes = 8192;
constexpr uint32_t kLutOff = 19;  // entry = (19 - length) | symbol << 8
constexpr uint32_t kLutMask = 0x1FFE;
constexpr uint32_t kGroupsPerCU = 3;
// inputs from this size on decode with streaming (non-temporal) second-half
// segment loads and output stores (see seg_fetch)
constexpr uint64_t kStreamBytes = 256ull << 20;
// LDS layout (bytes): the table, the two segment-start tables (this group's
// second halves, the next group's first halves), the leftover list and the
// group-failure flag, then the slots (16-byte aligned: the output transpose
// reuses them) and 4 spare words for window reads past the last slot.
constexpr uint32_t kOffStartsA = kLutBytes;
constexpr uint32_t kOffStartsB = kOffStartsA + 4 * kThreads;
constexpr uint32_t kOffLeft = kOffStartsB + 4 * kThreads;
constexpr uint32_t kOffFlag = kOffLeft + 264;
constexpr uint32_t kOffSlots = kOffLeft + 272;
constexpr uint32_t kLdsBytes = kOffSlots + (kThreads * kSlotWords + 4) * 4;
static_assert(kOffSlots % 16 == 0, "slots hold 16-byte quads for the output transpose");
// each wave's output transpose (8 KiB) fits inside its own lanes' slots
constexpr uint32_t kWaveSlotQuads = 64 * kSlotWords / 4;
static_assert(64 * kSlotWords % 4 == 0 && kWaveSlotQuads * 16 >= 8192, "the output transpose fits a wave's slots");
// three workgroups per CU, with room for an LDS allocation granularity of
// 512 or 1280 bytes
static_assert(3 * ((kLdsBytes + 1279) / 1280 * 1280) <= 160 * 1024, "three workgroups per CU");

// First error wins.  The plain read first keeps a corrupt stream, where
// every lane may report, from serialising millions of atomics on one word.
__device__ __forceinline__ void flag_corrupt(uint32_t *status) {
    if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        atomicCAS(status, 0u, (uint32_t)PC_ERR_CORRUPT);
}

// Payload word sources.  Indices are clamped so that corrupt positions never
// read outside the staged words or the payload.  fetch4 reads words a .. a+3;
// fetch4m reads words q-1 .. q+2 (the window of the table decoder, see
// lut16_step8; word -1 of a segment is the LDS word before it, read but
// never used, as are words past the segment).
struct LdsWords {
    const uint32_t *w;
    uint32_t last;  // last staged word (relative)
    __device__ __forceinline__ void fetch4(uint32_t a, uint32_t (&v)[4]) const {
        a = a < last ? a : last;
        v[0] = w[a];
        v[1] = w[a + 1];
        v[2] = w[a + 2];
        v[3] = w[a + 3];
    }
    __device__ __forceinline__ void fetch4m(uint32_t q, uint32_t (&v)[4]) const {
        // q = last + 1 is a lane whose remaining bits all lie in the last
        // word (read as word q - 1); the next segment, or the spare words
        // after the last one, keep the reads of q .. q + 2 inside the
        // allocation
        q = min(q, last + 1);
        const uint32_t *p = w + q - 1;
        v[0] = p[0];
        v[1] = p[1];
        v[2] = p[2];
        v[3] = p[3];
    }
};

struct GlobalWords {
    const uint32_t *w;  // payload + wbase
    uint64_t last;      // last readable index relative to w
    __device__ __forceinline__ void fetch4(uint32_t a, uint32_t (&v)[4]) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = w[(uint64_t)a + k < last ? (uint64_t)a + k : last];
    }
    __device__ __forceinline__ void fetch4m(uint32_t q, uint32_t (&v)[4]) const {
        const uint64_t a = (uint64_t)q - 1;  // wraps for q = 0: clamped, and then unused
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = w[a + k < last ? a + k : last];
    }
};

struct Tables {
    const uint32_t *lut;  // LDS: 4096 x u16 ((19 - length) | symbol << 8), 0 = no codeword
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

// Whether a sub-stream met a bit pattern that is no codeword: LUT mode keeps
// the least table entry read (a codeword's entry is at least 7, "no
// codeword" is 0), QLC mode the largest window seen.
template <int MODE>
__device__ __forceinline__ uint32_t no_invalid_yet() { return MODE == kDecodeLut12 ? ~0u : 0u; }

template <int MODE>
__device__ __forceinline__ bool saw_invalid(uint32_t bad, const Tables &t) {
    return MODE == kDecodeLut12 ? bad == 0 : (t.qlc_check && bad >= t.qlc_lim);
}

// Table decoder with one 16-bit entry per 12-bit peek: (19 - length) in the
// low 5 bits (0 = no codeword), the symbol in byte 1.  The next entry's byte
// offset comes from the window before it is advanced: the 12 bits after a
// codeword of length len start len bits into h, so (h >> (19 - len)) &
// 0x1FFE is twice their value; the window's funnel shifts (by 32 - len =
// entry + 13 in the low 5 bits) run beside the next table read.  Per symbol
// the chain of dependent instructions is one LDS read, one shift and one
// mask.  The 8 KiB table leaves room for three workgroups' segments per CU.
// The bit position is kept negated (npos =
// -pos, mod 2^32): the window is the 96 bits from pos, funnelled from the
// words q-1 .. q+2 with q = (pos + 31) / 32 by v_alignbit with shift npos (its
// low 5 bits are (32 - pos % 32) % 32; pos % 32 == 0 shifts by 0 and takes
// word q itself).  (96 valid bits, and 7 codewords take <= 84, so the 12
// bits after any of the first 7 are valid.)  Symbols at index >= lim (masked
// variant only) consume nothing.  Returns the 8 symbols packed little-endian
// in o0, o1.
template <bool MASKED, bool CHECK, class Src>
__device__ __forceinline__ void lut16_step8(const Src &src, uint32_t &npos, uint32_t &bad, const uint32_t *lut,
                                            uint32_t k0, uint32_t lim, uint32_t &o0, uint32_t &o1) {
    uint32_t w[4];
    src.fetch4m((31u - npos) >> 5, w);
    uint32_t h = __builtin_amdgcn_alignbit(w[0], w[1], npos);
    uint32_t m = __builtin_amdgcn_alignbit(w[1], w[2], npos);
    uint32_t l = __builtin_amdgcn_alignbit(w[2], w[3], npos);
    uint32_t a = (h >> kLutOff) & kLutMask;
    uint32_t e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool masked = MASKED && k0 + k >= lim;
        uint32_t ek = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(lut) + a);
        if (CHECK) {
            const uint32_t c = masked ? ~0u : ek;
            bad = bad < c ? bad : c;
        }
        if (masked) ek = (ek & 0xFF00u) | kLutOff;  // length 0: the window is kept
        if (k < 7) a = (h >> (ek & 31)) & kLutMask;
        const uint32_t s = ek + (32 - kLutOff);  // 32 - length in the low 5 bits (32: masked, no advance)
        if (k < 7) {
            const uint32_t h2 = __builtin_amdgcn_alignbit(h, m, s);
            const uint32_t m2 = __builtin_amdgcn_alignbit(m, l, s);
            const uint32_t l2 = __builtin_amdgcn_alignbit(l, 0u, s);
            if (!masked) {
                h = h2;
                m = m2;
                l = l2;
            }
        }
        e[k] = ek;
    }
    // each low byte is 19 - length (<= 18): four of them sum below 256
    const uint32_t s0 = (e[0] + e[1] + e[2] + e[3]) & 0xFF, s1 = (e[4] + e[5] + e[6] + e[7]) & 0xFF;
    npos += s0 + s1 - 8 * kLutOff;  // -(bits consumed); masked entries count 19, i.e. nothing
    o0 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0501u) | __builtin_amdgcn_perm(e[3], e[2], 0x05010C0Cu);
    o1 = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0501u) | __builtin_amdgcn_perm(e[7], e[6], 0x05010C0Cu);
    // pack and check here: left to the scheduler, the packing sinks towards
    // the store and the checks towards the end of the stream, and both keep
    // all eight entries of every step alive until then
    asm volatile("" : "+v"(o0), "+v"(o1));
    if (CHECK) asm volatile("" : "+v"(bad));
}

// The same decoder for a complete code (no "no codeword" entries) and all 8
// symbols owed.  The next step's window word index is taken from the sum of
// the first 7 entries before the 8th arrives, so the chain from the 8th entry
// to the next window read is a subtract, a clamp, a shift and an address;
// that read is issued before the 8 symbols are packed and before the step's
// side work.  basem4 is the LDS byte address of the lane's words minus 4 (a
// window starts at word q - 1).
typedef const __attribute__((address_space(3))) uint32_t lds_u32;

struct Win4 {
    uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ Win4 read_win(uint32_t basem4, uint32_t q, uint32_t qlim) {
    lds_u32 *p = (lds_u32 *)(size_t)(basem4 + (min(q, qlim) << 2));
    return Win4{p[0], p[1], p[2], p[3]};
}

// One step from the window words read a step earlier; when NEXT, it also
// reads the next step's words.
template <bool NEXT, bool CHECK, class Side>
__device__ __forceinline__ void lut16_step8_fast(Win4 &win, uint32_t basem4, uint32_t qlim, uint32_t &npos,
                                                 uint32_t &bad, const uint32_t *lut, uint32_t &o0, uint32_t &o1,
                                                 Side &&side) {
    uint32_t h = __builtin_amdgcn_alignbit(win.w0, win.w1, npos);
    uint32_t m = __builtin_amdgcn_alignbit(win.w1, win.w2, npos);
    uint32_t l = __builtin_amdgcn_alignbit(win.w2, win.w3, npos);
    uint32_t a = (h >> kLutOff) & kLutMask;
    const uint32_t K = 31u - npos + 8 * kLutOff;
    const uint8_t *lb = reinterpret_cast<const uint8_t *>(lut);
    uint32_t ecur = *reinterpret_cast<const uint16_t *>(lb + a);
    uint32_t e[8];
    uint32_t T = 0, K6 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t ek = ecur;
        if (CHECK) bad = bad < ek ? bad : ek;
        if (k < 7) {
            a = (h >> (ek & 31)) & kLutMask;
            ecur = *reinterpret_cast<const uint16_t *>(lb + a);
            const uint32_t s = ek + (32 - kLutOff);
            h = __builtin_amdgcn_alignbit(h, m, s);
            m = __builtin_amdgcn_alignbit(m, l, s);
            l = __builtin_amdgcn_alignbit(l, 0u, s);
            T += ek;
        }
        if (k == 6) {
            // low bytes are 19 - length <= 18: their sum never carries out of byte 0
            K6 = K - (T & 0xFF);
            asm volatile("" : "+v"(K6));
        }
        e[k] = ek;
    }
    // (31 - npos') / 32 for npos' = npos + sum(19 - length) - 8 * 19
    if (NEXT) win = read_win(basem4, (K6 - (e[7] & 0xFF)) >> 5, qlim);
    asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]),
                 "+v"(e[7])::"memory");
    npos += ((T + e[7]) & 0xFF) - 8 * kLutOff;
    o0 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0501u) | __builtin_amdgcn_perm(e[3], e[2], 0x05010C0Cu);
    o1 = __builtin_amdgcn_perm(e[5], e[4], 0x0C0C0501u) | __builtin_amdgcn_perm(e[7], e[6], 0x05010C0Cu);
    asm volatile("" : "+v"(o0), "+v"(o1));
    side();
    asm volatile("" ::: "memory");  // the side work stays at this step
}

// QLC decoder, 8 symbols from the 96-bit window (h, m, l); returns them
// packed little-endian in two words and adds the bits consumed to pos.
// Symbols at index >= lim (masked variant only) consume nothing.
template <bool MASKED, bool CHECK>
__device__ __forceinline__ void qlc_step8(uint32_t h, uint32_t m, uint32_t l, uint32_t &pos, uint32_t &bad,
                                          const Tables &t, uint32_t k0, uint32_t lim, uint32_t &o0, uint32_t &o1) {
    uint32_t e[8], y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool masked = MASKED && k0 + k >= lim;  // length 0: the window is kept
        // the area number (3 bits) selects bytes of the area registers (the
        // other selector bytes, 0x0C, give zeros; one funnel shift forms the
        // selector: (0x01818180 << 3) | (h >> 29)); the chain per symbol is
        // funnel shift, v_perm, funnel shift, with the rank and the symbol
        // read beside it (a rank past 255 reads a zero of the 1 KiB table)
        const uint32_t sel = __builtin_amdgcn_alignbit(0x01818180u, h, 29);
        const uint32_t sh = __builtin_amdgcn_perm(t.sh_hi, t.sh_lo, sel);  // 32 - length
        const uint32_t bw = __builtin_amdgcn_perm(t.bw_hi, t.bw_lo, sel);
        const uint32_t r = __builtin_amdgcn_perm(t.st_hi, t.st_lo, sel) + __builtin_amdgcn_ubfe(h, sh, bw);
        if (CHECK && !masked) bad = bad > h ? bad : h;
        y[k] = t.sym[r];
        const uint32_t h2 = __builtin_amdgcn_alignbit(h, m, sh);
        const uint32_t m2 = __builtin_amdgcn_alignbit(m, l, sh);
        const uint32_t l2 = __builtin_amdgcn_alignbit(l, 0u, sh);
        if (!masked) {  // (a funnel shift by 32 would read as 0)
            h = h2;
            m = m2;
            l = l2;
        }
        e[k] = masked ? 32u : sh;
    }
    // e[k] = 32 - length (<= 32 each)
    pos += 8 * 32 - (e[0] + e[1] + e[2] + e[3]) - (e[4] + e[5] + e[6] + e[7]);
    o0 = __builtin_amdgcn_perm(y[1], y[0], 0x0C0C0400u) | __builtin_amdgcn_perm(y[3], y[2], 0x04000C0Cu);
    o1 = __builtin_amdgcn_perm(y[5], y[4], 0x0C0C0400u) | __builtin_amdgcn_perm(y[7], y[6], 0x04000C0Cu);
    asm volatile("" : "+v"(o0), "+v"(o1));
    if (CHECK) asm volatile("" : "+v"(bad));
}

// 8 symbols of either decoder from the current position.
template <int MODE, bool MASKED, bool CHECK, class Src>
__device__ __forceinline__ void step8(const Src &src, uint32_t &pos, uint32_t &bad, const Tables &t, uint32_t k0,
                                      uint32_t lim, uint32_t &o0, uint32_t &o1) {
    if (MODE == kDecodeLut12) {  // pos holds -position here
        lut16_step8<MASKED, CHECK>(src, pos, bad, t.lut, k0, lim, o0, o1);
    } else {
        uint32_t w[4];
        src.fetch4(pos >> 5, w);
        const uint32_t sh = pos & 31;
        const uint32_t h = (uint32_t)(((((uint64_t)w[0] << 32) | w[1]) << sh) >> 32);
        const uint32_t m = (uint32_t)(((((uint64_t)w[1] << 32) | w[2]) << sh) >> 32);
        const uint32_t l = (uint32_t)(((((uint64_t)w[2] << 32) | w[3]) << sh) >> 32);
        qlc_step8<MASKED, CHECK>(h, m, l, pos, bad, t, k0, lim, o0, o1);
    }
}

// Positions as the steps keep them: negated in LUT mode.
template <int MODE>
__device__ __forceinline__ uint32_t to_step_pos(uint32_t pos) { return MODE == kDecodeLut12 ? 0u - pos : pos; }

// Masked decode (the leftover groups): symbols [s_begin, s_end) of one
// sub-stream in blocks of 16; a lane writes only its bytes below lim (lanes
// past the end of the stream own none).
template <int MODE, class Src>
__device__ __forceinline__ uint32_t decode_masked(const Src &src, uint32_t pos, uint32_t lim, const Tables &t,
                                                  uint8_t *dst, uint32_t &bad, uint32_t s_begin, uint32_t s_end) {
    pos = to_step_pos<MODE>(pos);
#pragma unroll 1
    for (uint32_t base = s_begin; base < s_end; base += 16) {
        uint32_t o[4];
#pragma unroll
        for (uint32_t q = 0; q < 2; ++q)
            step8<MODE, true, true>(src, pos, bad, t, base + q * 8, lim, o[2 * q], o[2 * q + 1]);
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
    return to_step_pos<MODE>(pos);
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
// [0, n), decoded into registers (stored with the other half once the group
// is decoded, see store_group).
constexpr uint32_t kHalf = kSub / 2;
constexpr uint32_t kHalfWords = kHalf / 4;

// side(q) runs after step q (8 symbols) of the 16: the memory instructions
// of a group are spread over its decode steps, where the wave mostly waits
// for LDS results, instead of being issued in bursts that stall the waves
// of a workgroup together behind the CU's memory pipeline.
template <int MODE, bool CHECK, class Side>
__device__ __forceinline__ uint32_t decode_half(const LdsWords &src, uint32_t pos, const Tables &t, uint32_t &bad,
                                                uint32_t (&o)[kHalfWords], Side &&side) {
    pos = to_step_pos<MODE>(pos);
    if (MODE == kDecodeLut12) {
        const uint32_t basem4 = (uint32_t)(size_t)(lds_u32 *)src.w - 4u;
        Win4 win = read_win(basem4, (31u - pos) >> 5, src.last + 1);
#pragma unroll
        for (uint32_t q = 0; q < kHalf / 8 - 1; ++q)
            lut16_step8_fast<true, CHECK>(win, basem4, src.last + 1, pos, bad, t.lut, o[2 * q], o[2 * q + 1],
                                          [&] { side(q); });
        constexpr uint32_t ql = kHalf / 8 - 1;
        lut16_step8_fast<false, CHECK>(win, basem4, src.last + 1, pos, bad, t.lut, o[2 * ql], o[2 * ql + 1],
                                       [&] { side(ql); });
        if (CHECK) asm volatile("" : "+v"(bad));
    } else {
#pragma unroll
        for (uint32_t q = 0; q < kHalf / 8; ++q) {
            step8<MODE, false, CHECK>(src, pos, bad, t, 0, kHalf, o[2 * q], o[2 * q + 1]);
            side(q);
            asm volatile("" ::: "memory");  // the side work stays at this step
        }
    }
    return to_step_pos<MODE>(pos);
}

// A group's output goes out through LDS, half a sub-stream (128 bytes per
// lane) at a time: each wave writes its lanes' 8 quads into the first 8 KiB
// of its own lanes' segment slots, then reads them back so that every store
// instruction writes eight whole 128-byte lines (8 lanes per line) instead of
// 16 bytes into each of 64 lines; with STREAM the stores are non-temporal
// (the output is not read again here).  Quad q of lane l sits at slot
// l * 8 + (q ^ (l % 8)).  A wave starts this as soon as its own lanes have
// decoded their second halves: no other wave reads those slots by then
// (window reads that run past a segment's end read words they never use).
template <bool STREAM>
__device__ __forceinline__ void store_group(uint4 *buf, uint8_t *out, uint32_t tid, const uint32_t (&o1)[kHalfWords],
                                            const uint32_t (&o2)[kHalfWords]) {
    const uint32_t w = tid >> 6, l = tid & 63;
    uint4 *wb = buf + w * kWaveSlotQuads;
    uint8_t *wout = out + (size_t)w * 64 * kSub;
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t *o = h ? o2 : o1;
        if (h) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the first half's reads are done
#pragma unroll
        for (uint32_t q = 0; q < 8; ++q)
            wb[l * 8 + (q ^ (l & 7))] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own writes, read by its other lanes
#pragma unroll
        for (uint32_t t = 0; t < 8; ++t) {
            const uint32_t L = 8 * t + (l >> 3), Q = l & 7;
            const uint4 v = wb[L * 8 + (Q ^ (L & 7))];
            uint8_t *dst = wout + L * kSub + h * kHalf + Q * 16;
            if (STREAM) {
                const u32x4 w4 = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(w4, reinterpret_cast<u32x4 *>(dst));
            } else {
                *reinterpret_cast<uint4 *>(dst) = v;
            }
        }
    }
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

__device__ __forceinline__ void span_words(const SpanEntries &e, uint64_t payload_words, uint64_t &lo, uint64_t &hi) {
    uint64_t a, b;
    span_bits(e, a, b);
    lo = uniform64(a >> 5);
    hi = uniform64((b + 31) >> 5);
    if (lo > payload_words) lo = payload_words;
    if (hi > payload_words) hi = payload_words;
    if (hi < lo) hi = lo;
}

// Segment loads.  A set: the first-half (or second-half) segments of a
// group's 256 sub-streams, one start word per segment (relative to the
// group's base word) in an LDS table.  The set's 2560 16-byte quads are
// loaded by the 256 lanes in turn, 10 loads per lane, one per decode step,
// unconditional and branch-free (control flow here would make the
// compiler's wait counting conservative for the whole loop).  Quads are
// 4-byte aligned (a segment starts at any word).  Start words are clamped
// so that nothing at or past payload_words is read: a quad clamped back to
// the payload's last four words is written to the segment at its true
// position, so the words before the end stay right.
struct SegFetch {
    uint4 q[kSegQuads];
};

// Quad k of a set's loads by lane tid: load tid + 256 k of the set, i.e.
// quad part_of of segment seg_of (consecutive lanes read consecutive quads
// of a segment, so one load instruction touches few 128-byte lines).
__device__ __forceinline__ uint32_t seg_of(uint32_t k, uint32_t tid) { return (tid + kThreads * k) / kSegQuads; }
__device__ __forceinline__ uint32_t part_of(uint32_t k, uint32_t tid) { return (tid + kThreads * k) % kSegQuads; }

typedef const __attribute__((address_space(1))) uint32_t gword;
typedef uint32_t u32x4w __attribute__((ext_vector_type(4), aligned(4)));
typedef const __attribute__((address_space(1))) u32x4w gquadw;

// The payload as the loads see it: a global pointer passed through an
// empty asm, so that the compiler no longer knows that nothing writes the
// words and keeps each load at the decode step it is issued at (loads of
// memory known to be read-only are moved freely, and end up together).
__device__ __forceinline__ gword *opaque_words(const uint32_t *p) {
    gword *g = (gword *)p;
    asm volatile("" : "+s"(g));
    return g;
}

// Load k of a set (k = 0..9); `start` is the start of the segment quad k
// belongs to (read from the table a step earlier).  On inputs larger than
// the 256 MB MALL (STREAM), the second-half sets, the last reads of their
// lines, load non-temporally, as the output is stored: the L2 then keeps
// the lines the first-half loads brought in, most of which the second-half
// loads of the same group read again half a group later (a sub-stream's
// first-half segment covers about three quarters of its words).  On
// smaller inputs both stay ordinary (measured faster there).
template <bool STREAM>
__device__ __forceinline__ void seg_fetch(SegFetch &f, uint32_t k, uint32_t start, gword *gb, uint32_t pwr,
                                          uint32_t tid) {
    const uint32_t r = min(start + 4 * part_of(k, tid), pwr - 4);
    gquadw *p = (gquadw *)((const __attribute__((address_space(1))) uint8_t *)gb + (r << 2));
    const u32x4w v = STREAM ? __builtin_nontemporal_load(p) : *p;
    f.q[k] = make_uint4(v.x, v.y, v.z, v.w);
}

// The set's words into the segment area (every lane's loads are complete).
__device__ __forceinline__ void seg_stage(const SegFetch &f, const uint32_t *starts, uint32_t pwr, uint32_t *slots,
                                          uint32_t tid) {
#pragma unroll
    for (uint32_t k = 0; k < kSegQuads; ++k) {
        const uint32_t seg = seg_of(k, tid), p4 = 4 * part_of(k, tid);
        const uint32_t s = starts[seg];
        // p4 unless the load was clamped (a start within the last words of
        // the payload only occurs in a corrupt container: its words then
        // land anywhere inside the segment)
        const uint32_t d = min(min(s + p4, pwr - 4) - s, kSlotData - 4);
        uint32_t *dst = slots + seg * kSlotWords + d;
        dst[0] = f.q[k].x;
        dst[1] = f.q[k].y;
        dst[2] = f.q[k].z;
        dst[3] = f.q[k].w;
    }
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
            lut[i] = (uint16_t)(len ? ((kLutOff - len) | ((uint32_t)ds[i] << 8)) : 0u);
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

// A lane's two segments, as start words relative to the group's base word:
// a holds the sub-stream's first bit (the first half is decoded from words
// a .. a + 39), b = max(e - 39, a) with e the word of its last bit (the
// second half from b .. b + 39).  Rejected lanes use 0.
struct SegJob {
    LaneJob j;
    uint32_t a, b;
};

__device__ __forceinline__ SegJob seg_job(const LaneMeta &m, bool kind_ok, uint64_t payload_words, uint64_t wbase,
                                          uint64_t hi, uint32_t *status) {
    SegJob s;
    s.j = lane_job(m, kind_ok, payload_words, wbase, hi, status);
    s.a = s.j.pos0 >> 5;
    const uint32_t e = s.j.pos_want > 0 ? (s.j.pos_want - 1) >> 5 : 0;
    s.b = max(e >= kSlotData - 1 ? e - (kSlotData - 1) : 0u, s.a);
    return s;
}

// The base word of a group's relative indices (its first word, moved back so
// that 4 words follow it: the kernel runs only when the payload has 4), and
// the words from there to the end of the payload (capped at 2^28, so that
// byte offsets fit 32 bits; relative indices of accepted lanes stay below
// 2^26).
__device__ __forceinline__ uint64_t group_base(uint64_t lo, uint64_t payload_words) {
    return lo < payload_words - 4 ? lo : payload_words - 4;
}

__device__ __forceinline__ uint32_t words_left(uint64_t wbase, uint64_t payload_words) {
    const uint64_t r = payload_words - wbase;
    return (uint32_t)(r < (1ull << 28) ? r : (1ull << 28));
}

// One group from global memory (the leftover groups, and a group whose
// halves do not fit their segments): each lane reads its words straight
// from the payload and writes only bytes below its symbol count.
template <int MODE>
__device__ __forceinline__ void decode_group_global(uint64_t grp, const Tables &t, bool kind_ok,
                                                    const uint32_t *payload, uint64_t payload_words,
                                                    const uint32_t *chunk_bits, const uint64_t *cwo,
                                                    const uint32_t *sub_off, uint64_t n, uint32_t chunk,
                                                    uint64_t num_sub, uint64_t num_chunks, uint8_t *out,
                                                    uint32_t *status, uint32_t tid) {
    uint64_t lo, hi;
    span_words(load_span(grp, num_sub, chunk, num_chunks, cwo, sub_off), payload_words, lo, hi);
    const uint64_t wbase = lo;
    const LaneMeta meta = load_meta(grp * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
    const LaneJob job = lane_job(meta, kind_ok, payload_words, wbase, hi, status);
    if (payload_words <= wbase) return;  // nothing readable: every lane was flagged
    uint8_t *dst = out + (grp * kThreads + tid) * kSub;
    GlobalWords src{payload + wbase, payload_words - wbase - 1};
    uint32_t bad = no_invalid_yet<MODE>();
    const uint32_t pos_end = decode_masked<MODE>(src, job.pos0, job.lim, t, dst, bad, 0, kSub);
    if (job.ok && (saw_invalid<MODE>(bad, t) || pos_end != job.pos_want)) flag_corrupt(status);
}

// The group loop of a workgroup (CHECK: test every table entry for "no
// codeword", needed only when the code is incomplete).  Per group:
//   B1  the segment area is free; the first-half segments (loaded during
//       the previous group's second half) are written into it;
//   B2  first half decoded; its steps issue the loads of the second-half
//       segments; the next group's entries are loaded;
//   B3  every lane checks that its first half ended inside its first
//       segment and starts inside its second; the second-half segments are
//       written into the segment area;
//   B4  second half decoded; its steps issue the loads of the next group's
//       first-half segments; then each wave, without waiting for the
//       others, sends its lanes' output out through their slots.
// A group where any lane's half does not fit its segment (more than ~9.8
// bits per symbol over 128 symbols) is decoded again from global memory, and
// nothing of the staged pass is stored.
template <int MODE, bool CHECK, bool STREAM>
__device__ __forceinline__ void decode_groups(uint64_t grp, uint32_t tid0, const Tables &t, bool kind_ok,
                                              uint8_t *lds, const uint32_t *payload, uint64_t payload_words,
                                              const uint32_t *chunk_bits, const uint64_t *cwo,
                                              const uint32_t *sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub,
                                              uint64_t num_full, uint64_t num_chunks, uint8_t *out,
                                              uint32_t *status) {
    uint32_t *starts_a = reinterpret_cast<uint32_t *>(lds + kOffStartsA);  // first halves, one group ahead
    uint32_t *starts_b = reinterpret_cast<uint32_t *>(lds + kOffStartsB);  // second halves of this group
    uint32_t *flag = reinterpret_cast<uint32_t *>(lds + kOffFlag);
    uint32_t *slots = reinterpret_cast<uint32_t *>(lds + kOffSlots);
    gword *gp = opaque_words(payload);
    // ---- prologue: the first group's entries and first-half segments ------
    LaneMeta meta = load_meta(grp * kThreads + tid0, num_sub, n, chunk, chunk_bits, cwo, sub_off);
    uint64_t lo, hi;
    span_words(load_span(grp, num_sub, chunk, num_chunks, cwo, sub_off), payload_words, lo, hi);
    uint64_t wbase = group_base(lo, payload_words);
    SegJob sj = seg_job(meta, kind_ok, payload_words, wbase, hi, status);
    // the next group's span entries, one group ahead
    SpanEntries nspan = load_span(grp + gridDim.x < num_full ? grp + gridDim.x : grp, num_sub, chunk, num_chunks,
                                  cwo, sub_off);
    starts_a[tid0] = sj.a;
    if (tid0 == 0) *flag = 0;
    __syncthreads();
    SegFetch pf;
    {
        gword *gb = gp + wbase;
        const uint32_t pwr = words_left(wbase, payload_words);
#pragma unroll
        for (uint32_t k = 0; k < kSetLoads; ++k)
            seg_fetch<false>(pf, k, starts_a[seg_of(k, tid0)], gb, pwr, tid0);
    }
    uint32_t o1[kHalfWords], o2[kHalfWords];

    for (;;) {
        // the lane index as an opaque value: computations from it are not
        // hoisted out of the loop to hold dozens of registers across it
        const uint32_t tid = vgpr_copy(tid0);
        gword *gb = gp + wbase;
        const uint32_t pwr = words_left(wbase, payload_words);
        starts_b[tid] = sj.b;
        __syncthreads();  // B1
        // wait for every load of the set here (waits left to the compiler
        // would sit at each use, and every later write of these registers
        // would wait again, for whatever is in flight)
#pragma unroll
        for (uint32_t k = 0; k < kSegQuads; ++k) {
            pin(pf.q[k].x);
            pin(pf.q[k].y);
            pin(pf.q[k].z);
            pin(pf.q[k].w);
        }
        seg_stage(pf, starts_a, pwr, slots, tid);
        __syncthreads();  // B2

        // ---- the next group's entries ---------------------------------
        // loaded on every pass (for the last, this group's own again):
        // control flow around loads makes the compiler's wait counting
        // conservative
        const uint64_t nxt = grp + gridDim.x;
        const bool more = nxt < num_full;
        const uint64_t nxt_c = more ? nxt : grp;
        const LaneMeta nmeta = load_meta(nxt_c * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
        const uint64_t nn = nxt + gridDim.x;
        const SpanEntries nspan2 = load_span(nn < num_full ? nn : nxt_c, num_sub, chunk, num_chunks, cwo, sub_off);
        uint64_t nlo, nhi;
        span_words(nspan, payload_words, nlo, nhi);
        const LdsWords src{slots + tid * kSlotWords, kSlotData - 1};
        uint32_t bad = no_invalid_yet<MODE>();

        // ---- first half; its steps load the second-half segments --------
        uint32_t st = starts_b[seg_of(0, tid)];
        uint32_t pos = decode_half<MODE, CHECK>(src, sj.j.pos0 & 31, t, bad, o1, [&](uint32_t q) {
            if (q < kSetLoads) {
                seg_fetch<STREAM>(pf, q, st, gb, pwr, tid);
                if (q + 1 < kSegQuads) st = starts_b[seg_of(q + 1, tid)];
            }
        });
        // bits from the base word a to the end of the first half; the half
        // must have ended inside segment a, and segment b must hold it
        const uint32_t m = sj.a * 32 + pos;
        const bool fail = sj.j.ok && (pos > kSlotBits || m < sj.b * 32);
        const uint32_t pos2 = fail ? 0u : m - sj.b * 32;
        // the next group's lane checks and first-half starts
        const uint64_t nwbase = group_base(nlo, payload_words);
        const SegJob nsj = seg_job(nmeta, kind_ok, payload_words, nwbase, nhi, status);
        starts_a[tid] = nsj.a;
        if (fail) atomicOr(flag, 1u);
        __syncthreads();  // B3
        const bool gfail = *flag != 0;
#pragma unroll
        for (uint32_t k = 0; k < kSegQuads; ++k) {
            pin(pf.q[k].x);
            pin(pf.q[k].y);
            pin(pf.q[k].z);
            pin(pf.q[k].w);
        }
        seg_stage(pf, starts_b, pwr, slots, tid);
        __syncthreads();  // B4
        if (tid == 0) *flag = 0;

        // ---- second half; its steps load the next group's first halves --
        gword *ngb = gp + nwbase;
        const uint32_t npwr = words_left(nwbase, payload_words);
        st = starts_a[seg_of(0, tid)];
        pos = decode_half<MODE, CHECK>(src, pos2, t, bad, o2, [&](uint32_t q) {
            if (q < kSetLoads) {
                seg_fetch<false>(pf, q, st, ngb, npwr, tid);
                if (q + 1 < kSegQuads) st = starts_a[seg_of(q + 1, tid)];
            }
        });
        if (!gfail && sj.j.ok && (saw_invalid<MODE>(bad, t) || pos != sj.j.pos_want - sj.b * 32))
            flag_corrupt(status);
        if (!gfail)
            store_group<STREAM>(reinterpret_cast<uint4 *>(slots), out + grp * kThreads * kSub, tid, o1, o2);
        else
            decode_group_global<MODE>(grp, t, kind_ok, payload, payload_words, chunk_bits, cwo, sub_off, n, chunk,
                                      num_sub, num_chunks, out, status, tid);

        if (!more) break;
        grp = nxt;
        wbase = nwbase;
        sj = nsj;
        nspan = nspan2;
    }
}

// The groups the main kernel leaves: the last group when it is not full
// (decoded from global memory, see decode_group_global).  Workgroup b owns
// the groups b, b + G, b + 2G, ... (G workgroups); its first wave tests 64
// of them at once (one per lane).
constexpr uint32_t kTestBatch = 64;

struct Leftovers {
    uint32_t todo[kTestBatch];
    uint32_t ntodo;
};

// Test the batch of groups base + l G, l = 0 .. 63: the ones for the
// global-memory path go to lo.todo; returns their number (uniform).
__device__ __forceinline__ uint32_t test_batch(Leftovers &lo_, uint64_t base, uint64_t G, uint64_t num_groups,
                                               uint64_t num_full, uint32_t tid) {
    if (tid == 0) lo_.ntodo = 0;
    __syncthreads();
    if (tid < kTestBatch && base + tid * G < num_groups) {
        const uint64_t g = base + tid * G;
        if (g >= num_full) lo_.todo[atomicAdd(&lo_.ntodo, 1u)] = tid;
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
    for (uint32_t i = 0; i < nt; ++i)
        decode_group_global<MODE>(base + lo_.todo[i] * G, t, kind_ok, payload, payload_words, chunk_bits, cwo,
                                  sub_off, n, chunk, num_sub, num_chunks, out, status, tid);
}

// Main kernel: the full groups (all 256 sub-streams of 256 symbols inside
// [0, n)), so no lane needs masking, then the workgroup's leftover groups.
// Lanes of a corrupt sub-stream decode from somewhere in their segments (LDS
// reads are clamped) and write unspecified bytes into their own 256-byte
// range.  Three workgroups share a CU (LDS: the table and one 41-word
// segment slot per lane, which the two halves use in turn; at most 170
// VGPRs).
template <int MODE, bool STREAM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_kernel(
    const pc_codebook *__restrict__ cb, const uint32_t *__restrict__ payload, uint64_t payload_words,
    const uint32_t *__restrict__ chunk_bits, const uint64_t *__restrict__ cwo,
    const uint32_t *__restrict__ sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub, uint64_t num_full,
    uint64_t num_chunks, uint64_t num_groups, uint8_t *__restrict__ out, uint32_t *__restrict__ status) {
    // everything at fixed LDS addresses (folded into the instructions'
    // offset fields)
    __shared__ uint4 lds4[kLdsBytes / 16];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);
    Leftovers &left = *reinterpret_cast<Leftovers *>(lds + kOffLeft);
    const uint32_t tid = threadIdx.x;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
    const pc_codebook *cbp = reinterpret_cast<const pc_codebook *>(cb);
    load_tables<MODE>(cbb, lds4, tid);
    const bool kind_ok = MODE == kDecodeLut12 || cbp->kind == PC_CODEBOOK_QLC;
    Tables t;
    t.lut = reinterpret_cast<const uint32_t *>(lds4);
    t.sym = reinterpret_cast<const uint8_t *>(lds4);
    if (MODE == kDecodeQlc) qlc_area_regs(cbb, t);

    // this workgroup's first batch of leftover groups, tested while the
    // tables arrive; decoded after the full groups
    const uint64_t G = gridDim.x;
    const uint32_t nt0 = test_batch(left, blockIdx.x, G, num_groups, num_full, tid);
    const uint64_t grp = blockIdx.x;
    if (grp < num_full) {
        if (cbp->complete == 1)
            decode_groups<MODE, false, STREAM>(grp, tid, t, kind_ok, lds, payload, payload_words, chunk_bits, cwo,
                                               sub_off, n, chunk, num_sub, num_full, num_chunks, out, status);
        else
            decode_groups<MODE, true, STREAM>(grp, tid, t, kind_ok, lds, payload, payload_words, chunk_bits, cwo,
                                              sub_off, n, chunk, num_sub, num_full, num_chunks, out, status);
    }
    __syncthreads();  // the tables are in LDS
    decode_batch<MODE>(left, nt0, blockIdx.x, G, t, kind_ok, payload, payload_words, chunk_bits, cwo, sub_off, n,
                       chunk, num_sub, num_chunks, out, status, tid);
    for (uint64_t base = blockIdx.x + G * kTestBatch; base < num_groups; base += G * kTestBatch) {
        __syncthreads();  // the previous batch's list is read
        const uint32_t nt = test_batch(left, base, G, num_groups, num_full, tid);
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
    uint64_t num_full, uint64_t num_chunks, uint8_t *__restrict__ out, uint32_t *__restrict__ status) {
    __shared__ uint4 tab4[MODE == kDecodeLut12 ? kLutBytes / 16 : 64];
    __shared__ Leftovers left;
    const uint32_t tid = threadIdx.x;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
    const pc_codebook *cbp = reinterpret_cast<const pc_codebook *>(cb);
    bool loaded = false;
    const bool kind_ok = MODE == kDecodeLut12 || cbp->kind == PC_CODEBOOK_QLC;
    Tables t;
    t.lut = reinterpret_cast<const uint32_t *>(tab4);
    t.sym = reinterpret_cast<const uint8_t *>(tab4);
    if (MODE == kDecodeQlc) qlc_area_regs(cbb, t);
    const uint64_t G = gridDim.x;
    for (uint64_t base = blockIdx.x; base < num_groups; base += G * kTestBatch) {
        const uint32_t nt = test_batch(left, base, G, num_groups, num_full, tid);
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
    // Per device (the current one), its CU count, queried once.  Concurrent
    // first calls may both query; they store the same value.
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus_of[kMaxDevices];
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
    // groups whose 256 sub-streams all hold 256 symbols inside [0, n)
    // (the main kernel's segment loads need four words of payload)
    const uint64_t num_full = payload_words >= 4 ? n / ((uint64_t)kThreads * kSub) : 0;
    uint64_t grid = (uint64_t)num_cus * kGroupsPerCU;
    if (grid > num_full) grid = num_full;
    uint64_t grid_g = (uint64_t)num_cus * kGroupsPerCU;
    if (grid_g > num_groups) grid_g = num_groups;
    if (num_sub >= kMaxDecodeSubstreams) return hipErrorInvalidValue;  // the entry point checks first
    const bool streaming = n >= kStreamBytes;
#define PC_DEC(K)                                                                                             \
    hipLaunchKernelGGL(K, dim3((uint32_t)grid), dim3(kThreads), 0, stream, cb, payload, payload_words,         \
                       chunk_bits, cwo, sub_off, n, chunk, num_sub, num_full, nc, num_groups, out, status)
#define PC_DEC_G(K)                                                                                           \
    hipLaunchKernelGGL(K, dim3((uint32_t)grid_g), dim3(kThreads), 0, stream, cb, payload, payload_words,       \
                       chunk_bits, cwo, sub_off, n, chunk, num_sub, num_groups, num_full, nc, out, status)
    // with a full group the main kernel also takes the leftover groups;
    // without one, only the leftover kernel runs
    if (mode == kDecodeLut12) {
        if (grid && streaming) PC_DEC((decode_kernel<kDecodeLut12, true>));
        else if (grid) PC_DEC((decode_kernel<kDecodeLut12, false>));
        else PC_DEC_G(decode_global_kernel<kDecodeLut12>);
    } else {
        if (grid && streaming) PC_DEC((decode_kernel<kDecodeQlc, true>));
        else if (grid) PC_DEC((decode_kernel<kDecodeQlc, false>));
        else PC_DEC_G(decode_global_kernel<kDecodeQlc>);
    }
#undef PC_DEC
#undef PC_DEC_G
    return hipGetLastError();
}

}  // namespace pc
