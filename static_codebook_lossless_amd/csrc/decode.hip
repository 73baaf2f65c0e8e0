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
// container entries and its payload span, into registers) are in flight, so
// HBM latency is hidden behind decoding.  Per group:
//   1. the staged span sits in LDS in rows of 34 words: 32 payload words plus
//      copies of the next row's first two, so any 3-word window read stays in
//      one row, and lanes whose sub-streams start ~50 words apart spread over
//      the LDS banks instead of falling on a few;
//   2. per lane and per 4 symbols: fetch 3 words at the current bit, funnel
//      them into a 64-bit window (>= 64 valid bits), then 4 times: read the
//      16-bit table entry (length | symbol << 8) at the top 12 window bits and
//      shift the window by the length;
//   3. 16 decoded bytes per lane go out as one 16-byte store;
//   4. the sub-stream must end exactly at the next sub-stream's first bit (or
//      at chunk_bits); any mismatch sets *status = PC_ERR_CORRUPT.
// A group whose span does not fit the LDS budget is decoded from global
// memory directly.  The QLC variant replaces the 12-bit table with the
// page's own decoder: a 3-bit area number, that area's fixed-width index, and
// the 256-entry rank -> symbol table.
#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kRow = 32;     // payload words per LDS row
constexpr uint32_t kRowPad = 34;  // row + copies of the next row's first 2 words
// Largest staged span: 56 KiB of payload (14 x 16 B per lane in flight).
constexpr uint32_t kPrefetch = 14;
constexpr uint32_t kMaxStageWords = kPrefetch * 4 * kThreads;  // 14336
constexpr uint32_t kGroupsPerCU = 2;

__device__ __forceinline__ void flag_corrupt(uint32_t *status) {
    atomicCAS(status, 0u, (uint32_t)PC_ERR_CORRUPT);
}

__device__ __forceinline__ uint32_t row_index(uint32_t a) { return a + 2 * (a >> 5); }

// Payload word sources.  Indices are clamped so that corrupt positions never
// read outside the staged words or the payload.
struct LdsWords {
    const uint32_t *w;
    uint32_t last;  // last staged word (relative)
    __device__ __forceinline__ void fetch3(uint32_t a, uint32_t &w0, uint32_t &w1, uint32_t &w2) const {
        a = a < last ? a : last;
        const uint32_t i = row_index(a);
        w0 = w[i];
        w1 = w[i + 1];
        w2 = w[i + 2];
    }
};

struct GlobalWords {
    const uint32_t *w;  // payload + wbase
    uint64_t last;      // last readable index relative to w
    __device__ __forceinline__ void fetch3(uint32_t a, uint32_t &w0, uint32_t &w1, uint32_t &w2) const {
        const uint64_t i0 = a < last ? a : last;
        const uint64_t i1 = a + 1 < last ? a + 1 : last;
        const uint64_t i2 = a + 2 < last ? a + 2 : last;
        w0 = w[i0];
        w1 = w[i1];
        w2 = w[i2];
    }
};

struct Tables {
    const uint16_t *lut;   // LDS: 4096 x (length | symbol << 8), length 0 = no codeword
    const uint8_t *sym;    // LDS: sym_of_rank[256] (QLC mode)
    const uint32_t *area;  // LDS: per area (index bits | first rank << 8) (QLC mode)
};

// Decode 4 symbols from the 64-bit window; returns them packed little-endian.
// Symbols at index >= lim (masked variant only) consume nothing.
template <int MODE, bool MASKED, bool CHECK>
__device__ __forceinline__ uint32_t decode4(uint64_t win, uint32_t &pos, uint32_t &bad, const Tables &t,
                                            uint32_t k0, uint32_t lim) {
    uint32_t e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t hi = (uint32_t)(win >> 32);
        uint32_t ek, inv;
        if (MODE == kDecodeLut12) {
            ek = t.lut[hi >> (32 - kPeek)];
            inv = (ek & 0xFF) == 0;
        } else {
            const uint32_t a = t.area[hi >> 29];
            const uint32_t b = a & 15;
            const uint32_t r = (a >> 8) + __builtin_amdgcn_ubfe(hi, 29 - b, b);
            inv = r >= 256;
            ek = (3 + b) | ((uint32_t)t.sym[r & 255] << 8);
        }
        if (MASKED && k0 + k >= lim) {
            ek &= 0xFF00;  // no length: the window stays
            inv = 0;
        }
        if (CHECK) bad |= inv;
        // the shift uses the low 6 bits only: the length
        win <<= (ek & 63);
        e[k] = ek;
    }
    pos += (e[0] + e[1] + e[2] + e[3]) & 0xFF;  // lengths sum to at most 48
    const uint32_t lo2 = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0501u);
    const uint32_t hi2 = __builtin_amdgcn_perm(e[3], e[2], 0x05010C0Cu);
    return lo2 | hi2;
}

template <int MODE, bool MASKED, bool CHECK, class Src>
__device__ __forceinline__ uint32_t decode_lane(const Src &src, uint32_t pos, uint32_t lim, const Tables &t,
                                                uint8_t *dst, uint32_t &bad) {
#pragma unroll 1
    for (uint32_t g16 = 0; g16 < kSub / 16; ++g16) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t w0, w1, w2;
            src.fetch3(pos >> 5, w0, w1, w2);
            const uint32_t s = pos & 31;
            const uint64_t a = (((uint64_t)w0 << 32) | w1) << s;
            const uint64_t b = (((uint64_t)w1 << 32) | w2) << s;
            const uint64_t win = (a & 0xFFFFFFFF00000000ull) | (b >> 32);
            o[q] = decode4<MODE, MASKED, CHECK>(win, pos, bad, t, g16 * 16 + q * 4, lim);
        }
        if (!MASKED) {
            *reinterpret_cast<uint4 *>(dst + g16 * 16) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (g16 * 16 + q * 4 + k < lim) dst[g16 * 16 + q * 4 + k] = (uint8_t)(o[q] >> (8 * k));
        }
    }
    return pos;
}

// Container entries a lane depends on (loaded one group ahead).
struct LaneMeta {
    uint64_t w0, w1;      // chunk_word_offset[c], [c + 1]
    uint32_t cbits;       // chunk_bits[c]
    uint32_t start, end;  // sub-stream start; next start (all ones: chunk_bits)
    uint32_t lim;         // symbols owed by this lane (0 if inactive)
    uint32_t first;       // first sub-stream of its chunk
};

__device__ __forceinline__ LaneMeta load_meta(uint64_t g, uint64_t num_sub, uint64_t n, uint32_t chunk,
                                              const uint32_t *chunk_bits, const uint64_t *cwo,
                                              const uint32_t *sub_off) {
    LaneMeta m{0, 0, 0, 0, 0, 0, 0};
    if (g < num_sub) {
        const uint32_t spc = chunk / kSub;
        const uint64_t c = g / spc;
        const uint32_t j = (uint32_t)(g - c * spc);
        const uint64_t cbase = c * chunk;
        const uint32_t lenc = (uint32_t)((n - cbase) < chunk ? (n - cbase) : chunk);
        const uint32_t nsub_c = (lenc + kSub - 1) / kSub;
        const uint32_t left = lenc - j * kSub;
        m.lim = left < kSub ? left : kSub;
        m.first = j == 0;
        m.w0 = cwo[c];
        m.w1 = cwo[c + 1];
        m.cbits = chunk_bits[c];
        m.start = sub_off[g];
        m.end = (j + 1 < nsub_c) ? sub_off[g + 1] : 0xFFFFFFFFu;
    }
    return m;
}

// Words [lo, hi) of the payload a group needs, from the first sub-stream's
// start and the next group's first sub-stream (or the end of the payload).
// Uniform across the workgroup; every lane later checks its own range.
__device__ __forceinline__ void group_span(uint64_t grp, uint64_t num_sub, uint32_t chunk, uint64_t num_chunks,
                                           const uint64_t *cwo, const uint32_t *sub_off, uint64_t payload_words,
                                           uint64_t &lo, uint64_t &hi) {
    const uint32_t spc = chunk / kSub;
    const uint64_t g0 = grp * kThreads, g1 = g0 + kThreads;
    const uint64_t a = cwo[g0 / spc] * 32 + sub_off[g0];
    const uint64_t b = g1 < num_sub ? cwo[g1 / spc] * 32 + sub_off[g1] : cwo[num_chunks] * 32;
    lo = a >> 5;
    hi = (b + 31) >> 5;
    if (lo > payload_words) lo = payload_words;
    if (hi > payload_words) hi = payload_words;
    if (hi < lo) hi = lo;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const pc_codebook *__restrict__ cb, const uint32_t *__restrict__ payload, uint64_t payload_words,
    const uint32_t *__restrict__ chunk_bits, const uint64_t *__restrict__ cwo,
    const uint32_t *__restrict__ sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub, uint64_t num_groups,
    uint64_t num_chunks, uint8_t *__restrict__ out, uint32_t *__restrict__ status, uint32_t stage_cap) {
    // Tables at fixed LDS addresses (folded into the instructions' offset
    // fields); the payload staging rows are the dynamic part.
    __shared__ uint4 tab4[MODE == kDecodeLut12 ? 512 : 16];
    __shared__ uint32_t area_tab[8];
    extern __shared__ uint4 stage4[];
    uint32_t *stage = reinterpret_cast<uint32_t *>(stage4);
    const uint32_t tid = threadIdx.x;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);
    const pc_codebook *cbp = reinterpret_cast<const pc_codebook *>(cb);

    if (MODE == kDecodeLut12) {
        // interleave dec_len / dec_sym into 16-bit entries
        for (uint32_t i = tid; i < 256; i += kThreads) {
            const uint4 s = reinterpret_cast<const uint4 *>(cbb + kOffDecSym)[i];
            const uint4 l = reinterpret_cast<const uint4 *>(cbb + kOffDecSym + 4096)[i];
            const uint32_t sv[4] = {s.x, s.y, s.z, s.w}, lv[4] = {l.x, l.y, l.z, l.w};
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                o[2 * k] = __builtin_amdgcn_perm(sv[k], lv[k], 0x05010400u);
                o[2 * k + 1] = __builtin_amdgcn_perm(sv[k], lv[k], 0x07030602u);
            }
            tab4[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
            tab4[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    } else {
        if (tid < 64)
            reinterpret_cast<uint32_t *>(tab4)[tid] = reinterpret_cast<const uint32_t *>(cbb + kOffSymOfRank)[tid];
        if (tid < 8) {
            const uint32_t b = cbb[kOffQlcBits + tid];
            const uint32_t st = reinterpret_cast<const uint16_t *>(cbb + kOffQlcStart)[tid];
            area_tab[tid] = b | (st << 8);
        }
    }
    const bool kind_ok = MODE == kDecodeLut12 || cbp->kind == PC_CODEBOOK_QLC;
    const bool complete = cbp->complete == 1;
    Tables t;
    t.lut = reinterpret_cast<const uint16_t *>(tab4);
    t.sym = reinterpret_cast<const uint8_t *>(tab4);
    t.area = area_tab;

    // ---- prologue: loads of the first group --------------------------
    uint64_t grp = blockIdx.x;
    if (grp >= num_groups) return;
    LaneMeta meta = load_meta(grp * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
    uint64_t lo, hi;
    group_span(grp, num_sub, chunk, num_chunks, cwo, sub_off, payload_words, lo, hi);
    uint4 pre[kPrefetch];
    auto issue_payload = [&](uint64_t lo_, uint64_t hi_) {
        const uint64_t wb = lo_ & ~(uint64_t)(kRow - 1);
        const uint64_t cnt = hi_ - wb;
        if (cnt <= stage_cap) {
            const uint32_t nq = (uint32_t)((cnt + 3) / 4);
            const uint4 *src = reinterpret_cast<const uint4 *>(payload + wb);
            const uint64_t full_q = (payload_words - wb) / 4;  // 16-byte loads fully inside the payload
#pragma unroll
            for (uint32_t k = 0; k < kPrefetch; ++k) {
                const uint32_t q = tid + k * kThreads;
                if (q < nq) {
                    if (q < full_q) {
                        pre[k] = load_stream16(src + q);
                    } else {
                        uint32_t v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            v[i] = (wb + 4 * q + i < payload_words) ? payload[wb + 4 * q + i] : 0u;
                        pre[k] = make_uint4(v[0], v[1], v[2], v[3]);
                    }
                }
            }
        }
    };
    issue_payload(lo, hi);

    for (;;) {
        // ---- stage the current group (its loads were issued earlier) --
        const uint64_t wbase = lo & ~(uint64_t)(kRow - 1);
        const uint64_t cnt = hi - wbase;
        const bool staged = cnt <= stage_cap;
        __syncthreads();  // every lane is done with the previous group's rows
        if (staged) {
            const uint32_t nq = (uint32_t)((cnt + 3) / 4);
#pragma unroll
            for (uint32_t k = 0; k < kPrefetch; ++k) {
                const uint32_t q = tid + k * kThreads;
                if (q < nq) {
                    const uint32_t i = row_index(4 * q);
                    uint2 *d = reinterpret_cast<uint2 *>(stage + i);
                    d[0] = make_uint2(pre[k].x, pre[k].y);
                    d[1] = make_uint2(pre[k].z, pre[k].w);
                    if ((q & 7) == 0 && q) *reinterpret_cast<uint2 *>(stage + i - 2) = make_uint2(pre[k].x, pre[k].y);
                }
            }
        }
        __syncthreads();

        // ---- this lane's checks -----------------------------------------
        const uint32_t end = meta.end == 0xFFFFFFFFu ? meta.cbits : meta.end;
        const uint64_t abs_s = meta.w0 * 32 + meta.start, abs_e = meta.w0 * 32 + end;
        const bool active = meta.lim > 0;
        const bool ok = active && kind_ok && meta.w1 >= meta.w0 &&
                        (meta.w1 - meta.w0) == ((uint64_t)meta.cbits + 31) / 32 && meta.w1 <= payload_words &&
                        (!meta.first || meta.start == 0) && meta.start <= end && end <= meta.cbits &&
                        abs_s >= wbase * 32 && abs_e <= hi * 32 && cnt < (1u << 26);
        if (active && !ok) flag_corrupt(status);
        const uint32_t lim = ok ? meta.lim : 0;
        const uint32_t pos0 = ok ? (uint32_t)(abs_s - wbase * 32) : 0;
        const uint32_t pos_want = ok ? (uint32_t)(abs_e - wbase * 32) : 0;
        uint8_t *dst = out + (grp * kThreads + tid) * kSub;
        const bool allfull = __syncthreads_count(lim == kSub) == (int)kThreads;

        // ---- issue the next group's loads ------------------------------
        const uint64_t nxt = grp + gridDim.x;
        const bool more = nxt < num_groups;
        uint64_t nlo = 0, nhi = 0;
        LaneMeta nmeta{0, 0, 0, 0, 0, 0, 0};
        if (more) {
            nmeta = load_meta(nxt * kThreads + tid, num_sub, n, chunk, chunk_bits, cwo, sub_off);
            group_span(nxt, num_sub, chunk, num_chunks, cwo, sub_off, payload_words, nlo, nhi);
            issue_payload(nlo, nhi);
        }

        // ---- decode --------------------------------------------------
        uint32_t bad = 0, pos_end = 0;
        if (staged) {
            LdsWords src{stage, (uint32_t)(cnt > 0 ? cnt - 1 : 0)};
            if (allfull) {
                if (complete)
                    pos_end = decode_lane<MODE, false, false>(src, pos0, lim, t, dst, bad);
                else
                    pos_end = decode_lane<MODE, false, true>(src, pos0, lim, t, dst, bad);
            } else if (active) {
                pos_end = decode_lane<MODE, true, true>(src, pos0, lim, t, dst, bad);
            }
        } else if (cnt > 0) {
            GlobalWords src{payload + wbase, cnt - 1};
            if (allfull)
                pos_end = decode_lane<MODE, false, true>(src, pos0, lim, t, dst, bad);
            else if (active)
                pos_end = decode_lane<MODE, true, true>(src, pos0, lim, t, dst, bad);
        }
        if (ok && (bad || pos_end != pos_want)) flag_corrupt(status);

        if (!more) break;
        grp = nxt;
        meta = nmeta;
        lo = nlo;
        hi = nhi;
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
    // LDS budget for a staged span: the average span of a group plus 1/16
    // slack and two rows, at most kMaxStageWords; stored as rows of 34 words.
    const uint64_t avg_words = (payload_words * kThreads + num_sub - 1) / (num_sub ? num_sub : 1);
    uint64_t cap = avg_words + avg_words / 16 + 2 * kRow;
    if (cap > kMaxStageWords) cap = kMaxStageWords;
    cap = (cap + kRow - 1) / kRow * kRow;
    const size_t shmem = (cap / kRow + 1) * kRowPad * 4;
    static bool attr_set[2] = {false, false};
    static int num_cus = 0;
    if (!num_cus) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const void *fn = mode == kDecodeLut12 ? (const void *)decode_kernel<kDecodeLut12>
                                          : (const void *)decode_kernel<kDecodeQlc>;
    if (!attr_set[mode]) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (kMaxStageWords / kRow + 1) * kRowPad * 4);
        if (e != hipSuccess) return e;
        attr_set[mode] = true;
    }
    uint64_t grid = (uint64_t)num_cus * kGroupsPerCU;
    if (grid > num_groups) grid = num_groups;
    if (mode == kDecodeLut12)
        hipLaunchKernelGGL(decode_kernel<kDecodeLut12>, dim3((uint32_t)grid), dim3(kThreads), shmem, stream, cb,
                           payload, payload_words, chunk_bits, cwo, sub_off, n, chunk, num_sub, num_groups, nc, out,
                           status, (uint32_t)cap);
    else
        hipLaunchKernelGGL(decode_kernel<kDecodeQlc>, dim3((uint32_t)grid), dim3(kThreads), shmem, stream, cb,
                           payload, payload_words, chunk_bits, cwo, sub_off, n, chunk, num_sub, num_groups, nc, out,
                           status, (uint32_t)cap);
    return hipGetLastError();
}

}  // namespace pc
