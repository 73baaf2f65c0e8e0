// Fixed-codebook decoder for gfx950.
//
// One lane decodes one 256-symbol sub-stream; the side index gives every
// sub-stream's first bit, so lanes are independent ("Quad Length Codes for
// Lossless Compression of e4m3", abstract, blames bit-sequential tree walks
// for slow Huffman decoding; here every codeword costs one table lookup).
//
// Workgroup = 256 consecutive sub-streams.  Steps:
//   1. copy the 12-bit peek tables (dec_sym / dec_len, 8 KiB) into LDS;
//   2. check the container entries every lane depends on;
//   3. stage the workgroup's contiguous payload span in LDS with coalesced
//      16-byte loads when it fits the LDS budget the host chose (otherwise
//      lanes read payload words from global memory directly);
//   4. per lane, per group of 4 symbols: fetch 3 words at the current bit
//      position, funnel-shift them into a 64-bit window (>= 64 valid bits),
//      then 4 times: peek the top 12 bits -> (symbol, length) from LDS,
//      shift the window by the length;
//   5. 16 decoded bytes per lane go out as one 16-byte store;
//   6. the sub-stream must end exactly at the next sub-stream's first bit
//      (or at chunk_bits); any mismatch sets *status = PC_ERR_CORRUPT.
// The QLC variant replaces step 4's table with the page's own decoder: a
// 3-bit area number, that area's fixed-width index, and the 256-entry
// rank -> symbol table.
#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kGuardWords = 4;

__device__ __forceinline__ void flag_corrupt(uint32_t *status) {
    atomicCAS(status, 0u, (uint32_t)PC_ERR_CORRUPT);
}

// Payload word source: LDS staging buffer (words [0, limit]) or global
// memory (words [0, limit]); indices are clamped so corrupt positions never
// read outside either.
struct LdsWords {
    const uint32_t *w;
    uint32_t limit;
    __device__ __forceinline__ void fetch3(uint32_t a, uint32_t &w0, uint32_t &w1, uint32_t &w2) const {
        a = a < limit ? a : limit;
        w0 = w[a];
        w1 = w[a + 1];
        w2 = w[a + 2];
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
    const uint8_t *sym;   // LDS: dec_sym[4096]  (LUT mode) / sym_of_rank[256] (QLC mode)
    const uint8_t *len;   // LDS: dec_len[4096]  (LUT mode)
    const uint32_t *area; // LDS: per area (index bits | first rank << 8) (QLC mode)
};

// Decode up to 4 symbols from the 64-bit window; returns them packed
// little-endian.  `lim` is the number of symbols still owed by this lane
// (only the masked variant looks at it).
template <int MODE, bool MASKED>
__device__ __forceinline__ uint32_t decode4(uint64_t &win, uint32_t &pos, uint32_t &bad, const Tables &t,
                                            uint32_t k0, uint32_t lim) {
    uint32_t out = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t hi = (uint32_t)(win >> 32);
        uint32_t sym, l, inv;
        if (MODE == kDecodeLut12) {
            const uint32_t peek = hi >> (32 - kPeek);
            sym = t.sym[peek];
            l = t.len[peek];
            inv = (l == 0);
        } else {
            const uint32_t e = t.area[hi >> 29];
            const uint32_t b = e & 15;
            const uint32_t r = (e >> 8) + __builtin_amdgcn_ubfe(hi, 29 - b, b);
            inv = (r >= 256);
            sym = t.sym[r & 255];
            l = 3 + b;
        }
        if (MASKED && k0 + k >= lim) {
            l = 0;
            inv = 0;
        }
        bad |= inv;
        win <<= l;
        pos += l;
        out |= sym << (8 * k);
    }
    return out;
}

template <int MODE, bool MASKED, class Src>
__device__ __forceinline__ void decode_lane(const Src &src, uint32_t pos, uint32_t lim, const Tables &t,
                                            uint8_t *dst, uint32_t &pos_out, uint32_t &bad) {
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
            uint64_t win = (a & 0xFFFFFFFF00000000ull) | (b >> 32);
            o[q] = decode4<MODE, MASKED>(win, pos, bad, t, g16 * 16 + q * 4, lim);
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
    pos_out = pos;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const pc_codebook *__restrict__ cb, const uint32_t *__restrict__ payload, uint64_t payload_words,
    const uint32_t *__restrict__ chunk_bits, const uint64_t *__restrict__ cwo,
    const uint32_t *__restrict__ sub_off, uint64_t n, uint32_t chunk, uint64_t num_sub,
    uint8_t *__restrict__ out, uint32_t *__restrict__ status, uint32_t stage_cap) {
    extern __shared__ uint4 smem4[];
    __shared__ uint64_t red[3][4];
    __shared__ uint32_t area_tab[8];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t *cbb = reinterpret_cast<const uint8_t *>(cb);

    // 1. tables into LDS
    uint8_t *tab = reinterpret_cast<uint8_t *>(smem4);
    uint32_t tab_bytes;
    if (MODE == kDecodeLut12) {
        tab_bytes = 8192;
        const uint4 *src = reinterpret_cast<const uint4 *>(cbb + kOffDecSym);
        for (uint32_t i = tid; i < 512; i += kThreads) smem4[i] = src[i];
    } else {
        tab_bytes = 256;
        if (tid < 64)
            reinterpret_cast<uint32_t *>(smem4)[tid] = reinterpret_cast<const uint32_t *>(cbb + kOffSymOfRank)[tid];
        if (tid < 8) {
            const uint32_t b = cbb[kOffQlcBits + tid];
            const uint32_t st = reinterpret_cast<const uint16_t *>(cbb + kOffQlcStart)[tid];
            area_tab[tid] = b | (st << 8);
        }
    }
    uint32_t *stage = reinterpret_cast<uint32_t *>(tab + tab_bytes);
    const bool qlc_ok = MODE == kDecodeLut12 || reinterpret_cast<const pc_codebook *>(cb)->kind == PC_CODEBOOK_QLC;

    // 2. per-lane container checks
    const uint64_t g = (uint64_t)blockIdx.x * kThreads + tid;
    const bool active = g < num_sub;
    const uint32_t spc = chunk / kSub;
    uint32_t lim = 0;
    uint64_t abs_s = 0, abs_e = 0;
    bool ok = false;
    if (active) {
        const uint64_t c = g / spc;
        const uint32_t j = (uint32_t)(g - c * spc);
        const uint64_t cbase = c * chunk;
        const uint32_t lenc = (uint32_t)((n - cbase) < chunk ? (n - cbase) : chunk);
        const uint32_t nsub_c = (lenc + kSub - 1) / kSub;
        const uint32_t left = lenc - j * kSub;
        lim = left < kSub ? left : kSub;
        const uint64_t w0 = cwo[c], w1 = cwo[c + 1];
        const uint32_t cbits = chunk_bits[c];
        const uint32_t start = sub_off[g];
        const uint32_t end = (j + 1 < nsub_c) ? sub_off[g + 1] : cbits;
        ok = qlc_ok && w1 >= w0 && (w1 - w0) == ((uint64_t)cbits + 31) / 32 && w1 <= payload_words &&
             (j != 0 || start == 0) && start <= end && end <= cbits;
        abs_s = w0 * 32 + start;
        abs_e = w0 * 32 + end;
    }
    if (active && !ok) flag_corrupt(status);
    if (!ok) lim = 0;

    // workgroup span of payload words
    uint64_t lo = ok ? (abs_s >> 5) : ~0ull;
    uint64_t hi = ok ? ((abs_e + 31) >> 5) : 0;
    const uint64_t full = (lim == kSub) ? 1 : 0;
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    const uint64_t nfull = wave_sum_u64(full);
    if (lane == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
        red[2][wave] = nfull;
    }
    __syncthreads();
    lo = red[0][0];
    hi = red[1][0];
    uint64_t allfull = red[2][0];
    for (int w = 1; w < 4; ++w) {
        lo = red[0][w] < lo ? red[0][w] : lo;
        hi = red[1][w] > hi ? red[1][w] : hi;
        allfull += red[2][w];
    }
    const bool masked = allfull != kThreads;
    if (lo > hi) lo = hi = 0;  // no healthy lane in this workgroup
    const uint64_t wbase = lo & ~3ull;
    uint64_t wend = hi + kGuardWords;
    if (wend > payload_words) wend = payload_words;
    const uint64_t cnt = wend > wbase ? wend - wbase : 0;
    const bool staged = cnt + kGuardWords <= stage_cap;

    Tables t;
    if (MODE == kDecodeLut12) {
        t.sym = tab;
        t.len = tab + 4096;
        t.area = nullptr;
    } else {
        t.sym = tab;
        t.len = nullptr;
        t.area = area_tab;
    }

    // 3. stage the span
    if (staged) {
        const uint32_t c32 = (uint32_t)cnt;
        const uint32_t nq = c32 / 4;
        const uint4 *src = reinterpret_cast<const uint4 *>(payload + wbase);
        uint4 *dq = reinterpret_cast<uint4 *>(stage);
        for (uint32_t i = tid; i < nq; i += kThreads) dq[i] = src[i];
        for (uint32_t i = nq * 4 + tid; i < c32 + kGuardWords; i += kThreads)
            stage[i] = i < c32 ? payload[wbase + i] : 0u;
    }
    __syncthreads();

    // 4-6. decode
    uint32_t bad = 0;
    uint32_t pos_end = 0;
    const uint32_t pos0 = ok ? (uint32_t)(abs_s - wbase * 32) : 0;
    uint8_t *dst = out + g * kSub;
    if (staged) {
        LdsWords src{stage, (uint32_t)(cnt > 0 ? cnt - 1 : 0)};
        if (!masked)
            decode_lane<MODE, false>(src, pos0, lim, t, dst, pos_end, bad);
        else if (active)
            decode_lane<MODE, true>(src, pos0, lim, t, dst, pos_end, bad);
    } else {
        GlobalWords src{payload + wbase, cnt > 0 ? cnt - 1 : 0};
        if (cnt == 0) {
            // nothing readable: every healthy lane would be corrupt anyway
            if (ok) flag_corrupt(status);
        } else if (!masked)
            decode_lane<MODE, false>(src, pos0, lim, t, dst, pos_end, bad);
        else if (active)
            decode_lane<MODE, true>(src, pos0, lim, t, dst, pos_end, bad);
    }
    if (ok && (bad || (uint64_t)pos_end != abs_e - wbase * 32)) flag_corrupt(status);
}

}  // namespace

hipError_t launch_decode(int mode, const pc_codebook *cb, const uint32_t *payload, uint64_t payload_words,
                         const uint32_t *chunk_bits, const uint64_t *cwo, const uint32_t *sub_off,
                         uint64_t n, uint32_t chunk, uint8_t *out, uint32_t *status, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint64_t nc = (n + chunk - 1) / chunk;
    const uint64_t last = n - (nc - 1) * chunk;
    const uint64_t num_sub = (nc - 1) * (chunk / kSub) + (last + kSub - 1) / kSub;
    const uint64_t blocks = (num_sub + kThreads - 1) / kThreads;
    // LDS budget for the staged payload: the average span of a workgroup
    // plus 1/16 slack, capped so that two workgroups fit in a CU's LDS.
    const uint32_t tab_bytes = mode == kDecodeLut12 ? 8192 : 256;
    const uint64_t avg_words = (payload_words * kThreads + num_sub - 1) / (num_sub ? num_sub : 1);
    uint64_t cap = avg_words + avg_words / 16 + 64;
    const uint64_t max_cap = (72 * 1024 - tab_bytes) / 4;
    if (cap > max_cap) cap = max_cap;
    cap = (cap + 3) & ~3ull;
    const size_t shmem = tab_bytes + cap * 4;
    // Dynamic LDS above 64 KiB must be allowed once per kernel.
    static bool attr_set[2] = {false, false};
    const void *fn = mode == kDecodeLut12 ? (const void *)decode_kernel<kDecodeLut12>
                                          : (const void *)decode_kernel<kDecodeQlc>;
    if (!attr_set[mode]) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 72 * 1024);
        if (e != hipSuccess) return e;
        attr_set[mode] = true;
    }
    if (mode == kDecodeLut12)
        hipLaunchKernelGGL(decode_kernel<kDecodeLut12>, dim3((uint32_t)blocks), dim3(kThreads), shmem, stream, cb,
                           payload, payload_words, chunk_bits, cwo, sub_off, n, chunk, num_sub, out, status,
                           (uint32_t)cap);
    else
        hipLaunchKernelGGL(decode_kernel<kDecodeQlc>, dim3((uint32_t)blocks), dim3(kThreads), shmem, stream, cb,
                           payload, payload_words, chunk_bits, cwo, sub_off, n, chunk, num_sub, out, status,
                           (uint32_t)cap);
    return hipGetLastError();
}

}  // namespace pc
