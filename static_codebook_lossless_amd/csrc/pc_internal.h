// Internal declarations of libpc.so (device helpers and kernel launchers).
// Target: CDNA4 (gfx950), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pc.h"

namespace pc {

constexpr uint32_t kWave = 64;
constexpr uint32_t kSub = PC_SUBSTREAM;  // symbols per decode sub-stream
constexpr uint32_t kPeek = PC_MAX_LEN;   // bits looked at per codeword
constexpr size_t kMaxChunk = (size_t)1 << 24;
// decode: sub-stream indices, and an index plus 256, stay below 2^32
constexpr uint64_t kMaxDecodeSubstreams = 0xFFFFFF00ull;

// Byte offsets inside pc_codebook (checked by static_asserts in codebook.cpp).
constexpr uint32_t kOffLength = 32;
constexpr uint32_t kOffCode = 288;
constexpr uint32_t kOffDecSym = 800;
constexpr uint32_t kOffQlcBits = 8992;
constexpr uint32_t kOffQlcStart = 9000;
constexpr uint32_t kOffSymOfRank = 9272;

// ---------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    // Lanes whose DPP source is outside the pattern (or whose row is masked
    // off) receive 0.
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (row shifts inside rows
// of 16, then the row broadcasts of lane 15 and lane 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += dpp_u32<0x111>(v);        // row_shr:1
    v += dpp_u32<0x112>(v);        // row_shr:2
    v += dpp_u32<0x114>(v);        // row_shr:4
    v += dpp_u32<0x118>(v);        // row_shr:8
    v += dpp_u32<0x142, 0xA>(v);   // row_bcast:15 -> rows 1 and 3
    v += dpp_u32<0x143, 0xC>(v);   // row_bcast:31 -> rows 2 and 3
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m, 64);
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m, 64);
        v = o > v ? o : v;
    }
    return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data read once (non-temporal: not kept in the caches).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    uint32_t lo = uniform((uint32_t)v), hi = uniform((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files, called from api.hip).
// ---------------------------------------------------------------------------

// max_polls: polls of the cross-chunk scan's bounded wait before it gives up
// and writes PC_ERR_TIMEOUT to *status (which the launch first zeroes).
constexpr uint32_t kDefaultWaitPolls = 1u << 20;

hipError_t launch_encode(const pc_codebook *cb, const uint8_t *in, uint64_t n, uint32_t chunk,
                         uint32_t *payload, uint32_t *chunk_bits, uint64_t *cwo, uint32_t *sub_off,
                         uint64_t *ws, uint32_t *status, uint32_t max_polls, hipStream_t stream);

enum DecodeMode { kDecodeLut12 = 0, kDecodeQlc = 1 };

hipError_t launch_decode(int mode, const pc_codebook *cb, const uint32_t *payload, uint64_t payload_words,
                         const uint32_t *chunk_bits, const uint64_t *cwo, const uint32_t *sub_off,
                         uint64_t n, uint32_t chunk, uint8_t *out, uint32_t *status, hipStream_t stream);

hipError_t launch_histogram(const uint8_t *in, uint64_t n, uint64_t *counts, hipStream_t stream);

}  // namespace pc
