// C-ABI entry points of libpc.so that touch the device: argument checks,
// launch geometry, and HIP error mapping.  The kernels live in encode.hip,
// decode.hip and histogram.hip; host-only entry points in codebook.cpp.
#include <atomic>

#include "pc_internal.h"

// Workspace of pc_encode_noalloc: the ticket word and one look-back
// descriptor per workgroup unit (at most one per chunk), for up to
// kNoAllocMaxChunks chunks (fewer for chunks of several 64 KiB units, whose
// per-unit counts share the array): 8 MiB + 8 bytes on every GPU the library runs
// on, held until the process ends.  Host code never uses the array's name
// as an address: each device's copy is reached through the pointer
// hipGetSymbolAddress returns for it (noalloc_scratch below).
static constexpr size_t kNoAllocMaxChunks = (size_t)1 << 20;
static __device__ __align__(256) uint64_t scratch[1 + kNoAllocMaxChunks];

namespace {

std::atomic<uint32_t> g_wait_polls{pc::kDefaultWaitPolls};

constexpr int kMaxDevices = 64;
std::atomic<uint64_t *> g_scratch_of[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current).  Concurrent first calls may both look it up; they
// store the same address.
hipError_t noalloc_scratch(uint64_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint64_t *p = g_scratch_of[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!addr) return hipErrorInvalidSymbol;
        p = static_cast<uint64_t *>(addr);
        g_scratch_of[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool chunk_ok(size_t chunk) {
    return chunk >= PC_SUBSTREAM && chunk % PC_SUBSTREAM == 0 && chunk <= pc::kMaxChunk;
}

pc_status map_hip(hipError_t e) { return e == hipSuccess ? PC_OK : PC_ERR_HIP; }

pc_status check_decode_args(const pc_codebook *d_cb, const uint32_t *d_payload, const uint32_t *d_chunk_bits,
                            const uint64_t *d_cwo, const uint32_t *d_sub_off, size_t n, size_t chunk,
                            uint8_t *d_out, uint32_t *d_status) {
    if (!chunk_ok(chunk)) return PC_ERR_INVALID_ARG;
    if (n == 0) return PC_OK;
    if (!d_cb || !d_payload || !d_chunk_bits || !d_cwo || !d_sub_off || !d_out || !d_status)
        return PC_ERR_INVALID_ARG;
    if (!aligned(d_cb, 16) || !aligned(d_payload, 16) || !aligned(d_out, 16) || !aligned(d_cwo, 8) ||
        !aligned(d_chunk_bits, 4) || !aligned(d_sub_off, 4) || !aligned(d_status, 4))
        return PC_ERR_INVALID_ARG;
    // sub-stream indices are 32-bit on the device (n below about 2^40)
    if (pc_num_substreams(n, chunk) >= pc::kMaxDecodeSubstreams) return PC_ERR_UNSUPPORTED;
    return PC_OK;
}

pc_status check_encode_args(const pc_codebook *d_cb, const uint8_t *d_in, size_t n, size_t chunk,
                            uint32_t *d_payload, size_t payload_capacity_words, uint32_t *d_chunk_bits,
                            uint64_t *d_chunk_word_offset, uint32_t *d_sub_off, uint32_t *d_status) {
    if (!chunk_ok(chunk) || !d_chunk_word_offset || !d_status) return PC_ERR_INVALID_ARG;
    if (!aligned(d_chunk_word_offset, 8) || !aligned(d_status, 4)) return PC_ERR_INVALID_ARG;
    if (n > 0) {
        if (!d_cb || !d_in || !d_payload || !d_chunk_bits || !d_sub_off) return PC_ERR_INVALID_ARG;
        if (!aligned(d_cb, 16) || !aligned(d_in, 16) || !aligned(d_payload, 16) || !aligned(d_chunk_bits, 4) ||
            !aligned(d_sub_off, 4))
            return PC_ERR_INVALID_ARG;
        if (pc_num_chunks(n, chunk) > 0x7FFFFFFFull) return PC_ERR_UNSUPPORTED;
        if (payload_capacity_words < pc_max_payload_words(n, chunk)) return PC_ERR_CAPACITY;
    }
    return PC_OK;
}

}  // namespace

extern "C" {

size_t pc_encode_workspace_bytes(size_t n, size_t chunk) {
    if (!chunk_ok(chunk)) return 0;
    // the ticket word and one look-back descriptor per chunk; chunks of
    // several 64 KiB units also keep a u32 per unit of their full chunks
    const size_t units = chunk > 65536 && chunk % 65536 == 0 ? (n / chunk) * (chunk / 65536) : 0;
    return (1 + pc_num_chunks(n, chunk)) * sizeof(uint64_t) + (units + 1) / 2 * sizeof(uint64_t);
}

uint32_t pc_encode_set_wait_limit(uint32_t polls) {
    return g_wait_polls.exchange(polls ? polls : pc::kDefaultWaitPolls);
}

pc_status pc_encode(const pc_codebook *d_cb, const uint8_t *d_in, size_t n, size_t chunk, uint32_t *d_payload,
                    size_t payload_capacity_words, uint32_t *d_chunk_bits, uint64_t *d_chunk_word_offset,
                    uint32_t *d_sub_off, void *d_ws, size_t ws_bytes, uint32_t *d_status, void *stream) {
    pc_status st = check_encode_args(d_cb, d_in, n, chunk, d_payload, payload_capacity_words, d_chunk_bits,
                                     d_chunk_word_offset, d_sub_off, d_status);
    if (st != PC_OK) return st;
    if (!d_ws || !aligned(d_ws, 8)) return PC_ERR_INVALID_ARG;
    if (ws_bytes < pc_encode_workspace_bytes(n, chunk)) return PC_ERR_CAPACITY;
    return map_hip(pc::launch_encode(d_cb, d_in, n, (uint32_t)chunk, d_payload, d_chunk_bits, d_chunk_word_offset,
                                     d_sub_off, static_cast<uint64_t *>(d_ws), d_status,
                                     g_wait_polls.load(std::memory_order_relaxed), static_cast<hipStream_t>(stream)));
}

pc_status pc_encode_noalloc(const pc_codebook *d_cb, const uint8_t *d_in, size_t n, size_t chunk,
                            uint32_t *d_payload, size_t payload_capacity_words, uint32_t *d_chunk_bits,
                            uint64_t *d_chunk_word_offset, uint32_t *d_sub_off, uint32_t *d_status, void *stream) {
    pc_status st = check_encode_args(d_cb, d_in, n, chunk, d_payload, payload_capacity_words, d_chunk_bits,
                                     d_chunk_word_offset, d_sub_off, d_status);
    if (st != PC_OK) return st;
    if (pc_num_chunks(n, chunk) > kNoAllocMaxChunks || pc_encode_workspace_bytes(n, chunk) > sizeof(scratch))
        return PC_ERR_CAPACITY;
    uint64_t *ws = nullptr;
    const hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return PC_ERR_HIP;
    return map_hip(pc::launch_encode(d_cb, d_in, n, (uint32_t)chunk, d_payload, d_chunk_bits, d_chunk_word_offset,
                                     d_sub_off, ws, d_status, g_wait_polls.load(std::memory_order_relaxed),
                                     static_cast<hipStream_t>(stream)));
}

pc_status pc_decode(const pc_codebook *d_cb, const uint32_t *d_payload, size_t payload_words,
                    const uint32_t *d_chunk_bits, const uint64_t *d_chunk_word_offset, const uint32_t *d_sub_off,
                    size_t n, size_t chunk, uint8_t *d_out, uint32_t *d_status, void *stream) {
    pc_status st = check_decode_args(d_cb, d_payload, d_chunk_bits, d_chunk_word_offset, d_sub_off, n, chunk,
                                     d_out, d_status);
    if (st != PC_OK || n == 0) return st;
    return map_hip(pc::launch_decode(pc::kDecodeLut12, d_cb, d_payload, payload_words, d_chunk_bits,
                                     d_chunk_word_offset, d_sub_off, n, (uint32_t)chunk, d_out, d_status,
                                     static_cast<hipStream_t>(stream)));
}

pc_status pc_decode_qlc(const pc_codebook *d_cb, const uint32_t *d_payload, size_t payload_words,
                        const uint32_t *d_chunk_bits, const uint64_t *d_chunk_word_offset, const uint32_t *d_sub_off,
                        size_t n, size_t chunk, uint8_t *d_out, uint32_t *d_status, void *stream) {
    pc_status st = check_decode_args(d_cb, d_payload, d_chunk_bits, d_chunk_word_offset, d_sub_off, n, chunk,
                                     d_out, d_status);
    if (st != PC_OK || n == 0) return st;
    return map_hip(pc::launch_decode(pc::kDecodeQlc, d_cb, d_payload, payload_words, d_chunk_bits,
                                     d_chunk_word_offset, d_sub_off, n, (uint32_t)chunk, d_out, d_status,
                                     static_cast<hipStream_t>(stream)));
}

pc_status pc_histogram(const uint8_t *d_in, size_t n, uint64_t *d_counts, void *stream) {
    if (n == 0) return PC_OK;
    if (!d_in || !d_counts || !aligned(d_counts, 8)) return PC_ERR_INVALID_ARG;
    return map_hip(pc::launch_histogram(d_in, n, d_counts, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
