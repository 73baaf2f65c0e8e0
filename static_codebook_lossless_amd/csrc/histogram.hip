// Byte histogram on the device: the statistics step that precedes the
// codebook build ("Single-Stage Huffman Encoder for ML Compression",
// abstract: the fixed codebook comes from the average distribution of
// previous batches).  HBM-bound: each input byte is read once.
//
// Every group of 4 lanes counts into its own 256-bin LDS copy (16 per wave):
// same-address atomics then come from at most 4 lanes, and the copies are
// 257 words apart so that one bin of different copies sits in different
// banks.  Each lane keeps 8 loads of 16 bytes in flight, non-temporal (the
// bytes are read once).  A workgroup adds its 64 copies into the caller's
// 64-bit bins at the end.
#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kWaves = kThreads / 64;
constexpr uint32_t kCopies = 16;  // per wave
constexpr uint32_t kStride = 257;
constexpr int kUnroll = 8;
// 66 KB of LDS each: two resident workgroups per CU on 256 CUs
constexpr uint64_t kMaxBlocks = 512;

__device__ __forceinline__ void count16(uint32_t *my, const uint4 &x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        atomicAdd(&my[w[k] & 0xFF], 1u);
        atomicAdd(&my[(w[k] >> 8) & 0xFF], 1u);
        atomicAdd(&my[(w[k] >> 16) & 0xFF], 1u);
        atomicAdd(&my[w[k] >> 24], 1u);
    }
}

__global__ __launch_bounds__(kThreads) void histogram_kernel(const uint8_t *__restrict__ in, uint64_t n,
                                                             uint64_t head, uint64_t *__restrict__ counts) {
    __shared__ uint32_t bins[kWaves * kCopies * kStride];
    const uint32_t tid = threadIdx.x, wave = tid >> 6;
    for (uint32_t i = tid; i < kWaves * kCopies * kStride; i += kThreads) bins[i] = 0;
    __syncthreads();
    uint32_t *my = bins + (wave * kCopies + (tid & 63) / (64 / kCopies)) * kStride;
    // unaligned head bytes and the tail are counted by the first workgroup
    if (blockIdx.x == 0) {
        for (uint64_t i = tid; i < head; i += kThreads) atomicAdd(&my[in[i]], 1u);
        const uint64_t body_end = head + ((n - head) & ~15ull);
        for (uint64_t i = body_end + tid; i < n; i += kThreads) atomicAdd(&my[in[i]], 1u);
    }
    const uint4 *q = reinterpret_cast<const uint4 *>(in + head);
    const uint64_t nq = (n - head) / 16;
    const uint64_t step = (uint64_t)gridDim.x * kThreads;
    uint64_t i = (uint64_t)blockIdx.x * kThreads + tid;
    for (; i + (kUnroll - 1) * step < nq; i += kUnroll * step) {
        uint4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = load_stream16(q + i + u * step);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) count16(my, x[u]);
    }
    for (; i < nq; i += step) count16(my, q[i]);
    __syncthreads();
    uint64_t s = 0;
    for (uint32_t c = 0; c < kWaves * kCopies; ++c) s += bins[c * kStride + tid];
    if (s) atomicAdd(reinterpret_cast<unsigned long long *>(&counts[tid]), (unsigned long long)s);
}

}  // namespace

hipError_t launch_histogram(const uint8_t *in, uint64_t n, uint64_t *counts, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint64_t mis = (uint64_t)(reinterpret_cast<uintptr_t>(in) & 15);
    uint64_t head = mis ? 16 - mis : 0;
    if (head > n) head = n;
    const uint64_t nq = (n - head) / 16;
    // a u32 LDS bin per workgroup must not overflow: <= 2^30 bytes each
    uint64_t blocks = (nq + kThreads * 16 - 1) / (kThreads * 16);
    const uint64_t min_blocks = (n >> 30) + 1;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < min_blocks) blocks = min_blocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(histogram_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, in, n, head, counts);
    return hipGetLastError();
}

}  // namespace pc
