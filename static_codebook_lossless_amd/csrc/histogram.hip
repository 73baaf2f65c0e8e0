// Byte histogram on the device: the statistics step that precedes the
// codebook build ("Single-Stage Huffman Encoder for ML Compression",
// abstract: the fixed codebook comes from the average distribution of
// previous batches).  HBM-bound: each input byte is read once.
//
// Every wave counts into its own 256-bin LDS copy (fewer same-address
// atomics than one shared copy); a workgroup adds its copies into the
// caller's 64-bit bins at the end.
#include "pc_internal.h"

namespace pc {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void histogram_kernel(const uint8_t *__restrict__ in, uint64_t n,
                                                             uint64_t head, uint64_t *__restrict__ counts) {
    __shared__ uint32_t bins[kWaves][256];
    const uint32_t tid = threadIdx.x, wave = tid >> 6;
    for (uint32_t i = tid; i < kWaves * 256; i += kThreads) (&bins[0][0])[i] = 0;
    __syncthreads();
    uint32_t *my = bins[wave];
    // unaligned head bytes and the tail are counted by the first workgroup
    if (blockIdx.x == 0) {
        for (uint64_t i = tid; i < head; i += kThreads) atomicAdd(&my[in[i]], 1u);
        const uint64_t body_end = head + ((n - head) & ~15ull);
        for (uint64_t i = body_end + tid; i < n; i += kThreads) atomicAdd(&my[in[i]], 1u);
    }
    const uint4 *q = reinterpret_cast<const uint4 *>(in + head);
    const uint64_t nq = (n - head) / 16;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + tid; i < nq; i += (uint64_t)gridDim.x * kThreads) {
        const uint4 x = q[i];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&my[w[k] & 0xFF], 1u);
            atomicAdd(&my[(w[k] >> 8) & 0xFF], 1u);
            atomicAdd(&my[(w[k] >> 16) & 0xFF], 1u);
            atomicAdd(&my[w[k] >> 24], 1u);
        }
    }
    __syncthreads();
    uint64_t s = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; ++w) s += bins[w][tid];
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
    if (blocks > 2048) blocks = 2048;
    if (blocks < min_blocks) blocks = min_blocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(histogram_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, in, n, head, counts);
    return hipGetLastError();
}

}  // namespace pc
