// Counter calibration: a copy made of the coder kernels' own memory
// instructions (16-byte non-temporal loads and stores), so that the bytes
// the hardware counters report for a known transfer can scale the counts
// taken on the coder kernels.  Not part of the coding method.
#include "pc_internal.h"

namespace pc {
namespace {

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         uint64_t nq) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace
}  // namespace pc

extern "C" pc_status pc_traffic_probe(const void *d_src, void *d_dst, size_t bytes, void *stream) {
    if (bytes == 0) return PC_OK;
    if (!d_src || !d_dst || bytes % 16 || (uintptr_t)d_src % 16 || (uintptr_t)d_dst % 16) return PC_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PC_ERR_HIP;
    const uint64_t nq = bytes / 16;
    uint64_t grid = (uint64_t)cus * 8;
    if (grid > (nq + 255) / 256) grid = (nq + 255) / 256;
    hipLaunchKernelGGL(pc::probe_copy_kernel, dim3((uint32_t)grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const pc::u32x4 *>(d_src), static_cast<pc::u32x4 *>(d_dst), nq);
    return hipGetLastError() == hipSuccess ? PC_OK : PC_ERR_HIP;
}
