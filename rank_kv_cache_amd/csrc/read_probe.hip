// Streaming-read probe: the read bandwidth a plain kernel reaches on this GPU, the practical ceiling
// that the decode's bandwidth (also a read-only stream of the caches) is compared to. Every
// workgroup of 8 waves reads one contiguous chunk with 16-byte loads, eight loads in flight per
// lane, and folds what it read (XOR) into one word, so no load can be left out.
#include "lra_device.h"
#include "lra_kernels.h"

namespace lra {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ x, int64_t per, uint32_t* out) {
    const uint4* p = x + per * int64_t(blockIdx.x);
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < per; i += int64_t(kProbeThreads) * kProbeUnroll) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + int64_t(u) * kProbeThreads;
            v[u] = j < per ? p[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // fold the workgroup: lanes, then waves through LDS
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), o));
    __shared__ uint32_t red[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t f = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / 64; ++w) f ^= red[w];
        out[blockIdx.x] = f;
    }
}

}  // namespace

hipError_t launch_read_probe(const void* x, int64_t bytes, int n_workgroups, uint32_t* out, hipStream_t stream) {
    const int64_t per = bytes / 16 / n_workgroups;
    hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(n_workgroups)), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(x), per, out);
    return hipGetLastError();
}

}  // namespace lra
