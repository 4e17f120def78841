// Memory-system reference kernels (declared in include/pkv_probe.h): a
// read-only stream that gives the practical HBM read ceiling, and a plain
// copy of known size for scaling traffic counters. Both read with the
// non-temporal 16-byte loads the attention kernels use for K/V.

#include "pkv_probe.h"
#include "pkv_device.hpp"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;                 // 16-byte pieces per thread per round
constexpr long long kProbeGroupPieces = (long long)kProbeThreads * kProbeUnroll;
constexpr unsigned kProbeMaxGroups = 256 * 32;  // 32 workgroups per compute unit

unsigned probe_groups(long long pieces) {
    const long long want = (pieces + kProbeGroupPieces - 1) / kProbeGroupPieces;
    return (unsigned)(want < (long long)kProbeMaxGroups ? want : (long long)kProbeMaxGroups);
}

// Workgroup w reads rounds w, w + G, w + 2G, ... of kProbeGroupPieces pieces;
// inside a round, thread t reads pieces t, t + 256, ... (each load
// instruction covers 4 KB of consecutive bytes).
__global__ __launch_bounds__(kProbeThreads)
void probe_read_kernel(const u32x4* __restrict__ src, long long pieces, uint32_t* sink) {
    uint32_t x = 0;
    const long long stride = (long long)gridDim.x * kProbeGroupPieces;
    for (long long base = (long long)blockIdx.x * kProbeGroupPieces; base < pieces;
         base += stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const long long p = base + (long long)u * kProbeThreads + threadIdx.x;
            v[u] = p < pieces ? __builtin_nontemporal_load(src + p) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    // fold the workgroup's values into one word through LDS
    __shared__ uint32_t red[kProbeThreads];
    red[threadIdx.x] = x;
    __syncthreads();
    for (int s = kProbeThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kProbeThreads)
void probe_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, long long pieces) {
    const long long stride = (long long)gridDim.x * kProbeGroupPieces;
    for (long long base = (long long)blockIdx.x * kProbeGroupPieces; base < pieces;
         base += stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const long long p = base + (long long)u * kProbeThreads + threadIdx.x;
            if (p < pieces) v[u] = __builtin_nontemporal_load(src + p);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const long long p = base + (long long)u * kProbeThreads + threadIdx.x;
            if (p < pieces) dst[p] = v[u];
        }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pkv

extern "C" {

size_t pkv_probe_read_sink_words(size_t bytes) {
    if (bytes == 0 || bytes % 16 != 0) return 0;
    return pkv::probe_groups((long long)(bytes / 16));
}

int pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !pkv::aligned16(src))
        return PKV_ERR_INVALID;
    const long long pieces = (long long)(bytes / 16);
    hipLaunchKernelGGL(pkv::probe_read_kernel, dim3(pkv::probe_groups(pieces)),
                       dim3(pkv::kProbeThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<const pkv::u32x4*>(src), pieces, sink);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 || !pkv::aligned16(src) ||
        !pkv::aligned16(dst))
        return PKV_ERR_INVALID;
    const long long pieces = (long long)(bytes / 16);
    hipLaunchKernelGGL(pkv::probe_copy_kernel, dim3(pkv::probe_groups(pieces)),
                       dim3(pkv::kProbeThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<pkv::u32x4*>(dst),
                       reinterpret_cast<const pkv::u32x4*>(src), pieces);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
