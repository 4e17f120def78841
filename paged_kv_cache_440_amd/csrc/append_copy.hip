// KV-cache append and block copy for gfx950: bit-exact 16-byte moves.
//
// Append (supersilo.blog vLLM/PagedAttention summary, section "자기회귀 생성과
// KV 캐시"): each decode step stores the new token's K/V after the cached
// ones, i.e. at position L-1 of a sequence of (new) length L, which lives in
// slot (L-1) % block_size of the physical block its table names for logical
// block (L-1) / block_size.
//
// Copy (same page, section "블록 공유"; blog.aqudi.me section 3): a block
// shared by several sequences is copied before one of them writes to it.
// A block image is contiguous in the [num_blocks][kv heads][block_size][D]
// pool, so the copy is one flat run of 16-byte pieces per pair.

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kCopyUnroll = 4;

// One thread per 16-byte piece of one (sequence, kv head) row of K or of V.
__global__ __launch_bounds__(kThreads)
void append_kernel(const AppendParams a, long long total) {
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (t >= total) return;
    const int pieces = a.row_bytes / 16;
    const int piece = (int)(t % pieces);
    long long r = t / pieces;
    const int g = (int)(r % a.num_kv_heads);
    r /= a.num_kv_heads;
    const int seq = (int)(r % a.num_seqs);
    const int which = (int)(r / a.num_seqs);      // 0: K, 1: V
    const int L = a.seq_lens[seq];
    if (L <= 0) return;
    const int pos = L - 1;
    const int blk = pos >> a.log2_bs;
    if (blk >= a.max_blocks) return;
    const int phys = a.block_tables[(size_t)seq * a.max_blocks + blk];
    if (phys < 0 || phys >= a.num_blocks) return;
    const int slot = pos & ((1 << a.log2_bs) - 1);
    const size_t row = (((size_t)phys * a.num_kv_heads + g) << a.log2_bs) + (size_t)slot;
    const size_t dst = row * a.row_bytes + (size_t)piece * 16;
    const size_t src = ((size_t)seq * a.num_kv_heads + g) * a.row_bytes + (size_t)piece * 16;
    const char* s = reinterpret_cast<const char*>(which ? a.v_new : a.k_new);
    char* d = reinterpret_cast<char*>(which ? a.v_pool : a.k_pool);
    store16(d + dst, load16(s + src));
}

// Grid: chunks_per_block * num_pairs * 2 workgroups; each moves
// kThreads * kCopyUnroll pieces of one block image of K or of V.
__global__ __launch_bounds__(kThreads)
void copy_blocks_kernel(const CopyParams a, int chunks_per_block) {
    const int chunk = blockIdx.x % chunks_per_block;
    const int r = blockIdx.x / chunks_per_block;
    const int pair = r >> 1;
    const int which = r & 1;
    const int src = a.mapping[2 * pair];
    const int dst = a.mapping[2 * pair + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
    char* pool = reinterpret_cast<char*>(which ? a.v_pool : a.k_pool);
    const char* s = pool + (size_t)src * a.block_bytes;
    char* d = pool + (size_t)dst * a.block_bytes;
    const long long pieces = a.block_bytes / 16;
    const long long base = (long long)chunk * kThreads * kCopyUnroll + threadIdx.x;
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const long long p = base + (long long)u * kThreads;
        if (p < pieces) v[u] = load16(s + p * 16);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const long long p = base + (long long)u * kThreads;
        if (p < pieces) store16(d + p * 16, v[u]);
    }
}

}  // namespace

hipError_t launch_append(const AppendParams& a, hipStream_t stream) {
    const long long total = 2LL * a.num_seqs * a.num_kv_heads * (a.row_bytes / 16);
    if (total == 0) return hipSuccess;
    const long long blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, total);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyParams& a, hipStream_t stream) {
    if (a.num_pairs == 0) return hipSuccess;
    const long long pieces = a.block_bytes / 16;
    const int chunks = (int)((pieces + kThreads * kCopyUnroll - 1) / (kThreads * kCopyUnroll));
    const long long blocks = (long long)chunks * a.num_pairs * 2;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                       chunks);
    return hipGetLastError();
}

}  // namespace pkv
