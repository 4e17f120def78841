// KV-cache append (plain and quantising into FP8) and block copy for gfx950.
//
// Append (supersilo.blog vLLM/PagedAttention summary, section "자기회귀 생성과
// KV 캐시"): each decode step stores the new token's K/V after the cached
// ones, i.e. at position L-1 of a sequence of (new) length L, which lives in
// slot (L-1) % block_size of the physical block its table names for logical
// block (L-1) / block_size.
//
// Copy (same page, section "블록 공유"; blog.aqudi.me section 3): a block
// shared by several sequences is copied before one of them writes to it.
// Swap (same page, section "적용 범위와 관련 연구"): blocks of preempted
// sequences move to a pool in pinned host memory and back; the same kernel
// does it, reading or writing host memory over the host link.
// A block image is contiguous in the [num_blocks][kv heads][block_size][D]
// pool, so the copy is one flat run of 16-byte pieces per pair.

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kCopyUnroll = 4;

// One thread per 16-byte piece of one (sequence, new token, kv head) row of
// K or of V. New token j of a sequence of (new) length L goes to position
// L - nq + j; positions below 0 are skipped.
__global__ __launch_bounds__(kThreads)
void append_kernel(const AppendParams a, long long total) {
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (t >= total) return;
    const int pieces = a.row_bytes / 16;
    const int piece = (int)(t % pieces);
    long long r = t / pieces;
    const int g = (int)(r % a.num_kv_heads);
    r /= a.num_kv_heads;
    const int j = (int)(r % a.num_queries);
    r /= a.num_queries;
    const int seq = (int)(r % a.num_seqs);
    const int which = (int)(r / a.num_seqs);      // 0: K, 1: V
    const int L = a.seq_lens[seq];
    const int pos = L - a.num_queries + j;
    if (L <= 0 || pos < 0) return;
    const int blk = pos >> a.log2_bs;
    if (blk >= a.max_blocks) {
        report_if(a.err, piece == 0, PKV_ERRBIT_APPEND);
        return;
    }
    const int phys = a.block_tables[(size_t)seq * a.max_blocks + blk];
    if (phys < 0 || phys >= a.num_blocks) {
        report_if(a.err, piece == 0, PKV_ERRBIT_APPEND);
        return;
    }
    const int slot = pos & ((1 << a.log2_bs) - 1);
    const size_t row = (((size_t)phys * a.num_kv_heads + g) << a.log2_bs) + (size_t)slot;
    const size_t dst = row * a.row_bytes + (size_t)piece * 16;
    const size_t src = (((size_t)seq * a.num_queries + j) * a.num_kv_heads + g) * a.row_bytes +
                       (size_t)piece * 16;
    const char* s = reinterpret_cast<const char*>(which ? a.v_new : a.k_new);
    char* d = reinterpret_cast<char*>(which ? a.v_pool : a.k_pool);
    // Non-temporal store: the attention walk reads these rows next, and
    // lines left dirty in the caches would be written back in the middle of
    // its read stream, which costs it more than the bytes (the appended rows
    // of 4 new tokens on the OPT-13B layer: walk 230.5 -> 224.0 us)
    __builtin_nontemporal_store(load16(s + src), reinterpret_cast<u32x4*>(d + dst));
}

// -- FP8 (OCP E4M3) quantisation for the FP8 append ----------------------
// The code nearest to y, ties to the even code; |y| >= 448 saturates to 448;
// NaN gives 0x7F. Integer rounding on the float32 bits, so the result does
// not depend on any conversion instruction's rounding mode.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t b = f2u(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t mag = b & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0x7fu;                       // NaN
    const float a = u2f(mag);
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0.015625f) {                                        // below 2^-6: steps of 2^-9
        // a * 512 is exact; round half to even (0..8; 8 is the code of 2^-6)
        return sign | (uint32_t)__builtin_rintf(a * 512.0f);
    }
    const uint32_t e = (mag >> 23) - 127u + 7u;                 // 1 .. 15
    const uint32_t mant = mag & 0x7fffffu;
    uint32_t r = mant >> 20;                                    // 3 kept bits
    const uint32_t rest = mant & 0xfffffu, half = 0x80000u;
    if (rest > half || (rest == half && (r & 1u))) ++r;        // a carry moves to e + 1
    return sign | ((e << 3) + r);
}

template <int NEW_BYTES>
__device__ __forceinline__ void load8_f32(const char* p, int new_dtype, float (&x)[8]) {
    if constexpr (NEW_BYTES == 4) {
        const u32x4 a = load16(p), b = load16(p + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = u2f(a[i]);
            x[4 + i] = u2f(b[i]);
        }
    } else {
        const u32x4 a = load16(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (new_dtype == PKV_F16) {
                x[2 * i] = lo_to_f32(F16{}, a[i]);
                x[2 * i + 1] = hi_to_f32(F16{}, a[i]);
            } else {
                x[2 * i] = lo_to_f32(BF16{}, a[i]);
                x[2 * i + 1] = hi_to_f32(BF16{}, a[i]);
            }
        }
    }
}

// One thread per 8 elements of one (sequence, new token, kv head) row of K
// or of V: 8 inputs -> 8 codes (one 8-byte store). New token j of a sequence
// of (new) length L goes to position L - nq + j; positions below 0 are skipped.
template <int NEW_BYTES>
__global__ __launch_bounds__(kThreads)
void append_fp8_kernel(const AppendFp8Params a, long long total) {
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (t >= total) return;
    const int groups = a.head_dim / 8;
    const int grp = (int)(t % groups);
    long long r = t / groups;
    const int g = (int)(r % a.num_kv_heads);
    r /= a.num_kv_heads;
    const int j = (int)(r % a.num_queries);
    r /= a.num_queries;
    const int seq = (int)(r % a.num_seqs);
    const int which = (int)(r / a.num_seqs);      // 0: K, 1: V
    const int L = a.seq_lens[seq];
    const int pos = L - a.num_queries + j;
    if (L <= 0 || pos < 0) return;
    const int blk = pos >> a.log2_bs;
    if (blk >= a.max_blocks) {
        report_if(a.err, grp == 0, PKV_ERRBIT_APPEND);
        return;
    }
    const int phys = a.block_tables[(size_t)seq * a.max_blocks + blk];
    if (phys < 0 || phys >= a.num_blocks) {
        report_if(a.err, grp == 0, PKV_ERRBIT_APPEND);
        return;
    }
    const int slot = pos & ((1 << a.log2_bs) - 1);
    const float scale = (which ? a.v_scales : a.k_scales)[g];
    const char* src = reinterpret_cast<const char*>(which ? a.v_new : a.k_new) +
                      ((((size_t)seq * a.num_queries + j) * a.num_kv_heads + g) * a.head_dim +
                       (size_t)grp * 8) * NEW_BYTES;
    float x[8];
    load8_f32<NEW_BYTES>(src, a.new_dtype, x);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo |= e4m3_encode(x[i] / scale) << (8 * i);
        hi |= e4m3_encode(x[4 + i] / scale) << (8 * i);
    }
    const size_t row = (((size_t)phys * a.num_kv_heads + g) << a.log2_bs) + (size_t)slot;
    uint8_t* dst = (which ? a.v_pool : a.k_pool) + row * a.head_dim + (size_t)grp * 8;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    // non-temporal for the reason given in append_kernel
    __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(dst));
}

// Grid: chunks_per_block * num_pairs * 2 workgroups; each moves
// kThreads * kCopyUnroll pieces of one block image of K or of V from the
// source pool to the destination pool (the same pool for copy-on-write).
__global__ __launch_bounds__(kThreads)
void copy_blocks_kernel(const CopyParams a, int chunks_per_block) {
    const int chunk = blockIdx.x % chunks_per_block;
    const int r = blockIdx.x / chunks_per_block;
    const int pair = r >> 1;
    const int which = r & 1;
    const int src = a.mapping[2 * pair];
    const int dst = a.mapping[2 * pair + 1];
    if (src < 0 || src >= a.src_num_blocks || dst < 0 || dst >= a.dst_num_blocks) {
        report_if(a.err, threadIdx.x == 0 && chunk == 0, PKV_ERRBIT_COPY);
        return;
    }
    const char* s = reinterpret_cast<const char*>(which ? a.src_v : a.src_k) +
                    (size_t)src * a.block_bytes;
    char* d = reinterpret_cast<char*>(which ? a.dst_v : a.dst_k) + (size_t)dst * a.block_bytes;
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
        if (p < pieces)   // non-temporal for the reason given in append_kernel
            __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + p * 16));
    }
}

}  // namespace

hipError_t launch_append(const AppendParams& a, hipStream_t stream) {
    const long long total = 2LL * a.num_seqs * a.num_queries * a.num_kv_heads * (a.row_bytes / 16);
    if (total == 0) return hipSuccess;
    const long long blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, total);
    return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendFp8Params& a, hipStream_t stream) {
    const long long total = 2LL * a.num_seqs * a.num_queries * a.num_kv_heads * (a.head_dim / 8);
    if (total == 0) return hipSuccess;
    const long long blocks = (total + kThreads - 1) / kThreads;
    if (a.new_dtype == PKV_F32)
        hipLaunchKernelGGL((append_fp8_kernel<4>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           a, total);
    else
        hipLaunchKernelGGL((append_fp8_kernel<2>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           a, total);
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
