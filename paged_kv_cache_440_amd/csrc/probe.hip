// Memory-system reference kernels (declared in include/pkv_probe.h): a
// read-only stream that gives the practical HBM read ceiling, a plain copy of
// known size for scaling traffic counters, and a gather of exactly the K/V
// rows a decode launch reads (the ceiling of the paged access pattern). All
// read with the non-temporal 16-byte loads the attention kernels use for K/V.

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

// -- paged gather: the K/V rows a decode launch reads, and nothing else -------
struct GatherParams {
    const char* k_pool;
    const char* v_pool;
    const int32_t* tables;
    const int32_t* lens;
    uint32_t* sink;
    int max_blocks, num_seqs, num_kv_heads, row_bytes, log2_bs, num_blocks, waves;
};

constexpr int kGatherUnit = 32;           // tokens per unit of the equal split
constexpr int kGatherWavesPerGroup = 4;

__device__ __forceinline__ long long gather_scan(long long x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ __forceinline__ int gather_units(const GatherParams& a, int i) {
    const int L = a.lens[i];
    return L > 0 ? (L + kGatherUnit - 1) / kGatherUnit : 0;
}

// Wave w of `waves` takes the w-th of `waves` equal runs of the 32-token
// units of all (sequence, kv head) segments laid end to end, and reads every
// K and V row of its run through the block table: lane l loads 16-byte piece
// l % LPT of token l / LPT of a TPL-token group (one wave load = TPL whole
// rows, consecutive bytes of one block), NL groups of K and NL of V per
// round, with non-temporal loads. Rows at or past a range's end are not
// loaded (exec-masked). The XOR of everything read goes to sink[w].
template <int LPT, int NL>
__global__ __launch_bounds__(64 * kGatherWavesPerGroup)
void probe_gather_kernel(const GatherParams a) {
    constexpr int TPL = 64 / LPT, CH = TPL * NL;
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kGatherWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.waves) return;
    long long total = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
        const int i = b0 + lane;
        total += __shfl(gather_scan(i < a.num_seqs ? gather_units(a, i) : 0), 63, 64);
    }
    total *= a.num_kv_heads;
    const long long q = (total + a.waves - 1) / a.waves;
    const long long u0 = (long long)w * q, u1 = u0 + q < total ? u0 + q : total;
    uint32_t x = 0;
    long long base = 0;
    int seq = a.num_seqs;
    if (u0 < u1) {
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int i = b0 + lane;
            const long long span = i < a.num_seqs ? (long long)a.num_kv_heads * gather_units(a, i) : 0;
            const long long incl = gather_scan(span);
            const unsigned long long past = __ballot(base + incl > u0);
            if (past) {
                const int j = __builtin_ctzll(past);
                seq = b0 + j;
                base += __shfl(incl - span, j, 64);
                break;
            }
            base += __shfl(incl, 63, 64);
        }
    }
    const int bs_mask = (1 << a.log2_bs) - 1;
    const size_t tile = (size_t)a.row_bytes << a.log2_bs;
    const size_t blk_stride = (size_t)a.num_kv_heads * tile;
    const int tok = lane / LPT, piece = lane % LPT;
    long long u = u0;
    while (u < u1 && seq < a.num_seqs) {
        const int L = a.lens[seq];
        const int nu = L > 0 ? (L + kGatherUnit - 1) / kGatherUnit : 0;
        if (nu == 0) { ++seq; continue; }
        const int g = (int)((u - base) / nu);
        const long long seg0 = base + (long long)g * nu, seg1 = seg0 + nu;
        const int k0 = (int)(u - seg0);
        const int k1 = (int)((u1 < seg1 ? u1 : seg1) - seg0);
        const int t_stop = k1 * kGatherUnit < L ? k1 * kGatherUnit : L;
        const int* trow = a.tables + (size_t)seq * a.max_blocks;
        int nblk = (L + bs_mask) >> a.log2_bs;
        nblk = nblk < a.max_blocks ? nblk : a.max_blocks;   // never read past the table row
        for (int w0 = k0 * kGatherUnit; w0 < t_stop;) {
            const int fb = w0 >> a.log2_bs;
            const int win_end = (fb + 64) << a.log2_bs;
            const int w_end = win_end < t_stop ? win_end : t_stop;
            int tv = fb + lane < nblk ? trow[fb + lane] : 0;
            tv = (uint32_t)tv < (uint32_t)a.num_blocks ? tv : a.num_blocks - 1;
            const int last_group = ((w_end - 1) / TPL) * TPL;
            for (int c = w0; c < w_end; c += CH) {
                u32x4 kr[NL], vr[NL];
#pragma unroll
                for (int j = 0; j < NL; ++j) {
                    int tg = c + j * TPL;
                    const bool live = tg + tok < w_end;
                    tg = tg < last_group ? tg : last_group;      // keep the lookup in the window
                    const uint32_t p = (uint32_t)__builtin_amdgcn_readlane(tv, (tg >> a.log2_bs) - fb);
                    const size_t off = (size_t)p * blk_stride + (size_t)g * tile +
                                       (size_t)(((tg & bs_mask) + tok) * a.row_bytes + piece * 16);
                    kr[j] = u32x4{0u, 0u, 0u, 0u};
                    vr[j] = u32x4{0u, 0u, 0u, 0u};
                    if (live) {
                        kr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k_pool + off));
                        vr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v_pool + off));
                    }
                }
#pragma unroll
                for (int j = 0; j < NL; ++j) x ^= kr[j][0] ^ kr[j][3] ^ vr[j][1] ^ vr[j][2];
            }
            w0 = w_end;
        }
        u = seg0 + k1;
        if (g == a.num_kv_heads - 1 && u == seg1) {
            base = u;
            ++seq;
        }
    }
    // fold the wave's lanes and store one word per wave (a vector store)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if (lane == 0) a.sink[w] = x;
}

// The same rows as probe_gather_kernel, split the same way, read with the
// matrix-core walker's load shapes (its operand layouts), a chunk of 32
// tokens at a time: K as two 16-token tiles, each wave load taking 16 bytes
// at byte 64 s + 16 q of row n of the tile in lane (n, q) (RB / 64 loads per
// tile: 64 bytes of each of 16 rows per load); V as eight loads, lane (n, q)
// taking bytes VB n .. VB n + VB - 1 of token 16 h + 4 q + j (VB = RB / 16:
// each load covers 4 whole rows). CPR chunks are requested per round before
// any is used. As in the walker, rows at or past a range's end re-read the
// range's last row and block lookups go through the lanes' window of table
// entries (one per token tile for K, one per four tokens for V). Sink: the
// XOR of words 0 and 3 of every 16-byte K piece and of words 1 and 2 of
// every 16-byte V piece of the rows in range, as probe_gather_kernel.
template <int RB, int CPR>
__global__ __launch_bounds__(64 * kGatherWavesPerGroup)
void probe_gather_mfma_kernel(const GatherParams a) {
    constexpr int KS = RB / 64, VB = RB / 16;
    const int lane = threadIdx.x & 63, n = lane & 15, qd = lane >> 4;
    const int w = blockIdx.x * kGatherWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.waves) return;
    long long total = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
        const int i = b0 + lane;
        total += __shfl(gather_scan(i < a.num_seqs ? gather_units(a, i) : 0), 63, 64);
    }
    total *= a.num_kv_heads;
    const long long q = (total + a.waves - 1) / a.waves;
    const long long u0 = (long long)w * q, u1 = u0 + q < total ? u0 + q : total;
    uint32_t x = 0;
    long long base = 0;
    int seq = a.num_seqs;
    if (u0 < u1) {
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int i = b0 + lane;
            const long long span = i < a.num_seqs ? (long long)a.num_kv_heads * gather_units(a, i) : 0;
            const long long incl = gather_scan(span);
            const unsigned long long past = __ballot(base + incl > u0);
            if (past) {
                const int j = __builtin_ctzll(past);
                seq = b0 + j;
                base += __shfl(incl - span, j, 64);
                break;
            }
            base += __shfl(incl, 63, 64);
        }
    }
    const int bs_mask = (1 << a.log2_bs) - 1;
    const size_t tile = (size_t)a.row_bytes << a.log2_bs;
    const size_t blk_stride = (size_t)a.num_kv_heads * tile;
    long long u = u0;
    while (u < u1 && seq < a.num_seqs) {
        const int L = a.lens[seq];
        const int nu = L > 0 ? (L + kGatherUnit - 1) / kGatherUnit : 0;
        if (nu == 0) { ++seq; continue; }
        const int g = (int)((u - base) / nu);
        const long long seg0 = base + (long long)g * nu, seg1 = seg0 + nu;
        const int k0 = (int)(u - seg0);
        const int k1 = (int)((u1 < seg1 ? u1 : seg1) - seg0);
        const int t_stop = k1 * kGatherUnit < L ? k1 * kGatherUnit : L;
        const int* trow = a.tables + (size_t)seq * a.max_blocks;
        int nblk = (L + bs_mask) >> a.log2_bs;
        nblk = nblk < a.max_blocks ? nblk : a.max_blocks;   // never read past the table row
        for (int w0 = k0 * kGatherUnit; w0 < t_stop;) {
            const int fb = w0 >> a.log2_bs;
            const int win_end = (fb + 64) << a.log2_bs;
            const int w_end = win_end < t_stop ? win_end : t_stop;
            int tv = fb + lane < nblk ? trow[fb + lane] : 0;
            tv = (uint32_t)tv < (uint32_t)a.num_blocks ? tv : a.num_blocks - 1;
            const int last = w_end - 1;
            // physical block of window block blk (per lane)
            auto phys = [&](int blk) -> size_t {
                return (size_t)(uint32_t)__builtin_amdgcn_ds_bpermute(blk << 2, tv);
            };
            for (int c = w0; c < w_end; c += CPR * kGatherUnit) {
                u32x4 kr[CPR][2][KS];
                u32x4 vr[CPR][8];
#pragma unroll
                for (int r = 0; r < CPR; ++r) {
                    const int c0 = c + r * kGatherUnit;
                    // as the walker: rows past the range end re-read its last
                    // row (in cache); their pieces are left out of the fold
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int row = c0 + 16 * t + n;
                        const int rc = row < w_end ? row : last;
                        const size_t off = phys((rc >> a.log2_bs) - fb) * blk_stride + (size_t)g * tile +
                                           (size_t)((rc & bs_mask) * a.row_bytes + 16 * qd);
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            kr[r][t][s] = __builtin_nontemporal_load(
                                reinterpret_cast<const u32x4*>(a.k_pool + off + 64 * s));
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // four aligned consecutive tokens share a block (bs >= 8)
                        const int tb = c0 + 16 * h + 4 * qd;
                        const int t0 = tb < last ? tb : last;
                        const size_t blk_off = phys((t0 >> a.log2_bs) - fb) * blk_stride +
                                               (size_t)g * tile + (size_t)(VB * n);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int tj = tb + j < last ? tb + j : last;
                            const char* pj = a.v_pool + blk_off + (size_t)((tj & bs_mask) * a.row_bytes);
                            if constexpr (VB == 16) {
                                vr[r][4 * h + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pj));
                            } else {
                                const u32x2 v2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pj));
                                // bytes 8n .. 8n+7: words 0, 1 (n even) or 2, 3 (n odd) of piece n/2
                                vr[r][4 * h + j] = (n & 1) ? u32x4{0u, 0u, v2[0], 0u}
                                                           : u32x4{0u, v2[1], 0u, 0u};
                            }
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < CPR; ++r) {
                    const int c0 = c + r * kGatherUnit;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bool live = c0 + 16 * t + n < w_end;
#pragma unroll
                        for (int s = 0; s < KS; ++s) x ^= live ? kr[r][t][s][0] ^ kr[r][t][s][3] : 0u;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const bool live = c0 + 16 * (j >> 2) + 4 * qd + (j & 3) < w_end;
                        x ^= live ? vr[r][j][1] ^ vr[r][j][2] : 0u;
                    }
                }
            }
            w0 = w_end;
        }
        u = seg0 + k1;
        if (g == a.num_kv_heads - 1 && u == seg1) {
            base = u;
            ++seq;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if (lane == 0) a.sink[w] = x;
}

template <int RB>
hipError_t launch_gather_mfma(const GatherParams& a, int chunks, hipStream_t stream) {
    const dim3 grid((a.waves + kGatherWavesPerGroup - 1) / kGatherWavesPerGroup);
    const dim3 block(64 * kGatherWavesPerGroup);
    switch (chunks) {
        case 1: hipLaunchKernelGGL((probe_gather_mfma_kernel<RB, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((probe_gather_mfma_kernel<RB, 2>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int LPT>
hipError_t launch_gather(const GatherParams& a, int loads, hipStream_t stream) {
    const dim3 grid((a.waves + kGatherWavesPerGroup - 1) / kGatherWavesPerGroup);
    const dim3 block(64 * kGatherWavesPerGroup);
    switch (loads) {
        case 2: hipLaunchKernelGGL((probe_gather_kernel<LPT, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((probe_gather_kernel<LPT, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((probe_gather_kernel<LPT, 8>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace pkv

namespace {

// Checks and parameters shared by both gather probes: PKV_OK and a filled
// `a`, or the status to return.
int gather_params(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                  int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_kv_heads,
                  int row_bytes, int block_size, int num_blocks, int waves, uint32_t* sink,
                  pkv::GatherParams& a) {
    int log2_bs = -1;
    for (int s = 3; s <= 8; ++s)
        if (block_size == (1 << s)) log2_bs = s;
    if (!k_pool || !v_pool || !block_tables || !seq_lens || !sink || num_seqs <= 0 ||
        num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || waves <= 0 ||
        !pkv::aligned16(k_pool) || !pkv::aligned16(v_pool))
        return PKV_ERR_INVALID;
    if ((row_bytes != 128 && row_bytes != 256) || log2_bs < 0) return PKV_ERR_UNSUPPORTED;
    if ((long long)num_seqs * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
    a = pkv::GatherParams{};
    a.k_pool = reinterpret_cast<const char*>(k_pool);
    a.v_pool = reinterpret_cast<const char*>(v_pool);
    a.tables = block_tables;
    a.lens = seq_lens;
    a.sink = sink;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.row_bytes = row_bytes;
    a.log2_bs = log2_bs;
    a.num_blocks = num_blocks;
    a.waves = waves;
    return PKV_OK;
}

}  // namespace

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

int pkv_probe_gather_mfma(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                          int num_kv_heads, int row_bytes, int block_size, int num_blocks,
                          int waves, int chunks_per_round, uint32_t* sink, void* stream) {
    pkv::GatherParams a;
    const int st = gather_params(k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens,
                                 num_seqs, num_kv_heads, row_bytes, block_size, num_blocks, waves,
                                 sink, a);
    if (st != PKV_OK) return st;
    if (chunks_per_round != 1 && chunks_per_round != 2) return PKV_ERR_UNSUPPORTED;
    const hipError_t err =
        row_bytes == 128 ? pkv::launch_gather_mfma<128>(a, chunks_per_round, (hipStream_t)stream)
                         : pkv::launch_gather_mfma<256>(a, chunks_per_round, (hipStream_t)stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_probe_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                     int num_kv_heads, int row_bytes, int block_size, int num_blocks, int waves,
                     int loads_per_round, uint32_t* sink, void* stream) {
    pkv::GatherParams a;
    const int st = gather_params(k_pool, v_pool, block_tables, max_blocks_per_seq, seq_lens,
                                 num_seqs, num_kv_heads, row_bytes, block_size, num_blocks, waves,
                                 sink, a);
    if (st != PKV_OK) return st;
    if (!(loads_per_round == 2 || loads_per_round == 4 || loads_per_round == 8))
        return PKV_ERR_UNSUPPORTED;
    const hipError_t err = row_bytes == 128 ? pkv::launch_gather<8>(a, loads_per_round, (hipStream_t)stream)
                                            : pkv::launch_gather<16>(a, loads_per_round, (hipStream_t)stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
