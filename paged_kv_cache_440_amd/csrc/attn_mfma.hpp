// Matrix-core walker for paged attention (gfx950), 16-bit K/V, head_dim 128.
// It serves every case where several query columns read the same K/V: 4 or
// 8 query heads per kv head (grouped-query decode), several new tokens per
// sequence (multi-query attention, each column with its own causal limit)
// and the samples of a prompt over their shared blocks (grouped decode).
// With N columns every K/V byte feeds 2N flops; on the vector units that is
// ALU-bound for N = 8, so both contractions of a 32-token chunk run as
// v_mfma_f32_16x16x32_{bf16,f16} (fp32 accumulation):
//
//   S^T = K . Q^T     M = 16 tokens (two tiles), N = 16 columns (the unused
//                     ones zero), K = 128 dims in four steps of 32.
//   O^T += V^T . P^T  M = 16 dims (eight tiles), N = 16 columns,
//                     K = the chunk's 32 tokens.
//
// Operand layouts (16x16x32): lane l, with n = l % 16 and q = l / 16, holds
// row n of A and column n of B for the 8 k-slots of group q; the 16x16
// result holds rows 4q .. 4q+3 of column n. The order of the k-slots inside
// a contraction is free as long as A and B agree, and the rows of V^T may be
// any permutation of the dims as long as the output is written accordingly:
//   * QK, step s: k-slots of group q are dims 32s + 8q .. +7, i.e. 16 bytes
//     at byte 64s + 16q of a token row -- K rows (A) and q rows (B) load
//     straight from memory;
//   * the S^T result gives lane (n, q) head n's scores of tokens 4q + i
//     (tile 0) and 16 + 4q + i (tile 1), i = 0..3. These eight tokens, in
//     that order, are the k-slots of group q of PV, so P^T (B) is the
//     lane's own softmax weights, no data movement;
//   * V^T (A) row n of dim tile c is dim 8n + c. Lane (n, q) loads the 16
//     bytes at dims 8n .. 8n+7 of each of its eight tokens (each wave load
//     covers four whole 256-byte rows) and transposes that 8x8 block of
//     16-bit values in registers: element c of the eight pieces forms the
//     operand of tile c;
//   * O^T tile c, row 4q + i, column n is head n, dim 8(4q + i) + c: lane
//     (n, q) ends with dims 32q .. 32q+31 of head n.
// The softmax of head n lives in the four lanes n, n+16, n+32, n+48: the
// chunk max is combined across them (permlane swaps), each keeps a partial
// sum, and the sums are added once at the end. P enters the matrix core as a
// 16-bit high part plus a 16-bit residual, two products per tile, so the
// weights keep about 16 significant bits.
//
// Masking: tokens at or past the range end (tail chunk only) get score -inf
// and their V pieces are zeroed by select before the products; a token past
// a column's causal limit (multi-query) gets score -inf in that column only,
// and its V piece stays, since other columns see it.
//
// FP8 pools (FP8 = true; blog.aqudi.me "벤치마크가 다가 아니야! vLLM으로 보는
// LLM 추론 최적화", section 4: a lower-precision KV cache): K/V rows are 128
// bytes of E4M3 codes times a per-kv-head scale; S is then q's 16-bit type,
// and the codes are widened to it (exact: every E4M3 value is an fp16 and a
// bf16 value) on their way into the operands, two per
// v_cvt_scalef32_pk_{f16,bf16}_fp8. K: one 16-byte load of codes at byte
// 16q (64 + 16q) gives dims 16q .. 16q+15 (64 + ...), the k-slots of two
// steps, so step s = 2h + s' takes dims 64h + 16q + 8s' .. +7 (q is loaded
// in the same order). V: lane (n, q) loads the 8 codes of dims 8n .. 8n+7
// of each of its tokens (an 8-byte load). The K scale is folded into the
// score scale and the V scale into the output.
#pragma once

#include <type_traits>

#include "attn_common.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_16x16x32(BF16, const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(F16, const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 values -> two 16-bit values (round to nearest even) in one dword,
// x in the low half: one v_cvt_pk_{bf16,f16}_f32
__device__ __forceinline__ uint32_t pack16(BF16, float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
__device__ __forceinline__ uint32_t pack16(F16, float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
}
// the low / high 16-bit value of a dword, widened to fp32 (exact)
__device__ __forceinline__ float lo16(BF16, uint32_t h) { return u2f(h << 16); }
__device__ __forceinline__ float hi16(BF16, uint32_t h) { return u2f(h & 0xffff0000u); }
__device__ __forceinline__ float lo16(F16, uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float hi16(F16, uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
}

// E4M3 codes H*2, H*2 + 1 (bytes) of w as two packed 16-bit values of type S,
// in one gfx950 conversion (scale 1; every E4M3 value is exact in fp16 and bf16).
template <typename S, bool H>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w);
template <> __device__ __forceinline__ uint32_t fp8_pair<F16, false>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t fp8_pair<F16, true>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true));
}
template <> __device__ __forceinline__ uint32_t fp8_pair<BF16, false>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t fp8_pair<BF16, true>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
}

// The results of up to 16 columns leave a matrix-core walker as a 16 x 128
// tile: lane (n, q) holds dims 32q .. 32q+31 of column n (acc[c][i] is dim
// 32q + 8i + c). Stored straight from registers, every store instruction
// would touch 16 rows at once; the tile is transposed through the wave's own
// LDS slice instead, so that each instruction writes two whole rows (lanes
// 0-31 one row, 32-63 the next). `row` is this lane's column's destination
// row, `active` whether the column is written; store(row, piece, v) writes
// dims 4 piece .. 4 piece + 3 of a row.
// The calling wave's 8 KB slice of LDS (one allocation per kernel, however
// many call sites).
// (NW waves per workgroup; one allocation per kernel and NW.)
template <int NW>
__device__ __forceinline__ f32x4 (*wave_tile_at(int wave))[32] {
    __shared__ f32x4 tile[NW][16][32];
    return tile[wave];
}

template <class Store>
__device__ __forceinline__ void store_column_tile(f32x4 (*t)[32], const f32x4 (&acc)[8], float scale,
                                                  size_t row, bool active, Store store) {
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        t[n][8 * q + 2 * i] = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]} * scale;
        t[n][8 * q + 2 * i + 1] = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]} * scale;
    }
    // the wave's own LDS operations complete in order; only keep the compiler
    // from moving the reads above the writes
    __builtin_amdgcn_wave_barrier();
    const unsigned long long act = __ballot(active);
    const uint32_t row_lo = (uint32_t)row, row_hi = (uint32_t)(row >> 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = 2 * k + (lane >> 5);           // lane r holds column r (q = 0)
        const size_t rr = ((size_t)(uint32_t)__shfl((int)row_hi, r, 64) << 32) |
                          (uint32_t)__shfl((int)row_lo, r, 64);
        const f32x4 v = t[r][lane & 31];
        if ((act >> r) & 1) store(rr, lane & 31, v);
    }
    __builtin_amdgcn_wave_barrier();
}

// dims 4 piece .. 4 piece + 3 of output row `row` (16-byte or 8-byte store)
__device__ __forceinline__ void store_out4(void* out, int out_dtype, size_t row, int piece,
                                           f32x4 v) {
    const size_t idx = row * 128 + 4 * (size_t)piece;
    if (out_dtype == PKV_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = v;
        return;
    }
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        h[k] = out_dtype == PKV_F16 ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[k])
                                    : (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[k]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) =
        u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// LDS-pointer form the direct-to-LDS load takes (its destination is M0-based).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N of this wave's vector-memory operations are in
// flight (gfx9 s_waitcnt encoding; N < 16). The memory clobber keeps the
// compiler from moving LDS reads of data those loads write above the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt");
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The workgroup's K/V chunk buffers for shared walks (16 KB each): chunks
// are requested kSharedBufs - 1 ahead (four buffers measured no faster than
// three on MI355X). Once a shared walk is over they hold the waves' output
// tiles (8 KB per wave), so a workgroup needs 48 KB of LDS and two fit a
// compute unit with room to spare.
#ifndef PKV_SHARED_BUFS
#define PKV_SHARED_BUFS 3
#endif
constexpr int kSharedBufs = PKV_SHARED_BUFS;
static_assert(kSharedBufs >= 3 && kSharedBufs <= 4 && kSharedBufs * 16384 >= kWaves * 8192,
              "shared chunk buffers");
__device__ __forceinline__ char* shared_chunk(int b) {
    __shared__ __attribute__((aligned(16))) char bufs[kSharedBufs][16384];
    return bufs[b];
}

template <typename S, int G_, bool STREAM, bool FP8 = false, int NT = 1,
          int WPS = (NT > 1 ? 1 : 2), bool SHARED = false, int NWG = kWaves>
struct MfmaWalker {
    static constexpr bool kStream = STREAM;     // K/V load policy
    // persistent waves per compute unit in the balanced schedule: for 16-bit
    // K/V one per SIMD for grouped heads (measured on MI355X: 4 waves beat 8
    // by 3-5% at 4 and 8 query heads per kv head) and two per SIMD for
    // multi-query columns of one head (8 beat 4 by 9%); two per SIMD for FP8
    // pools (8 beat 4 and 12 on the long FP8 GQA layer)
    static constexpr int kBalancedWavesPerCU = FP8 ? 8 : (G_ >= 4 ? 4 : 8);
    static constexpr int D = 128, G = G_;
    static constexpr int ROW = FP8 ? 128 : 256;   // bytes of one K/V token row of one kv head
    static constexpr int QROW = 256;              // bytes of one q row (16-bit)
    static constexpr int KS = FP8 ? 2 : 4;        // 16-byte K loads per token row and lane
    static constexpr int CHUNK = 32;              // tokens per chunk
    // NT 16-column tiles per wave share each K/V chunk (chunked prefill);
    // WPS waves per SIMD bound the registers (one for several tiles whose
    // K/V chunks are held in registers; the shared walk, which holds them
    // in LDS, fits two tiles at two)
    static constexpr int kTiles = NT;
    static constexpr int kMinWavesPerSimd = WPS;
    static constexpr int kBalancedMinWavesPerSimd = WPS;
    // one lane's V piece of one token: 8 dims, 16-bit or codes
    using VPiece = std::conditional_t<FP8, u32x2, u32x4>;
    static_assert(S::bytes == 2 && G_ <= 16, "16-bit operands, at most 16 query heads");

    // per tile t of the wave (lane (n, q) holds column n of each)
    f32x4 acc[NT][8];   // O^T tiles: acc[t][c][i] = column n, dim 32q + 8i + c (unnormalised)
    float m[NT], l[NT]; // column n: running max (log2 units), this lane's partial sum
    u32x4 qb[NT][4];    // B operand of Q^T for the four k-steps
    int ncols[NT];      // real columns of tile t: the rest are zero padding
    int lim[NT];        // last token position column n of tile t may see (causal rule)
    size_t orow[NT];    // output row of column n of tile t
    float kfac, vscale; // FP8: the kv head's K and V scales

    int wb, tv;         // table window: lane j holds the physical id of block wb + j
    int pre_tv = 0;     // a window read ahead (preload_window)
    bool pre = false;
    const char* kbase;
    const char* vbase;
    const int* trow;
    size_t head_stride_bytes;
    size_t kvhead_off;
    int log2_bs, bs_mask, nblk_valid, max_phys;
    int* err;           // error word, or null
    int lane, n, q;
    int t_end;
    int mask_from;      // first position some column may not see

    __device__ __forceinline__ void init(int lane_id) {
        lane = lane_id;
        n = lane_id & 15;
        q = lane_id >> 4;
    }

    __device__ __forceinline__ void begin_table(const AttnParams& a, int table_seq, int g, int L) {
        log2_bs = a.log2_bs;
        bs_mask = (1 << a.log2_bs) - 1;
        nblk_valid = (L + bs_mask) >> a.log2_bs;
        max_phys = a.num_blocks;
        err = a.err;
        trow = a.block_tables + (size_t)table_seq * a.max_blocks;
        head_stride_bytes = (size_t)a.num_kv_heads * ((size_t)ROW << a.log2_bs);
        kvhead_off = (size_t)g * ((size_t)ROW << a.log2_bs);
        kbase = reinterpret_cast<const char*>(a.k_pool);
        vbase = reinterpret_cast<const char*>(a.v_pool);
        if constexpr (FP8) {
            kfac = a.k_scales[g];
            vscale = a.v_scales[g];
        }
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            m[t] = -__builtin_inff();
            l[t] = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Point the walker at the NT 16-column tiles NT*group .. of segment
    // (seq, g) of length L: column c = 16 tile + n = (query token c / G, head
    // g*G + c % G); a new token at position L - nq + j sees positions <= its own.
    __device__ __forceinline__ void begin(const AttnParams& a, int seq, int g, int L, int group = 0) {
        begin_table(a, seq, g, L);
        const int nq = a.num_queries, cols = nq * G;
        mask_from = L - nq + (16 * NT * group) / G + 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c0 = 16 * (NT * group + t);
            ncols[t] = cols - c0 < 16 ? cols - c0 : 16;       // <= 0 past the last column
            const bool active = n < ncols[t];
            const int c = active ? c0 + n : (c0 < cols ? c0 : cols - 1);
            lim[t] = active ? L - nq + c / G : L - 1;
            orow[t] = out_row(a, seq, g, c);
            load_q(a, orow[t], active, qb[t]);
        }
        reset();
    }

    // Columns taken from several sequences that share the blocks of tokens
    // [0, L) (the samples of one prompt): the tables of table_seq are walked,
    // this lane's column n reads q row qrow_idx if active and a zero row
    // otherwise, and every token of the walked range is visible to every
    // column.
    __device__ __forceinline__ void begin_columns(const AttnParams& a, int table_seq, int g, int L,
                                                  size_t qrow_idx, bool active) {
        static_assert(NT == 1, "one tile of sampled columns");
        begin_table(a, table_seq, g, L);
        ncols[0] = 16;
        lim[0] = L - 1;
        mask_from = L;
        orow[0] = qrow_idx;
        load_q(a, qrow_idx, active, qb[0]);
        reset();
    }

    // q row `row` as the B operand of the four k-steps (zero if !active):
    // step s covers dims 32s + 8q .. +7 (16-bit K/V) or 64(s/2) + 16q +
    // 8(s%2) .. +7 (FP8 codes), 16 consecutive bytes of q either way
    __device__ __forceinline__ void load_q(const AttnParams& a, size_t row, bool active,
                                           u32x4 (&b)[4]) {
        const char* qrow = reinterpret_cast<const char*>(a.q) + row * QROW;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int d0 = FP8 ? 64 * (s >> 1) + 16 * q + 8 * (s & 1) : 32 * s + 8 * q;
            b[s] = active ? load16(qrow + 2 * d0) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Entries of blocks 0 .. 63 of the next segment's table row (lane j: block
    // j), read ahead by the caller while the previous segment was walked; the
    // next load_window(0) takes them instead of reading the table.
    __device__ __forceinline__ void preload_window(int entries) {
        pre_tv = entries;
        pre = true;
    }

    __device__ __forceinline__ void load_window(int first_block) {
        wb = first_block;
        const bool valid = wb + lane < nblk_valid;
        tv = (pre && first_block == 0) ? (valid ? pre_tv : 0) : (valid ? trow[wb + lane] : 0);
        pre = false;
        // an entry of a valid block outside the pool is read clamped; say so
        report_wave(err, wb + lane < nblk_valid && (uint32_t)tv >= (uint32_t)max_phys,
                    PKV_ERRBIT_TABLE);
    }

    // physical block of window block blk (per lane, 0 <= blk < 64)
    __device__ __forceinline__ uint32_t phys(int blk) {
        const uint32_t p = (uint32_t)__builtin_amdgcn_ds_bpermute(blk << 2, tv);
        return p < (uint32_t)max_phys ? p : (uint32_t)(max_phys - 1);
    }

    // K: kt[t][s] = row (c0 + 16t + n), bytes 64s + 16q .. +15. Rows at or
    // past the range end (masked by softmax_pv) re-read the range's last row,
    // which is in cache, instead of fetching unrelated blocks from HBM.
    __device__ __forceinline__ void load_k(int c0, u32x4 (&kt)[2][KS]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            int tok = c0 + 16 * t + n;
            tok = tok < t_end ? tok : t_end - 1;
            const char* p = kbase + (size_t)phys((tok >> log2_bs) - wb) * head_stride_bytes +
                            kvhead_off + (uint32_t)((tok & bs_mask) * ROW + 16 * q);
#pragma unroll
            for (int s = 0; s < KS; ++s) kt[t][s] = load16_kv<STREAM>(p + 64 * s);
        }
    }

    // V: vt[4h + j] = row (c0 + 16h + 4q + j), dims 8n .. 8n+7 (16 bytes, or
    // 8 bytes of codes). Four aligned consecutive tokens never straddle a
    // block (bs >= 8). Rows at or past the range end (zeroed by softmax_pv)
    // re-read the range's last row, which lies in the same block as the first
    // of the four rows once that one is clamped too.
    __device__ __forceinline__ void load_v(int c0, VPiece (&vt)[8]) {
        const int last = t_end - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tb = c0 + 16 * h + 4 * q;
            const int t0 = tb < last ? tb : last;
            const char* p = vbase + (size_t)phys((t0 >> log2_bs) - wb) * head_stride_bytes +
                            kvhead_off + (uint32_t)(sizeof(VPiece) * n);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tj = tb + j < last ? tb + j : last;
                const char* pj = p + (uint32_t)((tj & bs_mask) * ROW);
                if constexpr (FP8)
                    vt[4 * h + j] = load8_kv<STREAM>(pj);
                else
                    vt[4 * h + j] = load16_kv<STREAM>(pj);
            }
        }
    }

    // A operand of k-step s for token tile t: the K row piece itself, or
    // (FP8) codes 8(s%2) .. +7 of load s/2 widened to S
    __device__ __forceinline__ static u32x4 k_operand(const u32x4 (&kt)[KS], int s) {
        if constexpr (FP8) {
            const uint32_t w0 = kt[s >> 1][2 * (s & 1)], w1 = kt[s >> 1][2 * (s & 1) + 1];
            return u32x4{fp8_pair<S, false>(w0), fp8_pair<S, true>(w0), fp8_pair<S, false>(w1),
                         fp8_pair<S, true>(w1)};
        } else {
            return kt[s];
        }
    }

    // Scores of the chunk for every tile: k-slot j of group q is token
    // 16 (j / 4) + 4q + j % 4. The K operands are built once for all tiles.
    __device__ __forceinline__ void scores(const u32x4 (&kt)[2][KS], float scale_log2,
                                           float (&sc)[NT][8]) {
        f32x4 s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) s0[t] = s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 a0 = k_operand(kt[0], s), a1 = k_operand(kt[1], s);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                s0[t] = mfma_16x16x32(S{}, a0, qb[t][s], s0[t]);
                s1[t] = mfma_16x16x32(S{}, a1, qb[t][s], s1[t]);
            }
        }
        const float f = FP8 ? scale_log2 * kfac : scale_log2;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[t][i] = s0[t][i] * f;
                sc[t][4 + i] = s1[t][i] * f;
            }
    }

    template <bool TAIL>
    __device__ __forceinline__ void softmax_pv(int c0, float (&sc)[NT][8], VPiece (&vt)[8]) {
        // Scores are masked by the range end and by column n's causal limit;
        // V pieces only by the range end: lane n's V piece holds dims
        // 8n .. 8n+7 of a token for every column, and a token past one
        // column's limit is still real data (its weight there is 0).
        if constexpr (TAIL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in_range = c0 + 16 * (j >> 2) + 4 * q + (j & 3) < t_end;
#pragma unroll
                for (int w = 0; w < (int)(sizeof(VPiece) / 4); ++w)
                    vt[j][w] = in_range ? vt[j][w] : 0u;
            }
        }
        // P^T of every tile as a 16-bit high part and the 16-bit residual
        u32x4 bhi[NT], blo[NT];
        float alpha[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            bool valid[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tok = c0 + 16 * (j >> 2) + 4 * q + (j & 3);
                valid[j] = !TAIL || (tok < t_end && tok <= lim[t]);
                if constexpr (TAIL) sc[t][j] = valid[j] ? sc[t][j] : -__builtin_inff();
            }
            float mx = sc[t][0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mx = __builtin_fmaxf(mx, sc[t][j]);
            mx = strided_max<16>(mx);
            // Outside masked chunks every token is valid and mx is finite. In a
            // masked chunk a column may have seen no valid token yet: then m_new
            // is -inf, every p is 0 and alpha (1) only multiplies zeros.
            const float m_new = __builtin_fmaxf(m[t], mx);
            alpha[t] = (TAIL && m_new == -__builtin_inff()) ? 1.f : fast_exp2(m[t] - m_new);
            float p[8], ps = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = (TAIL && !valid[j]) ? 0.f : fast_exp2(sc[t][j] - m_new);
                ps += p[j];
            }
            l[t] = l[t] * alpha[t] + ps;
            m[t] = m_new;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t h = pack16(S{}, p[2 * w], p[2 * w + 1]);
                bhi[t][w] = h;
                blo[t][w] = pack16(S{}, p[2 * w] - lo16(S{}, h), p[2 * w + 1] - hi16(S{}, h));
            }
        }
        // the eight V pieces as pairs of S values: hv[j][k] = dims 2k, 2k+1 of token j
        uint32_t hv[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (FP8) {
                hv[j][0] = fp8_pair<S, false>(vt[j][0]);
                hv[j][1] = fp8_pair<S, true>(vt[j][0]);
                hv[j][2] = fp8_pair<S, false>(vt[j][1]);
                hv[j][3] = fp8_pair<S, true>(vt[j][1]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) hv[j][k] = vt[j][k];
            }
        }
        // Rescale the accumulators only when some column's max grew: alpha is
        // exactly 1 otherwise (exp2 of 0), and past the first chunks the
        // running max rarely moves, so most chunks skip these 32 products per
        // tile (the result bits are the same either way). One test for all
        // the wave's tiles: a branch per tile cost registers and made the
        // two-tile prefill walk 9% slower on MI355X; this one is 1% faster.
        {
            bool grew = false;
#pragma unroll
            for (int t = 0; t < NT; ++t) grew = grew || alpha[t] != 1.f;
            if (__ballot(grew) != 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[t][c] = acc[t][c] * alpha[t];
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // V^T tile c: element c of the eight V pieces, token order as k-slots
            u32x4 av;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x = hv[2 * w][c >> 1], y = hv[2 * w + 1][c >> 1];
                // low halves of x and y (c even) or high halves (c odd), x's
                // first, in one byte permute (v_perm_b32: selector bytes 0-3
                // pick bytes of the second operand, 4-7 of the first)
                av[w] = __builtin_amdgcn_perm(y, x, (c & 1) ? 0x07060302u : 0x05040100u);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 o = mfma_16x16x32(S{}, av, bhi[t], acc[t][c]);
                acc[t][c] = mfma_16x16x32(S{}, av, blo[t], o);
            }
        }
    }

    // One buffer each for K and V: the next chunk's K is requested as soon as
    // the scores have consumed this chunk's K, the next V as soon as the
    // products have consumed this V, so about one chunk stays in flight per
    // wave with half the registers of a double buffer (two waves per SIMD).
    __device__ __forceinline__ void walk(int t_begin, int t_stop, float scale_log2) {
        u32x4 kt[2][KS];
        VPiece vt[8];
        float sc[NT][8];
        for (int w0 = t_begin; w0 < t_stop;) {
            const int first_block = w0 >> log2_bs;
            const int win_end = (first_block + 64) << log2_bs;
            const int w_end = win_end < t_stop ? win_end : t_stop;
            load_window(first_block);
            t_end = w_end;
            int c = w0;
            load_k(c, kt);
            load_v(c, vt);
            for (;;) {
                const int nx = c + CHUNK;
                scores(kt, scale_log2, sc);
                if (nx >= w_end) { softmax_pv<true>(c, sc, vt); break; }
                load_k(nx, kt);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
                if (nx > mask_from)                  // causal limits of several new tokens
                    softmax_pv<true>(c, sc, vt);
                else
                    softmax_pv<false>(c, sc, vt);
                load_v(nx, vt);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
                c = nx;
            }
            w0 = w_end;
        }
    }

    // -- shared walks: the four waves of a workgroup walk the same range ----
    // Each 32-token chunk is 16 wave-wide loads (8 of K: token tile t, k-step
    // s; 8 of V: half h, row j), laid out in LDS in the lanes' operand order:
    // load i puts lane l's 16 bytes at i * 1024 + 16 l. Wave w issues loads
    // 4w .. 4w+3 straight into LDS (global_load_lds, no registers held), two
    // chunks ahead of the compute; after a wait and a workgroup barrier every
    // wave reads the whole chunk back conflict-free and runs its own tiles.
    static constexpr int kSharedLoads = 4;        // per wave and chunk (16-bit K/V)

    __device__ __forceinline__ void issue_shared(int c0, int b, int wave) {
        static_assert(!FP8, "shared walks read 16-bit K/V");
        char* base = shared_chunk(b);
#pragma unroll
        for (int u = 0; u < kSharedLoads; ++u) {
            const int i = wave * kSharedLoads + u;       // wave-uniform
            const char* p;
            if (i < 8) {                                 // K: tile t = i / 4, step s = i % 4
                int tok = c0 + 16 * (i >> 2) + n;
                tok = tok < t_end ? tok : t_end - 1;
                p = kbase + (size_t)phys((tok >> log2_bs) - wb) * head_stride_bytes + kvhead_off +
                    (uint32_t)((tok & bs_mask) * ROW + 16 * q + 64 * (i & 3));
            } else {                                     // V: half h = (i - 8) / 4, row j
                const int last = t_end - 1;
                int tok = c0 + 16 * ((i - 8) >> 2) + 4 * q + (i & 3);
                tok = tok < last ? tok : last;
                p = vbase + (size_t)phys((tok >> log2_bs) - wb) * head_stride_bytes + kvhead_off +
                    (uint32_t)((tok & bs_mask) * ROW + 16 * n);
            }
            __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)(base + i * 1024), 16, 0, 0);
        }
    }

    __device__ __forceinline__ void read_shared(int b, u32x4 (&kt)[2][KS], VPiece (&vt)[8]) {
        const char* base = shared_chunk(b) + 16 * lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) kt[i >> 2][i & 3] = *reinterpret_cast<const u32x4*>(base + i * 1024);
#pragma unroll
        for (int j = 0; j < 8; ++j) vt[j] = *reinterpret_cast<const u32x4*>(base + (8 + j) * 1024);
    }

    // Tokens [t_begin, t_stop) for this wave's tiles, the chunks shared with
    // the other three waves of the workgroup, which walk the same range
    // (every wave of the workgroup must call this with the same range).
    __device__ __forceinline__ void walk_shared(int t_begin, int t_stop, float scale_log2,
                                                int wave) {
        u32x4 kt[2][KS];
        VPiece vt[8];
        float sc[NT][8];
        for (int w0 = t_begin; w0 < t_stop;) {
            const int first_block = w0 >> log2_bs;
            const int win_end = (first_block + 64) << log2_bs;
            const int w_end = win_end < t_stop ? win_end : t_stop;
            load_window(first_block);
            t_end = w_end;
            const int nch = (w_end - w0 + CHUNK - 1) / CHUNK;
            constexpr int AHEAD = kSharedBufs - 1;     // chunks requested ahead of the one in use
#pragma unroll
            for (int k = 0; k < AHEAD; ++k)
                if (k < nch) issue_shared(w0 + k * CHUNK, k, wave);
            for (int k = 0; k < nch; ++k) {
                const int c = w0 + k * CHUNK;
                // this wave's loads of chunk k are done (those of the chunks
                // after it may fly)
                const int later = nch - 1 - k < AHEAD - 1 ? nch - 1 - k : AHEAD - 1;
                if (later >= 2)
                    wait_vmcnt<2 * kSharedLoads>();
                else if (later == 1)
                    wait_vmcnt<kSharedLoads>();
                else
                    wait_vmcnt<0>();
                // ... and every wave's: chunk k is in LDS, and chunk k - 1's
                // buffer, which chunk k + AHEAD takes next, has been read by all
                __syncthreads();
                if (k + AHEAD < nch) issue_shared(c + AHEAD * CHUNK, (k + AHEAD) % kSharedBufs, wave);
                read_shared(k % kSharedBufs, kt, vt);
                scores(kt, scale_log2, sc);
                if (k == nch - 1 || c + CHUNK > mask_from)
                    softmax_pv<true>(c, sc, vt);
                else
                    softmax_pv<false>(c, sc, vt);
            }
            // the next window's first loads reuse the first buffers
            __syncthreads();
            w0 = w_end;
        }
    }

    __device__ __forceinline__ float total_sum(int t) { return strided_sum<16>(l[t]); }

    // LDS for the output transposes: the wave's own slice, or, after a
    // shared walk (SHARED: the workgroup walks with walk_shared), the wave's
    // 8 KB of the chunk buffers, which the walk has finished with
    __device__ __forceinline__ static f32x4 (*out_tile())[32] {
        if constexpr (SHARED)
            return reinterpret_cast<f32x4(*)[32]>(shared_chunk(0) + 8192 * (threadIdx.x >> 6));
        else
            return wave_tile_at<NWG>(threadIdx.x >> 6);
    }

    __device__ __forceinline__ void write_final(const AttnParams& a, int seq, int g) {
        void* out = a.out;
        const int dt = a.out_dtype;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float lsum = total_sum(t);
            // 0: a query before the start; FP8 values carry the kv head's V scale
            const float inv = lsum > 0.f ? (FP8 ? vscale / lsum : 1.0f / lsum) : 0.f;
            store_column_tile(out_tile(), acc[t], inv, orow[t], n < ncols[t],
                              [&](size_t r, int piece, f32x4 v) { store_out4(out, dt, r, piece, v); });
        }
    }

    // Pieces of segments that the balanced schedule cuts, parked in LDS
    // until the workgroup is done, in record form: slot (K, wave) holds
    // column c's unnormalised accumulator row (value scale) at
    // slot_acc<K>(wave) + 128 c, its max and sum at slot_ml<K>(wave)[c] and
    // [16 + c]. Slot 1 is the wave's output tile, which a wave fills only
    // with its last piece.
    static constexpr int kSlotCols = 16;

    // Waves per workgroup (NWG): the balanced schedule runs its own instance,
    // with eight waves (a compute unit's two per SIMD) for 16-bit K/V at one
    // or two query heads per kv head, where one workgroup per compute unit
    // keeps the two waves of a SIMD from the same workgroup and halves the
    // cut segments that cross workgroups; four otherwise.
    static constexpr int kGroupWaves = NWG;
    using Balanced = MfmaWalker<S, G_, STREAM, FP8, NT, WPS, SHARED,
                                (!FP8 && G_ < 4 && NT == 1 && !SHARED) ? 2 * kWaves : kWaves>;

    __device__ __forceinline__ static float* slot_rows() {
        __shared__ __attribute__((aligned(16))) float rows[NWG * 16 * 128];
        return rows;
    }

    __device__ __forceinline__ static float* slot_mls() {
        __shared__ float ml[2 * NWG * 32];
        return ml;
    }

    template <int K>
    __device__ __forceinline__ static float* slot_acc(int wave) {
        static_assert(NT == 1 && !SHARED, "one tile per wave, own tiles");
        if constexpr (K == 0)
            return slot_rows() + wave * 16 * 128;
        else
            return reinterpret_cast<float*>(wave_tile_at<NWG>(wave));
    }

    template <int K>
    __device__ __forceinline__ static float* slot_ml(int wave) {
        return slot_mls() + (K * NWG + wave) * 32;
    }

    template <int K>
    __device__ __forceinline__ void deposit(int wave) const {
        f32x4 (*t)[32] = reinterpret_cast<f32x4(*)[32]>(slot_acc<K>(wave));
        const float scale = FP8 ? vscale : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t[n][8 * q + 2 * i] = f32x4{acc[0][0][i], acc[0][1][i], acc[0][2][i], acc[0][3][i]} * scale;
            t[n][8 * q + 2 * i + 1] =
                f32x4{acc[0][4][i], acc[0][5][i], acc[0][6][i], acc[0][7][i]} * scale;
        }
        const float lsum = strided_sum<16>(l[0]);
        if (q == 0) {
            slot_ml<K>(wave)[n] = m[0];
            slot_ml<K>(wave)[16 + n] = lsum;
        }
    }

    // Partial results: column n of tile t to workspace row row0 + (16 t + n) * row_stride.
    __device__ __forceinline__ void write_partial(const AttnParams& a, size_t row0,
                                                  size_t row_stride) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            write_tile_partial(a, t, row0 + (size_t)(16 * t + n) * row_stride, n < ncols[t]);
    }

    // Column n's partial result (tile 0) into workspace row `row` (this lane's), if active.
    __device__ __forceinline__ void write_partial_at(const AttnParams& a, size_t row, bool active) {
        write_tile_partial(a, 0, row, active);
    }

    __device__ __forceinline__ void write_tile_partial(const AttnParams& a, int t, size_t row,
                                                       bool active) {
        const float lsum = total_sum(t);
        float* ws = a.ws_acc;
        store_column_tile(out_tile(), acc[t], FP8 ? vscale : 1.f, row, active,
                          [&](size_t r, int piece, f32x4 v) {
            *reinterpret_cast<f32x4*>(ws + r * D + 4 * piece) = v;
        });
        if (!active) return;
        if (q == 0) {
            a.ws_ml[2 * row] = m[t];
            a.ws_ml[2 * row + 1] = lsum;
        }
    }
};

}  // namespace
}  // namespace pkv
