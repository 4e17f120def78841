// Vector walker for paged decode attention (gfx950): q.k by packed dot
// products and DPP row sums, p.v by fp32 FMAs. Used for fp32 inputs, for
// head_dim 64, and for one or two query heads per kv head.
//
// Lane layout (for one 16-byte piece per lane and load)
//   A token row of one kv head is D * eb bytes = LPT 16-byte pieces. Lane l
//   holds piece (l % LPT) of token (l / LPT) of a TPL-token group, so one
//   wave-wide 16-byte load reads TPL whole rows: 1 KB of consecutive bytes in
//   one physical block (block_size is a multiple of TPL). A chunk is NLOAD
//   such groups (CHUNK tokens); the next chunk's K and V are loaded before
//   the current one is consumed.
//
// Softmax
//   Scores are kept in the log2 domain (scale * log2(e) folded in). The lanes
//   of token class c = l / LPT see tokens c, c + TPL, c + 2 TPL, ... of the
//   range and keep their own running max m, sum l and unnormalised
//   accumulator acc (online rescaling by exp2(m_old - m_new) whenever m
//   grows). At the end of the range the TPL classes are merged with the
//   log-sum-exp rule.
//
// Masking
//   Only the last chunk of a range can hold tokens at or past its end; there
//   scores are replaced by -inf and values by 0 through selects, so stale
//   slot contents (NaN included) never reach the result.
#pragma once

#include "attn_common.hpp"

namespace pkv {
namespace {

#ifndef PKV_ATTN_NLOAD
#define PKV_ATTN_NLOAD 4
#endif

template <typename S, int D>
struct Geo {
    static constexpr int EB = S::bytes;
    static constexpr int ROW = D * EB;          // bytes of one token row of one kv head
    static constexpr int LPT = ROW / 16;        // lanes per token row
    static constexpr int TPL = 64 / LPT;        // tokens per wave-wide load
    static constexpr int NLOAD = PKV_ATTN_NLOAD;  // loads of K (and of V) per chunk
    static constexpr int CHUNK = TPL * NLOAD;   // tokens per chunk
    static constexpr int EPL = 16 / EB;         // elements per lane per load
    static_assert(LPT >= 8 && LPT <= 32, "row must span 8..32 lanes");
};

template <typename S, int D_, int G_, bool STREAM>
struct VecWalker {
    static constexpr bool kStream = STREAM;     // K/V load policy
    static constexpr int kBalancedWavesPerCU = 8;
    static constexpr int D = D_, G = G_;
    using Gm = Geo<S, D_>;
    static constexpr int LPT = Gm::LPT, TPL = Gm::TPL, NLOAD = Gm::NLOAD;
    static constexpr int CHUNK = Gm::CHUNK, EPL = Gm::EPL;
    static constexpr int kMinWavesPerSimd = 1;
    // the balanced schedule keeps three waves per SIMD at one query head per
    // kv head (its registers fit without spilling)
    static constexpr int kBalancedMinWavesPerSimd = G == 1 ? 3 : kMinWavesPerSimd;

    // per-lane running state for G query heads
    float m[G], l[G], acc[G][EPL];
    u32x4 qv[G];

    // block table window: lane j holds the physical id of logical block wb + j
    int wb, tv;
    int pre_tv = 0;     // a window read ahead (preload_window)
    bool pre = false;

    const char* kbase;
    const char* vbase;
    const int* trow;
    size_t head_stride_bytes;   // bytes from one physical block to the next
    size_t kvhead_off;          // bytes of kv head g inside a block
    int log2_bs, bs_mask, nblk_valid, max_phys;
    int* err;           // error word, or null
    int lane, tok, piece;
    int t_end, last_group;

    __device__ __forceinline__ void init(int lane_id) {
        lane = lane_id;
        tok = lane_id / LPT;
        piece = lane_id % LPT;
    }

    // Load the table entries of logical blocks wb .. wb + 63 (one per lane).
    // Called only between pipelined walks: a load issued inside the walk
    // would make every later table lookup wait for all loads in flight.
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

    // physical block of logical block blk (wave-uniform, inside the window)
    __device__ __forceinline__ uint32_t phys(int blk) {
        uint32_t p = (uint32_t)__builtin_amdgcn_readlane(tv, blk - wb);
        return p < (uint32_t)max_phys ? p : (uint32_t)(max_phys - 1);
    }

    __device__ __forceinline__ void load_chunk(int c0, u32x4 (&kr)[NLOAD], u32x4 (&vr)[NLOAD]) {
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) {
            int tg = c0 + j * TPL;
            tg = tg < last_group ? tg : last_group;   // a group past the end re-reads the last one
            const uint32_t p = phys(tg >> log2_bs);
            const size_t blk_off = (size_t)p * head_stride_bytes + kvhead_off;
            const uint32_t off = (uint32_t)(((tg & bs_mask) + tok) * Gm::ROW + piece * 16);
            kr[j] = load16_kv<STREAM>(kbase + blk_off + off);
            vr[j] = load16_kv<STREAM>(vbase + blk_off + off);
        }
    }

    template <bool TAIL>
    __device__ __forceinline__ void consume(int c0, const u32x4 (&kr)[NLOAD],
                                            const u32x4 (&vr)[NLOAD], float scale_log2) {
        bool valid[NLOAD];
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) valid[j] = !TAIL || (c0 + j * TPL + tok < t_end);

        float vf[NLOAD][EPL];
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) {
            Piece<S>::widen(vr[j], vf[j]);
            if constexpr (TAIL) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vf[j][e] = valid[j] ? vf[j][e] : 0.f;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s[NLOAD];
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) {
                s[j] = group_sum<LPT>(dot16(S{}, qv[h], kr[j])) * scale_log2;
                if constexpr (TAIL) s[j] = valid[j] ? s[j] : -__builtin_inff();
            }
            float mx = m[h];
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) mx = __builtin_fmaxf(mx, s[j]);
            // Outside the tail every token is valid, so mx is finite. In the tail a
            // class may have seen no valid token at all: then m = mx = -inf, every
            // p is 0 and alpha (1) only multiplies zeros.
            const float alpha = (TAIL && mx == -__builtin_inff()) ? 1.f : fast_exp2(m[h] - mx);
            float p[NLOAD], ps = 0.f;
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) {
                p[j] = (TAIL && !valid[j]) ? 0.f : fast_exp2(s[j] - mx);
                ps += p[j];
            }
            l[h] = l[h] * alpha + ps;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[h][e] * alpha;
#pragma unroll
                for (int j = 0; j < NLOAD; ++j) a = __builtin_fmaf(p[j], vf[j][e], a);
                acc[h][e] = a;
            }
            m[h] = mx;
        }
    }

    // -- one range of one segment --------------------------------------------

    // Point the state at segment (seq, g) of length L and reset it.
    __device__ __forceinline__ void begin(const AttnParams& a, int seq, int g, int L, int = 0) {
        log2_bs = a.log2_bs;
        bs_mask = (1 << a.log2_bs) - 1;
        nblk_valid = (L + bs_mask) >> a.log2_bs;
        max_phys = a.num_blocks;
        err = a.err;
        trow = a.block_tables + (size_t)seq * a.max_blocks;
        head_stride_bytes = (size_t)a.num_kv_heads * ((size_t)Gm::ROW << a.log2_bs);
        kvhead_off = (size_t)g * ((size_t)Gm::ROW << a.log2_bs);
        kbase = reinterpret_cast<const char*>(a.k_pool);
        vbase = reinterpret_cast<const char*>(a.v_pool);
        const char* qrow = reinterpret_cast<const char*>(a.q) +
                           ((size_t)seq * a.num_kv_heads * G + (size_t)g * G) * Gm::ROW + piece * 16;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            qv[h] = load16(qrow + (size_t)h * Gm::ROW);
            m[h] = -__builtin_inff();
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
        }
    }

    // Consume tokens [t_begin, t_stop) of the segment (t_begin a multiple of
    // 32). The walk goes one table window (64 blocks) at a time; inside a
    // window it is software-pipelined. Window ends fall on block boundaries,
    // which are multiples of CHUNK past t_begin, so no chunk crosses one.
    __device__ __forceinline__ void walk(int t_begin, int t_stop, float scale_log2) {
        u32x4 k0[NLOAD], v0[NLOAD], k1[NLOAD], v1[NLOAD];
        for (int w0 = t_begin; w0 < t_stop;) {
            const int first_block = w0 >> log2_bs;
            const int win_end = (first_block + 64) << log2_bs;
            const int w_end = win_end < t_stop ? win_end : t_stop;
            load_window(first_block);
            t_end = w_end;
            last_group = ((w_end - 1) / TPL) * TPL;
            int c = w0;
            load_chunk(c, k0, v0);
            for (;;) {
                const int n1 = c + CHUNK;
                if (n1 >= w_end) { consume<true>(c, k0, v0, scale_log2); break; }
                load_chunk(n1, k1, v1);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
                consume<false>(c, k0, v0, scale_log2);
                const int n2 = n1 + CHUNK;
                if (n2 >= w_end) { consume<true>(n1, k1, v1, scale_log2); break; }
                load_chunk(n2, k0, v0);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
                consume<false>(n1, k1, v1, scale_log2);
                c = n2;
            }
            w0 = w_end;
        }
    }

    // Merge the TPL token classes (lanes LPT apart) of head h with the
    // log-sum-exp rule: returns the range's max and sum, and leaves the merged
    // unnormalised accumulator in acc[h] (valid on every lane of a class).
    __device__ __forceinline__ void merge_classes(int h, float& mall, float& lsum) {
        mall = strided_max<LPT>(m[h]);
        const float w = (m[h] == -__builtin_inff()) ? 0.f : fast_exp2(m[h] - mall);
        lsum = strided_sum<LPT>(l[h] * w);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e] * w);
    }

    // Pieces of segments that the balanced schedule cuts, parked in LDS
    // until the workgroup is done, in record form (classes merged):
    // slot (K, wave) holds head h's unnormalised accumulator row at
    // slot_acc<K>(wave) + D h, its max and sum at slot_ml<K>(wave)[h] and [G + h].
    static constexpr int kSlotCols = G;
    // waves per workgroup in the balanced schedule, which runs this type
    static constexpr int kGroupWaves = kWaves;
    using Balanced = VecWalker;

    __device__ __forceinline__ static float* slot_rows() {
        __shared__ __attribute__((aligned(16))) float rows[2 * kWaves * G * D];
        return rows;
    }

    __device__ __forceinline__ static float* slot_mls() {
        __shared__ float ml[2 * kWaves * 2 * G];
        return ml;
    }

    template <int K>
    __device__ __forceinline__ static float* slot_acc(int wave) {
        return slot_rows() + (K * kWaves + wave) * G * D;
    }

    template <int K>
    __device__ __forceinline__ static float* slot_ml(int wave) {
        return slot_mls() + (K * kWaves + wave) * 2 * G;
    }

    template <int K>
    __device__ __forceinline__ void deposit(int wave) {
        float* rows = slot_acc<K>(wave);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mall, lsum;
            merge_classes(h, mall, lsum);
            if (tok == 0) {
                f32x4* dst = reinterpret_cast<f32x4*>(rows + h * D + piece * EPL);
#pragma unroll
                for (int r = 0; r < EPL / 4; ++r)
                    dst[r] = f32x4{acc[h][4 * r], acc[h][4 * r + 1], acc[h][4 * r + 2],
                                   acc[h][4 * r + 3]};
            }
            if (lane == 0) {
                slot_ml<K>(wave)[h] = mall;
                slot_ml<K>(wave)[G + h] = lsum;
            }
        }
    }

    // Write the finished segment (seq, g): out = acc / l for its G heads.
    __device__ __forceinline__ void write_final(const AttnParams& a, int seq, int g) {
        const size_t row0 = (size_t)seq * a.num_kv_heads * G + (size_t)g * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mall, lsum;
            merge_classes(h, mall, lsum);
            const float inv = 1.0f / lsum;
            if (tok == 0) {
                if constexpr (EPL == 8) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = acc[h][e] * inv;
                    store_out8(a.out, a.out_dtype, (row0 + h) * D + piece * EPL, v);
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        store_out(a.out, a.out_dtype, (row0 + h) * D + piece * EPL + e,
                                  acc[h][e] * inv);
                }
            }
        }
    }

    // Write a partial result of the G heads: the unnormalised accumulator to
    // ws_acc row (row0 + h * row_stride), (max, sum) to the same ws_ml row.
    __device__ __forceinline__ void write_partial(const AttnParams& a, size_t row0,
                                                  size_t row_stride) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mall, lsum;
            merge_classes(h, mall, lsum);
            const size_t row = row0 + (size_t)h * row_stride;
            if (tok == 0) {
                f32x4* dst = reinterpret_cast<f32x4*>(a.ws_acc + row * D + piece * EPL);
#pragma unroll
                for (int r = 0; r < EPL / 4; ++r)
                    dst[r] = f32x4{acc[h][4 * r], acc[h][4 * r + 1], acc[h][4 * r + 2],
                                   acc[h][4 * r + 3]};
            }
            if (lane == 0) {
                a.ws_ml[2 * row] = mall;
                a.ws_ml[2 * row + 1] = lsum;
            }
        }
    }
};

}  // namespace
}  // namespace pkv
