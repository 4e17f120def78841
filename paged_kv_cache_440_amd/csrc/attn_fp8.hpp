// Walkers for FP8 (OCP E4M3) pools: K/V are 8-bit codes times a per-kv-head
// scale (blog.aqudi.me "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론
// 최적화", section 4: a lower-precision KV cache halves the bytes decode
// streams). Codes are widened in registers with v_cvt_pk_f32_fp8 (exact: every
// E4M3 value is a float32); the K scale is folded into the score scale and
// the V scale into the output. head_dim 128: a token row of one kv head is
// 128 bytes.
#pragma once

#include "attn_common.hpp"
#include "attn_mfma.hpp"

namespace pkv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// the four E4M3 codes of a dword as float32, in byte order
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

// q elements [first, first + n) of one row as float32
template <typename Q>
__device__ __forceinline__ float q_elem(const char* row, int i);
template <> __device__ __forceinline__ float q_elem<F32>(const char* row, int i) {
    return reinterpret_cast<const float*>(row)[i];
}
template <> __device__ __forceinline__ float q_elem<F16>(const char* row, int i) {
    return (float)reinterpret_cast<const _Float16*>(row)[i];
}
template <> __device__ __forceinline__ float q_elem<BF16>(const char* row, int i) {
    return (float)reinterpret_cast<const __bf16*>(row)[i];
}

// ---------------------------------------------------------------------------
// Vector walker (one query head per kv head). Lane l holds 16-byte piece
// l % 8 (16 codes, dims 16 (l % 8) ..) of token l / 8 of an 8-token group;
// one wave load covers 8 whole rows (1 KB). With fp16 / bf16 q, K codes are
// widened to pairs of q's type and a score is 8 packed dot products plus a
// 3-step DPP row sum, scaled by scale * log2(e) * k_scale; with fp32 q, q is
// widened once per segment, pre-multiplied by that factor, and a score is a
// 16-term FMA chain. Softmax bookkeeping is
// that of the 16-bit vector walker (token classes merged at the end).
template <typename Q, int G_, bool STREAM, int NLOAD_>
struct Fp8VecWalker {
    static constexpr bool kStream = STREAM;     // K/V load policy
    static constexpr int kBalancedWavesPerCU = 8;
    static constexpr int D = 128, G = G_;
    // NLOAD_ wave loads of K (and of V) per chunk
    static constexpr int ROW = 128, LPT = 8, TPL = 8, NLOAD = NLOAD_, CHUNK = TPL * NLOAD, EPL = 16;
    static constexpr int kMinWavesPerSimd = 2;
    static constexpr int kBalancedMinWavesPerSimd = kMinWavesPerSimd;

    float qf[G][EPL];   // fp32 q: pre-multiplied by scale * log2(e) * k_scale
    u32x4 qh[G][2];     // 16-bit q: the lane's 16 values as 8 pairs, unscaled
    float qmul;         // scale * log2(e) * k_scale
    float m[G], l[G], acc[G][EPL];
    float vscale;

    int wb, tv;
    int pre_tv = 0;     // a window read ahead (preload_window)
    bool pre = false;
    const char* kbase;
    const char* vbase;
    const int* trow;
    size_t head_stride_bytes, kvhead_off;
    int log2_bs, bs_mask, nblk_valid, max_phys;
    int* err;           // error word, or null
    int lane, tok, piece;
    int t_end, last_group;

    __device__ __forceinline__ void init(int lane_id) {
        lane = lane_id;
        tok = lane_id / LPT;
        piece = lane_id % LPT;
    }

    __device__ __forceinline__ void begin(const AttnParams& a, int seq, int g, int L, int = 0) {
        log2_bs = a.log2_bs;
        bs_mask = (1 << a.log2_bs) - 1;
        nblk_valid = (L + bs_mask) >> a.log2_bs;
        max_phys = a.num_blocks;
        err = a.err;
        trow = a.block_tables + (size_t)seq * a.max_blocks;
        head_stride_bytes = (size_t)a.num_kv_heads * ((size_t)ROW << a.log2_bs);
        kvhead_off = (size_t)g * ((size_t)ROW << a.log2_bs);
        kbase = reinterpret_cast<const char*>(a.k_pool);
        vbase = reinterpret_cast<const char*>(a.v_pool);
        vscale = a.v_scales[g];
        qmul = a.scale * kLog2e * a.k_scales[g];
        const char* q0 = reinterpret_cast<const char*>(a.q) +
                         ((size_t)seq * a.num_kv_heads * G + (size_t)g * G) * D * Q::bytes;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if constexpr (Q::bytes == 2) {
                const char* qrow = q0 + (size_t)h * D * 2 + piece * EPL * 2;
                qh[h][0] = load16(qrow);
                qh[h][1] = load16(qrow + 16);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    qf[h][e] = q_elem<Q>(q0 + (size_t)h * D * Q::bytes, piece * EPL + e) * qmul;
            }
            m[h] = -__builtin_inff();
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
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

    __device__ __forceinline__ uint32_t phys(int blk) {
        uint32_t p = (uint32_t)__builtin_amdgcn_readlane(tv, blk - wb);
        return p < (uint32_t)max_phys ? p : (uint32_t)(max_phys - 1);
    }

    __device__ __forceinline__ void load_chunk(int c0, u32x4 (&kr)[NLOAD], u32x4 (&vr)[NLOAD]) {
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) {
            int tg = c0 + j * TPL;
            tg = tg < last_group ? tg : last_group;
            const uint32_t p = phys(tg >> log2_bs);
            const size_t blk_off = (size_t)p * head_stride_bytes + kvhead_off;
            const uint32_t off = (uint32_t)(((tg & bs_mask) + tok) * ROW + piece * 16);
            kr[j] = load16_kv<STREAM>(kbase + blk_off + off);
            vr[j] = load16_kv<STREAM>(vbase + blk_off + off);
        }
    }

    template <bool TAIL>
    __device__ __forceinline__ void consume(int c0, const u32x4 (&kr)[NLOAD],
                                            const u32x4 (&vr)[NLOAD], float) {
        bool valid[NLOAD];
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) valid[j] = !TAIL || (c0 + j * TPL + tok < t_end);
        // scores, one K piece widened at a time: for 16-bit q, to pairs of q's
        // type and packed dot products (exact products, fp32 sums); for fp32
        // q, to fp32 and FMAs
        float s[G][NLOAD];
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) {
            if constexpr (Q::bytes == 2) {
                const u32x4 k0 = {fp8_pair<Q, false>(kr[j][0]), fp8_pair<Q, true>(kr[j][0]),
                                  fp8_pair<Q, false>(kr[j][1]), fp8_pair<Q, true>(kr[j][1])};
                const u32x4 k1 = {fp8_pair<Q, false>(kr[j][2]), fp8_pair<Q, true>(kr[j][2]),
                                  fp8_pair<Q, false>(kr[j][3]), fp8_pair<Q, true>(kr[j][3])};
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float d = dot16(Q{}, qh[h][0], k0) + dot16(Q{}, qh[h][1], k1);
                    d = group_sum<LPT>(d) * qmul;
                    s[h][j] = (TAIL && !valid[j]) ? -__builtin_inff() : d;
                }
            } else {
                float kf[EPL];
#pragma unroll
                for (int w = 0; w < 4; ++w) fp8x4_to_f32(kr[j][w], kf + 4 * w);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float d = qf[h][0] * kf[0];
#pragma unroll
                    for (int e = 1; e < EPL; ++e) d = __builtin_fmaf(qf[h][e], kf[e], d);
                    d = group_sum<LPT>(d);
                    s[h][j] = (TAIL && !valid[j]) ? -__builtin_inff() : d;
                }
            }
        }
        // online softmax update, then the V pieces one at a time
        float p[G][NLOAD];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = m[h];
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) mx = __builtin_fmaxf(mx, s[h][j]);
            const float alpha = (TAIL && mx == -__builtin_inff()) ? 1.f : fast_exp2(m[h] - mx);
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) {
                p[h][j] = (TAIL && !valid[j]) ? 0.f : fast_exp2(s[h][j] - mx);
                ps += p[h][j];
            }
            l[h] = l[h] * alpha + ps;
            m[h] = mx;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        }
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) {
            float vf[EPL];
#pragma unroll
            for (int w = 0; w < 4; ++w) fp8x4_to_f32(vr[j][w], vf + 4 * w);
            if constexpr (TAIL) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vf[e] = valid[j] ? vf[e] : 0.f;
            }
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(p[h][j], vf[e], acc[h][e]);
        }
    }

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
                consume<false>(c, k0, v0, scale_log2);
                const int n2 = n1 + CHUNK;
                if (n2 >= w_end) { consume<true>(n1, k1, v1, scale_log2); break; }
                load_chunk(n2, k0, v0);
                consume<false>(n1, k1, v1, scale_log2);
                c = n2;
            }
            w0 = w_end;
        }
    }

    // classes merged with the log-sum-exp rule; acc[h] ends scaled to values
    __device__ __forceinline__ void merge_classes(int h, float& mall, float& lsum) {
        mall = strided_max<LPT>(m[h]);
        const float w = (m[h] == -__builtin_inff()) ? 0.f : fast_exp2(m[h] - mall);
        lsum = strided_sum<LPT>(l[h] * w);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e] * w) * vscale;
    }

    // Pieces of segments that the balanced schedule cuts, parked in LDS
    // until the workgroup is done, in record form (classes merged (value scale)):
    // slot (K, wave) holds head h's unnormalised accumulator row at
    // slot_acc<K>(wave) + D h, its max and sum at slot_ml<K>(wave)[h] and [G + h].
    static constexpr int kSlotCols = G;
    // waves per workgroup in the balanced schedule, which runs this type
    static constexpr int kGroupWaves = kWaves;
    using Balanced = Fp8VecWalker;

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

    __device__ __forceinline__ void write_final(const AttnParams& a, int seq, int g) {
        const size_t row0 = (size_t)seq * a.num_kv_heads * G + (size_t)g * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mall, lsum;
            merge_classes(h, mall, lsum);
            const float inv = 1.0f / lsum;
            if (tok == 0) {
#pragma unroll
                for (int r = 0; r < EPL / 8; ++r) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = acc[h][8 * r + e] * inv;
                    store_out8(a.out, a.out_dtype, (row0 + h) * D + piece * EPL + 8 * r, v);
                }
            }
        }
    }

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

// ---------------------------------------------------------------------------
// Matrix-core walker for FP8 pools (2, 4 or 8 query heads per kv head, several
// new tokens, or the samples of a group; q in fp16 or bf16): the matrix-core
// walker of attn_mfma.hpp on E4M3 codes, computing in q's type.
template <typename Q, int G, bool STREAM>
using Fp8MfmaWalker = MfmaWalker<Q, G, STREAM, true>;

}  // namespace
}  // namespace pkv
