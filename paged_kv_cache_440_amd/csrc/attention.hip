// Paged single-query decode attention for gfx950.
//
// What is computed (supersilo.blog vLLM/PagedAttention summary, sections
// "자기회귀 생성과 KV 캐시" and "PagedAttention의 설계"): for every sequence
// and query head, softmax(scale * q.k_t) over all valid tokens t, applied to
// the values, with K/V fetched through the sequence's block table in logical
// order and ONE normalisation over every valid token.
//
// Work decomposition
//   A work item is (kv head g, sequence i, partition p): up to part_len
//   consecutive tokens of sequence i, for the G query heads that read kv head
//   g. One wave64 runs one work item; a workgroup holds kWaves independent
//   waves (no LDS, no barriers). Items are numbered g fastest, then i, then p.
//
// Lane layout inside a wave (for one 16-byte piece per lane and load)
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
//   item and keep their own running max m, sum l and unnormalised
//   accumulator acc (online rescaling by exp2(m_old - m_new) whenever m
//   grows). At the end of the item the TPL classes are merged with the
//   log-sum-exp rule; with several partitions the reduce kernel merges the
//   partitions the same way. Every merge and every reduction order depends
//   only on logical token positions, so relabelling physical blocks or
//   aliasing them changes no output bit.
//
// Masking
//   Only the last chunk of an item can hold tokens at or past the item's end;
//   there scores are replaced by -inf and values by 0 through selects, so
//   stale slot contents (NaN included) never reach the result.

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kWaves = 4;                       // independent waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <typename S, int D>
struct Geo {
    static constexpr int EB = S::bytes;
    static constexpr int ROW = D * EB;          // bytes of one token row of one kv head
    static constexpr int LPT = ROW / 16;        // lanes per token row
    static constexpr int TPL = 64 / LPT;        // tokens per wave-wide load
    static constexpr int NLOAD = 4;             // loads of K (and of V) per chunk
    static constexpr int CHUNK = TPL * NLOAD;   // tokens per chunk
    static constexpr int EPL = 16 / EB;         // elements per lane per load
    static_assert(LPT >= 8 && LPT <= 32, "row must span 8..32 lanes");
};

template <typename S, int D, int G>
struct Attn {
    using Gm = Geo<S, D>;
    static constexpr int LPT = Gm::LPT, TPL = Gm::TPL, NLOAD = Gm::NLOAD;
    static constexpr int CHUNK = Gm::CHUNK, EPL = Gm::EPL;

    // per-lane running state for G query heads
    float m[G], l[G], acc[G][EPL];
    u32x4 qv[G];

    // block table window: lane j holds the physical id of logical block wb + j
    int wb, tv;

    const char* kbase;
    const char* vbase;
    const int* trow;
    size_t head_stride_bytes;   // bytes from one physical block to the next
    size_t kvhead_off;          // bytes of kv head g inside a block
    int log2_bs, bs_mask, nblk_valid, max_phys;
    int lane, tok, piece;
    int t_end, last_group;

    __device__ __forceinline__ uint32_t phys(int blk) {
        if (blk - wb >= 64) {                      // wave-uniform; rare (single pass only)
            wb = blk;
            tv = (wb + lane < nblk_valid) ? trow[wb + lane] : 0;
        }
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
            kr[j] = load16(kbase + blk_off + off);
            vr[j] = load16(vbase + blk_off + off);
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
};

template <typename S>
__device__ __forceinline__ void store_out(void* out, int out_dtype, size_t idx, float v) {
    if (out_dtype == PKV_F32) {
        reinterpret_cast<float*>(out)[idx] = v;
    } else if (out_dtype == PKV_F16) {
        reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
    } else {
        reinterpret_cast<__bf16*>(out)[idx] = (__bf16)v;
    }
}

template <typename S, int D, int G>
__global__ __launch_bounds__(64 * kWaves)
void paged_decode_kernel(const AttnParams a) {
    using A = Attn<S, D, G>;
    using Gm = Geo<S, D>;
    constexpr int LPT = Gm::LPT, TPL = Gm::TPL, NLOAD = Gm::NLOAD, EPL = Gm::EPL;
    constexpr int CHUNK = Gm::CHUNK;

    const int lane = threadIdx.x & 63;
    // the wave index is uniform; say so, so that item-derived values live in SGPRs
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.num_items) return;
    const int g = item % a.num_kv_heads;
    const int rest = item / a.num_kv_heads;
    const int seq = rest % a.num_seqs;
    const int part = rest / a.num_seqs;
    const int num_heads = a.num_kv_heads * G;

    int L = a.seq_lens[seq];
    L = L < 0 ? 0 : L;
    L = L < a.max_tokens ? L : a.max_tokens;
    const int part_len = a.part_tokens > 0 ? a.part_tokens : (L > 0 ? L : 1);
    const int nparts = (L + part_len - 1) / part_len;
    const int t_begin = part * part_len;
    const int t_end = (t_begin + part_len < L) ? t_begin + part_len : L;
    const int tok = lane / LPT;
    const int piece = lane % LPT;

    if (t_begin >= t_end) {
        if (part == 0 && lane < LPT) {          // empty sequence: zero output rows
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    store_out<S>(a.out, a.out_dtype,
                                 ((size_t)seq * num_heads + g * G + h) * D + piece * EPL + e, 0.f);
        }
        return;
    }

    A st;
    st.lane = lane;
    st.tok = tok;
    st.piece = piece;
    st.t_end = t_end;
    st.last_group = ((t_end - 1) / TPL) * TPL;
    st.log2_bs = a.log2_bs;
    st.bs_mask = (1 << a.log2_bs) - 1;
    st.nblk_valid = (L + st.bs_mask) >> a.log2_bs;
    st.max_phys = a.num_blocks;
    st.trow = a.block_tables + (size_t)seq * a.max_blocks;
    st.head_stride_bytes = (size_t)a.num_kv_heads * (Gm::ROW << a.log2_bs);
    st.kvhead_off = (size_t)g * (Gm::ROW << a.log2_bs);
    st.kbase = reinterpret_cast<const char*>(a.k_pool);
    st.vbase = reinterpret_cast<const char*>(a.v_pool);
    st.wb = t_begin >> a.log2_bs;
    st.tv = (st.wb + lane < st.nblk_valid) ? st.trow[st.wb + lane] : 0;

    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((size_t)seq * num_heads + (size_t)g * G) * Gm::ROW + piece * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.qv[h] = load16(qrow + (size_t)h * Gm::ROW);
        st.m[h] = -__builtin_inff();
        st.l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[h][e] = 0.f;
    }
    const float scale_log2 = a.scale * kLog2e;

    // software-pipelined walk over the item's chunks
    u32x4 k0[NLOAD], v0[NLOAD], k1[NLOAD], v1[NLOAD];
    int c = t_begin;
    st.load_chunk(c, k0, v0);
    for (;;) {
        const int n1 = c + CHUNK;
        if (n1 >= t_end) { st.template consume<true>(c, k0, v0, scale_log2); break; }
        st.load_chunk(n1, k1, v1);
        st.template consume<false>(c, k0, v0, scale_log2);
        const int n2 = n1 + CHUNK;
        if (n2 >= t_end) { st.template consume<true>(n1, k1, v1, scale_log2); break; }
        st.load_chunk(n2, k0, v0);
        st.template consume<false>(n1, k1, v1, scale_log2);
        c = n2;
    }

    // merge the TPL token classes (lanes LPT apart) with the log-sum-exp rule
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float mall = strided_max<LPT>(st.m[h]);
        const float w = (st.m[h] == -__builtin_inff()) ? 0.f : fast_exp2(st.m[h] - mall);
        const float lsum = strided_sum<LPT>(st.l[h] * w);
        const size_t row = (size_t)seq * num_heads + (size_t)g * G + h;
        if (nparts == 1) {
            const float inv = 1.0f / lsum;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float o = strided_sum<LPT>(st.acc[h][e] * w);
                if (tok == 0) store_out<S>(a.out, a.out_dtype, row * D + piece * EPL + e, o * inv);
            }
        } else {
            const size_t prow = row * a.max_parts + part;
            float* wacc = a.ws_acc + prow * D + piece * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float o = strided_sum<LPT>(st.acc[h][e] * w);
                if (tok == 0) wacc[e] = o;
            }
            if (lane == 0) {
                a.ws_ml[2 * prow] = mall;
                a.ws_ml[2 * prow + 1] = lsum;
            }
        }
    }
}

// Merge the partitions of every (sequence, query head) that has more than one:
//   M = max_p m_p,  out = sum_p exp2(m_p - M) acc_p / sum_p exp2(m_p - M) l_p
// One wave per (sequence, head); lane j owns dims j, j + 64, ...
template <int D>
__global__ __launch_bounds__(64 * kWaves)
void lse_reduce_kernel(const AttnParams a) {
    const int lane = threadIdx.x & 63;
    const int num_heads = a.num_kv_heads * a.group;
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.num_seqs * num_heads) return;
    const int seq = item / num_heads;
    int L = a.seq_lens[seq];
    L = L < 0 ? 0 : L;
    L = L < a.max_tokens ? L : a.max_tokens;
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
    if (nparts <= 1) return;
    const size_t prow0 = (size_t)item * a.max_parts;
    float mmax = -__builtin_inff();
    for (int p = 0; p < nparts; ++p) mmax = __builtin_fmaxf(mmax, a.ws_ml[2 * (prow0 + p)]);
    constexpr int PER = D / 64;
    float o[PER], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int p = 0; p < nparts; ++p) {
        const float mp = a.ws_ml[2 * (prow0 + p)];
        const float w = (mp == -__builtin_inff()) ? 0.f : fast_exp2(mp - mmax);
        lsum = __builtin_fmaf(w, a.ws_ml[2 * (prow0 + p) + 1], lsum);
        const float* acc = a.ws_acc + (prow0 + p) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(w, acc[lane + 64 * e], o[e]);
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const size_t idx = (size_t)item * D + lane + 64 * e;
        if (a.out_dtype == PKV_F32) reinterpret_cast<float*>(a.out)[idx] = o[e] * inv;
        else if (a.out_dtype == PKV_F16) reinterpret_cast<_Float16*>(a.out)[idx] = (_Float16)(o[e] * inv);
        else reinterpret_cast<__bf16*>(a.out)[idx] = (__bf16)(o[e] * inv);
    }
}

template <typename S, int D, int G>
hipError_t launch_typed(const AttnParams& a, hipStream_t stream) {
    const int blocks = (a.num_items + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((paged_decode_kernel<S, D, G>), dim3(blocks), dim3(64 * kWaves), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.max_parts <= 1) return err;
    const int rblocks = (a.num_seqs * a.num_kv_heads * G + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((lse_reduce_kernel<D>), dim3(rblocks), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

template <typename S, int D>
hipError_t launch_group(const AttnParams& a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_typed<S, D, 1>(a, stream);
        case 2: return launch_typed<S, D, 2>(a, stream);
        case 4: return launch_typed<S, D, 4>(a, stream);
        case 8: return launch_typed<S, D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename S>
hipError_t launch_dim(const AttnParams& a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return launch_group<S, 64>(a, stream);
        case 128: return launch_group<S, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_paged_attention(const AttnParams& a, hipStream_t stream) {
    switch (a.dtype) {
        case PKV_F32: return launch_dim<F32>(a, stream);
        case PKV_F16: return launch_dim<F16>(a, stream);
        case PKV_BF16: return launch_dim<BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
