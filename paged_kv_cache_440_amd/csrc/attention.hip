// Paged single-query decode attention for gfx950.
//
// What is computed (supersilo.blog vLLM/PagedAttention summary, sections
// "자기회귀 생성과 KV 캐시" and "PagedAttention의 설계"): for every sequence
// and query head, softmax(scale * q.k_t) over all valid tokens t, applied to
// the values, with K/V fetched through the sequence's block table in logical
// order and ONE normalisation over every valid token.
//
// A segment is (sequence i, kv head g): the L_i tokens of one kv head, read
// for the G query heads that share it. One wave64 walks a contiguous token
// range of one segment at a time; workgroups hold kWaves independent waves
// (no LDS, no barriers). Three schedules decide the ranges:
//   single pass      one wave per segment (partition_size 0);
//   fixed partitions one wave per (segment, partition of part_len tokens),
//                    numbered g fastest, then i, then the partition; the
//                    hardware dispatcher hands them out, and waves of
//                    neighbouring sequences run side by side (blocks those
//                    sequences share are read from cache);
//   balanced         a fixed number W of persistent waves; the segments, cut
//                    into 32-token units and laid end to end in (i, g) order,
//                    are split into W equal runs, one per wave, so every wave
//                    streams the same number of bytes whatever the lengths.
// Partial results of split segments are merged by a log-sum-exp reduce.
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
//   range and keep their own running max m, sum l and unnormalised
//   accumulator acc (online rescaling by exp2(m_old - m_new) whenever m
//   grows). At the end of the range the TPL classes are merged with the
//   log-sum-exp rule; the reduce kernel merges the ranges of a split segment
//   the same way. Every merge and reduction order depends only on logical
//   token positions and on the lengths of the batch, so relabelling physical
//   blocks or aliasing them changes no output bit.
//
// Masking
//   Only the last chunk of a range can hold tokens at or past its end; there
//   scores are replaced by -inf and values by 0 through selects, so stale
//   slot contents (NaN included) never reach the result.

#include <atomic>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

#ifndef PKV_ATTN_WAVES
#define PKV_ATTN_WAVES 4
#endif
#ifndef PKV_ATTN_NLOAD
#define PKV_ATTN_NLOAD 4
#endif
constexpr int kWaves = PKV_ATTN_WAVES;          // independent waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

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

    // Load the table entries of logical blocks wb .. wb + 63 (one per lane).
    // Called only between pipelined walks: a load issued inside the walk
    // would make every later table lookup wait for all loads in flight.
    __device__ __forceinline__ void load_window(int first_block) {
        wb = first_block;
        tv = (wb + lane < nblk_valid) ? trow[wb + lane] : 0;
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

    // -- one range of one segment --------------------------------------------

    // Point the state at segment (seq, g) of length L and reset it.
    __device__ __forceinline__ void begin(const AttnParams& a, int seq, int g, int L) {
        log2_bs = a.log2_bs;
        bs_mask = (1 << a.log2_bs) - 1;
        nblk_valid = (L + bs_mask) >> a.log2_bs;
        max_phys = a.num_blocks;
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
};

__device__ __forceinline__ void store_out(void* out, int out_dtype, size_t idx, float v) {
    if (out_dtype == PKV_F32) {
        reinterpret_cast<float*>(out)[idx] = v;
    } else if (out_dtype == PKV_F16) {
        reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
    } else {
        reinterpret_cast<__bf16*>(out)[idx] = (__bf16)v;
    }
}

__device__ __forceinline__ int clamp_len(const AttnParams& a, int L) {
    L = L < 0 ? 0 : L;
    return L < a.max_tokens ? L : a.max_tokens;
}

// Write the finished segment (seq, g): out = acc / l for its G heads.
template <typename S, int D, int G>
__device__ __forceinline__ void write_final(Attn<S, D, G>& st, const AttnParams& a, int seq, int g) {
    constexpr int EPL = Attn<S, D, G>::EPL;
    const size_t row0 = (size_t)seq * a.num_kv_heads * G + (size_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mall, lsum;
        st.merge_classes(h, mall, lsum);
        const float inv = 1.0f / lsum;
        if (st.tok == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                store_out(a.out, a.out_dtype, (row0 + h) * D + st.piece * EPL + e,
                             st.acc[h][e] * inv);
        }
    }
}

// Write a partial result of G heads: unnormalised acc to rows
// ws_acc[row0 + h], (max, sum) to ws_ml[row0 + h].
template <typename S, int D, int G>
__device__ __forceinline__ void write_partial(Attn<S, D, G>& st, const AttnParams& a,
                                              size_t row0, size_t row_stride) {
    constexpr int EPL = Attn<S, D, G>::EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mall, lsum;
        st.merge_classes(h, mall, lsum);
        const size_t row = row0 + (size_t)h * row_stride;
        if (st.tok == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.ws_acc[row * D + st.piece * EPL + e] = st.acc[h][e];
        }
        if (st.lane == 0) {
            a.ws_ml[2 * row] = mall;
            a.ws_ml[2 * row + 1] = lsum;
        }
    }
}

template <typename S, int D, int G>
__device__ __forceinline__ void write_zero_rows(const AttnParams& a, int seq, int g, int lane) {
    constexpr int LPT = Geo<S, D>::LPT, EPL = Geo<S, D>::EPL;
    if (lane >= LPT) return;
    const size_t row0 = (size_t)seq * a.num_kv_heads * G + (size_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            store_out(a.out, a.out_dtype, (row0 + h) * D + lane * EPL + e, 0.f);
}

// ---------------------------------------------------------------------------
// Single pass and fixed partitions: one wave per (segment, partition).
// Partial rows: ws_acc[((seq * H + h) * max_parts + part)], the same for ws_ml.
template <typename S, int D, int G>
__global__ __launch_bounds__(64 * kWaves)
void paged_decode_kernel(const AttnParams a) {
    using A = Attn<S, D, G>;
    const int lane = threadIdx.x & 63;
    // the wave index is uniform; say so, so that item-derived values live in SGPRs
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.num_items) return;
    const int g = item % a.num_kv_heads;
    const int rest = item / a.num_kv_heads;
    const int seq = rest % a.num_seqs;
    const int part = rest / a.num_seqs;

    const int L = clamp_len(a, a.seq_lens[seq]);
    if (L == 0) {                                   // padding row: zero output
        if (part == 0) write_zero_rows<S, D, G>(a, seq, g, lane);
        return;
    }
    const int part_len = a.part_tokens > 0 ? a.part_tokens : L;
    const int nparts = (L + part_len - 1) / part_len;
    if (part >= nparts) return;
    const int t_begin = part * part_len;
    const int t_stop = (t_begin + part_len < L) ? t_begin + part_len : L;

    A st;
    st.lane = lane;
    st.tok = lane / A::LPT;
    st.piece = lane % A::LPT;
    st.begin(a, seq, g, L);
    st.walk(t_begin, t_stop, a.scale * kLog2e);
    if (nparts == 1) {
        write_final(st, a, seq, g);
    } else {
        const size_t row0 = ((size_t)seq * a.num_kv_heads * G + (size_t)g * G) * a.max_parts + part;
        write_partial(st, a, row0, (size_t)a.max_parts);
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
    const int L = clamp_len(a, a.seq_lens[seq]);
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
    for (int e = 0; e < PER; ++e)
        store_out(a.out, a.out_dtype, (size_t)item * D + lane + 64 * e, o[e] * inv);
}

// ---------------------------------------------------------------------------
// Balanced schedule.
//
// Segment (i, g) is cut into nu_i = ceil(L_i / kUnit) units of kUnit tokens;
// segments are laid end to end in (i, g) order, giving U = Hkv * sum_i nu_i
// units. Wave w of W takes units [w * q, (w + 1) * q), q = ceil(U / W). A
// segment inside one wave's run is finished by that wave. A segment cut by
// run boundaries gets one partial record per wave: the wave in which it
// starts writes record 2w + 1, every later wave writes record 2w (a wave's
// run begins inside at most one segment that started earlier, and ends inside
// at most one that goes on). Record r holds G rows: ws_acc[r * G + h],
// ws_ml[r * G + h].

constexpr int kUnit = 32;

__device__ __forceinline__ int units_of(int L) { return (L + kUnit - 1) / kUnit; }

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ long long wave_inclusive_scan(long long x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ __forceinline__ long long wave_total(long long x) {
    return __shfl(wave_inclusive_scan(x), 63, 64);
}

// Units of all segments of sequences [0, end): Hkv * sum nu_i.
__device__ __forceinline__ long long units_before(const AttnParams& a, int end) {
    const int lane = threadIdx.x & 63;
    long long total = 0;
    for (int b0 = 0; b0 < end; b0 += 64) {
        const int i = b0 + lane;
        const int nu = i < end ? units_of(clamp_len(a, a.seq_lens[i])) : 0;
        total += wave_total(nu);
    }
    return total * a.num_kv_heads;
}

template <typename S, int D, int G>
__global__ __launch_bounds__(64 * kWaves)
void paged_decode_balanced_kernel(const AttnParams a) {
    using A = Attn<S, D, G>;
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.num_items) return;
    const int W = a.num_items;
    const long long total = units_before(a, a.num_seqs);
    const long long q = (total + W - 1) / W;
    const long long u0 = (long long)w * q;
    const long long u1 = (u0 + q < total) ? u0 + q : total;
    if (u0 >= u1) return;

    // the sequence whose segments hold unit u0, and the units before it
    long long base = 0;
    int seq = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
        const int i = b0 + lane;
        const long long span =
            i < a.num_seqs ? (long long)a.num_kv_heads * units_of(clamp_len(a, a.seq_lens[i])) : 0;
        const long long incl = wave_inclusive_scan(span);
        const unsigned long long past = __ballot(base + incl > u0);
        if (past) {
            const int j = __builtin_ctzll(past);
            seq = b0 + j;
            base += __shfl(incl - span, j, 64);
            break;
        }
        base += __shfl(incl, 63, 64);
    }

    A st;
    st.lane = lane;
    st.tok = lane / A::LPT;
    st.piece = lane % A::LPT;
    const float scale_log2 = a.scale * kLog2e;
    long long u = u0;
    while (u < u1 && seq < a.num_seqs) {
        const int L = clamp_len(a, a.seq_lens[seq]);
        const int nu = units_of(L);
        if (nu == 0) { ++seq; continue; }        // empty sequences own no units
        const int g = (int)((u - base) / nu);
        const long long seg0 = base + (long long)g * nu;
        const long long seg1 = seg0 + nu;
        const int k0 = (int)(u - seg0);
        const int k1 = (int)((u1 < seg1 ? u1 : seg1) - seg0);
        const int t_stop = (k1 * kUnit < L) ? k1 * kUnit : L;
        st.begin(a, seq, g, L);
        st.walk(k0 * kUnit, t_stop, scale_log2);
        if (k0 == 0 && k1 == nu) {
            write_final(st, a, seq, g);
        } else {
            const size_t rec = 2 * (size_t)w + (k0 == 0 ? 1 : 0);
            write_partial(st, a, rec * G, 1);
        }
        u = seg0 + k1;
        if (g == a.num_kv_heads - 1 && u == seg1) {
            base = u;
            ++seq;
        }
    }
}

// Finish the balanced schedule: one wave per (sequence, query head). Rows
// of empty sequences are zeroed; rows of segments cut by run boundaries are
// merged from their records with the log-sum-exp rule.
template <int D>
__global__ __launch_bounds__(64 * kWaves)
void balanced_reduce_kernel(const AttnParams a) {
    const int lane = threadIdx.x & 63;
    const int num_heads = a.num_kv_heads * a.group;
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.num_seqs * num_heads) return;
    const int seq = item / num_heads;
    const int h = item % num_heads;
    const int g = h / a.group;
    constexpr int PER = D / 64;
    const int nu = units_of(clamp_len(a, a.seq_lens[seq]));
    if (nu == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            store_out(a.out, a.out_dtype, (size_t)item * D + lane + 64 * e, 0.f);
        return;
    }
    const int W = a.num_items;
    const long long total = units_before(a, a.num_seqs);
    const long long q = (total + W - 1) / W;
    const long long seg0 = units_before(a, seq) + (long long)g * nu;
    const long long wf = seg0 / q;
    const long long wl = (seg0 + nu - 1) / q;
    if (wf == wl) return;                        // finished by one wave
    const int hh = h % a.group;
    float mmax = -__builtin_inff();
    for (long long wv = wf; wv <= wl; ++wv) {
        const size_t rec = 2 * (size_t)wv + (wv == wf ? 1 : 0);
        mmax = __builtin_fmaxf(mmax, a.ws_ml[2 * (rec * a.group + hh)]);
    }
    float o[PER], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (long long wv = wf; wv <= wl; ++wv) {
        const size_t row = (2 * (size_t)wv + (wv == wf ? 1 : 0)) * a.group + hh;
        const float mp = a.ws_ml[2 * row];
        const float wgt = (mp == -__builtin_inff()) ? 0.f : fast_exp2(mp - mmax);
        lsum = __builtin_fmaf(wgt, a.ws_ml[2 * row + 1], lsum);
        const float* acc = a.ws_acc + row * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(wgt, acc[lane + 64 * e], o[e]);
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        store_out(a.out, a.out_dtype, (size_t)item * D + lane + 64 * e, o[e] * inv);
}

// Waves of the balanced kernel instance that fit on one compute unit at once
// (register-limited), queried once per instance.
template <typename S, int D, int G>
int balanced_resident_waves_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int groups = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &groups, reinterpret_cast<const void*>(&paged_decode_balanced_kernel<S, D, G>),
            64 * kWaves, 0) != hipSuccess || groups <= 0)
        return -1;
    v = groups * kWaves;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

template <typename S, int D, int G>
hipError_t launch_typed(const AttnParams& a_in, hipStream_t stream) {
    AttnParams a = a_in;
    if (a.balanced) {
        // a.num_items holds the compute-unit count; launch at most as many
        // persistent waves as are resident together, so that all of them
        // start at once and finish together
        const int resident = balanced_resident_waves_per_cu<S, D, G>();
        if (resident <= 0) return hipErrorInvalidValue;
        const int per_cu = resident < kBalancedWavesPerCU ? resident : kBalancedWavesPerCU;
        const long long w = (long long)a.num_items * per_cu;
        a.num_items = (int)(w < kMaxBalancedWaves ? w : kMaxBalancedWaves);
    }
    const int blocks = (a.num_items + kWaves - 1) / kWaves;
    const int rblocks = (a.num_seqs * a.num_kv_heads * G + kWaves - 1) / kWaves;
    if (a.balanced) {
        hipLaunchKernelGGL((paged_decode_balanced_kernel<S, D, G>), dim3(blocks),
                           dim3(64 * kWaves), 0, stream, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((balanced_reduce_kernel<D>), dim3(rblocks), dim3(64 * kWaves), 0,
                           stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((paged_decode_kernel<S, D, G>), dim3(blocks), dim3(64 * kWaves), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.max_parts <= 1) return err;
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
