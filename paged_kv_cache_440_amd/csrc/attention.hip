// Paged single-query decode attention for gfx950: schedules, reduce kernels
// and dispatch.
//
// What is computed (supersilo.blog vLLM/PagedAttention summary, sections
// "자기회귀 생성과 KV 캐시" and "PagedAttention의 설계"): for every sequence
// and query head, softmax(scale * q.k_t) over all valid tokens t, applied to
// the values, with K/V fetched through the sequence's block table in logical
// order and ONE normalisation over every valid token.
//
// A segment is (sequence i, kv head g): the L_i tokens of one kv head, read
// for the G query heads that share it. One wave64 walks a contiguous token
// range of one segment at a time (a "walker": attn_vec.hpp on the vector
// units, attn_mfma.hpp on the matrix cores for grouped-query attention);
// workgroups hold kWaves waves that share nothing, except under the balanced
// schedule (its workgroups of Walker::kGroupWaves waves fold the pieces of cut
// segments in LDS after one end-of-run barrier). Three schedules decide the
// ranges:
//   single pass      one wave per segment (partition_size 0);
//   fixed partitions one wave per (segment, partition of part_len tokens),
//                    handed out by the hardware dispatcher; numbered g
//                    fastest, then i, then the partition for streamed K/V,
//                    and i fastest, then g, then the partition for the
//                    cached-load policy, so that neighbouring sequences run
//                    side by side and blocks they share come from cache;
//   balanced         a fixed number W of persistent waves; the segments, cut
//                    into 32-token units and laid end to end in (i, g) order,
//                    are split into W equal runs, one per wave, so every wave
//                    streams the same number of bytes whatever the lengths.
// Partial results of split segments are merged by a log-sum-exp reduce. Every
// merge and reduction order depends only on logical token positions and on
// the lengths of the batch, so relabelling physical blocks or aliasing them
// changes no output bit.

#include <atomic>
#include <type_traits>

#include "attn_common.hpp"
#include "attn_fp8.hpp"
#include "attn_mfma.hpp"
#include "attn_vec.hpp"

namespace pkv {

namespace {

// Sampling groups: partition `part` of sequence seq (length L) lies inside
// the tokens its group shares, so the group kernel computes it for all the
// group's sequences at once. The same predicate decides on both sides, so
// every (sequence, partition) is computed exactly once. The last token of a
// sequence is never in a shared partition.
__device__ __forceinline__ bool in_shared_part(const AttnParams& a, int seq, int part, int L) {
    const int P = a.shared_tokens[seq / a.group_size];
    const int lim = P < L - 1 ? P : L - 1;
    return (part + 1) * a.part_tokens <= lim;
}

// ---------------------------------------------------------------------------
// Single pass and fixed partitions: one wave per (segment, 16-column tile,
// partition); a segment has one tile unless it has more than 16 columns
// (several new tokens per sequence on the matrix cores). Partial rows:
// ws_acc[((seq * Hkv + g) * cols + c) * max_parts + part] for column c, the
// same for ws_ml.
template <class Walker>
__device__ __forceinline__ void decode_partition(const AttnParams& a, int item_in) {
    constexpr int D = Walker::D, G = Walker::G;
    const int lane = threadIdx.x & 63;
    if (item_in >= a.num_items) return;
    // the tile groups of one partition are neighbours: they read the same blocks
    const int groups = (a.col_tiles + a.tiles_per_item - 1) / a.tiles_per_item;
    const int tile = item_in % groups;           // the group of tiles this wave walks
    const int item = item_in / groups;
    int g, seq, part;
    if constexpr (Walker::kStream) {
        // the kv heads of one sequence side by side: their tiles are neighbours
        g = item % a.num_kv_heads;
        const int rest = item / a.num_kv_heads;
        seq = rest % a.num_seqs;
        part = rest / a.num_seqs;
    } else {
        // neighbouring sequences side by side, in the same workgroup: blocks
        // they share are read from HBM once and then found in cache
        seq = item % a.num_seqs;
        const int rest = item / a.num_seqs;
        g = rest % a.num_kv_heads;
        part = rest / a.num_kv_heads;
    }

    const int raw_len = a.seq_lens[seq];
    report_if(a.err, lane == 0 && g == 0 && part == 0 && (raw_len < 0 || raw_len > a.max_tokens),
              PKV_ERRBIT_LENGTH);
    const int L = clamp_len(a, raw_len);
    if (L == 0) {                                   // padding row: zero output
        if (part == 0 && tile == 0) write_zero_rows<D>(a, seq, g, lane);
        return;
    }
    // the tokens the group's columns see (L unless several tiles)
    const int reach = a.col_tiles > 1 ? group_reach(a, L, tile) : L;
    if (reach <= 0) {                               // every column before the start
        const int c0 = 16 * a.tiles_per_item * tile, cols = a.num_queries * G;
        const int c1 = c0 + 16 * a.tiles_per_item < cols ? c0 + 16 * a.tiles_per_item : cols;
        if (part == 0) write_zero_cols<D>(a, seq, g, c0, c1, lane);
        return;
    }
    const int part_len = a.part_tokens > 0 ? a.part_tokens : reach;
    const int nparts = (reach + part_len - 1) / part_len;
    if (part >= nparts) return;
    if (a.shared_tokens != nullptr && a.part_tokens > 0 && in_shared_part(a, seq, part, L)) return;
    const int t_begin = part * part_len;
    const int t_stop = (t_begin + part_len < reach) ? t_begin + part_len : reach;

    Walker st;
    st.init(lane);
    st.begin(a, seq, g, L, tile);
    st.walk(t_begin, t_stop, a.scale * kLog2e);
    if (nparts == 1) {
        st.write_final(a, seq, g);
    } else {
        const int cols = a.num_queries * G;
        const size_t row0 =
            ((size_t)seq * a.num_kv_heads * cols + (size_t)g * cols +
             16 * (size_t)a.tiles_per_item * tile) * a.max_parts + part;
        st.write_partial(a, row0, (size_t)a.max_parts);
    }
}

template <class Walker>
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(Walker::kMinWavesPerSimd)))
void paged_decode_kernel(const AttnParams a) {
    // the wave index is uniform; say so, so that item-derived values live in SGPRs
    decode_partition<Walker>(a, blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
}

// Sampling groups: a wave per (group k, kv head g, partition). Column n of
// the matrix-core walker is sample n / G of the group with query head
// g*G + n % G; the partition's K/V are read once for all of them. A column
// whose sequence does not share the partition is left to the sequence
// kernel. Partial rows as in paged_decode_kernel.
template <class Walker>
__device__ __forceinline__ void group_partition(const AttnParams& a, int item) {
    const int lane = threadIdx.x & 63;
    const int num_groups = a.num_seqs / a.group_size;
    if (item >= num_groups * a.num_kv_heads * a.max_parts) return;
    const int g = item % a.num_kv_heads;
    const int rest = item / a.num_kv_heads;
    const int k = rest % num_groups;
    const int part = rest / num_groups;
    const int G = a.group;
    const int n = lane & 15;
    const int sample = n / G < a.group_size ? n / G : a.group_size - 1;
    const int seq = k * a.group_size + sample;
    bool active = false;
    if (n < a.group_size * G) {
        const int L = clamp_len(a, a.seq_lens[seq]);
        active = L > 0 && in_shared_part(a, seq, part, L);
    }
    const unsigned long long act = __ballot(active);
    if (act == 0) return;
    // the blocks of the partition, through the table of a sequence that shares it
    const int table_seq = __shfl(seq, __builtin_ctzll(act), 64);
    const int t_begin = part * a.part_tokens;
    const int t_stop = t_begin + a.part_tokens;
    const size_t head_row = (size_t)seq * a.num_kv_heads * G + (size_t)g * G + n % G;
    Walker st;
    st.init(lane);
    st.begin_columns(a, table_seq, g, t_stop, head_row, active);
    st.walk(t_begin, t_stop, a.scale * kLog2e);
    st.write_partial_at(a, head_row * a.max_parts + part, active);
}

// Both kinds of work of a grouped call in one launch: the group items first
// (long, one per group, kv head and partition), then the sequence items,
// which fill the machine while the last group items finish.
template <class GroupWalker, class SeqWalker>
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(GroupWalker::kMinWavesPerSimd)))
void paged_decode_grouped_kernel(const AttnParams a, int group_items) {
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item < group_items)
        group_partition<GroupWalker>(a, item);
    else
        decode_partition<SeqWalker>(a, item - group_items);
}

// Log-sum-exp fold of one output row's partial records (D floats of
// unnormalised accumulator plus (max, sum) in base-2 units each). The wave
// reads RPW records side by side: LPR = D / 4 lanes cover a record row with
// one 16-byte load each, and lane group k folds records k, k + RPW, ... in
// order with a running max,
//   M' = max(M, m_r),  o' = o 2^(M - M') + acc_r 2^(m_r - M'),
//   l' = l 2^(M - M') + l_r 2^(m_r - M'),
// issuing the loads of many records before the first result is needed. The
// groups are then merged pairwise by the same rule and out = o / l is written
// by group 0. row_of(r) gives the workspace row of record r (0 <= r < nrec).
template <int D, class RowOf>
__device__ __forceinline__ void fold_records(const AttnParams& a, int nrec, RowOf row_of,
                                             size_t orow) {
    constexpr int LPR = D / 4, RPW = 64 / LPR;
    static_assert(LPR * RPW == 64, "record rows of 16 to 64 lanes");
    const int lane = threadIdx.x & 63, grp = lane / LPR, sub = lane % LPR;
    float mrun = -__builtin_inff(), lsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int r = grp; r < nrec; r += RPW) {
        const size_t row = row_of(r);
        const float mr = a.ws_ml[2 * row], lr = a.ws_ml[2 * row + 1];
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.ws_acc + row * D + 4 * sub);
        const float mnew = __builtin_fmaxf(mrun, mr);
        const float keep = (mrun == -__builtin_inff()) ? 0.f : fast_exp2(mrun - mnew);
        const float take = (mr == -__builtin_inff()) ? 0.f : fast_exp2(mr - mnew);
        lsum = __builtin_fmaf(take, lr, lsum * keep);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = __builtin_fmaf(take, x[k], o[k] * keep);
        mrun = mnew;
    }
#pragma unroll
    for (int step = LPR; step < 64; step <<= 1) {
        const float mo = __shfl_xor(mrun, step, 64), lo = __shfl_xor(lsum, step, 64);
        const float mnew = __builtin_fmaxf(mrun, mo);
        const float ka = (mrun == -__builtin_inff()) ? 0.f : fast_exp2(mrun - mnew);
        const float kb = (mo == -__builtin_inff()) ? 0.f : fast_exp2(mo - mnew);
        lsum = lsum * ka + lo * kb;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = o[k] * ka + __shfl_xor(o[k], step, 64) * kb;
        mrun = mnew;
    }
    if (grp != 0) return;
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;   // 0: a query before the start
    const size_t idx = orow * D + 4 * sub;
    if (a.out_dtype == PKV_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + idx) = o * inv;
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) store_out(a.out, a.out_dtype, idx + k, o[k] * inv);
}

// Merge the partitions of every (segment, column) that has more than one:
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
// One wave per (sequence, kv head, column), folding its partitions with
// fold_records.
template <int D>
__global__ __launch_bounds__(64 * kWaves)
void lse_reduce_kernel(const AttnParams a) {
    const int cols = a.num_queries * a.group;
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= a.num_seqs * a.num_kv_heads * cols) return;
    const int seq = item / (a.num_kv_heads * cols);
    const int g = (item / cols) % a.num_kv_heads;
    const int n = item % cols;
    const int L = clamp_len(a, a.seq_lens[seq]);
    // partitions of the tokens column n's tile group reaches, as the walk cut them
    const int reach = a.col_tiles > 1 ? group_reach(a, L, n / (16 * a.tiles_per_item)) : L;
    const int nparts = reach > 0 ? (reach + a.part_tokens - 1) / a.part_tokens : 0;
    if (nparts <= 1) return;
    const size_t prow0 = (size_t)item * a.max_parts;
    fold_records<D>(a, nparts, [&](int p) { return prow0 + p; }, out_row(a, seq, g, n));
}

// ---------------------------------------------------------------------------
// Balanced schedule.
//
// Segment (i, g) is cut into nu_i = ceil(L_i / kUnit) units of kUnit tokens;
// segments are laid end to end in (i, g) order, giving U = Hkv * sum_i nu_i
// units. Wave w of W takes units [w * q, (w + 1) * q), q = ceil(U / W). A
// segment inside one wave's run is finished by that wave. A wave's run
// begins inside at most one segment that started earlier and ends inside at
// most one that goes on; the pieces of such cut segments first meet in LDS.
// Each wave parks its cut pieces there (the first of its run in slot 0, the
// last in slot 1), and once the whole workgroup is done, the pieces that fall
// in one workgroup are folded by one of its waves. If the segment starts and
// ends in the workgroup, that wave writes the output; otherwise it writes
// the workgroup's one partial record: the wave w where the segment starts
// record 2w + 1, the first wave w of every later workgroup record 2w.
// Record r holds one row per column: ws_acc[r * cols + c], ws_ml[r * cols + c].
// The merge kernel folds those records.

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

// Per wave of the workgroup: the segment (seq * Hkv + g) whose piece it
// holds in its LDS slot 0 (-1: none), and, if that segment ends in its run
// after beginning in an earlier workgroup, the first wave holding a piece of
// it (-1 otherwise).
template <int NW>
__device__ __forceinline__ int* slot_tags() {
    __shared__ int tags[2 * NW];
    return tags;
}

// 16-byte (fp32) or 8-byte (16-bit) store of outputs idx .. idx + 3.
__device__ __forceinline__ void store_out_quad(void* out, int out_dtype, size_t idx, f32x4 v) {
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

// Fold nslots pieces of segment (seq, g) parked in LDS (record form, as the
// walkers' deposit writes them; slot k at acc_of(k), ml_of(k)) by the
// log-sum-exp rule, and write its cols columns: the outputs if `final`,
// else workspace record rec (rows rec * cols + c).
template <class Walker, class AccOf, class MlOf>
__device__ __forceinline__ void fold_slots(const AttnParams& a, int nslots, AccOf acc_of, MlOf ml_of,
                                           bool final, int seq, int g, size_t rec) {
    constexpr int D = Walker::D, SC = Walker::kSlotCols, LPR = D / 4, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, grp = lane / LPR, sub = lane % LPR;
    const int cols = a.num_queries * Walker::G;
    for (int c0 = 0; c0 < cols; c0 += RPW) {
        const int c = c0 + grp;
        if (c >= cols) break;
        float mrun = -__builtin_inff(), lsum = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < nslots; ++k) {
            const float* ml = ml_of(k);
            const float mk = ml[c], lk = ml[SC + c];
            const f32x4 x = *reinterpret_cast<const f32x4*>(acc_of(k) + c * D + 4 * sub);
            const float mnew = __builtin_fmaxf(mrun, mk);
            const float keep = (mrun == -__builtin_inff()) ? 0.f : fast_exp2(mrun - mnew);
            const float take = (mk == -__builtin_inff()) ? 0.f : fast_exp2(mk - mnew);
            lsum = __builtin_fmaf(take, lk, lsum * keep);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = __builtin_fmaf(take, x[j], o[j] * keep);
            mrun = mnew;
        }
        if (final) {
            const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;   // 0: a query before the start
            store_out_quad(a.out, a.out_dtype, out_row(a, seq, g, c) * D + 4 * sub, o * inv);
        } else {
            const size_t row = rec * cols + c;
            *reinterpret_cast<f32x4*>(a.ws_acc + row * D + 4 * sub) = o;
            if (sub == 0) {
                a.ws_ml[2 * row] = mrun;
                a.ws_ml[2 * row + 1] = lsum;
            }
        }
    }
}

// Wave w's run of the balanced schedule. Its cut pieces go to its LDS slots:
// the first piece, if it continues a segment begun before the run, to slot
// 0 (tagged with the segment, seq * Hkv + g), the last, if it begins a
// segment that goes on past the run, to slot 1. Returns that last piece's
// segment (-1: none), and in *ends_here whether the segment ends inside the
// workgroup.
template <class Walker>
__device__ __forceinline__ int balanced_run(const AttnParams& a, int w, Walker& st,
                                            bool* ends_here) {
    constexpr int NW = Walker::kGroupWaves;
    const int lane = threadIdx.x & 63;
    const int wl = w % NW;
    const int W = a.num_items;
    // padding sequences (length 0) own no units: wave w zeroes the rows of
    // sequences w, w + W, ...
    for (int i = w; i < a.num_seqs; i += W) {
        const int raw_len = a.seq_lens[i];
        report_if(a.err, lane == 0 && (raw_len < 0 || raw_len > a.max_tokens), PKV_ERRBIT_LENGTH);
        if (clamp_len(a, raw_len) == 0)
            for (int g = 0; g < a.num_kv_heads; ++g) write_zero_rows<Walker::D>(a, i, g, lane);
    }
    const long long total = units_before(a, a.num_seqs);
    const long long q = (total + W - 1) / W;
    const long long u0 = (long long)w * q;
    const long long u1 = (u0 + q < total) ? u0 + q : total;
    if (u0 >= u1) return -1;                     // holds no piece of any segment
    // The workgroup's waves hold units [g_lo, g_hi). A segment that starts
    // before u0 lies inside the workgroup if it starts at or after g_lo and
    // ends by g_hi; one that starts in this run and goes on past u1, if its
    // units past u1 number at most g_room.
    const long long g_lo = (long long)(w - wl) * q, g_hi = g_lo + NW * q;
    const int g_room = __builtin_amdgcn_readfirstlane(
        (int)(g_hi - u1 < 0x7fffffff ? g_hi - u1 : 0x7fffffff));

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

    // Whether this wave ends a segment begun in an earlier workgroup (the
    // one holding unit u0), which the merge kernel finishes.
    {
        const int nu = units_of(clamp_len(a, a.seq_lens[seq]));
        const int g = (int)((u0 - base) / nu);
        const long long seg0 = base + (long long)g * nu;
        if (lane == 0 && seg0 < g_lo && seg0 + nu <= u1) slot_tags<NW>()[NW + wl] = (int)(seg0 / q);
    }

    st.init(lane);
    const float scale_log2 = a.scale * kLog2e;
    int pending = -1;
    long long u = u0;
    // the next segment's length and first table window, read while the
    // current segment is walked (sequence -1: nothing read ahead)
    int pf_seq = -1, pf_g = -1, pf_len = 0, pf_tv = 0;
    while (u < u1 && seq < a.num_seqs) {
        const int raw_len = seq == pf_seq ? pf_len : a.seq_lens[seq];
        const int L = clamp_len(a, raw_len);
        const int nu = units_of(L);
        if (nu == 0) { ++seq; continue; }        // empty sequences own no units
        const int g = (int)((u - base) / nu);
        const long long seg0 = base + (long long)g * nu;
        const long long seg1 = seg0 + nu;
        const int k0 = (int)(u - seg0);
        const int k1 = (int)((u1 < seg1 ? u1 : seg1) - seg0);
        const int t_stop = (k1 * kUnit < L) ? k1 * kUnit : L;
        st.begin(a, seq, g, L);
        if (seq == pf_seq && g == pf_g) st.preload_window(pf_tv);
        // the segment after this one, if this wave's run goes on into it
        const int nseq = g + 1 < a.num_kv_heads ? seq : seq + 1;
        const int ng = g + 1 < a.num_kv_heads ? g + 1 : 0;
        if (seg0 + k1 < u1 && nseq < a.num_seqs) {
            pf_seq = nseq;
            pf_g = ng;
            pf_len = nseq == seq ? raw_len : a.seq_lens[nseq];
            pf_tv = lane < a.max_blocks ? a.block_tables[(size_t)nseq * a.max_blocks + lane] : 0;
        } else {
            pf_seq = -1;
        }
        st.walk(k0 * kUnit, t_stop, scale_log2);
        if (k0 == 0 && k1 == nu) {
            st.write_final(a, seq, g);
        } else if (k0 > 0) {
            // a later piece of a segment begun before this run (its first piece)
            st.template deposit<0>(wl);
            if (lane == 0) slot_tags<NW>()[wl] = seq * a.num_kv_heads + g;
        } else {
            // the first piece of a segment that goes on past this run (its last)
            st.template deposit<1>(wl);
            pending = __builtin_amdgcn_readfirstlane(seq * a.num_kv_heads + g);
            *ends_here = nu - k1 <= g_room;
        }
        u = seg0 + k1;
        if (g == a.num_kv_heads - 1 && u == seg1) {
            base = u;
            ++seq;
        }
    }
    return pending;
}

template <class Walker>
__global__ __launch_bounds__(64 * Walker::kGroupWaves)
__attribute__((amdgpu_waves_per_eu(Walker::kBalancedMinWavesPerSimd)))
void paged_decode_balanced_kernel(const AttnParams a) {
    constexpr int NW = Walker::kGroupWaves;
    const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x * NW + wl;
    int* tags = slot_tags<NW>();
    if ((threadIdx.x & 63) == 0) {
        tags[wl] = -1;
        tags[NW + wl] = -1;
    }
    Walker st;
    bool ends_here = false;
    const int pending = w < a.num_items ? balanced_run<Walker>(a, w, st, &ends_here) : -1;
    // every wave of the workgroup reaches this barrier (no early exits
    // above): the parked pieces and their tags are in place
    __syncthreads();
    const int hkv = a.num_kv_heads;
    if (pending >= 0) {
        // the segment this wave begins: its piece in slot 1, the later ones
        // in slot 0 of the next waves of the workgroup
        int n = 1;
        while (wl + n < NW && tags[wl + n] == pending) ++n;
        auto acc_of = [&](int k) {
            return k == 0 ? Walker::template slot_acc<1>(wl) : Walker::template slot_acc<0>(wl + k);
        };
        auto ml_of = [&](int k) {
            return k == 0 ? Walker::template slot_ml<1>(wl) : Walker::template slot_ml<0>(wl + k);
        };
        fold_slots<Walker>(a, n, acc_of, ml_of, ends_here, pending / hkv, pending % hkv,
                           2 * (size_t)w + 1);
    }
    if (wl != 0) return;
    const int s0 = tags[0];
    if (s0 >= 0) {
        // the segment begun in an earlier workgroup that goes on into this
        // one: its pieces in slot 0 of the first waves
        int n = 1;
        while (n < NW && tags[n] == s0) ++n;
        fold_slots<Walker>(
            a, n, [&](int k) { return Walker::template slot_acc<0>(k); },
            [&](int k) { return Walker::template slot_ml<0>(k); }, false, s0 / hkv, s0 % hkv,
            2 * (size_t)w);
    }
    // the merge kernel's entry for this workgroup: the segment that ends
    // here after beginning in an earlier workgroup (only s0 can), and its
    // first wave
    int wf = -1;
    for (int j = 0; j < NW; ++j) wf = tags[NW + j] >= 0 ? tags[NW + j] : wf;
    if ((threadIdx.x & 63) == 0) {
        a.ws_info[2 * blockIdx.x] = wf >= 0 ? s0 : -1;
        a.ws_info[2 * blockIdx.x + 1] = wf;
    }
}

// Finish the balanced schedule. Wave (b, n) merges column n of the segment
// that ends in workgroup b after beginning in an earlier one, if any
// (ws_info[2b] = seq * Hkv + g, ws_info[2b + 1] = wf, the first wave holding
// a piece). Wave wf wrote record 2 wf + 1, the first wave of each later
// workgroup up to b record 2 v; a record holds one row per column. The
// records are folded with the log-sum-exp rule (fold_records). NW: waves per
// workgroup of the decode kernel.
template <int D, int NW>
__global__ __launch_bounds__(64 * kWaves)
void balanced_reduce_kernel(const AttnParams a) {
    const int cols = a.num_queries * a.group;
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int groups = (a.num_items + NW - 1) / NW;
    if (item >= groups * cols) return;
    const int b = item / cols, n = item % cols;
    const int seg = a.ws_info[2 * b];
    if (seg < 0) return;
    const int wf = a.ws_info[2 * b + 1];
    const int wg0 = wf / NW;
    fold_records<D>(a, 1 + b - wg0,
                    [&](int r) {
                        return (r == 0 ? 2 * (size_t)wf + 1 : 2 * (size_t)(wg0 + r) * NW) *
                                   cols + n;
                    },
                    out_row(a, seg / a.num_kv_heads, seg % a.num_kv_heads, n));
}

// Waves of a balanced kernel instance that fit on one compute unit at once
// (register-limited), queried once per instance.
template <class Walker>
int balanced_resident_waves_per_cu() {
    constexpr int NW = Walker::kGroupWaves;
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int groups = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &groups, reinterpret_cast<const void*>(&paged_decode_balanced_kernel<Walker>),
            64 * NW, 0) != hipSuccess || groups <= 0)
        return -1;
    v = groups * NW;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

// The balanced schedule: persistent waves, then the merge of split segments.
// It runs the walker's own instance for the schedule (Walker::Balanced, whose
// workgroups hold kGroupWaves waves).
template <class AnyWalker>
hipError_t launch_balanced(const AttnParams& a_in, hipStream_t stream) {
    using Walker = typename AnyWalker::Balanced;
    constexpr int D = Walker::D, G = Walker::G, NW = Walker::kGroupWaves;
    AttnParams a = a_in;
    // the LDS slots hold kSlotCols columns of a segment
    if (a.num_queries * G > Walker::kSlotCols) return hipErrorInvalidValue;
    // a.num_items holds the compute-unit count; launch at most as many
    // persistent waves as are resident together, so that all of them start
    // at once and finish together
    const int resident = balanced_resident_waves_per_cu<Walker>();
    if (resident <= 0) return hipErrorInvalidValue;
    // A wave that moves on to the next segment waits for two dependent reads
    // (the table window, then the first K/V chunk) with little else in
    // flight. When segments outnumber twice the waves, every wave switches
    // several times, and as many waves as fit keep the links busy meanwhile
    // (LLaMA-13B, 10,240 segments: 426 -> 414 us); with fewer segments the
    // walker's own count is faster (OPT-13B, 2,560 segments: 224 vs 228 us).
    int want = Walker::kBalancedWavesPerCU;
    if ((long long)a.num_seqs * a.num_kv_heads > 2LL * a.num_items * want) want = resident;
    const int per_cu = resident < want ? resident : want;
    const long long w = (long long)a.num_items * per_cu;
    a.num_items = (int)(w < kMaxBalancedWaves ? w : kMaxBalancedWaves);
    const int cols = a.num_queries * G;
    if (stage_walks(a.stage)) {
        hipLaunchKernelGGL((paged_decode_balanced_kernel<Walker>),
                           dim3((a.num_items + NW - 1) / NW), dim3(64 * NW), 0, stream, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess || !stage_merges(a.stage)) return err;
    }
    const int groups = (a.num_items + NW - 1) / NW;
    hipLaunchKernelGGL((balanced_reduce_kernel<D, NW>), dim3((groups * cols + kWaves - 1) / kWaves),
                       dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

// Single pass or fixed partitions, then the reduce of split sequences.
template <class Walker>
hipError_t launch_partitioned(const AttnParams& a, hipStream_t stream) {
    constexpr int D = Walker::D, G = Walker::G;
    const int cols = a.num_queries * G;
    if (stage_walks(a.stage)) {
        hipLaunchKernelGGL((paged_decode_kernel<Walker>), dim3((a.num_items + kWaves - 1) / kWaves),
                           dim3(64 * kWaves), 0, stream, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.max_parts <= 1 || !stage_merges(a.stage)) return hipSuccess;
    hipLaunchKernelGGL((lse_reduce_kernel<D>),
                       dim3((a.num_seqs * a.num_kv_heads * cols + kWaves - 1) / kWaves),
                       dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

template <class Walker>
hipError_t launch_walker(const AttnParams& a, hipStream_t stream) {
    return a.balanced ? launch_balanced<Walker>(a, stream) : launch_partitioned<Walker>(a, stream);
}

// Matrix cores for 16-bit K/V with head_dim 128 and 4 or 8 query heads per
// kv head; the vector walker otherwise. STREAM selects the K/V load policy.
template <typename S, int D, int G, bool STREAM>
using DecodeWalker = std::conditional_t<S::bytes == 2 && D == 128 && (G == 4 || G == 8),
                                        MfmaWalker<S, G, STREAM>, VecWalker<S, D, G, STREAM>>;

template <typename S, int D, int G, bool STREAM>
hipError_t launch_typed(const AttnParams& a, hipStream_t stream) {
    using Vec = VecWalker<S, D, G, STREAM>;
    if constexpr (STREAM && !std::is_same_v<DecodeWalker<S, D, G, STREAM>, Vec>) {
        // PKV_WALKER_VECTOR: grouped heads on the vector units, for comparison
        if (a.force_vector) return launch_walker<Vec>(a, stream);
    }
    return launch_walker<DecodeWalker<S, D, G, STREAM>>(a, stream);
}

// The decode walker for FP8 pools under fixed partitions: the vector walker
// for one query head per kv head (q in Q), the matrix cores for more.
template <typename Q, int G, bool STREAM>
using Fp8DecodeWalker = std::conditional_t<G == 1, Fp8VecWalker<Q, 1, STREAM, 4>,
                                           MfmaWalker<Q, G, STREAM, true>>;

// Sampling groups: one launch of the shared partitions on the matrix cores
// (one wave per group, kv head and partition) and every sequence's own
// partitions, then the reduce over both. (Measured on MI355X: one launch
// beats two back-to-back launches by 11% on the 32 x 8 sampling layer.)
// FP8: E4M3 pools, S is q's type.
template <typename S, int G, bool STREAM, bool FP8>
hipError_t launch_grouped_typed(const AttnParams& a, hipStream_t stream) {
    using SeqWalker = std::conditional_t<FP8, Fp8DecodeWalker<S, G, STREAM>,
                                         DecodeWalker<S, 128, G, STREAM>>;
    if (a.max_parts <= 1) return launch_partitioned<SeqWalker>(a, stream);
    const long long group_items =
        (long long)(a.num_seqs / a.group_size) * a.num_kv_heads * a.max_parts;
    const long long total = group_items + a.num_items;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    if (stage_walks(a.stage)) {
        hipLaunchKernelGGL((paged_decode_grouped_kernel<MfmaWalker<S, G, STREAM, FP8>, SeqWalker>),
                           dim3((unsigned)((total + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0,
                           stream, a, (int)group_items);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess || !stage_merges(a.stage)) return err;
    }
    hipLaunchKernelGGL((lse_reduce_kernel<128>),
                       dim3((a.num_seqs * a.num_kv_heads * G + kWaves - 1) / kWaves),
                       dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

template <typename S, bool STREAM, bool FP8>
hipError_t launch_grouped_group(const AttnParams& a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_grouped_typed<S, 1, STREAM, FP8>(a, stream);
        case 2: return launch_grouped_typed<S, 2, STREAM, FP8>(a, stream);
        case 4: return launch_grouped_typed<S, 4, STREAM, FP8>(a, stream);
        case 8: return launch_grouped_typed<S, 8, STREAM, FP8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename S, bool FP8>
hipError_t launch_grouped_policy(const AttnParams& a, hipStream_t stream) {
    return a.kv_stream ? launch_grouped_group<S, true, FP8>(a, stream)
                       : launch_grouped_group<S, false, FP8>(a, stream);
}

template <typename S, int D, bool STREAM>
hipError_t launch_group(const AttnParams& a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_typed<S, D, 1, STREAM>(a, stream);
        case 2: return launch_typed<S, D, 2, STREAM>(a, stream);
        case 4: return launch_typed<S, D, 4, STREAM>(a, stream);
        case 8: return launch_typed<S, D, 8, STREAM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename S, bool STREAM>
hipError_t launch_dim(const AttnParams& a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return launch_group<S, 64, STREAM>(a, stream);
        case 128: return launch_group<S, 128, STREAM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename S>
hipError_t launch_policy(const AttnParams& a, hipStream_t stream) {
    return a.kv_stream ? launch_dim<S, true>(a, stream) : launch_dim<S, false>(a, stream);
}

// FP8 pools: the vector walker for one query head per kv head, the matrix
// cores for 2, 4 or 8 (q in fp16 / bf16; the entry point rejects fp32 q
// there). head_dim is 128.
template <typename Q, int G, bool STREAM>
hipError_t launch_fp8_typed(const AttnParams& a, hipStream_t stream) {
    // the vector walker keeps four loads of K and V per chunk in flight, two
    // under the balanced schedule with fp32 q (four spill registers there)
    if constexpr (G == 1)
        return a.balanced ? launch_balanced<Fp8VecWalker<Q, G, STREAM, Q::bytes == 2 ? 4 : 2>>(a, stream)
                          : launch_partitioned<Fp8VecWalker<Q, G, STREAM, 4>>(a, stream);
    else if constexpr (Q::bytes == 2)
        return launch_walker<Fp8MfmaWalker<Q, G, STREAM>>(a, stream);
    else
        return hipErrorInvalidValue;
}

template <typename Q, bool STREAM>
hipError_t launch_fp8_group(const AttnParams& a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_fp8_typed<Q, 1, STREAM>(a, stream);
        case 2: return launch_fp8_typed<Q, 2, STREAM>(a, stream);
        case 4: return launch_fp8_typed<Q, 4, STREAM>(a, stream);
        case 8: return launch_fp8_typed<Q, 8, STREAM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename Q>
hipError_t launch_fp8_policy(const AttnParams& a, hipStream_t stream) {
    return a.kv_stream ? launch_fp8_group<Q, true>(a, stream) : launch_fp8_group<Q, false>(a, stream);
}

// Chunked prefill (more than 16 columns per kv head) with 16-bit K/V: one
// workgroup per (sequence, kv head, partition, group of kWaves * NT
// 16-column tiles). Its waves share every K/V chunk (MfmaWalker::walk_shared:
// loaded once, straight into LDS, two chunks ahead) and each runs NT tiles
// on it, so the cache is read once per group instead of once per tile.
// Partial rows as in paged_decode_kernel.
// The sequence of rank r when sequences are ordered by decreasing length
// (ties by index), for up to 64 sequences; sequence r beyond that. Workgroups
// take sequences in this order, so the longest walks start first and the
// ones that wait for a free compute unit are the shortest.
__device__ __forceinline__ int seq_of_length_rank(const AttnParams& a, int r) {
    if (a.num_seqs > 64) return r;
    const int lane = threadIdx.x & 63;
    const int Lj = lane < a.num_seqs ? clamp_len(a, a.seq_lens[lane]) : -1;
    int rank = 0;
    for (int k = 0; k < a.num_seqs; ++k) {
        const int Lk = __shfl(Lj, k, 64);
        rank += (Lk > Lj || (Lk == Lj && k < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(lane < a.num_seqs && rank == r);
    return hit ? __builtin_ctzll(hit) : r;
}

template <class Walker>
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(Walker::kMinWavesPerSimd)))
void paged_prefill_kernel(const AttnParams a) {
    constexpr int D = Walker::D, G = Walker::G;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int groups = (a.col_tiles + a.tiles_per_item - 1) / a.tiles_per_item;
    const int sg = blockIdx.x % groups;              // the group of tiles of this workgroup
    const int rest = blockIdx.x / groups;
    const int g = rest % a.num_kv_heads;
    const int seq = __builtin_amdgcn_readfirstlane(
        seq_of_length_rank(a, (rest / a.num_kv_heads) % a.num_seqs));
    const int part = rest / (a.num_kv_heads * a.num_seqs);
    const int raw_len = a.seq_lens[seq];
    report_if(a.err, threadIdx.x == 0 && g == 0 && part == 0 && sg == 0 &&
                     (raw_len < 0 || raw_len > a.max_tokens), PKV_ERRBIT_LENGTH);
    const int L = clamp_len(a, raw_len);
    const int cols = a.num_queries * G;
    // the columns of this wave: tiles tiles_per_item * sg + Walker::kTiles * wave ..
    const int c0 = 16 * (a.tiles_per_item * sg + Walker::kTiles * wave);
    const int c1 = c0 + 16 * Walker::kTiles < cols ? c0 + 16 * Walker::kTiles : cols;
    // every branch below is uniform over the workgroup: the walk's barriers
    // need all four waves
    const int reach = L > 0 ? group_reach(a, L, sg) : 0;
    if (reach <= 0) {                                // padding row, or queries before the start
        if (part == 0 && c0 < cols) write_zero_cols<D>(a, seq, g, c0, c1, lane);
        return;
    }
    const int part_len = a.part_tokens > 0 ? a.part_tokens : reach;
    const int nparts = (reach + part_len - 1) / part_len;
    if (part >= nparts) return;
    const int t_begin = part * part_len;
    const int t_stop = (t_begin + part_len < reach) ? t_begin + part_len : reach;
    Walker st;
    st.init(lane);
    st.begin(a, seq, g, L, kWaves * sg + wave);
    st.walk_shared(t_begin, t_stop, a.scale * kLog2e, wave);
    if (c0 >= cols) return;                          // a wave past the last column
    if (nparts == 1) {
        st.write_final(a, seq, g);
    } else {
        const size_t row0 =
            ((size_t)seq * a.num_kv_heads * cols + (size_t)g * cols + c0) * a.max_parts + part;
        st.write_partial(a, row0, (size_t)a.max_parts);
    }
}

// Tiles each wave runs: with shared chunks (16-bit K/V) four waves of
// kPrefillTiles tiles walk together, two waves per SIMD (measured on MI355X
// on the OPT-13B prefill layer: 289 us, against 306 us for one tile per wave
// and 385-397 us for two or four tiles at one wave per SIMD; with the output
// tiles moved into the chunk buffers, so that two workgroups fit a compute
// unit's LDS, and the longest sequences dispatched first: 243 us); FP8 pools
// use one wave of kPrefillTilesFp8 tiles per work item, one wave per SIMD
// (two tiles per wave: 316 us against 622 us for one, on 16-bit pools).
#ifndef PKV_PREFILL_TILES
#define PKV_PREFILL_TILES 2
#endif
#ifndef PKV_PREFILL_WAVES_PER_SIMD
#define PKV_PREFILL_WAVES_PER_SIMD 2
#endif
constexpr int kPrefillTiles = PKV_PREFILL_TILES;
constexpr int kPrefillWavesPerSimd = PKV_PREFILL_WAVES_PER_SIMD;
constexpr int kPrefillTilesFp8 = 2;

template <typename S, int G, bool STREAM, bool FP8>
hipError_t launch_multi_typed(const AttnParams& a, hipStream_t stream) {
    if (a.col_tiles > 1) {
        AttnParams b = a;
        if constexpr (FP8) {
            b.tiles_per_item = kPrefillTilesFp8;
            const long long groups = (b.col_tiles + b.tiles_per_item - 1) / b.tiles_per_item;
            b.num_items = (int)((long long)b.max_parts * b.num_seqs * b.num_kv_heads * groups);
            return launch_partitioned<MfmaWalker<S, G, STREAM, FP8, kPrefillTilesFp8>>(b, stream);
        } else {
            using W = MfmaWalker<S, G, STREAM, false, kPrefillTiles, kPrefillWavesPerSimd, true>;
            b.tiles_per_item = kWaves * kPrefillTiles;
            const long long groups = (b.col_tiles + b.tiles_per_item - 1) / b.tiles_per_item;
            const long long wgs = (long long)b.max_parts * b.num_seqs * b.num_kv_heads * groups;
            if (wgs > INT32_MAX) return hipErrorInvalidValue;
            if (stage_walks(b.stage)) {
                hipLaunchKernelGGL((paged_prefill_kernel<W>), dim3((unsigned)wgs),
                                   dim3(64 * kWaves), 0, stream, b);
                const hipError_t err = hipGetLastError();
                if (err != hipSuccess) return err;
            }
            if (b.max_parts <= 1 || !stage_merges(b.stage)) return hipSuccess;
            hipLaunchKernelGGL((lse_reduce_kernel<128>),
                               dim3((b.num_seqs * b.num_kv_heads * b.num_queries * G + kWaves - 1) /
                                    kWaves),
                               dim3(64 * kWaves), 0, stream, b);
            return hipGetLastError();
        }
    }
    return launch_walker<MfmaWalker<S, G, STREAM, FP8>>(a, stream);
}

template <typename S, bool STREAM, bool FP8>
hipError_t launch_multi_group(const AttnParams& a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_multi_typed<S, 1, STREAM, FP8>(a, stream);
        case 2: return launch_multi_typed<S, 2, STREAM, FP8>(a, stream);
        case 4: return launch_multi_typed<S, 4, STREAM, FP8>(a, stream);
        case 8: return launch_multi_typed<S, 8, STREAM, FP8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename S, bool FP8>
hipError_t launch_multi_policy(const AttnParams& a, hipStream_t stream) {
    return a.kv_stream ? launch_multi_group<S, true, FP8>(a, stream)
                       : launch_multi_group<S, false, FP8>(a, stream);
}

}  // namespace

// Several new tokens per sequence: always the matrix-core walker, whose 16
// columns hold (new token, query head) pairs with their own causal limits.
// FP8 pools: E4M3 codes widened to q's type on the way into the matrix cores.
hipError_t launch_paged_attention_multi(const AttnParams& a, hipStream_t stream) {
    if (a.head_dim != 128 || (a.col_tiles > 1 && a.balanced)) return hipErrorInvalidValue;
    const int t = a.dtype == PKV_FP8_E4M3 ? a.q_dtype : a.dtype;
    const bool fp8 = a.dtype == PKV_FP8_E4M3;
    switch (t) {
        case PKV_F16:
            return fp8 ? launch_multi_policy<F16, true>(a, stream)
                       : launch_multi_policy<F16, false>(a, stream);
        case PKV_BF16:
            return fp8 ? launch_multi_policy<BF16, true>(a, stream)
                       : launch_multi_policy<BF16, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// Parallel-sampling groups: 16-bit K/V or FP8 pools with 16-bit q, head_dim
// 128, fixed partitions.
hipError_t launch_paged_attention_grouped(const AttnParams& a, hipStream_t stream) {
    if (a.head_dim != 128 || a.balanced || a.group_size * a.group > 16) return hipErrorInvalidValue;
    const int t = a.dtype == PKV_FP8_E4M3 ? a.q_dtype : a.dtype;
    const bool fp8 = a.dtype == PKV_FP8_E4M3;
    switch (t) {
        case PKV_F16:
            return fp8 ? launch_grouped_policy<F16, true>(a, stream)
                       : launch_grouped_policy<F16, false>(a, stream);
        case PKV_BF16:
            return fp8 ? launch_grouped_policy<BF16, true>(a, stream)
                       : launch_grouped_policy<BF16, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_attention_fp8(const AttnParams& a, hipStream_t stream) {
    if (a.head_dim != 128) return hipErrorInvalidValue;
    switch (a.q_dtype) {
        case PKV_F32: return launch_fp8_policy<F32>(a, stream);
        case PKV_F16: return launch_fp8_policy<F16>(a, stream);
        case PKV_BF16: return launch_fp8_policy<BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_attention(const AttnParams& a, hipStream_t stream) {
    switch (a.dtype) {
        case PKV_F32: return launch_policy<F32>(a, stream);
        case PKV_F16: return launch_policy<F16>(a, stream);
        case PKV_BF16: return launch_policy<BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
