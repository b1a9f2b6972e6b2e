// Steps 2 and 3: indexer scores and the causal top-k block selection, fused.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache",
// section "Selection is a weighted ReLU score, not attention softmax": for
// query t and provider group g the score of historical block r sums, over the
// group's four indexer heads, a signed weight times ReLU of the dot product
// of the BF16 indexer query with the (E4M3-valued, BF16-widened) summary; no
// softmax; only r < floor(t/8) compete for the K slots, equal scores go to
// the lower block id.  Section "A configured million-token window is not a
// validated million-token launch" shows why the [G*N, R] FP32 score matrix
// must not be materialised (512 GiB per rank at 1M tokens): here no score
// leaves the wavefront that computed it unless it may still be selected.
//
// Mapping (one wavefront per query and candidate split):
//   * the query's 4 groups x 4 heads of q_hat are exactly the 16 rows of a
//     v_mfma_f32_16x16x32_bf16 A operand, so the four groups share every
//     store row the wavefront reads;
//   * a 16-block tile of the store is the B operand, read straight from HBM /
//     L2 into registers (16 B per lane per 32-wide k step), two tiles ahead;
//   * the result layout puts all 4 heads of (group, block) in one lane, so
//     the weighted ReLU sum is in-lane;
//   * each group's selection is a streaming top-k: an LDS buffer of `cap`
//     (key, block) entries in ascending block order, an acceptance threshold
//     (the current k-th key) and a radix-select compaction back to k entries
//     when the buffer is nearly full.  Keys are order-preserving uint32 images
//     of the fp32 scores (-0 folded into +0); ties keep the earlier entry,
//     which is the lower block id because blocks arrive in ascending order.
// A decode-sized call (few queries) splits each query's candidates over
// several wavefronts; index_merge_kernel then selects from their lists.
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;


__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
    return v;
}

// Keep the k entries with the largest keys among (key, idx)[0..n), n > k,
// preferring earlier entries among equal keys, in their original order.
// Runs on one wavefront; `hist` is 256 words of LDS owned by it.  Radix
// select with 8-bit digits starting at the highest bit in which the keys
// differ (all-equal rows, e.g. rows of zero scores, need no histogram).
// Returns the smallest kept key: the acceptance threshold for later,
// higher-numbered candidates.
__device__ uint32_t compact_topk(uint32_t* key, int32_t* idx, int n, int k, uint32_t* hist) {
    const int lane = lane_id();
    const uint32_t k0 = key[0];
    uint32_t diff = 0;
    for (int i = lane; i < n; i += 64) diff |= key[i] ^ k0;
    diff = wave_or(diff);
    uint32_t prefix = k0;
    int krem = k;
    if (diff != 0) {
        const int hb = 31 - __builtin_clz(diff);
        uint32_t pmask = hb == 31 ? 0u : (0xFFFFFFFFu << (hb + 1));
        prefix = k0 & pmask;
#pragma unroll 1
        for (int hi = hb; hi >= 0;) {
            const int lo = hi >= 7 ? hi - 7 : 0;
            const int nbins = 1 << (hi - lo + 1);
            const uint32_t dmask = (uint32_t)nbins - 1u;
            for (int b = lane; b < 256; b += 64) hist[b] = 0u;
            wave_lds_sync();
            for (int i = lane; i < n; i += 64) {
                const uint32_t kk = key[i];
                if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> lo) & dmask], 1u);
            }
            wave_lds_sync();
            // lane L owns digits nbins-1-4L down to nbins-4-4L
            uint32_t h[4];
            uint32_t tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = nbins - 1 - 4 * lane - j;
                h[j] = d >= 0 ? hist[d] : 0u;
                tot += h[j];
            }
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t up = __shfl_up(incl, o, 64);
                if (lane >= o) incl += up;
            }
            uint32_t above = incl - tot;   // entries with a larger digit
            int found = -1;
            uint32_t above_found = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (found < 0 && h[j] > 0 && above + h[j] >= (uint32_t)krem) {
                    found = nbins - 1 - 4 * lane - j;
                    above_found = above;
                }
                above += h[j];
            }
            const uint64_t fm = __ballot(found >= 0);
            const int src = (int)__builtin_ctzll(fm);
            const int digit = __shfl(found, src, 64);
            const uint32_t ab = __shfl(above_found, src, 64);
            prefix |= (uint32_t)digit << lo;
            pmask |= dmask << lo;
            krem -= (int)ab;
            wave_lds_sync();
            hi = lo - 1;
        }
    }
    // stable in-place compaction: all keys > v, and the first krem keys == v
    const uint32_t v = prefix;
    int out = 0, eq_seen = 0;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        uint32_t kk = 0;
        int32_t ii = 0;
        if (i < n) {
            kk = key[i];
            ii = idx[i];
        }
        const bool gt = (i < n) && kk > v;
        const bool eq = (i < n) && kk == v;
        const uint64_t em = __ballot(eq);
        const int er = eq_seen + (int)lanes_below(em);
        const bool keep = gt || (eq && er < krem);
        const uint64_t km = __ballot(keep);
        const int pos = out + (int)lanes_below(km);
        if (keep) {
            key[pos] = kk;
            idx[pos] = ii;
        }
        out += __popcll(km);
        eq_seen += __popcll(em);
    }
    wave_lds_sync();
    return v;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *(const uint4*)p; }

// Indexer query of (row, t): RMSNorm, rotary span at position t, bf16; the
// lane's A-operand fragments (row m = 4*group + head, k-chunk qq).  Writes
// q_hat when asked.
__device__ __forceinline__ void index_query_fragments(const IndexArgs& a, int64_t row, int64_t t,
                                                      int qq, int m, bool write_qhat,
                                                      bf16x8 (&afrag)[4]) {
    // ---- indexer query: RMSNorm, rotary span, bf16 (A operand rows) ----
    const uint16_t* qrow = a.q_idx + (row * (kGroups * kIdxHeads) + m) * kIdxDim + 8 * qq;
    float x[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 raw = load16(qrow + 32 * kk);
        uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[kk][2 * e] = bf16_to_f32(w4[e] & 0xFFFFu);
            x[kk][2 * e + 1] = bf16_to_f32(w4[e] >> 16);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kIdxDim) + a.eps);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float gam[8];
        if (a.rms_gamma) {
            uint4 gr = load16(a.rms_gamma + 32 * kk + 8 * qq);
            uint32_t g4[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gam[2 * e] = bf16_to_f32(g4[e] & 0xFFFFu);
                gam[2 * e + 1] = bf16_to_f32(g4[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gam[e] = 1.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[kk][e] = x[kk][e] * inv * gam[e];
    }
    // rotary span = dims 0..31 = k-chunk 0: lanes qq=0,1 hold pairs' first
    // halves (dims 8qq+e), lanes qq=2,3 the second halves; partner = lane ^ 32
    {
        const bool first = qq < 2;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __shfl_xor(x[0][e], 32, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float c, s;
            rope_cos_sin(t, a.theta[8 * (qq & 1) + e], &c, &s);
            x[0][e] = first ? (x[0][e] * c - p[e] * s) : (p[e] * s + x[0][e] * c);
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 packed;
        packed.x = f32_to_bf16(x[kk][0]) | (f32_to_bf16(x[kk][1]) << 16);
        packed.y = f32_to_bf16(x[kk][2]) | (f32_to_bf16(x[kk][3]) << 16);
        packed.z = f32_to_bf16(x[kk][4]) | (f32_to_bf16(x[kk][5]) << 16);
        packed.w = f32_to_bf16(x[kk][6]) | (f32_to_bf16(x[kk][7]) << 16);
        afrag[kk] = as_bf16x8(packed);
        if (a.q_hat_out && write_qhat)
            *(uint4*)(a.q_hat_out + (row * (kGroups * kIdxHeads) + m) * kIdxDim + 32 * kk + 8 * qq) =
                packed;
    }

}

__global__ __launch_bounds__(64) void index_topk_kernel(SeqTable seqs, IndexArgs a) {
    extern __shared__ uint32_t lds[];
    const int cap = a.cap;
    uint32_t* keys = lds;                               // [4][cap]
    int32_t* idxs = (int32_t*)(lds + 4 * cap);          // [4][cap]
    uint32_t* hist = lds + 8 * cap;                     // [256]

    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / a.n_split;
    const int split = blockIdx.x % a.n_split;
    if (qi >= sq.n_q) return;
    const int64_t t = sq.pos0 + qi;
    const int64_t row = sq.q_offset + qi;
    const int lane = lane_id();
    const int qq = lane >> 4;     // operand k-chunk; result group
    const int m = lane & 15;      // operand row (4*group + head); result column
    bf16x8 afrag[4];
    index_query_fragments(a, row, t, qq, m, true, afrag);

    // this lane's results belong to group qq, heads 0..3
    const float4 wv = *(const float4*)(a.w + (row * kGroups + qq) * kIdxHeads);

    // ---- candidates of this split: r in [r_lo, r_hi), r < floor(t/B) ----
    const int64_t nb = t / a.block_size;
    const int64_t r_lo = (int64_t)split * a.split_blocks;
    const int64_t r_hi = nb < r_lo + a.split_blocks ? nb : r_lo + a.split_blocks;
    const uint16_t* store = a.store + sq.store_offset * kIdxDim + 8 * qq;

    uint32_t thr = 0u;             // accept keys above it (0: accept every score)
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, cnt3 = 0;
    uint32_t* const mykeys = keys + qq * cap;
    int32_t* const myidx = idxs + qq * cap;

    // B operand of tile r0: lane holds store[r0 + m][32kk + 8qq .. +7]
    uint4 b0[4], b1[4];
    auto row_of = [&](int64_t r0) { return (r0 + m < r_hi ? r0 + m : r_lo) * kIdxDim; };
    if (r_lo < r_hi) {
        const int64_t o = row_of(r_lo);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = load16(store + o + 32 * kk);
    }
    if (r_lo + 16 < r_hi) {
        const int64_t o = row_of(r_lo + 16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b1[kk] = load16(store + o + 32 * kk);
    }
    for (int64_t r0 = r_lo; r0 < r_hi; r0 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_16x16x32(afrag[kk], as_bf16x8(b0[kk]), acc);
        // rotate the two-tile register pipeline: tile r0+32 goes in flight
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = b1[kk];
        if (r0 + 32 < r_hi) {
            const int64_t o = row_of(r0 + 32);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) b1[kk] = load16(store + o + 32 * kk);
        }
        float s = wv.x * fmaxf(acc[0], 0.f);
        s += wv.y * fmaxf(acc[1], 0.f);
        s += wv.z * fmaxf(acc[2], 0.f);
        s += wv.w * fmaxf(acc[3], 0.f);
        const int64_t rr = r0 + m;
        const uint32_t key = score_key(s);
        const bool take = (rr < r_hi) && key > thr;
        const uint64_t am = __ballot(take);
        if (am == 0) continue;                    // the common case once the threshold is up
        const uint32_t seg = (uint32_t)(am >> (16 * qq)) & 0xFFFFu;
        const int mycnt = qq == 0 ? cnt0 : qq == 1 ? cnt1 : qq == 2 ? cnt2 : cnt3;
        if (take) {
            const int pos = mycnt + __popc(seg & ((1u << m) - 1u));
            mykeys[pos] = key;
            myidx[pos] = (int32_t)rr;
        }
        cnt0 += __popc((uint32_t)am & 0xFFFFu);
        cnt1 += __popc((uint32_t)(am >> 16) & 0xFFFFu);
        cnt2 += __popc((uint32_t)(am >> 32) & 0xFFFFu);
        cnt3 += __popc((uint32_t)(am >> 48) & 0xFFFFu);
        if (cnt0 > cap - 16 || cnt1 > cap - 16 || cnt2 > cap - 16 || cnt3 > cap - 16) {
            wave_lds_sync();
            if (cnt0 > cap - 16) {
                const uint32_t v = compact_topk(keys, idxs, cnt0, a.topk, hist);
                cnt0 = a.topk;
                if (qq == 0) thr = v;
            }
            if (cnt1 > cap - 16) {
                const uint32_t v = compact_topk(keys + cap, idxs + cap, cnt1, a.topk, hist);
                cnt1 = a.topk;
                if (qq == 1) thr = v;
            }
            if (cnt2 > cap - 16) {
                const uint32_t v = compact_topk(keys + 2 * cap, idxs + 2 * cap, cnt2, a.topk, hist);
                cnt2 = a.topk;
                if (qq == 2) thr = v;
            }
            if (cnt3 > cap - 16) {
                const uint32_t v = compact_topk(keys + 3 * cap, idxs + 3 * cap, cnt3, a.topk, hist);
                cnt3 = a.topk;
                if (qq == 3) thr = v;
            }
        }
    }
    wave_lds_sync();

    // ---- final selection and output ----
    int cnts[4] = {cnt0, cnt1, cnt2, cnt3};
#pragma unroll 1
    for (int g = 0; g < kGroups; ++g) {
        int c = cnts[g];
        if (c > a.topk) {
            compact_topk(keys + g * cap, idxs + g * cap, c, a.topk, hist);
            c = a.topk;
        }
        const int64_t rg = row * kGroups + g;
        int32_t* sel = a.sel + rg * a.topk;
        float* ssc = a.sel_scores ? a.sel_scores + rg * a.topk : nullptr;
        for (int j = lane; j < a.topk; j += 64) {
            const bool in = j < c;
            sel[j] = in ? idxs[g * cap + j] : -1;
            if (ssc) ssc[j] = in ? key_score(keys[g * cap + j]) : 0.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode-sized calls (few queries, long histories): the candidates of each
// query are spread over many wavefronts that only score (same MFMA mapping as
// above) and write the order-preserving score keys to the workspace at their
// block ids; one workgroup per (query, group) then selects.  Keys cost 4 B
// per (query, group, candidate): 33 MB for 64 sequences of 256K tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void index_score_kernel(SeqTable seqs, IndexArgs a) {
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / a.n_split;
    const int split = blockIdx.x % a.n_split;
    if (qi >= sq.n_q) return;
    const int64_t t = sq.pos0 + qi;
    const int64_t row = sq.q_offset + qi;
    const int64_t nb = t / a.block_size;
    const int64_t r_lo = (int64_t)split * a.split_blocks;
    const int64_t r_hi = nb < r_lo + a.split_blocks ? nb : r_lo + a.split_blocks;
    if (r_lo >= r_hi && !(split == 0 && a.q_hat_out)) return;
    const int lane = lane_id();
    const int qq = lane >> 4;
    const int m = lane & 15;
    bf16x8 afrag[4];
    index_query_fragments(a, row, t, qq, m, split == 0, afrag);
    if (r_lo >= r_hi) return;
    const float4 wv = *(const float4*)(a.w + (row * kGroups + qq) * kIdxHeads);
    const uint16_t* store = a.store + sq.store_offset * kIdxDim + 8 * qq;
    uint32_t* keys = a.part_key + (row * kGroups + qq) * a.key_stride;
    uint4 b0[4], b1[4];
    auto row_of = [&](int64_t r0) { return (r0 + m < r_hi ? r0 + m : r_lo) * kIdxDim; };
    {
        const int64_t o = row_of(r_lo);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = load16(store + o + 32 * kk);
    }
    if (r_lo + 16 < r_hi) {
        const int64_t o = row_of(r_lo + 16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b1[kk] = load16(store + o + 32 * kk);
    }
    for (int64_t r0 = r_lo; r0 < r_hi; r0 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_16x16x32(afrag[kk], as_bf16x8(b0[kk]), acc);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = b1[kk];
        if (r0 + 32 < r_hi) {
            const int64_t o = row_of(r0 + 32);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) b1[kk] = load16(store + o + 32 * kk);
        }
        float s = wv.x * fmaxf(acc[0], 0.f);
        s += wv.y * fmaxf(acc[1], 0.f);
        s += wv.z * fmaxf(acc[2], 0.f);
        s += wv.w * fmaxf(acc[3], 0.f);
        if (r0 + m < r_hi) keys[r0 + m] = score_key(s);
    }
}

// Top-k of one (query, group) from its score keys: the k largest, equal keys
// to the lower block id, output in ascending block id.  Four wavefronts:
// keys staged in LDS when they fit, one histogram per wavefront per radix
// digit (summed by wavefront 0), and the ordered output written from four
// contiguous segments whose offsets come from one exchange.
constexpr int kSelectLdsKeys = 36864;

__global__ __launch_bounds__(256) void index_select_kernel(SeqTable seqs, IndexArgs a) {
    extern __shared__ uint32_t skeys[];
    __shared__ uint32_t hist[4][256];
    __shared__ uint32_t red[4];
    __shared__ int s_cnt[2][4];
    __shared__ int s_digit, s_above;
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / kGroups;
    const int g = blockIdx.x % kGroups;
    if (qi >= sq.n_q) return;
    const int64_t t = sq.pos0 + qi;
    const int64_t rg = (sq.q_offset + qi) * kGroups + g;
    const int n = (int)(t / a.block_size);
    const int K = a.topk;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint32_t* gkeys = a.part_key + rg * a.key_stride;
    const bool in_lds = n <= kSelectLdsKeys;
    if (in_lds)
        for (int i = tid; i < n; i += 256) skeys[i] = gkeys[i];
    const uint32_t* keys = in_lds ? skeys : gkeys;
    int32_t* sel = a.sel + rg * K;
    float* ssc = a.sel_scores ? a.sel_scores + rg * K : nullptr;
    __syncthreads();

    // selection rule: an entry is kept iff (key & pmask) > prefix, or
    // (key & pmask) == prefix and fewer than krem such entries precede it
    uint32_t prefix = 0, pmask = 0;   // n <= K: pmask 0 keeps everything
    int krem = K;
    if (n > K) {
        const uint32_t k0 = keys[0];
        uint32_t diff = 0;
        for (int i = tid; i < n; i += 256) diff |= keys[i] ^ k0;
        diff = wave_or(diff);
        if (lane == 0) red[w] = diff;
        __syncthreads();
        diff = red[0] | red[1] | red[2] | red[3];
        prefix = k0;
        pmask = 0xFFFFFFFFu;
        if (diff != 0) {
            const int hb = 31 - __builtin_clz(diff);
            pmask = hb == 31 ? 0u : (0xFFFFFFFFu << (hb + 1));
            prefix = k0 & pmask;
            for (int hi = hb; hi >= 0;) {
                const int lo = hi >= 7 ? hi - 7 : 0;
                const int nbins = 1 << (hi - lo + 1);
                const uint32_t dmask = (uint32_t)nbins - 1u;
                for (int b = lane; b < 256; b += 64) hist[w][b] = 0u;
                __syncthreads();
                for (int i = tid; i < n; i += 256) {
                    const uint32_t kk = keys[i];
                    if ((kk & pmask) == prefix) atomicAdd(&hist[w][(kk >> lo) & dmask], 1u);
                }
                __syncthreads();
                if (w == 0) {
                    uint32_t h[4], tot = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int d = nbins - 1 - 4 * lane - j;
                        h[j] = d >= 0 ? hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d] : 0u;
                        tot += h[j];
                    }
                    uint32_t incl = tot;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const uint32_t up = __shfl_up(incl, o, 64);
                        if (lane >= o) incl += up;
                    }
                    uint32_t above = incl - tot;
                    int found = -1;
                    uint32_t above_found = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (found < 0 && h[j] > 0 && above + h[j] >= (uint32_t)krem) {
                            found = nbins - 1 - 4 * lane - j;
                            above_found = above;
                        }
                        above += h[j];
                    }
                    const uint64_t fm = __ballot(found >= 0);
                    if (lane == (int)__builtin_ctzll(fm)) {
                        s_digit = found;
                        s_above = (int)above_found;
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)s_digit << lo;
                pmask |= dmask << lo;
                krem -= s_above;
                hi = lo - 1;
            }
        }
    }
    // ordered output: wavefront w owns entries [w*seg, (w+1)*seg)
    const int seg = (n + 255) / 256 * 64;
    const int b0 = w * seg;
    const int b1 = b0 + seg < n ? b0 + seg : n;
    int n_gt = 0, n_eq = 0;
    for (int base = b0; base < b1; base += 64) {
        const int i = base + lane;
        const uint32_t kk = i < b1 ? keys[i] & pmask : 0u;
        n_gt += __popcll(__ballot(i < b1 && kk > prefix));
        n_eq += __popcll(__ballot(i < b1 && kk == prefix));
    }
    if (lane == 0) {
        s_cnt[0][w] = n_gt;
        s_cnt[1][w] = n_eq;
    }
    __syncthreads();
    // kept before this segment: every larger masked key, min(krem, equal ones)
    int out = 0, eq_seen = 0;
    for (int j = 0; j < w; ++j) {
        out += s_cnt[0][j];
        eq_seen += s_cnt[1][j];
    }
    out += eq_seen < krem ? eq_seen : krem;
    for (int base = b0; base < b1; base += 64) {
        const int i = base + lane;
        const uint32_t kk = i < b1 ? keys[i] : 0u;
        const bool eq = i < b1 && (kk & pmask) == prefix;
        const uint64_t em = __ballot(eq);
        const int er = eq_seen + (int)lanes_below(em);
        const bool keep = i < b1 && ((kk & pmask) > prefix || (eq && er < krem));
        const uint64_t km = __ballot(keep);
        if (keep) {
            const int pos = out + (int)lanes_below(km);
            sel[pos] = i;
            if (ssc) ssc[pos] = key_score(kk);
        }
        out += __popcll(km);
        eq_seen += __popcll(em);
    }
    const int total = n <= K ? n : K;
    for (int j = total + tid; j < K; j += 256) {
        sel[j] = -1;
        if (ssc) ssc[j] = 0.0f;
    }
}

}  // namespace

size_t index_lds_bytes(int cap) { return (size_t)cap * 32u + 1024u; }

hipError_t launch_index_topk(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                             hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    const size_t lds = index_lds_bytes(a.cap);
    hipError_t e = hipFuncSetAttribute((const void*)index_topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * a.n_split), (unsigned)seqs.n);
    hipLaunchKernelGGL(index_topk_kernel, grid, dim3(64), lds, stream, seqs, a);
    return hipGetLastError();
}

hipError_t launch_index_split(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                              hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)(max_nq * a.n_split), (unsigned)seqs.n);
    hipLaunchKernelGGL(index_score_kernel, grid, dim3(64), 0, stream, seqs, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t max_b = a.key_stride;
    const size_t lds = (size_t)(max_b < kSelectLdsKeys ? max_b : kSelectLdsKeys) * sizeof(uint32_t);
    e = hipFuncSetAttribute((const void*)index_select_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid2((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL(index_select_kernel, grid2, dim3(256), lds, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
