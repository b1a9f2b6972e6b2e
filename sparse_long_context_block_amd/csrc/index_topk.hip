// Steps 2 and 3: indexer scores and the causal top-k block selection.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache",
// section "Selection is a weighted ReLU score, not attention softmax": for
// query t and provider group g the score of historical block r sums, over the
// group's four indexer heads, a signed weight times ReLU of the dot product
// of the BF16 indexer query with the (E4M3-valued, BF16-widened) summary; no
// softmax; only r < floor(t/8) compete for the K slots, equal scores go to
// the lower block id.  Section "A configured million-token window is not a
// validated million-token launch" shows why the [G*N, R] FP32 score matrix
// must not be materialised (512 GiB per rank at 1M tokens): the fused kernel
// keeps scores in the wavefront that computed them, the other paths write
// 4-byte keys for a bounded number of query rows at a time.
//
// Common MFMA mapping (every score kernel):
//   * the query's 4 groups x 4 heads of q_hat are exactly the 16 rows of a
//     v_mfma_f32_16x16x32_bf16 A operand, so the four groups share every
//     store row read;
//   * a 16-block tile of the store is the B operand (16 B per lane per
//     32-wide k step);
//   * the result layout puts all 4 heads of (group, block) in one lane, so
//     the weighted ReLU sum is in-lane.
// Keys are order-preserving uint32 images of the fp32 scores (-0 folded into
// +0).  Three paths (the host picks one per call):
//   * index_topk_kernel -- one wavefront per query, store tiles straight from
//     memory two tiles ahead, and per group a streaming top-k: an LDS buffer
//     of `cap` (key, block) entries in ascending block order, an acceptance
//     threshold (the current k-th key) and a radix-select compaction back to
//     k entries when the buffer is nearly full; ties keep the earlier entry,
//     which is the lower block id because blocks arrive in ascending order;
//   * index_score_kernel + index_select_kernel -- decode-sized calls spread
//     each query's candidates over many score wavefronts that write keys;
//   * index_score_tile_kernel + index_select_kernel -- calls of 1024+
//     queries score 16 queries per workgroup against store tiles in LDS.
#include "compress_block.hpp"

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

// Store rows as the score kernels read them: bf16 (256 B per block) or
// E4M3 codes (128 B per block).  A load leaves Raw in registers; widen()
// gives the 8 bf16 values of one MFMA operand (E4M3 -> bf16 is exact; the
// gfx950 conversion takes two codes per instruction, OCP E4M3FN).
template <bool FP8>
struct StoreFmt {
    using Raw = uint4;
    static constexpr int kRowBytes = kIdxDim * 2;
    // row 0 of the sequence's store, at coordinate 8 qq
    __device__ static const uint8_t* rows(const void* store, int64_t store_offset, int qq) {
        return (const uint8_t*)store + store_offset * kRowBytes + 16 * qq;
    }
    // coordinates 32 kk + [0, 8) relative to p (a row as rows() places it)
    __device__ static Raw load(const uint8_t* p, int kk) { return *(const uint4*)(p + 64 * kk); }
    __device__ static bf16x8 widen(Raw r) { return as_bf16x8(r); }
};

// codes of bytes 2 HI, 2 HI + 1 of the word -> two bf16 (low half first)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HI));
}

template <>
struct StoreFmt<true> {
    using Raw = uint2;
    static constexpr int kRowBytes = kIdxDim;
    __device__ static const uint8_t* rows(const void* store, int64_t store_offset, int qq) {
        return (const uint8_t*)store + store_offset * kRowBytes + 8 * qq;
    }
    __device__ static Raw load(const uint8_t* p, int kk) { return *(const uint2*)(p + 32 * kk); }
    __device__ static bf16x8 widen(Raw r) {
        uint4 o;
        o.x = e4m3x2_to_bf16x2<false>(r.x);
        o.y = e4m3x2_to_bf16x2<true>(r.x);
        o.z = e4m3x2_to_bf16x2<false>(r.y);
        o.w = e4m3x2_to_bf16x2<true>(r.y);
        return as_bf16x8(o);
    }
};

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

template <bool FP8>
__global__ __launch_bounds__(64) void index_topk_kernel(SeqTable seqs, IndexArgs a) {
    using F = StoreFmt<FP8>;
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
    const uint8_t* store = F::rows(a.store, sq.store_offset, qq);

    uint32_t thr = 0u;             // accept keys above it (0: accept every score)
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, cnt3 = 0;
    uint32_t* const mykeys = keys + qq * cap;
    int32_t* const myidx = idxs + qq * cap;

    // B operand of tile r0: lane holds store[r0 + m][32kk + 8qq .. +7]
    typename F::Raw b0[4], b1[4];
    auto row_of = [&](int64_t r0) { return (r0 + m < r_hi ? r0 + m : r_lo) * F::kRowBytes; };
    if (r_lo < r_hi) {
        const int64_t o = row_of(r_lo);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = F::load(store + o, kk);
    }
    if (r_lo + 16 < r_hi) {
        const int64_t o = row_of(r_lo + 16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b1[kk] = F::load(store + o, kk);
    }
    for (int64_t r0 = r_lo; r0 < r_hi; r0 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_16x16x32(afrag[kk], F::widen(b0[kk]), acc);
        // rotate the two-tile register pipeline: tile r0+32 goes in flight
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b0[kk] = b1[kk];
        if (r0 + 32 < r_hi) {
            const int64_t o = row_of(r0 + 32);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) b1[kk] = F::load(store + o, kk);
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
// Store tiles in the decode scorer's lane-contiguous order: lane (qq, m)
// holds coordinates 32 qq .. 32 qq + 31 of row m (64 B of bf16 or 32 B of
// E4M3 codes, read with whole 16 B loads that together cover whole cache
// lines), and MFMA step kk takes coordinates 32 qq + 8 kk .. + 7 of it; the
// query fragments are permuted to the same order.
template <bool FP8>
struct LaneRows {
    static constexpr int kLoads = FP8 ? 2 : 4;
    static constexpr int kRowBytes = FP8 ? kIdxDim : 2 * kIdxDim;
    struct Tile {
        uint4 v[kLoads];
    };
    __device__ static const uint8_t* rows(const void* store, int64_t store_offset, int qq) {
        return (const uint8_t*)store + store_offset * kRowBytes + qq * (kRowBytes / 4);
    }
    __device__ static Tile load(const uint8_t* p) {
        Tile t;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) t.v[i] = *(const uint4*)(p + 16 * i);
        return t;
    }
    __device__ static bf16x8 operand(const Tile& t, int kk) {
        if constexpr (FP8) {
            const uint4 u = t.v[kk >> 1];
            return (kk & 1) ? StoreFmt<true>::widen(uint2{u.z, u.w}) : StoreFmt<true>::widen(uint2{u.x, u.y});
        } else {
            return as_bf16x8(t.v[kk]);
        }
    }
};

// one scoring wavefront: column bx of sequence entry sq (query bx / n_split,
// candidate split bx % n_split); xp is the wavefront's 1 KiB of LDS
template <bool FP8>
__device__ __forceinline__ void score_split_wave(const DevSeq& sq, int64_t bx, const IndexArgs& a,
                                                 uint4 (*xp)[4][16]) {
    using F = LaneRows<FP8>;
    const int64_t qi = bx / a.n_split;
    const int split = (int)(bx % a.n_split);
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
    // lane (qq, m) takes for step kk the fragment of chunk qq that lane
    // (kk, m) formed: q_hat coordinates 32 qq + 8 kk .. + 7 of row m
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xp[kk][qq][m] = __builtin_bit_cast(uint4, afrag[kk]);
    wave_lds_sync();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) afrag[kk] = as_bf16x8(xp[qq][kk][m]);
    const float4 wv = *(const float4*)(a.w + (row * kGroups + qq) * kIdxHeads);
    const uint8_t* store = F::rows(a.store, sq.store_offset, qq);
    uint32_t* keys = a.part_key + ((sq.ws_row + qi) * kGroups + qq) * a.key_stride;
    // 16-block store tiles, kDepth of them in flight (a ring refilled kDepth
    // tiles ahead as each is used)
    constexpr int kDepth = 4;
    typename F::Tile b[kDepth];
    auto row_of = [&](int64_t r0) { return (r0 + m < r_hi ? r0 + m : r_lo) * F::kRowBytes; };
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        if (r_lo + 16 * d < r_hi) b[d] = F::load(store + row_of(r_lo + 16 * d));
    for (int64_t r00 = r_lo; r00 < r_hi; r00 += 16 * kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int64_t r0 = r00 + 16 * d;
            if (r0 >= r_hi) break;                     // wavefront-uniform
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma_16x16x32(afrag[kk], F::operand(b[d], kk), acc);
            if (r0 + 16 * kDepth < r_hi) b[d] = F::load(store + row_of(r0 + 16 * kDepth));
            float s = wv.x * fmaxf(acc[0], 0.f);
            s += wv.y * fmaxf(acc[1], 0.f);
            s += wv.z * fmaxf(acc[2], 0.f);
            s += wv.w * fmaxf(acc[3], 0.f);
            if (r0 + m < r_hi) keys[r0 + m] = score_key(s);
        }
    }
}

template <bool FP8>
__global__ __launch_bounds__(64) void index_score_kernel(SeqTable seqs, IndexArgs a) {
    __shared__ uint4 xp[4][4][16];
    score_split_wave<FP8>(seqs.s[blockIdx.y], blockIdx.x, a, xp);
}

// The same scoring launch carrying step 1 for calls whose queries read none
// of the blocks the call completes (each sequence's queries lie inside one
// block, e.g. one new token per sequence): column 0 of each sequence merges
// its completed block, if any, into the store row that no score of the
// launch reads; the other columns score.  One launch fewer per decode step.
template <bool FP8, int B>
__global__ __launch_bounds__(64) void index_score_merge_kernel(SeqTable seqs, IndexArgs a, CompressArgs c) {
    __shared__ uint4 xp[4][4][16];
    const DevSeq sq = seqs.s[blockIdx.y];
    if (blockIdx.x == 0) {
        const int64_t r = sq.pos0 / B;
        if (r < (sq.pos0 + sq.n_q) / B) compress_block<B>(sq, r, c);
        return;
    }
    score_split_wave<FP8>(sq, (int64_t)blockIdx.x - 1, a, xp);
}

// ---------------------------------------------------------------------------
// Prefill-sized calls, first step: every query's indexer rows (RMSNorm,
// rotary span, bf16) once, written to the workspace in the score kernel's
// A-operand order: per query 4 k-chunks x 64 lanes x 16 B, so a score
// workgroup loads its fragments with one coalesced 16-byte read per lane and
// k-chunk instead of recomputing them for every candidate range.  One
// wavefront per query; q_hat is written here when asked.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_qfrag_kernel(SeqTable seqs, IndexArgs a) {
    // the call's first launch clears its diagnostics block (the list select
    // of this and later launches appends to it)
    if (a.diag && a.diag_clear && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kDiagWords)
        a.diag[threadIdx.x] = 0u;
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (qi >= sq.n_q) return;
    // a row of at most k candidates takes all of them: without score or q_hat
    // outputs nothing reads its fragments
    if (!a.sel_scores && !a.q_hat_out && (sq.pos0 + qi) / a.block_size <= a.topk) return;
    const int lane = lane_id();
    bf16x8 af[4];
    index_query_fragments(a, sq.q_offset + qi, sq.pos0 + qi, lane >> 4, lane & 15, true, af);
    uint4* dst = a.q_frag + (sq.ws_row + qi) * 256;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) dst[kk * 64 + lane] = __builtin_bit_cast(uint4, af[kk]);
}

// ---------------------------------------------------------------------------
// Prefill-sized calls: a workgroup of four wavefronts scores 16 consecutive
// queries (four per wavefront) against one range of candidate blocks.  The
// range streams through LDS in tiles of 64 store rows (double-buffered, rows
// padded to 68 dwords so the 16 rows a B-operand read touches hit distinct
// banks); every B fragment a wavefront reads serves the MFMAs of its four
// queries, so the store is read once per 16 queries instead of once per
// query.  LISTED = false writes every key to the workspace, as the
// decode-sized path does; LISTED = true (tiles with long rows) keeps only the
// keys >= the row's sampled threshold, with their block ids, in per-segment
// lists (in block order: lanes append in block order, segments lie inside
// one workgroup's range) plus one count per segment.
// ---------------------------------------------------------------------------
constexpr int kStoreTile = 64;
constexpr int kStoreStrideU = kIdxDim + 8;    // bf16 per LDS store row (68 dwords = 4 x 17)
static_assert(kSegBlocks % kStoreTile == 0, "a store tile lies inside one segment");

template <bool LISTED, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void index_score_tile_kernel(
    SeqTable seqs, IndexArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tiles[2][kStoreTile * kStoreStrideU];
    // indexer weights of the 16 queries (query, group): read by the score
    // epilogues from LDS (the 16 lanes of a group read one address) rather
    // than held in registers
    __shared__ float4 wlds[kScoreTileQueries][kGroups];
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t n_qt = (sq.n_q + kScoreTileQueries - 1) / kScoreTileQueries;
    // Keyed tiles: a query tile's candidate ranges in dispatch order, so
    // neighbouring workgroups write neighbouring pieces of the same key rows.
    // Listed tiles (long rows, few writes, the store read once per query
    // tile): workgroups go out round-robin over the 8 XCDs, and each XCD
    // takes a contiguous run of the range-major order, so the query tiles
    // that read one store range run on one XCD close together in time and
    // find it in that XCD's L2 (the remap is a bijection on the first
    // multiple of 8 workgroups and the identity on the rest).
    const uint32_t nwg = gridDim.x, full = nwg / 8 * 8, b = blockIdx.x;
    const uint32_t n_qt_grid = nwg / (uint32_t)a.n_split;
    const uint32_t l = b < full ? (b % 8) * (full / 8) + b / 8 : b;
    const int64_t qt = LISTED ? l % n_qt_grid : b / (uint32_t)a.n_split;
    const int split = (int)(LISTED ? l / n_qt_grid : b % (uint32_t)a.n_split);
    if (qt >= n_qt) return;
    const int64_t q0 = qt * kScoreTileQueries;
    if ((a.listed && list_tile((sq.pos0 + q0) / a.block_size, a.topk)) != LISTED) return;
    const int n_valid = (int)(sq.n_q - q0 < kScoreTileQueries ? sq.n_q - q0 : kScoreTileQueries);
    // every row of the tile has at most k candidates and takes them all: the
    // keys are read only for score outputs
    if (!a.sel_scores && (sq.pos0 + q0 + n_valid - 1) / a.block_size <= a.topk) return;
    // the candidate range as wavefront-uniform values (the 64-bit division
    // runs in vector registers), so the store resource and the per-query
    // limits below stay in scalar registers
    const int64_t nb_max = uniform_i64((sq.pos0 + q0 + n_valid - 1) / a.block_size);
    const int64_t r_lo = (int64_t)split * a.split_blocks;
    const int64_t r_hi = nb_max < r_lo + a.split_blocks ? nb_max : r_lo + a.split_blocks;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qq = lane >> 4;     // operand k-chunk; result group
    const int m = lane & 15;      // operand row (4*group + head); result column

    // ---- the wavefront's four queries: A fragments, weights, candidates ----
    bf16x8 af[4][4];
    int lim[4];                   // candidates r_lo + [0, lim) of (query, group qq)
    float tauf[4];                // listed: its threshold as a score
    // byte offset of the key row of (query 4 * wave + j, group qq): kofs0 +
    // j * krow_bytes (keys: from block r_lo)
    const uint32_t krow_bytes = (uint32_t)(kGroups * a.key_stride * 4);
    const uint32_t kofs0 = (uint32_t)((4 * wave * kGroups + qq) * a.key_stride * 4) +
                           (LISTED ? 0u : 4u * (uint32_t)r_lo);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int qo = 4 * wave + j;
        const bool ok = qo < n_valid;
        const int64_t qi = q0 + (ok ? qo : 0);
        const int64_t row = sq.q_offset + qi;
        const int64_t t = sq.pos0 + qi;
        const uint4* qf = a.q_frag + (sq.ws_row + qi) * 256;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) af[j][kk] = as_bf16x8(qf[kk * 64 + lane]);
        if (m == 0) wlds[qo][qq] = *(const float4*)(a.w + (row * kGroups + qq) * kIdxHeads);
        const int64_t nb = ok ? t / a.block_size : 0;
        const int64_t hi = nb < r_hi ? nb : r_hi;
        lim[j] = hi > r_lo ? (int)(hi - r_lo) : 0;
        // the threshold key as the score it stands for: scores are never
        // -0, and on other finite values the key map is strictly increasing,
        // so key >= tau exactly when score >= this value
        if (LISTED) tauf[j] = key_score(a.part_key[((sq.ws_row + qi) * kGroups + qq) * a.key_stride + a.tau_off]);
    }
    if (r_lo >= r_hi) return;                       // workgroup-uniform

    // key rows of the workgroup's 16 queries through a buffer resource: 32-bit
    // offsets (the host keeps 64 key rows below 4 GiB), and a store at an
    // offset past the resource's end is dropped, which is how candidates
    // outside a query's range (or below its threshold) are skipped without a
    // branch
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.part_key + (sq.ws_row + q0) * kGroups * a.key_stride), (short)0,
        (int)(uint32_t)(kScoreTileQueries * kGroups * a.key_stride * 4), 0x00020000);
    constexpr uint32_t kDropped = 0xFFFFFFF0u;

    // ---- store tiles: 64 rows of 16 B chunks (16 per bf16 row, four per
    //      thread; 8 per E4M3 row, two per thread, widened to bf16 on the way
    //      into LDS); rows past the range read as zero (their scores are
    //      dropped) ----
    constexpr int kRowBytes = FP8 ? kIdxDim : kIdxDim * 2;
    constexpr int kChunkShift = FP8 ? 3 : 4;        // log2 chunks per row
    constexpr int kStage = FP8 ? 2 : 4;             // chunks per thread
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)a.store + (sq.store_offset + r_lo) * kRowBytes), (short)0,
        (int)((r_hi - r_lo) * kRowBytes), 0x00020000);
    auto gload = [&](int rt, uint4 (&v)[kStage]) {
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
            const int c = tid + 256 * k;
            const int ch = c & ((1 << kChunkShift) - 1);
            v[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 srs, (rt + (c >> kChunkShift)) * kRowBytes + 16 * ch, 0, 0));
        }
    };
    auto lstore = [&](uint16_t* buf, const uint4 (&v)[kStage]) {
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
            const int c = tid + 256 * k;
            const int ch = c & ((1 << kChunkShift) - 1);
            uint16_t* dst = buf + (c >> kChunkShift) * kStoreStrideU;
            if constexpr (FP8) {
                *(uint4*)(dst + 16 * ch) = __builtin_bit_cast(uint4, StoreFmt<true>::widen(uint2{v[k].x, v[k].y}));
                *(uint4*)(dst + 16 * ch + 8) =
                    __builtin_bit_cast(uint4, StoreFmt<true>::widen(uint2{v[k].z, v[k].w}));
            } else {
                *(uint4*)(dst + 8 * ch) = v[k];
            }
        }
    };
    uint4 stage[kStage];
    gload(0, stage);
    lstore(tiles[0], stage);
    int cur = 0;
    // steps of 16 blocks below lim_min are candidates of all four queries
    const int lim_min = min(min(lim[0], lim[1]), min(lim[2], lim[3]));
    // listed: entries of the current segment per query (above kSegCap when
    // entries were dropped)
    uint32_t cnt[4] = {0u, 0u, 0u, 0u};
    const uint32_t below = (1u << m) - 1u;          // group lanes below this one
    for (int64_t r0 = r_lo; r0 < r_hi; r0 += kStoreTile) {
        const int rt = (int)(r0 - r_lo);
        const bool more = r0 + kStoreTile < r_hi;
        if (more) gload(rt + kStoreTile, stage);
        __syncthreads();
        const uint16_t* buf = tiles[cur];
        const uint32_t seg = (uint32_t)(r0 / kSegBlocks);
#pragma unroll
        for (int sub = 0; sub < kStoreTile / 16; ++sub) {
            if (r0 + 16 * sub >= r_hi) break;       // workgroup-uniform
            bf16x8 bf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                bf[kk] = as_bf16x8(*(const uint4*)(buf + (16 * sub + m) * kStoreStrideU + 32 * kk + 8 * qq));
            // the four queries' weights, read ahead of the epilogue's branches
            float4 wq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wq[j] = wlds[4 * wave + j][qq];
            // the four queries' chains interleaved, one accumulator each
            f32x4 acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = mfma_16x16x32(af[j][kk], bf[kk], acc[j]);
            const int rb = rt + 16 * sub;
            const int rr = rb + m;
            // every row of the step is a candidate of the four queries
            // (wavefront-uniform): no per-row limit test
            const bool full = rb + 16 <= lim_min;
            float sc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] = head_score(acc[j], wq[j]);
            if (!LISTED) {
                if (full) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            score_key_nz(sc[j]), krs, (int)(kofs0 + (uint32_t)j * krow_bytes + 4u * (uint32_t)rr), 0, 0);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t off = rr < lim[j] ? kofs0 + (uint32_t)j * krow_bytes + 4u * (uint32_t)rr
                                                         : kDropped;
                        __builtin_amdgcn_raw_buffer_store_b32(score_key_nz(sc[j]), krs, (int)off, 0, 0);
                    }
                }
            } else {
                // append (key, block id) to the segment's list of (query j,
                // group qq): the 16 lanes of the group count the passing
                // lanes below them.  Few candidates pass the threshold, so a
                // query whose lanes all fail skips the bookkeeping.
                uint64_t bal[4];
                if (full) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bal[j] = __ballot(sc[j] >= tauf[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bal[j] = __ballot(rr < lim[j] && sc[j] >= tauf[j]);
                }
                const uint32_t blk = (uint32_t)(r_lo + rr);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (bal[j] == 0u) continue;                           // wavefront-uniform
                    const uint32_t gm = (uint32_t)(bal[j] >> (16 * qq)) & 0xFFFFu;
                    const uint32_t pos = cnt[j] + (uint32_t)__builtin_popcount(gm & below);
                    const uint32_t off = ((gm >> m) & 1u) && pos < (uint32_t)kSegCap
                        ? kofs0 + (uint32_t)j * krow_bytes +
                              4u * ((uint32_t)a.list_off + seg * (2 * kSegCap) + 2u * pos)
                        : kDropped;
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{score_key_nz(sc[j]), blk}, krs, (int)off, 0, 0);
                    cnt[j] += (uint32_t)__builtin_popcount(gm);
                }
            }
        }
        if (LISTED && (((r0 + kStoreTile) % kSegBlocks) == 0 || r0 + kStoreTile >= r_hi)) {
            // the segment ends: its count, for every query whose range
            // reaches into it
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool wr = m == 0 && (int64_t)seg * kSegBlocks - r_lo < lim[j];
                __builtin_amdgcn_raw_buffer_store_b32(cnt[j], krs,
                                                      (int)(wr ? kofs0 + (uint32_t)j * krow_bytes + 4u * seg
                                                               : kDropped), 0, 0);
                cnt[j] = 0u;
            }
        }
        if (more) lstore(tiles[cur ^ 1], stage);
        cur ^= 1;
    }
}

// Top-k of one (query, group) from its score keys: the k largest, equal keys
// to the lower block id, output in ascending block id.  Rows of at most
// kWaveSelectKeys keys take one wavefront each (index_select_wave_kernel);
// longer ones a workgroup of NW wavefronts (4; 16 for the rows of calls with
// few rows, and for rescued rows).
// The k-th largest key v and the number krem of entries equal to v that are
// kept come from a radix select (8-bit digits from the highest bit in which
// the keys differ, one histogram per wavefront per digit).  A workgroup
// first bounds v from below with a sample (a sixteenth of the row, at most
// 2048 keys, in groups of 16 consecutive keys spread over the row): the
// sample's j-th largest key tau, j chosen so that about m k keys are expected
// at or above it (m = 1 + 5 / sqrt(k S / n), as for the candidate lists).
// One pass over the row then streams every key >= tau, with its block id,
// into an LDS candidate list kept in block order; when a step would overflow
// it (the sample misjudged a row whose high keys cluster), the list is cut to
// its top k and the threshold raised, as in the fused kernel's streaming
// top-k.  The list then holds every key >= v, so the select and the ordered
// output run on it alone.  Only a row with fewer than k keys >= tau falls
// back to selecting over the whole row in global memory.  Outputs are written
// in block order from NW contiguous segments whose offsets come from one
// exchange.
constexpr int kWaveSelectKeys = 1024;
constexpr int kSelectSampleMax = 2048;     // sample keys (LDS words)

// keys a wavefront scans per step of the candidate pass.  Four-wavefront
// workgroups take many rows of a few thousand keys: short steps keep the
// list, and so each workgroup's LDS, small, and more rows run at once per
// CU.  Sixteen-wavefront workgroups take few long rows: long steps keep more
// loads in flight per row.
__host__ __device__ constexpr int select_step(int nw) { return nw == 4 ? 256 : 1024; }
// candidate list capacity: k plus one step of every wavefront (a step always
// fits after a cut to the top k)
__host__ __device__ constexpr int select_capacity(int k, int nw) { return k + select_step(nw) * nw; }
static_assert(2 * select_capacity(1, 4) >= kSelectSampleMax, "the sample fits the candidate area");

// shared state of a select workgroup of NW wavefronts
template <int NW>
struct SelectShared {
    uint32_t hist[NW][256];
    uint32_t total[256];        // NW > 4: the wavefronts' histograms summed
    uint32_t red[NW];
    int cnt[2][NW];
    int digit, above, count;
};

// v (as prefix under pmask) and krem of the k-th largest of keys[0..n),
// 1 <= k <= n.  Called by all 64*NW threads.  With stop_bit > 0 only the
// key bits >= stop_bit are resolved: prefix (its lower bits zero) is then a
// lower bound of the k-th largest key that at least k keys reach.
template <int NW>
__device__ void radix_kth(const uint32_t* keys, int n, int k, SelectShared<NW>& sh, uint32_t& prefix,
                          uint32_t& pmask, int& krem, int stop_bit = 0) {
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    krem = k;
    const uint32_t k0 = keys[0];
    uint32_t diff = 0;
    for (int i = tid; i < n; i += NT) diff |= keys[i] ^ k0;
    diff = wave_or(diff);
    if (lane == 0) sh.red[w] = diff;
    __syncthreads();
    diff = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) diff |= sh.red[j];
    __syncthreads();
    prefix = k0;
    pmask = 0xFFFFFFFFu;
    if (diff == 0) return;
    const int hb = 31 - __builtin_clz(diff);
    pmask = hb == 31 ? 0u : (0xFFFFFFFFu << (hb + 1));
    prefix = k0 & pmask;
    for (int hi = hb; hi >= stop_bit;) {
        const int lo = hi - 7 > stop_bit ? hi - 7 : stop_bit;
        const int nbins = 1 << (hi - lo + 1);
        const uint32_t dmask = (uint32_t)nbins - 1u;
        for (int b = lane; b < 256; b += 64) sh.hist[w][b] = 0u;
        __syncthreads();
        int i = tid;
        for (; i + 3 * NT < n; i += 4 * NT) {
            const uint32_t k0 = keys[i], k1 = keys[i + NT], k2 = keys[i + 2 * NT], k3 = keys[i + 3 * NT];
            if ((k0 & pmask) == prefix) atomicAdd(&sh.hist[w][(k0 >> lo) & dmask], 1u);
            if ((k1 & pmask) == prefix) atomicAdd(&sh.hist[w][(k1 >> lo) & dmask], 1u);
            if ((k2 & pmask) == prefix) atomicAdd(&sh.hist[w][(k2 >> lo) & dmask], 1u);
            if ((k3 & pmask) == prefix) atomicAdd(&sh.hist[w][(k3 >> lo) & dmask], 1u);
        }
        for (; i < n; i += NT) {
            const uint32_t kk = keys[i];
            if ((kk & pmask) == prefix) atomicAdd(&sh.hist[w][(kk >> lo) & dmask], 1u);
        }
        __syncthreads();
        if constexpr (NW > 4) {
            // many wavefronts: 256 threads sum the histograms, so the scan
            // below reads one total per bin instead of NW partial counts
            if (tid < nbins) {
                uint32_t hs = 0;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) hs += sh.hist[ww][tid];
                sh.total[tid] = hs;
            }
            __syncthreads();
        }
        if (w == 0) {
            uint32_t h[4], tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = nbins - 1 - 4 * lane - j;
                uint32_t hs = 0;
                if (d >= 0) {
                    if constexpr (NW > 4) {
                        hs = sh.total[d];
                    } else {
#pragma unroll
                        for (int ww = 0; ww < NW; ++ww) hs += sh.hist[ww][d];
                    }
                }
                h[j] = hs;
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
                sh.digit = found;
                sh.above = (int)above_found;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh.digit << lo;
        pmask |= dmask << lo;
        krem -= sh.above;
        hi = lo - 1;
        __syncthreads();
    }
}

// Cut an LDS candidate list (keys, block ids, in block order) to its top k in
// place, order kept, and return the k-th key v: kept are the keys > v and the
// first entries equal to v.  Called by every thread of the workgroup; one
// wavefront moves the entries (each to an index <= its own).
template <int NW>
__device__ uint32_t compact_to_topk(uint32_t* ckeys, int32_t* cidx, int pool, int K, SelectShared<NW>& sh) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t v, vm;
    int vr;
    radix_kth(ckeys, pool, K, sh, v, vm, vr);
    if (w == 0) {
        int out = 0, eq_seen = 0;
        for (int i0 = 0; i0 < pool; i0 += 64) {
            const int i = i0 + lane;
            const uint32_t kk = i < pool ? ckeys[i] : 0u;
            const int32_t ii = i < pool ? cidx[i] : 0;
            const bool eq = i < pool && kk == v;
            const uint64_t em = __ballot(eq);
            const bool keep = i < pool && (kk > v || (eq && eq_seen + (int)lanes_below(em) < vr));
            const uint64_t km = __ballot(keep);
            wave_lds_sync();
            if (keep) {
                ckeys[out + (int)lanes_below(km)] = kk;
                cidx[out + (int)lanes_below(km)] = ii;
            }
            wave_lds_sync();
            out += __popcll(km);
            eq_seen += __popcll(em);
        }
    }
    __syncthreads();
    return v;
}

// Keep rule over entries [0, n) of keys (block ids idx, or the entry index
// when idx is null): key & pmask > prefix, or == prefix among the first krem
// such; written in order to sel / ssc.
template <int NW>
__device__ void select_ordered_output(const uint32_t* keys, const int32_t* idx, int n, uint32_t prefix,
                                      uint32_t pmask, int krem, int32_t* sel, float* ssc, SelectShared<NW>& sh) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int seg = (n + 64 * NW - 1) / (64 * NW) * 64;
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
        sh.cnt[0][w] = n_gt;
        sh.cnt[1][w] = n_eq;
    }
    __syncthreads();
    // kept before this segment: every larger masked key, min(krem, equal ones)
    int out = 0, eq_seen = 0;
    for (int jw = 0; jw < w; ++jw) {
        out += sh.cnt[0][jw];
        eq_seen += sh.cnt[1][jw];
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
            sel[pos] = idx ? idx[i] : i;
            if (ssc) ssc[pos] = key_score(kk);
        }
        out += __popcll(km);
        eq_seen += __popcll(em);
    }
}

template <int NW>
__device__ void select_row(const DevSeq& sq, int64_t qi, int g, const IndexArgs& a, uint32_t* lds_keys,
                           SelectShared<NW>& sh) {
    constexpr int NT = 64 * NW;
    const int64_t t = sq.pos0 + qi;
    const int64_t row = sq.q_offset + qi;
    const int64_t rg = row * kGroups + g;
    const int n = (int)(t / a.block_size);
    const int K = a.topk;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint32_t* gkeys = a.part_key + ((sq.ws_row + qi) * kGroups + g) * a.key_stride;
    int32_t* sel = a.sel + rg * K;
    float* ssc = a.sel_scores ? a.sel_scores + rg * K : nullptr;
    if (n <= K) {
        // every candidate is selected, in block order, then -1 padding
        for (int jj = tid; jj < K; jj += NT) {
            sel[jj] = jj < n ? jj : -1;
            if (ssc) ssc[jj] = jj < n ? key_score(gkeys[jj]) : 0.0f;
        }
        return;
    }

    uint32_t prefix = 0, pmask = 0;
    int krem = K;

    // ---- threshold tau: the j-th largest of a sample of S keys taken as
    //      S/16 groups of 16 consecutive keys spread over the row ----
    const int smax = kSelectSampleMax < n / 16 ? kSelectSampleMax : n / 16;
    const int S = smax / 16 * 16;
    const int ngrp = S / 16;
    for (int i = tid; i < S; i += NT) {
        const int gi = i >> 4;
        const int64_t start = (int64_t)gi * (n - 16) / (ngrp > 1 ? ngrp - 1 : 1);
        lds_keys[i] = gkeys[start + (i & 15)];
    }
    __syncthreads();
    // j such that about m k keys are expected at or above tau, m = 1 +
    // 5 / sqrt(k S / n): the sample's estimate of a share has relative spread
    // 1 / sqrt(j), so fewer than k keys pass only about five spreads out
    const double ks = (double)K * S / (double)n;
    const int64_t jt = (int64_t)ceil((1.0 + 5.0 / sqrt(ks)) * ks);
    const int j = (int)(jt < 1 ? 1 : (jt > S ? S : jt));
    // (tau only bounds the list: its top 16 bits suffice -- the keys it
    // admits beyond the exact j-th lie within one part in 128 of it)
    uint32_t tau, tmask;
    int trem;
    radix_kth(lds_keys, S, j, sh, tau, tmask, trem, 16);

    // ---- candidates: the wavefronts scan the row in steps of STEP keys
    //      per wavefront (wavefront w takes the w-th STEP, STEP / 64 loads in
    //      flight per lane) and append the (key, block) pairs that pass the threshold
    //      to one list in block order, counts exchanged once per step.  A
    //      step that would overflow the list first compacts it to its top k
    //      (block order kept) and raises the threshold to the k-th key: only
    //      larger keys can still enter (an equal one would lose the tie).
    //      The capacity leaves room for a whole step after a compaction. ----
    const int cap = select_capacity(K, NW);
    uint32_t* ckeys = lds_keys;
    int32_t* cidx = (int32_t*)(lds_keys + cap);
    uint32_t thr = tau;
    bool strict = false;          // accept key > thr (after a compaction) or key >= thr
    int pool = 0, par = 0;
    constexpr int STEP = select_step(NW), NU = STEP / 64;
    for (int base = 0; base < n; base += STEP * NW) {
        const int wb = base + STEP * w;
        uint32_t kv[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int i = wb + 64 * u + lane;
            kv[u] = i < n ? gkeys[i] : 0u;
        }
        int pos[NU];
        int total = 0, off = 0;
#pragma unroll 1
        for (int attempt = 0; attempt < 2; ++attempt) {
            int cw = 0;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int i = wb + 64 * u + lane;
                const bool take = i < n && (strict ? kv[u] > thr : kv[u] >= thr);
                const uint64_t m = __ballot(take);
                pos[u] = take ? cw + (int)lanes_below(m) : -1;
                cw += __popcll(m);
            }
            if (lane == 0) sh.cnt[par][w] = cw;
            __syncthreads();
            total = 0;
            off = pool;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const int cj = sh.cnt[par][j];
                total += cj;
                off += j < w ? cj : 0;
            }
            par ^= 1;
            if (pool + total <= cap) break;              // workgroup-uniform
            thr = compact_to_topk(ckeys, cidx, pool, K, sh);
            pool = K;
            strict = true;
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (pos[u] >= 0) {
                ckeys[off + pos[u]] = kv[u];
                cidx[off + pos[u]] = wb + 64 * u + lane;
            }
        }
        pool += total;
    }
    __syncthreads();
    const int c = pool;
    if (c < K) {
        // the sample's threshold was above the k-th key: select over the row
        radix_kth(gkeys, n, K, sh, prefix, pmask, krem);
        select_ordered_output(gkeys, nullptr, n, prefix, pmask, krem, sel, ssc, sh);
        return;
    }
    radix_kth(ckeys, c, K, sh, prefix, pmask, krem);
    select_ordered_output(ckeys, cidx, c, prefix, pmask, krem, sel, ssc, sh);
}

// Rows of at most kWaveSelectKeys candidates, one wavefront each: the row's
// keys sit in registers (lane l holds keys l, l + 64, ...); the k-th largest
// key v comes from four 8-bit digit passes over a wavefront-private LDS
// histogram (bins scanned from the top by a wavefront prefix sum), and the
// output goes out in block order from ballots -- no workgroup barrier.

__global__ __launch_bounds__(256) void index_select_wave_kernel(SeqTable seqs, IndexArgs a) {
    constexpr int KPL = kWaveSelectKeys / 64;
    __shared__ uint32_t hist[4][256];
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x;
    const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (qi >= sq.n_q) return;
    const int n = (int)((sq.pos0 + qi) / a.block_size);
    if (n > kWaveSelectKeys) return;
    const int K = a.topk;
    const int64_t rg = (sq.q_offset + qi) * kGroups + g;
    int32_t* sel = a.sel + rg * K;
    float* ssc = a.sel_scores ? a.sel_scores + rg * K : nullptr;
    const uint32_t* gkeys = a.part_key + ((sq.ws_row + qi) * kGroups + g) * a.key_stride;
    if (n <= K) {
        for (int jj = lane; jj < K; jj += 64) {
            sel[jj] = jj < n ? jj : -1;
            if (ssc) ssc[jj] = jj < n ? key_score(gkeys[jj]) : 0.0f;
        }
        return;
    }
    uint32_t key[KPL];
#pragma unroll
    for (int u = 0; u < KPL; ++u) key[u] = 64 * u + lane < n ? gkeys[64 * u + lane] : 0u;
    uint32_t* h = hist[g];
    uint32_t pref = 0u, pmask = 0u;
    int need = K;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        wave_lds_sync();                               // the previous pass's bin reads are done
#pragma unroll
        for (int j = 0; j < 4; ++j) h[lane + 64 * j] = 0u;
        wave_lds_sync();
#pragma unroll
        for (int u = 0; u < KPL; ++u)
            if (64 * u + lane < n && (key[u] & pmask) == pref) atomicAdd(&h[(key[u] >> shift) & 255u], 1u);
        wave_lds_sync();
        // lane l holds bins 255 - 4l - j; counts above a bin by a prefix sum
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = h[255 - 4 * lane - j];
            tot += c[j];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        uint32_t above = incl - tot, above_found = 0;
        int found = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (found < 0 && c[j] > 0 && above + c[j] >= (uint32_t)need) {
                found = 255 - 4 * lane - j;
                above_found = above;
            }
            above += c[j];
        }
        const int src = (int)__builtin_ctzll(__ballot(found >= 0));
        const int digit = __shfl(found, src, 64);
        need -= (int)__shfl(above_found, src, 64);
        pref |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
    }
    // keep every key > v and the first `need` keys == v, in block order
    int out = 0, eq_seen = 0;
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
        const bool ok = 64 * u + lane < n;
        const bool eq = ok && key[u] == pref;
        const uint64_t em = __ballot(eq);
        const bool keep = ok && (key[u] > pref || (eq && eq_seen + (int)lanes_below(em) < need));
        const uint64_t km = __ballot(keep);
        if (keep) {
            const int pos = out + (int)lanes_below(km);
            sel[pos] = 64 * u + lane;
            if (ssc) ssc[pos] = key_score(key[u]);
        }
        out += __popcll(km);
        eq_seen += __popcll(em);
    }
}

// a listed row of a tiled call (its key row holds candidate lists)
__device__ __forceinline__ bool listed_row(const DevSeq& sq, int64_t qi, const IndexArgs& a) {
    return a.listed && list_tile((sq.pos0 + (qi & ~(int64_t)(kScoreTileQueries - 1))) / a.block_size, a.topk);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void index_select_kernel(SeqTable seqs, IndexArgs a) {
    extern __shared__ uint32_t lds_keys[];    // the sample, then candidate keys + block ids
    __shared__ SelectShared<NW> sh;
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / kGroups;
    const int g = blockIdx.x % kGroups;
    if (qi >= sq.n_q) return;
    const int64_t n = (sq.pos0 + qi) / a.block_size;
    if (n <= kWaveSelectKeys) return;              // one wavefront per row
    if (listed_row(sq, qi, a)) return;             // selected from its lists
    select_row<NW>(sq, qi, g, a, lds_keys, sh);
}

// ---------------------------------------------------------------------------
// Listed rows (tiled calls, long histories), before the score step: the
// scores of each tile's sample, S blocks in S/16 groups of 16 consecutive
// blocks spread over [0, n0) (n0 = the tile's first query's candidates, so
// every sample block is a candidate of all 16 queries), written to the key
// rows' sample area.  Workgroups of four wavefronts, four queries each, an
// eighth of the groups per workgroup; B fragments straight from memory.
// ---------------------------------------------------------------------------
constexpr int kSampleParts = 8;

template <bool FP8>
__global__ __launch_bounds__(256) void index_sample_kernel(SeqTable seqs, IndexArgs a) {
    using F = StoreFmt<FP8>;
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t n_qt = (sq.n_q + kScoreTileQueries - 1) / kScoreTileQueries;
    const int64_t qt = blockIdx.x / kSampleParts;
    const int part = blockIdx.x % kSampleParts;
    if (qt >= n_qt) return;
    const int64_t q0 = qt * kScoreTileQueries;
    const int64_t n0 = (sq.pos0 + q0) / a.block_size;
    if (!(a.listed && list_tile(n0, a.topk))) return;
    const int ngrp = list_sample(n0) / 16;
    const int g_lo = part * ngrp / kSampleParts, g_hi = (part + 1) * ngrp / kSampleParts;
    const int n_valid = (int)(sq.n_q - q0 < kScoreTileQueries ? sq.n_q - q0 : kScoreTileQueries);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qq = lane >> 4, m = lane & 15;
    bf16x8 af[4][4];
    float4 wv[4];
    uint32_t* sk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int qo = 4 * wave + j;
        const int64_t qi = q0 + (qo < n_valid ? qo : 0);
        const uint4* qf = a.q_frag + (sq.ws_row + qi) * 256;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) af[j][kk] = as_bf16x8(qf[kk * 64 + lane]);
        wv[j] = *(const float4*)(a.w + ((sq.q_offset + qi) * kGroups + qq) * kIdxHeads);
        sk[j] = qo < n_valid ? a.part_key + ((sq.ws_row + qi) * kGroups + qq) * a.key_stride + a.samp_off
                             : nullptr;
    }
    const uint8_t* store = F::rows(a.store, sq.store_offset, qq);
    auto start = [&](int gi) { return (int64_t)gi * (n0 - 16) / (ngrp > 1 ? ngrp - 1 : 1); };
    typename F::Raw b[4];
    if (g_lo < g_hi) {
        const uint8_t* src = store + (start(g_lo) + m) * F::kRowBytes;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b[kk] = F::load(src, kk);
    }
    for (int gi = g_lo; gi < g_hi; ++gi) {
        bf16x8 bf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bf[kk] = F::widen(b[kk]);
        if (gi + 1 < g_hi) {
            const uint8_t* src = store + (start(gi + 1) + m) * F::kRowBytes;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) b[kk] = F::load(src, kk);
        }
        f32x4 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma_16x16x32(af[j][kk], bf[kk], acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (sk[j]) sk[j][16 * gi + m] = score_key_nz(head_score(acc[j], wv[j]));
    }
}

// Listed rows: the threshold tau of each (query, group), the j-th largest of
// its S sample keys (list_rank), into the key row's tau slot.  The first
// workgroup also clears the failed-row count of the launch.
__global__ __launch_bounds__(256) void index_tau_kernel(SeqTable seqs, IndexArgs a) {
    __shared__ uint32_t skeys[kListSampleMax];
    __shared__ SelectShared<4> sh;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.ctl[0] = 0u;
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / kGroups;
    const int g = blockIdx.x % kGroups;
    if (qi >= sq.n_q || !listed_row(sq, qi, a)) return;
    const int64_t n0 = (sq.pos0 + (qi & ~(int64_t)(kScoreTileQueries - 1))) / a.block_size;
    const int S = list_sample(n0);
    uint32_t* krow = a.part_key + ((sq.ws_row + qi) * kGroups + g) * a.key_stride;
    for (int i = threadIdx.x; i < S; i += 256) skeys[i] = krow[a.samp_off + i];
    __syncthreads();
    uint32_t tau, tmask;
    int trem;
    radix_kth(skeys, S, list_rank(n0, a.topk), sh, tau, tmask, trem);
    if (threadIdx.x == 0) krow[a.tau_off] = tau;
}

// exclusive prefix sum over the 256 threads of a workgroup (4 wavefronts)
__device__ __forceinline__ int block_scan256(int v, int* part, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
    }
    if (lane == 63) part[w] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        before += j < w ? part[j] : 0;
        total += part[j];
    }
    __syncthreads();
    return before + incl - v;
}

// Listed rows: the top k from the candidate lists.  Thread i takes the
// contiguous segments [i*spt, (i+1)*spt) of the row, reads their counts, and one workgroup scan gives each thread the offset
// of its entries in block order.  Then:
//  * the row's entries fit the LDS pool: each thread copies its entries
//    there (several loads in flight), and the pool is selected exactly;
//  * they do not (scores tied at the threshold tau: a row whose indexer
//    weights are all negative scores 0 on every block whose four dot
//    products are <= 0, and its tau is that 0): the entries are streamed
//    again, counting the keys > tau.  With at least k of them (and no more
//    than the pool holds) only those go to the pool and are selected; with
//    fewer, the answer is every key > tau plus the first keys == tau in
//    block order, written straight to the output in block order.
// A row whose lists cannot give the exact answer -- a segment that dropped
// entries, fewer than k entries (tau was above the k-th score), or more
// than the pool holds above tau -- is appended to the launch's failed rows
// instead, to be scored again in full.
// f(entry) for the entries of segments [s0, s1), in block order.  A
// segment's count and its first 8 entries (two 16-byte loads per 4 entries;
// a segment owns all kSegCap slots, so reading past its count stays inside
// its list) are loaded together, the next segment's while this one's are
// used; longer segments take their remaining entries 8 at a time.
template <class F>
__device__ __forceinline__ void list_entries(const uint32_t* krow, const uint2* lists, int s0, int s1, F&& f) {
    if (s0 >= s1) return;
    int c_nx = (int)krow[s0];
    uint4 e_nx[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) e_nx[x] = ((const uint4*)(lists + (int64_t)s0 * kSegCap))[x];
    for (int sg = s0; sg < s1; ++sg) {
        const int c = c_nx < kSegCap ? c_nx : kSegCap;
        uint4 e[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = e_nx[x];
        if (sg + 1 < s1) {
            c_nx = (int)krow[sg + 1];
#pragma unroll
            for (int x = 0; x < 4; ++x) e_nx[x] = ((const uint4*)(lists + (int64_t)(sg + 1) * kSegCap))[x];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (2 * x < c) f(make_uint2(e[x].x, e[x].y));
            if (2 * x + 1 < c) f(make_uint2(e[x].z, e[x].w));
        }
        for (int e0 = 8; e0 < c; e0 += 8) {
            const uint4* l = (const uint4*)(lists + (int64_t)sg * kSegCap + e0);
            uint4 r[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) r[x] = l[x];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if (e0 + 2 * x < c) f(make_uint2(r[x].x, r[x].y));
                if (e0 + 2 * x + 1 < c) f(make_uint2(r[x].z, r[x].w));
            }
        }
    }
}

__global__ __launch_bounds__(256) void index_list_select_kernel(SeqTable seqs, IndexArgs a) {
    extern __shared__ uint32_t lds[];            // keys [cap], block ids [cap]
    __shared__ SelectShared<4> sh;
    __shared__ int part[4];
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / kGroups;
    const int g = blockIdx.x % kGroups;
    if (qi >= sq.n_q || !listed_row(sq, qi, a)) return;
    const int K = a.topk;
    const int cap = a.list_cap;
    const int n = (int)((sq.pos0 + qi) / a.block_size);
    const int nseg = (n + kSegBlocks - 1) / kSegBlocks;
    const uint32_t* krow = a.part_key + ((sq.ws_row + qi) * kGroups + g) * a.key_stride;
    const uint2* lists = (const uint2*)(krow + a.list_off);
    uint32_t* ckeys = lds;
    int32_t* cidx = (int32_t*)(lds + cap);
    const int tid = threadIdx.x;
    // contiguous runs of segments per thread: one, or a multiple of 4 (the
    // counts then come as 16-byte loads; counts past the row's last segment
    // lie inside its key row and are masked)
    const int spt0 = (nseg + 255) / 256;
    const int spt = spt0 == 1 ? 1 : (spt0 + 3) / 4 * 4;
    const int s0 = tid * spt;
    const int s1 = s0 + spt < nseg ? s0 + spt : nseg;
    const int64_t rg = (sq.q_offset + qi) * kGroups + g;
    int32_t* sel = a.sel + rg * K;
    float* ssc = a.sel_scores ? a.sel_scores + rg * K : nullptr;

    // the thread's entry count
    int mine = 0, bad = 0;
    if (spt == 1) {
        const int c = s0 < nseg ? (int)krow[s0] : 0;
        bad = c > kSegCap;
        mine = c < kSegCap ? c : kSegCap;
    } else {
        for (int u = 0; u < spt; u += 4) {
            const uint4 c4 = *(const uint4*)(krow + s0 + u);
            const int cc[4] = {(int)c4.x, (int)c4.y, (int)c4.z, (int)c4.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = s0 + u + v < nseg ? cc[v] : 0;
                bad |= c > kSegCap;
                mine += c < kSegCap ? c : kSegCap;
            }
        }
    }
    int total;
    const int off = block_scan256(mine, part, total);
    bad = __syncthreads_or(bad);
    auto fail = [&]() {
        if (tid == 0) {
            const uint32_t slot = atomicAdd(&a.ctl[0], 1u);
            a.ctl[1 + slot] = ((uint32_t)qi << 8) | ((uint32_t)blockIdx.y << 2) | (uint32_t)g;
            if (a.diag) {
                const uint32_t d = atomicAdd(&a.diag[0], 1u);
                if (d < (uint32_t)kDiagRows) {
                    a.diag[2 + 2 * d] = (uint32_t)(sq.q_offset + qi);
                    a.diag[3 + 2 * d] = (uint32_t)g;
                }
            }
        }
    };
    if (bad || total < K) {
        fail();
        return;
    }
    uint32_t prefix, pmask;
    int krem;
    if (total <= cap) {
        int o = off;
        list_entries(krow, lists, s0, s1, [&](uint2 kv) {
            ckeys[o] = kv.x;
            cidx[o] = (int32_t)kv.y;
            ++o;
        });
        __syncthreads();
        radix_kth(ckeys, total, K, sh, prefix, pmask, krem);
        select_ordered_output(ckeys, cidx, total, prefix, pmask, krem, sel, ssc, sh);
        return;
    }

    // more entries than the pool holds: the keys strictly above tau
    const uint32_t thr = krow[a.tau_off];
    int gt = 0;
    list_entries(krow, lists, s0, s1, [&](uint2 kv) { gt += kv.x > thr; });
    int n_gt;
    const int gt_off = block_scan256(gt, part, n_gt);
    if (n_gt >= K) {
        if (n_gt > cap) {
            fail();
            return;
        }
        int o = gt_off;
        list_entries(krow, lists, s0, s1, [&](uint2 kv) {
            if (kv.x > thr) {
                ckeys[o] = kv.x;
                cidx[o] = (int32_t)kv.y;
                ++o;
            }
        });
        __syncthreads();
        radix_kth(ckeys, n_gt, K, sh, prefix, pmask, krem);
        select_ordered_output(ckeys, cidx, n_gt, prefix, pmask, krem, sel, ssc, sh);
        return;
    }
    // every key > tau and the first K - n_gt keys == tau, in block order: an
    // entry's output slot is the number of kept entries before it
    const int quota = K - n_gt;
    int gt_run = gt_off, eq_run = off - gt_off;   // every listed key is >= tau
    // (both counters advance by value, not through a selected reference,
    // which kept them in scratch memory)
    list_entries(krow, lists, s0, s1, [&](uint2 kv) {
        const bool gt = kv.x > thr;
        const int eq_kept = eq_run < quota ? eq_run : quota;
        if (gt || eq_run < quota) {
            const int pos = gt_run + eq_kept;
            sel[pos] = (int32_t)kv.y;
            if (ssc) ssc[pos] = key_score(kv.x);
        }
        gt_run += gt ? 1 : 0;
        eq_run += gt ? 0 : 1;
    });
}

// Failed listed rows, again in full: every key of the row's query (all four
// groups, one wavefront per range of kRescoreBlocks candidates: a range is a
// chain of dependent MFMAs, so short ranges keep the few failed rows' latency
// low) into its key rows, over the launch's failed-row list (a grid-stride
// loop: the count is known only on the device).
constexpr int kRescoreBlocks = 256;

template <bool FP8>
__global__ __launch_bounds__(256) void index_rescore_kernel(SeqTable seqs, IndexArgs a) {
    using F = StoreFmt<FP8>;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qq = lane >> 4, m = lane & 15;
    // ranges per row: enough for the longest row (a key row holds at least
    // every candidate of its query)
    const int64_t n_rng = (a.key_stride + kRescoreBlocks - 1) / kRescoreBlocks;
    const int64_t units = (int64_t)a.ctl[0] * n_rng;
    for (int64_t u = (int64_t)blockIdx.x * 4 + wave; u < units; u += (int64_t)gridDim.x * 4) {
        const uint32_t item = a.ctl[1 + u / n_rng];
        const int64_t rng = u % n_rng;
        const DevSeq sq = seqs.s[(item >> 2) & 63];
        const int64_t qi = item >> 8;
        const int64_t nb = (sq.pos0 + qi) / a.block_size;
        const int64_t r_lo = rng * kRescoreBlocks;
        const int64_t r_hi = nb < r_lo + kRescoreBlocks ? nb : r_lo + kRescoreBlocks;
        if (r_lo >= r_hi) continue;
        bf16x8 af[4];
        const uint4* qf = a.q_frag + (sq.ws_row + qi) * 256;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) af[kk] = as_bf16x8(qf[kk * 64 + lane]);
        const float4 wv = *(const float4*)(a.w + ((sq.q_offset + qi) * kGroups + qq) * kIdxHeads);
        const uint8_t* store = F::rows(a.store, sq.store_offset, qq);
        uint32_t* keys = a.part_key + ((sq.ws_row + qi) * kGroups + qq) * a.key_stride;
        for (int64_t r0 = r_lo; r0 < r_hi; r0 += 16) {
            const int64_t r = r0 + m < r_hi ? r0 + m : r_lo;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mfma_16x16x32(af[kk], F::widen(F::load(store + r * F::kRowBytes, kk)), acc);
            if (r0 + m < r_hi) keys[r0 + m] = score_key_nz(head_score(acc, wv));
        }
    }
}

// Failed listed rows: the long-row select over the keys just written.  The
// failed rows are few, so each gets sixteen wavefronts when the candidate
// list of k plus one 16384-key step fits LDS (k <= 1024), else four.
template <int NW>
__global__ __launch_bounds__(64 * NW) void index_select_rescue_kernel(SeqTable seqs, IndexArgs a) {
    extern __shared__ uint32_t lds_keys[];
    __shared__ SelectShared<NW> sh;
    const uint32_t count = a.ctl[0];
    for (uint32_t it = blockIdx.x; it < count; it += gridDim.x) {
        const uint32_t item = a.ctl[1 + it];
        select_row<NW>(seqs.s[(item >> 2) & 63], item >> 8, (int)(item & 3), a, lds_keys, sh);
        __syncthreads();
    }
}

}  // namespace

// the candidate list (keys, then block ids), which the sample uses first
template <int NW>
static size_t select_long_lds(const IndexArgs& a) {
    return (size_t)2 * select_capacity(a.topk, NW) * sizeof(uint32_t);
}

template <int NW>
static hipError_t launch_select_long(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a, hipStream_t stream) {
    const size_t lds = select_long_lds<NW>(a);
    hipError_t e = set_dynamic_lds((const void*)index_select_kernel<NW>, lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL((index_select_kernel<NW>), grid, dim3(64 * NW), lds, stream, seqs, a);
    return hipGetLastError();
}

// keyed_long = false: no long row of the launch selects from its keys (every
// one is listed), so the long-row select is not launched
static hipError_t launch_select(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                                hipStream_t stream, bool keyed_long = true) {
    const int64_t max_b = a.key_stride;
    // short rows (skipped when every sequence's first query already has a
    // long row): a wavefront per row up to kWaveSelectKeys keys
    int64_t min_b = INT64_MAX, rows = 0;
    for (int i = 0; i < seqs.n; ++i) {
        const int64_t b = seqs.s[i].pos0 / a.block_size;
        min_b = b < min_b ? b : min_b;
        rows += seqs.s[i].n_q * kGroups;
    }
    hipError_t e = hipSuccess;
    if (min_b <= kWaveSelectKeys) {
        hipLaunchKernelGGL(index_select_wave_kernel, dim3((unsigned)max_nq, (unsigned)seqs.n), dim3(256), 0,
                           stream, seqs, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (max_b <= kWaveSelectKeys || !keyed_long) return e;
    // longer rows: a few rows (decode) get sixteen wavefronts each, with
    // 1024-key steps, so each row's scan has sixteen times the loads in
    // flight (the candidate list then takes k plus one 16384-key step:
    // k <= 1024 keeps it within LDS)
    return rows <= 1024 && a.topk <= 1024 ? launch_select_long<16>(seqs, max_nq, a, stream)
                                          : launch_select_long<4>(seqs, max_nq, a, stream);
}

size_t index_lds_bytes(int cap) { return (size_t)cap * 32u + 1024u; }

hipError_t launch_index_topk(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                             hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    const size_t lds = index_lds_bytes(a.cap);
    const void* fn = a.store_fp8 ? (const void*)index_topk_kernel<true> : (const void*)index_topk_kernel<false>;
    hipError_t e = set_dynamic_lds(fn, lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * a.n_split), (unsigned)seqs.n);
    if (a.store_fp8)
        hipLaunchKernelGGL(index_topk_kernel<true>, grid, dim3(64), lds, stream, seqs, a);
    else
        hipLaunchKernelGGL(index_topk_kernel<false>, grid, dim3(64), lds, stream, seqs, a);
    return hipGetLastError();
}

template <bool FP8>
hipError_t launch_score_merge(const SeqTable& seqs, dim3 grid, const IndexArgs& a, const CompressArgs& c,
                              hipStream_t stream) {
    switch (c.block_size) {
        case 1: hipLaunchKernelGGL((index_score_merge_kernel<FP8, 1>), grid, dim3(64), 0, stream, seqs, a, c); break;
        case 2: hipLaunchKernelGGL((index_score_merge_kernel<FP8, 2>), grid, dim3(64), 0, stream, seqs, a, c); break;
        case 4: hipLaunchKernelGGL((index_score_merge_kernel<FP8, 4>), grid, dim3(64), 0, stream, seqs, a, c); break;
        case 8: hipLaunchKernelGGL((index_score_merge_kernel<FP8, 8>), grid, dim3(64), 0, stream, seqs, a, c); break;
        case 16: hipLaunchKernelGGL((index_score_merge_kernel<FP8, 16>), grid, dim3(64), 0, stream, seqs, a, c); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_index_split(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                              hipStream_t stream, const CompressArgs* merge) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)(max_nq * a.n_split), (unsigned)seqs.n);
    hipError_t e;
    if (merge) {
        grid.x += 1;
        e = a.store_fp8 ? launch_score_merge<true>(seqs, grid, a, *merge, stream)
                        : launch_score_merge<false>(seqs, grid, a, *merge, stream);
    } else {
        if (a.store_fp8)
            hipLaunchKernelGGL(index_score_kernel<true>, grid, dim3(64), 0, stream, seqs, a);
        else
            hipLaunchKernelGGL(index_score_kernel<false>, grid, dim3(64), 0, stream, seqs, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return launch_select(seqs, max_nq, a, stream);
}

hipError_t launch_index_tiled(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                              hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    const int64_t n_qt = (max_nq + kScoreTileQueries - 1) / kScoreTileQueries;
    // which kinds of tiles the launch holds (listed: long rows, candidate
    // lists; keyed: every key written)
    bool any_listed = false, any_keyed = false, keyed_long = false;
    int64_t n0_listed = 0;        // the largest first-query candidate count of a listed tile
    for (int i = 0; i < seqs.n; ++i) {
        const DevSeq& d = seqs.s[i];
        for (int64_t q0 = 0; q0 < d.n_q; q0 += kScoreTileQueries) {
            const int64_t n0 = (d.pos0 + q0) / a.block_size;
            const bool l = a.listed && list_tile(n0, a.topk);
            any_listed |= l;
            if (l && n0 > n0_listed) n0_listed = n0;
            any_keyed |= !l;
            const int64_t q1 = q0 + kScoreTileQueries < d.n_q ? q0 + kScoreTileQueries : d.n_q;
            keyed_long |= !l && (d.pos0 + q1 - 1) / a.block_size > kWaveSelectKeys;
        }
    }
    hipError_t e;
    hipLaunchKernelGGL(index_qfrag_kernel, dim3((unsigned)((max_nq + 3) / 4), (unsigned)seqs.n),
                       dim3(256), 0, stream, seqs, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 rows_grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    if (any_listed) {
        const dim3 sgrid((unsigned)(n_qt * kSampleParts), (unsigned)seqs.n);
        if (a.store_fp8)
            hipLaunchKernelGGL(index_sample_kernel<true>, sgrid, dim3(256), 0, stream, seqs, a);
        else
            hipLaunchKernelGGL(index_sample_kernel<false>, sgrid, dim3(256), 0, stream, seqs, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(index_tau_kernel, rows_grid, dim3(256), 0, stream, seqs, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(n_qt * a.n_split), (unsigned)seqs.n);
    if (any_keyed) {
        if (a.store_fp8)
            hipLaunchKernelGGL((index_score_tile_kernel<false, true>), grid, dim3(256), 0, stream, seqs, a);
        else
            hipLaunchKernelGGL((index_score_tile_kernel<false, false>), grid, dim3(256), 0, stream, seqs, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (any_listed) {
        if (a.store_fp8)
            hipLaunchKernelGGL((index_score_tile_kernel<true, true>), grid, dim3(256), 0, stream, seqs, a);
        else
            hipLaunchKernelGGL((index_score_tile_kernel<true, false>), grid, dim3(256), 0, stream, seqs, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (any_keyed && (e = launch_select(seqs, max_nq, a, stream, keyed_long)) != hipSuccess) return e;
    if (!any_listed) return hipSuccess;
    IndexArgs al = a;
    al.list_cap = list_capacity(n0_listed, a.topk);
    const size_t lds_l = (size_t)al.list_cap * 8;
    if ((e = set_dynamic_lds((const void*)index_list_select_kernel, lds_l)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(index_list_select_kernel, rows_grid, dim3(256), lds_l, stream, seqs, al);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // rows whose lists failed (usually none): scored again, then selected
    // from their keys; grid-stride loops over the count the device holds
    if (a.store_fp8)
        hipLaunchKernelGGL(index_rescore_kernel<true>, dim3(1024), dim3(256), 0, stream, seqs, a);
    else
        hipLaunchKernelGGL(index_rescore_kernel<false>, dim3(1024), dim3(256), 0, stream, seqs, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.topk <= 1024) {
        const size_t lds_r = select_long_lds<16>(a);
        if ((e = set_dynamic_lds((const void*)index_select_rescue_kernel<16>, lds_r)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(index_select_rescue_kernel<16>, dim3(256), dim3(1024), lds_r, stream, seqs, a);
    } else {
        const size_t lds_r = select_long_lds<4>(a);
        if ((e = set_dynamic_lds((const void*)index_select_rescue_kernel<4>, lds_r)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(index_select_rescue_kernel<4>, dim3(512), dim3(256), lds_r, stream, seqs, a);
    }
    return hipGetLastError();
}

}  // namespace sgqa
