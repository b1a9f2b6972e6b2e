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
//   * the 4 groups x 4 heads of one query's indexer queries are exactly the
//     16 rows of a v_mfma_f32_16x16x32_bf16 A operand, so the four groups
//     share every summary tile the wave streams (4x reuse of the store);
//   * a 16-block tile of the store is the B operand, read straight from HBM /
//     L2 into registers (16 B per lane per 32-wide k step, double-buffered);
//   * the result layout puts all 4 heads of (group, block) in one lane, so
//     the weighted ReLU sum is in-lane;
//   * each group's selection is a streaming top-k: a per-group LDS buffer of
//     `cap` (key, block) entries in ascending block order, an acceptance
//     threshold (the current k-th key), and a radix-select compaction back to
//     k entries when the buffer is nearly full.  Keys are order-preserving
//     uint32 images of the fp32 scores (-0 folded into +0); ties keep the
//     earlier entry, which is the lower block id because blocks arrive in
//     ascending order.
// A decode-sized call (few queries) splits each query's candidates over
// several wavefronts; index_merge_kernel then selects from their lists.
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;

// Keep the k entries with the largest keys among (key, idx)[0..n), n > k,
// preferring earlier entries among equal keys, in their original order.
// Runs on one wavefront; `hist` is 256 words of LDS.  Returns the k-th key.
__device__ uint32_t compact_topk(uint32_t* key, int32_t* idx, int n, int k, uint32_t* hist) {
    const int lane = lane_id();
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = lane; b < 256; b += 64) hist[b] = 0u;
        wave_lds_sync();
        for (int i = lane; i < n; i += 64) {
            uint32_t kk = key[i];
            if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
        }
        wave_lds_sync();
        // lane L owns digits 255-4L down to 252-4L
        uint32_t h[4];
        uint32_t tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = hist[255 - 4 * lane - j];
            tot += h[j];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        uint32_t above = incl - tot;   // entries with a larger digit
        int found = -1;
        uint32_t above_found = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (found < 0 && above + h[j] >= (uint32_t)krem) {
                found = 255 - 4 * lane - j;
                above_found = above;
            }
            above += h[j];
        }
        const uint64_t fm = __ballot(found >= 0);
        const int src = (int)__builtin_ctzll(fm);
        const int digit = __shfl(found, src, 64);
        const uint32_t ab = __shfl(above_found, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xFFu << shift;
        krem -= (int)ab;
        wave_lds_sync();
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
            const int j = 8 * (qq & 1) + e;
            float c, s;
            rope_cos_sin(t, rope_theta(j, a.rope_base), &c, &s);
            x[0][e] = first ? (x[0][e] * c - p[e] * s) : (p[e] * s + x[0][e] * c);
        }
    }
    bf16x8 afrag[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 packed;
        packed.x = f32_to_bf16(x[kk][0]) | (f32_to_bf16(x[kk][1]) << 16);
        packed.y = f32_to_bf16(x[kk][2]) | (f32_to_bf16(x[kk][3]) << 16);
        packed.z = f32_to_bf16(x[kk][4]) | (f32_to_bf16(x[kk][5]) << 16);
        packed.w = f32_to_bf16(x[kk][6]) | (f32_to_bf16(x[kk][7]) << 16);
        afrag[kk] = as_bf16x8(packed);
        if (a.q_hat_out && split == 0)
            *(uint4*)(a.q_hat_out + (row * (kGroups * kIdxHeads) + m) * kIdxDim + 32 * kk + 8 * qq) =
                packed;
    }

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

    uint4 bcur[4], bnxt[4];
    if (r_lo < r_hi) {
        const int64_t rr = r_lo + m < r_hi ? r_lo + m : r_lo;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bcur[kk] = load16(store + rr * kIdxDim + 32 * kk);
    }
    for (int64_t r0 = r_lo; r0 < r_hi; r0 += 16) {
        const int64_t rn = r0 + 16;
        if (rn < r_hi) {
            const int64_t rr = rn + m < r_hi ? rn + m : rn;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) bnxt[kk] = load16(store + rr * kIdxDim + 32 * kk);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_16x16x32(afrag[kk], as_bf16x8(bcur[kk]), acc);
        float s = wv.x * fmaxf(acc[0], 0.f);
        s += wv.y * fmaxf(acc[1], 0.f);
        s += wv.z * fmaxf(acc[2], 0.f);
        s += wv.w * fmaxf(acc[3], 0.f);
        const int64_t rr = r0 + m;
        const uint32_t key = score_key(s);
        const bool take = (rr < r_hi) && key > thr;
        const uint64_t am = __ballot(take);
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
        if (cnt0 > a.cap - 16 || cnt1 > a.cap - 16 || cnt2 > a.cap - 16 || cnt3 > a.cap - 16) {
            wave_lds_sync();
            if (cnt0 > a.cap - 16) {
                uint32_t v = compact_topk(keys, idxs, cnt0, a.topk, hist);
                cnt0 = a.topk;
                if (qq == 0) thr = v;
            }
            if (cnt1 > a.cap - 16) {
                uint32_t v = compact_topk(keys + cap, idxs + cap, cnt1, a.topk, hist);
                cnt1 = a.topk;
                if (qq == 1) thr = v;
            }
            if (cnt2 > a.cap - 16) {
                uint32_t v = compact_topk(keys + 2 * cap, idxs + 2 * cap, cnt2, a.topk, hist);
                cnt2 = a.topk;
                if (qq == 2) thr = v;
            }
            if (cnt3 > a.cap - 16) {
                uint32_t v = compact_topk(keys + 3 * cap, idxs + 3 * cap, cnt3, a.topk, hist);
                cnt3 = a.topk;
                if (qq == 3) thr = v;
            }
        }
        if (rn < r_hi) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) bcur[kk] = bnxt[kk];
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
        if (a.n_split == 1) {
            int32_t* sel = a.sel + rg * a.topk;
            float* ssc = a.sel_scores ? a.sel_scores + rg * a.topk : nullptr;
            for (int j = lane; j < a.topk; j += 64) {
                const bool in = j < c;
                sel[j] = in ? idxs[g * cap + j] : -1;
                if (ssc) ssc[j] = in ? key_score(keys[g * cap + j]) : 0.0f;
            }
        } else {
            const int64_t part = rg * a.n_split + split;
            for (int j = lane; j < c; j += 64) {
                a.part_key[part * a.topk + j] = keys[g * cap + j];
                a.part_idx[part * a.topk + j] = idxs[g * cap + j];
            }
            if (lane == 0) a.part_cnt[part] = c;
        }
    }
}

// Final selection of a split call: concatenate the splits' lists (ascending
// block order), keep the k best.  One wavefront per (query, group).
__global__ __launch_bounds__(64) void index_merge_kernel(SeqTable seqs, IndexMergeArgs a) {
    extern __shared__ uint32_t lds[];
    const int capm = a.n_split * a.topk;
    uint32_t* keys = lds;
    int32_t* idxs = (int32_t*)(lds + capm);
    uint32_t* hist = lds + 2 * capm;

    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t qi = blockIdx.x / kGroups;
    const int g = blockIdx.x % kGroups;
    if (qi >= sq.n_q) return;
    const int lane = lane_id();
    const int64_t rg = (sq.q_offset + qi) * kGroups + g;

    int n = 0;
    for (int s = 0; s < a.n_split; ++s) {
        const int64_t part = rg * a.n_split + s;
        const int c = a.part_cnt[part];
        for (int j = lane; j < c; j += 64) {
            keys[n + j] = a.part_key[part * a.topk + j];
            idxs[n + j] = a.part_idx[part * a.topk + j];
        }
        n += c;
    }
    wave_lds_sync();
    if (n > a.topk) {
        compact_topk(keys, idxs, n, a.topk, hist);
        n = a.topk;
    }
    int32_t* sel = a.sel + rg * a.topk;
    float* ssc = a.sel_scores ? a.sel_scores + rg * a.topk : nullptr;
    for (int j = lane; j < a.topk; j += 64) {
        const bool in = j < n;
        sel[j] = in ? idxs[j] : -1;
        if (ssc) ssc[j] = in ? key_score(keys[j]) : 0.0f;
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

hipError_t launch_index_merge(const SeqTable& seqs, int64_t max_nq, const IndexMergeArgs& a,
                              hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    const size_t lds = (size_t)a.n_split * a.topk * 8u + 1024u;
    hipError_t e = hipFuncSetAttribute((const void*)index_merge_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL(index_merge_kernel, grid, dim3(64), lds, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
