// Step 4: sparse GQA attention over the original K/V of the selected blocks.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache":
//   * "Main attention still reads original K/V" -- head h uses group
//     g(h) = floor(h/16); ordinary scaled dot products and a softmax over the
//     group's selected original tokens (not over summaries).
//   * "Selection is a weighted ReLU score, not attention softmax" -- the
//     current block is appended unconditionally, restricted to positions <= t.
//   * "What gets cheaper, and what stays length-dependent?" -- at most
//     512*8 + 8 = 4,104 positions per query and group.
//
// Gather mapping (one workgroup of 4 wavefronts per (query, group, split)):
// the query's token list (selected blocks in ascending order, then the
// current block up to t) is cut into 16-token chunks; wavefront w takes
// chunks w, w+4, ..., with the rows of its next chunk in flight while the
// current one is processed (two register sets alternate).  Per chunk it
//   * loads the 16 K rows straight into the A operand of S^T = K Q^T
//     (v_mfma_f32_16x16x32_bf16; the group's 16 heads are the N dimension,
//     so every gathered K/V byte serves all 16 heads);
//   * runs the online softmax on the result layout, where each lane holds 4
//     tokens of one head, with a lazily raised reference max: the
//     exponentiated tile is directly the B operand (P^T) of O^T = V^T P^T
//     (v_mfma_f32_16x16x16bf16_1k), no LDS round trip;
//   * writes the 16 V rows to a per-wave LDS tile and reads the A operand
//     V^T back with transposed reads.
// The four wavefronts' (max, sum, O) are merged in LDS; a split call (decode:
// few queries) writes partials that attn_merge_kernel combines.  Workgroups
// run group-major.
#include "attn_common.hpp"

namespace sgqa {
namespace {

using namespace dev;
using namespace attn;

constexpr int kGVStride = kHeadDim + 8;             // bf16 per row of a wave's V tile (100 dwords)
constexpr int kWaveBufFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;
static_assert(16 * kGVStride * 2 <= kWaveBufFloats * 4, "a wave's V tile fits its merge buffer");

// Cache row of entry i of the query's token list.  Contiguous caches:
// sel[j] holds selected block ids, rows are positions (cur0 = first position
// of the current block).  Paged caches: sel[j] already holds the pool row of
// block j's first position, cur0 the pool row of the current block's (a
// block never straddles a 16-token page).
__device__ __forceinline__ int64_t token_at(int64_t i, int n_sel, int shift_b, int B, bool paged,
                                            const int32_t* sel, int64_t cur0) {
    const int64_t j = i >> shift_b;
    if (j < n_sel) return (paged ? (int64_t)sel[j] : (int64_t)sel[j] * B) + (i & (B - 1));
    return cur0 + (i - ((int64_t)n_sel << shift_b));
}

// K/V rows of chunk c for this lane (token 16c + m; K dims 32kk + 8qq, V
// dims 8(qq + 4j)); chunks past the token list read the current token (row
// t_row), whose values stay finite and are masked.  Rows are clamped to
// [0, row_max], so malformed ids never read outside the cache or pool.
struct GatherRegs {
    uint4 k[6], v[6];
};

__device__ __forceinline__ GatherRegs gather_chunk(int64_t c, int m, int qq, int64_t n_tok, int n_sel, int shift_b,
                                                   int B, bool paged, const int32_t* sel_lds, int64_t cur0,
                                                   int64_t t_row, int64_t row_max, const uint16_t* kbase,
                                                   const uint16_t* vbase) {
    constexpr int64_t kRowStride = (int64_t)kGroups * kHeadDim;
    const int64_t ti = 16 * c + m;
    int64_t tok = ti < n_tok ? token_at(ti, n_sel, shift_b, B, paged, sel_lds, cur0) : t_row;
    tok = tok < 0 ? 0 : (tok > row_max ? row_max : tok);
    const uint16_t* krow = kbase + tok * kRowStride + 8 * qq;
    const uint16_t* vrow = vbase + tok * kRowStride;
    GatherRegs r;
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) r.k[kk] = *(const uint4*)(krow + 32 * kk);
#pragma unroll
    for (int j = 0; j < 6; ++j) r.v[j] = *(const uint4*)(vrow + 8 * (qq + 4 * j));
    return r;
}

struct GatherState {
    f32x4 o[12];       // O^T: dims 16nt + 4qq + i of head m
    float m_use;       // reference max of head m (raw score units), raised lazily
    float lsum;        // this lane's tokens' sum relative to it
};

struct GatherLane {
    uint16_t* vtile;   // this wavefront's V tile in LDS
    int tr_off;        // this lane's transposed-read offset in it
    int m, qq;
    int64_t n_tok;
    float sl2;
};

// One 16-token chunk.  The V rows go into the wavefront's tile (100-dword
// rows: the b128 row writes are conflict-free); the O^T A operand comes out
// of it with ds_read_b64_tr_b16: lane 16G + 4i + c supplies row 4G + i, dims
// 4c..4c+3 of a 16-dim block, and lane 16G + j receives dim j of tokens
// 4G..4G+3 -- row j, k = 4G + i of v_mfma_f32_16x16x16bf16_1k.  The softmax
// runs on the S^T result layout (lane: tokens 16c + 4qq + i of head m) with
// a lazily raised reference max; the exponentiated tile is the B operand.
__device__ __forceinline__ void gather_step(GatherState& st, const GatherRegs& r, const bf16x8 (&qf)[6], int64_t c,
                                            const GatherLane& gl) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) s = mfma_16x16x32(as_bf16x8(r.k[kk]), qf[kk], s);
#pragma unroll
    for (int j = 0; j < 6; ++j) *(uint4*)(gl.vtile + gl.m * kGVStride + 8 * (gl.qq + 4 * j)) = r.v[j];
    float xv[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool valid = 16 * c + 4 * gl.qq + i < gl.n_tok;
        xv[i] = valid ? s[i] : -INFINITY;
        tmax = fmaxf(tmax, xv[i]);
    }
    tmax = xor32_max(xor16_max(tmax));
    const float sl2 = gl.sl2;
    const float ts = tmax * sl2;
    float ms = st.m_use * sl2;
    const bool need = ts > ms + kLazyRescale;
    if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(ms - ts) : 1.0f;
#pragma unroll
        for (int nt = 0; nt < 12; ++nt) st.o[nt] *= alpha;
        st.lsum *= alpha;
        if (need) st.m_use = tmax;
        ms = st.m_use * sl2;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(xv[i] * sl2 - ms);   // ms finite: token 16c is valid
        st.lsum += p[i];
    }
    uint2 pb;
    pb.x = pack_bf16(p[0], p[1]);
    pb.y = pack_bf16(p[2], p[3]);
    const i16x4 pbv = as_i16x4(pb);
    wave_lds_sync();
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
        const i16x4 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(gl.vtile + gl.tr_off + 16 * nt));
        st.o[nt] = mfma_16x16x16(av, pbv, st.o[nt]);
    }
    wave_lds_sync();
}

template <bool PAGED>
__global__ __launch_bounds__(256) void sparse_attn_kernel(SeqTable seqs, AttnArgs a) {
    extern __shared__ int32_t sel_lds[];                        // [K]
    __shared__ float wave_buf[4][kWaveBufFloats];
    __shared__ int s_nsel;

    // group-major order: the workgroups in flight read one group's K/V
    // (disjoint cache lines per group), a quarter of the cache's footprint,
    // which keeps the re-read rows of neighbouring queries in the last-level
    // cache
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t per_group = (int64_t)(gridDim.x / kGroups);
    const int g = (int)(blockIdx.x / per_group);
    const int64_t rem = blockIdx.x - g * per_group;
    const int split = (int)(rem % a.n_split);
    const int64_t qi = rem / a.n_split;
    if (qi >= sq.n_q) return;
    const int64_t t = sq.pos0 + qi;
    const int64_t row = sq.q_offset + qi;
    const int B = a.block_size;
    const int shift_b = __builtin_ctz(B);
    const int64_t cur_first = (t / B) * B;

    // selection of (t, g): ids before the first -1
    if (threadIdx.x == 0) s_nsel = a.topk;
    __syncthreads();
    const int32_t* selrow = a.sel + (row * kGroups + g) * a.topk;
    for (int j = threadIdx.x; j < a.topk; j += 256) {
        const int32_t v = selrow[j];
        sel_lds[j] = v;
        if (v < 0) atomicMin(&s_nsel, j);
    }
    __syncthreads();
    const int n_sel = s_nsel;
    // rows: positions of the contiguous cache, or pool rows through the
    // sequence's page table (the selection list becomes pool rows; block ids
    // outside [0, floor(t/B)] are clamped first, so the table is read only
    // inside the sequence's pages)
    int64_t cur0 = cur_first, t_row = t, row_max = t;
    if (PAGED) {
        const int32_t* pt = a.page_table + sq.kv_offset;
        const int64_t b_max = t / B;
        for (int j = threadIdx.x; j < n_sel; j += 256) {
            const int64_t r = sel_lds[j] > b_max ? b_max : sel_lds[j];
            sel_lds[j] = (int32_t)paged_row(pt, a.n_pages, r * B);
        }
        cur0 = paged_row(pt, a.n_pages, cur_first);
        t_row = cur0 + (t - cur_first);
        row_max = a.n_pages * kPageTokens - 1;
        __syncthreads();
    }
    const int64_t n_tok = ((int64_t)n_sel << shift_b) + (t - cur_first + 1);
    const int64_t n_chunks = (n_tok + 15) >> 4;
    const int64_t c_lo = (int64_t)split * a.chunks_per_split;
    const int64_t c_hi = n_chunks < c_lo + a.chunks_per_split ? n_chunks : c_lo + a.chunks_per_split;

    const int w = threadIdx.x >> 6;
    const int lane = lane_id();
    const int qq = lane >> 4;
    const int m = lane & 15;

    // Q^T as the B operand: lane holds Q[head m][32kk + 8qq .. +7]
    const uint16_t* qrow = a.q + (row * kHeads + g * kHeadsPerGroup + m) * kHeadDim + 8 * qq;
    bf16x8 qf[6];
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) qf[kk] = as_bf16x8(*(const uint4*)(qrow + 32 * kk));

    GatherState st;
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) st.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_use = -INFINITY;
    st.lsum = 0.f;
    GatherLane gl;
    gl.vtile = (uint16_t*)wave_buf[w];
    gl.tr_off = (4 * qq + ((lane >> 2) & 3)) * kGVStride + 4 * (lane & 3);
    gl.m = m;
    gl.qq = qq;
    gl.n_tok = n_tok;
    gl.sl2 = a.scale_log2;
    const int64_t row0 = PAGED ? 0 : sq.kv_offset;
    const uint16_t* kbase = a.k + (row0 * kGroups + g) * kHeadDim;
    const uint16_t* vbase = a.v + (row0 * kGroups + g) * kHeadDim;

    // two register sets alternate: one chunk's rows are in flight while the
    // other chunk is processed
    if (c_lo + w < c_hi) {
        GatherRegs ra = gather_chunk(c_lo + w, m, qq, n_tok, n_sel, shift_b, B, PAGED, sel_lds, cur0, t_row, row_max, kbase,
                                     vbase);
        for (int64_t c = c_lo + w; c < c_hi; c += 8) {
            const GatherRegs rb =
                gather_chunk(c + 4, m, qq, n_tok, n_sel, shift_b, B, PAGED, sel_lds, cur0, t_row, row_max, kbase, vbase);
            gather_step(st, ra, qf, c, gl);
            if (c + 4 >= c_hi) break;
            ra = gather_chunk(c + 8, m, qq, n_tok, n_sel, shift_b, B, PAGED, sel_lds, cur0, t_row, row_max, kbase, vbase);
            gather_step(st, rb, qf, c + 4, gl);
        }
    }
    float lsum = st.lsum;
    f32x4 (&o)[12] = st.o;
    const float m_use = st.m_use;
    const float sl2 = a.scale_log2;
    // the head's sum over its four token lanes; the merge takes the max in
    // log2 units
    lsum = xor32_sum(xor16_sum(lsum));
    const float mrow = m_use * sl2;

    // ---- merge the four wavefronts ----
    __syncthreads();
    float* buf = wave_buf[w];
#pragma unroll
    for (int nt = 0; nt < 12; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[m * kHeadDim + 16 * nt + 4 * qq + i] = o[nt][i];
    if (qq == 0) {
        buf[kHeadsPerGroup * kHeadDim + m] = mrow;
        buf[kHeadsPerGroup * kHeadDim + kHeadsPerGroup + m] = lsum;
    }
    __syncthreads();

    const int64_t rg = (sq.ws_row + qi) * kGroups + g;     // partials row
    for (int e = threadIdx.x; e < kHeadsPerGroup * kHeadDim; e += 256) {
        const int head = e / kHeadDim;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            mw[ww] = wave_buf[ww][kHeadsPerGroup * kHeadDim + head];
            M = fmaxf(M, mw[ww]);
        }
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float sc = exp2f(mw[ww] - M);
                L += wave_buf[ww][kHeadsPerGroup * kHeadDim + kHeadsPerGroup + head] * sc;
                O += wave_buf[ww][e] * sc;
            }
        }
        const int d = e - head * kHeadDim;
        if (a.n_split == 1) {
            const int64_t oi = (row * kHeads + g * kHeadsPerGroup + head) * kHeadDim + d;
            a.out[oi] = (uint16_t)f32_to_bf16(a.gate ? O / L * gate_sigmoid(a.gate[oi]) : O / L);
            if (a.lse && d == 0) a.lse[row * kHeads + g * kHeadsPerGroup + head] = (M + log2f(L)) * kLn2;
        } else {
            const int64_t part = rg * a.n_split + split;
            a.part_o[(part * kHeadsPerGroup + head) * kHeadDim + d] = O;
            if (d == 0) {
                a.part_ml[(part * kHeadsPerGroup + head) * 2] = M;
                a.part_ml[(part * kHeadsPerGroup + head) * 2 + 1] = L;
            }
        }
    }
}

// Combine the splits' partial softmax states of one (query, group): each
// split's (max, sum) becomes one weight per head, then every output element
// is a weighted sum of the splits' partial outputs.
__global__ __launch_bounds__(256) void attn_merge_kernel(SeqTable seqs, AttnMergeArgs a) {
    __shared__ float wsc[kMaxAttnSplits][kHeadsPerGroup];
    const DevSeq sq = seqs.s[blockIdx.y];
    const int g = blockIdx.x % kGroups;
    const int64_t qi = blockIdx.x / kGroups;
    if (qi >= sq.n_q) return;
    const int64_t row = sq.q_offset + qi;
    const int64_t rg = (sq.ws_row + qi) * kGroups + g;     // partials row
    const int tid = threadIdx.x;
    if (tid < kHeadsPerGroup) {
        const int head = tid;
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s)
            M = fmaxf(M, a.part_ml[((rg * a.n_split + s) * kHeadsPerGroup + head) * 2]);
        float L = 0.f;
        for (int s = 0; s < a.n_split; ++s) {
            const int64_t pi = ((rg * a.n_split + s) * kHeadsPerGroup + head) * 2;
            const float ms = a.part_ml[pi];
            const float sc = ms == -INFINITY ? 0.0f : exp2f(ms - M);
            wsc[s][head] = sc;
            L += a.part_ml[pi + 1] * sc;
        }
        const float inv = 1.0f / L;
        for (int s = 0; s < a.n_split; ++s) wsc[s][head] *= inv;
        if (a.lse) a.lse[row * kHeads + g * kHeadsPerGroup + head] = (M + log2f(L)) * kLn2;
    }
    __syncthreads();
    for (int e = tid; e < kHeadsPerGroup * kHeadDim; e += 256) {
        const int head = e / kHeadDim;
        float O = 0.f;
        for (int s = 0; s < a.n_split; ++s)
            O += wsc[s][head] * a.part_o[((rg * a.n_split + s) * kHeadsPerGroup) * kHeadDim + e];
        const int64_t oi = (row * kHeads + g * kHeadsPerGroup) * kHeadDim + e;
        a.out[oi] = (uint16_t)f32_to_bf16(a.gate ? O * gate_sigmoid(a.gate[oi]) : O);
    }
}

}  // namespace

template <bool PAGED>
static hipError_t launch_sparse_attn_t(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                                       hipStream_t stream) {
    const size_t lds = (size_t)a.topk * sizeof(int32_t);
    hipError_t e = set_dynamic_lds((const void*)sparse_attn_kernel<PAGED>, lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * kGroups * a.n_split), (unsigned)seqs.n);
    hipLaunchKernelGGL((sparse_attn_kernel<PAGED>), grid, dim3(256), lds, stream, seqs, a);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                              hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    return a.page_table ? launch_sparse_attn_t<true>(seqs, max_nq, a, stream)
                        : launch_sparse_attn_t<false>(seqs, max_nq, a, stream);
}

hipError_t launch_attn_merge(const SeqTable& seqs, int64_t max_nq, const AttnMergeArgs& a,
                             hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL(attn_merge_kernel, grid, dim3(256), 0, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
