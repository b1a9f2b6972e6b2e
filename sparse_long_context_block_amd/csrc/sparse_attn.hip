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
// chunks w, w+4, ...  Per chunk it
//   * loads the 16 K rows straight into the A operand of S^T = K Q^T
//     (v_mfma_f32_16x16x32_bf16; the group's 16 heads are the N dimension,
//     so every gathered K/V byte serves all 16 heads);
//   * runs the online softmax on the result layout, where each lane holds 4
//     tokens of one head: the exponentiated tile is directly the B operand
//     (P^T) of O^T = V^T P^T (v_mfma_f32_16x16x16bf16_1k), no LDS round trip;
//   * transposes the 16 V rows through a small per-wave LDS tile to form the
//     A operand V^T.
// The four wavefronts' (max, sum, O) are merged in LDS; a split call (decode:
// few queries) writes partials that attn_merge_kernel combines.
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;

constexpr int kVtStride = 20;                       // bf16 per V^T row: 16 tokens + pad
constexpr int kWaveBufFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int64_t token_at(int64_t i, int n_sel, int shift_b, int B,
                                            const int32_t* sel, int64_t cur_first) {
    const int64_t j = i >> shift_b;
    if (j < n_sel) return (int64_t)sel[j] * B + (i & (B - 1));
    return cur_first + (i - ((int64_t)n_sel << shift_b));
}

__global__ __launch_bounds__(256) void sparse_attn_kernel(SeqTable seqs, AttnArgs a) {
    extern __shared__ int32_t sel_lds[];                        // [K]
    __shared__ float wave_buf[4][kWaveBufFloats];
    __shared__ int s_nsel;

    const DevSeq sq = seqs.s[blockIdx.y];
    const int split = blockIdx.x % a.n_split;
    const int g = (blockIdx.x / a.n_split) % kGroups;
    const int64_t qi = blockIdx.x / (a.n_split * kGroups);
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

    float mrow = -INFINITY;   // running max of head m, log2 domain
    float lsum = 0.f;
    f32x4 o[12];
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint16_t* vt = (uint16_t*)wave_buf[w];
    const uint16_t* kbase = a.k + (sq.kv_offset * kGroups + g) * kHeadDim;
    const uint16_t* vbase = a.v + (sq.kv_offset * kGroups + g) * kHeadDim;
    constexpr int64_t kRowStride = (int64_t)kGroups * kHeadDim;

    for (int64_t c = c_lo + w; c < c_hi; c += 4) {
        // this lane's token for the K/V loads
        const int64_t ti = 16 * c + m;
        int64_t tok = ti < n_tok ? token_at(ti, n_sel, shift_b, B, sel_lds, cur_first) : t;
        tok = tok < 0 ? 0 : (tok > t ? t : tok);   // malformed ids never read past the cache
        const uint16_t* krow = kbase + tok * kRowStride + 8 * qq;
        const uint16_t* vrow = vbase + tok * kRowStride;
        uint4 kr[6], vr[6];
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) kr[kk] = *(const uint4*)(krow + 32 * kk);
#pragma unroll
        for (int j = 0; j < 6; ++j) vr[j] = *(const uint4*)(vrow + 8 * (qq + 4 * j));

        // S^T[token][head] = K Q^T
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) s = mfma_16x16x32(as_bf16x8(kr[kk]), qf[kk], s);

        // online softmax; lane holds tokens 16c + 4qq + i of head m
        float xv[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = 16 * c + 4 * qq + i < n_tok;
            xv[i] = valid ? s[i] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, xv[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mnew = fmaxf(mrow, tmax);           // finite: token 16c is valid
        const float alpha = exp2f(mrow - mnew);
        float p[4], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = exp2f(xv[i] - mnew);
            psum += p[i];
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        lsum = lsum * alpha + psum;
        mrow = mnew;
#pragma unroll
        for (int nt = 0; nt < 12; ++nt) o[nt] *= alpha;

        // V^T tile: lane wrote token m, dims 8(qq+4j) .. +7
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const uint32_t w4[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
            const int d0 = 8 * (qq + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(d0 + 2 * e) * kVtStride + m] = (uint16_t)(w4[e] & 0xFFFFu);
                vt[(d0 + 2 * e + 1) * kVtStride + m] = (uint16_t)(w4[e] >> 16);
            }
        }
        wave_lds_sync();

        uint2 pb;
        pb.x = f32_to_bf16(p[0]) | (f32_to_bf16(p[1]) << 16);
        pb.y = f32_to_bf16(p[2]) | (f32_to_bf16(p[3]) << 16);
        const i16x4 pbv = as_i16x4(pb);
#pragma unroll
        for (int nt = 0; nt < 12; ++nt) {
            const uint2 av = *(const uint2*)(vt + (16 * nt + m) * kVtStride + 4 * qq);
            o[nt] = mfma_16x16x16(as_i16x4(av), pbv, o[nt]);
        }
        wave_lds_sync();
    }

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

    const int64_t rg = row * kGroups + g;
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
            a.out[(row * kHeads + g * kHeadsPerGroup + head) * kHeadDim + d] =
                (uint16_t)f32_to_bf16(O / L);
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

// Combine the splits' partial softmax states of one (query, group).
__global__ __launch_bounds__(256) void attn_merge_kernel(SeqTable seqs, AttnMergeArgs a) {
    const DevSeq sq = seqs.s[blockIdx.y];
    const int g = blockIdx.x % kGroups;
    const int64_t qi = blockIdx.x / kGroups;
    if (qi >= sq.n_q) return;
    const int64_t row = sq.q_offset + qi;
    const int64_t rg = row * kGroups + g;
    for (int e = threadIdx.x; e < kHeadsPerGroup * kHeadDim; e += 256) {
        const int head = e / kHeadDim;
        const int d = e - head * kHeadDim;
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s)
            M = fmaxf(M, a.part_ml[((rg * a.n_split + s) * kHeadsPerGroup + head) * 2]);
        float L = 0.f, O = 0.f;
        for (int s = 0; s < a.n_split; ++s) {
            const int64_t part = rg * a.n_split + s;
            const float ms = a.part_ml[(part * kHeadsPerGroup + head) * 2];
            if (ms == -INFINITY) continue;
            const float sc = exp2f(ms - M);
            L += a.part_ml[(part * kHeadsPerGroup + head) * 2 + 1] * sc;
            O += a.part_o[(part * kHeadsPerGroup + head) * kHeadDim + d] * sc;
        }
        a.out[(row * kHeads + g * kHeadsPerGroup + head) * kHeadDim + d] = (uint16_t)f32_to_bf16(O / L);
        if (a.lse && d == 0) a.lse[row * kHeads + g * kHeadsPerGroup + head] = (M + log2f(L)) * kLn2;
    }
}

}  // namespace

hipError_t launch_sparse_attn(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                              hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    const size_t lds = (size_t)a.topk * sizeof(int32_t);
    hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(max_nq * kGroups * a.n_split), (unsigned)seqs.n);
    hipLaunchKernelGGL(sparse_attn_kernel, grid, dim3(256), lds, stream, seqs, a);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const SeqTable& seqs, int64_t max_nq, const AttnMergeArgs& a,
                             hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL(attn_merge_kernel, grid, dim3(256), 0, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
