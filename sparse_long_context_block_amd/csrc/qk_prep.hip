// Neighbour of the path, before it: the main Q/K producer.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache",
// section "Two paths leave the same hidden state": the main path normalizes
// Q and K and applies the layer's partial rotary span (its width is
// head_dim times a partial-rotary factor the page names but does not give,
// so span and base are parameters).  For each new token t of a sequence:
//   q_out[t, h]     = bf16(RoPE_t(RMSNorm(q_raw[t, h]) * q_gamma)),  h < 64
//   k_cache[t, g]   = bf16(RoPE_t(RMSNorm(k_raw[t, g]) * k_gamma)),  g < 4
//   v_cache[t, g]   = v_raw[t, g]                                   (optional)
// RMSNorm over the head's 192 dims in fp32; the rotary span rotates pairs
// (j, j + span/2) by t * base^(-2j/span) (the indexer's convention), the
// angle reduced in fp64.  Cache rows: kv_offset + t, or the pool row of t
// through the sequence's page table.
//
// Mapping: one wavefront per 192-element row (the token's 64 Q heads, 4 K
// groups and, with v_raw, 4 V groups: 72 rows per token), lane l holding
// elements l, l + 64 and l + 128 (three coalesced 128-byte loads); the
// rotary partners are exchanged through a per-wavefront LDS row.
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;

constexpr int kRowsPerToken = kHeads + 2 * kGroups;   // Q heads, K groups, V groups

__global__ __launch_bounds__(256) void qk_prep_kernel(SeqTable seqs, QkPrepArgs a) {
    __shared__ float ybuf[4][kHeadDim];
    const DevSeq sq = seqs.s[blockIdx.y];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;          // (token, row) index
    const int64_t i = r / kRowsPerToken;
    const int rr = (int)(r - i * kRowsPerToken);
    if (i >= sq.n_q) return;
    const bool is_q = rr < kHeads, is_k = !is_q && rr < kHeads + kGroups;
    const int g = is_q ? 0 : (is_k ? rr - kHeads : rr - kHeads - kGroups);
    const int64_t t = sq.pos0 + i;
    const int64_t crow = a.page_table ? paged_row(a.page_table + sq.kv_offset, a.n_pages, t) : sq.kv_offset + t;
    if (!is_q && !is_k) {                                       // V: a copy
        if (!a.v_raw) return;
        const uint16_t* src = a.v_raw + ((sq.q_offset + i) * kGroups + g) * kHeadDim;
        uint16_t* dst = a.v_cache + (crow * kGroups + g) * kHeadDim;
#pragma unroll
        for (int e = 0; e < 3; ++e) dst[lane + 64 * e] = src[lane + 64 * e];
        return;
    }
    const uint16_t* src = is_q ? a.q_raw + ((sq.q_offset + i) * kHeads + rr) * kHeadDim
                               : a.k_raw + ((sq.q_offset + i) * kGroups + g) * kHeadDim;
    const uint16_t* gam = is_q ? a.q_gamma : a.k_gamma;
    float x[3];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
        x[e] = bf16_to_f32(src[lane + 64 * e]);
        ss += x[e] * x[e];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
    for (int e = 0; e < 3; ++e) {
        x[e] *= inv;
        if (gam) x[e] *= bf16_to_f32(gam[lane + 64 * e]);
        ybuf[wave][lane + 64 * e] = x[e];
    }
    wave_lds_sync();
    const int half = a.rope_dim >> 1;
    uint16_t* dst = is_q ? a.q_out + ((sq.q_offset + i) * kHeads + rr) * kHeadDim
                         : a.k_cache + (crow * kGroups + g) * kHeadDim;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
        const int d = lane + 64 * e;
        float y = x[e];
        if (d < 2 * half) {
            const bool first = d < half;
            const int j = first ? d : d - half;
            const float p = ybuf[wave][first ? d + half : d - half];
            float c, s;
            rope_cos_sin(t, exp(-(2.0 * j / a.rope_dim) * a.log_base), &c, &s);
            y = first ? y * c - p * s : p * s + y * c;
        }
        dst[d] = (uint16_t)f32_to_bf16(y);
    }
}

}  // namespace

hipError_t launch_qk_prep(const SeqTable& seqs, int64_t max_nq, const QkPrepArgs& a, hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)((max_nq * kRowsPerToken + 3) / 4), (unsigned)seqs.n);
    hipLaunchKernelGGL(qk_prep_kernel, grid, dim3(256), 0, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
