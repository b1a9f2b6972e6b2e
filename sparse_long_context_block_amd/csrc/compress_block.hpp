// Step 1 body: the merge of one completed block into the store, run by one
// wavefront (shared by the compress kernel and the decode scoring launch,
// which carries the merges of calls whose queries read none of the blocks
// they complete).
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache":
//   * "Two paths leave the same hidden state" -- proxy keys are LayerNorm'd
//     and carry a 32-dim rotary span; compression logits are a separate
//     projection.
//   * "Eight tokens become one search key, coordinate by coordinate" -- per
//     completed block and per coordinate d, a max-subtracted softmax of the
//     block's logits for d weights the tokens' coordinate d; FP32
//     accumulation; stored through BF16 into E4M3.
//
// Mapping: lane l owns coordinates 2l and 2l+1 of all B tokens, so the
// per-coordinate softmax over the block is in-lane and the only cross-lane
// work is the LayerNorm statistics and the rotary pair exchange.  Each token
// row is one coalesced 256-byte (proxy key) and 512-byte (logits) wave load;
// the store row is one 256-byte wave store.
#pragma once
#include "sgqa_internal.hpp"

namespace sgqa {
namespace dev {

// store row sq.store_offset + r from the B tokens of block r of sequence sq
template <int B>
__device__ __forceinline__ void compress_block(const DevSeq& sq, int64_t r, const CompressArgs& a) {
    const int lane = lane_id();
    const int d0 = 2 * lane;                        // coordinates d0, d0+1

    float g0 = 1.f, g1 = 1.f, b0 = 0.f, b1 = 0.f;
    if (a.ln_gamma) {
        uint32_t gg = *(const uint32_t*)(a.ln_gamma + d0);
        g0 = bf16_to_f32(gg & 0xFFFFu);
        g1 = bf16_to_f32(gg >> 16);
    }
    if (a.ln_beta) {
        uint32_t bb = *(const uint32_t*)(a.ln_beta + d0);
        b0 = bf16_to_f32(bb & 0xFFFFu);
        b1 = bf16_to_f32(bb >> 16);
    }

    // rotary span: lanes 0..7 hold the first halves (pairs j = d0, d0+1),
    // lanes 8..15 the second halves (pairs j = d0-16, d0-15)
    constexpr int kHalf = kRopeDim / 2;
    const bool first_half = d0 < kHalf;
    const bool in_rope = d0 < kRopeDim;
    const int pair_j = first_half ? d0 : d0 - kHalf;
    const int partner = first_half ? lane + kHalf / 2 : lane - kHalf / 2;
    const double th0 = in_rope ? a.theta[pair_j] : 0.0;
    const double th1 = in_rope ? a.theta[pair_j + 1] : 0.0;

    // the block's B tokens are consecutive rows (a 16-token page holds whole
    // blocks: B divides 16)
    const int64_t row0 = a.page_table ? paged_row(a.page_table + sq.kv_offset, a.n_pages, (int64_t)B * r)
                                      : sq.kv_offset + (int64_t)B * r;
    float k0[B], k1[B], c0[B], c1[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int64_t pos = (int64_t)B * r + j;
        const int64_t row = row0 + j;
        uint32_t xx = *(const uint32_t*)(a.proxy_k + row * kIdxDim + d0);
        float2 cc = *(const float2*)(a.logits + row * kIdxDim + d0);
        c0[j] = cc.x;
        c1[j] = cc.y;
        float x0 = bf16_to_f32(xx & 0xFFFFu), x1 = bf16_to_f32(xx >> 16);
        // LayerNorm, population variance, two-pass in fp32
        float mean = wave_sum(x0 + x1) * (1.0f / kIdxDim);
        float e0 = x0 - mean, e1 = x1 - mean;
        float var = wave_sum(e0 * e0 + e1 * e1) * (1.0f / kIdxDim);
        float inv = 1.0f / sqrtf(var + a.eps);
        float y0 = e0 * inv * g0 + b0;
        float y1 = e1 * inv * g1 + b1;
        // rotary: (y_j, y_{j+16}) <- (y_j c - y_{j+16} s, y_j s + y_{j+16} c)
        float p0 = __shfl(y0, partner, 64);
        float p1 = __shfl(y1, partner, 64);
        if (in_rope) {
            float cs0, sn0, cs1, sn1;
            rope_cos_sin(pos, th0, &cs0, &sn0);
            rope_cos_sin(pos, th1, &cs1, &sn1);
            if (first_half) {
                y0 = y0 * cs0 - p0 * sn0;
                y1 = y1 * cs1 - p1 * sn1;
            } else {
                y0 = p0 * sn0 + y0 * cs0;
                y1 = p1 * sn1 + y1 * cs1;
            }
        }
        k0[j] = y0;
        k1[j] = y1;
    }

    // per-coordinate softmax over the block's tokens, maximum subtracted
    float m0 = c0[0], m1 = c1[0];
#pragma unroll
    for (int j = 1; j < B; ++j) {
        m0 = fmaxf(m0, c0[j]);
        m1 = fmaxf(m1, c1[j]);
    }
    float n0 = 0.f, n1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < B; ++j) {
        float w0 = expf(c0[j] - m0), w1 = expf(c1[j] - m1);
        s0 += w0;
        s1 += w1;
        n0 += w0 * k0[j];
        n1 += w1 * k1[j];
    }
    uint32_t o0 = f32_to_bf16(n0 / s0);
    uint32_t o1 = f32_to_bf16(n1 / s1);
    if (a.store_q8) {
        o0 = bf16_to_e4m3_as_bf16(o0);
        o1 = bf16_to_e4m3_as_bf16(o1);
    }
    if (a.store_q8 == 2)        // E4M3 codes, one byte per coordinate
        *(uint16_t*)((uint8_t*)a.store + (sq.store_offset + r) * kIdxDim + d0) =
            (uint16_t)(e4m3_code(o0) | (e4m3_code(o1) << 8));
    else
        *(uint32_t*)(a.store + (sq.store_offset + r) * kIdxDim + d0) = o0 | (o1 << 16);
}

}  // namespace dev
}  // namespace sgqa
