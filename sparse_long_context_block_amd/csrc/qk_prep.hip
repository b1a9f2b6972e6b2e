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
// Mapping (an HBM-bound stream of 384-byte rows): a workgroup of 4
// wavefronts takes 4 consecutive tokens, i.e. 4 x 72 rows (64 Q heads,
// 4 K groups, 4 V groups per token), as 72 quads of 4 rows of one token and
// one kind.  It first writes the 4 tokens' rotary cosines and sines and
// cache rows to LDS.  A wavefront then takes every fourth quad, three quads
// at a time with all their loads issued before any arithmetic (4.5 KB in
// flight per wavefront): 16 lanes per row, lane l holding elements
// 4l..4l+3 of each 64-element third of the row (three coalesced 128-byte
// pieces per row).  The row's sum of squares is reduced over its 16 lanes;
// rotary partners are exchanged through a per-wavefront LDS block.
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;

constexpr int kTokensPerBlock = 4;
constexpr int kQuadsPerToken = kHeads / 4 + 2;        // 16 Q quads, 1 K quad, 1 V quad
constexpr int kQuadsPerBlock = kTokensPerBlock * kQuadsPerToken;
constexpr int kQuadsPerWave = kQuadsPerBlock / 4;
constexpr int kBatch = 3;                             // quads in flight per wavefront
constexpr int64_t kMaxGridTokens = 1 << 22;           // longer calls loop over token groups
static_assert(kQuadsPerWave % kBatch == 0, "quads split into whole batches");
static_assert(kHeadDim == 3 * 64, "a row is three 64-element thirds");

__device__ __forceinline__ float lo_f(uint32_t u) { return bf16_to_f32(u & 0xFFFFu); }
__device__ __forceinline__ float hi_f(uint32_t u) { return bf16_to_f32(u >> 16); }

__global__ __launch_bounds__(256) void qk_prep_kernel(SeqTable seqs, QkPrepArgs a) {
    __shared__ float2 rot[kTokensPerBlock][kHeadDim / 2];   // (cos, sin) of pair j per token
    __shared__ int64_t crow_s[kTokensPerBlock];
    __shared__ float ybuf[4][4][kHeadDim];                  // per wavefront: its quad's 4 rows
    const DevSeq sq = seqs.s[blockIdx.y];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = lane >> 4, l16 = lane & 15;
    const int half = a.rope_dim >> 1;
    const int64_t groups = (sq.n_q + kTokensPerBlock - 1) / kTokensPerBlock;

    // per-lane gammas of the lane's 12 elements (1.0 when absent)
    uint2 qg[3], kg[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const int d = 64 * c + 4 * l16;
        qg[c] = a.q_gamma ? *(const uint2*)(a.q_gamma + d) : make_uint2(0x3F803F80u, 0x3F803F80u);
        kg[c] = a.k_gamma ? *(const uint2*)(a.k_gamma + d) : make_uint2(0x3F803F80u, 0x3F803F80u);
    }

    // token groups in a grid-stride loop (the trip count is uniform over the workgroup)
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
        const int64_t i0 = grp * kTokensPerBlock;
        for (int k = threadIdx.x; k < kTokensPerBlock * half; k += blockDim.x) {
            const int tt = k / half, j = k - tt * half;
            float c, s;
            rope_cos_sin(sq.pos0 + i0 + tt, exp(-(2.0 * j / a.rope_dim) * a.log_base), &c, &s);
            rot[tt][j] = make_float2(c, s);
        }
        // cache rows of the group's tokens (slots past the last token stay
        // unread: their page-table entries may lie past the sequence's)
        if (threadIdx.x < kTokensPerBlock && i0 + threadIdx.x < sq.n_q) {
            const int64_t t = sq.pos0 + i0 + threadIdx.x;
            crow_s[threadIdx.x] = a.page_table ? paged_row(a.page_table + sq.kv_offset, a.n_pages, t)
                                               : sq.kv_offset + t;
        }
        __syncthreads();

#pragma unroll 1
        for (int b = 0; b < kQuadsPerWave / kBatch; ++b) {
            const uint16_t* src[kBatch];
            uint16_t* dst[kBatch];
            int kind[kBatch], tt[kBatch];              // kind: 0 Q, 1 K, 2 V, -1 none
            uint2 raw[kBatch][3];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int qd = wave + 4 * (b * kBatch + u);
                tt[u] = qd / kQuadsPerToken;
                const int kq = qd - tt[u] * kQuadsPerToken;
                const int64_t i = i0 + tt[u];
                const int64_t qrow = sq.q_offset + i;
                const int64_t crow = crow_s[tt[u]];
                kind[u] = i >= sq.n_q ? -1 : (kq < kHeads / 4 ? 0 : (kq == kHeads / 4 ? 1 : 2));
                if (kind[u] == 2 && !a.v_raw) kind[u] = -1;
                src[u] = nullptr;
                dst[u] = nullptr;
                if (kind[u] == 0) {
                    src[u] = a.q_raw + (qrow * kHeads + 4 * kq + row) * kHeadDim;
                    dst[u] = a.q_out + (qrow * kHeads + 4 * kq + row) * kHeadDim;
                } else if (kind[u] == 1) {
                    src[u] = a.k_raw + (qrow * kGroups + row) * kHeadDim;
                    dst[u] = a.k_cache + (crow * kGroups + row) * kHeadDim;
                } else if (kind[u] == 2) {
                    src[u] = a.v_raw + (qrow * kGroups + row) * kHeadDim;
                    dst[u] = a.v_cache + (crow * kGroups + row) * kHeadDim;
                }
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    raw[u][c] = kind[u] >= 0 ? *(const uint2*)(src[u] + 64 * c + 4 * l16)
                                             : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (kind[u] < 0) continue;                 // wave-uniform
                if (kind[u] == 2) {                        // V: a copy
#pragma unroll
                    for (int c = 0; c < 3; ++c) *(uint2*)(dst[u] + 64 * c + 4 * l16) = raw[u][c];
                    continue;
                }
                float x[12];
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    x[4 * c + 0] = lo_f(raw[u][c].x);
                    x[4 * c + 1] = hi_f(raw[u][c].x);
                    x[4 * c + 2] = lo_f(raw[u][c].y);
                    x[4 * c + 3] = hi_f(raw[u][c].y);
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 12; ++e) ss += x[e] * x[e];
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);   // the row's 16 lanes
                const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
                const uint2* gw = kind[u] == 0 ? qg : kg;
                wave_lds_sync();                           // the previous quad's partner reads are done
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const float g[4] = {lo_f(gw[c].x), hi_f(gw[c].x), lo_f(gw[c].y), hi_f(gw[c].y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[4 * c + e] = x[4 * c + e] * inv * g[e];
                        ybuf[wave][row][64 * c + 4 * l16 + e] = x[4 * c + e];
                    }
                }
                wave_lds_sync();
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int d = 64 * c + 4 * l16 + e;
                        const float y = x[4 * c + e];
                        o[e] = y;
                        if (d < 2 * half) {
                            const bool first = d < half;
                            const int j = first ? d : d - half;
                            const float p = ybuf[wave][row][first ? d + half : d - half];
                            const float2 cs = rot[tt[u]][j];
                            o[e] = first ? y * cs.x - p * cs.y : p * cs.y + y * cs.x;
                        }
                    }
                    *(uint2*)(dst[u] + 64 * c + 4 * l16) =
                        make_uint2(f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16),
                                   f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16));
                }
            }
        }
        __syncthreads();                                   // rot[] and crow_s[] reused by the next group
    }
}

}  // namespace

hipError_t launch_qk_prep(const SeqTable& seqs, int64_t max_nq, const QkPrepArgs& a, hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    int64_t groups = (max_nq + kTokensPerBlock - 1) / kTokensPerBlock;
    if (groups > kMaxGridTokens / kTokensPerBlock) groups = kMaxGridTokens / kTokensPerBlock;
    dim3 grid((unsigned)groups, (unsigned)seqs.n);
    hipLaunchKernelGGL(qk_prep_kernel, grid, dim3(256), 0, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
