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

// ---------------------------------------------------------------------------
// Tiled kernel for dense-ish selections (selected share of the candidates
// >= 1/4, e.g. every query of an 8K prefill at k = 512 blocks).
//
// One workgroup = 2*NW consecutive queries x one group; wavefront w owns two
// queries x 16 heads = 32 columns.  The workgroup walks the causal range in
// contiguous 32-token tiles; K and V rows go through LDS once (row-major,
// padded) and serve 32*NW (query, head) columns.  A per-query bitmap of the
// selected blocks (plus the current block, positions <= t) masks the scores,
// so every query still attends over exactly its own token set.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128),
//                 B = Q^T (registers)
//   O^T = V^T P^T v_mfma_f32_32x32x16_bf16, A = V^T read from the row-major
//                 V tile with ds_read_b64_tr_b16 (each 16-lane group gets a
//                 4-token x 16-dim block transposed), B = P^T: the
//                 exponentiated S^T result layout with the token order
//                 permuted identically in A and B, so P never leaves
//                 registers.
// Each lane holds one (query, head) column, so the running max / sum are
// per lane; the max is rescaled lazily (only when it grows by more than
// 2^8), which keeps O exact because O and the sum share the reference max.
// Global loads run two tiles ahead through registers (3 x 16 B per thread
// per tile), LDS is double-buffered.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4v;
typedef __attribute__((ext_vector_type(8))) short i16x8v;

constexpr int kTileTok = 32;
constexpr int kKStrideU = kHeadDim + 8;       // bf16 per K row in LDS (400 B: b128 reads conflict-free)
constexpr int kVStrideU = kHeadDim + 32;      // bf16 per V row in LDS (448 B: transposed reads conflict-free)
constexpr int kKTileElems = kTileTok * kKStrideU;
constexpr int kVTileElems = kTileTok * kVStrideU;
constexpr int kBufElems = kKTileElems + kVTileElems;
constexpr int kHalfChunks = kTileTok * kHeadDim / 8;       // 16-byte chunks of one K (or V) tile
constexpr int kOutStride = kHeadDim + 8;      // bf16 per staged output row (400 B)
constexpr float kLazyRescale = 8.0f;          // log2 units

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4v lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4v*)(p));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// three 16-byte chunks per thread per tile (512 threads x 3 = 2 x 768 chunks)
struct KVStage {
    uint4 c0, c1, c2;
};

struct UnionCtx {
    const uint16_t* kb;
    const uint16_t* vb;
    int64_t t_last;
    int tid;
};

__device__ __forceinline__ uint4 load_chunk(const UnionCtx& u, int tile, int c) {
    const bool is_v = c >= kHalfChunks;
    const int cc = is_v ? c - kHalfChunks : c;
    const int tok = cc / 24, d8 = (cc - tok * 24) * 8;
    int64_t pos = (int64_t)tile * kTileTok + tok;
    pos = pos > u.t_last ? u.t_last : pos;
    return *(const uint4*)((is_v ? u.vb : u.kb) + pos * ((int64_t)kGroups * kHeadDim) + d8);
}

__device__ __forceinline__ void store_chunk(uint16_t* buf, int c, uint4 v) {
    const bool is_v = c >= kHalfChunks;
    const int cc = is_v ? c - kHalfChunks : c;
    const int tok = cc / 24, d8 = (cc - tok * 24) * 8;
    *(uint4*)(buf + (is_v ? kKTileElems + tok * kVStrideU : tok * kKStrideU) + d8) = v;
}

__device__ __forceinline__ void gload(const UnionCtx& u, int tile, KVStage& r) {
    r.c0 = load_chunk(u, tile, u.tid);
    r.c1 = load_chunk(u, tile, u.tid + 512);
    r.c2 = load_chunk(u, tile, u.tid + 1024);
}

__device__ __forceinline__ void lstore(uint16_t* buf, int tid, const KVStage& r) {
    store_chunk(buf, tid, r.c0);
    store_chunk(buf, tid + 512, r.c1);
    store_chunk(buf, tid + 1024, r.c2);
}

// state of one lane's (query, head) column
struct ColState {
    f32x16 o[6];
    float m_use, lsum;
};

template <int LOG2B>
__device__ __forceinline__ void union_tile(ColState& st, const bf16x8 (&qf)[12], const uint16_t* buf,
                                           int i, uint32_t word, int64_t tq, bool q_ok, int lane,
                                           float sl2) {
    const int hgrp = lane >> 5, col = lane & 31;
    const uint16_t* kt = buf;
    const uint16_t* vt = buf + kKTileElems;
    // S^T = K Q^T for this lane's column
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const uint16_t* kl = kt + col * kKStrideU + 8 * hgrp;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) s = mfma_32x32x16(as_bf16x8(*(const uint4*)(kl + 16 * kk)), qf[kk], s);

    // mask: this query's selected blocks, and positions <= t
    const int64_t tok0 = (int64_t)i * kTileTok;
    const int blk0 = (int)(tok0 >> LOG2B);
    constexpr uint32_t kTileBits = LOG2B == 0 ? 0xFFFFFFFFu : ((1u << (kTileTok >> LOG2B)) - 1u);
    const uint32_t tb = (LOG2B == 0 ? word : (word >> (blk0 & 31))) & kTileBits;
    const int64_t lim64 = tq - tok0;                       // last visible offset in the tile
    const int lim = lim64 > 64 ? 64 : (int)lim64;          // (negative: nothing visible)
    const bool full = q_ok && tb == kTileBits && lim >= kTileTok - 1;
    float x[16];
    if (__ballot(!full) == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = s[r];
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mm = 8 * (r >> 2) + 4 * hgrp + (r & 3);
            const bool valid = q_ok && ((tb >> (mm >> LOG2B)) & 1u) && mm <= lim;
            x[r] = valid ? s[r] : -INFINITY;
        }
    }
    float tmax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, x[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float ts = tmax * sl2;
    float ms = st.m_use * sl2;
    const bool need = ts > ms + kLazyRescale;
    if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(ms - ts) : 1.0f;
#pragma unroll
        for (int dt = 0; dt < 6; ++dt) st.o[dt] *= alpha;
        st.lsum *= alpha;
        if (need) st.m_use = tmax;
        ms = st.m_use * sl2;
    }
    const float msub = st.m_use == -INFINITY ? 0.0f : ms;
    float p[16], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(x[r] * sl2 - msub);
        psum += p[r];
    }
    psum += __shfl_xor(psum, 32, 64);
    st.lsum += psum;
    bf16x8 pb[2];
#pragma unroll
    for (int sgi = 0; sgi < 2; ++sgi) {
        uint4 pk;
        pk.x = pack_bf16(p[8 * sgi + 0], p[8 * sgi + 1]);
        pk.y = pack_bf16(p[8 * sgi + 2], p[8 * sgi + 3]);
        pk.z = pack_bf16(p[8 * sgi + 4], p[8 * sgi + 5]);
        pk.w = pack_bf16(p[8 * sgi + 6], p[8 * sgi + 7]);
        pb[sgi] = as_bf16x8(pk);
    }
    // O^T += V^T P^T; k index 8*hgrp+e <-> token 16*sgi + 4*hgrp + (e&3) + 8*(e>>2).
    // Transposed read: this lane supplies row tr_row (+16 sgi, +8), column
    // tr_col + 32 dt; its 16-lane group receives a 4-token x 16-dim block.
    const int tr_grp = lane >> 4;
    const int tr_row = 4 * (tr_grp >> 1) + ((lane >> 2) & 3);
    const int tr_col = 16 * (tr_grp & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < 6; ++dt) {
#pragma unroll
        for (int sgi = 0; sgi < 2; ++sgi) {
            const uint16_t* vr = vt + (16 * sgi + tr_row) * kVStrideU + 32 * dt + tr_col;
            const i16x4v lo = lds_read_tr16(vr);
            const i16x4v hi = lds_read_tr16(vr + 8 * kVStrideU);
            const i16x8v av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            st.o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, av), pb[sgi], st.o[dt]);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel for dense-ish selections (selected share of the candidates
// >= 1/4, e.g. every query of an 8K prefill at k = 512 blocks).
//
// One workgroup = 16 consecutive queries x one group on 8 wavefronts;
// wavefront w owns two queries x 16 heads = 32 columns.  The workgroup walks
// the causal range in contiguous 32-token tiles; K and V rows go through LDS
// once (row-major, padded) and serve 256 (query, head) columns.  A per-query
// bitmap of the selected blocks (plus the current block, positions <= t)
// masks the scores, so every query still attends over exactly its own token
// set.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128),
//                 B = Q^T (registers)
//   O^T = V^T P^T v_mfma_f32_32x32x16_bf16, A = V^T read from the row-major
//                 V tile with ds_read_b64_tr_b16 (each 16-lane group gets a
//                 4-token x 16-dim block transposed), B = P^T: the
//                 exponentiated S^T result layout with the token order
//                 permuted identically in A and B, so P never leaves
//                 registers.
// Each lane holds one (query, head) column, so the running max / sum are
// per lane; the max is rescaled lazily (only when it grows by more than
// 2^8), which keeps O exact because O and the sum share the reference max.
// Global loads run two tiles ahead through registers (3 x 16 B per thread
// per tile), LDS is double-buffered, and the output is staged through LDS so
// each query's 16 heads leave as one contiguous 6 KB row block.
// ---------------------------------------------------------------------------
template <int LOG2B>
__global__ __launch_bounds__(512) void attn_union_kernel(SeqTable seqs, AttnArgs a, int words) {
    constexpr int NW = 8, TQ = 16, NT = 512;
    extern __shared__ uint32_t bitmap[];                         // [TQ][words]
    __shared__ __attribute__((aligned(16))) uint16_t kv_lds[2 * kBufElems];
    __shared__ int s_nsel[TQ];
    static_assert(2 * kBufElems >= NW * 16 * kOutStride, "output staging fits the tile buffers");

    const DevSeq sq = seqs.s[blockIdx.y];
    const int g = blockIdx.x & 3;
    const int64_t n_qt = (sq.n_q + TQ - 1) / TQ;
    const int64_t rank = blockIdx.x >> 2;
    if (rank >= n_qt) return;
    const int64_t q0 = (n_qt - 1 - rank) * TQ;                  // longest tiles first
    const int n_valid = (int)(sq.n_q - q0 < TQ ? sq.n_q - q0 : TQ);
    const int64_t t0 = sq.pos0 + q0;
    const int64_t t_last = t0 + n_valid - 1;
    const int nwords = (int)((t_last >> LOG2B) >> 5) + 1;
    const int tid = threadIdx.x;
    const int K = a.topk;

    UnionCtx u;
    u.kb = a.k + (sq.kv_offset * kGroups + g) * kHeadDim;
    u.vb = a.v + (sq.kv_offset * kGroups + g) * kHeadDim;
    u.t_last = t_last;
    u.tid = tid;
    const int n_tiles = (int)(t_last / kTileTok) + 1;
    KVStage ra, rb;
    gload(u, 0, ra);
    if (n_tiles > 1) gload(u, 1, rb);

    // ---- per-query bitmaps of the selected blocks and the current block ----
    for (int i = tid; i < TQ * nwords; i += NT) bitmap[(i / nwords) * words + i % nwords] = 0u;
    if (tid < TQ) s_nsel[tid] = K;
    __syncthreads();
    const int32_t* selbase = a.sel + ((sq.q_offset + q0) * kGroups + g) * (int64_t)K;
    for (int i = tid; i < n_valid * K; i += NT) {
        const int q = i / K, j = i - q * K;
        if (selbase[(int64_t)q * kGroups * K + j] < 0) atomicMin(&s_nsel[q], j);
    }
    __syncthreads();
    for (int i = tid; i < n_valid * K; i += NT) {
        const int q = i / K, j = i - q * K;
        if (j >= s_nsel[q]) continue;
        const int32_t v = selbase[(int64_t)q * kGroups * K + j];
        const int64_t nb = (t0 + q) >> LOG2B;
        if (v >= 0 && v < nb) atomicOr(&bitmap[q * words + (v >> 5)], 1u << (v & 31));
    }
    if (tid < n_valid) {
        const int64_t cb = (t0 + tid) >> LOG2B;
        atomicOr(&bitmap[tid * words + (int)(cb >> 5)], 1u << (int)(cb & 31));
    }

    // ---- this lane's column: query qw (2 per wave), head ----
    const int wave = tid >> 6, lane = tid & 63, hgrp = lane >> 5, col = lane & 31;
    const int qw = 2 * wave + (col >> 4);
    const int head = col & 15;
    const bool q_ok = qw < n_valid;
    const int64_t tq = t0 + qw;
    const int64_t qrow = sq.q_offset + q0 + (q_ok ? qw : 0);
    bf16x8 qf[12];
    {
        const uint16_t* qp = a.q + (qrow * kHeads + g * kHeadsPerGroup + head) * kHeadDim + 8 * hgrp;
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) qf[kk] = as_bf16x8(*(const uint4*)(qp + 16 * kk));
    }
    const uint32_t* mybits = bitmap + (q_ok ? qw : 0) * words;

    ColState st;
#pragma unroll
    for (int dt = 0; dt < 6; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][r] = 0.f;
    st.m_use = -INFINITY;
    st.lsum = 0.f;
    const float sl2 = a.scale_log2;

    lstore(kv_lds, tid, ra);
    __syncthreads();
    // tile i: compute from buffer i&1; registers of tile i+1 go to the other
    // buffer afterwards; tile i+2 is loaded into the registers just freed
    int i = 0;
    for (; i + 1 < n_tiles; i += 2) {
        if (i + 2 < n_tiles) gload(u, i + 2, ra);
        union_tile<LOG2B>(st, qf, kv_lds, i, mybits[(int)((i * kTileTok) >> LOG2B) >> 5], tq, q_ok,
                          lane, sl2);
        lstore(kv_lds + kBufElems, tid, rb);
        __syncthreads();
        if (i + 3 < n_tiles) gload(u, i + 3, rb);
        union_tile<LOG2B>(st, qf, kv_lds + kBufElems, i + 1,
                          mybits[(int)(((i + 1) * kTileTok) >> LOG2B) >> 5], tq, q_ok, lane, sl2);
        if (i + 2 < n_tiles) lstore(kv_lds, tid, ra);
        __syncthreads();
    }
    if (i < n_tiles) {
        union_tile<LOG2B>(st, qf, kv_lds, i, mybits[(int)((i * kTileTok) >> LOG2B) >> 5], tq, q_ok,
                          lane, sl2);
        __syncthreads();
    }

    // ---- epilogue: O^T[d][col] for d = 32dt + 8j + 4hgrp + i, normalised,
    //      staged per query in LDS, then written as contiguous 6 KB rows ----
    const float inv = 1.0f / st.lsum;
    if (hgrp == 0 && q_ok && a.lse)
        a.lse[qrow * kHeads + g * kHeadsPerGroup + head] = (st.m_use * sl2 + log2f(st.lsum)) * kLn2;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
        if ((col >> 4) == phase) {
            uint16_t* orow = kv_lds + (wave * 16 + head) * kOutStride;
#pragma unroll
            for (int dt = 0; dt < 6; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint2 pk;
                    pk.x = pack_bf16(st.o[dt][4 * j] * inv, st.o[dt][4 * j + 1] * inv);
                    pk.y = pack_bf16(st.o[dt][4 * j + 2] * inv, st.o[dt][4 * j + 3] * inv);
                    *(uint2*)(orow + 32 * dt + 8 * j + 4 * hgrp) = pk;
                }
        }
        __syncthreads();
        // 8 queries x 16 heads x 24 chunks of 16 B
        for (int c = tid; c < NW * 16 * 24; c += NT) {
            const int w = c / (16 * 24);
            const int rem = c - w * 16 * 24;
            const int h = rem / 24, c16 = rem - h * 24;
            const int q = 2 * w + phase;
            if (q < n_valid) {
                const int64_t row = sq.q_offset + q0 + q;
                *(uint4*)(a.out + (row * kHeads + g * kHeadsPerGroup + h) * kHeadDim + 8 * c16) =
                    *(const uint4*)(kv_lds + (w * 16 + h) * kOutStride + 8 * c16);
            }
        }
        __syncthreads();
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
    const int64_t rg = row * kGroups + g;
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
        a.out[(row * kHeads + g * kHeadsPerGroup) * kHeadDim + e] = (uint16_t)f32_to_bf16(O);
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

template <int LOG2B>
static hipError_t launch_union_t(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                                 int words, hipStream_t stream) {
    const size_t lds = (size_t)16 * words * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute((const void*)attn_union_kernel<LOG2B>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t n_qt = (max_nq + 15) / 16;
    dim3 grid((unsigned)(n_qt * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL((attn_union_kernel<LOG2B>), grid, dim3(512), lds, stream, seqs, a, words);
    return hipGetLastError();
}

int union_queries_per_block() { return 16; }

hipError_t launch_attn_union(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                             int words, hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    switch (a.block_size) {
        case 1: return launch_union_t<0>(seqs, max_nq, a, words, stream);
        case 2: return launch_union_t<1>(seqs, max_nq, a, words, stream);
        case 4: return launch_union_t<2>(seqs, max_nq, a, words, stream);
        case 8: return launch_union_t<3>(seqs, max_nq, a, words, stream);
        case 16: return launch_union_t<4>(seqs, max_nq, a, words, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_merge(const SeqTable& seqs, int64_t max_nq, const AttnMergeArgs& a,
                             hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)(max_nq * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL(attn_merge_kernel, grid, dim3(256), 0, stream, seqs, a);
    return hipGetLastError();
}

}  // namespace sgqa
