// Step 4, tiled kernel: sparse GQA attention for dense-ish selections.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache":
//   * "Main attention still reads original K/V" -- head h uses group
//     g(h) = floor(h/16); ordinary scaled dot products and a softmax over the
//     group's selected original tokens.
//   * "Selection is a weighted ReLU score, not attention softmax" -- the
//     current block is appended unconditionally, restricted to positions <= t.
// Queries whose selection covers at least a quarter of their candidates (the
// host routes them here) share most of their K/V tiles with their
// neighbours, so this kernel walks the causal range once per 16 queries and
// masks each query's scores to its own token set; the gather kernel
// (sparse_attn.hip) takes the rest.
#include "attn_common.hpp"

namespace sgqa {
namespace {

using namespace dev;
using namespace attn;

// ---------------------------------------------------------------------------
// Tiled kernel for dense-ish selections: tile constants and helpers
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kTileTok = 32;
constexpr int kKStrideU = kHeadDim + 8;       // bf16 per K row in LDS (100 dwords = 4 x odd: b128 reads conflict-free)
constexpr int kVtStrideU = kTileTok + 8;      // bf16 per V^T row (one dim, 32 tokens) in LDS (20 dwords = 4 x odd)
constexpr int kKTileElems = kTileTok * kKStrideU;
constexpr int kVTileElems = kHeadDim * kVtStrideU;
constexpr int kBufElems = kKTileElems + kVTileElems;
constexpr int kVSlots = (kHeadDim / 2) * (kTileTok / 8);   // (dim pair, token octet) slots of one V tile
constexpr int kOutStride = kHeadDim + 8;      // bf16 per staged output row (400 B)
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Staging of one 32-token tile (12 dwords per thread).  Threads below
// kVSlots each carry one V slot -- one dim pair of eight tokens, loaded as
// dwords and transposed with byte permutes into two V^T row pieces -- and
// one K chunk; the remaining threads carry three K chunks.  The eight
// tokens of V slot octet o are the ones the O^T MFMA takes as k = 8o..8o+7:
// 16(o>>1) + 4(o&1) + {0,1,2,3,8,9,10,11}, the token order of the
// exponentiated scores a lane holds.
struct KVStage {
    uint4 a, b, c;
};

struct UnionCtx {
    const uint16_t* kb;        // group slice of the sequence's row 0, or of the page pool
    const uint16_t* vb;
    const int32_t* pt;         // paged: the sequence's page table
    int64_t n_pages;
    int64_t t_last;
    bool vwave;        // this wavefront carries V slots (wave-uniform)
    int o, pr;         // V slot: token octet, dim pair
    int kc[3];         // K chunks carried (one for V wavefronts, three otherwise)
    uint32_t voff;     // byte offset of the V slot's first token within a tile
    uint32_t koff[3];  // byte offsets of the K chunks within a tile
};

constexpr int64_t kRowElems = (int64_t)kGroups * kHeadDim;   // cache row stride in bf16
constexpr int kRowBytes = (int)kRowElems * 2;

__device__ __forceinline__ constexpr int octet_token(int o, int e) {
    return 16 * (o >> 1) + 4 * (o & 1) + (e & 3) + 8 * (e >> 2);
}

__device__ __forceinline__ uint32_t k_chunk_bytes(int c) {
    const int tok = c / 24;
    return (uint32_t)(tok * kRowBytes + (c - tok * 24) * 16);
}

__device__ __forceinline__ void union_ctx_init(UnionCtx& u, int tid) {
    // readfirstlane makes the V/K split a scalar branch: the split falls on a
    // wavefront boundary (kVSlots is a multiple of 64)
    static_assert(kVSlots % 64 == 0, "V slots fill whole wavefronts");
    u.vwave = __builtin_amdgcn_readfirstlane(tid) < kVSlots;
    u.o = tid / 96;
    u.pr = tid - u.o * 96;
    u.kc[0] = tid;                 // V wavefronts: chunks 0..383; others: 384..767 in three strides
    u.kc[1] = tid + 128;
    u.kc[2] = tid + 256;
    u.voff = (uint32_t)(octet_token(u.o, 0) * kRowBytes + 4 * u.pr);
#pragma unroll
    for (int j = 0; j < 3; ++j) u.koff[j] = k_chunk_bytes(u.kc[j]);
}

// Buffer resource over the tile's rows of one group: records end after the
// group's slice of row t_last, so rows past the last query read as zeros
// (finite, and masked out of the softmax) without any clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t tile0, int64_t t_last) {
    const int64_t rows = t_last - tile0 + 1;
    const int nrec = rows >= kTileTok ? kTileTok * kRowBytes : (int)(rows - 1) * kRowBytes + kHeadDim * 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + tile0 * kRowElems), (short)0, nrec, 0x00020000);
}

// Paged caches: rows 0..15 and 16..31 of a tile are two 16-token pages, and
// every load of a wavefront falls in one of them (the V slots of octets 0
// and 1 and the one K chunk of each V wavefront: rows 0..15, V wavefronts 0
// to 2; octets 2 and 3: rows 16..31, V wavefronts 3 to 5; the three K chunks
// of wavefronts 6 and 7: rows 16..31), so a wavefront takes one page's
// resource.  Its records end at the group's slice of row t_last as in
// tile_rsrc; a page wholly past t_last gets no records (reads zeros) and its
// page-table entry is not read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* pool, const UnionCtx& u, int64_t p0) {
    const int64_t rows = u.t_last - p0 + 1;
    if (rows <= 0) return __builtin_amdgcn_make_buffer_rsrc((void*)pool, (short)0, 0, 0x00020000);
    // p0 is wave-uniform: one scalar load, and the resource stays in SGPRs
    int64_t pid = __builtin_amdgcn_readfirstlane(u.pt[p0 / kPageTokens]);
    pid = pid < 0 ? 0 : (pid >= u.n_pages ? u.n_pages - 1 : pid);
    const int nrec = rows >= kPageTokens ? kPageTokens * kRowBytes : (int)(rows - 1) * kRowBytes + kHeadDim * 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(pool + pid * kPageTokens * kRowElems), (short)0, nrec,
                                             0x00020000);
}

template <bool PAGED>
__device__ __forceinline__ void gload(const UnionCtx& u, int tile, KVStage& r) {
    const int64_t tile0 = (int64_t)tile * kTileTok;
    if (PAGED) {
        constexpr uint32_t kHalf = kPageTokens * kRowBytes;
        if (u.vwave) {
            const bool hi = __builtin_amdgcn_readfirstlane(u.o) >= 2;   // V wavefronts 3..5
            const __amdgpu_buffer_rsrc_t vr = page_rsrc(u.vb, u, tile0 + (hi ? kPageTokens : 0));
            const __amdgpu_buffer_rsrc_t kr = page_rsrc(u.kb, u, tile0);
            const uint32_t vo = u.voff - (hi ? kHalf : 0u);
            uint32_t d[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                d[e] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(vo + octet_token(0, e) * kRowBytes), 0, 0);
            r.a = make_uint4(d[0], d[1], d[2], d[3]);
            r.b = make_uint4(d[4], d[5], d[6], d[7]);
            r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)u.koff[0], 0, 0));
        } else {
            const __amdgpu_buffer_rsrc_t kr = page_rsrc(u.kb, u, tile0 + kPageTokens);
            r.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)(u.koff[0] - kHalf), 0, 0));
            r.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)(u.koff[1] - kHalf), 0, 0));
            r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)(u.koff[2] - kHalf), 0, 0));
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(u.kb, tile0, u.t_last);
    if (u.vwave) {
        const __amdgpu_buffer_rsrc_t vr = tile_rsrc(u.vb, tile0, u.t_last);
        uint32_t d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            d[e] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(u.voff + octet_token(0, e) * kRowBytes), 0, 0);
        r.a = make_uint4(d[0], d[1], d[2], d[3]);
        r.b = make_uint4(d[4], d[5], d[6], d[7]);
        r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)u.koff[0], 0, 0));
    } else {
        r.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)u.koff[0], 0, 0));
        r.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)u.koff[1], 0, 0));
        r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)u.koff[2], 0, 0));
    }
}

__device__ __forceinline__ void store_k_chunk(uint16_t* buf, int c, uint4 v) {
    const int tok = c / 24, d8 = (c - tok * 24) * 8;
    *(uint4*)(buf + tok * kKStrideU + d8) = v;
}

__device__ __forceinline__ void lstore(uint16_t* buf, const UnionCtx& u, const KVStage& r) {
    if (u.vwave) {
        // dims 2pr (low halves) and 2pr+1 (high halves) of the eight tokens
        uint4 lo, hi;
        lo.x = __builtin_amdgcn_perm(r.a.y, r.a.x, 0x05040100u);
        lo.y = __builtin_amdgcn_perm(r.a.w, r.a.z, 0x05040100u);
        lo.z = __builtin_amdgcn_perm(r.b.y, r.b.x, 0x05040100u);
        lo.w = __builtin_amdgcn_perm(r.b.w, r.b.z, 0x05040100u);
        hi.x = __builtin_amdgcn_perm(r.a.y, r.a.x, 0x07060302u);
        hi.y = __builtin_amdgcn_perm(r.a.w, r.a.z, 0x07060302u);
        hi.z = __builtin_amdgcn_perm(r.b.y, r.b.x, 0x07060302u);
        hi.w = __builtin_amdgcn_perm(r.b.w, r.b.z, 0x07060302u);
        uint16_t* vt = buf + kKTileElems + (2 * u.pr) * kVtStrideU + 8 * u.o;
        *(uint4*)vt = lo;
        *(uint4*)(vt + kVtStrideU) = hi;
        store_k_chunk(buf, u.kc[0], r.c);
    } else {
        store_k_chunk(buf, u.kc[0], r.a);
        store_k_chunk(buf, u.kc[1], r.b);
        store_k_chunk(buf, u.kc[2], r.c);
    }
}

// S^T = K Q^T for this lane's column over one 32-token tile
__device__ __forceinline__ f32x16 tile_scores(const uint16_t* buf, const bf16x8 (&qf)[12], int lane) {
    const int hgrp = lane >> 5, col = lane & 31;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const uint16_t* kl = buf + col * kKStrideU + 8 * hgrp;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) s = mfma_32x32x16(as_bf16x8(*(const uint4*)(kl + 16 * kk)), qf[kk], s);
    return s;
}

struct UnionState {
    f32x16 o[6];       // O^T accumulators, 192 dims x this lane's column
    f32x16 s;          // newest scores S^T
    bf16x8 pb[2];      // exponentiated scores of the current tile, packed
    float m_use, lsum; // reference max (raw score units) and running sum
};

struct UnionLane {
    const uint32_t* mybits;
    int64_t tq;
    bool q_ok;
    int lane, hgrp, col;
    float sl2;
};

// Matrix work of a tile step: O^T += V^T P^T with the tile's exponentiated
// scores, then S^T = K Q^T for the next tile.  k index
// 8*hgrp+e of half sgi is V^T column 16*sgi + 8*hgrp + e, i.e. token
// 16*sgi + 4*hgrp + (e&3) + 8*(e>>2), the token of S^T register 8*sgi + e.
__device__ __forceinline__ void union_matrix(UnionState& st, const bf16x8 (&qf)[12], const uint16_t* kbuf,
                                             const uint16_t* vbuf, const UnionLane& ln) {
    const uint16_t* vt = vbuf + kKTileElems + ln.col * kVtStrideU + 8 * ln.hgrp;
#pragma unroll
    for (int sgi = 0; sgi < 2; ++sgi)
#pragma unroll
        for (int dt = 0; dt < 6; ++dt) {
            const bf16x8 av = as_bf16x8(*(const uint4*)(vt + 32 * dt * kVtStrideU + 16 * sgi));
            st.o[dt] = mfma_32x32x16(av, st.pb[sgi], st.o[dt]);
        }
    st.s = tile_scores(kbuf, qf, ln.lane);
}

// Vector work of a tile step: mask the scores of tile ti (every score when
// ti is not a tile of the range), update the lazily rescaled max and the
// sum, and pack the exponentiated scores for the matrix work.
template <int LOG2B>
__device__ __forceinline__ void union_vector(UnionState& st, int ti, int n_tiles, const UnionLane& ln) {
    constexpr uint32_t kTileBits = LOG2B == 0 ? 0xFFFFFFFFu : ((1u << (kTileTok >> LOG2B)) - 1u);
    const bool live = ti >= 0 && ti < n_tiles;
    const int64_t tok0 = (int64_t)(live ? ti : 0) * kTileTok;
    const int blk0 = (int)(tok0 >> LOG2B);
    const uint32_t word = ln.mybits[blk0 >> 5];
    const uint32_t tb = (LOG2B == 0 ? word : (word >> (blk0 & 31))) & kTileBits;
    const int64_t lim64 = ln.tq - tok0;
    const int lim = ln.q_ok && live ? (lim64 > 64 ? 64 : (int)lim64) : -1;
    float tmax = -INFINITY;
    if (__ballot(lim < kTileTok - 1) == 0) {
        // no lane's query lies inside the tile: only the block bits mask
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mm = 8 * (r >> 2) + 4 * ln.hgrp + (r & 3);
            st.s[r] = (tb >> (mm >> LOG2B)) & 1u ? st.s[r] : -INFINITY;
            tmax = fmaxf(tmax, st.s[r]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mm = 8 * (r >> 2) + 4 * ln.hgrp + (r & 3);
            const bool valid = ((tb >> (mm >> LOG2B)) & 1u) && mm <= lim;
            st.s[r] = valid ? st.s[r] : -INFINITY;
            tmax = fmaxf(tmax, st.s[r]);
        }
    }
    tmax = xor32_max(tmax);
    const float sl2 = ln.sl2;
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
    float psum = 0.f;
#pragma unroll
    for (int sgi = 0; sgi < 2; ++sgi) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(st.s[8 * sgi + e] * sl2 - msub);
            psum += p[e];
        }
        uint4 pk;
        pk.x = pack_bf16(p[0], p[1]);
        pk.y = pack_bf16(p[2], p[3]);
        pk.z = pack_bf16(p[4], p[5]);
        pk.w = pack_bf16(p[6], p[7]);
        st.pb[sgi] = as_bf16x8(pk);
    }
    psum = xor32_sum(psum);
    st.lsum += psum;
}

// ---------------------------------------------------------------------------
// Tiled kernel for dense-ish selections (selected share of the candidates
// >= 1/4, e.g. every query of an 8K prefill at k = 512 blocks).
//
// One workgroup = 16 consecutive queries x one group on 8 wavefronts;
// wavefront w owns two queries x 16 heads = 32 columns.  The workgroup walks
// the causal range in contiguous 32-token tiles; K and V rows go through LDS
// once and serve 256 (query, head) columns.  A per-query bitmap of the
// selected blocks (plus the current block, positions <= t) masks the
// scores, so every query still attends over exactly its own token set.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows (ds_read_b128 from a
//                 row-major tile padded to 100 dwords per row),
//                 B = Q^T (registers)
//   O^T = V^T P^T v_mfma_f32_32x32x16_bf16, A = V^T rows (ds_read_b128)
//                 from a dim-major V tile written with its tokens in the
//                 order of the S^T result layout, B = P^T: the
//                 exponentiated S^T registers, so P never leaves registers.
//                 (Transposing on the way into LDS costs eight byte
//                 permutes per thread per tile; transposed LDS reads run at
//                 about a third of the b128 rate.)
// Each lane holds one (query, head) column, so the running max / sum are
// per lane; the max is rescaled lazily (only when it grows by more than
// 2^8), which keeps O exact because O and the sum share the reference max.
// K/V tiles circulate through a ring of three LDS buffers with one barrier
// per tile: tile i+2 is fetched with buffer loads at the top of step i (a
// per-tile buffer resource ends at row t_last, so rows past the last query
// read as zeros) and stored at its end.  The output is staged through LDS so
// each query's 16 heads leave as one contiguous 6 KB row block.
// ---------------------------------------------------------------------------
template <int LOG2B, bool PAGED>
__global__ __launch_bounds__(512) void attn_union_kernel(SeqTable seqs, AttnArgs a, int words) {
    constexpr int NW = 8, TQ = 16, NT = 512;
    extern __shared__ uint32_t bitmap[];                         // [TQ][words]
    __shared__ __attribute__((aligned(16))) uint16_t kv_lds[3 * kBufElems];
    __shared__ int s_nsel[TQ];
    static_assert(3 * kBufElems >= NW * 16 * kOutStride, "output staging fits the tile buffers");

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
    const int64_t row0 = PAGED ? 0 : sq.kv_offset;
    u.kb = a.k + (row0 * kGroups + g) * kHeadDim;
    u.vb = a.v + (row0 * kGroups + g) * kHeadDim;
    u.pt = PAGED ? a.page_table + sq.kv_offset : nullptr;
    u.n_pages = a.n_pages;
    u.t_last = t_last;
    union_ctx_init(u, tid);
    const int n_tiles = (int)(t_last / kTileTok) + 1;
    KVStage rs;
    gload<PAGED>(u, 0, rs);

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
    UnionState st;
#pragma unroll
    for (int dt = 0; dt < 6; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.s[r] = 0.f;
    st.pb[0] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
    st.pb[1] = st.pb[0];
    st.m_use = -INFINITY;
    st.lsum = 0.f;
    UnionLane ln;
    ln.mybits = mybits;
    ln.tq = tq;
    ln.q_ok = q_ok;
    ln.lane = lane;
    ln.hgrp = hgrp;
    ln.col = col;
    ln.sl2 = a.scale_log2;
    const float sl2 = a.scale_log2;

    // ---- tile loop: the scores of tile i+1 are issued in the same straight
    //      line as the softmax of tile i and the O update with it; tile i+2
    //      is loaded at the top and stored into the third buffer at the end
    //      (past the end the last tile is fetched again into a buffer no
    //      longer read, which keeps loads and stores unconditional) ----
    lstore(kv_lds, u, rs);
    gload<PAGED>(u, n_tiles > 1 ? 1 : 0, rs);
    lstore(kv_lds + kBufElems, u, rs);
    __syncthreads();
    st.s = tile_scores(kv_lds, qf, lane);
    int b_cur = 0;
    for (int i = 0; i < n_tiles; ++i) {
        const int b_nxt = b_cur == 2 ? 0 : b_cur + 1;
        const int b_new = b_nxt == 2 ? 0 : b_nxt + 1;
        gload<PAGED>(u, i + 2 < n_tiles ? i + 2 : n_tiles - 1, rs);
        union_vector<LOG2B>(st, i, n_tiles, ln);
        union_matrix(st, qf, kv_lds + b_nxt * kBufElems, kv_lds + b_cur * kBufElems, ln);
        lstore(kv_lds + b_new * kBufElems, u, rs);
        __syncthreads();
        b_cur = b_nxt;
    }
    f32x16 (&o)[6] = st.o;
    const float m_use = st.m_use, lsum = st.lsum;

    // ---- epilogue: O^T[d][col] for d = 32dt + 8j + 4hgrp + i, normalised,
    //      staged per query in LDS, then written as contiguous 6 KB rows ----
    const float inv = 1.0f / lsum;
    if (hgrp == 0 && q_ok && a.lse)
        a.lse[qrow * kHeads + g * kHeadsPerGroup + head] = (m_use * sl2 + log2f(lsum)) * kLn2;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
        if ((col >> 4) == phase) {
            uint16_t* orow = kv_lds + (wave * 16 + head) * kOutStride;
            // output gate (sigmoid of the logits), applied before rounding
            const uint16_t* grow =
                a.gate && q_ok ? a.gate + (qrow * kHeads + g * kHeadsPerGroup + head) * kHeadDim : nullptr;
#pragma unroll
            for (int dt = 0; dt < 6; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = o[dt][4 * j + i] * inv;
                    if (grow) {
                        const uint2 gw = *(const uint2*)(grow + 32 * dt + 8 * j + 4 * hgrp);
                        v[0] *= gate_sigmoid((uint16_t)(gw.x & 0xFFFFu));
                        v[1] *= gate_sigmoid((uint16_t)(gw.x >> 16));
                        v[2] *= gate_sigmoid((uint16_t)(gw.y & 0xFFFFu));
                        v[3] *= gate_sigmoid((uint16_t)(gw.y >> 16));
                    }
                    uint2 pk;
                    pk.x = pack_bf16(v[0], v[1]);
                    pk.y = pack_bf16(v[2], v[3]);
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

}  // namespace

template <int LOG2B, bool PAGED>
static hipError_t launch_union_t(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                                 int words, hipStream_t stream) {
    const size_t lds = (size_t)16 * words * sizeof(uint32_t);
    hipError_t e = set_dynamic_lds((const void*)attn_union_kernel<LOG2B, PAGED>, lds);
    if (e != hipSuccess) return e;
    const int64_t n_qt = (max_nq + 15) / 16;
    dim3 grid((unsigned)(n_qt * kGroups), (unsigned)seqs.n);
    hipLaunchKernelGGL((attn_union_kernel<LOG2B, PAGED>), grid, dim3(512), lds, stream, seqs, a, words);
    return hipGetLastError();
}

template <bool PAGED>
static hipError_t launch_union_b(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a, int words,
                                 hipStream_t stream) {
    switch (a.block_size) {
        case 1: return launch_union_t<0, PAGED>(seqs, max_nq, a, words, stream);
        case 2: return launch_union_t<1, PAGED>(seqs, max_nq, a, words, stream);
        case 4: return launch_union_t<2, PAGED>(seqs, max_nq, a, words, stream);
        case 8: return launch_union_t<3, PAGED>(seqs, max_nq, a, words, stream);
        case 16: return launch_union_t<4, PAGED>(seqs, max_nq, a, words, stream);
        default: return hipErrorInvalidValue;
    }
}

int union_queries_per_block() { return 16; }

hipError_t launch_attn_union(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                             int words, hipStream_t stream) {
    if (max_nq <= 0 || seqs.n <= 0) return hipSuccess;
    return a.page_table ? launch_union_b<true>(seqs, max_nq, a, words, stream)
                        : launch_union_b<false>(seqs, max_nq, a, words, stream);
}

}  // namespace sgqa
