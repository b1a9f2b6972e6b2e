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
#include "sgqa_internal.hpp"

namespace sgqa {
namespace {

using namespace dev;

constexpr int kGVStride = kHeadDim + 8;             // bf16 per row of a wave's V tile (100 dwords)
constexpr int kWaveBufFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;
static_assert(16 * kGVStride * 2 <= kWaveBufFloats * 4, "a wave's V tile fits its merge buffer");
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;          // log2 units

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Reductions across lanes through v_permlane16_swap / v_permlane32_swap
// (VALU ops: no LDS round trip as with ds_bpermute): xor16 combines lanes
// l and l ^ 16, xor32 lanes l and l ^ 32.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int64_t token_at(int64_t i, int n_sel, int shift_b, int B,
                                            const int32_t* sel, int64_t cur_first) {
    const int64_t j = i >> shift_b;
    if (j < n_sel) return (int64_t)sel[j] * B + (i & (B - 1));
    return cur_first + (i - ((int64_t)n_sel << shift_b));
}

// K/V rows of chunk c for this lane (token 16c + m; K dims 32kk + 8qq, V
// dims 8(qq + 4j)); chunks past the token list read the current token, whose
// values stay finite and are masked
struct GatherRegs {
    uint4 k[6], v[6];
};

__device__ __forceinline__ GatherRegs gather_chunk(int64_t c, int m, int qq, int64_t n_tok, int n_sel, int shift_b,
                                                   int B, const int32_t* sel_lds, int64_t cur_first, int64_t t,
                                                   const uint16_t* kbase, const uint16_t* vbase) {
    constexpr int64_t kRowStride = (int64_t)kGroups * kHeadDim;
    const int64_t ti = 16 * c + m;
    int64_t tok = ti < n_tok ? token_at(ti, n_sel, shift_b, B, sel_lds, cur_first) : t;
    tok = tok < 0 ? 0 : (tok > t ? t : tok);   // malformed ids never read past the cache
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
    const uint16_t* kbase = a.k + (sq.kv_offset * kGroups + g) * kHeadDim;
    const uint16_t* vbase = a.v + (sq.kv_offset * kGroups + g) * kHeadDim;

    // two register sets alternate: one chunk's rows are in flight while the
    // other chunk is processed
    if (c_lo + w < c_hi) {
        GatherRegs ra = gather_chunk(c_lo + w, m, qq, n_tok, n_sel, shift_b, B, sel_lds, cur_first, t, kbase, vbase);
        for (int64_t c = c_lo + w; c < c_hi; c += 8) {
            const GatherRegs rb =
                gather_chunk(c + 4, m, qq, n_tok, n_sel, shift_b, B, sel_lds, cur_first, t, kbase, vbase);
            gather_step(st, ra, qf, c, gl);
            if (c + 4 >= c_hi) break;
            ra = gather_chunk(c + 8, m, qq, n_tok, n_sel, shift_b, B, sel_lds, cur_first, t, kbase, vbase);
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
    const uint16_t* kb;
    const uint16_t* vb;
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

__device__ __forceinline__ void gload(const UnionCtx& u, int tile, KVStage& r) {
    const int64_t tile0 = (int64_t)tile * kTileTok;
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
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int mm = 8 * (r >> 2) + 4 * ln.hgrp + (r & 3);
        const bool valid = ((tb >> (mm >> LOG2B)) & 1u) && mm <= lim;
        st.s[r] = valid ? st.s[r] : -INFINITY;
        tmax = fmaxf(tmax, st.s[r]);
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
template <int LOG2B>
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
    u.kb = a.k + (sq.kv_offset * kGroups + g) * kHeadDim;
    u.vb = a.v + (sq.kv_offset * kGroups + g) * kHeadDim;
    u.t_last = t_last;
    union_ctx_init(u, tid);
    const int n_tiles = (int)(t_last / kTileTok) + 1;
    KVStage rs;
    gload(u, 0, rs);

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
    gload(u, n_tiles > 1 ? 1 : 0, rs);
    lstore(kv_lds + kBufElems, u, rs);
    __syncthreads();
    st.s = tile_scores(kv_lds, qf, lane);
    int b_cur = 0;
    for (int i = 0; i < n_tiles; ++i) {
        const int b_nxt = b_cur == 2 ? 0 : b_cur + 1;
        const int b_new = b_nxt == 2 ? 0 : b_nxt + 1;
        gload(u, i + 2 < n_tiles ? i + 2 : n_tiles - 1, rs);
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
#pragma unroll
            for (int dt = 0; dt < 6; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint2 pk;
                    pk.x = pack_bf16(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv);
                    pk.y = pack_bf16(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
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
