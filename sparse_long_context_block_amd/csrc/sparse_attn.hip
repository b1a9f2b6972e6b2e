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
// chunks w, w+4, ...  A chunk's 16 K rows and 16 V rows (384 bytes each for
// the group) are fetched with coalesced loads -- each group of four lanes
// reads 64 contiguous bytes of one row, so a 1 KB load instruction touches
// about eight cache lines instead of sixteen half lines, one per lane
// (reading the rows straight into MFMA operand order made every lane a
// separate cache access and the address unit the bottleneck) -- and written
// to the wavefront's padded LDS tiles.  Per chunk the wavefront
//   * reads K back as the A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16;
//     the group's 16 heads are the N dimension, so every gathered K/V byte
//     serves all 16 heads);
//   * runs the online softmax on the result layout, where each lane holds 4
//     tokens of one head, with a lazily raised reference max: the
//     exponentiated tile is directly the B operand (P^T) of O^T = V^T P^T
//     (v_mfma_f32_16x16x16bf16_1k), no LDS round trip;
//   * reads V^T from the V tile with transposed reads.
// Two register sets hold the rows of the next two chunks in flight while a
// chunk is processed from LDS.  The four wavefronts' (max, sum, O) are merged
// in LDS; a split call (decode: few queries) writes partials that
// attn_merge_kernel combines.  Workgroups run group-major.
#include <type_traits>

#include "attn_common.hpp"

namespace sgqa {
namespace {

using namespace dev;
using namespace attn;

// Padded tile rows.  K tile: 100 dwords per row, so the b128 operand reads
// of eight (and of sixteen) consecutive lanes -- rows m, m+1, ... -- start
// in distinct bank groups.  V tile: 104 dwords per row, so the 8-byte
// transposed reads of the 16 lanes of a lane group (4 rows x 4 column
// quads) cover 32 distinct banks.
constexpr int kTileRow = kHeadDim + 8;                 // K: bf16 per row (100 dwords)
constexpr int kTileRowV = kHeadDim + 16;               // V: bf16 per row (104 dwords)
constexpr int kTileBytes = 16 * kTileRow * 2;          // K tile: 6,400 B
constexpr int kTileBytesV = 16 * kTileRowV * 2;        // V tile: 6,656 B
constexpr int kWaveLds = kTileBytes + kTileBytesV;     // a wavefront's K and V tiles
constexpr int kWaveBufFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;
static_assert(kWaveBufFloats * 4 <= kWaveLds, "a wavefront's merge buffer fits its tiles");
// wavefronts per gather workgroup: every per-wavefront array, the chunk
// stride and the merge below are sized by this one constant
constexpr int kGatherWaves = 4;
constexpr int kGatherThreads = 64 * kGatherWaves;
constexpr uint32_t kRowBytes = kGroups * kHeadDim * 2;  // bytes between a tensor's token rows

// Token list of a (query, group): entry i < n_sel*B is token i%B of block
// sel[i/B] (contiguous caches: sel holds block ids; paged: the pool row of
// the block's first position), later entries are the current block's tokens
// up to t.  Entries past the list, or chunks at or past c_hi, read row t_row
// (finite values, masked).  Rows are clamped to [0, row_max], so malformed
// ids never read outside the cache or the pool.
struct ChunkMap {
    const int32_t* sel_lds;
    int n_sel, shift_b, n_tok, c_hi;
    int64_t cur0, t_row, row_max;
};

// Cache row (contiguous: relative to the sequence's first row; paged: pool
// row) of token 16c + tau of the list.  Branch-free: the selection entry is
// read for every lane (index 0 when the token is not a historical one).
__device__ __forceinline__ uint32_t token_row(int c, int tau, bool paged, const ChunkMap& cm) {
    const int ti = 16 * c + tau;
    const bool listed = (c < cm.c_hi) & (ti < cm.n_tok);
    const int j = ti >> cm.shift_b;
    const bool hist = j < cm.n_sel;
    const int64_t e = cm.sel_lds[hist ? j : 0];
    const int64_t within = ti & ((1 << cm.shift_b) - 1);
    const int64_t tok_h = (paged ? e : e << cm.shift_b) + within;
    const int64_t tok_c = cm.cur0 + (ti - (cm.n_sel << cm.shift_b));
    int64_t tok = listed ? (hist ? tok_h : tok_c) : cm.t_row;
    tok = tok < 0 ? 0 : (tok > cm.row_max ? cm.row_max : tok);
    return (uint32_t)tok;
}

// Coalesced piece map.  A tensor's chunk is 16 rows x 24 pieces of 16 bytes;
// load instruction i (< 6) of lane L fetches piece x = 64 i + L: row
// tau = x / 24, piece p = x % 24, so consecutive lanes read consecutive
// 16-byte pieces of a row.  Packed per i: the piece's LDS byte offset in the
// K tile (tau * 400 + 16 p, bits 0..12; the V tile adds 16 tau), its byte
// offset in the row (16 p, bits 13..21) and tau (bits 22..25).
__device__ __forceinline__ uint32_t piece_code(int i, int lane) {
    const int x = 64 * i + lane;
    const int tau = x / 24, p = x - 24 * (x / 24);
    return (uint32_t)(tau * kTileRow * 2 + 16 * p) | ((uint32_t)(16 * p) << 13) | ((uint32_t)tau << 22);
}

// Byte offset from the K (or V) base of this lane's piece i of chunk c:
// 32-bit for contiguous caches (the host keeps a sequence's capacity below
// 2^32 / 1536 rows), 64-bit into a page pool.
template <bool PAGED>
using RowOff = typename std::conditional<PAGED, uint64_t, uint32_t>::type;

// The rows of chunk c into registers (k[i], v[i]: piece i of the K and V
// rows): lanes 0..15 find the chunk's 16 rows, every lane takes the rows of
// its six pieces from them (ds_bpermute).
// Native vectors (not the HIP uint4 struct, whose copies become memcpys that
// keep the staging arrays in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool PAGED>
__device__ __forceinline__ void load_chunk(int c, int lane, const uint32_t (&pc)[6], const ChunkMap& cm,
                                           const char* kbase, const char* vbase, u32x4 (&k)[6], u32x4 (&v)[6]) {
    const uint32_t row = token_row(c, lane & 15, PAGED, cm);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const uint32_t tau = pc[i] >> 22;
        const uint32_t rw = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(tau << 2), (int)row);
        const RowOff<PAGED> off = (RowOff<PAGED>)rw * kRowBytes + ((pc[i] >> 13) & 0x1FFu);
        k[i] = *(const u32x4*)(kbase + off);
        v[i] = *(const u32x4*)(vbase + off);
    }
}

// The staged rows into the wavefront's tiles (row tau at tau * 400 bytes of
// the K tile, tau * 416 bytes of the V tile).
__device__ __forceinline__ void store_chunk(const u32x4 (&k)[6], const u32x4 (&v)[6], const uint32_t (&pc)[6],
                                            char* ktile, char* vtile) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const uint32_t o = pc[i] & 0x1FFFu;
        *(u32x4*)(ktile + o) = k[i];
        *(u32x4*)(vtile + o + ((pc[i] >> 22) << 4)) = v[i];
    }
}

struct GatherState {
    f32x4 o[12];       // O^T: dims 16nt + 4qq + i of head m
    float m_use;       // reference max of head m (raw score units), raised lazily
    float lsum;        // this lane's tokens' sum relative to it
};

struct GatherLane {
    const char* ktile;   // this wavefront's K tile in LDS
    const char* vtile;   // and its V tile
    int k_off;           // this lane's A-operand offset in the K tile (bytes)
    int tr_off;          // its transposed-read offset in the V tile (bytes)
    int qq;
    int n_tok;
    float sl2;
};

// One 16-token chunk from the tiles.  S^T A operand: lane (m, qq) reads row
// m, dims 32kk + 8qq .. +7 (100-dword rows: the b128 reads of eight lanes
// fall in distinct banks).  O^T A operand with ds_read_b64_tr_b16: lane
// 16G + 4i + c supplies row 4G + i, dims 4c..4c+3 of a 16-dim block, and lane
// 16G + j receives dim j of tokens 4G..4G+3 -- row j, k = 4G + i of
// v_mfma_f32_16x16x16bf16_1k.  The softmax runs on the S^T result layout
// (lane: tokens 16c + 4qq + i of head m) with a lazily raised reference max;
// the exponentiated tile is the B operand.
__device__ __forceinline__ void gather_step(GatherState& st, const bf16x8 (&qf)[6], int c, const GatherLane& gl) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 6; ++kk)
        s = mfma_16x16x32(*(const bf16x8*)(gl.ktile + gl.k_off + 64 * kk), qf[kk], s);
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
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
        const i16x4 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(gl.vtile + gl.tr_off + 32 * nt));
        st.o[nt] = mfma_16x16x16(av, pbv, st.o[nt]);
    }
}

template <bool PAGED>
__global__ __launch_bounds__(kGatherThreads, 2) void sparse_attn_kernel(SeqTable seqs, AttnArgs a) {
    extern __shared__ int32_t sel_lds[];                        // [K]
    __shared__ __align__(16) char tiles[kGatherWaves][kWaveLds];
    __shared__ int s_nsel;

    // Group-major order: the workgroups in flight read one group's K/V
    // (disjoint cache lines per group), a quarter of the cache's footprint,
    // which keeps the re-read rows in the last-level cache.  Within a group,
    // workgroups are dealt to the 8 XCDs round-robin by id; each XCD takes a
    // contiguous run of queries (and, for range splits, the same range for
    // all of them), so queries that run together on one XCD are neighbours
    // and share whatever blocks their selections have in common through
    // that XCD's L2.  (Any bijection is correct; this one needs the group's
    // workgroup count to be a multiple of 8 and n_split to divide 8.)
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t per_group = (int64_t)(gridDim.x / kGroups);
    const int g = (int)(blockIdx.x / per_group);
    const int64_t loc = blockIdx.x - g * per_group;
    int split;
    int64_t qi;
    if (per_group % 8 == 0 && 8 % a.n_split == 0) {
        const int xcd = (int)(loc % 8);
        split = xcd % a.n_split;
        qi = (int64_t)(xcd / a.n_split) * (per_group / 8) + loc / 8;
    } else {
        split = (int)(loc % a.n_split);
        qi = loc / a.n_split;
    }
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
    for (int j = threadIdx.x; j < a.topk; j += kGatherThreads) {
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
        for (int j = threadIdx.x; j < n_sel; j += kGatherThreads) {
            const int64_t r = sel_lds[j] > b_max ? b_max : sel_lds[j];
            sel_lds[j] = (int32_t)paged_row(pt, a.n_pages, r * B);
        }
        cur0 = paged_row(pt, a.n_pages, cur_first);
        t_row = cur0 + (t - cur_first);
        row_max = a.n_pages * kPageTokens - 1;
        __syncthreads();
    }
    const int n_tok = (n_sel << shift_b) + (int)(t - cur_first + 1);
    const int n_chunks = (n_tok + 15) >> 4;
    const int c_lo = split * a.chunks_per_split;
    const int c_hi = n_chunks < c_lo + a.chunks_per_split ? n_chunks : c_lo + a.chunks_per_split;

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
    char* ktile = tiles[w];
    char* vtile = tiles[w] + kTileBytes;
    GatherLane gl;
    gl.ktile = ktile;
    gl.vtile = vtile;
    gl.k_off = m * kTileRow * 2 + 16 * qq;
    gl.tr_off = ((4 * qq + ((lane >> 2) & 3)) * kTileRowV + 4 * (lane & 3)) * 2;
    gl.qq = qq;
    // tokens past this split's chunks are masked (a pair's second chunk may
    // lie past c_hi; its rows are row t_row's)
    gl.n_tok = n_tok < 16 * c_hi ? n_tok : 16 * c_hi;
    gl.sl2 = a.scale_log2;
    // contiguous caches: rows relative to the sequence's first row
    const int64_t row0 = PAGED ? 0 : sq.kv_offset;
    const char* kbase = (const char*)(a.k + (row0 * kGroups + g) * kHeadDim);
    const char* vbase = (const char*)(a.v + (row0 * kGroups + g) * kHeadDim);
    ChunkMap cm;
    cm.sel_lds = sel_lds;
    cm.n_sel = n_sel;
    cm.shift_b = shift_b;
    cm.n_tok = n_tok;
    cm.c_hi = c_hi;
    cm.cur0 = cur0;
    cm.t_row = t_row;
    cm.row_max = row_max;
    uint32_t pc[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) pc[i] = piece_code(i, lane);

    // Chunks w, w + W, ... (W = kGatherWaves) in pairs.  Two register sets:
    // a set's rows go to the tiles just before their chunk is processed, and
    // the set is refilled at once with the chunk 2W ahead, so the next two
    // chunks' rows are in flight while a chunk is processed.  A pair's second chunk
    // may lie past c_hi (fully masked: it adds nothing); loads of chunks past
    // the wavefront's last read row t_row (the same lines for every lane).
    // The loop has a single exit at its end, which keeps the compiler's wait
    // counts exact: each store waits only for its own set's rows.
    int c = c_lo + w;
    if (c < c_hi) {
        u32x4 ak[6], av[6], bk[6], bv[6];
        load_chunk<PAGED>(c, lane, pc, cm, kbase, vbase, ak, av);
        load_chunk<PAGED>(c + kGatherWaves, lane, pc, cm, kbase, vbase, bk, bv);
        do {
            store_chunk(ak, av, pc, ktile, vtile);
            wave_lds_sync();
            load_chunk<PAGED>(c + 2 * kGatherWaves, lane, pc, cm, kbase, vbase, ak, av);
            gather_step(st, qf, c, gl);
            wave_lds_sync();
            store_chunk(bk, bv, pc, ktile, vtile);
            wave_lds_sync();
            load_chunk<PAGED>(c + 3 * kGatherWaves, lane, pc, cm, kbase, vbase, bk, bv);
            gather_step(st, qf, c + kGatherWaves, gl);
            wave_lds_sync();
            c += 2 * kGatherWaves;
        } while (c < c_hi);
    }
    float lsum = st.lsum;
    f32x4 (&o)[12] = st.o;
    const float m_use = st.m_use;
    const float sl2 = a.scale_log2;
    // the head's sum over its four token lanes; the merge takes the max in
    // log2 units
    lsum = xor32_sum(xor16_sum(lsum));
    const float mrow = m_use * sl2;

    // ---- merge the wavefronts ----
    __syncthreads();
    float* buf = (float*)tiles[w];
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
    for (int e = threadIdx.x; e < kHeadsPerGroup * kHeadDim; e += kGatherThreads) {
        const int head = e / kHeadDim;
        float mw[kGatherWaves], M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kGatherWaves; ++ww) {
            mw[ww] = ((const float*)tiles[ww])[kHeadsPerGroup * kHeadDim + head];
            M = fmaxf(M, mw[ww]);
        }
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < kGatherWaves; ++ww) {
                const float sc = exp2f(mw[ww] - M);
                L += ((const float*)tiles[ww])[kHeadsPerGroup * kHeadDim + kHeadsPerGroup + head] * sc;
                O += ((const float*)tiles[ww])[e] * sc;
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
    hipLaunchKernelGGL((sparse_attn_kernel<PAGED>), grid, dim3(kGatherThreads), lds, stream, seqs, a);
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
