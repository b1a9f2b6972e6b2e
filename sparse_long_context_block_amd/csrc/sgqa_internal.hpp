// Internal declarations shared by the HIP kernels and the host dispatch of
// libsgqa.so.  Nothing here is part of the public ABI (include/sgqa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sgqa {

// ---------------------------------------------------------------------------
// compiled shape set
// ---------------------------------------------------------------------------
constexpr int kHeads = 64;        // query heads
constexpr int kGroups = 4;        // KV groups (16 heads each)
constexpr int kHeadsPerGroup = 16;
constexpr int kHeadDim = 192;     // main Q/K/V head dim
constexpr int kIdxHeads = 4;      // indexer heads per group
constexpr int kIdxDim = 128;      // indexer dim
constexpr int kRopeDim = 32;      // indexer rotary span
constexpr int kMaxTopK = 3072;
constexpr int kMaxSeqsPerLaunch = 64;
// diagnostics block of a tiled index call (uint32 words): [0] rows whose
// candidate lists failed and were scored again in full, [1] reserved, then
// (query row, group) of the first kDiagRows of them
constexpr int kDiagWords = 64;
constexpr int kDiagRows = (kDiagWords - 2) / 2;

// Raise a kernel's dynamic-LDS limit to at least `bytes` on the current
// device; the limit already set per (device, kernel) is remembered, so the
// runtime is called only when a launch needs more than before.
hipError_t set_dynamic_lds(const void* kernel, size_t bytes);
constexpr int kMaxAttnSplits = 64;

// Per-sequence descriptor as the kernels see it (passed by value in the
// kernel arguments, up to kMaxSeqsPerLaunch per launch).
struct DevSeq {
    int64_t q_offset;
    int64_t n_q;
    int64_t pos0;
    int64_t kv_offset;
    int64_t store_offset;
    int64_t ws_row;      // first workspace row of this entry's queries: the
                         // host numbers the queries of one launch table
                         // 0, 1, ... in table order (split index keys and
                         // split attention partials are addressed by it)
};

struct SeqTable {
    int32_t n;
    int32_t pad_;
    DevSeq s[kMaxSeqsPerLaunch];
};

// ---------------------------------------------------------------------------
// launch parameter blocks (host-chosen, passed by value)
// ---------------------------------------------------------------------------
// Paged caches (per-token tensors in pages of 16 positions): position pos of
// a sequence lives in row page_table[kv_offset + pos / 16] * 16 + pos % 16 of
// the page pool; the kv_offset of a sequence is the index of its first page
// table entry.  page_table == nullptr: contiguous, row kv_offset + pos.
constexpr int kPageTokens = 16;

struct CompressArgs {
    const uint16_t* proxy_k;
    const float* logits;
    const int32_t* page_table;  // paged proxy keys / logits, or null
    int64_t n_pages;
    const uint16_t* ln_gamma;  // may be null
    const uint16_t* ln_beta;   // may be null
    uint16_t* store;
    int32_t block_size;
    int32_t store_q8;
    float eps;
    double theta[kRopeDim / 2]; // rotary frequencies base^(-2j/32)
};

struct IndexArgs {
    const uint16_t* q_idx;
    const float* w;
    const uint16_t* rms_gamma;  // may be null
    const uint16_t* store;      // bf16 rows, or E4M3 codes when store_fp8 (128 B rows)
    int32_t* sel;
    float* sel_scores;          // may be null
    uint16_t* q_hat_out;        // may be null
    uint32_t* part_key;         // split calls: score keys [launch rows, G, key_stride],
                                // row = DevSeq::ws_row + query index
    uint4* q_frag;              // tiled calls: indexer A fragments [launch rows, 4, 64]
    uint32_t* ctl;              // tiled calls: [0] rows whose list failed, [1..] those rows
    uint32_t* diag;             // tiled calls: the call's diagnostics block (kDiagWords),
                                // or null
    int32_t diag_clear;         // this launch is the call's first: clear diag first
    int64_t key_stride;
    int32_t listed;             // tiled calls: long rows may select from candidate lists
    int32_t list_off;           // listed rows: u32 offsets inside a key row of the
    int32_t samp_off;           //   candidate lists, the sample keys and the threshold
    int32_t tau_off;            //   (segment counts at offset 0)
    int32_t block_size;
    int32_t topk;               // K
    int32_t cap;                // per-row LDS buffer capacity C (fused kernel)
    int32_t n_split;
    int32_t split_blocks;       // candidate blocks per split (multiple of 16)
    int32_t list_cap;           // listed rows: entries of the LDS pool (list_capacity)
    int32_t store_fp8;          // store rows hold E4M3 codes
    float eps;
    double theta[kRopeDim / 2]; // rotary frequencies base^(-2j/32)
};

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;          // cache, or page pool [n_pages, 16, G, D]
    const uint16_t* v;
    const int32_t* page_table;  // paged K/V, or null
    int64_t n_pages;
    const uint16_t* gate;       // bf16 [Nq, H, D] output-gate logits, or null
    const int32_t* sel;
    uint16_t* out;
    float* lse;            // may be null
    float* part_o;         // split mode: [launch rows, G, n_split, 16, 192]
    float* part_ml;        // split mode: [launch rows, G, n_split, 16, 2]
    int32_t block_size;
    int32_t topk;
    int32_t n_split;
    int32_t chunks_per_split;  // 16-token chunks per split
    float scale_log2;          // softmax_scale * log2(e)
};

struct AttnMergeArgs {
    const float* part_o;
    const float* part_ml;
    const uint16_t* gate;       // as AttnArgs::gate
    uint16_t* out;
    float* lse;
    int32_t n_split;
};

// ---------------------------------------------------------------------------
// candidate lists of long rows (tiled calls)
//
// A 16-query tile whose first query has n0 candidate blocks is "listed" when
// n0 is large: its queries' selections then come from candidate lists
// instead of every score key.  A sample of S scores per (query, group) gives
// a threshold tau, the j-th largest sample score, j = ceil(m k S / n0) with
// m = 1 + 5 / sqrt(k S / n0), so that about m k scores are expected at or
// above tau and fewer than k only five standard deviations out.  The score
// step keeps the scores >= tau, with their block ids, in lists of at most
// kSegCap entries per segment of kSegBlocks blocks (m k kSegBlocks / n0 <= 21
// expected per segment).  A row whose lists overflow, or hold fewer than k
// entries, or more than the select can stage, is scored again in full and
// selected from its keys, so the result is always the exact top k.
// ---------------------------------------------------------------------------
constexpr int kSegBlocks = 256;
constexpr int kSegCap = 64;
constexpr int64_t kListMinBlocks = 32768;
constexpr int64_t kListMaxBlocks = (int64_t)1 << 21;
constexpr int kListSampleMax = 2048;

__host__ __device__ inline int list_sample(int64_t n0) {
    const int64_t s = n0 / 4 < kListSampleMax ? n0 / 4 : kListSampleMax;
    return (int)(s / 16 * 16);
}
__host__ __device__ inline double list_margin(int64_t n0, int k) {
    return 1.0 + 5.0 / sqrt((double)k * list_sample(n0) / (double)n0);
}
__host__ __device__ inline bool list_tile(int64_t n0, int k) {
    return n0 >= kListMinBlocks && n0 <= kListMaxBlocks &&
           list_margin(n0, k) * k * kSegBlocks <= 21.0 * (double)n0;
}
__host__ __device__ inline int list_rank(int64_t n0, int k) {
    const int S = list_sample(n0);
    const double j = ceil(list_margin(n0, k) * k * S / (double)n0);
    return j < 1.0 ? 1 : (j > S ? S : (int)j);
}
// entries of the LDS pool (8 B each) of listed rows whose tiles start at
// most n0 candidates in: the expected list length (j/S of the row, about
// m k entries) plus five times its spread (the share of a row above the
// sample's j-th largest key has relative spread 1/sqrt(j)), at least k +
// 1024, at most 16384.  A row with more entries takes the list select's
// other paths.
__host__ __device__ inline int list_capacity(int64_t n0, int k) {
    const int j = list_rank(n0, k);
    const double e = (double)j * (double)n0 / (double)list_sample(n0);
    int c = (int)((e * (1.0 + 5.0 / sqrt((double)j)) + 1023.0) / 1024.0) * 1024;
    const int lo = (k + 1024 + 1023) / 1024 * 1024;
    c = c < lo ? lo : c;
    return c > 16384 ? 16384 : c;
}

// Main-path Q/K producer: RMSNorm over each head's D dims (one gamma per
// tensor, shared by the heads), the rotary span [0, rope_dim) at the token's
// position, bf16; V rows copied.  Q rows go to q_out, K/V rows into the
// caches (contiguous, or paged as in CompressArgs).
struct QkPrepArgs {
    const uint16_t* q_raw;      // [Nq, H, D]
    const uint16_t* k_raw;      // [Nq, G, D]
    const uint16_t* v_raw;      // [Nq, G, D] or null
    const uint16_t* q_gamma;    // [D] or null
    const uint16_t* k_gamma;    // [D] or null
    uint16_t* q_out;
    uint16_t* k_cache;
    uint16_t* v_cache;
    const int32_t* page_table;
    int64_t n_pages;
    double log_base;            // ln(rope base)
    int32_t rope_dim;
    float eps;
};

// a launch table travels in the kernel arguments, which hold at most 4 KiB
static_assert(sizeof(SeqTable) + sizeof(IndexArgs) <= 4096, "index kernel arguments fit");
static_assert(sizeof(SeqTable) + sizeof(AttnArgs) + 8 <= 4096, "attention kernel arguments fit");
static_assert(sizeof(SeqTable) + sizeof(CompressArgs) <= 4096, "compress kernel arguments fit");
static_assert(sizeof(SeqTable) + sizeof(IndexArgs) + sizeof(CompressArgs) <= 4096,
              "scoring-with-merge kernel arguments fit");

// ---------------------------------------------------------------------------
// launchers (defined next to their kernels); return hipError_t of the launch
// ---------------------------------------------------------------------------
hipError_t launch_compress(const SeqTable& seqs, int64_t max_blocks, const CompressArgs& a,
                           hipStream_t stream);
hipError_t launch_qk_prep(const SeqTable& seqs, int64_t max_nq, const QkPrepArgs& a, hipStream_t stream);
size_t index_lds_bytes(int cap);
constexpr size_t kMaxLds = 160 * 1024;
hipError_t launch_index_topk(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                             hipStream_t stream);
// decode-sized calls: score wavefronts over candidate splits, then one
// select workgroup per (query, group).  merge: step 1 carried in the
// scoring launch (calls whose queries read none of the blocks they
// complete), or null
hipError_t launch_index_split(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                              hipStream_t stream, const CompressArgs* merge = nullptr);
// prefill-sized calls: 16-query workgroups score candidate ranges of
// a.split_blocks blocks against store tiles shared through LDS, then one
// select workgroup per (query, group)
constexpr int kScoreTileQueries = 16;
hipError_t launch_index_tiled(const SeqTable& seqs, int64_t max_nq, const IndexArgs& a,
                              hipStream_t stream);
hipError_t launch_sparse_attn(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a,
                              hipStream_t stream);
hipError_t launch_attn_merge(const SeqTable& seqs, int64_t max_nq, const AttnMergeArgs& a,
                             hipStream_t stream);
// tiled kernel for dense-ish selections; `words` = 32-bit words per query
// bitmap (>= floor(t_max/B)/32 + 1 over the launch)
int union_queries_per_block();
hipError_t launch_attn_union(const SeqTable& seqs, int64_t max_nq, const AttnArgs& a, int words,
                             hipStream_t stream);

}  // namespace sgqa

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
namespace sgqa {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// sigmoid of a bf16 gate logit (fp32; 0 and 1 at the extremes)
__device__ __forceinline__ float gate_sigmoid(uint16_t bits) {
    return 1.0f / (1.0f + __expf(-__uint_as_float((uint32_t)bits << 16)));
}

// pool row of position pos through a sequence's page table pt (ids outside
// [0, n_pages) are clamped, so a bad table never reads outside the pool)
__device__ __forceinline__ int64_t paged_row(const int32_t* pt, int64_t n_pages, int64_t pos) {
    int64_t p = pt[pos / kPageTokens];
    p = p < 0 ? 0 : (p >= n_pages ? n_pages - 1 : p);
    return p * kPageTokens + pos % kPageTokens;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// bf16 value -> nearest OCP E4M3FN value (ties to even, saturating at 448),
// returned as bf16 bits.  Exact: scaling by powers of two and rint.
__device__ __forceinline__ uint32_t bf16_to_e4m3_as_bf16(uint32_t b) {
    float x = bf16_to_f32(b);
    float a = fabsf(x);
    float r;
    if (a < 0.015625f) {                         // below 2^-6: quantum 2^-9
        r = rintf(a * 512.0f) * (1.0f / 512.0f);
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // a in [2^e, 2^(e+1))
        float up = __uint_as_float((uint32_t)(127 + 3 - e) << 23);   // 2^(3-e)
        float dn = __uint_as_float((uint32_t)(127 - 3 + e) << 23);   // 2^(e-3)
        r = rintf(a * up) * dn;
    }
    r = fminf(r, 448.0f);
    r = copysignf(r, x);
    return __float_as_uint(r) >> 16;             // exactly representable in bf16
}

// OCP E4M3FN code of a bf16 value that E4M3 represents exactly (what
// bf16_to_e4m3_as_bf16 returns): normals (bf16 exponent >= 121, i.e. >= 2^-6)
// take the exponent rebiased by -120 and the top three mantissa bits;
// smaller values are multiples of 2^-9 (the code's low bits), zero included.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t h) {
    const uint32_t sign = (h >> 8) & 0x80u;
    const uint32_t e = (h >> 7) & 0xFFu;
    const uint32_t mt = h & 0x7Fu;
    if (e >= 121) return sign | ((e - 120) << 3) | (mt >> 4);
    if (e < 118) return sign;
    return sign | ((0x80u | mt) >> (125 - e));
}

// Order-preserving map of a score to uint32 (larger score -> larger key);
// -0.0 is first folded into +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The indexer score of one (query, group, block) from the MFMA result of its
// four heads: sum_i w_i * max(0, dot_i), accumulated from +0 with fused
// multiply-adds, so an exactly zero score is +0, never -0 (equal scores
// compare equal as keys).  max(0, x) is an integer max on the bits (a
// negative float, -0 included, is a negative integer); the inputs are finite.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }
__device__ __forceinline__ float head_score(f32x4 acc, float4 w) {
    float s = fmaf(w.x, relu_bits(acc[0]), 0.0f);
    s = fmaf(w.y, relu_bits(acc[1]), s);
    s = fmaf(w.z, relu_bits(acc[2]), s);
    return fmaf(w.w, relu_bits(acc[3]), s);
}
// score_key for a score that is not -0 (head_score's results)
__device__ __forceinline__ uint32_t score_key_nz(float s) {
    const uint32_t u = __float_as_uint(s);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// a value the wavefront holds in every lane, as a uniform (scalar) value
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// number of set bits of `mask` at lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// make this wave's LDS writes visible to its other lanes
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(uint2 v) { return __builtin_bit_cast(i16x4, v); }

// cos / sin of the rotary angle pos * theta.  The angle is reduced modulo
// 2*pi in fp64 (an fp32 product would lose ~0.06 rad near position 1e6),
// then evaluated in fp32 on the reduced argument.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double theta, float* c, float* s) {
    const double kTwoPiHi = 6.283185307179586;
    const double kTwoPiLo = 2.4492935982947064e-16;
    const double phi = (double)pos * theta;
    const double k = rint(phi * 0.15915494309189535);
    const double r = (phi - k * kTwoPiHi) - k * kTwoPiLo;
    sincosf((float)r, s, c);
}

}  // namespace dev
}  // namespace sgqa
#endif
