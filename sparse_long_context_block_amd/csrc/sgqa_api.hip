// Host side of libsgqa.so: argument validation, launch policy, workspace
// carving and the extern "C" entry points declared in include/sgqa.h.
//
// Every check runs before the first HIP call, so rejected calls are testable
// on a machine without a GPU and enqueue nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <map>
#include <mutex>
#include <utility>
#include <string>
#include <vector>

#include "sgqa.h"
#include "sgqa_internal.hpp"

namespace sgqa {

hipError_t set_dynamic_lds(const void* kernel, size_t bytes) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, size_t> set;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    size_t& have = set[{dev, kernel}];
    if (bytes <= have) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

}  // namespace sgqa

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SGQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// the stream must belong to the current device: kernel attributes, the
// static scratch and the forward's second stream are kept per current device
int check_stream(void* hip_stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (!hip_stream) return SGQA_OK;
    int sdev = 0;
    e = hipStreamGetDevice((hipStream_t)hip_stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
        return fail(SGQA_ERR_CONFIG, "hip_stream belongs to device %d, the current device is %d", sdev, dev);
    return SGQA_OK;
}

constexpr int64_t kMaxExtent = (int64_t)1 << 40;   // bound on offsets / lengths
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_config(const sgqa_config* c) {
    if (!c) return fail(SGQA_ERR_NULL, "cfg is NULL");
    if (c->num_q_heads <= 0 || c->num_kv_groups <= 0 || c->head_dim <= 0 || c->idx_heads <= 0 ||
        c->idx_dim <= 0 || c->rope_dim < 0 || c->block_size <= 0 || c->topk_blocks <= 0)
        return fail(SGQA_ERR_CONFIG, "config sizes must be positive");
    if (c->num_q_heads % c->num_kv_groups != 0)
        return fail(SGQA_ERR_CONFIG, "num_q_heads (%d) is not a multiple of num_kv_groups (%d)",
                    c->num_q_heads, c->num_kv_groups);
    if (c->rope_dim % 2 != 0 || c->rope_dim > c->idx_dim)
        return fail(SGQA_ERR_CONFIG, "rope_dim (%d) must be even and <= idx_dim", c->rope_dim);
    if (!(isfinite(c->rope_base) && c->rope_base > 0.f))
        return fail(SGQA_ERR_CONFIG, "rope_base must be finite and positive");
    if (!(isfinite(c->softmax_scale) && c->softmax_scale > 0.f))
        return fail(SGQA_ERR_CONFIG, "softmax_scale must be finite and positive");
    if (!(isfinite(c->eps_rms) && c->eps_rms >= 0.f && isfinite(c->eps_ln) && c->eps_ln >= 0.f))
        return fail(SGQA_ERR_CONFIG, "eps_rms / eps_ln must be finite and >= 0");
    if (c->store_q8 < 0 || c->store_q8 > 2)
        return fail(SGQA_ERR_CONFIG, "store_q8 must be 0, 1 or 2");
    if (c->num_q_heads != sgqa::kHeads || c->num_kv_groups != sgqa::kGroups ||
        c->head_dim != sgqa::kHeadDim || c->idx_heads != sgqa::kIdxHeads ||
        c->idx_dim != sgqa::kIdxDim || c->rope_dim != sgqa::kRopeDim)
        return fail(SGQA_ERR_UNSUPPORTED,
                    "compiled shapes are H=64, G=4, D=192, idx_heads=4, idx_dim=128, rope_dim=32");
    const int B = c->block_size;
    if (B != 1 && B != 2 && B != 4 && B != 8 && B != 16)
        return fail(SGQA_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16}", B);
    if (c->topk_blocks > sgqa::kMaxTopK)
        return fail(SGQA_ERR_UNSUPPORTED, "topk_blocks %d above %d", c->topk_blocks, sgqa::kMaxTopK);
    return SGQA_OK;
}

int check_seqs(const sgqa_config* c, const sgqa_seq* s, int32_t n) {
    if (!s) return fail(SGQA_ERR_NULL, "seqs is NULL");
    if (n <= 0) return fail(SGQA_ERR_SHAPE, "n_seqs must be >= 1 (got %d)", n);
    for (int32_t i = 0; i < n; ++i) {
        const sgqa_seq& q = s[i];
        const int64_t f[8] = {q.q_offset, q.n_q, q.pos0, q.cache_len,
                              q.kv_offset, q.kv_capacity, q.store_offset, q.store_capacity};
        for (int k = 0; k < 8; ++k)
            if (f[k] < 0 || f[k] > kMaxExtent)
                return fail(SGQA_ERR_SHAPE, "seqs[%d]: field %d out of range [0, 2^40]", i, k);
        if (q.cache_len != q.pos0 + q.n_q)
            return fail(SGQA_ERR_CAUSAL, "seqs[%d]: cache_len %lld != pos0 %lld + n_q %lld", i,
                        (long long)q.cache_len, (long long)q.pos0, (long long)q.n_q);
        if (q.cache_len > q.kv_capacity)
            return fail(SGQA_ERR_CAPACITY, "seqs[%d]: cache_len %lld > kv_capacity %lld", i,
                        (long long)q.cache_len, (long long)q.kv_capacity);
        if (q.cache_len / c->block_size > q.store_capacity)
            return fail(SGQA_ERR_CAPACITY, "seqs[%d]: %lld blocks exceed store_capacity %lld", i,
                        (long long)(q.cache_len / c->block_size), (long long)q.store_capacity);
    }
    return SGQA_OK;
}

// Paged per-token tensors: a page table of int32 physical page ids (device
// memory), table_len entries, over a pool of n_pages pages of 16 positions.
struct Paging {
    const int32_t* table = nullptr;     // null: contiguous caches
    int64_t n_pages = 0;
};

int check_paging(const sgqa_seq* s, int32_t n, const int32_t* table, int64_t table_len, int64_t n_pages) {
    if (!table) return fail(SGQA_ERR_NULL, "page_table is NULL");
    if (table_len <= 0 || n_pages <= 0)
        return fail(SGQA_ERR_SHAPE, "page_table_len (%lld) and n_pages (%lld) must be positive",
                    (long long)table_len, (long long)n_pages);
    if (n_pages > ((int64_t)1 << 31) / sgqa::kPageTokens)
        return fail(SGQA_ERR_SHAPE, "n_pages %lld above 2^27", (long long)n_pages);
    for (int32_t i = 0; i < n; ++i) {
        const int64_t pages = (s[i].kv_capacity + sgqa::kPageTokens - 1) / sgqa::kPageTokens;
        if (s[i].kv_offset + pages > table_len)
            return fail(SGQA_ERR_CAPACITY,
                        "seqs[%d]: page-table entries %lld .. %lld past page_table_len %lld", i,
                        (long long)s[i].kv_offset, (long long)(s[i].kv_offset + pages - 1),
                        (long long)table_len);
    }
    return SGQA_OK;
}

// ---------------------------------------------------------------------------
// launch policy
// ---------------------------------------------------------------------------
enum class IndexMode { Fused, Split, Tiled };

struct IndexPlan {
    IndexMode mode = IndexMode::Fused;
    int n_split = 1;
    int split_blocks = 0;
    int cap = 0;
    int64_t key_stride = 0;
    int64_t rows = 0;           // key-workspace rows: queries of the largest launch
    int64_t chunk_rows = 0;     // tiled mode: queries per launch (one key pass)
    size_t frag_off = 0;        // tiled mode: byte offset of the query fragments
    size_t ctl_off = 0;         // tiled mode: byte offset of the failed-row list
    size_t diag_off = 0;        // tiled mode: byte offset of the diagnostics block
    bool listed = false;        // tiled mode: long rows may use candidate lists
    int32_t list_off = 0, samp_off = 0, tau_off = 0;
    size_t ws = 0;
};

// tiled mode: bytes of one query's indexer A fragments (16 rows x 128 bf16)
constexpr size_t kQueryFragBytes = (size_t)sgqa::kGroups * sgqa::kIdxHeads * sgqa::kIdxDim * 2;
// tiled mode: the score kernel addresses the keys of 16 queries with 32-bit
// byte offsets
constexpr int64_t kTiledMaxStride = ((int64_t)1 << 32) / (16 * sgqa::kGroups * 4) - 64;

// key workspace of the tiled mode: query rows are processed in passes whose
// keys (4 B per row, group and candidate) fit this budget (4 GiB: a 1M-token
// prefill at B = 1 then runs 192 queries per launch instead of 48, so the
// launches' fixed costs -- sample, threshold, list select, rescue -- are paid
// a quarter as often; 8 and 16 GiB measured no faster)
constexpr size_t kTiledKeyBudget = (size_t)1 << 32;
constexpr int kTiledSplitBlocks = 2048;

struct AttnPlan {
    int n_split = 1;
    int chunks_per_split = 0;
    int64_t rows = 0;           // workspace rows: gather queries of one launch
    bool range_split = false;   // splits are ranges of the token list, one per XCD (pair)
    size_t ws = 0;
};

// Range splits across XCDs.  Workgroups go to the eight XCDs round-robin in
// launch order, and the gather grid is (group, query, split)-major, so with
// 4 or 8 splits every split of every unit runs on the same XCD(s): each
// XCD's L2 then holds only its split's range of the group's selected rows.
// Measured on the 64K-token prefill's late rows: 21 TB/s of gathered rows
// with each XCD's reads confined to an eighth or a quarter of the block
// range, 9 TB/s unconfined.  Worth it while a sequence's K+V rows of one
// group (768 B per token) split in four or eight stay near 12 MB, i.e. up to
// 128K tokens; the partials of at most kRangeSplitPassBytes go per launch.
constexpr int64_t kRangeSplitMaxTokens = 131072;
constexpr int64_t kRangeSplitMinUnits = 2048;
constexpr size_t kRangeSplitPassBytes = (size_t)1 << 30;

// Workspace rows are numbered per launch table (DevSeq::ws_row), so a
// workspace holds the queries of the largest table, whatever the queries'
// row offsets.  With tables of kMaxSeqsPerLaunch sequences in call order,
// that is the largest sum of nq(seq) over such a group.
template <typename Rows>
int64_t max_launch_rows(const sgqa_seq* s, int32_t n, Rows nq) {
    int64_t best = 0;
    for (int32_t first = 0; first < n; first += sgqa::kMaxSeqsPerLaunch) {
        const int32_t end = std::min<int32_t>(n, first + sgqa::kMaxSeqsPerLaunch);
        int64_t sum = 0;
        for (int32_t i = first; i < end; ++i) sum += std::max<int64_t>(0, nq(s[i]));
        best = std::max(best, sum);
    }
    return best;
}

// Three ways to run the indexer and the selection:
//  * Tiled (1024 queries or more, fewer than 16.7M candidates): each query's
//    indexer rows are prepared once, 16-query workgroups score candidate
//    ranges against store tiles shared in LDS, keys go to the workspace in
//    passes of at most kTiledKeyBudget bytes, one workgroup per (query,
//    group) selects;
//  * Split (fewer queries, long histories, keys within 1 GiB): each query's
//    candidates are spread over score wavefronts, then the same selection;
//  * Fused (the rest): one wavefront per query scores and keeps a streaming
//    top-k in LDS; no workspace.
IndexPlan plan_index(const sgqa_config* c, const sgqa_seq* s, int32_t n) {
    IndexPlan p;
    const int K = c->topk_blocks;
    p.cap = (K + 256 + 63) / 64 * 64;
    while (p.cap > K + 64 && sgqa::index_lds_bytes(p.cap) > sgqa::kMaxLds) p.cap -= 64;
    int64_t total_q = 0, max_b = 0;
    for (int32_t i = 0; i < n; ++i) {
        total_q += s[i].n_q;
        if (s[i].n_q > 0) max_b = std::max(max_b, (s[i].cache_len - 1) / c->block_size);
    }
    p.n_split = 1;
    p.split_blocks = 0x7FFFFFF0;
    p.key_stride = 0;
    // key rows are 256 B x an odd number apart, so the rows that score and
    // select workgroups touch at the same time spread over the memory
    // channels instead of all starting at one power-of-two alignment
    int64_t stride = std::max<int64_t>(64, (max_b + 63) / 64 * 64);
    if ((stride / 64) % 2 == 0) stride += 64;
    if (total_q >= 1024 && stride <= kTiledMaxStride) {
        const size_t row_bytes = (size_t)sgqa::kGroups * stride * 4;
        int64_t chunk = (int64_t)(kTiledKeyBudget / row_bytes) / 16 * 16;
        chunk = std::max<int64_t>(16, std::min<int64_t>(chunk, (total_q + 15) / 16 * 16));
        p.mode = IndexMode::Tiled;
        p.chunk_rows = chunk;
        p.rows = chunk;
        p.key_stride = stride;
        p.split_blocks = kTiledSplitBlocks;
        p.n_split = (int)std::max<int64_t>(1, (max_b + kTiledSplitBlocks - 1) / kTiledSplitBlocks);
        p.frag_off = align_up((size_t)chunk * row_bytes);
        p.ctl_off = p.frag_off + align_up((size_t)chunk * kQueryFragBytes);
        p.diag_off = p.ctl_off + align_up((size_t)(1 + chunk * sgqa::kGroups) * 4);
        p.ws = p.diag_off + align_up((size_t)sgqa::kDiagWords * 4);
        // candidate lists share a key row with one count per segment, the
        // sample and the threshold; rows short enough to hold them all are
        // long enough to be listed
        const int64_t nseg = (stride + sgqa::kSegBlocks - 1) / sgqa::kSegBlocks;
        const int64_t list_off = (nseg + 63) / 64 * 64;
        const int64_t samp_off = list_off + 2 * sgqa::kSegCap * nseg;
        const int64_t tau_off = samp_off + sgqa::kListSampleMax;
        p.listed = max_b >= sgqa::kListMinBlocks && tau_off < stride;
        p.list_off = (int32_t)list_off;
        p.samp_off = (int32_t)samp_off;
        p.tau_off = (int32_t)tau_off;
        return p;
    }
    p.rows = max_launch_rows(s, n, [](const sgqa_seq& q) { return q.n_q; });
    const size_t key_bytes = (size_t)p.rows * sgqa::kGroups * stride * 4;
    if (total_q == 0 || max_b <= K || key_bytes > ((size_t)1 << 30)) return p;
    // about 8192 score wavefronts, at least 256 candidate blocks each (measured
    // on the 64-sequence decode against 2048..16384)
    int64_t split = std::min<int64_t>((8192 + total_q - 1) / total_q, std::max<int64_t>(1, max_b / 256));
    int64_t per = (max_b + split - 1) / split;
    per = (per + 15) / 16 * 16;
    p.mode = IndexMode::Split;
    p.split_blocks = (int)per;
    p.n_split = (int)((max_b + per - 1) / per);
    p.key_stride = stride;
    p.ws = align_up(key_bytes);
    return p;
}

void rope_table(const sgqa_config* c, double* theta) {
    for (int j = 0; j < sgqa::kRopeDim / 2; ++j)
        theta[j] = pow((double)c->rope_base, -2.0 * j / (double)sgqa::kRopeDim);
}

// Queries of a sequence [0, n_dense) whose selection covers at least a
// quarter of their candidates (floor(t/B) <= 4K) take the tiled kernel when
// the sequence brings enough queries to fill its workgroups; the rest take
// the gather kernel.
int64_t dense_queries(const sgqa_config* c, const sgqa_seq& q) {
    if (q.n_q < 64) return 0;
    const int64_t limit = 4 * (int64_t)c->topk_blocks * c->block_size;   // t < limit
    return std::max<int64_t>(0, std::min<int64_t>(q.n_q, limit - q.pos0));
}

AttnPlan plan_attn(const sgqa_config* c, const sgqa_seq* s, int32_t n) {
    AttnPlan p;
    p.rows = max_launch_rows(s, n, [c](const sgqa_seq& q) { return q.n_q - dense_queries(c, q); });
    int64_t total_q = 0;
    for (int32_t i = 0; i < n; ++i) total_q += s[i].n_q - dense_queries(c, s[i]);
    const int64_t max_chunks =
        ((int64_t)c->topk_blocks * c->block_size + c->block_size + 15) / 16;
    const int64_t units = total_q * sgqa::kGroups;
    int64_t max_cache = 0;
    for (int32_t i = 0; i < n; ++i)
        if (s[i].n_q - dense_queries(c, s[i]) > 0) max_cache = std::max(max_cache, s[i].cache_len);
    if (units >= kRangeSplitMinUnits && max_cache <= kRangeSplitMaxTokens && max_chunks >= 64) {
        p.range_split = true;
        p.n_split = max_cache > 65536 ? 8 : 4;
        p.chunks_per_split = (int)((max_chunks + p.n_split - 1) / p.n_split);
        const size_t row_bytes =
            (size_t)sgqa::kGroups * p.n_split * sgqa::kHeadsPerGroup * (sgqa::kHeadDim + 2) * 4;
        p.rows = std::max<int64_t>(1, std::min<int64_t>(p.rows, (int64_t)(kRangeSplitPassBytes / row_bytes)));
        const size_t parts = (size_t)p.rows * sgqa::kGroups * p.n_split * sgqa::kHeadsPerGroup;
        p.ws = align_up(parts * sgqa::kHeadDim * 4) + align_up(parts * 2 * 4);
        return p;
    }
    // otherwise split only calls too small to give each CU a workgroup
    // (measured on the 64-sequence decode: 256 unsplit workgroups beat 1024
    // split ones and the merge they need)
    int64_t want = units > 0 ? (256 + units - 1) / units : 1;
    int64_t split = std::min<int64_t>({want, std::max<int64_t>(1, max_chunks / 8),
                                       (int64_t)sgqa::kMaxAttnSplits});
    if (split <= 1) {
        p.n_split = 1;
        p.chunks_per_split = (int)std::min<int64_t>(max_chunks + 4, 0x7FFFFFF0);
        return p;
    }
    int64_t per = (max_chunks + split - 1) / split;
    per = (per + 3) / 4 * 4;
    p.chunks_per_split = (int)per;
    p.n_split = (int)((max_chunks + per - 1) / per);
    if (p.n_split <= 1) {
        p.n_split = 1;
        p.chunks_per_split = (int)(max_chunks + 4);
        return p;
    }
    const size_t parts = (size_t)p.rows * sgqa::kGroups * p.n_split * sgqa::kHeadsPerGroup;
    p.ws = align_up(parts * sgqa::kHeadDim * 4) + align_up(parts * 2 * 4);
    return p;
}

// The gather kernel addresses a contiguous cache's rows with 32-bit byte
// offsets from the sequence's first row (1536 bytes per row of one tensor).
constexpr int64_t kMaxGatherRows = (((int64_t)1 << 32) - 1024) / (sgqa::kGroups * sgqa::kHeadDim * 2);

int check_gather_rows(const sgqa_seq* s, int32_t n) {
    for (int32_t i = 0; i < n; ++i)
        if (s[i].kv_capacity > kMaxGatherRows)
            return fail(SGQA_ERR_UNSUPPORTED,
                        "seqs[%d]: kv_capacity %lld above %lld rows (contiguous K/V caches are "
                        "addressed with 32-bit offsets per sequence; use the paged calls)",
                        i, (long long)s[i].kv_capacity, (long long)kMaxGatherRows);
    return SGQA_OK;
}

// Tensor rows are read and written with vector accesses of up to 16 bytes.
int check_aligned(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
    for (const auto& p : ptrs)
        if (p.first && ((uintptr_t)p.first & 15u))
            return fail(SGQA_ERR_SHAPE, "%s is not 16-byte aligned", p.second);
    return SGQA_OK;
}

int check_ws(size_t need, void* ws, size_t ws_bytes) {
    if (need == 0) return SGQA_OK;
    if (!ws) return fail(SGQA_ERR_WORKSPACE, "workspace of %zu bytes required, ws is NULL", need);
    if (ws_bytes < need)
        return fail(SGQA_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, ws_bytes);
    if (((uintptr_t)ws) % kAlign != 0)
        return fail(SGQA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    return SGQA_OK;
}

// Fill a launch table with sequences [first, first+count) that have queries
// (or blocks to compress); returns the largest per-sequence extent `ext`.
template <typename Extent>
int64_t fill_table(sgqa::SeqTable& tab, const sgqa_seq* s, int32_t first, int32_t count,
                   Extent ext) {
    tab.n = 0;
    tab.pad_ = 0;
    int64_t mx = 0, rows = 0;
    for (int32_t i = first; i < first + count; ++i) {
        const int64_t e = ext(s[i]);
        if (e <= 0) continue;
        sgqa::DevSeq& d = tab.s[tab.n++];
        d.q_offset = s[i].q_offset;
        d.n_q = s[i].n_q;
        d.pos0 = s[i].pos0;
        d.kv_offset = s[i].kv_offset;
        d.store_offset = s[i].store_offset;
        d.ws_row = rows;
        rows += s[i].n_q;
        mx = std::max(mx, e);
    }
    return mx;
}

// ---------------------------------------------------------------------------
// the three steps (arguments already validated)
// ---------------------------------------------------------------------------
sgqa::CompressArgs compress_args(const sgqa_config* c, const void* proxy_k, const float* logits,
                                 const Paging& pg, const void* ln_gamma, const void* ln_beta, void* store) {
    sgqa::CompressArgs a;
    a.proxy_k = (const uint16_t*)proxy_k;
    a.logits = logits;
    a.page_table = pg.table;
    a.n_pages = pg.n_pages;
    a.ln_gamma = (const uint16_t*)ln_gamma;
    a.ln_beta = (const uint16_t*)ln_beta;
    a.store = (uint16_t*)store;
    a.block_size = c->block_size;
    a.store_q8 = c->store_q8;
    a.eps = c->eps_ln;
    rope_table(c, a.theta);
    return a;
}

// true when no query of the call has a block the call completes among its
// candidates: every sequence's queries lie inside one block (query t sees
// blocks below t / B; the call completes the blocks below (pos0 + n_q) / B
// from pos0 / B on, so at most the block of its queries)
bool merge_unread_by_call(const sgqa_config* c, const sgqa_seq* s, int32_t n) {
    const int64_t B = c->block_size;
    for (int32_t i = 0; i < n; ++i)
        if (s[i].n_q > 0 && (s[i].pos0 + s[i].n_q - 1) / B != s[i].pos0 / B) return false;
    return true;
}

int run_compress(const sgqa_config* c, const sgqa_seq* s, int32_t n, const void* proxy_k,
                 const float* logits, const Paging& pg, const void* ln_gamma, const void* ln_beta,
                 void* store, hipStream_t st) {
    const sgqa::CompressArgs a = compress_args(c, proxy_k, logits, pg, ln_gamma, ln_beta, store);
    const int B = c->block_size;
    for (int32_t first = 0; first < n; first += sgqa::kMaxSeqsPerLaunch) {
        const int32_t cnt = std::min<int32_t>(sgqa::kMaxSeqsPerLaunch, n - first);
        sgqa::SeqTable tab;
        const int64_t mx = fill_table(tab, s, first, cnt, [B](const sgqa_seq& q) {
            return q.cache_len / B - q.pos0 / B;
        });
        if (tab.n == 0) continue;
        hipError_t e = sgqa::launch_compress(tab, mx, a, st);
        if (e != hipSuccess) return hip_fail(e, "compress launch");
    }
    return SGQA_OK;
}

// diag_at: the diagnostics block to use instead of the plan's own (the
// pieces of a split forward call share one), cleared by this call only when
// diag_clear is set
// merge: step 1 for split-mode calls whose queries read none of the blocks
// they complete, carried in the scoring launch (null: run separately)
int run_index(const sgqa_config* c, const sgqa_seq* s, int32_t n, const IndexPlan& p,
              const void* q_idx, const float* w, const void* rms_gamma, const void* store,
              int32_t* sel, float* sel_scores, void* q_hat_out, void* ws, hipStream_t st,
              uint32_t* diag_at = nullptr, bool diag_clear = true,
              const sgqa::CompressArgs* merge = nullptr) {
    sgqa::IndexArgs a;
    a.q_idx = (const uint16_t*)q_idx;
    a.w = w;
    a.rms_gamma = (const uint16_t*)rms_gamma;
    a.store = (const uint16_t*)store;
    a.store_fp8 = c->store_q8 == 2;
    a.sel = sel;
    a.sel_scores = sel_scores;
    a.q_hat_out = (uint16_t*)q_hat_out;
    a.block_size = c->block_size;
    a.topk = c->topk_blocks;
    a.cap = p.cap;
    a.n_split = p.n_split;
    a.split_blocks = p.split_blocks;
    a.eps = c->eps_rms;
    rope_table(c, a.theta);
    a.part_key = nullptr;
    a.q_frag = nullptr;
    a.ctl = nullptr;
    a.diag = nullptr;
    a.diag_clear = 0;
    a.key_stride = p.key_stride;
    a.listed = p.listed ? 1 : 0;
    a.list_off = p.list_off;
    a.samp_off = p.samp_off;
    a.tau_off = p.tau_off;
    if (p.key_stride > 0) a.part_key = (uint32_t*)ws;
    if (p.frag_off > 0) a.q_frag = (uint4*)((char*)ws + p.frag_off);
    if (p.ctl_off > 0) a.ctl = (uint32_t*)((char*)ws + p.ctl_off);
    if (p.diag_off > 0) {
        a.diag = diag_at ? diag_at : (uint32_t*)((char*)ws + p.diag_off);
        a.diag_clear = diag_clear ? 1 : 0;
    }
    if (p.mode == IndexMode::Tiled) {
        // launches of at most chunk_rows queries (one pass over the key
        // workspace each) and kMaxSeqsPerLaunch entries, filled in call
        // order; a sequence that does not fit the room left is cut
        sgqa::SeqTable tab;
        tab.n = 0;
        tab.pad_ = 0;
        int64_t used = 0, mx = 0;
        for (int32_t i = 0; i < n; ++i) {
            const sgqa_seq& q = s[i];
            for (int64_t done = 0; done < q.n_q;) {
                const int64_t take = std::min(q.n_q - done, p.chunk_rows - used);
                sgqa::DevSeq& d = tab.s[tab.n++];
                d.q_offset = q.q_offset + done;
                d.n_q = take;
                d.pos0 = q.pos0 + done;
                d.kv_offset = q.kv_offset;
                d.store_offset = q.store_offset;
                d.ws_row = used;
                used += take;
                done += take;
                mx = std::max(mx, take);
                if (used == p.chunk_rows || tab.n == sgqa::kMaxSeqsPerLaunch) {
                    hipError_t e = sgqa::launch_index_tiled(tab, mx, a, st);
                    if (e != hipSuccess) return hip_fail(e, "index_topk launch");
                    a.diag_clear = 0;
                    tab.n = 0;
                    used = 0;
                    mx = 0;
                }
            }
        }
        if (tab.n > 0) {
            hipError_t e = sgqa::launch_index_tiled(tab, mx, a, st);
            if (e != hipSuccess) return hip_fail(e, "index_topk launch");
        }
        return SGQA_OK;
    }
    for (int32_t first = 0; first < n; first += sgqa::kMaxSeqsPerLaunch) {
        const int32_t cnt = std::min<int32_t>(sgqa::kMaxSeqsPerLaunch, n - first);
        sgqa::SeqTable tab;
        const int64_t mx = fill_table(tab, s, first, cnt, [](const sgqa_seq& q) { return q.n_q; });
        if (tab.n == 0) continue;
        hipError_t e = p.mode == IndexMode::Split ? sgqa::launch_index_split(tab, mx, a, st, merge)
                                                  : sgqa::launch_index_topk(tab, mx, a, st);
        if (e != hipSuccess) return hip_fail(e, "index_topk launch");
    }
    return SGQA_OK;
}

int run_attn(const sgqa_config* c, const sgqa_seq* s, int32_t n, const AttnPlan& p,
             const void* q, const void* k_cache, const void* v_cache, const Paging& pg,
             const int32_t* sel, void* out, float* lse, const void* gate, void* ws, hipStream_t st) {
    sgqa::AttnArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_cache;
    a.v = (const uint16_t*)v_cache;
    a.page_table = pg.table;
    a.n_pages = pg.n_pages;
    a.gate = (const uint16_t*)gate;
    a.sel = sel;
    a.out = (uint16_t*)out;
    a.lse = lse;
    a.block_size = c->block_size;
    a.topk = c->topk_blocks;
    a.n_split = p.n_split;
    a.chunks_per_split = p.chunks_per_split;
    a.scale_log2 = c->softmax_scale * 1.4426950408889634f;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    if (p.n_split > 1) {
        const size_t parts = (size_t)p.rows * sgqa::kGroups * p.n_split * sgqa::kHeadsPerGroup;
        a.part_o = (float*)ws;
        a.part_ml = (float*)((char*)ws + align_up(parts * sgqa::kHeadDim * 4));
    }
    // the gather queries in launches of at most p.rows queries (the
    // workspace rows) and kMaxSeqsPerLaunch entries; a sequence that does not
    // fit the room left is cut
    sgqa::SeqTable gt;
    gt.n = 0;
    gt.pad_ = 0;
    int64_t gmax = 0, grows = 0;
    auto flush_gather = [&]() -> int {
        if (gt.n == 0) return SGQA_OK;
        hipError_t e = sgqa::launch_sparse_attn(gt, gmax, a, st);
        if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
        if (p.n_split > 1) {
            sgqa::AttnMergeArgs ma;
            ma.part_o = a.part_o;
            ma.part_ml = a.part_ml;
            ma.gate = a.gate;
            ma.out = (uint16_t*)out;
            ma.lse = lse;
            ma.n_split = p.n_split;
            e = sgqa::launch_attn_merge(gt, gmax, ma, st);
            if (e != hipSuccess) return hip_fail(e, "attn_merge launch");
        }
        gt.n = 0;
        gmax = 0;
        grows = 0;
        return SGQA_OK;
    };
    for (int32_t first = 0; first < n; first += sgqa::kMaxSeqsPerLaunch) {
        const int32_t cnt = std::min<int32_t>(sgqa::kMaxSeqsPerLaunch, n - first);
        // dense-ish leading queries -> tiled kernel
        sgqa::SeqTable ut;
        ut.n = 0;
        ut.pad_ = 0;
        int64_t umax = 0, ublk = 0;
        for (int32_t i = first; i < first + cnt; ++i) {
            const sgqa_seq& q = s[i];
            const int64_t nd = dense_queries(c, q);
            if (nd > 0) {
                sgqa::DevSeq& d = ut.s[ut.n++];
                d.q_offset = q.q_offset;
                d.n_q = nd;
                d.pos0 = q.pos0;
                d.kv_offset = q.kv_offset;
                d.store_offset = q.store_offset;
                d.ws_row = 0;   // the tiled kernel uses no workspace
                umax = std::max(umax, nd);
                ublk = std::max(ublk, (q.pos0 + nd - 1) / c->block_size);
            }
        }
        if (ut.n > 0) {
            const int words = (int)(ublk / 32 + 1);
            hipError_t e = sgqa::launch_attn_union(ut, umax, a, words, st);
            if (e != hipSuccess) return hip_fail(e, "sparse_attn (tiled) launch");
        }
        for (int32_t i = first; i < first + cnt; ++i) {
            const sgqa_seq& q = s[i];
            const int64_t nd = dense_queries(c, q);
            for (int64_t done = nd; done < q.n_q;) {
                const int64_t take = std::min(q.n_q - done, p.rows - grows);
                sgqa::DevSeq& d = gt.s[gt.n++];
                d.q_offset = q.q_offset + done;
                d.n_q = take;
                d.pos0 = q.pos0 + done;
                d.kv_offset = q.kv_offset;
                d.store_offset = q.store_offset;
                d.ws_row = grows;
                grows += take;
                done += take;
                gmax = std::max(gmax, take);
                if (grows == p.rows || gt.n == sgqa::kMaxSeqsPerLaunch) {
                    const int rc = flush_gather();
                    if (rc) return rc;
                }
            }
        }
    }
    {
        const int rc = flush_gather();
        if (rc) return rc;
    }
    return SGQA_OK;
}

// ---------------------------------------------------------------------------
// Forward calls: the index step beside the attention
// ---------------------------------------------------------------------------
// A call whose queries all take the gather kernel and whose index step runs
// tiled (long histories, e.g. an 8,192-query chunk over a 1M-token cache) is
// split into pieces of at least kPieceQueries queries.  Piece i's index step
// runs on the caller's stream; piece i's attention waits for it (an event)
// on a second stream the library keeps per device, so it runs while the
// index step of piece i + 1 does: the index step is compute-bound and the
// gather bound by the memory system.  The caller's stream waits for the
// second stream before its next work, so the call keeps the stream order of
// a single-stream call.  The pieces use disjoint workspace regions (the
// index region first, then the attention region) and write disjoint rows of
// sel / out / lse.  Only calls whose every query takes the unsplit gather
// kernel are split, so each query's index and attention run exactly as in a
// single-stream call and the outputs are the same bit for bit.  Measured on the 1M chunk: 19.5 ->
// 18.5 ms per call with eight pieces.
constexpr int64_t kPieceQueries = 1024;     // each piece's index step stays tiled
constexpr int kMaxPieces = 16;

struct ForwardLayout {
    bool pieces = false;
    std::vector<std::vector<sgqa_seq>> piece;
    size_t idx_ws = 0, attn_off = 0, diag_off = 0, ws = 0;
};

// the queries of [s, s + n) in call order cut into np pieces: `per` queries
// each, the last one the rest (a sequence may be cut; each part keeps
// cache_len = pos0 + n_q)
std::vector<std::vector<sgqa_seq>> cut_pieces(const sgqa_seq* s, int32_t n, int64_t per, int64_t np) {
    std::vector<std::vector<sgqa_seq>> out(1);
    int64_t room = per;
    for (int32_t i = 0; i < n; ++i) {
        for (int64_t done = 0; done < s[i].n_q;) {
            if (room == 0) {
                out.emplace_back();
                room = (int64_t)out.size() < np ? per : INT64_MAX;
            }
            const int64_t take = std::min(s[i].n_q - done, room);
            sgqa_seq q = s[i];
            q.q_offset = s[i].q_offset + done;
            q.n_q = (int32_t)take;
            q.pos0 = s[i].pos0 + done;
            q.cache_len = q.pos0 + take;
            out.back().push_back(q);
            done += take;
            room -= take;
        }
    }
    return out;
}

ForwardLayout plan_forward(const sgqa_config* c, const sgqa_seq* s, int32_t n, bool allow_pieces) {
    ForwardLayout f;
    const IndexPlan ip = plan_index(c, s, n);
    const AttnPlan ap = plan_attn(c, s, n);
    f.ws = std::max(ip.ws, ap.ws);
    // pieces only where the gather takes queries (whose memory-bound
    // attention can run beside the next piece's index step), and only when
    // every query's attention runs in the pieces exactly as in a
    // single-stream call (checked below)
    if (!allow_pieces || ip.mode != IndexMode::Tiled) return f;
    int64_t total_q = 0, gather_q = 0;
    for (int32_t i = 0; i < n; ++i) {
        total_q += s[i].n_q;
        gather_q += s[i].n_q - dense_queries(c, s[i]);
    }
    if (total_q < 2 * kPieceQueries || gather_q < kPieceQueries) return f;
    // pieces of a multiple of 16 queries (the index tiles keep their
    // boundaries) and at least kPieceQueries each (their index steps stay
    // tiled)
    const int64_t np = std::min<int64_t>(kMaxPieces, total_q / kPieceQueries);
    const int64_t per = total_q / np / 16 * 16;
    const auto piece = cut_pieces(s, n, per, np);
    // each query keeps its kernel (the tiled kernel for a sequence's leading
    // dense-ish queries, else the gather) and the gather keeps its ranges
    // (the same split count and split length), so every query's attention is
    // the same arithmetic as in the single-stream call
    std::vector<int64_t> dense(n);
    for (int32_t i = 0; i < n; ++i) dense[i] = dense_queries(c, s[i]);
    size_t idx_ws = 0, attn_ws = 0;
    int32_t si = 0;                   // the call's sequence of the next part (parts
    int64_t done = 0;                 // follow the sequences in order), its queries so far
    for (const auto& pc : piece) {
        const IndexPlan pi = plan_index(c, pc.data(), (int32_t)pc.size());
        const AttnPlan pa = plan_attn(c, pc.data(), (int32_t)pc.size());
        if (pi.mode != IndexMode::Tiled) return f;
        int64_t pg = 0;
        for (const sgqa_seq& q : pc) {
            while (si < n && done >= s[si].n_q) {
                ++si;
                done = 0;
            }
            if (si == n) return f;
            const int64_t want = std::max<int64_t>(0, std::min<int64_t>(q.n_q, dense[si] - done));
            if (dense_queries(c, q) != want) return f;
            pg += q.n_q - want;
            done += q.n_q;
        }
        if (pg > 0 && (pa.n_split != ap.n_split || pa.range_split != ap.range_split ||
                       (ap.n_split > 1 && pa.chunks_per_split != ap.chunks_per_split)))
            return f;
        idx_ws = std::max(idx_ws, pi.ws);
        attn_ws = std::max(attn_ws, pa.ws);
    }
    f.piece = piece;
    f.pieces = true;
    f.idx_ws = idx_ws;
    f.attn_off = align_up(idx_ws);
    // the pieces' index steps share one diagnostics block, after the
    // attention region
    f.diag_off = f.attn_off + align_up(attn_ws);
    f.ws = f.diag_off + align_up((size_t)sgqa::kDiagWords * 4);
    return f;
}

// the second stream of the current device and the events that order the
// two streams (created on a device's first split call, kept until the
// process ends; default priority), or nullptr if they cannot be created
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t ev[kMaxPieces + 2] = {};
    std::mutex mu;            // one call's fork / join sequence at a time
};

SideStream* side_stream() {
    static std::mutex mu;
    static std::map<int, SideStream*> per_dev;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    auto it = per_dev.find(dev);
    if (it != per_dev.end()) return it->second;
    SideStream* ss = new SideStream();
    bool ok = hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < kMaxPieces + 2; ++i)
        ok = hipEventCreateWithFlags(&ss->ev[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        for (int i = 0; i < kMaxPieces + 2; ++i)
            if (ss->ev[i]) (void)hipEventDestroy(ss->ev[i]);
        if (ss->s) (void)hipStreamDestroy(ss->s);
        delete ss;
        per_dev[dev] = nullptr;      // not tried again: calls run on one stream
        return nullptr;
    }
    per_dev[dev] = ss;
    return ss;
}

// steps 1 -> 2+3 -> 4 (arguments validated): on the caller's stream, or in
// pieces over it and the side stream (see above) when the layout says so
int run_forward(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs, const void* proxy_k,
                const float* comp_logits, const void* ln_gamma, const void* ln_beta, void* store,
                const void* q_idx, const float* w, const void* rms_gamma, int32_t* sel, float* sel_scores,
                const void* q, const void* k_cache, const void* v_cache, const Paging& pg, void* out,
                float* lse, const void* gate, void* ws, size_t ws_bytes, hipStream_t st,
                bool allow_pieces = true) {
    const ForwardLayout fl = plan_forward(cfg, seqs, n_seqs, allow_pieces);
    int rc = check_ws(fl.ws, ws, ws_bytes);
    if (rc) return rc;
    if (!fl.pieces) {
        const IndexPlan ip = plan_index(cfg, seqs, n_seqs);
        const AttnPlan ap = plan_attn(cfg, seqs, n_seqs);
        // decode-shaped calls: the merge rides in the scoring launch (no
        // score of the call reads the rows it writes)
        const bool carry = ip.mode == IndexMode::Split && merge_unread_by_call(cfg, seqs, n_seqs);
        const sgqa::CompressArgs ca = compress_args(cfg, proxy_k, comp_logits, pg, ln_gamma, ln_beta, store);
        if (!carry &&
            (rc = run_compress(cfg, seqs, n_seqs, proxy_k, comp_logits, pg, ln_gamma, ln_beta, store, st)))
            return rc;
        if ((rc = run_index(cfg, seqs, n_seqs, ip, q_idx, w, rms_gamma, store, sel, sel_scores, nullptr, ws,
                            st, nullptr, true, carry ? &ca : nullptr)))
            return rc;
        return run_attn(cfg, seqs, n_seqs, ap, q, k_cache, v_cache, pg, sel, out, lse, gate, ws, st);
    }
    if ((rc = run_compress(cfg, seqs, n_seqs, proxy_k, comp_logits, pg, ln_gamma, ln_beta, store, st)))
        return rc;
    // pieces: over the side stream, or one after the other on the caller's
    // stream if the side stream could not be created (same layout)
    SideStream* side = side_stream();
    std::unique_lock<std::mutex> lock;
    if (side) lock = std::unique_lock<std::mutex>(side->mu);
    hipStream_t ast = side ? side->s : st;
    void* ws_attn = (char*)ws + fl.attn_off;
    uint32_t* diag = (uint32_t*)((char*)ws + fl.diag_off);
    const int np = (int)fl.piece.size();
    hipError_t e = hipSuccess;
    if (side) {
        e = hipEventRecord(side->ev[0], st);
        if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->ev[0], 0);
        if (e != hipSuccess) return hip_fail(e, "forward: ordering the side stream after the caller's");
    }
    for (int i = 0; i < np && rc == SGQA_OK; ++i) {
        const sgqa_seq* pc = fl.piece[i].data();
        const int32_t pn = (int32_t)fl.piece[i].size();
        rc = run_index(cfg, pc, pn, plan_index(cfg, pc, pn), q_idx, w, rms_gamma, store, sel, sel_scores,
                       nullptr, ws, st, diag, i == 0);
        if (rc) break;
        if (side) {
            e = hipEventRecord(side->ev[1 + i], st);
            if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->ev[1 + i], 0);
            if (e != hipSuccess) {
                rc = hip_fail(e, "forward: ordering a piece's attention after its index step");
                break;
            }
        }
        rc = run_attn(cfg, pc, pn, plan_attn(cfg, pc, pn), q, k_cache, v_cache, pg, sel, out, lse, gate,
                      ws_attn, ast);
    }
    if (side) {
        // the caller's stream waits for the side stream, also after an error
        e = hipEventRecord(side->ev[kMaxPieces + 1], side->s);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, side->ev[kMaxPieces + 1], 0);
        if (rc == SGQA_OK && e != hipSuccess) rc = hip_fail(e, "forward: joining the side stream");
    }
    return rc;
}

}  // namespace

// ---------------------------------------------------------------------------
// The workspace of sgqa_forward_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): each device's address comes from hipGetSymbolAddress, called once
// per device with that device current, and only that address is used.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// address of `scratch` on the current device (resolved on the first call
// per device), or nullptr with the status in *rc
void* scratch_address(int* rc) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = hip_fail(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *rc = fail(SGQA_ERR_UNSUPPORTED, "device %d above the %d devices the static scratch covers", dev,
                   kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *rc = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        addr[dev] = ptr;
    }
    *rc = SGQA_OK;
    return addr[dev];
}

}  // namespace

// ---------------------------------------------------------------------------
// extern "C" entry points
// ---------------------------------------------------------------------------
extern "C" {

int32_t sgqa_abi_version(void) { return 1; }

const char* sgqa_last_error(void) { return g_last_error.c_str(); }

const char* sgqa_status_string(int status) {
    switch (status) {
        case SGQA_OK: return "SGQA_OK";
        case SGQA_ERR_NULL: return "SGQA_ERR_NULL";
        case SGQA_ERR_CONFIG: return "SGQA_ERR_CONFIG";
        case SGQA_ERR_SHAPE: return "SGQA_ERR_SHAPE";
        case SGQA_ERR_CAUSAL: return "SGQA_ERR_CAUSAL";
        case SGQA_ERR_CAPACITY: return "SGQA_ERR_CAPACITY";
        case SGQA_ERR_WORKSPACE: return "SGQA_ERR_WORKSPACE";
        case SGQA_ERR_UNSUPPORTED: return "SGQA_ERR_UNSUPPORTED";
        case SGQA_ERR_HIP: return "SGQA_ERR_HIP";
        default: return "SGQA_UNKNOWN_STATUS";
    }
}

int64_t sgqa_index_diag_offset(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs) {
    if (check_config(cfg) != SGQA_OK || check_seqs(cfg, seqs, n_seqs) != SGQA_OK) return -1;
    const IndexPlan p = plan_index(cfg, seqs, n_seqs);
    return p.diag_off > 0 ? (int64_t)p.diag_off : -1;
}

int64_t sgqa_forward_diag_offset(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs) {
    if (check_config(cfg) != SGQA_OK || check_seqs(cfg, seqs, n_seqs) != SGQA_OK) return -1;
    const ForwardLayout fl = plan_forward(cfg, seqs, n_seqs, true);
    if (fl.pieces) return (int64_t)fl.diag_off;
    const IndexPlan p = plan_index(cfg, seqs, n_seqs);
    return p.diag_off > 0 ? (int64_t)p.diag_off : -1;
}

size_t sgqa_workspace_size(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           int32_t op) {
    if (check_config(cfg) != SGQA_OK || check_seqs(cfg, seqs, n_seqs) != SGQA_OK) return 0;
    switch (op) {
        case SGQA_OP_COMPRESS: return 0;
        case SGQA_OP_INDEX_TOPK: return plan_index(cfg, seqs, n_seqs).ws;
        case SGQA_OP_SPARSE_ATTN: return plan_attn(cfg, seqs, n_seqs).ws;
        case SGQA_OP_FORWARD: return plan_forward(cfg, seqs, n_seqs, true).ws;
        default: fail(SGQA_ERR_CONFIG, "unknown op %d", op); return 0;
    }
}

int sgqa_compress(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                  const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                  const void* ln_beta, void* store, void* ws, size_t ws_bytes,
                  void* hip_stream) {
    (void)ws;
    (void)ws_bytes;
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!proxy_k || !comp_logits || !store)
        return fail(SGQA_ERR_NULL, "proxy_k, comp_logits and store are required");
    if ((rc = check_aligned({{proxy_k, "proxy_k"}, {comp_logits, "comp_logits"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}}))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_compress(cfg, seqs, n_seqs, proxy_k, comp_logits, Paging(), ln_gamma, ln_beta, store,
                        (hipStream_t)hip_stream);
}

int sgqa_compress_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                        const void* proxy_pages, const float* logit_pages, const int32_t* page_table,
                        int64_t page_table_len, int64_t n_pages, const void* ln_gamma,
                        const void* ln_beta, void* store, void* ws, size_t ws_bytes,
                        void* hip_stream) {
    (void)ws;
    (void)ws_bytes;
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!proxy_pages || !logit_pages || !store)
        return fail(SGQA_ERR_NULL, "proxy_pages, logit_pages and store are required");
    if ((rc = check_aligned({{proxy_pages, "proxy_pages"}, {logit_pages, "logit_pages"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}}))) return rc;
    if ((rc = check_paging(seqs, n_seqs, page_table, page_table_len, n_pages))) return rc;
    Paging pg;
    pg.table = page_table;
    pg.n_pages = n_pages;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_compress(cfg, seqs, n_seqs, proxy_pages, logit_pages, pg, ln_gamma, ln_beta, store,
                        (hipStream_t)hip_stream);
}

int sgqa_index_topk(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                    const void* q_idx, const float* w, const void* rms_gamma,
                    const void* store, int32_t* sel, float* sel_scores, void* q_hat_out,
                    void* ws, size_t ws_bytes, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!q_idx || !w || !store || !sel)
        return fail(SGQA_ERR_NULL, "q_idx, w, store and sel are required");
    if ((rc = check_aligned({{q_idx, "q_idx"}, {w, "w"}, {rms_gamma, "rms_gamma"}, {store, "store"}, {sel, "sel"}, {sel_scores, "sel_scores"}, {q_hat_out, "q_hat_out"}}))) return rc;
    const IndexPlan p = plan_index(cfg, seqs, n_seqs);
    if ((rc = check_ws(p.ws, ws, ws_bytes))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_index(cfg, seqs, n_seqs, p, q_idx, w, rms_gamma, store, sel, sel_scores,
                     q_hat_out, ws, (hipStream_t)hip_stream);
}

int sgqa_sparse_attn(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                     const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* sel, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if ((rc = check_gather_rows(seqs, n_seqs))) return rc;
    if (!q || !k_cache || !v_cache || !sel || !out)
        return fail(SGQA_ERR_NULL, "q, k_cache, v_cache, sel and out are required");
    if ((rc = check_aligned({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {sel, "sel"}, {out, "out"}, {lse, "lse"}}))) return rc;
    const AttnPlan p = plan_attn(cfg, seqs, n_seqs);
    if ((rc = check_ws(p.ws, ws, ws_bytes))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_attn(cfg, seqs, n_seqs, p, q, k_cache, v_cache, Paging(), sel, out, lse, nullptr, ws,
                    (hipStream_t)hip_stream);
}

int sgqa_sparse_attn_gated(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           const void* q, const void* k_cache, const void* v_cache, const int32_t* sel,
                           void* out, float* lse, const void* gate, void* ws, size_t ws_bytes,
                           void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if ((rc = check_gather_rows(seqs, n_seqs))) return rc;
    if (!q || !k_cache || !v_cache || !sel || !out || !gate)
        return fail(SGQA_ERR_NULL, "q, k_cache, v_cache, sel, out and gate are required");
    if ((rc = check_aligned({{q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {sel, "sel"}, {out, "out"}, {lse, "lse"}, {gate, "gate"}}))) return rc;
    const AttnPlan p = plan_attn(cfg, seqs, n_seqs);
    if ((rc = check_ws(p.ws, ws, ws_bytes))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_attn(cfg, seqs, n_seqs, p, q, k_cache, v_cache, Paging(), sel, out, lse, gate, ws,
                    (hipStream_t)hip_stream);
}

int sgqa_sparse_attn_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* page_table, int64_t page_table_len, int64_t n_pages,
                           const int32_t* sel, void* out, float* lse, const void* gate, void* ws,
                           size_t ws_bytes, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!q || !k_pages || !v_pages || !sel || !out)
        return fail(SGQA_ERR_NULL, "q, k_pages, v_pages, sel and out are required");
    if ((rc = check_aligned({{q, "q"}, {k_pages, "k_pages"}, {v_pages, "v_pages"}, {sel, "sel"}, {out, "out"}, {lse, "lse"}, {gate, "gate"}}))) return rc;
    if ((rc = check_paging(seqs, n_seqs, page_table, page_table_len, n_pages))) return rc;
    const AttnPlan p = plan_attn(cfg, seqs, n_seqs);
    if ((rc = check_ws(p.ws, ws, ws_bytes))) return rc;
    Paging pg;
    pg.table = page_table;
    pg.n_pages = n_pages;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_attn(cfg, seqs, n_seqs, p, q, k_pages, v_pages, pg, sel, out, lse, gate, ws,
                    (hipStream_t)hip_stream);
}

int sgqa_forward(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                 const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                 const void* ln_beta, void* store, const void* q_idx, const float* w,
                 const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                 const void* k_cache, const void* v_cache, void* out, float* lse, void* ws,
                 size_t ws_bytes, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if ((rc = check_gather_rows(seqs, n_seqs))) return rc;
    if (!proxy_k || !comp_logits || !store || !q_idx || !w || !sel || !q || !k_cache ||
        !v_cache || !out)
        return fail(SGQA_ERR_NULL,
                    "proxy_k, comp_logits, store, q_idx, w, sel, q, k_cache, v_cache and out "
                    "are required");
    if ((rc = check_aligned({{proxy_k, "proxy_k"}, {comp_logits, "comp_logits"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}, {q_idx, "q_idx"}, {w, "w"}, {rms_gamma, "rms_gamma"}, {sel, "sel"}, {sel_scores, "sel_scores"}, {q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {out, "out"}, {lse, "lse"}}))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_forward(cfg, seqs, n_seqs, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                       rms_gamma, sel, sel_scores, q, k_cache, v_cache, Paging(), out, lse, nullptr, ws,
                       ws_bytes, (hipStream_t)hip_stream);
}

int sgqa_forward_noalloc(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                         const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                         const void* ln_beta, void* store, const void* q_idx, const float* w,
                         const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                         const void* k_cache, const void* v_cache, void* out, float* lse,
                         void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if ((rc = check_gather_rows(seqs, n_seqs))) return rc;
    if (!proxy_k || !comp_logits || !store || !q_idx || !w || !sel || !q || !k_cache ||
        !v_cache || !out)
        return fail(SGQA_ERR_NULL,
                    "proxy_k, comp_logits, store, q_idx, w, sel, q, k_cache, v_cache and out "
                    "are required");
    if ((rc = check_aligned({{proxy_k, "proxy_k"}, {comp_logits, "comp_logits"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}, {q_idx, "q_idx"}, {w, "w"}, {rms_gamma, "rms_gamma"}, {sel, "sel"}, {sel_scores, "sel_scores"}, {q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {out, "out"}, {lse, "lse"}}))) return rc;
    // one stream: no pieces (the side stream would be created on first use)
    const size_t need = plan_forward(cfg, seqs, n_seqs, false).ws;
    if (need > kNoAllocScratchBytes)
        return fail(SGQA_ERR_WORKSPACE,
                    "these sequences need %zu bytes of workspace; sgqa_forward_noalloc's static "
                    "scratch holds %zu (use sgqa_forward with a caller workspace)",
                    need, kNoAllocScratchBytes);
    void* ws = scratch_address(&rc);
    if (!ws) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_forward(cfg, seqs, n_seqs, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                       rms_gamma, sel, sel_scores, q, k_cache, v_cache, Paging(), out, lse, nullptr, ws,
                       kNoAllocScratchBytes, (hipStream_t)hip_stream, false);
}

int sgqa_forward_gated(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                       const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                       const void* ln_beta, void* store, const void* q_idx, const float* w,
                       const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                       const void* k_cache, const void* v_cache, void* out, float* lse, const void* gate,
                       void* ws, size_t ws_bytes, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if ((rc = check_gather_rows(seqs, n_seqs))) return rc;
    if (!proxy_k || !comp_logits || !store || !q_idx || !w || !sel || !q || !k_cache ||
        !v_cache || !out || !gate)
        return fail(SGQA_ERR_NULL,
                    "proxy_k, comp_logits, store, q_idx, w, sel, q, k_cache, v_cache, out and gate "
                    "are required");
    if ((rc = check_aligned({{proxy_k, "proxy_k"}, {comp_logits, "comp_logits"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}, {q_idx, "q_idx"}, {w, "w"}, {rms_gamma, "rms_gamma"}, {sel, "sel"}, {sel_scores, "sel_scores"}, {q, "q"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {out, "out"}, {lse, "lse"}, {gate, "gate"}}))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_forward(cfg, seqs, n_seqs, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                       rms_gamma, sel, sel_scores, q, k_cache, v_cache, Paging(), out, lse, gate, ws,
                       ws_bytes, (hipStream_t)hip_stream);
}

int sgqa_forward_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                       const void* proxy_pages, const float* logit_pages, const void* ln_gamma,
                       const void* ln_beta, void* store, const void* q_idx, const float* w,
                       const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                       const void* k_pages, const void* v_pages, const int32_t* page_table,
                       int64_t page_table_len, int64_t n_pages, void* out, float* lse,
                       const void* gate, void* ws, size_t ws_bytes, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!proxy_pages || !logit_pages || !store || !q_idx || !w || !sel || !q || !k_pages ||
        !v_pages || !out)
        return fail(SGQA_ERR_NULL,
                    "proxy_pages, logit_pages, store, q_idx, w, sel, q, k_pages, v_pages and out "
                    "are required");
    if ((rc = check_aligned({{proxy_pages, "proxy_pages"}, {logit_pages, "logit_pages"}, {ln_gamma, "ln_gamma"}, {ln_beta, "ln_beta"}, {store, "store"}, {q_idx, "q_idx"}, {w, "w"}, {rms_gamma, "rms_gamma"}, {sel, "sel"}, {sel_scores, "sel_scores"}, {q, "q"}, {k_pages, "k_pages"}, {v_pages, "v_pages"}, {out, "out"}, {lse, "lse"}, {gate, "gate"}}))) return rc;
    if ((rc = check_paging(seqs, n_seqs, page_table, page_table_len, n_pages))) return rc;
    Paging pg;
    pg.table = page_table;
    pg.n_pages = n_pages;
    if ((rc = check_stream(hip_stream))) return rc;
    return run_forward(cfg, seqs, n_seqs, proxy_pages, logit_pages, ln_gamma, ln_beta, store, q_idx, w,
                       rms_gamma, sel, sel_scores, q, k_pages, v_pages, pg, out, lse, gate, ws, ws_bytes,
                       (hipStream_t)hip_stream);
}

int sgqa_qk_prep(const sgqa_config* cfg, const sgqa_qk_config* qk, const sgqa_seq* seqs, int32_t n_seqs,
                 const void* q_raw, const void* k_raw, const void* v_raw, const void* q_gamma,
                 const void* k_gamma, void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                 int64_t page_table_len, int64_t n_pages, void* hip_stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!qk) return fail(SGQA_ERR_NULL, "qk is NULL");
    if (qk->rope_dim < 0 || qk->rope_dim > cfg->head_dim || qk->rope_dim % 2 != 0)
        return fail(SGQA_ERR_CONFIG, "qk rope_dim %d must be even and in [0, %d]", qk->rope_dim,
                    cfg->head_dim);
    if (!(isfinite(qk->rope_base) && qk->rope_base > 0.f) || !(isfinite(qk->eps) && qk->eps >= 0.f))
        return fail(SGQA_ERR_CONFIG, "qk rope_base must be finite and positive, eps finite and >= 0");
    if ((rc = check_seqs(cfg, seqs, n_seqs))) return rc;
    if (!q_raw || !k_raw || !q_out || !k_cache)
        return fail(SGQA_ERR_NULL, "q_raw, k_raw, q_out and k_cache are required");
    if ((v_raw == nullptr) != (v_cache == nullptr))
        return fail(SGQA_ERR_NULL, "v_raw and v_cache go together");
    if ((rc = check_aligned({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {q_gamma, "q_gamma"}, {k_gamma, "k_gamma"}, {q_out, "q_out"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}}))) return rc;
    if (page_table && (rc = check_paging(seqs, n_seqs, page_table, page_table_len, n_pages))) return rc;
    if ((rc = check_stream(hip_stream))) return rc;
    sgqa::QkPrepArgs a;
    a.q_raw = (const uint16_t*)q_raw;
    a.k_raw = (const uint16_t*)k_raw;
    a.v_raw = (const uint16_t*)v_raw;
    a.q_gamma = (const uint16_t*)q_gamma;
    a.k_gamma = (const uint16_t*)k_gamma;
    a.q_out = (uint16_t*)q_out;
    a.k_cache = (uint16_t*)k_cache;
    a.v_cache = (uint16_t*)v_cache;
    a.page_table = page_table;
    a.n_pages = page_table ? n_pages : 0;
    a.log_base = log((double)qk->rope_base);
    a.rope_dim = qk->rope_dim;
    a.eps = qk->eps;
    for (int32_t first = 0; first < n_seqs; first += sgqa::kMaxSeqsPerLaunch) {
        const int32_t cnt = std::min<int32_t>(sgqa::kMaxSeqsPerLaunch, n_seqs - first);
        sgqa::SeqTable tab;
        const int64_t mx = fill_table(tab, seqs, first, cnt, [](const sgqa_seq& q) { return q.n_q; });
        if (tab.n == 0) continue;
        hipError_t e = sgqa::launch_qk_prep(tab, mx, a, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(e, "qk_prep launch");
    }
    return SGQA_OK;
}

}  // extern "C"
