/*
 * sgqa.h -- C ABI of the sparse GQA global-attention library (libsgqa.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The library computes, for one attention layer, the four steps of
 * Step-5-Preview's sparse global attention as described on the page
 * "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache":
 *
 *   1. sgqa_compress    block-wise token merging of proxy keys into the
 *                       compressed store (section "Eight tokens become one
 *                       search key, coordinate by coordinate");
 *   2.+3. sgqa_index_topk  weighted-ReLU indexer scores per KV group and the
 *                       causal top-k block selection (section "Selection is a
 *                       weighted ReLU score, not attention softmax");
 *   4. sgqa_sparse_attn GQA attention of each group's 16 query heads over the
 *                       original K/V of the selected blocks plus the current
 *                       block (section "Main attention still reads original
 *                       K/V");
 *   sgqa_forward        1 -> 2+3 -> 4 on one stream.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor pointer is a DEVICE pointer to memory the caller
 *           owns (allocated e.g. by PyTorch); the library never allocates,
 *           frees or synchronises.  Tensors are dense, row-major, without
 *           padding, and start at a 16-byte aligned address (every torch
 *           allocation does; a misaligned pointer returns SGQA_ERR_SHAPE).
 *           bf16 is the 16-bit brain-float bit pattern.  Scratch
 *           memory comes from the caller as (ws, ws_bytes) of at least
 *           sgqa_workspace_size(...) bytes, 256-byte aligned; ws may be NULL
 *           when that size is 0.  Workspace contents need no initialisation
 *           and are meaningless after the call.
 * Streams.  Work is enqueued on hip_stream (a hipStream_t; NULL = the null
 *           stream) and returns before it completes.  Buffers must stay alive
 *           until the stream reaches the end of the call's work.  hip_stream
 *           must belong to the calling thread's current device (kernel
 *           attributes and the library's per-device state follow the current
 *           device); a stream of another device returns SGQA_ERR_CONFIG
 *           before any work is enqueued.
 * Sequences. A call processes n_seqs >= 1 independent sequences described by
 *           a HOST array of sgqa_seq.  Query-side tensors are packed over all
 *           sequences (rows q_offset .. q_offset+n_q-1 belong to a sequence);
 *           cache-side tensors hold each sequence at its own row offset.
 *           Positions are zero-based; query i of a sequence sits at position
 *           pos0 + i and cache_len == pos0 + n_q (the new tokens' K/V, proxy
 *           keys and compression logits are already written into the caches).
 * Errors.   Every check of arguments, shapes and descriptors runs on the host
 *           before any work is enqueued (the only HIP calls before that are
 *           device and stream queries), so a rejected call has enqueued
 *           nothing and touched no memory.  Entry points return SGQA_OK (0) or a
 *           negative sgqa_status; sgqa_last_error() then holds a message for
 *           the calling thread.  A failing HIP launch returns SGQA_ERR_HIP
 *           (work enqueued before it may still run).  Nothing aborts and no
 *           C++ exception crosses this boundary.
 * Threads.  Calls are re-entrant; concurrent calls must not write the same
 *           output or workspace memory.
 * Results.  Deterministic: identical inputs and arguments give bit-identical
 *           outputs.
 */
#ifndef SGQA_H
#define SGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sgqa_status {
    SGQA_OK = 0,
    SGQA_ERR_NULL = -1,        /* a required pointer is NULL                          */
    SGQA_ERR_CONFIG = -2,      /* inconsistent or out-of-range sgqa_config field      */
    SGQA_ERR_SHAPE = -3,       /* bad sequence descriptor, or a misaligned tensor     */
    SGQA_ERR_CAUSAL = -4,      /* cache_len != pos0 + n_q                             */
    SGQA_ERR_CAPACITY = -5,    /* cache_len exceeds kv_capacity, or store too small  */
    SGQA_ERR_WORKSPACE = -6,   /* ws_bytes below sgqa_workspace_size, or misaligned  */
    SGQA_ERR_UNSUPPORTED = -7, /* valid but outside the compiled shape set           */
    SGQA_ERR_HIP = -8          /* a HIP runtime call failed                          */
} sgqa_status;

/*
 * Layer configuration.  The compiled shape set is the one the page describes
 * for Step-5-Preview's global layers (section "Two paths leave the same hidden
 * state"): num_q_heads 64 in num_kv_groups 4 (16 heads per group), head_dim
 * 192, idx_heads 4 indexer heads per group of idx_dim 128, rope_dim 32 (even,
 * <= idx_dim).  block_size B is 1, 2, 4, 8 or 16 (8 on the page; 1 in the
 * architecture blog's ablation); topk_blocks K is 1..3072 (512 on the page:
 * 4,096 tokens at B=8).  Other values are SGQA_ERR_UNSUPPORTED.
 */
typedef struct sgqa_config {
    int32_t num_q_heads;   /* H: query heads (64)                                   */
    int32_t num_kv_groups; /* G: KV groups; head h uses group h / (H/G)  (4)        */
    int32_t head_dim;      /* D: main Q/K/V head dim (192)                          */
    int32_t idx_heads;     /* indexer heads per group (4)                           */
    int32_t idx_dim;       /* indexer query / proxy-key dim (128)                   */
    int32_t rope_dim;      /* indexer rotary span: dims [0, rope_dim) (32)          */
    float rope_base;       /* rotary base (10000)                                   */
    int32_t block_size;    /* B: tokens merged per summary (8)                      */
    int32_t topk_blocks;   /* K: historical blocks kept per query and group (512)   */
    float softmax_scale;   /* main attention logit scale (1/sqrt(192))              */
    float eps_rms;         /* RMSNorm epsilon of the indexer queries (1e-6)         */
    float eps_ln;          /* LayerNorm epsilon of the proxy keys (1e-6)            */
    int32_t store_q8;      /* 1: round summaries fp32 -> bf16 -> E4M3 (held as bf16
                              values); 2: the same E4M3 values held as OCP E4M3FN
                              codes, one byte each (a uint8 store, half the bytes
                              the scorers stream; the scores are bit-identical to
                              those of 1); 0: round to bf16 only                    */
} sgqa_config;

/* One sequence of a call.  All fields are validated on the host. */
typedef struct sgqa_seq {
    int64_t q_offset;       /* first row of this sequence in the packed query-side
                               tensors (q, q_idx, w, out, lse, sel, ...)             */
    int64_t n_q;            /* new query tokens (>= 0)                              */
    int64_t pos0;           /* position of the first new token                      */
    int64_t cache_len;      /* tokens cached, new ones included; == pos0 + n_q     */
    int64_t kv_offset;      /* row of position 0 in k_cache / v_cache / proxy_k /
                               comp_logits                                          */
    int64_t kv_capacity;    /* rows reserved from kv_offset; >= cache_len           */
    int64_t store_offset;   /* row of block 0 in the store                          */
    int64_t store_capacity; /* store rows reserved; >= cache_len / block_size       */
} sgqa_seq;

/* Operation codes for sgqa_workspace_size. */
enum {
    SGQA_OP_COMPRESS = 0,
    SGQA_OP_INDEX_TOPK = 1,
    SGQA_OP_SPARSE_ATTN = 2,
    SGQA_OP_FORWARD = 3
};

/*
 * Bytes of workspace the operation needs for these arguments (0 when none),
 * or 0 with sgqa_last_error() set when the arguments are invalid.  What it
 * holds: for SGQA_OP_INDEX_TOPK, the 4-byte score keys of every candidate of
 * the queries processed at once -- calls of 1024+ queries work in passes of
 * at most 4 GiB of keys and also hold each query's prepared indexer rows
 * (4 KiB per query of a pass), smaller calls with long histories keep the queries
 * of 64 consecutive seqs[] entries at a time (at most 1 GiB, else they need
 * none); for SGQA_OP_SPARSE_ATTN, the per-split partial outputs of calls
 * whose queries are spread over several workgroups (decode-sized calls), for
 * 64 consecutive seqs[] entries at a time.  The size depends on the entries'
 * n_q, pos0 and order, not on their q_offset.  SGQA_OP_FORWARD needs the
 * larger of the two (the steps run one after the other), except for calls
 * sgqa_forward runs in pieces (see there): those hold the pieces' index
 * region, then their attention region, then one 256-byte diagnostics block.
 */
size_t sgqa_workspace_size(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           int32_t op);

/*
 * Diagnostics of the index step (for checking and monitoring).  Calls whose
 * index step works in the tiled mode (1024 or more queries) keep, in their
 * workspace at the byte offset returned here, a block of 64 uint32 words:
 *   [0]  the number of (query, group) rows whose candidate lists could not
 *        give the exact top k and were scored again over every candidate;
 *   [1]  reserved (0);
 *   [2 + 2j], [3 + 2j]  for j < min([0], 31): query row (q_offset + index in
 *        the sequence, low 32 bits) and group of the j-th such row (in the
 *        order the device found them).
 * The block is cleared at the start of the call's index step and written by
 * its kernels; the attention of the same sgqa_forward call leaves it alone
 * (calls of that size never split their attention).  Returns -1, with no
 * block kept, when the index step of these arguments does not use the tiled
 * mode or the arguments are invalid (sgqa_last_error() says which).  The
 * offset is for sgqa_index_topk workspaces; sgqa_forward_diag_offset gives
 * it for sgqa_forward's.
 */
int64_t sgqa_index_diag_offset(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs);

/*
 * The same diagnostics block in an sgqa_forward workspace: for calls run in
 * pieces, one block at the end of the workspace that every piece's index
 * step adds to (cleared by the first); otherwise the offset
 * sgqa_index_diag_offset gives.  -1 as there.
 */
int64_t sgqa_forward_diag_offset(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs);

/*
 * Step 1 -- block-wise token merging (page section "Eight tokens become one
 * search key, coordinate by coordinate"; norms and rotary span from section
 * "Two paths leave the same hidden state").
 *
 * For every sequence, every block r with floor(pos0/B) <= r < floor(cache_len/B)
 * (the blocks completed by the new tokens) gets
 *   k_hat[s]   = RoPE_s(LayerNorm(proxy_k[s]) * ln_gamma + ln_beta)  per token s,
 *   store[r,d] = sum_j softmax_j(comp_logits[B r + j, d]) * k_hat[B r + j, d],
 * the softmax over the block's B tokens per coordinate d with its maximum
 * subtracted, accumulated in fp32, then rounded to bf16 (and from bf16 to
 * E4M3 when cfg->store_q8).  Rows [B*floor(pos0/B), cache_len) of proxy_k /
 * comp_logits must hold valid data (the incomplete-block buffer of earlier
 * calls is the caller's rows).  Other store rows are left untouched.
 *
 *   proxy_k      bf16 [rows, idx_dim]   raw proxy keys, row kv_offset + s
 *   comp_logits  fp32 [rows, idx_dim]   compression logits, same rows
 *   ln_gamma     bf16 [idx_dim] or NULL (= 1)
 *   ln_beta      bf16 [idx_dim] or NULL (= 0)
 *   store        bf16 [store_rows, idx_dim], row store_offset + r  (written);
 *                uint8 E4M3 codes, same shape, when cfg->store_q8 == 2
 */
int sgqa_compress(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                  const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                  const void* ln_beta, void* store, void* ws, size_t ws_bytes,
                  void* hip_stream);

/*
 * Steps 2 and 3 -- indexer scores and causal top-k (page section "Selection is
 * a weighted ReLU score, not attention softmax").
 *
 * For query position t and group g (4 groups share one store):
 *   q_hat[t,g,i] = bf16(RoPE_t(RMSNorm(q_idx[t,g,i]) * rms_gamma)),  i < idx_heads
 *   s[t,g,r]     = sum_i w[t,g,i] * max(0, q_hat[t,g,i] . store[r])   (fp32)
 * for the candidates r < floor(t/B).  sel[t,g,:] receives the K candidates
 * with the largest s (equal scores, -0 == +0, go to the lower r), or all
 * candidates when there are at most K, in ascending r, padded with -1.  The
 * current block floor(t/B) is never listed; attention appends it.
 * Store rows 0 .. floor((cache_len-1)/B)-1 of each sequence must be written.
 *
 *   q_idx       bf16 [Nq, G, idx_heads, idx_dim]   raw indexer queries
 *   w           fp32 [Nq, G, idx_heads]            signed head weights
 *   rms_gamma   bf16 [idx_dim] or NULL (= 1)
 *   store       bf16 [store_rows, idx_dim] (uint8 E4M3 codes when
 *               cfg->store_q8 == 2)
 *   sel         int32 [Nq, G, K]                   (written)
 *   sel_scores  fp32 [Nq, G, K] or NULL: s of each listed block, 0 at padding
 *   q_hat_out   bf16 [Nq, G, idx_heads, idx_dim] or NULL: q_hat (for checking)
 * Nq = max over sequences of q_offset + n_q.
 */
int sgqa_index_topk(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                    const void* q_idx, const float* w, const void* rms_gamma,
                    const void* store, int32_t* sel, float* sel_scores, void* q_hat_out,
                    void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Step 4 -- sparse GQA attention (page sections "Main attention still reads
 * original K/V" and "What gets cheaper, and what stays length-dependent?").
 *
 * Query t, head h, group g = h / (H/G) attends over
 *   U = { B*r + j : r in sel[t,g,:], r >= 0, j < B } U { B*floor(t/B) .. t }
 * (at most K*B + B positions) with an exact softmax:
 *   out[t,h] = sum_{u in U} softmax_u(softmax_scale * q[t,h] . k_cache[u,g]) v_cache[u,g]
 *   lse[t,h] = log sum_{u in U} exp(softmax_scale * q[t,h] . k_cache[u,g])
 * Listed ids must satisfy 0 <= r < floor(t/B) (as sgqa_index_topk writes them);
 * entries after the first -1 are ignored.
 *
 *   q        bf16 [Nq, H, D]
 *   k_cache  bf16 [rows, G, D], v_cache bf16 [rows, G, D]  (row kv_offset + position);
 *            a sequence's kv_capacity must be at most 2,796,202 rows
 *            (SGQA_ERR_UNSUPPORTED otherwise; the paged calls have no such limit)
 *   sel      int32 [Nq, G, K]
 *   out      bf16 [Nq, H, D]    (written)
 *   lse      fp32 [Nq, H] or NULL (natural log)
 */
int sgqa_sparse_attn(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                     const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* sel, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* hip_stream);

/*
 * Steps 1 -> 2+3 -> 4: sgqa_compress, sgqa_index_topk, sgqa_sparse_attn with
 * the arguments above (sel is written and then read), ordered on hip_stream.
 * ws_bytes must be at least sgqa_workspace_size(..., SGQA_OP_FORWARD).
 *
 * Decode-shaped calls (the index step scores with per-query wavefronts and
 * every sequence's queries lie inside one block, e.g. one new token per
 * sequence) read none of the blocks they complete, so step 1 runs inside the
 * index step's scoring launch instead of a launch of its own; the store rows
 * written are the same.
 *
 * Calls of at least 2048 queries whose index step works in the tiled mode and
 * whose gather attention takes at least 1024 of them (long histories, e.g. a
 * prefill chunk over a 1M-token cache or a 64K-token prefill) run in pieces
 * of at least 1024 queries, when cutting them into pieces leaves every
 * query's attention kernel and the gather's ranges unchanged: each piece's
 * index step on hip_stream, its attention on a second
 * stream of the same device that the library creates on the device's first
 * such call (default priority, kept until the process ends), after an event
 * recorded behind that index step -- so a piece's attention overlaps the next
 * piece's index step.  hip_stream then waits for the second stream, so work
 * the caller puts on hip_stream later, and an event the caller records there,
 * come after the whole call, and HIP graph capture of hip_stream captures
 * both streams.  The outputs equal those of the three calls above run in
 * order.  Concurrent calls from several host threads on one device are
 * serialised while they queue their work.
 */
int sgqa_forward(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                 const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                 const void* ln_beta, void* store, const void* q_idx, const float* w,
                 const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                 const void* k_cache, const void* v_cache, void* out, float* lse, void* ws,
                 size_t ws_bytes, void* hip_stream);

/*
 * sgqa_forward for callers that cannot allocate memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation: the
 * same three steps with the same arguments and results, but the workspace is
 * a static 64 MiB device array inside the library (one per GPU, held until
 * the process ends) instead of a caller buffer.  No memory is allocated or
 * freed by the call.  Calls whose workspace (sgqa_workspace_size(...,
 * SGQA_OP_FORWARD)) exceeds 64 MiB return SGQA_ERR_WORKSPACE before any HIP
 * call; decode-sized calls (e.g. 64 sequences of up to 262,144 cached tokens)
 * fit.  All calls on one GPU share its array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  The first call on each
 * device resolves that device's copy (hipGetSymbolAddress) with it current.
 */
int sgqa_forward_noalloc(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                         const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                         const void* ln_beta, void* store, const void* q_idx, const float* w,
                         const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                         const void* k_cache, const void* v_cache, void* out, float* lse,
                         void* hip_stream);

/*
 * Paged caches (page section "Cache capacity: 4,104 reads do not mean 4,104
 * stored tokens": global capacity rounded up to 16-token pages, with page
 * tables).  The per-token tensors live in a pool of n_pages pages of 16
 * positions each:
 *   k_pages, v_pages       bf16 [n_pages, 16, G, D]
 *   proxy_pages            bf16 [n_pages, 16, Di]
 *   logit_pages            fp32 [n_pages, 16, Di]
 * page_table: int32 [page_table_len], device memory, owned by the caller.
 * For a sequence, kv_offset is the index in page_table of its logical page 0:
 * position u lives in physical page page_table[kv_offset + u / 16], slot
 * u % 16 (the same table serves all four tensors).  kv_capacity (tokens) must
 * satisfy kv_offset + ceil(kv_capacity / 16) <= page_table_len, else
 * SGQA_ERR_CAPACITY; n_pages must be at most 2^27.  Page ids are read on the
 * device only: an id outside [0, n_pages) is clamped into the pool, so it never
 * reads outside it (the results are then meaningless).  A block never
 * straddles two pages (B divides 16).  The store, queries, selections and
 * outputs keep the layouts above, and the results equal those of the
 * contiguous calls for the same logical contents.  Workspace: as the
 * corresponding contiguous call (sgqa_workspace_size with SGQA_OP_COMPRESS,
 * SGQA_OP_SPARSE_ATTN or SGQA_OP_FORWARD).
 */
int sgqa_compress_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                        const void* proxy_pages, const float* logit_pages, const int32_t* page_table,
                        int64_t page_table_len, int64_t n_pages, const void* ln_gamma,
                        const void* ln_beta, void* store, void* ws, size_t ws_bytes,
                        void* hip_stream);

int sgqa_sparse_attn_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* page_table, int64_t page_table_len, int64_t n_pages,
                           const int32_t* sel, void* out, float* lse, const void* gate, void* ws,
                           size_t ws_bytes, void* hip_stream);

int sgqa_forward_paged(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                       const void* proxy_pages, const float* logit_pages, const void* ln_gamma,
                       const void* ln_beta, void* store, const void* q_idx, const float* w,
                       const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                       const void* k_pages, const void* v_pages, const int32_t* page_table,
                       int64_t page_table_len, int64_t n_pages, void* out, float* lse,
                       const void* gate, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * The neighbours of the path, fused into it (page sections "Two paths leave
 * the same hidden state" and "Main attention still reads original K/V").
 *
 * Output gate: each head's output vector is sigmoid-gated before the heads
 * are concatenated; here elementwise,
 *   out[t,h,d] = bf16( o[t,h,d] * 1 / (1 + exp(-gate[t,h,d])) )
 * with o the attention result of sgqa_sparse_attn in fp32 and gate bf16
 * [Nq, H, D] logits from the caller (the projection needs trained weights),
 * applied in the attention kernels before rounding; lse is the attention's,
 * unchanged.  The _paged entry points above take the same gate (NULL: no
 * gate).  Everything else as sgqa_sparse_attn / sgqa_forward.
 */
int sgqa_sparse_attn_gated(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                           const void* q, const void* k_cache, const void* v_cache, const int32_t* sel,
                           void* out, float* lse, const void* gate, void* ws, size_t ws_bytes,
                           void* hip_stream);

int sgqa_forward_gated(const sgqa_config* cfg, const sgqa_seq* seqs, int32_t n_seqs,
                       const void* proxy_k, const float* comp_logits, const void* ln_gamma,
                       const void* ln_beta, void* store, const void* q_idx, const float* w,
                       const void* rms_gamma, int32_t* sel, float* sel_scores, const void* q,
                       const void* k_cache, const void* v_cache, void* out, float* lse, const void* gate,
                       void* ws, size_t ws_bytes, void* hip_stream);

/* Main-path Q/K producer parameters (sgqa_qk_prep). */
typedef struct {
    int32_t rope_dim;   /* rotary span of the main Q/K: even, 0 .. head_dim       */
    float rope_base;    /* finite, > 0                                            */
    float eps;          /* RMSNorm epsilon, finite, >= 0                          */
    int32_t reserved;   /* 0                                                      */
} sgqa_qk_config;

/*
 * Main-path Q/K producer: the main path normalizes Q and K and applies the
 * layer's partial rotary span (its width is head_dim times a partial-rotary
 * factor the page names but does not give: rope_dim and rope_base are the
 * caller's).  For every new token t of each sequence (rows as in the calls
 * above: q rows at q_offset, cache rows at kv_offset + t, or through
 * page_table when it is not NULL, with the paged checks above):
 *   q_out[t, h]   = bf16(RoPE_t(RMSNorm(q_raw[t, h]) * q_gamma))    h < H
 *   k_cache[t, g] = bf16(RoPE_t(RMSNorm(k_raw[t, g]) * k_gamma))    g < G
 *   v_cache[t, g] = v_raw[t, g]               (when v_raw is not NULL)
 * RMSNorm over each head's D dims with one gamma [D] per tensor (NULL: 1),
 * epsilon qk->eps, fp32; RoPE_t rotates pairs (j, j + rope_dim/2) of dims
 * [0, rope_dim) by t * rope_base^(-2j/rope_dim) (the indexer's convention).
 * q_raw bf16 [Nq, H, D], k_raw / v_raw bf16 [Nq, G, D], q_out bf16 [Nq, H, D].
 * v_raw and v_cache are both NULL or both set.  No workspace.
 */
int sgqa_qk_prep(const sgqa_config* cfg, const sgqa_qk_config* qk, const sgqa_seq* seqs, int32_t n_seqs,
                 const void* q_raw, const void* k_raw, const void* v_raw, const void* q_gamma,
                 const void* k_gamma, void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                 int64_t page_table_len, int64_t n_pages, void* hip_stream);

/* Static name of a status code. */
const char* sgqa_status_string(int status);

/* Message of the calling thread's most recent failing call ("" if none). */
const char* sgqa_last_error(void);

/* Library ABI version, currently 1. */
int32_t sgqa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGQA_H */
