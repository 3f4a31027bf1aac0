/*
 * hysparse.h -- C ABI of the HySparse hybrid-block attention hot path on AMD
 * MI355X (gfx950).
 *
 * A hybrid block is one full causal attention layer followed by N sparse
 * layers (HySparse paper, section 3.1 "HySparse Overview"; explainer page
 * section 3.2 "Big-Picture Architecture").  The full layer computes ordinary
 * causal GQA attention and, in the same pass, per-64-token-block scores
 * (explainer section 3.4.1, "Block-Level Max Attention Scores" and "Modified
 * FlashAttention Kernel"; paper section 3.2).  The scores are normalised,
 * reduced over the query heads of each GQA group and turned into a per-query
 * top-k block list (explainer 3.4.1 "Grouped-Query Attention (GQA)
 * Aggregation", 3.4.2 "TopK Block Selection").  Every sparse layer then
 * attends to those blocks of the full layer's own K/V plus a sliding window
 * of its own K'/V', and merges the two with sigmoid gates (explainer 3.4.3;
 * paper sections 3.1, 3.3).  Decode runs the same path for one new token per
 * sequence; the token-level variant of the HySparse2 explainer ("Precise
 * retrieval without a separate indexer") selects single tokens plus the
 * newest ones instead of blocks.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, densely packed in the layouts stated below (row-major, last
 *     index fastest).  The library never allocates or frees device memory;
 *     scratch space comes from a caller workspace of hs_workspace_size() bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is only enqueued; nothing synchronises the host.
 *   - Arguments are validated before anything is launched; on an error the
 *     call returns a non-zero hs_status, writes nothing, and hs_last_error()
 *     (thread-local) describes the problem.  HS_ERR_LAUNCH reports a failed
 *     kernel launch.
 *   - Query head h belongs to kv head floor(h / G), G = hq / hkv (contiguous
 *     GQA grouping).  G must be a power of two <= 32 (<= 16 for the sparse
 *     layers and for decode); head_dim is 64 or 128.
 *   - Value tensors use a block-major layout: each run of 64 consecutive
 *     positions of one kv head is stored as a [head_dim][64] tile, i.e. a
 *     value tensor is [batch][hkv][ceil(len/64)][head_dim][64].  The one
 *     exception is the fp8 value cache of token-level decode, which is
 *     position-major like the keys.  Key tensors are position-major
 *     [batch][hkv][len][head_dim].  Tail entries of the last value tile
 *     (positions >= len) are never used and may hold anything.
 *   - The softmax scale is shape.scale, or 1/sqrt(head_dim) when it is 0.
 */
#ifndef HYSPARSE_H
#define HYSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hs_status {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = 1, /* a null pointer, a bad size or a misaligned pointer */
  HS_ERR_UNSUPPORTED = 2, /* a valid but unimplemented combination            */
  HS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  HS_ERR_LAUNCH = 4       /* the HIP runtime refused a launch                 */
} hs_status;

typedef enum hs_dtype {
  HS_F32 = 0,      /* IEEE binary32                                   */
  HS_BF16 = 1,     /* bfloat16                                        */
  HS_FP8_E4M3 = 2  /* OCP fp8 e4m3fn codes (key/value caches only)    */
} hs_dtype;

/* flags of hs_full_attn_fwd_scores */
#define HS_SCORE_MAX 0 /* block score = max logit of the block (the pages' rule) */
#define HS_SCORE_LSE 1 /* block score = log-sum-exp of the block's logits        */
/* flags of hs_block_topk */
#define HS_SEL_FULLY_PAST 0   /* candidates j < floor(t/64)                      */
#define HS_SEL_INCLUDE_DIAG 2 /* candidates j <= floor(t/64) (diagonal clipped)  */

typedef struct hs_shape {
  size_t struct_size;     /* = sizeof(hs_shape); lets the struct grow          */
  int batch;              /* number of sequences                               */
  int q_len;              /* prefill: T (queries = keys = T); decode: 1        */
  int kv_len;             /* prefill: T; decode: cache capacity per sequence    */
  int hq, hkv, head_dim;  /* query heads, kv heads, head dimension (64|128)    */
  int dtype;              /* hs_dtype of queries/outputs (and K/V in prefill)  */
  int kv_dtype;           /* decode: hs_dtype of the caches; prefill: = dtype  */
  float scale;            /* softmax scale tau; 0 -> 1/sqrt(head_dim)          */
  const int32_t* kv_lens; /* decode: device [batch] context lengths L_b (the
                             query sits at position L_b-1), 1 <= L_b <= C; the
                             kernels hold a value outside [0, C] to that range
                             rather than read past the caches.  NULL = prefill */
  const float* kv_scale;  /* fp8 caches: device [2][hkv] scales (K, V); value
                             = decoded code * scale.  NULL otherwise           */
  /* fields below were appended; a caller whose struct_size stops before one
     of them is read as passing NULL there */
  const float* q_scale;   /* fp8 prefill: device [hq] scales of the queries (q
                             of the full layer, q_sp of a sparse layer)        */
  const float* swa_scale; /* fp8 prefill sparse layer: device [2][hkv] scales
                             of the window cache (k_swa, v_swa)               */
} hs_shape;

/*
 * Full causal attention layer with per-block scores in one pass
 * (explainer 3.4.1 eq. o_t and eq. S_t^i; "Modified FlashAttention Kernel",
 * first pass; paper 3.2).
 *
 * Prefill (kv_lens == NULL), T = q_len = kv_len, nblk = ceil(T/64):
 *   q  [batch][T][hq][head_dim]          dtype
 *   k  [batch][hkv][T][head_dim]         dtype
 *   v  [batch][hkv][nblk][head_dim][64]  dtype (block-major)
 *   o  [batch][T][hq][head_dim]          dtype (out; bf16 for fp8 inputs)
 *   lse     [batch][hq][T] fp32 (out): log sum_{i<=t} exp(tau q_t.k_i)
 *   blk_raw [batch][hq][T][nblk] fp32 (out): for j <= floor(t/64) only,
 *           HS_SCORE_MAX: max_{i in block j, i<=t} tau q_t.k_i
 *           HS_SCORE_LSE: log sum_{i in block j, i<=t} exp(tau q_t.k_i)
 *     Both are log-domain and independent of the row normaliser: the
 *     post-softmax score of the pages is exp(blk_raw - lse).  Entries
 *     j > floor(t/64) are not written.
 * Decode (kv_lens != NULL, q_len == 1), capacity C = kv_len (multiple of 64):
 *   q [batch][hq][head_dim] (dtype, bf16); k [batch][hkv][C][head_dim];
 *   block = 64: bf16 caches, v [batch][hkv][C/64][head_dim][64];
 *   block = 1 (token-level variant): fp8 e4m3 caches with kv_scale,
 *     v [batch][hkv][C][head_dim] (position-major);
 *   o [batch][hq][head_dim]; lse [batch][hq];
 *   blk_raw [batch][hq][C/block]: block = 64 gives block scores as above for
 *   j <= floor((L_b-1)/64); block = 1 gives every token's logit tau q.k_i for
 *   i < L_b.  Needs a workspace of hs_workspace_size(HS_FN_FULL_ATTN, ...)
 *   bytes (the split-K partial states).
 * `block` must be 64 in prefill and 64 or 1 in decode.
 * fp8 prefill (dtype = kv_dtype = HS_FP8_E4M3, head_dim 128, hq/hkv <= 16):
 *   q, k, v hold OCP e4m3 codes; the values are code * scale with
 *   shape.q_scale [hq] for the queries and shape.kv_scale [2][hkv] for the
 *   keys and values.  Logits are exact in fp32; the probabilities are
 *   rounded to e4m3 for the value product (lse and blk_raw are those of the
 *   exact logits).  o is bf16.
 */
hs_status hs_full_attn_fwd_scores(const hs_shape* shape, const void* q, const void* k,
                                  const void* v, void* o, float* lse, float* blk_raw,
                                  int block, int flags, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Finalisation, GQA group maximum and top-k selection
 * (explainer 3.4.1 "Modified FlashAttention Kernel" second pass, eq. S_g;
 * 3.4.2 "TopK Block Selection"; paper 3.2).
 *
 * For each query row t and group g:
 *   S_g[t][j] = max_{h in g} exp(blk_raw[h][t][j] - lse[h][t])
 * and idx receives the `topk` candidates with the largest S_g, ties to the
 * smaller index, written in ascending order and padded with -1 when there are
 * fewer candidates.  Candidates: j < floor(t/64) (HS_SEL_FULLY_PAST) or
 * j <= floor(t/64) (HS_SEL_INCLUDE_DIAG).
 * Prefill: blk_raw/lse as produced above; idx [batch][hkv][T][topk] int32;
 *   grp_score (nullable) [batch][hkv][T][nblk] fp32 receives S_g for
 *   j <= floor(t/64).
 * Decode, block = 64: t = L_b-1, idx [batch][hkv][topk].
 * Decode, block = 1 (token mode): candidates are the tokens i < L_b-n_recent;
 *   the n_recent newest tokens are always added and do not count against
 *   topk; idx [batch][hkv][topk+n_recent] holds token ids, ascending, -1
 *   padded.  grp_score (nullable) [batch][hkv][C] receives S_g for i < L_b.
 * topk is 1..1024 in block mode and 1..4096 in token mode.  Block mode takes
 * at most 4096 blocks per row (T, or the cache capacity, up to 262144);
 * longer rows return HS_ERR_UNSUPPORTED.
 */
hs_status hs_block_topk(const hs_shape* shape, const float* blk_raw, const float* lse,
                        int block, int topk, int n_recent, int flags, float* grp_score,
                        int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * One sparse layer, prefill (explainer 3.4.3: "Branch 1: Block Sparse
 * Attention" eq. K~,V~ and eq. o~_t, "Branch 2: Sliding Window Attention"
 * eq. o'_t, "Gated Fusion"; paper 3.1 and 3.3).
 *   q_sp  [batch][T][hq][head_dim]          the layer's own queries q'
 *   k, v  the full layer's K (position-major) and V (block-major), shared
 *   idx   [batch][hkv][T][topk] int32 block ids, read as a set per row (any
 *         order; repeats count once; negative or j > floor(t/64) ids, and
 *         -1 padding, are ignored)
 *   k_swa [batch][hkv][T][head_dim], v_swa [batch][hkv][nblk][head_dim][64]
 *         the layer's own window cache (NULL together with window == 0)
 *   window   W >= 0: keys t-W+1 .. t of k_swa/v_swa
 *   gate_logits [batch][T][hq][2] fp32 (sparse, window) or NULL (both gates 1)
 *   sinks [2][hq] fp32 device per-head sink logits (row 0: sparse branch,
 *         row 1: window branch), in the units of tau q.k, or NULL (none)
 *   o     [batch][T][hq][head_dim] (out)
 * o_t = sigmoid(G0) o~_t + sigmoid(G1) o'_t; an empty selection gives o~ = 0.
 * Keys after t inside a selected block are excluded.  The selection bitsets
 * of one work group must fit 48 KiB of LDS: T <= 83968 for G = hq/hkv = 1,
 * 147456 for G = 2, 239616 for G = 4, 262144 for G >= 8 (G <= 16); longer
 * sequences return HS_ERR_UNSUPPORTED.  Sinks (paper 4.1,
 * "Experiments Setup": per-head learnable sink biases in both branches,
 * following gpt-oss): each branch's softmax takes one more logit b_h that
 * carries no value, o = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{b_h}).
 */
hs_status hs_sparse_attn_fwd(const hs_shape* shape, const void* q_sp, const void* k,
                             const void* v, const int32_t* idx, int topk,
                             const void* k_swa, const void* v_swa, int window,
                             const float* gate_logits, const float* sinks, void* o,
                             void* stream);

/*
 * One sparse layer at decode time, one query per sequence (explainer 3.4.3;
 * HySparse2 explainer, decode_one_token pseudocode).
 *   q_sp [batch][hq][head_dim]; k, v: the full layer's caches as in
 *   hs_full_attn_fwd_scores decode mode; idx [batch][hkv][n_sel] from
 *   hs_block_topk (block ids for block = 64, token ids for block = 1).
 *   Each idx row is read as a set (the sparse branch attends the union of
 *   the selected blocks or tokens): the order does not matter, an id listed
 *   more than once counts once, and ids that are negative or out of range
 *   (block mode: 64*j >= L_b; token mode: i >= L_b) are ignored, wherever
 *   they stand in the row.  idx may be NULL when n_sel == 0.
 *   k_ring, v_ring: the layer's own window ring [batch][hkv][W][head_dim]
 *   and [batch][hkv][ceil(W/64)][head_dim][64] (slot = position mod W), or
 *   NULL with window == 0.  gate_logits [batch][hq][2] or NULL.  sinks
 *   [2][hq] or NULL, as in hs_sparse_attn_fwd (token mode uses row 0).
 *   o [batch][hq][head_dim] (out).
 * Token mode (block = 1, fp8 caches as in hs_full_attn_fwd_scores) has no
 * window branch and no gate (the newest tokens are part of idx).  Block mode
 * takes no workspace.  Token mode takes an optional one: with
 * ws_bytes >= hs_workspace_size(HS_FN_DECODE_SELECT, shape, 1, 0, 0) every
 * (sequence, kv head) is spread over several work groups (about one 64-token
 * tile per wave, and no more work groups in all than the device has compute
 * units) and merged by a second kernel; with less (or NULL) one work group
 * handles it.  Results agree to rounding either way.
 */
hs_status hs_decode_select_attn(const hs_shape* shape, const void* q_sp, const void* k,
                                const void* v, const int32_t* idx, int n_sel, int block,
                                const void* k_ring, const void* v_ring, int window,
                                const float* gate_logits, const float* sinks, void* o,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * hs_decode_select_attn without a workspace, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments and
 * results are those of hs_decode_select_attn.  The token-mode split partial
 * states go to a fixed device array inside the library instead of a caller
 * workspace: HS_STATIC_SCRATCH_BYTES per GPU, held until the process ends.
 * The split uses at most as many work groups as the device has compute
 * units, so its partials take at most (compute units) * 16 * (head_dim + 2)
 * * 4 bytes: 2.1 MB on a 256-CU device.  A shape whose split partials need
 * more than HS_STATIC_SCRATCH_BYTES returns HS_ERR_WORKSPACE; block mode
 * needs no scratch.  All calls on one GPU share that GPU's array, so
 * calls that overlap in time on one GPU (on different streams) race; calls
 * on one stream are ordered and safe.  The first call on a device looks up
 * that device's copy of the array (no allocation).
 */
#define HS_STATIC_SCRATCH_BYTES (8u << 20)
hs_status hs_decode_select_attn_static(const hs_shape* shape, const void* q_sp, const void* k,
                                       const void* v, const int32_t* idx, int n_sel, int block,
                                       const void* k_ring, const void* v_ring, int window,
                                       const float* gate_logits, const float* sinks, void* o,
                                       void* stream);

/*
 * Gather of the selected blocks (explainer 3.4.3 eq. K~,V~: the selected
 * blocks' keys and values concatenated), block-mode decode caches:
 *   k [batch][hkv][C][head_dim], v [batch][hkv][C/64][head_dim][64] (bf16),
 *   idx [batch][hkv][n_sel] block ids, read as a set of fully-past blocks
 *   (order free, repeats once; ids outside 0 <= j < floor((L_b-1)/64), the
 *   block-mode decode candidates, are dropped: a gathered block is whole);
 *   k_sel [batch][hkv][n_sel*64][head_dim], v_sel [batch][hkv][n_sel][head_dim][64]
 *   (out): slot p < n holds the p-th live block in ascending id order;
 *   idx_sel [batch][hkv][n_sel] (out): p for p < n, then -1.  Slots p >= n
 *   are not written.
 * The compact cache is a block-mode cache of capacity n_sel*64: a sparse
 * layer over it is hs_decode_select_attn with shape.kv_len = 64*n_sel (which
 * must be >= window), the same kv_lens, k_sel/v_sel and idx_sel, and gives
 * the same result as over the full cache with idx.
 */
hs_status hs_gather_blocks(const hs_shape* shape, const void* k, const void* v, const int32_t* idx,
                           int n_sel, void* k_sel, void* v_sel, int32_t* idx_sel, void* stream);

/*
 * One decode step's full layer, selection and gather over a full-layer cache
 * held in host memory (paper section 5, "Potential of HySparse for Efficient
 * KV Cache Offloading": the full layer's cache lives in external memory and
 * is prefetched before the computation; only the selected blocks stay on
 * the GPU for the sparse layers).  Block mode, bf16 caches.
 *   lens_host [batch]: host copy of shape.kv_lens (sizes of the copies);
 *   q, o, lse, blk_raw, idx: as hs_full_attn_fwd_scores + hs_block_topk in
 *   decode mode (device); k_host, v_host: the caches in the decode layouts,
 *   in pinned host memory; k_sel, v_sel, idx_sel: as hs_gather_blocks with
 *   n_sel = topk (device).
 * Sequences are processed in chunks of `chunk`: the live key rows and value
 * blocks of chunk c+1 are copied (hipMemcpyAsync) on copy_stream into one of
 * two device staging buffers while the full layer, the top-k and the gather
 * of chunk c run on `stream`.  Results equal those of the device-resident
 * calls.  ws: hs_offload_workspace_size(shape, chunk) bytes, 256-byte
 * aligned.  copy_stream should be a second stream of default priority; all
 * work is complete once `stream` reaches the end of what this call enqueued.
 * The library keeps one set of events per device for the pipeline and
 * enqueues each call's work under a lock, so calls may come from several
 * host threads (each with its own workspace).
 */
size_t hs_offload_workspace_size(const hs_shape* shape, int chunk);
hs_status hs_offload_full_select(const hs_shape* shape, const int32_t* lens_host, const void* q,
                                 const void* k_host, const void* v_host, void* o, float* lse,
                                 float* blk_raw, int topk, int32_t* idx, void* k_sel, void* v_sel,
                                 int32_t* idx_sel, int chunk, void* ws, size_t ws_bytes, void* stream,
                                 void* copy_stream);

/*
 * Token-level decode step's full layer and selection in one call, without the
 * per-token logits (HySparse2 explainer, "Precise retrieval without a
 * separate indexer" and the decode_one_token pseudocode).  o, lse and idx are
 * those of hs_full_attn_fwd_scores + hs_block_topk with block = 1 and no
 * grp_score: the same selection rule (top-k older tokens by
 * x_i = max_h (logit_hi - LSE_h), ties to the smaller token id, then the
 * n_recent newest tokens), and the same full-layer arithmetic for o and lse.
 * Instead of every head's logit, the full layer leaves one value per token and
 * kv group plus one offset per 64-token tile and head, which bound x_i from
 * both sides once the LSEs are known; the tokens whose bounds reach the k-th
 * largest lower bound are rescored exactly from their key rows, and the
 * selection runs on them.  The scores are therefore rounded differently from
 * the two-call path (both within fp32 rounding of the exact value), so rows
 * whose k-th and (k+1)-th scores differ by rounding only may pick different
 * tokens among those ties.
 *   shape: decode (kv_lens set), fp8 e4m3 caches with kv_scale, head_dim 64
 *   or 128, group size <= 16; q [batch][hq][head_dim] bf16; k, v the
 *   position-major fp8 caches; o [batch][hq][head_dim] bf16 and lse
 *   [batch][hq] (out); idx [batch][hkv][topk + n_recent] int32 (out),
 *   topk 1..4096, n_recent 0..4096.
 * ws: hs_workspace_size(HS_FN_DECODE_TOKEN_SELECT, shape, 1, topk, 0) bytes,
 * 16-byte aligned.
 */
hs_status hs_decode_token_select(const hs_shape* shape, const void* q, const void* k, const void* v,
                                 void* o, float* lse, int topk, int n_recent, int32_t* idx, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Training forward of one sparse layer: hs_sparse_attn_fwd (bf16), plus what
 * its backward needs, each branch's own ungated output and LSE:
 *   o_branch   [2][batch][T][hq][head_dim] bf16 (out): [0] the block-sparse
 *              branch o~, [1] the window branch o' (explainer 3.4.3)
 *   lse_branch [2][batch][hq][T] fp32 (out): log of each branch's softmax
 *              denominator, its sink included (-inf for an empty branch
 *              without a sink)
 * Takes the shapes the default sparse kernel serves (selection bitsets of a
 * work group within 16 KiB of LDS: T <= 32768 for G = 1, more for larger
 * groups); longer sequences return HS_ERR_UNSUPPORTED.
 */
hs_status hs_sparse_attn_fwd_train(const hs_shape* shape, const void* q_sp, const void* k,
                                   const void* v, const int32_t* idx, int topk, const void* k_swa,
                                   const void* v_swa, int window, const float* gate_logits,
                                   const float* sinks, void* o, void* o_branch, float* lse_branch,
                                   void* stream);

/*
 * Backward pass of the full layer (bf16 prefill, head_dim 64/128, hq/hkv <=
 * 16).  The paper trains this architecture (section 4.1); gradients follow
 * the chain rule of eq. o_t (explainer 3.4.1):
 *   dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO o)), dQ = tau dS K,
 *   dK = tau dS^T Q.
 *   q, o, dout [batch][T][hq][head_dim]; k, v as hs_full_attn_fwd_scores;
 *   lse [batch][hq][T] from the forward;
 *   dq [batch][T][hq][head_dim], dk, dv [batch][hkv][T][head_dim] fp32
 *   (out, overwritten; dv is position-major).
 * ws: hs_workspace_size(HS_FN_FULL_ATTN_BWD, shape, 64, 0, 0) bytes,
 * 256-byte aligned (layout copies of K, V, Q and dO; row terms).
 */
hs_status hs_full_attn_bwd(const hs_shape* shape, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, float* dq, float* dk,
                           float* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass of one sparse layer (bf16): the block-sparse branch over the
 * shared K/V at the forward's indices (read as in the forward; they get no
 * gradient), the window branch over the layer's own K'/V', the sigmoid gates
 * (explainer 3.4.3), the sink logits (paper 4.1).  With s = sigmoid(G):
 * each branch sees dO~ = s dO; dG = s (1 - s) dO.o_branch; a sink gets
 * -sum_t p_sink dO~.o_branch.
 *   q_sp, dout [batch][T][hq][head_dim]; k, v, idx, topk, k_swa, v_swa,
 *   window, gate_logits, sinks: as in the forward call;
 *   o_branch, lse_branch: from hs_sparse_attn_fwd_train;
 *   dq_sp [batch][T][hq][head_dim] fp32 (out);
 *   dk, dv [batch][hkv][T][head_dim] fp32: the shared K/V's gradients, to
 *     which this layer's share is ADDED (pass those of the full layer's
 *     backward, then every sparse layer's in turn);
 *   dk_swa, dv_swa [batch][hkv][T][head_dim] fp32 (out; with window > 0);
 *   dgate [batch][T][hq][2] fp32 (out; with gate_logits); dsinks [2][hq]
 *   fp32 (out; with sinks).
 * ws: hs_workspace_size(HS_FN_SPARSE_ATTN_BWD, shape, 64, topk, window)
 * bytes, 256-byte aligned.  Gradients are sums taken in a fixed order (no
 * atomics), so a call repeated on the same inputs gives the same bits.
 */
hs_status hs_sparse_attn_bwd(const hs_shape* shape, const void* q_sp, const void* k, const void* v,
                             const int32_t* idx, int topk, const void* k_swa, const void* v_swa,
                             int window, const float* gate_logits, const float* sinks,
                             const void* o_branch, const float* lse_branch, const void* dout,
                             float* dq_sp, float* dk, float* dv, float* dk_swa, float* dv_swa,
                             float* dgate, float* dsinks, void* ws, size_t ws_bytes, void* stream);

/* Function ids for hs_workspace_size */
#define HS_FN_FULL_ATTN 0
#define HS_FN_BLOCK_TOPK 1
#define HS_FN_SPARSE_ATTN 2
#define HS_FN_DECODE_SELECT 3
#define HS_FN_FULL_ATTN_BWD 4   /* prefill shape (kv_lens NULL) */
#define HS_FN_SPARSE_ATTN_BWD 5 /* prefill shape (kv_lens NULL) */
#define HS_FN_DECODE_TOKEN_SELECT 6

/* Workspace bytes the given entry point needs (or, for token-mode
 * hs_decode_select_attn, can use) for this shape; 0 if none.  `block`,
 * `topk` and `window` are the values that will be passed to it.  The
 * workspace is scratch: its contents need no initialisation and are not
 * preserved. */
size_t hs_workspace_size(int fn_id, const hs_shape* shape, int block, int topk, int window);

/* Thread-local description of the last error of this thread ("" if none). */
const char* hs_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYSPARSE_H */
