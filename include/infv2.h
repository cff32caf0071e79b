/*
 * infv2.h -- C ABI of the InfLLM v2 sparse-attention hot path for AMD MI355X (gfx950).
 *
 * InfLLM v2 (MiniCPM4 summary page, section "InfLLM v2: Trainable Sparse
 * Attention for Both Prefilling and Decoding") splits attention into two
 * stages: (1) score every KV block against the query's group through
 * mean-pooled "semantic kernels" and pick the top-k blocks, and (2) run exact
 * softmax attention over the chosen blocks only (paragraph "Complexity
 * analysis").  The library exposes each step as one call:
 *
 *   infv2_compress_keys        step 1a: compressed keys  kbar_j = Mean(K[j s : j s + p])
 *   infv2_select_blocks        step 1b: kernel softmax, group mean, block max, top-k
 *   infv2_select_blocks_coarse step 1b with the coarse-kernel LogSumExp approximation
 *   infv2_sparse_attn_decode   step 2 for one new token per sequence
 *   infv2_sparse_attn_prefill  step 2 for a chunk of consecutive query rows
 *   infv2_sparse_attn_prefill_bwd  gradients of step 2 (training)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them after the call returns.  Scratch
 *    memory comes only from the caller's workspace (see infv2_workspace_bytes).
 *  - Every call enqueues work on `stream` (a hipStream_t; NULL = the default
 *    stream) and returns without synchronising.  Results are valid once the
 *    caller has synchronised that stream.  No host<->device copies are made.
 *  - Arguments are validated on the host BEFORE any HIP call: an invalid call
 *    returns an error status and enqueues nothing.  Values that live in device
 *    memory (offsets, lengths, indices) cannot be checked on the host; if they
 *    are inconsistent with the buffers the result is undefined.
 *  - Launch failures are reported as INFV2_ERR_DEVICE.
 *  - The method's calls hold no mutable global state (the benchmark timing
 *    session at the end of this header is the only global state).
 *    Concurrent calls on different streams need distinct workspaces.
 *
 * Layouts (row-major, contiguous; element type given by the config):
 *  - Query heads h = g*G + r (r < G) belong to KV head g, G = Hq / Hkv.
 *  - K / V of sequence b: tokens [kv_offsets[b], kv_offsets[b+1]) of a packed
 *    buffer; inside, layout [Hkv][cap_b][d] with cap_b = kv_offsets[b+1] -
 *    kv_offsets[b] (each KV head's keys contiguous).  The valid length is
 *    kv_lens[b] <= cap_b (kv_lens == NULL: the length is cap_b).
 *  - Compressed keys of sequence b: kernels [ck_offsets[b], ck_offsets[b+1])
 *    of a packed buffer, layout [Hkv][ccap_b][d], element type ck_dtype, with
 *    ccap_b >= n_c(kv_lens[b]).
 *  - block_idx: int32 [rows][Hkv][topk], ascending, padded with -1.
 *
 * Readings of the pages that fix the arithmetic:
 *  - kernels: only complete ones, n_c(n) = floor((n - p) / s) + 1 (0 if n < p);
 *  - a query at absolute position i sees kernel j only if j*s + p <= i + 1;
 *  - logits z = score_scale * q.kbar; LogSumExp per query head; group score
 *    = mean over the group's heads of the per-head softmax; block score = max
 *    over the visible kernels that share a token with the block;
 *  - forced blocks F = {0..init-1} U {c-local+1..c}, c = floor(i/m); k counts
 *    F; if c + 1 <= k every block 0..c is taken (dense); score ties go to the
 *    lower block index;
 *  - attention: softmax(attn_scale * q.k) over the tokens t <= i (and t < n)
 *    of the selected blocks.
 *
 * Supported on the GPU: head_dim = 128, group size Hq/Hkv = 16 (one token's
 * group forms the 16-row side of a 16x16 MFMA tile), block_size a multiple of
 * 16 in [16, 256], 1 <= kernel_stride <= kernel_size <= 256, topk <= 1024,
 * at most 16384 blocks per sequence.  Other values return INFV2_ERR_UNSUPPORTED.
 * bf16 inputs run on the matrix cores (prefill attention there needs
 * block_size 64 and topk <= 128); fp32 inputs and the other bf16 prefill
 * shapes run on vector-ALU kernels with fp32 accumulation.
 */
#ifndef INFV2_H
#define INFV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INFV2_ABI_VERSION 9   /* 9: infv2_decode_step_append */

typedef enum infv2_status {
    INFV2_OK = 0,
    INFV2_ERR_NULL = 1,         /* a required pointer is NULL */
    INFV2_ERR_SHAPE = 2,        /* sizes inconsistent (e.g. Hq % Hkv != 0, k < |F|), or a
                                   negative or non-finite scale */
    INFV2_ERR_UNSUPPORTED = 3,  /* valid but not implemented on this device path */
    INFV2_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than infv2_workspace_bytes */
    INFV2_ERR_DEVICE = 5,       /* a HIP launch failed */
    INFV2_ERR_SCRATCH = 6       /* the call needs more than the library's static scratch */
} infv2_status;

typedef enum infv2_dtype {
    INFV2_FP32 = 0,
    INFV2_BF16 = 1
} infv2_dtype;

typedef enum infv2_mode {
    INFV2_MODE_DECODE = 0,      /* one query row per sequence, at position kv_lens[b] - 1 */
    INFV2_MODE_PREFILL = 1      /* one sequence, rows at positions q_start .. q_start + rows - 1 */
} infv2_mode;

typedef enum infv2_op {         /* operation ids for infv2_workspace_bytes */
    INFV2_OP_COMPRESS = 0,
    INFV2_OP_SELECT_DECODE = 1,
    INFV2_OP_SELECT_PREFILL = 2,
    INFV2_OP_ATTN_DECODE = 3,
    INFV2_OP_ATTN_PREFILL = 4,
    INFV2_OP_ATTN_PREFILL_BWD = 5,
    INFV2_OP_SELECT_COARSE_DECODE = 6,
    INFV2_OP_SELECT_COARSE_PREFILL = 7,
    INFV2_OP_DECODE_STEP = 8
} infv2_op;

/* Method hyper-parameters (names follow the pages' notation). */
typedef struct infv2_config {
    int32_t head_dim;       /* d */
    int32_t num_q_heads;    /* Hq */
    int32_t num_kv_heads;   /* Hkv; group size G = Hq / Hkv */
    int32_t block_size;     /* m: tokens per KV block ("Block-level key-value partitioning") */
    int32_t kernel_size;    /* p: tokens per semantic kernel ("Semantic kernels"), 32 recommended */
    int32_t kernel_stride;  /* s: stride between kernel starts, 16 recommended */
    int32_t topk;           /* k: blocks attended per query token, forced blocks included */
    int32_t init_blocks;    /* leading blocks always selected ("Initial and local tokens") */
    int32_t local_blocks;   /* blocks of the local window ending at the query's block */
    int32_t io_dtype;       /* infv2_dtype of q, k, v and out */
    int32_t ck_dtype;       /* infv2_dtype of the compressed keys (FP32 default) */
    float   score_scale;    /* selection logit scale, > 0; 0 selects the default 1.0 (the
                               pages print the kernel softmax with no scale) */
    float   attn_scale;     /* attention logit scale, > 0; 0 selects the default 1/sqrt(d) */
} infv2_config;

/*
 * infv2_compress_keys -- step 1a, "Semantic kernels" paragraph: the kernel
 * j of sequence b covers tokens [j*s, j*s + p) and its compressed key is the
 * mean of those keys ("What this computes" / "Why mean pooling").
 *
 * Computes, for every sequence b and KV head, the kernels
 * j in [ck_begin[b], n_c(kv_lens[b])) and stores them at their index j in the
 * sequence's compressed-key region (incremental update: earlier kernels are
 * left untouched).  The mean is formed exactly (float64 sum) and rounded once
 * to ck_dtype.
 *
 *   k            device, io_dtype, packed K (see Layouts)
 *   kv_offsets   device int64 [batch+1], token offsets (capacities) of the K buffer
 *   kv_lens      device int64 [batch] valid lengths, or NULL (= capacities)
 *   ck_offsets   device int64 [batch+1], kernel offsets (capacities) of the CK buffer
 *   ck_begin     device int64 [batch] first kernel to compute, or NULL (= 0)
 *   batch        number of sequences, >= 1
 *   max_len      host upper bound of every kv_lens[b] (sizes the grid)
 *   max_new      host upper bound of n_c(kv_lens[b]) - ck_begin[b] over b;
 *                < 0 means n_c(max_len)
 *   ck           device, ck_dtype, packed compressed keys (written)
 */
int32_t infv2_compress_keys(const infv2_config* cfg, const void* k, const int64_t* kv_offsets,
                            const int64_t* kv_lens, const int64_t* ck_offsets,
                            const int64_t* ck_begin, int32_t batch, int64_t max_len,
                            int64_t max_new, void* ck, void* stream);

/*
 * infv2_append_kv -- the step before decoding attention: one new token per
 * sequence enters the cache, and the compressed keys follow incrementally
 * ("Semantic kernels": kernel j covers [j*s, j*s + p); with complete kernels
 * only, the token at position n completes kernel (n + 1 - p) / s exactly when
 * n + 1 >= p and s divides n + 1 - p, i.e. one new kernel every s tokens).
 *
 * For every sequence b with n = kv_lens[b] < capacity: writes k_new[b] and
 * v_new[b] at position n of its cache region, stores the compressed key of
 * the kernel the token completes (same float64 mean and single rounding as
 * infv2_compress_keys; skipped if ck_offsets leave no room for it), and sets
 * kv_lens[b] = n + 1.  A sequence whose cache is full is left unchanged.
 *
 *   k_new, v_new device, io_dtype [batch][Hkv][d]
 *   k, v         device, io_dtype, packed caches (see Layouts), updated in place
 *   kv_offsets   device int64 [batch+1] (capacities)
 *   kv_lens      device int64 [batch], read and advanced in place
 *   ck_offsets, ck   as for infv2_compress_keys (ck updated in place)
 */
int32_t infv2_append_kv(const infv2_config* cfg, const void* k_new, const void* v_new, void* k,
                        void* v, const int64_t* kv_offsets, int64_t* kv_lens,
                        const int64_t* ck_offsets, void* ck, int32_t batch, void* stream);

/*
 * infv2_select_blocks -- step 1b, paragraphs "Semantic kernels" (eqs.
 * r_kernel, r_block), "Query group sharing" (eq. r_group), "Top-K
 * implementation and the LSE bottleneck" (two passes: LogSumExp, then
 * normalised scores) and "Initial and local tokens always selected".
 *
 * For every query row and KV head g: logits of the group's G heads against
 * every kernel visible to the row, per-head LogSumExp, group score per kernel
 * (mean of the per-head softmax), block score (max over the kernels meeting
 * the block), and the forced blocks plus the top (k - |F|) other blocks.
 *
 *   mode         INFV2_MODE_DECODE: rows == batch, q [batch][Hq][d], row b at
 *                position kv_lens[b] - 1 of sequence b.
 *                INFV2_MODE_PREFILL: batch == 1, q [rows][Hq][d], row r at
 *                position q_start + r; compressed keys up to n_c(q_start + rows)
 *                must be present.
 *   q            device, io_dtype
 *   ck, ck_offsets, kv_offsets, kv_lens, batch, max_len   as above
 *                (prefill: max_len >= q_start + rows)
 *   block_idx    device int32 [rows][Hkv][topk] (written)
 *   block_score  device float [rows][Hkv][topk] or NULL: the block score of
 *                each selected block (-inf if no kernel is visible in it,
 *                NaN in padding slots).  With NULL and every row shorter than
 *                topk*block_size (max_len, or q_start + rows, <= topk*m) the
 *                selection is dense by definition and no score is computed:
 *                only the ids are written and ws is not touched.
 *   ws           device workspace of ws_bytes >= infv2_workspace_bytes(op =
 *                SELECT_DECODE or SELECT_PREFILL).  No initial contents are
 *                needed: the call clears and writes everything it reads.
 *                Calls that overlap in time need distinct workspaces.
 */
int32_t infv2_select_blocks(const infv2_config* cfg, int32_t mode, const void* q, int32_t rows,
                            int64_t q_start, const void* ck, const int64_t* ck_offsets,
                            const int64_t* kv_offsets, const int64_t* kv_lens, int32_t batch,
                            int64_t max_len, int32_t* block_idx, float* block_score, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * infv2_select_blocks_coarse -- infv2_select_blocks with the pages' cheaper
 * first pass ("Efficient LSE approximation"; "Complexity analysis", Stage 1):
 * the per-head LogSumExp is taken over coarse kernels -- spans of `coarse`
 * tokens at stride `coarse`, complete ones only, seen by a row when they lie
 * wholly at or before it, their keys the mean of the span -- and the second
 * pass scores the fine kernels against that normaliser.  Selections and scores
 * can differ from the exact call's: that is the approximation.  A row that sees
 * no coarse kernel keeps the exact normaliser (such rows are dense, since
 * coarse <= topk * block_size).
 *
 *   coarse       s_c, with kernel_size <= coarse <= min(256, topk * block_size)
 *                (256: the largest kernel infv2_compress_keys builds)
 *   ck_coarse    device, ck_dtype: the coarse compressed keys, as written by
 *                infv2_compress_keys with kernel_size = kernel_stride = coarse
 *                (same layout as ck)
 *   ckc_offsets  device int64 [batch+1], kernel offsets of ck_coarse
 *   ws           infv2_workspace_bytes(op = SELECT_COARSE_DECODE or
 *                SELECT_COARSE_PREFILL); no initial contents are needed
 *   all else     as for infv2_select_blocks (INFV2_ERR_SHAPE for a coarse size
 *                out of range)
 */
int32_t infv2_select_blocks_coarse(const infv2_config* cfg, int32_t coarse, int32_t mode,
                                   const void* q, int32_t rows, int64_t q_start, const void* ck,
                                   const int64_t* ck_offsets, const void* ck_coarse,
                                   const int64_t* ckc_offsets, const int64_t* kv_offsets,
                                   const int64_t* kv_lens, int32_t batch, int64_t max_len,
                                   int32_t* block_idx, float* block_score, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * infv2_sparse_attn_decode -- step 2 for decoding ("Complexity analysis",
 * Stage 2: each query token attends the k*m tokens of its selected blocks;
 * "Query group sharing": the group's heads read the same blocks once).
 *
 *   q            device, io_dtype [batch][Hq][d]; row b at position kv_lens[b] - 1
 *   k, v         device, io_dtype, packed K/V (see Layouts)
 *   kv_offsets, kv_lens, batch, max_len   as above
 *   block_idx    device int32 [batch][Hkv][topk] from infv2_select_blocks
 *                (entries -1 are skipped)
 *   out          device, io_dtype [batch][Hq][d] (written)
 *   ws           workspace (infv2_workspace_bytes op = ATTN_DECODE); no initial
 *                contents are needed
 */
int32_t infv2_sparse_attn_decode(const infv2_config* cfg, const void* q, const void* k,
                                 const void* v, const int64_t* kv_offsets, const int64_t* kv_lens,
                                 int32_t batch, int64_t max_len, const int32_t* block_idx,
                                 void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * infv2_decode_step -- one decode step of the whole path for every sequence of
 * a batch, in one call: the compressed key of the kernel that the newest token
 * completes ("Semantic kernels": with complete kernels only, token n - 1
 * completes kernel (n - p) / s when n >= p and s divides n - p), block
 * selection (step 1b) and sparse attention (step 2).  The results are those of
 * infv2_compress_keys for that kernel, then infv2_select_blocks (decode, no
 * scores) and infv2_sparse_attn_decode, bit for bit; with bf16 inputs the
 * compression runs inside the selection's first kernel (one launch fewer).
 *
 *   q, k, v, kv_offsets, kv_lens, batch, max_len   as for infv2_sparse_attn_decode;
 *                kv_lens[b] = n_b counts the newest token, whose K/V row must
 *                already be at position n_b - 1 of the cache (infv2_append_kv
 *                or the caller's own write); kv_lens == NULL: the capacities
 *   ck_offsets, ck   compressed keys (see Layouts), kernels up to the newest
 *                token's present except the one it completes, which is written
 *   block_idx    device int32 [batch][Hkv][topk] (written)
 *   out          device, io_dtype [batch][Hq][d] (written)
 *   ws           infv2_workspace_bytes(op = DECODE_STEP); no initial contents needed
 */
int32_t infv2_decode_step(const infv2_config* cfg, const void* q, const void* k, const void* v,
                          const int64_t* kv_offsets, const int64_t* kv_lens,
                          const int64_t* ck_offsets, void* ck, int32_t batch, int64_t max_len,
                          int32_t* block_idx, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * infv2_decode_step_append -- the serving loop's step: infv2_append_kv (the new
 * token of every sequence enters the cache, "Semantic kernels": it completes
 * kernel (n - p) / s when s divides n - p) followed by infv2_decode_step, with
 * the same results bit for bit (caches, compressed keys, kv_lens, block_idx,
 * out), in the decode step's launches: with bf16 inputs the first kernel also
 * writes the new K/V rows and the last one advances kv_lens (one launch fewer
 * than the two calls).  Other inputs run the two calls.
 *
 *   q            device, io_dtype [batch][Hq][d], the new tokens' queries
 *   k_new, v_new device, io_dtype [batch][Hkv][d], the new tokens' keys / values
 *   k, v, kv_offsets, kv_lens, ck_offsets, ck, batch   as for infv2_append_kv
 *                (caches, compressed keys and kv_lens updated in place; a full
 *                sequence is left as it is and decodes over its cache)
 *   max_len      >= every sequence's length after the append
 *   block_idx, out, ws, ws_bytes   as for infv2_decode_step (op = DECODE_STEP)
 * Concurrent calls on one cache race; calls ordered on one stream are safe.
 */
int32_t infv2_decode_step_append(const infv2_config* cfg, const void* q, const void* k_new,
                                 const void* v_new, void* k, void* v, const int64_t* kv_offsets,
                                 int64_t* kv_lens, const int64_t* ck_offsets, void* ck,
                                 int32_t batch, int64_t max_len, int32_t* block_idx, void* out,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * infv2_sparse_attn_prefill -- step 2 for a chunk of consecutive query rows
 * of one sequence ("Design principles summary": every query token selects its
 * own blocks; rows are causal, t <= i).
 *
 *   q            device, io_dtype [rows][Hq][d]; row r at position q_start + r
 *   k, v         device, io_dtype, one sequence [Hkv][cap][d] with
 *                cap = kv_offsets[1] - kv_offsets[0] >= q_start + rows
 *   kv_offsets   device int64 [2]
 *   block_idx    device int32 [rows][Hkv][topk]
 *   out          device, io_dtype [rows][Hq][d] (written)
 *   ws           workspace (op = ATTN_PREFILL); infv2_workspace_bytes returns 0
 *                for this op, so NULL is allowed; kept for ABI stability
 */
int32_t infv2_sparse_attn_prefill(const infv2_config* cfg, const void* q, int32_t rows,
                                  int64_t q_start, const void* k, const void* v,
                                  const int64_t* kv_offsets, const int32_t* block_idx, void* out,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * infv2_sparse_attn_decode_noalloc -- infv2_sparse_attn_decode for callers that
 * cannot allocate device memory (code captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc): no workspace argument.  The split
 * partials go to a static device array of INFV2_NOALLOC_SCRATCH_BYTES inside the
 * library (one per GPU, held until the process ends); the call allocates
 * nothing.  Same arguments, results and errors as infv2_sparse_attn_decode,
 * plus INFV2_ERR_SCRATCH (nothing enqueued) when infv2_workspace_bytes(op =
 * ATTN_DECODE) for these sizes exceeds INFV2_NOALLOC_SCRATCH_BYTES, and
 * INFV2_ERR_DEVICE if the scratch address cannot be obtained.  Every call on a
 * GPU uses that GPU's one array, so calls that overlap in time on one GPU (on
 * different streams) race; calls ordered on one stream are safe.  The scratch
 * needs no initial contents (every partial is written before it is read).
 */
#define INFV2_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t infv2_sparse_attn_decode_noalloc(const infv2_config* cfg, const void* q, const void* k,
                                         const void* v, const int64_t* kv_offsets,
                                         const int64_t* kv_lens, int32_t batch, int64_t max_len,
                                         const int32_t* block_idx, void* out, void* stream);

/*
 * Varlen prefill: several sequences in one call (serving-style prefill).  The
 * rows of the call are packed sequence after sequence: rows_per_seq[b] rows of
 * sequence b, the first at position q_start_per_seq[b] ("Design principles
 * summary": every query token selects its own blocks, so sequences are
 * independent).  Both arrays are HOST arrays of `batch` entries, checked
 * before anything is launched; everything else is as for the single-sequence
 * calls, with kv_offsets / ck_offsets describing all `batch` sequences ([batch+1]).
 * Compressed keys up to n_c(q_start_per_seq[b] + rows_per_seq[b]) must be
 * present (infv2_compress_keys over the batch).  The workspace must hold at
 * least the largest single-sequence need: infv2_workspace_bytes(op, rows = max
 * rows, batch = 1, max_len = max (q_start + rows)).  The bf16 matrix-core
 * attention (block size 64) runs up to 64 sequences per launch, from a table of
 * the sequences passed with the launch.  The bf16 selection does the same when
 * the workspace holds all rows of the call: infv2_workspace_bytes(
 * INFV2_OP_SELECT_PREFILL, rows = total rows, batch = number of sequences with
 * rows, max_len); with less it runs sequence after sequence.  Both give the
 * same bits.  fp32 calls run sequence after sequence through the
 * single-sequence kernels.
 *
 *   q, block_idx, block_score, out   packed over all rows of the call
 */
int32_t infv2_select_blocks_varlen(const infv2_config* cfg, const void* q, int32_t batch,
                                   const int32_t* rows_per_seq, const int64_t* q_start_per_seq,
                                   const void* ck, const int64_t* ck_offsets,
                                   const int64_t* kv_offsets, int32_t* block_idx,
                                   float* block_score, void* ws, size_t ws_bytes, void* stream);
int32_t infv2_sparse_attn_prefill_varlen(const infv2_config* cfg, const void* q, int32_t batch,
                                         const int32_t* rows_per_seq,
                                         const int64_t* q_start_per_seq, const void* k,
                                         const void* v, const int64_t* kv_offsets,
                                         const int32_t* block_idx, void* out, void* ws,
                                         size_t ws_bytes, void* stream);

/*
 * infv2_sparse_attn_prefill_bwd -- gradients of step 2 for a chunk of rows
 * ("Training-time considerations": top-k is not differentiable, so the
 * selection is held fixed and no gradient reaches the compressed keys, which
 * only feed it; K and V receive gradient only through the attention over the
 * selected blocks, and "Why mean pooling": that is how training still shapes
 * the keys the selection pools).
 *
 * For the loss L with dL/dout = dout, per query head and with P the softmax
 * of attn_scale * q.k over the row's selected tokens (t <= i):
 *   dq = attn_scale * sum_t P_t (dout.v_t - dout.out) k_t,
 *   dk_t = attn_scale * sum over the rows and heads attending t of P_t (dout.v_t - dout.out) q,
 *   dv_t = sum over the rows and heads attending t of P_t dout.
 *
 *   q, rows, q_start, k, v, kv_offsets, block_idx   as for infv2_sparse_attn_prefill
 *                (the entries of one row of block_idx must be distinct, as
 *                infv2_select_blocks writes them; entries < 0 or past the
 *                row's block range are ignored)
 *   out          device, io_dtype [rows][Hq][d]: the forward output for these inputs
 *   dout         device, io_dtype [rows][Hq][d]: gradient of the loss w.r.t. out
 *   dq           device, io_dtype [rows][Hq][d] (written)
 *   dk, dv       device, io_dtype, same layout as k and v: tokens 0 .. q_start +
 *                rows - 1 of every KV head are written with the sum over this
 *                call's rows (0 where no row attends the token); later tokens
 *                are not touched.  A chunked caller sums the calls' results.
 *   ws           workspace (op = ATTN_PREFILL_BWD, rows, max_len = q_start + rows);
 *                no initial contents are needed
 * rows * topk must not exceed 2^30.  rows == 0 writes nothing.
 */
int32_t infv2_sparse_attn_prefill_bwd(const infv2_config* cfg, const void* q, int32_t rows,
                                      int64_t q_start, const void* k, const void* v,
                                      const int64_t* kv_offsets, const int32_t* block_idx,
                                      const void* out, const void* dout, void* dq, void* dk,
                                      void* dv, void* ws, size_t ws_bytes, void* stream);

/* Workspace size in bytes for operation `op` (infv2_op) at the given sizes.
 * SELECT_PREFILL with batch > 1: the varlen selection's one-launch workspace
 * for `rows` rows of `batch` sequences (see infv2_select_blocks_varlen). */
int32_t infv2_workspace_bytes(const infv2_config* cfg, int32_t op, int32_t rows, int32_t batch,
                              int64_t max_len, size_t* bytes);

/* Number of complete kernels over n keys: floor((n - p) / s) + 1, or 0 if n < p. */
int64_t infv2_num_kernels(const infv2_config* cfg, int64_t n);

/* Human-readable name of a status code (static string). */
const char* infv2_status_str(int32_t status);

/* INFV2_ABI_VERSION of the loaded library. */
int32_t infv2_abi_version(void);

/*
 * Kernel timing, for benchmarks and profiling only (not part of the method).
 * While a timing session is open, every launch of the chosen kernel family gets
 * a pair of HIP events, so one kernel can be timed on its own although an entry
 * point launches several.  For a family of one kernel per launch site (the
 * attention, scoring, append and backward-pass kernels) the launch itself
 * stamps the pair with the kernel's own begin and end (hipExtLaunchKernel);
 * for the others (compression, top-k, the backward's inverse index) the pair
 * is recorded on the stream before and after the launches of one call.  The
 * backward column family times its main kernel, not the small work-list and
 * reduction kernels around it.  Launches on a stream that is being captured
 * into a graph are not timed.  This is the only global state of the library: one session at a
 * time per process, guarded by a mutex.
 *
 * infv2_timing_start  opens a session for `kernel` (an infv2_kernel id);
 *                     INFV2_ERR_SHAPE for an unknown id or a session already
 *                     open.
 * infv2_timing_stop   closes it, waits for the recorded events and returns
 *                     the summed duration in milliseconds and the number of
 *                     timed launches; INFV2_ERR_SHAPE if no session is
 *                     open, INFV2_ERR_DEVICE if an event failed.
 */
typedef enum infv2_kernel {
    INFV2_KERNEL_COMPRESS = 0,          /* compressed keys */
    INFV2_KERNEL_SELECT_LOGITS = 1,     /* decode: kernel logits + per-chunk (max, sum exp) */
    INFV2_KERNEL_SELECT_SCORES = 2,     /* decode: LSE, group scores, block max */
    INFV2_KERNEL_SELECT_PREFILL = 3,    /* prefill: the two scoring passes */
    INFV2_KERNEL_SELECT_TOPK = 4,       /* top-k kernels that read keys from memory */
    INFV2_KERNEL_ATTN_DECODE = 5,       /* decode: attention over the selected blocks (partials) */
    INFV2_KERNEL_ATTN_MERGE = 6,        /* decode: merge of the partials */
    INFV2_KERNEL_ATTN_PREFILL = 7,      /* prefill: attention over the selected blocks */
    INFV2_KERNEL_VT_BUILD = 8,          /* reserved: no kernel is timed under this id */
    INFV2_KERNEL_APPEND = 9,            /* decode: cache append + incremental compressed key */
    INFV2_KERNEL_BWD_ROW = 10,          /* backward: dq, LogSumExp and dout.out per row */
    INFV2_KERNEL_BWD_INDEX = 11,        /* backward: the rows that selected each block */
    INFV2_KERNEL_BWD_COL = 12,          /* backward: dk and dv per block */
    INFV2_KERNEL_COUNT = 13
} infv2_kernel;

int32_t infv2_timing_start(int32_t kernel);
int32_t infv2_timing_stop(double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* INFV2_H */
