/*
 * dsa.h — C ABI of libdsa, the DeepSeek Sparse Attention (DSA) hot path on AMD MI355X (gfx950).
 *
 * DSA runs in three steps, and each step is one call here:
 *   1. dsa_indexer_scores  — the lightning indexer gives every causal (query, key) pair a relevance score.
 *   2. dsa_topk            — each query keeps the k best-scoring earlier positions.
 *   3. dsa_sparse_attn     — exact softmax attention over the gathered rows of a shared MLA latent cache,
 *                            read in multi-query mode (all heads score against the same cached row).
 * Upstream of a decode step, dsa_cache_append writes the new tokens into the caches (FP8 indexer keys with a
 * per-token scale, latent rows).
 * Sources (web pages on DSA):
 *   - "Linear and Sparse Attention — Featuring Kimi and DeepSeek", section "DeepSeek Sparse Attention":
 *     the two-stage pipeline (score everything, then attend over the top-k).
 *   - the GLM sparse-attention essay (thethings.ai), paragraphs on MLA's absorbed read, on the two DSA
 *     stages and the ReLU in the indexer, and on the gather kernels.
 *   - "Sparse Attention Architecture Evolution in LLMs: From Uniform Attention to Hybrid Gated DSA",
 *     sections "Indexer: A Lightweight 'Attention Router'" and "Top-K Selection: A Hard Filtering Mechanism".
 *   - "DeepSeek Sparse Attention" (attention-lab explainer), sections "Make a shortlist first",
 *     "Indexing and main attention are separate", "The lightning indexer" and "The top-k budget".
 *
 * Conventions shared by every call
 *   - Every tensor argument is a caller-owned DEVICE pointer to row-major, densely packed data unless a
 *     leading dimension is given. libdsa allocates no device memory, keeps no pointer after it returns and
 *     holds no global mutable state: calls are reentrant. (The one exception is dsa_topk_noalloc, which uses
 *     a device array the library holds; see there.) Buffers must stay alive until the stream has run the
 *     kernels. Outputs must not alias inputs.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Every call is asynchronous on it.
 *   - All argument checks run on the host, before any launch. A call that fails a check launches nothing
 *     and returns a non-zero dsa_status; dsa_last_error() then gives a message for the calling thread.
 *   - Device-side contract violations are not checked on the device and their results are undefined: a
 *     page id outside the pool, a q_pos or q_seq outside the ranges dsa_batch states, NaN scores given to
 *     dsa_topk. (Index entries outside 0 .. q_pos[r] are not a violation: dsa_sparse_attn skips them.)
 *   - Tensor pointers must be 16-byte aligned (vector loads); otherwise DSA_ERR_INVALID_ARGUMENT.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, negative size, k < 1, ld too small ... */
  DSA_ERR_UNSUPPORTED = 2,      /* a shape or dtype with no compiled kernel */
  DSA_ERR_WORKSPACE = 3,        /* workspace pointer NULL or smaller than the *_workspace_size query */
  DSA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} dsa_status;

typedef enum {
  DSA_BF16 = 0,       /* bfloat16 */
  DSA_FP8_E4M3FN = 1  /* OCP FP8 E4M3 (finite-only, max 448), one byte per element */
} dsa_dtype;

/*
 * dsa_batch — which query rows exist and where their sequence's cached tokens live.
 *
 * Query row r (0 <= r < num_q) belongs to sequence b = q_seq[r] and sits at logical position p = q_pos[r]
 * in that sequence. Its causal candidates are the positions s = 0 .. p (the query's own token included).
 * Logical position s of sequence b lives in cache row ("slot"):
 *   contiguous (page_table == NULL):  slot(b, s) = b * seq_stride + s
 *   paged      (page_table != NULL):  slot(b, s) = page_table[b * max_pages + s / page_size] * page_size
 *                                                 + s % page_size
 * The same slot map addresses the indexer key cache and the latent cache.
 *
 * Host fields size the launch grids and are never read on the device. The caller guarantees, for every r:
 * 0 <= q_pos[r] < max_kv_len, 0 <= q_seq[r] < num_seqs, and rows of one sequence are stored
 * consecutively (q_seq non-decreasing), which lets the indexer share a key tile across such rows.
 */
typedef struct {
  int32_t num_seqs;          /* host: number of sequences (>= 1) */
  int32_t num_q;             /* host: number of query rows (>= 0; 0 = nothing to do) */
  int32_t max_kv_len;        /* host: > every q_pos[r]; row length bound of the score matrix */
  int32_t page_size;         /* host: tokens per page when paged (64 is compiled); ignored otherwise */
  int32_t max_pages;         /* host: row length of page_table when paged */
  int32_t reserved;          /* must be 0 */
  int64_t seq_stride;        /* host: contiguous layout only, >= max_kv_len when num_seqs > 1 */
  const int32_t *q_seq;      /* device [num_q] */
  const int32_t *q_pos;      /* device [num_q] */
  const int32_t *page_table; /* device [num_seqs * max_pages], or NULL for the contiguous layout */
} dsa_batch;

/* Human-readable name of a status code. Never NULL; the string is static. */
const char *dsa_status_string(dsa_status s);

/* Detail of the calling thread's last non-OK return ("" if none). Valid until the thread's next call. */
const char *dsa_last_error(void);

/*
 * dsa_indexer_scores — lightning-indexer scores for every causal (query row, key) pair.
 *   scores[r * ld_scores + s] = sum_{j < H_I} w[r, j] * ReLU( sigma_s * dot(q_idx[r, j, :], k_idx[slot(b, s), :]) )
 *   for s = 0 .. q_pos[r]; entries with s > q_pos[r] are left untouched.
 * Defined by: GLM sparse-attention essay, the paragraph on the indexer's ReLU (a non-negative sum of
 * per-head evidence, robust in low precision); "DeepSeek Sparse Attention" explainer, sections
 * "Make a shortlist first" and "The lightning indexer" (the indexer scans every earlier token; its scores
 * pick positions and are not attention weights).
 *   q_idx   [num_q, H_I, d_I] bf16            indexer queries
 *   w       [num_q, H_I]      fp32            per-(query, head) weights, any finite value
 *   k_idx   [slots, d_I]      bf16 or fp8     indexer key cache (k_dtype)
 *   k_scale [slots]           fp32 > 0        per-token dequantisation scale sigma_s; required iff fp8,
 *                                              must be NULL for bf16 (sigma_s = 1)
 *   scores  [num_q, ld_scores] fp32           output; ld_scores >= max_kv_len, multiple of 4
 * Products are exact (fp8 keys up-convert exactly to bf16); sums accumulate in fp32. Since sigma_s > 0 the
 * scale is applied after the head sum, which is the same value.
 * Compiled shapes: (H_I, d_I) in {(4, 32), (64, 128)}; otherwise DSA_ERR_UNSUPPORTED.
 */
dsa_status dsa_indexer_scores(const dsa_batch *b, const void *q_idx, const float *w, const void *k_idx,
                              dsa_dtype k_dtype, const float *k_scale, int32_t H_I, int32_t d_I,
                              float *scores, int64_t ld_scores, void *stream);

/* Bytes of device workspace dsa_topk needs for this batch and k (may be 0). */
dsa_status dsa_topk_workspace_size(const dsa_batch *b, int32_t k, size_t *bytes);

/*
 * dsa_topk — per-row causal top-k selection.
 *   Row r reads scores[r * ld_scores + s] for s = 0 .. q_pos[r] only. If q_pos[r] + 1 <= k every candidate
 *   is kept; otherwise the k candidates with the largest score are kept. Scores compare as fp32 values
 *   (-0.0 == +0.0); among equal scores the lower position wins.
 *   idx[r * k + i], i < k: the kept positions in ascending order, then -1 up to length k.
 * Defined by: GLM sparse-attention essay, the paragraph on the needle (the cut-off falls to the k-th best
 * score); "Sparse Attention Architecture Evolution in LLMs", section "Top-K Selection: A Hard Filtering
 * Mechanism" (a fixed budget k per query token, 2048 in a shipped model); "DeepSeek Sparse Attention"
 * explainer, sections "Select individual positions" and "The top-k budget" (token-level choice; a token
 * not kept cannot contribute).
 *   scores [num_q, ld_scores] fp32, ld_scores >= max_kv_len;  idx [num_q, k] int32 (output)
 *   ws / ws_bytes: device workspace of at least dsa_topk_workspace_size bytes (NULL allowed when 0).
 * Limits: 1 <= k <= 4096, max_kv_len <= 1 << 20; otherwise DSA_ERR_UNSUPPORTED.
 */
dsa_status dsa_topk(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t k, int32_t *idx,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_topk_noalloc — dsa_topk for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, rules and result as dsa_topk, without the
 * workspace: the plans that need one (few rows over long contexts, e.g. decode batches) use a device array the
 * library holds, DSA_TOPK_NOALLOC_SCRATCH_BYTES per GPU, from the first call on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine); it resolves the array's
 * device address once per device, on the calling thread's current device, which must be the stream's device.
 *   A batch whose dsa_topk_workspace_size exceeds DSA_TOPK_NOALLOC_SCRATCH_BYTES: DSA_ERR_UNSUPPORTED, nothing
 *   launched. Every call on one GPU shares that GPU's array and nothing in it must start at any value (each call
 *   writes the parts it reads), but calls that overlap on one GPU (other streams, other threads) race on it.
 */
#define DSA_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dsa_status dsa_topk_noalloc(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t k, int32_t *idx,
                            void *stream);

/* Bytes of device workspace dsa_sparse_attn needs for this batch and shape (may be 0). */
dsa_status dsa_sparse_attn_workspace_size(const dsa_batch *b, int32_t k, int32_t H, int32_t D_v,
                                          size_t *bytes);

/*
 * dsa_sparse_attn — exact softmax attention of every query head over the rows its row's idx selects.
 *   For row r with sequence b and head h, over the valid entries i (idx[r, i] != -1), c_i = latent[slot(b, idx[r, i])]:
 *     z_i = sm_scale * dot(q[r, h, 0:D_qk], c_i[0:D_qk])
 *     out[r, h, :] = sum_i softmax(z)_i * c_i[0:D_v]          lse[r, h] = log(sum_i exp(z_i))
 *   A row with no valid entry gets out = 0 and lse = -inf. Duplicate entries count as listed. Entries
 *   outside 0 .. q_pos[r] are skipped like -1 (the library never reads a cache row past the query).
 * Defined by: GLM sparse-attention essay, the paragraphs on the exact softmax over the survivors, on MLA's
 * absorbed read (one cached latent per token serves every head, MQA-like) and on the gather kernels;
 * "DeepSeek Sparse Attention" explainer, section "Indexing and main attention are separate".
 *   q      [num_q, H, D_qk] bf16      absorbed queries
 *   latent [slots, D_qk]    bf16      latent cache; the value is its first D_v columns
 *   idx    [num_q, k]       int32     logical positions (0 .. q_pos[r]) or -1
 *   out    [num_q, H, D_v]  bf16      output;   lse [num_q, H] fp32 output, or NULL
 * sm_scale must be finite and > 0 (it is 1/sqrt(head dim) in practice), else DSA_ERR_INVALID_ARGUMENT.
 * The softmax is computed in fp32 with an online max; products run on bf16 MFMA with fp32 accumulation.
 * Compiled shapes: (H, D_qk, D_v) in {(8, 80, 64), (128, 576, 512)}, 1 <= k <= 4096. Rows whose list is longer
 * than 2048 entries, or batches of few rows, are split across workgroups and merged through the workspace.
 */
dsa_status dsa_sparse_attn(const dsa_batch *b, const void *q, const void *latent, const int32_t *idx,
                           int32_t k, int32_t H, int32_t D_qk, int32_t D_v, float sm_scale, void *out,
                           float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_cache_append — write the batch's query tokens into the caches the three calls above read (the step
 * before a decode step: the cache holds the query tokens, q_pos[r] = kv_len - num_new + i).
 *   For every row r, with slot = slot(q_seq[r], q_pos[r]) (the batch's slot map):
 *     sigma = max(max_d |k_new[r, d]|, FLT_MIN) / 448                      (fp32, correctly rounded)
 *     k_pool[slot, d] = E4M3( clamp(k_new[r, d] / sigma, -448, 448) )       (fp32 quotient, round to nearest even)
 *     k_scale[slot] = sigma;   latent_pool[slot, :] = latent_new[r, :]       (bit copy)
 * Defined by: GLM sparse-attention essay, the paragraphs on MLA (one cached latent row per token) and on the
 * indexer's ReLU (the indexer runs in FP8); the per-token absolute-maximum scale is a reading (the pages do
 * not say how the FP8 keys are scaled), and it is the format dsa_indexer_scores reads (k_dtype FP8, k_scale).
 *   k_new       [num_q, d_I]  fp32     new indexer keys (finite)
 *   latent_new  [num_q, D_qk] bf16     new latent rows
 *   k_pool      [slots, d_I]  E4M3     indexer key cache (written at the rows' slots only)
 *   k_scale     [slots]       fp32     its per-token scales (written at the rows' slots only)
 *   latent_pool [slots, D_qk] bf16     latent cache (written at the rows' slots only)
 * Two rows with the same slot race (undefined which one lands). Compiled d_I: 128, 32; D_qk a multiple of 8
 * up to 8192; otherwise DSA_ERR_UNSUPPORTED. Pointers 16-byte aligned (k_scale 4).
 */
dsa_status dsa_cache_append(const dsa_batch *b, const float *k_new, int32_t d_I, const void *latent_new,
                            int32_t D_qk, void *k_pool, float *k_scale, void *latent_pool, void *stream);

/*
 * dsa_indexer_topk — the indexer and the top-k in one call: the scores never reach device memory.
 *   idx[r, :] = the selection dsa_topk makes (same rules: ties to the lower position, ascending, -1 padded)
 *   from the fp32 scores of dsa_indexer_scores' formula, summed in a fixed order (per 32-head tile, heads in
 *   accumulator order, the two half-waves added, sigma applied last) — the order dsa_indexer_scores uses for
 *   decode batches (fewer than 8 rows per sequence, or FP8 or paged keys), so there the two paths select the
 *   same positions.
 * Defined by: "Sparse Attention Architecture Evolution in LLMs", section "Deployment Practice: Memory Planning
 * and Optimization" (fusing the indexer operators), over the definitions of dsa_indexer_scores and dsa_topk.
 *   Arguments as dsa_indexer_scores (q_idx, w, k_idx, k_dtype, k_scale, H_I, d_I) and dsa_topk (k, idx).
 *   ws: at least dsa_indexer_topk_workspace_size bytes (per row and 8192-key chunk, k candidates).
 * Compiled: (H_I, d_I) = (64, 128); 1 <= k <= 4096 with ceil(max_kv_len / 8192) * k <= 65536. Built for decode
 * batches: each workgroup scores one row's 8192-key chunk, so rows of one sequence do not share key reads.
 */
dsa_status dsa_indexer_topk_workspace_size(const dsa_batch *b, int32_t H_I, int32_t d_I, int32_t k, size_t *bytes);
dsa_status dsa_indexer_topk(const dsa_batch *b, const void *q_idx, const float *w, const void *k_idx,
                            dsa_dtype k_dtype, const float *k_scale, int32_t H_I, int32_t d_I, int32_t k,
                            int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/*
 * Block-versus-token comparator. The "DeepSeek Sparse Attention" explainer (section "Select individual
 * positions") contrasts DSA's selection of individual positions with reading every token of a selected block:
 * scattered useful tokens make a block reader pay for whole blocks ("tokens actually read", "extra work").
 *
 * dsa_block_topk — block selection with the token budget k_blocks * block, for comparison with dsa_topk.
 *   Block j of row r covers the causal positions j*block .. min((j+1)*block, q_pos[r]+1) - 1 and scores as the
 *   largest of their scores (a reading: the pages do not say how a block is ranked). The k_blocks best blocks
 *   are kept (ranked like dsa_topk: fp32 compare, ties to the lower block; all blocks when there are at most
 *   k_blocks) and idx[r, :] lists every causal position of the kept blocks, ascending, then -1 up to
 *   k_blocks * block entries — an index list dsa_sparse_attn takes as it is.
 *   scores [num_q, ld_scores] fp32 (ld_scores >= max_kv_len, multiple of 4); idx [num_q, k_blocks*block] int32
 *   ws: at least dsa_block_topk_workspace_size bytes, 256-byte aligned (block scores, block positions, the
 *   block-level top-k and its own workspace).
 * Compiled block sizes: 16, 32, 64, 128, 256; 1 <= k_blocks <= 4096.
 */
dsa_status dsa_block_topk_workspace_size(const dsa_batch *b, int32_t block, int32_t k_blocks, size_t *bytes);
dsa_status dsa_block_topk(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t block,
                          int32_t k_blocks, int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_block_cover — what reading whole blocks would cost for a token selection.
 *   idx [num_q, k] int32 in dsa_topk's form (ascending, -1 padded; entries outside 0 .. q_pos[r] ignored).
 *   counts[r, 0..2] = useful tokens (distinct valid entries), distinct blocks touched (position / block), and
 *   tokens read, i.e. the causal positions of those blocks (the block holding q_pos[r] stops there).
 * Any block >= 1. An unsorted list gives undefined counts.
 */
dsa_status dsa_block_cover(const dsa_batch *b, const int32_t *idx, int32_t k, int32_t block, int32_t *counts,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
