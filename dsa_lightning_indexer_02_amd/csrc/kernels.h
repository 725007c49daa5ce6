// Internal launch functions of the libdsa kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

struct IndexerArgs {
  const void *q_idx;        // [num_q, H_I, d_I] bf16
  const float *w;           // [num_q, H_I]
  const void *k_idx;        // [slots, d_I] bf16 or fp8
  const float *k_scale;     // [slots] (fp8) or nullptr
  const int32_t *q_seq;
  const int32_t *q_pos;
  SlotMap slot;
  float *scores;
  int64_t ld;
  int num_q;
  int max_kv_len;
  bool fp8;
  int H_I, d_I;
};
hipError_t launch_indexer(const IndexerArgs &a, int rows_per_wg, int target_wgs, hipStream_t s);
hipError_t launch_indexer_topk(const IndexerArgs &a, int k, uint32_t *cand_key, int32_t *cand_pos, int32_t *idx,
                               hipStream_t s);
size_t indexer_topk_ws_bytes(int num_q, int max_kv_len, int k);
hipError_t launch_topk_merge(const int32_t *q_pos, int num_q, int k, int chunk, int n_chunks, const uint32_t *cand_key,
                             const int32_t *cand_pos, int32_t *idx, hipStream_t s);

hipError_t launch_topk_rows(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k,
                            int32_t *idx, int items, hipStream_t s);
hipError_t launch_topk_stream(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k, int32_t *idx,
                              hipStream_t s);
hipError_t launch_topk_windowed(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int k, int chunk,
                                int n_chunks, void *ws, int32_t *idx, hipStream_t s);
size_t topk_windowed_ws_bytes(int num_q, int n_chunks, int cap);

struct AttnArgs {
  const void *q;            // [num_q, H, D_qk] bf16
  const void *latent;       // [slots, D_qk] bf16
  const int32_t *idx;       // [num_q, k]
  const int32_t *q_seq;
  const int32_t *q_pos;
  SlotMap slot;
  void *out;                // [num_q, H, D_v] bf16
  float *lse;               // [num_q, H] or nullptr
  float *ws;                // split partials (fp32) or nullptr
  int num_q, k, H, D_qk, D_v;
  float sm_scale;
  int splits;               // key-list splits per row (1 = no combine pass)
  int64_t max_slots;        // contiguous caches: an upper bound on the slots the batch addresses; 0 = unknown
};
hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t s);
size_t sparse_attn_ws_floats(int num_q, int splits, int H, int D_v);

struct AppendArgs {
  const float *k_new;       // [num_q, d_I] fp32
  const void *latent_new;   // [num_q, D_qk] bf16
  const int32_t *q_seq;
  const int32_t *q_pos;
  SlotMap slot;
  void *k_pool;             // [slots, d_I] e4m3fn
  float *k_scale;           // [slots]
  void *latent_pool;        // [slots, D_qk] bf16
  int num_q, D_qk;
};
hipError_t launch_cache_append(const AppendArgs &a, int d_I, hipStream_t s);

hipError_t launch_block_scores(const float *scores, int64_t ld, const int32_t *q_pos, int num_q, int max_kv_len,
                               int B, float *bs, int64_t ldb, int32_t *blk_pos, hipStream_t s);
hipError_t launch_block_expand(const int32_t *blk, int kb, int B, const int32_t *q_pos, int num_q, int32_t *idx,
                               hipStream_t s);
hipError_t launch_block_cover(const int32_t *idx, int k, int B, const int32_t *q_pos, int num_q, int32_t *counts,
                              hipStream_t s);

}  // namespace dsa
