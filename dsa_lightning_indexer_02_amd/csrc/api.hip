// libdsa C ABI: argument checks, kernel dispatch and workspace sizing for the three DSA calls.
// The contract of every entry point is stated in include/dsa.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dsa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status ok() { return DSA_OK; }

dsa_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

int pow2_ceil(long long x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

#define DSA_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

dsa_status check_batch(const dsa_batch *b) {
  DSA_CHECK(b != nullptr, DSA_ERR_INVALID_ARGUMENT, "batch is NULL");
  DSA_CHECK(b->num_seqs >= 1, DSA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1 (got %d)", b->num_seqs);
  DSA_CHECK(b->num_q >= 0, DSA_ERR_INVALID_ARGUMENT, "num_q must be >= 0 (got %d)", b->num_q);
  DSA_CHECK(b->max_kv_len >= 1, DSA_ERR_INVALID_ARGUMENT, "max_kv_len must be >= 1 (got %d)", b->max_kv_len);
  DSA_CHECK(b->reserved == 0, DSA_ERR_INVALID_ARGUMENT, "reserved field must be 0");
  if (b->num_q > 0) {
    DSA_CHECK(b->q_seq != nullptr && b->q_pos != nullptr, DSA_ERR_INVALID_ARGUMENT, "q_seq / q_pos is NULL");
    DSA_CHECK(aligned(b->q_seq, 4) && aligned(b->q_pos, 4), DSA_ERR_INVALID_ARGUMENT,
              "q_seq / q_pos must be 4-byte aligned");
  }
  if (b->page_table != nullptr) {
    DSA_CHECK(aligned(b->page_table, 4), DSA_ERR_INVALID_ARGUMENT, "page_table must be 4-byte aligned");
    DSA_CHECK(b->page_size >= 1 && (b->page_size & (b->page_size - 1)) == 0 && b->page_size <= (1 << 20),
              DSA_ERR_UNSUPPORTED, "page_size must be a power of two in [1, 2^20] (got %d)", b->page_size);
    DSA_CHECK(b->max_pages >= 1 && (long long)b->max_pages * b->page_size >= b->max_kv_len,
              DSA_ERR_INVALID_ARGUMENT, "max_pages * page_size (%d * %d) must cover max_kv_len %d", b->max_pages,
              b->page_size, b->max_kv_len);
  } else {
    DSA_CHECK(b->seq_stride >= 0, DSA_ERR_INVALID_ARGUMENT, "seq_stride must be >= 0");
    DSA_CHECK(b->num_seqs == 1 || b->seq_stride >= b->max_kv_len, DSA_ERR_INVALID_ARGUMENT,
              "seq_stride (%lld) must be >= max_kv_len (%d) when num_seqs > 1", (long long)b->seq_stride,
              b->max_kv_len);
  }
  return ok();
}

dsa::SlotMap slot_map(const dsa_batch *b) {
  dsa::SlotMap m;
  m.page_table = b->page_table;
  m.seq_stride = b->seq_stride;
  m.max_pages = b->max_pages;
  int sh = 0;
  if (b->page_table != nullptr)
    while ((1 << sh) < b->page_size) ++sh;
  m.page_shift = sh;
  return m;
}

// ---- top-k plan: batches that fill the GPU take one workgroup per row, rows of at least
//      kTopkStreamMinLen through the streaming form (sampled window, nothing held in registers) and shorter
//      ones held in registers; otherwise (few rows: decode) each row splits into chunks that keep only the keys
//      of a sampled window, and a merge pass selects among them (the windowed form).
constexpr long long kTopkStreamMinLen = 8192;
struct TopkPlan {
  bool windowed, stream;
  int items_a, chunk, n_chunks;
  size_t ws_bytes;
};

TopkPlan plan_topk(const dsa_batch *b, int k) {
  TopkPlan p{};
  const long long L = b->max_kv_len;
  if (L > k && b->num_q >= 512 && L >= kTopkStreamMinLen) {
    p.stream = true;
    return p;
  }
  if ((L <= 65536 && b->num_q >= 512) || L <= k) {
    p.items_a = pow2_ceil(ceil_div(L, 1024));
    return p;
  }
  // about 256 chunk workgroups in all (chunks of 4096, 8192 or 16384 keys, one 256-thread workgroup each, at most
  // 256 per row: L <= 2^20 needs at most 64)
  const int chunk = std::min(16384, std::max(4096, pow2_ceil(ceil_div(L * b->num_q, 256))));
  p.windowed = true;
  p.chunk = chunk;
  p.n_chunks = ceil_div(L, chunk);
  p.ws_bytes = dsa::topk_windowed_ws_bytes(b->num_q, p.n_chunks, std::min(k, chunk));
  return p;
}

// ---- attention plan: split the key list across workgroups when the batch has too few rows to fill the GPU.
// Key-list splits per row: at least enough that one workgroup attends to at most kAttnKeysPerWorkgroup
// entries (its compacted row list lives in LDS), more when few rows would leave the chip idle, but no split
// shorter than 256 entries: every split reads the row's Q and writes a partial output (128 KB each at 128
// heads), which would outweigh its share of the gather (16 rows of 2048: 8 splits 39 us, 16 splits 45 us).
constexpr int kAttnKeysPerWorkgroup = 2048;
int plan_attn_splits(const dsa_batch *b, int k) {
  const int need = ceil_div(k, kAttnKeysPerWorkgroup);
  if (b->num_q >= 256) return need;
  const int cap = std::max(1, k / 256);
  return std::max(need, std::min(cap, std::max(1, ceil_div(256, std::max(1, b->num_q)))));
}

// Launches of dsa_topk's plan (arguments already checked; ws holds the plan's workspace bytes).
dsa_status topk_launch(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t k, int32_t *idx, void *ws,
                       hipStream_t stream) {
  const TopkPlan p = plan_topk(b, k);
  hipError_t e;
  if (p.stream) {
    e = dsa::launch_topk_stream(scores, ld_scores, b->q_pos, b->num_q, k, idx, stream);
  } else if (!p.windowed) {
    e = dsa::launch_topk_rows(scores, ld_scores, b->q_pos, b->num_q, k, idx, p.items_a, stream);
  } else {
    e = dsa::launch_topk_windowed(scores, ld_scores, b->q_pos, b->num_q, k, p.chunk, p.n_chunks, ws, idx, stream);
  }
  return from_hip(e, "dsa_topk launch");
}

// ---- the no-allocation top-k: its workspace is this file-scope device array. In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the address hipGetSymbolAddress reports, taken
// once per device with that device current (each device holds its own copy of the array).
constexpr size_t kNoallocScratchBytes = DSA_TOPK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "dsa_topk_noalloc: hipGetDevice");
  DSA_CHECK(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED, "dsa_topk_noalloc: device %d (at most %d devices)",
            dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "dsa_topk_noalloc: hipGetSymbolAddress");
    DSA_CHECK(p != nullptr, DSA_ERR_HIP, "dsa_topk_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

const char *dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char *dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status dsa_indexer_scores(const dsa_batch *b, const void *q_idx, const float *w, const void *k_idx,
                              dsa_dtype k_dtype, const float *k_scale, int32_t H_I, int32_t d_I, float *scores,
                              int64_t ld_scores, void *stream) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3FN, DSA_ERR_INVALID_ARGUMENT, "unknown k_dtype %d",
            (int)k_dtype);
  DSA_CHECK((H_I == 64 && d_I == 128) || (H_I == 4 && d_I == 32), DSA_ERR_UNSUPPORTED,
            "no indexer kernel for (H_I, d_I) = (%d, %d); compiled: (64, 128), (4, 32)", H_I, d_I);
  DSA_CHECK(ld_scores >= b->max_kv_len && ld_scores % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) must be >= max_kv_len (%d) and a multiple of 4", (long long)ld_scores, b->max_kv_len);
  if (b->num_q == 0) return ok();
  DSA_CHECK(q_idx && w && k_idx && scores, DSA_ERR_INVALID_ARGUMENT, "q_idx, w, k_idx and scores must be non-NULL");
  DSA_CHECK(aligned(q_idx, 16) && aligned(w, 16) && aligned(k_idx, 16) && aligned(scores, 16),
            DSA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if (k_dtype == DSA_FP8_E4M3FN) {
    DSA_CHECK(k_scale != nullptr && aligned(k_scale, 4), DSA_ERR_INVALID_ARGUMENT,
              "FP8 keys need a 4-byte aligned per-token k_scale");
  } else {
    DSA_CHECK(k_scale == nullptr, DSA_ERR_INVALID_ARGUMENT, "k_scale must be NULL for bf16 keys");
  }
  dsa::IndexerArgs a{};
  a.q_idx = q_idx;
  a.w = w;
  a.k_idx = k_idx;
  a.k_scale = k_scale;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.slot = slot_map(b);
  a.scores = scores;
  a.ld = ld_scores;
  a.num_q = b->num_q;
  a.max_kv_len = b->max_kv_len;
  a.fp8 = (k_dtype == DSA_FP8_E4M3FN);
  a.H_I = H_I;
  a.d_I = d_I;
  const double rows_per_seq = (double)b->num_q / b->num_seqs;
  const int rows_per_wg = rows_per_seq >= 8 ? 8 : (rows_per_seq >= 2 ? 2 : 1);
  // Few rows per sequence (decode): the key range of each row is split so that the batch makes about one
  // workgroup per CU, each streaming a long stretch of keys (a second round of workgroups would pay the
  // row-operand load and the tile pipeline's fill again; measured 95 -> 79 us on 64 x 32K FP8 keys).
  const int target_wgs = rows_per_wg >= 8 ? 1024 : 256;
  return from_hip(dsa::launch_indexer(a, rows_per_wg, target_wgs, (hipStream_t)stream), "dsa_indexer_scores launch");
}

dsa_status dsa_topk_workspace_size(const dsa_batch *b, int32_t k, size_t *bytes) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(bytes != nullptr, DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DSA_CHECK(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k must be >= 1 (got %d)", k);
  DSA_CHECK(k <= 4096 && b->max_kv_len <= (1 << 20), DSA_ERR_UNSUPPORTED,
            "top-k supports k <= 4096 and max_kv_len <= 2^20 (got k=%d, max_kv_len=%d)", k, b->max_kv_len);
  *bytes = b->num_q == 0 ? 0 : plan_topk(b, k).ws_bytes;
  return ok();
}

dsa_status dsa_topk(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t k, int32_t *idx, void *ws,
                    size_t ws_bytes, void *stream) {
  size_t need = 0;
  dsa_status st = dsa_topk_workspace_size(b, k, &need);
  if (st != DSA_OK) return st;
  DSA_CHECK(ld_scores >= b->max_kv_len, DSA_ERR_INVALID_ARGUMENT, "ld_scores (%lld) must be >= max_kv_len (%d)",
            (long long)ld_scores, b->max_kv_len);
  if (b->num_q == 0) return ok();
  DSA_CHECK(scores && idx, DSA_ERR_INVALID_ARGUMENT, "scores and idx must be non-NULL");
  DSA_CHECK(aligned(scores, 16) && aligned(idx, 16), DSA_ERR_INVALID_ARGUMENT, "scores / idx must be 16-byte aligned");
  DSA_CHECK(ws_bytes >= need && (need == 0 || ws != nullptr), DSA_ERR_WORKSPACE,
            "top-k needs %zu bytes of workspace (got %zu)", need, ws_bytes);
  DSA_CHECK(need == 0 || aligned(ws, 16), DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return topk_launch(b, scores, ld_scores, k, idx, ws, (hipStream_t)stream);
}

dsa_status dsa_topk_noalloc(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t k, int32_t *idx,
                            void *stream) {
  size_t need = 0;
  dsa_status st = dsa_topk_workspace_size(b, k, &need);
  if (st != DSA_OK) return st;
  DSA_CHECK(need <= kNoallocScratchBytes, DSA_ERR_UNSUPPORTED,
            "dsa_topk_noalloc: this batch needs %zu bytes of scratch; the library holds %zu (use dsa_topk with a "
            "workspace)", need, kNoallocScratchBytes);
  DSA_CHECK(ld_scores >= b->max_kv_len, DSA_ERR_INVALID_ARGUMENT, "ld_scores (%lld) must be >= max_kv_len (%d)",
            (long long)ld_scores, b->max_kv_len);
  if (b->num_q == 0) return ok();
  DSA_CHECK(scores && idx, DSA_ERR_INVALID_ARGUMENT, "scores and idx must be non-NULL");
  DSA_CHECK(aligned(scores, 16) && aligned(idx, 16), DSA_ERR_INVALID_ARGUMENT, "scores / idx must be 16-byte aligned");
  void *ws = nullptr;
  if (need > 0) {
    st = scratch_of_current_device(&ws);
    if (st != DSA_OK) return st;
  }
  return topk_launch(b, scores, ld_scores, k, idx, ws, (hipStream_t)stream);
}

dsa_status dsa_sparse_attn_workspace_size(const dsa_batch *b, int32_t k, int32_t H, int32_t D_v, size_t *bytes) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(bytes != nullptr, DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DSA_CHECK(k >= 1 && H >= 1 && D_v >= 1, DSA_ERR_INVALID_ARGUMENT, "k, H and D_v must be >= 1");
  DSA_CHECK(k <= 4096, DSA_ERR_UNSUPPORTED, "sparse attention supports k <= 4096 (got %d)", k);
  *bytes = b->num_q == 0 ? 0 : dsa::sparse_attn_ws_floats(b->num_q, plan_attn_splits(b, k), H, D_v) * sizeof(float);
  return ok();
}

dsa_status dsa_sparse_attn(const dsa_batch *b, const void *q, const void *latent, const int32_t *idx, int32_t k,
                           int32_t H, int32_t D_qk, int32_t D_v, float sm_scale, void *out, float *lse, void *ws,
                           size_t ws_bytes, void *stream) {
  size_t need = 0;
  dsa_status st = dsa_sparse_attn_workspace_size(b, k, H, D_v, &need);
  if (st != DSA_OK) return st;
  DSA_CHECK((H == 128 && D_qk == 576 && D_v == 512) || (H == 8 && D_qk == 80 && D_v == 64), DSA_ERR_UNSUPPORTED,
            "no attention kernel for (H, D_qk, D_v) = (%d, %d, %d); compiled: (128, 576, 512), (8, 80, 64)", H, D_qk,
            D_v);
  DSA_CHECK(std::isfinite(sm_scale) && sm_scale > 0.f, DSA_ERR_INVALID_ARGUMENT,
            "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (b->num_q == 0) return ok();
  DSA_CHECK(q && latent && idx && out, DSA_ERR_INVALID_ARGUMENT, "q, latent, idx and out must be non-NULL");
  DSA_CHECK(aligned(q, 16) && aligned(latent, 16) && aligned(idx, 16) && aligned(out, 16) &&
                (lse == nullptr || aligned(lse, 4)),
            DSA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned (lse 4-byte)");
  DSA_CHECK(ws_bytes >= need && (need == 0 || ws != nullptr), DSA_ERR_WORKSPACE,
            "sparse attention needs %zu bytes of workspace (got %zu)", need, ws_bytes);
  DSA_CHECK(need == 0 || aligned(ws, 16), DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  dsa::AttnArgs a{};
  a.q = q;
  a.latent = latent;
  a.idx = idx;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.slot = slot_map(b);
  a.out = out;
  a.lse = lse;
  a.ws = static_cast<float *>(ws);
  a.num_q = b->num_q;
  a.k = k;
  a.H = H;
  a.D_qk = D_qk;
  a.D_v = D_v;
  a.sm_scale = sm_scale;
  a.splits = plan_attn_splits(b, k);
  // the contiguous slot map addresses rows below (num_seqs - 1) * seq_stride + max_kv_len (entries past q_pos
  // are skipped); a paged map's page ids are not known on the host
  a.max_slots = b->page_table != nullptr ? 0 : (int64_t)(b->num_seqs - 1) * b->seq_stride + b->max_kv_len;
  return from_hip(dsa::launch_sparse_attn(a, (hipStream_t)stream), "dsa_sparse_attn launch");
}

}  // extern "C"

extern "C" dsa_status dsa_cache_append(const dsa_batch *b, const float *k_new, int32_t d_I, const void *latent_new,
                                       int32_t D_qk, void *k_pool, float *k_scale, void *latent_pool, void *stream) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(d_I == 128 || d_I == 32, DSA_ERR_UNSUPPORTED, "no cache-append kernel for d_I = %d; compiled: 128, 32",
            d_I);
  DSA_CHECK(D_qk >= 8 && D_qk % 8 == 0 && D_qk <= 8192, DSA_ERR_UNSUPPORTED,
            "D_qk must be a multiple of 8 in [8, 8192] (got %d)", D_qk);
  if (b->num_q == 0) return ok();
  DSA_CHECK(k_new && latent_new && k_pool && k_scale && latent_pool, DSA_ERR_INVALID_ARGUMENT,
            "k_new, latent_new, k_pool, k_scale and latent_pool must be non-NULL");
  DSA_CHECK(aligned(k_new, 16) && aligned(latent_new, 16) && aligned(k_pool, 16) && aligned(k_scale, 4) &&
                aligned(latent_pool, 16),
            DSA_ERR_INVALID_ARGUMENT, "k_new, latent_new, k_pool and latent_pool must be 16-byte aligned, k_scale 4");
  dsa::AppendArgs a{};
  a.k_new = k_new;
  a.latent_new = latent_new;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.slot = slot_map(b);
  a.k_pool = k_pool;
  a.k_scale = k_scale;
  a.latent_pool = latent_pool;
  a.num_q = b->num_q;
  a.D_qk = D_qk;
  return from_hip(dsa::launch_cache_append(a, d_I, (hipStream_t)stream), "dsa_cache_append launch");
}

// ---- block-versus-token comparator
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
struct BlockPlan {
  int max_blocks;
  int64_t ldb;
  size_t off_pos, off_blk, off_tk, tk_bytes, total;
  dsa_batch bb;   // the rows over block positions (q_pos points into the workspace once it is known)
};
dsa_status plan_blocks(const dsa_batch *b, int block, int k_blocks, BlockPlan *pl) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(block == 16 || block == 32 || block == 64 || block == 128 || block == 256, DSA_ERR_UNSUPPORTED,
            "block must be 16, 32, 64, 128 or 256 (got %d)", block);
  DSA_CHECK(k_blocks >= 1, DSA_ERR_INVALID_ARGUMENT, "k_blocks must be >= 1 (got %d)", k_blocks);
  DSA_CHECK(k_blocks <= 4096, DSA_ERR_UNSUPPORTED, "k_blocks must be <= 4096 (got %d)", k_blocks);
  pl->max_blocks = ceil_div(b->max_kv_len, block);
  pl->ldb = (pl->max_blocks + 3) / 4 * 4;
  dsa_batch bb{};
  bb.num_seqs = 1;
  bb.num_q = b->num_q;
  bb.max_kv_len = pl->max_blocks;
  bb.seq_stride = pl->max_blocks;
  bb.q_seq = b->q_seq;
  bb.q_pos = b->q_pos;   // placeholder until the workspace address is known (sizes only depend on shapes)
  size_t tk = 0;
  st = dsa_topk_workspace_size(&bb, k_blocks, &tk);
  if (st != DSA_OK) return st;
  const size_t nq = (size_t)b->num_q;
  pl->off_pos = align256(nq * pl->ldb * 4);
  pl->off_blk = pl->off_pos + align256(nq * 4);
  pl->off_tk = pl->off_blk + align256(nq * (size_t)k_blocks * 4);
  pl->tk_bytes = tk;
  pl->total = nq == 0 ? 0 : pl->off_tk + align256(tk);
  pl->bb = bb;
  return ok();
}
}  // namespace

extern "C" dsa_status dsa_block_topk_workspace_size(const dsa_batch *b, int32_t block, int32_t k_blocks,
                                                     size_t *bytes) {
  DSA_CHECK(bytes != nullptr, DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BlockPlan pl{};
  dsa_status st = plan_blocks(b, block, k_blocks, &pl);
  if (st != DSA_OK) return st;
  *bytes = pl.total;
  return ok();
}

extern "C" dsa_status dsa_block_topk(const dsa_batch *b, const float *scores, int64_t ld_scores, int32_t block,
                                     int32_t k_blocks, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
  BlockPlan pl{};
  dsa_status st = plan_blocks(b, block, k_blocks, &pl);
  if (st != DSA_OK) return st;
  DSA_CHECK(ld_scores >= b->max_kv_len && ld_scores % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) must be >= max_kv_len (%d) and a multiple of 4", (long long)ld_scores, b->max_kv_len);
  if (b->num_q == 0) return ok();
  DSA_CHECK(scores && idx, DSA_ERR_INVALID_ARGUMENT, "scores and idx must be non-NULL");
  DSA_CHECK(aligned(scores, 16) && aligned(idx, 16), DSA_ERR_INVALID_ARGUMENT, "scores / idx must be 16-byte aligned");
  DSA_CHECK(ws != nullptr && ws_bytes >= pl.total, DSA_ERR_WORKSPACE, "block top-k needs %zu bytes of workspace (got %zu)",
            pl.total, ws_bytes);
  DSA_CHECK(aligned(ws, 256), DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  float *bs = reinterpret_cast<float *>(w8);
  int32_t *bpos = reinterpret_cast<int32_t *>(w8 + pl.off_pos);
  int32_t *bidx = reinterpret_cast<int32_t *>(w8 + pl.off_blk);
  hipStream_t s = (hipStream_t)stream;
  st = from_hip(dsa::launch_block_scores(scores, ld_scores, b->q_pos, b->num_q, b->max_kv_len, block, bs, pl.ldb, bpos, s),
                "dsa_block_topk block scores");
  if (st != DSA_OK) return st;
  pl.bb.q_pos = bpos;
  st = dsa_topk(&pl.bb, bs, pl.ldb, k_blocks, bidx, pl.tk_bytes ? w8 + pl.off_tk : nullptr, pl.tk_bytes, stream);
  if (st != DSA_OK) return st;
  return from_hip(dsa::launch_block_expand(bidx, k_blocks, block, b->q_pos, b->num_q, idx, s), "dsa_block_topk expand");
}

extern "C" dsa_status dsa_block_cover(const dsa_batch *b, const int32_t *idx, int32_t k, int32_t block, int32_t *counts,
                                      void *stream) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(k >= 1 && block >= 1, DSA_ERR_INVALID_ARGUMENT, "k and block must be >= 1 (got %d, %d)", k, block);
  if (b->num_q == 0) return ok();
  DSA_CHECK(idx && counts, DSA_ERR_INVALID_ARGUMENT, "idx and counts must be non-NULL");
  DSA_CHECK(aligned(idx, 4) && aligned(counts, 4), DSA_ERR_INVALID_ARGUMENT, "idx / counts must be 4-byte aligned");
  return from_hip(dsa::launch_block_cover(idx, k, block, b->q_pos, b->num_q, counts, (hipStream_t)stream),
                  "dsa_block_cover launch");
}

// ---- fused indexer -> top-k
namespace {
dsa_status check_indexer_topk(const dsa_batch *b, int32_t H_I, int32_t d_I, int32_t k) {
  dsa_status st = check_batch(b);
  if (st != DSA_OK) return st;
  DSA_CHECK(H_I == 64 && d_I == 128, DSA_ERR_UNSUPPORTED,
            "no fused indexer/top-k kernel for (H_I, d_I) = (%d, %d); compiled: (64, 128)", H_I, d_I);
  DSA_CHECK(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k must be >= 1 (got %d)", k);
  DSA_CHECK(k <= 4096 && (long long)ceil_div(b->max_kv_len, 8192) * k <= 65536, DSA_ERR_UNSUPPORTED,
            "fused indexer/top-k supports k <= 4096 and ceil(max_kv_len / 8192) * k <= 65536 (got k=%d, max_kv_len=%d)",
            k, b->max_kv_len);
  return ok();
}
}  // namespace

extern "C" dsa_status dsa_indexer_topk_workspace_size(const dsa_batch *b, int32_t H_I, int32_t d_I, int32_t k,
                                                       size_t *bytes) {
  DSA_CHECK(bytes != nullptr, DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  dsa_status st = check_indexer_topk(b, H_I, d_I, k);
  if (st != DSA_OK) return st;
  *bytes = b->num_q == 0 ? 0 : dsa::indexer_topk_ws_bytes(b->num_q, b->max_kv_len, k);
  return ok();
}

extern "C" dsa_status dsa_indexer_topk(const dsa_batch *b, const void *q_idx, const float *w, const void *k_idx,
                                       dsa_dtype k_dtype, const float *k_scale, int32_t H_I, int32_t d_I, int32_t k,
                                       int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
  dsa_status st = check_indexer_topk(b, H_I, d_I, k);
  if (st != DSA_OK) return st;
  DSA_CHECK(k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3FN, DSA_ERR_INVALID_ARGUMENT, "unknown k_dtype %d",
            (int)k_dtype);
  if (b->num_q == 0) return ok();
  DSA_CHECK(q_idx && w && k_idx && idx, DSA_ERR_INVALID_ARGUMENT, "q_idx, w, k_idx and idx must be non-NULL");
  DSA_CHECK(aligned(q_idx, 16) && aligned(w, 16) && aligned(k_idx, 16) && aligned(idx, 16), DSA_ERR_INVALID_ARGUMENT,
            "tensor pointers must be 16-byte aligned");
  if (k_dtype == DSA_FP8_E4M3FN) {
    DSA_CHECK(k_scale != nullptr && aligned(k_scale, 4), DSA_ERR_INVALID_ARGUMENT,
              "FP8 keys need a 4-byte aligned per-token k_scale");
  } else {
    DSA_CHECK(k_scale == nullptr, DSA_ERR_INVALID_ARGUMENT, "k_scale must be NULL for bf16 keys");
  }
  const size_t need = dsa::indexer_topk_ws_bytes(b->num_q, b->max_kv_len, k);
  DSA_CHECK(ws != nullptr && ws_bytes >= need && aligned(ws, 16), DSA_ERR_WORKSPACE,
            "fused indexer/top-k needs %zu bytes of 16-byte aligned workspace (got %zu)", need, ws_bytes);
  dsa::IndexerArgs a{};
  a.q_idx = q_idx;
  a.w = w;
  a.k_idx = k_idx;
  a.k_scale = k_scale;
  a.q_seq = b->q_seq;
  a.q_pos = b->q_pos;
  a.slot = slot_map(b);
  a.num_q = b->num_q;
  a.max_kv_len = b->max_kv_len;
  a.fp8 = (k_dtype == DSA_FP8_E4M3FN);
  a.H_I = H_I;
  a.d_I = d_I;
  uint32_t *ck = static_cast<uint32_t *>(ws);
  const size_t per = need / 8;
  int32_t *cp = reinterpret_cast<int32_t *>(ck + per);
  return from_hip(dsa::launch_indexer_topk(a, k, ck, cp, idx, (hipStream_t)stream), "dsa_indexer_topk launch");
}

