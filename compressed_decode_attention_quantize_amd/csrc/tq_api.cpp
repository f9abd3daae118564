// C ABI entry points that launch GPU work: argument validation on the host,
// parameter packing, then the launchers in the kernel translation units.
// Nothing is enqueued when validation fails.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "tq_internal.h"

using namespace tq;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tq_status hip_fail(const char *what, int err) {
  return fail(TQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(static_cast<hipError_t>(err)));
}

bool valid_dtype(tq_dtype d) { return d == TQ_F32 || d == TQ_BF16 || d == TQ_F16; }

}  // namespace

TQ_EXPORT tq_status tq_quantize_append(const tq_config *cfg, int layer_idx, const void *k, const void *v,
                                       tq_dtype in_dtype, int64_t num_tokens, int num_kv_heads,
                                       int64_t k_token_stride, int64_t v_token_stride,
                                       const int64_t *slot_mapping, uint8_t *kv_pool, int64_t num_blocks,
                                       int block_size, void *stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_quantize_append: negative num_tokens/num_blocks or non-positive heads/block_size");
  if (num_kv_heads > 65535) return fail(TQ_ERR_UNSUPPORTED, "tq_quantize_append: at most 65535 KV heads");
  if (!valid_dtype(in_dtype)) return fail(TQ_ERR_INVALID_ARG, "tq_quantize_append: unknown input dtype");
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !kv_pool) return fail(TQ_ERR_INVALID_ARG, "tq_quantize_append: NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(kv_pool))
    return fail(TQ_ERR_INVALID_ARG, "tq_quantize_append: k, v and kv_pool must be 16-byte aligned");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * cfg->head_dim;
  if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
    return fail(TQ_ERR_INVALID_ARG,
                "tq_quantize_append: token strides must be >= num_kv_heads*head_dim and multiples of 8 elements");
  QuantParams p;
  std::memset(&p, 0, sizeof(p));
  p.k = k;
  p.v = v;
  p.slot_mapping = slot_mapping;
  p.pool = kv_pool;
  p.num_tokens = num_tokens;
  p.k_stride = k_token_stride;
  p.v_stride = v_token_stride;
  p.total_slots = num_blocks * block_size;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.slot_bytes = cfg->slot_size_aligned;
  p.key_bytes = cfg->key_packed_size;
  layer_sign_mask(*cfg, layer_idx, p.sign_words);
  if (!cfg->key_fp8 && !lloyd_max_bins(*cfg, p))
    return fail(TQ_ERR_UNSUPPORTED, "tq_quantize_append: the config's midpoints do not fit the index bins");
  p.sqrt_block = static_cast<float>(std::sqrt(static_cast<double>(cfg->wht_block)));
  const int err = launch_quantize(*cfg, in_dtype, p, stream);
  if (err != hipSuccess) return hip_fail("tq_quantize_append launch", err);
  return TQ_OK;
}

TQ_EXPORT tq_status tq_ring_flush(const tq_config *cfg, int layer_idx, const uint16_t *ring_k, const uint16_t *ring_v,
                                  int ring_cap, int32_t *ring_lens, int32_t *seq_lens, const int32_t *block_tables,
                                  int max_blocks_per_seq, int batch, int num_kv_heads, uint8_t *kv_pool,
                                  int64_t num_blocks, int block_size, void *stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (batch < 0 || ring_cap <= 0 || num_kv_heads <= 0 || num_blocks < 0 || block_size <= 0 || max_blocks_per_seq < 0)
    return fail(TQ_ERR_INVALID_ARG,
                "tq_ring_flush: need batch >= 0, ring_cap > 0, num_kv_heads > 0, block_size > 0, non-negative sizes");
  if (num_kv_heads > 65535) return fail(TQ_ERR_UNSUPPORTED, "tq_ring_flush: at most 65535 KV heads");
  if (batch == 0) return TQ_OK;
  if (!ring_k || !ring_v || !ring_lens || !seq_lens || !block_tables || !kv_pool)
    return fail(TQ_ERR_INVALID_ARG, "tq_ring_flush: NULL pointer");
  if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned16(kv_pool))
    return fail(TQ_ERR_INVALID_ARG, "tq_ring_flush: ring_k, ring_v and kv_pool must be 16-byte aligned");
  QuantParams p;
  std::memset(&p, 0, sizeof(p));
  p.k = ring_k;
  p.v = ring_v;
  p.pool = kv_pool;
  p.num_tokens = static_cast<int64_t>(batch) * ring_cap;
  p.total_slots = num_blocks * block_size;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.slot_bytes = cfg->slot_size_aligned;
  p.key_bytes = cfg->key_packed_size;
  layer_sign_mask(*cfg, layer_idx, p.sign_words);
  if (!cfg->key_fp8 && !lloyd_max_bins(*cfg, p))
    return fail(TQ_ERR_UNSUPPORTED, "tq_ring_flush: the config's midpoints do not fit the index bins");
  p.sqrt_block = static_cast<float>(std::sqrt(static_cast<double>(cfg->wht_block)));
  p.ring_lens = ring_lens;
  p.seq_lens = seq_lens;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.ring_cap = ring_cap;
  int err = launch_quantize(*cfg, TQ_BF16, p, stream);
  if (err != hipSuccess) return hip_fail("tq_ring_flush launch", err);
  err = launch_ring_commit(ring_lens, seq_lens, batch, ring_cap, stream);
  if (err != hipSuccess) return hip_fail("tq_ring_flush commit launch", err);
  return TQ_OK;
}

TQ_EXPORT tq_status tq_ring_append(const tq_config *cfg, const uint16_t *k_new, const uint16_t *v_new, int batch,
                                   int num_kv_heads, uint16_t *ring_k, uint16_t *ring_v, int ring_cap,
                                   int32_t *ring_lens, void *stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (batch < 0 || ring_cap <= 0 || num_kv_heads <= 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_ring_append: need batch >= 0, ring_cap > 0 and num_kv_heads > 0");
  if (batch == 0) return TQ_OK;
  if (!k_new || !v_new || !ring_k || !ring_v || !ring_lens) return fail(TQ_ERR_INVALID_ARG, "tq_ring_append: NULL pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(ring_k) || !aligned16(ring_v))
    return fail(TQ_ERR_INVALID_ARG, "tq_ring_append: k_new, v_new, ring_k and ring_v must be 16-byte aligned");
  const int err = launch_ring_append(k_new, v_new, ring_k, ring_v, ring_lens, batch, num_kv_heads, cfg->head_dim,
                                     ring_cap, stream);
  if (err != hipSuccess) return hip_fail("tq_ring_append launch", err);
  return TQ_OK;
}

namespace {

// Work division and workspace of a continuation prefill. Row blocks of
// kPrefillRows query rows per (sequence, KV head); the history is cut into
// `splits` ranges of split_tokens tokens so that about kPrefillTargetWaves
// waves run (no range shorter than kPrefillMinSplitTokens). The workspace
// holds one partial per (row, split).
constexpr int64_t kPrefillTargetWaves = 2048;
constexpr int64_t kPrefillMinSplitTokens = 1024;

struct PrefillLayout {
  int row_blocks = 0, rows_pad = 0, row_sets = 0, splits = 1, split_tokens = 32, workgroups = 0;
  size_t total = 0;
};

tq_status prefill_layout(const tq_config &cfg, int batch, int num_q_heads, int num_kv_heads, int max_chunk,
                         int max_hist, PrefillLayout *L) {
  const int64_t group = num_q_heads / num_kv_heads;
  const int64_t rows = static_cast<int64_t>(max_chunk) * group;
  if (rows > INT32_MAX - kPrefillRows)
    return fail(TQ_ERR_UNSUPPORTED, "tq_prefill: max_chunk * (num_q_heads / num_kv_heads) must fit in 31 bits");
  const int64_t rb = (rows + kPrefillRows - 1) / kPrefillRows;
  const int64_t base = static_cast<int64_t>(batch) * num_kv_heads * rb;
  int64_t splits = 1, split_tokens = 32;
  if (max_hist > 0 && base > 0) {
    splits = std::max<int64_t>(1, std::min<int64_t>((kPrefillTargetWaves + base - 1) / base,
                                                    max_hist / kPrefillMinSplitTokens));
    split_tokens = ((max_hist + splits - 1) / splits + 31) / 32 * 32;
    splits = (max_hist + split_tokens - 1) / split_tokens;
  }
  const int64_t sets = (rb + kPrefillWaves - 1) / kPrefillWaves;
  const int64_t workgroups = static_cast<int64_t>(batch) * num_kv_heads * sets * splits;
  if (workgroups > INT32_MAX / 4)
    return fail(TQ_ERR_UNSUPPORTED, "tq_prefill: too many (sequence, KV head, row block) work items; split the batch");
  L->row_blocks = static_cast<int>(rb);
  L->rows_pad = static_cast<int>(rb * kPrefillRows);
  L->row_sets = static_cast<int>(sets);
  L->splits = static_cast<int>(splits);
  L->split_tokens = static_cast<int>(split_tokens);
  L->workgroups = static_cast<int>(workgroups);
  L->total = static_cast<size_t>(batch) * num_kv_heads * L->rows_pad * L->splits * (cfg.head_dim + 4) * sizeof(float);
  return TQ_OK;
}

}  // namespace

TQ_EXPORT tq_status tq_prefill_workspace_size(const tq_config *cfg, int batch, int num_q_heads, int num_kv_heads,
                                              int max_chunk, int max_hist, int max_blocks_per_seq,
                                              tq_dtype q_dtype, size_t *bytes_out) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (!bytes_out) return fail(TQ_ERR_INVALID_ARG, "tq_prefill_workspace_size: bytes_out is NULL");
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_chunk < 0 ||
      max_hist < 0 || max_blocks_per_seq < 0 || !valid_dtype(q_dtype))
    return fail(TQ_ERR_INVALID_ARG, "tq_prefill_workspace_size: invalid sizes or dtype");
  PrefillLayout L;
  st = prefill_layout(*cfg, batch, num_q_heads, num_kv_heads, max_chunk, max_hist, &L);
  if (st != TQ_OK) return st;
  *bytes_out = L.total;
  return TQ_OK;
}

TQ_EXPORT tq_status tq_prefill_attention(const tq_config *cfg, int layer_idx, const void *q, tq_dtype q_dtype,
                                         const uint16_t *k_chunk, const uint16_t *v_chunk, const int32_t *cu_chunk,
                                         int batch, int max_chunk, int num_q_heads, int num_kv_heads,
                                         const uint8_t *kv_pool, int64_t num_blocks, int block_size,
                                         const int32_t *block_tables, int max_blocks_per_seq,
                                         const int32_t *hist_lens, int max_hist, float softmax_scale, float *out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (batch < 0 || max_chunk < 0 || max_hist < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_prefill_attention: invalid sizes (num_q_heads must be a multiple of num_kv_heads)");
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(TQ_ERR_UNSUPPORTED, "tq_prefill_attention: block_size must be a positive multiple of 16");
  if (static_cast<int64_t>(num_kv_heads) * block_size * cfg->slot_size_aligned > INT32_MAX)
    return fail(TQ_ERR_UNSUPPORTED, "tq_prefill_attention: a pool block (num_kv_heads * block_size * slot bytes) must be below 2 GiB");
  if (!valid_dtype(q_dtype)) return fail(TQ_ERR_INVALID_ARG, "tq_prefill_attention: unknown q dtype");
  if (batch == 0 || max_chunk == 0) return TQ_OK;
  if (!q || !k_chunk || !v_chunk || !cu_chunk || !kv_pool || !block_tables || !hist_lens || !out)
    return fail(TQ_ERR_INVALID_ARG, "tq_prefill_attention: NULL pointer");
  if (!aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(kv_pool) || !aligned16(out))
    return fail(TQ_ERR_INVALID_ARG, "tq_prefill_attention: q, k_chunk, v_chunk, kv_pool and out must be 16-byte aligned");
  if (max_hist > 0 && num_blocks < 1)
    return fail(TQ_ERR_INVALID_ARG, "tq_prefill_attention: a history (max_hist > 0) needs a pool of at least one block");
  PrefillLayout L;
  st = prefill_layout(*cfg, batch, num_q_heads, num_kv_heads, max_chunk, max_hist, &L);
  if (st != TQ_OK) return st;
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(TQ_ERR_WORKSPACE, "tq_prefill_attention: workspace must be 256-byte aligned and hold " +
                                      std::to_string(L.total) + " bytes");
  PrefillParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_chunk = k_chunk;
  p.v_chunk = v_chunk;
  p.cu_chunk = cu_chunk;
  p.hist_lens = hist_lens;
  p.block_tables = block_tables;
  p.pool = kv_pool;
  p.partials = static_cast<float *>(workspace);
  p.out = out;
  p.num_blocks = num_blocks;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.max_chunk = max_chunk;
  p.max_hist = max_hist;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.row_blocks = L.row_blocks;
  p.rows_pad = L.rows_pad;
  p.splits = L.splits;
  p.split_tokens = L.split_tokens;
  p.row_sets = L.row_sets;
  p.workgroups = L.workgroups;
  const float scale = softmax_scale > 0.0f ? softmax_scale
                                           : static_cast<float>(1.0 / std::sqrt(static_cast<double>(cfg->head_dim)));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.centroid_scale = cfg->centroid_scale;
  layer_sign_mask(*cfg, layer_idx, p.sign_words);
  for (int i = 0; i < 16; ++i) p.centroids[i] = cfg->centroids[i];
  const int err = launch_prefill(*cfg, q_dtype, p, stream);
  if (err != hipSuccess) return hip_fail("tq_prefill_attention launch", err);
  return TQ_OK;
}

TQ_EXPORT tq_status tq_dequant(const tq_config *cfg, int layer_idx, const uint8_t *kv_pool, int64_t num_blocks,
                               int num_kv_heads, int block_size, const int64_t *slot_ids, int64_t n,
                               float *k_out, float *v_out, void *stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (n < 0 || num_kv_heads <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_dequant: negative n/num_blocks or non-positive heads/block_size");
  if (n == 0) return TQ_OK;
  if (!kv_pool || !slot_ids || !k_out || !v_out) return fail(TQ_ERR_INVALID_ARG, "tq_dequant: NULL pointer");
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(TQ_ERR_INVALID_ARG, "tq_dequant: outputs must be 16-byte aligned");
  DequantParams p;
  std::memset(&p, 0, sizeof(p));
  p.pool = kv_pool;
  p.slot_ids = slot_ids;
  p.k_out = k_out;
  p.v_out = v_out;
  p.n = n;
  p.total_slots = num_blocks * block_size;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.slot_bytes = cfg->slot_size_aligned;
  p.key_bytes = cfg->key_packed_size;
  p.norm_correction = cfg->norm_correction;
  layer_sign_mask(*cfg, layer_idx, p.sign_words);
  for (int i = 0; i < 16; ++i) p.centroids[i] = cfg->centroids[i];
  p.inv_sqrt_block = static_cast<float>(1.0 / std::sqrt(static_cast<double>(cfg->wht_block)));
  const int err = launch_dequant(*cfg, p, stream);
  if (err != hipSuccess) return hip_fail("tq_dequant launch", err);
  return TQ_OK;
}

namespace {

// Validates a decode call and fills everything but the workspace pointers.
// *run is false when there is nothing to launch (batch 0).
tq_status decode_setup(const char *fn, const tq_config *cfg, int layer_idx, const void *q, tq_dtype q_dtype,
                       int batch, int num_q_heads, int num_kv_heads, const uint8_t *kv_pool, int64_t num_blocks,
                       int block_size, const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens,
                       int max_seq_len, const void *ring_k, const void *ring_v, const int32_t *ring_lens,
                       int ring_cap, float softmax_scale, float *out, int split_tokens, DecodeParams *pp,
                       SplitPlan *plan, bool *run) {
  *run = false;
  const std::string f(fn);
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, f + ": need batch >= 0 and num_q_heads a positive multiple of num_kv_heads");
  if (batch > 8192)
    return fail(TQ_ERR_UNSUPPORTED, f + ": at most 8192 sequences per call");
  if (num_q_heads / num_kv_heads > 16)
    return fail(TQ_ERR_UNSUPPORTED, f + ": at most 16 query heads per KV head");
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(TQ_ERR_UNSUPPORTED, f + ": block_size must be a positive multiple of 16");
  if (static_cast<int64_t>(num_kv_heads) * block_size * cfg->slot_size_aligned > INT32_MAX)
    return fail(TQ_ERR_UNSUPPORTED, f + ": a pool block (num_kv_heads * block_size * slot bytes) must be below 2 GiB");
  if (max_seq_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0 || ring_cap < 0)
    return fail(TQ_ERR_INVALID_ARG, f + ": negative size argument");
  if (!valid_dtype(q_dtype)) return fail(TQ_ERR_INVALID_ARG, f + ": unknown q dtype");
  const bool has_ring = ring_k != nullptr || ring_v != nullptr;
  if (has_ring && (!ring_k || !ring_v || !ring_lens || ring_cap <= 0))
    return fail(TQ_ERR_INVALID_ARG, f + ": ring needs ring_k, ring_v, ring_lens and ring_cap > 0");
  if (!has_ring && ring_cap != 0)
    return fail(TQ_ERR_INVALID_ARG, f + ": ring_cap must be 0 without a ring");
  if (batch == 0) return TQ_OK;
  if (!q || !kv_pool || !block_tables || !seq_lens || !out)
    return fail(TQ_ERR_INVALID_ARG, f + ": NULL pointer");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || (has_ring && (!aligned16(ring_k) || !aligned16(ring_v))))
    return fail(TQ_ERR_INVALID_ARG, f + ": q, kv_pool, out, ring_k and ring_v must be 16-byte aligned");
  st = plan_decode(*cfg, batch, num_q_heads, max_seq_len, ring_cap, split_tokens, plan);
  if (st != TQ_OK) return st;
  DecodeParams &p = *pp;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.pool = kv_pool;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.ring_k = static_cast<const uint16_t *>(ring_k);
  p.ring_v = static_cast<const uint16_t *>(ring_v);
  p.ring_lens = ring_lens;
  p.out = out;
  p.num_blocks = num_blocks;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.ring_cap = has_ring ? ring_cap : 0;
  p.split_tokens = plan->split_tokens;
  p.ring_chunks = plan->ring_chunks;
  p.slot_bytes = cfg->slot_size_aligned;
  p.key_bytes = cfg->key_packed_size;
  p.norm_correction = cfg->norm_correction;
  const float scale = softmax_scale > 0.0f ? softmax_scale
                                           : static_cast<float>(1.0 / std::sqrt(static_cast<double>(cfg->head_dim)));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.centroid_scale = cfg->centroid_scale;
  layer_sign_mask(*cfg, layer_idx, p.sign_words);
  for (int i = 0; i < 16; ++i) p.centroids[i] = cfg->centroids[i];
  *run = true;
  return TQ_OK;
}

void bind_workspace(DecodeParams &p, const SplitPlan &plan, void *workspace) {
  char *ws = static_cast<char *>(workspace);
  p.plan = reinterpret_cast<int32_t *>(ws);
  p.partials = reinterpret_cast<float *>(ws + plan.header_bytes);
  p.ring_partials = reinterpret_cast<float *>(ws + plan.ring_offset);
}

}  // namespace

TQ_EXPORT tq_status tq_decode_attention(const tq_config *cfg, int layer_idx, const void *q, tq_dtype q_dtype,
                                        int batch, int num_q_heads, int num_kv_heads, const uint8_t *kv_pool,
                                        int64_t num_blocks, int block_size, const int32_t *block_tables,
                                        int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len,
                                        const void *ring_k, const void *ring_v, const int32_t *ring_lens,
                                        int ring_cap, float softmax_scale, float *out, void *workspace,
                                        size_t workspace_bytes, int split_tokens, void *stream) {
  DecodeParams p;
  SplitPlan plan;
  bool run = false;
  tq_status st = decode_setup("tq_decode_attention", cfg, layer_idx, q, q_dtype, batch, num_q_heads, num_kv_heads,
                              kv_pool, num_blocks, block_size, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                              ring_k, ring_v, ring_lens, ring_cap, softmax_scale, out, split_tokens, &p, &plan, &run);
  if (st != TQ_OK || !run) return st;
  if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned16(workspace))
    return fail(TQ_ERR_WORKSPACE, "tq_decode_attention: workspace must be 16-byte aligned and hold " +
                                      std::to_string(plan.workspace_bytes) + " bytes");
  bind_workspace(p, plan, workspace);
  const int err = launch_decode(*cfg, q_dtype, p, stream);
  if (err != hipSuccess) return hip_fail("tq_decode_attention launch", err);
  return TQ_OK;
}

TQ_EXPORT tq_status tq_decode_attention_no_alloc(const tq_config *cfg, int layer_idx, const void *q, tq_dtype q_dtype,
                                                 int batch, int num_q_heads, int num_kv_heads, const uint8_t *kv_pool,
                                                 int64_t num_blocks, int block_size, const int32_t *block_tables,
                                                 int max_blocks_per_seq, const int32_t *seq_lens, int max_seq_len,
                                                 const void *ring_k, const void *ring_v, const int32_t *ring_lens,
                                                 int ring_cap, float softmax_scale, float *out, int split_tokens,
                                                 void *stream) {
  DecodeParams p;
  SplitPlan plan;
  bool run = false;
  tq_status st = decode_setup("tq_decode_attention_no_alloc", cfg, layer_idx, q, q_dtype, batch, num_q_heads,
                              num_kv_heads, kv_pool, num_blocks, block_size, block_tables, max_blocks_per_seq,
                              seq_lens, max_seq_len, ring_k, ring_v, ring_lens, ring_cap, softmax_scale, out,
                              split_tokens, &p, &plan, &run);
  if (st != TQ_OK || !run) return st;
  // the partials this launch can write: its split waves + one row per segment
  const long long waves = decode_launch_waves(*cfg, p);
  if (waves < 0) return hip_fail("tq_decode_attention_no_alloc occupancy query", hipErrorInvalidValue);
  plan_for_launch(*cfg, batch, num_q_heads, num_kv_heads, waves, &plan);
  void *ws = nullptr;
  size_t cap = 0;
  const int e = static_scratch(&ws, &cap);
  if (e != hipSuccess) return hip_fail("tq_decode_attention_no_alloc scratch address", e);
  if (plan.workspace_bytes > cap)
    return fail(TQ_ERR_WORKSPACE, "tq_decode_attention_no_alloc: this call needs " +
                                      std::to_string(plan.workspace_bytes) + " bytes of scratch, more than the " +
                                      std::to_string(cap) + " the library holds per device; use tq_decode_attention "
                                      "with a caller workspace");
  bind_workspace(p, plan, ws);
  const int err = launch_decode(*cfg, q_dtype, p, stream);
  if (err != hipSuccess) return hip_fail("tq_decode_attention_no_alloc launch", err);
  return TQ_OK;
}
