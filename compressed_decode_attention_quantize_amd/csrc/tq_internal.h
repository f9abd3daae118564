// Internal declarations shared by the host core, the C-ABI layer and the
// kernel translation units. Not installed; the public surface is include/tq.h.
#pragma once

#include <cstdint>
#include <string>

#include "../../include/tq.h"

#define TQ_EXPORT extern "C" __attribute__((visibility("default")))

namespace tq {

// Records the message returned by tq_last_error() on this thread and returns
// the status, so call sites can write `return fail(TQ_ERR_..., "...")`.
tq_status fail(tq_status st, const std::string &msg);
void clear_error();

// Validates a config filled by tq_config_init (recomputes the derived sizes).
tq_status check_config(const tq_config *cfg);

struct QuantParams;
// Fills the Lloyd-Max bin fields of p from the config's midpoints: kLmBins
// equal bins, the first midpoint in bin 1 and the last in bin kLmBins - 1.
// Returns false when two midpoints fall in one bin (or are out of order),
// where the table cannot give the exact count.
bool lloyd_max_bins(const tq_config &cfg, QuantParams &p);

// Random signs of one layer as a bit mask: bit j of words[j / 32] is set when
// sign j is -1. head_dim <= 128.
void layer_sign_mask(const tq_config &cfg, int layer_idx, uint32_t words[4]);

// Bins of the Lloyd-Max index table (a power of two; at most one midpoint
// falls in each bin for every table tq_config_init makes).
constexpr int kLmBins = 64;

// Kernel parameter blocks. Plain structs passed by value to the kernels.
struct QuantParams {
  const void *k;
  const void *v;
  const int64_t *slot_mapping;
  uint8_t *pool;
  int64_t num_tokens;
  int64_t k_stride;     // elements
  int64_t v_stride;     // elements
  int64_t total_slots;  // num_blocks * block_size
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t slot_bytes;   // slot_size_aligned
  int32_t key_bytes;    // key_packed_size
  uint32_t sign_words[4];
  float sqrt_block;     // fp32(sqrt(B))
  // Lloyd-Max index by bins (MSE keys; see lloyd_max_bins): bin(u) =
  // trunc(min(max(fma(u, lm_scale, lm_offset), 0), kLmBins - 1)), entry j =
  // {bits of the midpoint in bin j (+inf if none), midpoints in bins < j}.
  float lm_scale;
  float lm_offset;
  uint32_t lm_table[2 * kLmBins];
  // Ring flush mode (ring_lens != nullptr): token n is ring position
  // n % ring_cap of sequence n / ring_cap, read at
  // (seq * num_kv_heads + h) * ring_cap * D + pos * D; it is written only if
  // that sequence's ring is full, at position seq_lens[seq] + pos through its
  // block table. slot_mapping, k_stride and v_stride are unused.
  const int32_t *ring_lens;
  const int32_t *seq_lens;
  const int32_t *block_tables;
  int32_t max_blocks_per_seq;
  int32_t ring_cap;
};

struct DequantParams {
  const uint8_t *pool;
  const int64_t *slot_ids;
  float *k_out;
  float *v_out;
  int64_t n;
  int64_t total_slots;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t slot_bytes;
  int32_t key_bytes;
  int32_t norm_correction;
  uint32_t sign_words[4];
  float centroids[16];
  float inv_sqrt_block;  // fp32(1/sqrt(B))
};

struct DecodeParams {
  const void *q;
  const uint8_t *pool;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  const uint16_t *ring_k;  // bf16 bits
  const uint16_t *ring_v;
  const int32_t *ring_lens;
  // Partials, rows of G query heads x [m, l, pad, pad, acc[D]] fp32:
  //  compressed tokens: wave w's partial of segment s = b * Hkv + h (the
  //  waves' ranges are consecutive, so w + s is unique) is row w + s;
  //  ring chunks: row (s * ring_chunks + chunk) of ring_partials.
  float *partials;
  float *ring_partials;
  float *out;
  int64_t num_blocks;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;
  int32_t ring_cap;
  int32_t split_tokens;    // minimum tokens per wave (multiple of 16)
  int32_t ring_chunks;     // ceil(ring_cap / kRingChunk)
  int32_t *plan;           // workspace header: [total tiles (int64), active waves, -, tile prefix[batch + 1]]
  int32_t slot_bytes;
  int32_t key_bytes;
  int32_t norm_correction;
  float scale_log2;        // softmax scale * log2(e)
  float centroid_scale;    // sigma of the f16 centroid table
  uint32_t sign_words[4];
  float centroids[16];
};

// Launchers (defined in the kernel translation units). Return hipSuccess or a
// HIP error code as int.
// Continuation prefill: one wave per (sequence, KV head, history split, row
// block of 16 * kPrefillRowGroups query rows), kPrefillWaves consecutive row
// blocks of one (sequence, KV head, split) per workgroup; rows of a KV head
// are ordered token-major (row r = t * group + g for query head h * group + g).
constexpr int kPrefillRowGroups = 2;
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = 16 * kPrefillRowGroups;
struct PrefillParams {
  const void *q;             // [N][num_q_heads][D], q_dtype
  const uint16_t *k_chunk;   // [N][num_kv_heads][D] bf16 bits
  const uint16_t *v_chunk;
  const int32_t *cu_chunk;   // [batch + 1]
  const int32_t *hist_lens;  // [batch]
  const int32_t *block_tables;
  const uint8_t *pool;
  // partials [batch][num_kv_heads][rows_pad][splits] x [m, l, -, -, acc[D]] fp32
  float *partials;
  float *out;                // [N][num_q_heads][D] fp32
  int64_t num_blocks;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;             // query heads per KV head
  int32_t max_chunk;
  int32_t max_hist;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t row_blocks;        // ceil(max_chunk * group / kPrefillRows)
  int32_t rows_pad;          // row_blocks * kPrefillRows
  int32_t splits;            // history ranges per row block
  int32_t split_tokens;      // tokens per history range (multiple of 32)
  int32_t row_sets;          // ceil(row_blocks / kPrefillWaves): workgroups per (sequence, KV head, split)
  int32_t workgroups;        // batch * num_kv_heads * splits * row_sets
  float scale_log2;          // softmax scale * log2(e)
  float centroid_scale;      // sigma of the f16 centroid table
  uint32_t sign_words[4];
  float centroids[16];
};

int launch_prefill(const tq_config &cfg, tq_dtype q_dtype, const PrefillParams &p, void *stream);
int launch_quantize(const tq_config &cfg, tq_dtype dtype, const QuantParams &p, void *stream);
int launch_dequant(const tq_config &cfg, const DequantParams &p, void *stream);
int launch_ring_commit(int32_t *ring_lens, int32_t *seq_lens, int batch, int ring_cap, void *stream);
int launch_ring_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *ring_k, uint16_t *ring_v,
                       int32_t *ring_lens, int batch, int num_kv_heads, int head_dim, int ring_cap, void *stream);
int launch_decode(const tq_config &cfg, tq_dtype q_dtype, const DecodeParams &p, void *stream);
// Waves the decode split kernel launch for these parameters uses on the
// current device (0 when none is launched); < 0 on a HIP error.
long long decode_launch_waves(const tq_config &cfg, const DecodeParams &p);
// The per-device static scratch of the no-allocation decode: its device
// address on the current device (looked up once per device) and its size.
int static_scratch(void **ptr, size_t *bytes);

// Split plan shared by tq_decode_workspace_size and tq_decode_attention.
struct SplitPlan {
  int32_t split_tokens;   // as given (0 = 256 tokens per wave at least)
  int32_t max_splits;     // partials per (sequence, KV head) at most: ceil(max_seq_len / split_tokens) + 1
  int32_t ring_chunks;    // one partial per kRingChunk ring tokens
  int64_t head_rows;      // compressed-token partial rows of one query head each
  size_t header_bytes;    // work-division header (16 + 4 (batch + 1), rounded to 256)
  size_t ring_offset;     // byte offset of the ring partials
  size_t workspace_bytes; // header + compressed partials + ring partials
};
// Shrinks a plan to a known split launch of `waves` waves over num_kv_heads
// KV heads: at most (waves + batch * num_kv_heads) rows of G heads.
void plan_for_launch(const tq_config &cfg, int batch, int num_q_heads, int num_kv_heads, long long waves,
                     SplitPlan *plan);
constexpr int kMinTokensPerWave = 256;     // default range of a decode wave (MSE keys)
constexpr int kMinTokensPerWaveFp8 = 512;  // FP8 keys: fewer, longer ranges
constexpr int kRingChunk = 32;  // ring tokens per partial slot
tq_status plan_decode(const tq_config &cfg, int batch, int num_q_heads, int max_seq_len,
                      int ring_cap, int split_tokens, SplitPlan *plan);

}  // namespace tq
