/*
 * tq.h -- C ABI of the TurboQuant KV-cache hot path for AMD Instinct MI355X
 * (gfx950): quantize-and-append K/V into packed per-head slots, and fused
 * decode attention directly over those slots.
 *
 * Sources the operations follow (cited by page and section):
 *  [API]  vLLM API page "vllm.model_executor.layers.quantization.turboquant",
 *         class TurboQuantConfig: docstring, fields, properties,
 *         from_cache_dtype.
 *  [PR]   prhub summary of vLLM PR #39931, "TurboQuant supports hybrid models
 *         and fixes page-size alignment", interface.py source snippet
 *         (TurboQuant page size = block_size * num_kv_heads * slot bytes).
 *  [ART]  hnwysp.cn article on the stand-alone turboquant project (full_tq
 *         zero-allocation mode): write-path section (128-token bf16 exact
 *         ring buffer, whole-chunk compression) and next-directions
 *         section, direction 1 (fused decode attention: single pass over the
 *         compressed data, online softmax block by block, query rotated
 *         forward instead of rotating keys back, no materialised FP16 KV),
 *         direction 2 (2-bit values beside 4-bit ones) and direction 3
 *         (initial_layers_key_bits: the first four layers get one more key
 *         bit).
 *  [PR]   also: implementation item 1 (hybrid models skip no layers) and
 *         the interface.py snippet (per-token attention page = lcm of the
 *         TurboQuant page and the unquantized skip-layer page).
 *
 * Conventions for every function:
 *  - Returns a tq_status; never throws or aborts. On failure nothing is
 *    enqueued and tq_last_error() describes the problem.
 *  - Device pointers are caller-owned; the library allocates no device memory.
 *    Its only mutable global state is a process-wide, mutex-guarded cache of
 *    the decode kernels' resident workgroups per (kernel, device), filled on
 *    first use; calls are reentrant and may run concurrently on different
 *    streams when they write disjoint memory.
 *  - GPU calls are asynchronous and ordered on `stream` (a hipStream_t passed
 *    as void*; NULL = the default stream).
 *  - Scalars and null pointers are validated on the host. Device contents
 *    (slot ids, block ids, lengths) are clamped or skipped by the kernels so
 *    that bad values cannot make them read or write out of bounds; such
 *    values give unspecified results, not faults.
 *  - Pool layout: uint8 [num_blocks][num_kv_heads][block_size][S] with
 *    S = slot_size_aligned; token position p of a sequence lives in physical
 *    block block_table[p / block_size] at offset p % block_size. The page of
 *    one block is block_size * num_kv_heads * S bytes ([PR]); the order inside
 *    it is this library's choice.
 *  - Slot layout ([API] slot_size): [key_packed | value_packed] where
 *    key_packed = MSE indices (LSB-first bitstream, ceil(D*kb/8) bytes) +
 *    fp16 vec_norm, or D FP8 E4M3FN bytes when key_quant_bits == 8; and
 *    value_packed = codes (LSB-first, ceil(D*vb/8) bytes) + fp16 scale +
 *    fp16 zero; fp16 fields little-endian; padded to an even size.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,    /* bad scalar, null pointer, misaligned pointer  */
  TQ_ERR_UNKNOWN_PRESET = 2, /* tq_config_from_preset with an unknown name    */
  TQ_ERR_UNSUPPORTED = 3,    /* valid but not built (e.g. head_dim 256)       */
  TQ_ERR_WORKSPACE = 4,      /* decode workspace missing or too small         */
  TQ_ERR_HIP = 5,            /* a HIP launch or runtime call failed           */
  TQ_STATUS_MAX_ENUM = 0x7fffffff /* no status: keeps the type a 32-bit integer */
} tq_status;

/* Element types of query / key / value inputs. TQ_DTYPE_MAX_ENUM is no
 * type: it keeps the enumeration a 32-bit integer whose every value is
 * representable, so a caller's invalid value reaches the library's
 * validation (TQ_ERR_INVALID_ARG) instead of being an out-of-range enum. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2, TQ_DTYPE_MAX_ENUM = 0x7fffffff } tq_dtype;

/*
 * Configuration: the five dataclass fields of TurboQuantConfig ([API]) plus
 * the derived properties, computed exactly as the printed properties do, and
 * the Lloyd-Max tables. A value type filled by tq_config_init or
 * tq_config_from_preset; callers must not edit it afterwards.
 *
 * centroids: the 2^mse_bits Lloyd-Max reconstruction levels of N(0, 1/D),
 *   ascending, fp32 (rounded from float64; exactly antisymmetric).
 * midpoints: the 2^mse_bits - 1 decision thresholds, fp32(mean of adjacent
 *   float64 levels).
 * wht_block: length B of the blockwise Walsh-Hadamard transform, the largest
 *   power of two dividing head_dim (128 -> 128, 96 -> 32, 64 -> 64).
 * centroid_scale: sigma = 1 + i / 2^18 (i < 2^18) minimising the largest
 *   relative round-off of fp16(fp32(sigma * centroid)) over the table.
 */
typedef struct {
  int32_t head_dim;          /* 64 | 96 | 128                                 */
  int32_t key_quant_bits;    /* 3 | 4 = Lloyd-Max MSE keys; 8 = FP8 keys      */
  int32_t value_quant_bits;  /* 2 | 3 | 4                                     */
  int32_t norm_correction;   /* 0 | 1                                         */
  int64_t seed;              /* base seed (default 42)                        */
  int32_t key_fp8;           /* key_quant_bits == 8                           */
  int32_t mse_bits;          /* key bits, or value bits in FP8 mode           */
  int32_t key_mse_bits;      /* 0 in FP8 mode                                 */
  int32_t centroid_bits;     /* == mse_bits                                   */
  int32_t n_centroids;       /* 2^mse_bits                                    */
  int32_t key_packed_size;   /* bytes                                         */
  int32_t value_packed_size; /* bytes                                         */
  int32_t slot_size;         /* key_packed_size + value_packed_size           */
  int32_t slot_size_aligned; /* slot_size rounded up to even                  */
  int32_t wht_block;
  float centroids[16];
  float midpoints[15];
  float centroid_scale;      /* sigma in [1, 2): the f16 images of sigma * centroids
                                are closest to exact; used by the decode kernel's
                                f16 centroid table (the score divides by sigma) */
} tq_config;

/* Dataclass constructor ([API] TurboQuantConfig fields). head_dim must be 64,
 * 96 or 128; key_bits 3, 4 or 8; value_bits 2, 3 or 4 (2 per [ART]
 * direction 2; the value field is then ceil(D*2/8) + 4 bytes by the [API]
 * value_packed_size formula). Host only. */
tq_status tq_config_init(int head_dim, int key_bits, int value_bits, int norm_correction,
                         int64_t seed, tq_config *out);

/* Named preset ([API] from_cache_dtype): turboquant_k8v4 (FP8 keys, 4-bit
 * values), turboquant_4bit_nc (4/4, norm correction), turboquant_k3v4_nc
 * (3/4, NC), turboquant_3bit_nc (3/3, NC); seed 42. Unknown names return
 * TQ_ERR_UNKNOWN_PRESET with the message
 * "Unknown TurboQuant cache dtype: '<name>'. Valid presets: turboquant_k8v4,
 * turboquant_4bit_nc, turboquant_k3v4_nc, turboquant_3bit_nc". Host only. */
tq_status tq_config_from_preset(const char *preset, int head_dim, tq_config *out);

/* Per-layer config for layer-adaptive key bits ([ART] direction 3). For
 * layer_idx < initial_layers, out = base with key_quant_bits =
 * initial_layers_key_bits, or base's key bits + 1 when that argument is 0
 * (an FP8 base then stays FP8: there is no wider FP8 key); for later layers
 * out = base. All other fields are base's (the layer's seed still comes from
 * seed + 1337 * layer_idx in the calls that take layer_idx). A width that
 * tq_config_init rejects (e.g. 5 from a 4-bit base) returns its error;
 * negative layer_idx or initial_layers returns TQ_ERR_INVALID_ARG. out may
 * alias base. Host only. */
tq_status tq_layer_config(const tq_config *base, int layer_idx, int initial_layers,
                          int initial_layers_key_bits, tq_config *out);

/* Boundary protection ([API] get_boundary_skip_layers): the layers that keep
 * the unquantized cache, ascending: the first n and the last n of a dense
 * model, n capped at num_layers / 2, each index once; none when n <= 0,
 * num_layers <= 0, or hybrid != 0 ([PR] item 1). Writes at most out_cap
 * indices to out and returns how many there are (the caller can size out
 * from a first call with out_cap = 0); -1 if out is NULL with out_cap > 0.
 * Host only. */
int tq_boundary_skip_layers(int num_layers, int n, int hybrid, int32_t *out, int out_cap);

/* Per-token page bytes every attention layer shares ([PR] interface.py):
 * the TurboQuant page num_kv_heads * slot_size_aligned, or, when skip layers
 * exist (skip_dtype_bytes > 0, the element size of their unquantized cache),
 * lcm(that, 2 * num_kv_heads * head_dim * skip_dtype_bytes): the least
 * common multiple, not the maximum, so both page kinds tile it. The skip
 * page formula (K and V rows of every head) is this library's reading.
 * Returns < 0 on invalid input. Host only. */
int64_t tq_attn_page_size_1_token(const tq_config *cfg, int num_kv_heads, int skip_dtype_bytes);

/* Slot bytes per head per position ([API] slot_size / slot_size_aligned):
 * aligned != 0 gives slot_size_aligned. Returns < 0 on a null or invalid
 * config. Host only. */
int32_t tq_slot_size(const tq_config *cfg, int aligned);

/* Bytes of one paged block: block_size * num_kv_heads * slot_size_aligned
 * ([PR] TurboQuant page size). Returns < 0 on invalid input. Host only. */
int64_t tq_page_size(const tq_config *cfg, int num_kv_heads, int block_size);

/* The layer's random signs as floats (+1/-1), head_dim of them, for layer
 * seed = seed + 1337 * layer_idx ([API] seed argument), drawn from
 * SplitMix64: sign j is -1 when bit 63 of output j is set. Host only; for
 * checking and for callers that rotate queries themselves. */
tq_status tq_layer_signs(const tq_config *cfg, int layer_idx, float *signs_out);

/*
 * Quantize-and-append ([API] docstring and slot layout; [ART] write path):
 * encodes K[t, h, :] and V[t, h, :] for t < num_tokens, h < num_kv_heads,
 * and writes the slot into kv_pool at physical slot slot_mapping[t].
 *
 *  k, v          device, dtype in_dtype (F32, BF16 or F16), element (t, h, j)
 *                at t * token_stride + h * head_dim + j; 16-byte aligned;
 *                token strides are multiples of 8 elements.
 *  slot_mapping  device int64 [num_tokens]; -1 skips the token; ids outside
 *                [0, num_blocks * block_size) are skipped too.
 *  kv_pool       device uint8, layout in the header comment, 16-byte aligned.
 *  num_kv_heads  at most 65535 (TQ_ERR_UNSUPPORTED otherwise; also for
 *                tq_ring_flush).
 * The index count is read from a table of equal bins over the midpoints with
 * at most one midpoint per bin; a config whose midpoints do not allow that
 * (never one tq_config_init made) gets TQ_ERR_UNSUPPORTED, here and in
 * tq_ring_flush.
 *
 * Keys (MSE mode): vec_norm = fp16(||k||), u = Pi k / ||k|| with
 * Pi = (1/sqrt(B)) H_B diag(signs), index j = number of midpoints strictly
 * below u_j. Keys (FP8 mode): E4M3FN, round to nearest even, saturating at
 * +-448. Values: scale = (max - min) / (2^vb - 1), zero = min, both fp16;
 * code_j = clamp(rint((v_j - zero') / scale'), 0, 2^vb - 1) using the
 * stored fp16 scale' and zero'. fp32 with a fixed operation order; the
 * bytes equal the CPU oracle's bit for bit.
 */
tq_status tq_quantize_append(const tq_config *cfg, int layer_idx,
                             const void *k, const void *v, tq_dtype in_dtype,
                             int64_t num_tokens, int num_kv_heads,
                             int64_t k_token_stride, int64_t v_token_stride,
                             const int64_t *slot_mapping,
                             uint8_t *kv_pool, int64_t num_blocks, int block_size,
                             void *stream);

/*
 * Ring flush ([ART] write path: decode tokens wait in a bf16 ring that is
 * compressed as one whole chunk when it overflows). For every sequence b whose
 * ring is full (ring_lens[b] >= ring_cap), its ring tokens 0..ring_cap-1 are
 * quantize-appended, exactly as tq_quantize_append would, at sequence
 * positions seq_lens[b] .. seq_lens[b] + ring_cap - 1 (slot
 * block_tables[b][p / block_size] * block_size + p % block_size); then
 * seq_lens[b] += ring_cap and ring_lens[b] = 0. Other sequences are left
 * alone. Everything runs on the device, in stream order, with no host sync:
 * a decode step calls tq_ring_flush, then tq_ring_append, then
 * tq_decode_attention.
 *
 *  ring_k/ring_v device bf16 [batch][num_kv_heads][ring_cap][head_dim],
 *                16-byte aligned (the layout tq_decode_attention reads).
 *  ring_lens, seq_lens   device int32 [batch], updated in place.
 *  block_tables  device int32 [batch][max_blocks_per_seq]; the caller has
 *                allocated the blocks the flushed positions fall in.
 *                Positions past max_blocks_per_seq, and negative or
 *                out-of-range block ids, are not written.
 *  kv_pool       device, 16-byte aligned, as for tq_quantize_append.
 */
tq_status tq_ring_flush(const tq_config *cfg, int layer_idx,
                        const uint16_t *ring_k, const uint16_t *ring_v, int ring_cap,
                        int32_t *ring_lens, int32_t *seq_lens,
                        const int32_t *block_tables, int max_blocks_per_seq,
                        int batch, int num_kv_heads,
                        uint8_t *kv_pool, int64_t num_blocks, int block_size,
                        void *stream);

/*
 * Ring append ([ART] write path): each sequence's new decode token, k_new /
 * v_new device bf16 [batch][num_kv_heads][head_dim] (16-byte aligned), is
 * copied to ring position ring_lens[b], which then grows by one. A full ring
 * (ring_lens[b] >= ring_cap) is left unchanged and that token is not
 * stored: flush first. Runs on the device, no host sync.
 */
tq_status tq_ring_append(const tq_config *cfg, const uint16_t *k_new, const uint16_t *v_new,
                         int batch, int num_kv_heads,
                         uint16_t *ring_k, uint16_t *ring_v, int ring_cap, int32_t *ring_lens,
                         void *stream);

/*
 * Continuation prefill over the compressed cache ([API] mse_bits docstring:
 * the centroid table is kept for continuation-prefill dequant; computed as
 * in [ART] direction 1, with the query rotated forward). Sequence b's new
 * chunk is rows cu_chunk[b] .. cu_chunk[b+1]-1 of q / k_chunk / v_chunk;
 * row t of it attends to the sequence's hist_lens[b] compressed tokens
 * (through its block table) and to the chunk's exact tokens 0..t (causal):
 *
 *   out[r, g, :] = sum_j softmax_j(scale * q[r, g] . k_j) v_j
 *
 * Query head g reads KV head g / (num_q_heads / num_kv_heads). The (token,
 * head) rows of one KV head are processed in blocks of 32, eight blocks to a
 * workgroup: each history tile is decoded once per workgroup and multiplied
 * with all of its rows, and the chunk's exact tokens are contracted on the
 * matrix cores with the causal limit of each row.
 *
 *  q             device [N][num_q_heads][head_dim], dtype q_dtype, 16-byte
 *                aligned (N = cu_chunk[batch]).
 *  k_chunk/v_chunk device bf16 [N][num_kv_heads][head_dim], 16-byte aligned.
 *  cu_chunk      device int32 [batch + 1], non-decreasing from 0, each chunk
 *                at most max_chunk rows (host bound).
 *  hist_lens     device int32 [batch], at most max_hist (host bound).
 *  kv_pool, block_tables, block_size: as for tq_decode_attention.
 *  out           device fp32 [N][num_q_heads][head_dim], 16-byte aligned.
 *  workspace     device, tq_prefill_workspace_size bytes, 256-byte aligned
 *                (one fp32 partial of head_dim + 4 floats per (row, history
 *                split)); contents on entry do not matter.
 * A history (max_hist > 0) needs num_blocks >= 1 (TQ_ERR_INVALID_ARG);
 * max_chunk * (num_q_heads / num_kv_heads) must fit in 31 bits
 * (TQ_ERR_UNSUPPORTED). The chunk itself is not written to the cache:
 * tq_quantize_append does that.
 */
tq_status tq_prefill_workspace_size(const tq_config *cfg, int batch, int num_q_heads, int num_kv_heads,
                                    int max_chunk, int max_hist, int max_blocks_per_seq,
                                    tq_dtype q_dtype, size_t *bytes_out);

tq_status tq_prefill_attention(const tq_config *cfg, int layer_idx,
                               const void *q, tq_dtype q_dtype,
                               const uint16_t *k_chunk, const uint16_t *v_chunk,
                               const int32_t *cu_chunk, int batch, int max_chunk,
                               int num_q_heads, int num_kv_heads,
                               const uint8_t *kv_pool, int64_t num_blocks, int block_size,
                               const int32_t *block_tables, int max_blocks_per_seq,
                               const int32_t *hist_lens, int max_hist,
                               float softmax_scale, float *out,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Workspace bytes for tq_decode_attention with the same arguments. The
 * decode flattens the batch's (sequence, KV head, 16-token tile) triples and
 * gives every resident wave an equal contiguous range of them, of at least
 * split_tokens tokens (a positive multiple of 16; 0 means 512 with FP8 keys
 * and 256 otherwise), so the work is balanced whatever the mix of lengths.
 * The workspace holds a header (16 + 4 (batch + 1) bytes, rounded up to
 * 256), then the fp32 partials (max, sum, acc[head_dim]) of the compressed
 * tokens: a wave writes one per query head of every (sequence, KV head) it
 * covers, at most max(Hq, batch Hq ceil(max_seq_len / 16) / (split_tokens /
 * 16)) + batch Hq of them (rounded up to 256 bytes), then one per (sequence,
 * query head) and 32 ring tokens (ceil(ring_cap / 32) each). num_splits_out
 * (nullable) receives the partials one (sequence, query head) can have:
 * ceil(max_seq_len / split_tokens) + 1 + ceil(ring_cap / 32).
 */
tq_status tq_decode_workspace_size(const tq_config *cfg, int batch, int num_q_heads,
                                   int max_seq_len, int ring_cap, int split_tokens,
                                   size_t *bytes_out, int *num_splits_out);

/*
 * Fused decode attention over the compressed cache ([ART] direction 1, ring
 * buffer from the write-path section):
 *
 *   out[b, g, :] = sum_t softmax_t(scale * q[b, g] . k_t) v_t
 *
 * over the sequence's compressed tokens 0..seq_lens[b]-1 (dequantized values
 * k_hat, v_hat) followed by its ring tokens 0..ring_lens[b]-1 (exact bf16).
 * Query head g reads KV head g / (num_q_heads / num_kv_heads). For MSE keys
 * the score is computed as n16 * <Pi q, c_idx> (divided by ||c_idx|| under
 * norm correction), never forming k_hat; FP8 and ring keys use q itself.
 * A sequence with no tokens outputs zeros.
 *
 *  q             device [batch][num_q_heads][head_dim], dtype q_dtype
 *                (F32, BF16 or F16), contiguous, 16-byte aligned.
 *  kv_pool       device, as written by tq_quantize_append; 16-byte aligned.
 *  block_tables  device int32 [batch][max_blocks_per_seq].
 *  seq_lens      device int32 [batch], compressed tokens per sequence; must
 *                be <= max_seq_len (the host hint used to size the splits);
 *                tokens beyond it are ignored.
 *  ring_k/ring_v device bf16 [batch][num_kv_heads][ring_cap][head_dim],
 *                16-byte aligned, or
 *                NULL (then ring_lens is ignored and ring_cap must be 0);
 *                ring_lens device int32 [batch], clamped to ring_cap.
 *  softmax_scale <= 0 means 1/sqrt(head_dim).
 *  out           device fp32 [batch][num_q_heads][head_dim], 16-byte aligned.
 *  workspace     device, at least tq_decode_workspace_size bytes, 16-byte
 *                aligned; its contents on entry do not matter.
 *  block_size    a multiple of 16; one pool block (num_kv_heads * block_size
 *                * slot_size_aligned bytes) below 2 GiB (TQ_ERR_UNSUPPORTED
 *                otherwise).
 */
tq_status tq_decode_attention(const tq_config *cfg, int layer_idx,
                              const void *q, tq_dtype q_dtype,
                              int batch, int num_q_heads, int num_kv_heads,
                              const uint8_t *kv_pool, int64_t num_blocks, int block_size,
                              const int32_t *block_tables, int max_blocks_per_seq,
                              const int32_t *seq_lens, int max_seq_len,
                              const void *ring_k, const void *ring_v,
                              const int32_t *ring_lens, int ring_cap,
                              float softmax_scale, float *out,
                              void *workspace, size_t workspace_bytes,
                              int split_tokens, void *stream);

/*
 * tq_decode_attention without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, meaning and result as tq_decode_attention.
 *
 * The header and partials go to a static scratch array of 32 MiB that the
 * library holds on every device it runs on until the process ends (its
 * device address is looked up once per device, on the first call there).
 * A call whose partials need more (its split waves plus batch *
 * num_kv_heads, times num_q_heads / num_kv_heads rows of head_dim + 4
 * floats, plus the ring partials) returns TQ_ERR_WORKSPACE before anything
 * is enqueued. All calls on one device share the array: calls that overlap
 * on one device (concurrent streams, or host threads) race and give wrong
 * results; serialise them. Nothing in the array needs clearing between
 * calls (every partial a call reads is written in that call).
 */
tq_status tq_decode_attention_no_alloc(const tq_config *cfg, int layer_idx,
                                       const void *q, tq_dtype q_dtype,
                                       int batch, int num_q_heads, int num_kv_heads,
                                       const uint8_t *kv_pool, int64_t num_blocks, int block_size,
                                       const int32_t *block_tables, int max_blocks_per_seq,
                                       const int32_t *seq_lens, int max_seq_len,
                                       const void *ring_k, const void *ring_v,
                                       const int32_t *ring_lens, int ring_cap,
                                       float softmax_scale, float *out,
                                       int split_tokens, void *stream);

/*
 * Dequantize slots back to the original basis ([API] docstring: centroids,
 * re-normalized under norm correction, then the inverse rotation; values
 * scale' * code + zero'), fp32 with the oracle's fixed operation order:
 *
 *  k_out[i, h, :], v_out[i, h, :] for i < n, h < num_kv_heads, from physical
 *  slot slot_ids[i] (device int64; -1 or out-of-range ids give zeros).
 *  k_out, v_out: device fp32 [n][num_kv_heads][head_dim].
 */
tq_status tq_dequant(const tq_config *cfg, int layer_idx,
                     const uint8_t *kv_pool, int64_t num_blocks, int num_kv_heads,
                     int block_size, const int64_t *slot_ids, int64_t n,
                     float *k_out, float *v_out, void *stream);

/*
 * Debug checks of caller data, in host memory (no device access, no stream).
 * The calls above clamp or skip bad device-side ids instead of failing: a
 * slot outside the pool is not written, a token of a block outside the pool
 * is masked, and two tokens mapped to one slot race. These checks, run on a
 * host copy before a call, report such inputs. The block/slot space is the
 * paged layout above ([PR] page-size snippet: block_size tokens per block;
 * slot = block * block_size + offset).
 *
 * tq_check_slot_mapping: every entry of slot_mapping[num_tokens] is -1 (skip)
 * or a slot in [0, num_blocks * block_size), and no slot appears twice.
 * TQ_OK, or TQ_ERR_INVALID_ARG with *bad_index (nullable) = the first
 * offending token (for a repeated slot: the later of the two tokens) and a
 * message naming it; *bad_index = -1 on success.
 *
 * tq_check_block_tables: for each sequence b, seq_lens[b] >= 0, its
 * ceil(seq_lens[b] / block_size) logical blocks fit the table row
 * (max_blocks_per_seq), and each of their ids in block_tables[b][i] lies in
 * [0, num_blocks). Blocks shared between sequences are allowed. TQ_OK, or
 * TQ_ERR_INVALID_ARG with *bad_seq / *bad_block (nullable; bad_block -1 when
 * the length itself is at fault).
 */
tq_status tq_check_slot_mapping(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                int block_size, int64_t *bad_index);
tq_status tq_check_block_tables(const int32_t *block_tables, int batch, int max_blocks_per_seq,
                                const int32_t *seq_lens, int64_t num_blocks, int block_size,
                                int *bad_seq, int *bad_block);

/* Message of the last failed call on this thread ("" if none). */
const char *tq_last_error(void);

/* Library version string, e.g. "tq-mi355x 0.1.0 gfx950". */
const char *tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
