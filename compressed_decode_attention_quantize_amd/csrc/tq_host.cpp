// Host core of the library: configuration (TurboQuantConfig arithmetic),
// Lloyd-Max tables, per-layer random signs, the decode split plan, and the
// thread-local error message. No HIP calls here.
//
// Sources: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
// TurboQuantConfig (fields, properties, named presets, from_cache_dtype);
// prhub summary of vLLM PR #39931 (TurboQuant page = block_size *
// num_kv_heads * slot bytes).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <string>
#include <utility>
#include <vector>

#include "tq_internal.h"

namespace tq {

namespace {
thread_local std::string g_last_error;

struct Preset {
  const char *name;
  int key_bits, value_bits, nc;
};
// In the order the TurboQuantConfig docstring lists them.
constexpr Preset kPresets[] = {
    {"turboquant_k8v4", 8, 4, 0},
    {"turboquant_4bit_nc", 4, 4, 1},
    {"turboquant_k3v4_nc", 3, 4, 1},
    {"turboquant_3bit_nc", 3, 3, 1},
};

int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Lloyd-Max quantizer of the standard normal (Lloyd's fixed-point iteration:
// thresholds at the midpoints of adjacent levels, each level the mean of the
// density over its cell). The positive half is iterated and mirrored, so the
// table is exactly antisymmetric. float64.
constexpr int kLloydIterations = 2000;

double normal_cell_mean(double a, double b) {  // 0 <= a < b <= inf
  const double inv_sqrt_2pi = 1.0 / std::sqrt(2.0 * M_PI);
  const double pa = std::exp(-0.5 * a * a) * inv_sqrt_2pi;
  const double pb = std::isinf(b) ? 0.0 : std::exp(-0.5 * b * b) * inv_sqrt_2pi;
  const double ea = std::erfc(a / std::sqrt(2.0));
  const double eb = std::isinf(b) ? 0.0 : std::erfc(b / std::sqrt(2.0));
  return (pa - pb) / (0.5 * (ea - eb));
}

void standard_normal_levels(int levels, double *out) {
  const int half = levels / 2;
  double c[8], edge[9];
  for (int k = 0; k < half; ++k) c[k] = (k + 0.5) * 3.0 / half;
  for (int it = 0; it < kLloydIterations; ++it) {
    edge[0] = 0.0;
    for (int k = 1; k < half; ++k) edge[k] = (c[k - 1] + c[k]) / 2.0;
    edge[half] = INFINITY;
    for (int k = 0; k < half; ++k) c[k] = normal_cell_mean(edge[k], edge[k + 1]);
  }
  for (int k = 0; k < half; ++k) {
    out[half + k] = c[k];
    out[half - 1 - k] = -c[k];
  }
}

// SplitMix64 (Steele, Lea and Flood 2014), one step.
uint64_t splitmix64_next(uint64_t &state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool supported_head_dim(int d) { return d == 64 || d == 96 || d == 128; }

// IEEE binary16 value of a positive normal float (round to nearest even).
double f16_round(float v) {
  int e;
  std::frexp(static_cast<double>(v), &e);  // v = m * 2^e, m in [0.5, 1)
  const double unit = std::ldexp(1.0, e - 11);  // f16 spacing in this binade
  return std::nearbyint(static_cast<double>(v) / unit) * unit;
}

// sigma = 1 + i/2^18 minimising the largest relative error of
// fp16(fp32(sigma * c_k)) over the table's positive levels.
float best_centroid_scale(const float *c, int n) {
  constexpr int kSteps = 1 << 18;
  float best_s = 1.0f;
  double best_e = INFINITY;
  for (int i = 0; i < kSteps; ++i) {
    const float sg = 1.0f + static_cast<float>(i) / static_cast<float>(kSteps);
    double worst = 0.0;
    for (int k = n / 2; k < n; ++k) {
      const float prod = c[k] * sg;
      const double e = std::fabs(f16_round(prod) - static_cast<double>(prod)) / static_cast<double>(prod);
      if (e > worst) worst = e;
      if (worst >= best_e) break;
    }
    if (worst < best_e) {
      best_e = worst;
      best_s = sg;
    }
  }
  return best_s;
}

}  // namespace

tq_status fail(tq_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

void clear_error() { g_last_error.clear(); }

tq_status check_config(const tq_config *cfg) {
  // Cheap per-call validation: the fields and the derived sizes (the tables
  // are trusted to be the ones tq_config_init wrote).
  if (!cfg) return fail(TQ_ERR_INVALID_ARG, "config is NULL");
  const int d = cfg->head_dim, kb = cfg->key_quant_bits, vb = cfg->value_quant_bits;
  if (!supported_head_dim(d) || (kb != 3 && kb != 4 && kb != 8) || (vb < 2 || vb > 4))
    return fail(TQ_ERR_INVALID_ARG, "config has an unsupported head_dim / bit width");
  const int fp8 = kb == 8;
  const int kp = fp8 ? d : ceil_div_i(d * kb, 8) + 2;
  const int vp = ceil_div_i(d * vb, 8) + 4;
  const int mse = fp8 ? vb : kb;
  if (cfg->key_fp8 != fp8 || cfg->key_packed_size != kp || cfg->value_packed_size != vp ||
      cfg->slot_size != kp + vp || cfg->slot_size_aligned != kp + vp + ((kp + vp) % 2) ||
      cfg->wht_block != (d & (-d)) || cfg->n_centroids != (1 << mse) ||
      !(cfg->centroid_scale >= 1.0f && cfg->centroid_scale < 2.0f))
    return fail(TQ_ERR_INVALID_ARG, "config was modified after tq_config_init");
  clear_error();
  return TQ_OK;
}

namespace {

// The bin of x exactly as the quantize kernel computes it: one correctly
// rounded fma, a clamp to [0, kLmBins - 1] (a NaN becomes 0), truncation.
// Every step is non-decreasing in x.
int lm_bin(float x, float scale, float offset) {
  const float t = std::fmin(std::fmax(std::fma(x, scale, offset), 0.0f), static_cast<float>(kLmBins - 1));
  return static_cast<int>(t);
}

}  // namespace

// The Lloyd-Max index of u is the number of midpoints strictly below u
// (vLLM API page, TurboQuantConfig: Lloyd-Max keys). With bin() non-decreasing
// and at most one midpoint per bin, every midpoint in a bin below bin(u) is
// below u and every one in a bin above is above it, so the count is the
// number of midpoints in lower bins plus (u > the midpoint in u's own bin).
// A NaN u falls in bin 0, below every midpoint's bin, and gets 0.
bool lloyd_max_bins(const tq_config &cfg, QuantParams &p) {
  const int nm = cfg.n_centroids - 1;
  if (nm < 1 || nm > 15) return false;
  const double lo = cfg.midpoints[0], hi = cfg.midpoints[nm - 1];
  if (!std::isfinite(lo) || !std::isfinite(hi) || !(hi > lo)) return false;
  const double w = (hi - lo) / (kLmBins - 2);
  p.lm_scale = static_cast<float>(1.0 / w);
  p.lm_offset = static_cast<float>(1.0 - lo / w);
  int bins[15];
  for (int k = 0; k < nm; ++k) {
    bins[k] = lm_bin(cfg.midpoints[k], p.lm_scale, p.lm_offset);
    if (k > 0 && bins[k] <= bins[k - 1]) return false;
  }
  const float inf = std::numeric_limits<float>::infinity();
  for (int j = 0; j < kLmBins; ++j) {
    float mid = inf;
    uint32_t below = 0;
    for (int k = 0; k < nm; ++k) {
      if (bins[k] < j) ++below;
      if (bins[k] == j) mid = cfg.midpoints[k];
    }
    std::memcpy(&p.lm_table[2 * j], &mid, sizeof(mid));
    p.lm_table[2 * j + 1] = below;
  }
  return true;
}

void layer_sign_mask(const tq_config &cfg, int layer_idx, uint32_t words[4]) {
  uint64_t state = static_cast<uint64_t>(cfg.seed) + static_cast<uint64_t>(layer_idx) * 1337ull;
  words[0] = words[1] = words[2] = words[3] = 0;
  for (int j = 0; j < cfg.head_dim; ++j) {
    const uint64_t z = splitmix64_next(state);
    if (z >> 63) words[j >> 5] |= 1u << (j & 31);
  }
}

namespace {

void plan_offsets(const tq_config &cfg, int batch, int num_q_heads, SplitPlan *plan) {
  const size_t row = static_cast<size_t>(cfg.head_dim + 4) * sizeof(float);  // [m, l, -, -, acc[D]]
  plan->header_bytes = ((16 + 4 * (static_cast<size_t>(batch) + 1) + 255) / 256) * 256;
  plan->ring_offset = plan->header_bytes + ((static_cast<size_t>(plan->head_rows) * row + 255) / 256) * 256;
  plan->workspace_bytes = plan->ring_offset + static_cast<size_t>(batch) * num_q_heads * plan->ring_chunks * row;
}

}  // namespace

tq_status plan_decode(const tq_config &cfg, int batch, int num_q_heads, int max_seq_len,
                      int ring_cap, int split_tokens, SplitPlan *plan) {
  if (batch < 0 || num_q_heads <= 0 || max_seq_len < 0 || ring_cap < 0)
    return fail(TQ_ERR_INVALID_ARG, "decode plan: negative batch/max_seq_len/ring_cap or num_q_heads <= 0");
  if (split_tokens < 0 || split_tokens % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "split_tokens must be 0 (auto) or a positive multiple of 16");
  // The automatic range: FP8-key decode streams bytes with little compute
  // per tile, and measures fastest with ~2 waves per SIMD on 512-token
  // ranges (fewer range start-ups and partials); the MSE-key decode is
  // latency-bound and keeps every resident wave busy on 256-token ranges.
  const int min_tokens = split_tokens > 0 ? split_tokens : (cfg.key_fp8 ? kMinTokensPerWaveFp8 : kMinTokensPerWave);
  plan->split_tokens = min_tokens;
  plan->max_splits = max_seq_len > 0 ? ceil_div_i(max_seq_len, min_tokens) + 1 : 0;
  plan->ring_chunks = (ring_cap + kRingChunk - 1) / kRingChunk;
  // Compressed partials: wave w writes row w + s for every (sequence, KV
  // head) segment s it covers, so rows < active waves + segments. The waves
  // activated are at most max(1, tiles / (min_tokens / 16)) with tiles <=
  // batch * Hkv * ceil(max_seq_len / 16); in rows of one query head that is
  // at most max(Hq, batch * Hq * tiles per sequence / tiles per wave)
  // + batch * Hq, whatever the number of KV heads.
  if (max_seq_len > 0) {
    const long long tiles = (static_cast<long long>(max_seq_len) + 15) / 16;
    const long long per_wave = min_tokens / 16;
    const long long wave_rows = (static_cast<long long>(batch) * num_q_heads * tiles + per_wave - 1) / per_wave;
    plan->head_rows = std::max<long long>(num_q_heads, wave_rows) + static_cast<long long>(batch) * num_q_heads;
  } else {
    plan->head_rows = 0;
  }
  plan_offsets(cfg, batch, num_q_heads, plan);
  return TQ_OK;
}

void plan_for_launch(const tq_config &cfg, int batch, int num_q_heads, int num_kv_heads, long long waves,
                     SplitPlan *plan) {
  if (plan->head_rows > 0) {
    const long long g = num_q_heads / num_kv_heads;
    const long long rows = (std::max(waves, 1LL) + static_cast<long long>(batch) * num_kv_heads) * g;
    plan->head_rows = std::min<long long>(plan->head_rows, rows);
  }
  plan_offsets(cfg, batch, num_q_heads, plan);
}

}  // namespace tq

using namespace tq;

TQ_EXPORT tq_status tq_config_init(int head_dim, int key_bits, int value_bits, int norm_correction,
                                   int64_t seed, tq_config *out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_config_init: out is NULL");
  if (!supported_head_dim(head_dim))
    return fail(TQ_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) + " not supported (64, 96, 128)");
  if (key_bits != 3 && key_bits != 4 && key_bits != 8)
    return fail(TQ_ERR_INVALID_ARG, "key_quant_bits must be 3, 4 (MSE) or 8 (FP8), got " + std::to_string(key_bits));
  if (value_bits < 2 || value_bits > 4)
    return fail(TQ_ERR_INVALID_ARG, "value_quant_bits must be 2, 3 or 4, got " + std::to_string(value_bits));
  tq_config c;
  std::memset(&c, 0, sizeof(c));
  c.head_dim = head_dim;
  c.key_quant_bits = key_bits;
  c.value_quant_bits = value_bits;
  c.norm_correction = norm_correction ? 1 : 0;
  c.seed = seed;
  // Derived properties, as the printed TurboQuantConfig properties compute them.
  c.key_fp8 = key_bits == 8;
  c.mse_bits = c.key_fp8 ? value_bits : key_bits;
  c.key_mse_bits = c.key_fp8 ? 0 : key_bits;
  c.centroid_bits = c.mse_bits;
  c.n_centroids = 1 << c.mse_bits;
  c.key_packed_size = c.key_fp8 ? head_dim : ceil_div_i(head_dim * c.key_mse_bits, 8) + 2;
  c.value_packed_size = ceil_div_i(head_dim * value_bits, 8) + 4;
  c.slot_size = c.key_packed_size + c.value_packed_size;
  c.slot_size_aligned = c.slot_size + (c.slot_size % 2);
  c.wht_block = head_dim & (-head_dim);
  // Lloyd-Max table of N(0, 1/D): the standard-normal levels scaled by 1/sqrt(D).
  double lv[16];
  standard_normal_levels(c.n_centroids, lv);
  const double sd = std::sqrt(static_cast<double>(head_dim));
  double c64[16];
  for (int k = 0; k < c.n_centroids; ++k) {
    c64[k] = lv[k] / sd;
    c.centroids[k] = static_cast<float>(c64[k]);
  }
  for (int k = 0; k + 1 < c.n_centroids; ++k) c.midpoints[k] = static_cast<float>((c64[k] + c64[k + 1]) / 2.0);
  c.centroid_scale = best_centroid_scale(c.centroids, c.n_centroids);
  *out = c;
  clear_error();
  return TQ_OK;
}

TQ_EXPORT tq_status tq_config_from_preset(const char *preset, int head_dim, tq_config *out) {
  if (!preset || !out) return fail(TQ_ERR_INVALID_ARG, "tq_config_from_preset: NULL argument");
  for (const Preset &p : kPresets)
    if (std::strcmp(p.name, preset) == 0) return tq_config_init(head_dim, p.key_bits, p.value_bits, p.nc, 42, out);
  std::string valid;
  for (const Preset &p : kPresets) {
    if (!valid.empty()) valid += ", ";
    valid += p.name;
  }
  return fail(TQ_ERR_UNKNOWN_PRESET,
              std::string("Unknown TurboQuant cache dtype: '") + preset + "'. Valid presets: " + valid);
}

TQ_EXPORT tq_status tq_layer_config(const tq_config *base, int layer_idx, int initial_layers,
                                    int initial_layers_key_bits, tq_config *out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_layer_config: out is NULL");
  const tq_status st = check_config(base);
  if (st != TQ_OK) return st;
  if (layer_idx < 0 || initial_layers < 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_layer_config: layer_idx and initial_layers must be >= 0");
  if (initial_layers_key_bits < 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_layer_config: initial_layers_key_bits must be >= 0 (0 = base + 1)");
  int kb = base->key_quant_bits;
  if (layer_idx < initial_layers) {
    if (initial_layers_key_bits > 0)
      kb = initial_layers_key_bits;
    else if (!base->key_fp8)
      kb = base->key_quant_bits + 1;
  }
  tq_config c;
  const tq_status s2 = tq_config_init(base->head_dim, kb, base->value_quant_bits, base->norm_correction,
                                      base->seed, &c);
  if (s2 != TQ_OK) return s2;
  *out = c;
  return TQ_OK;
}

TQ_EXPORT int tq_boundary_skip_layers(int num_layers, int n, int hybrid, int32_t *out, int out_cap) {
  if (out_cap < 0 || (out_cap > 0 && !out)) {
    fail(TQ_ERR_INVALID_ARG, "tq_boundary_skip_layers: out is NULL or out_cap < 0");
    return -1;
  }
  clear_error();
  if (hybrid || n <= 0 || num_layers <= 0) return 0;
  n = std::min(n, num_layers / 2);
  // first n, then last n, skipping the overlap (num_layers <= 2 n cannot
  // happen after the cap, but the loop keeps indices unique either way)
  int count = 0;
  for (int i = 0; i < num_layers; ++i) {
    if (i < n || i >= num_layers - n) {
      if (count < out_cap) out[count] = i;
      ++count;
    }
  }
  return count;
}

TQ_EXPORT int64_t tq_attn_page_size_1_token(const tq_config *cfg, int num_kv_heads, int skip_dtype_bytes) {
  if (check_config(cfg) != TQ_OK) return -1;
  if (num_kv_heads <= 0 || skip_dtype_bytes < 0) {
    fail(TQ_ERR_INVALID_ARG, "tq_attn_page_size_1_token: num_kv_heads must be positive, skip_dtype_bytes >= 0");
    return -1;
  }
  const int64_t tq = static_cast<int64_t>(num_kv_heads) * cfg->slot_size_aligned;
  if (skip_dtype_bytes == 0) return tq;
  const int64_t skip = 2ll * num_kv_heads * cfg->head_dim * skip_dtype_bytes;
  int64_t a = tq, b = skip;
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return tq / a * skip;
}

TQ_EXPORT int32_t tq_slot_size(const tq_config *cfg, int aligned) {
  if (check_config(cfg) != TQ_OK) return -1;
  return aligned ? cfg->slot_size_aligned : cfg->slot_size;
}

TQ_EXPORT int64_t tq_page_size(const tq_config *cfg, int num_kv_heads, int block_size) {
  if (check_config(cfg) != TQ_OK) return -1;
  if (num_kv_heads <= 0 || block_size <= 0) {
    fail(TQ_ERR_INVALID_ARG, "tq_page_size: num_kv_heads and block_size must be positive");
    return -1;
  }
  return static_cast<int64_t>(block_size) * num_kv_heads * cfg->slot_size_aligned;
}

TQ_EXPORT tq_status tq_layer_signs(const tq_config *cfg, int layer_idx, float *signs_out) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (!signs_out) return fail(TQ_ERR_INVALID_ARG, "tq_layer_signs: signs_out is NULL");
  uint32_t w[4];
  layer_sign_mask(*cfg, layer_idx, w);
  for (int j = 0; j < cfg->head_dim; ++j) signs_out[j] = ((w[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
  return TQ_OK;
}

TQ_EXPORT tq_status tq_decode_workspace_size(const tq_config *cfg, int batch, int num_q_heads,
                                             int max_seq_len, int ring_cap, int split_tokens,
                                             size_t *bytes_out, int *num_splits_out) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (!bytes_out) return fail(TQ_ERR_INVALID_ARG, "tq_decode_workspace_size: bytes_out is NULL");
  SplitPlan plan;
  st = plan_decode(*cfg, batch, num_q_heads, max_seq_len, ring_cap, split_tokens, &plan);
  if (st != TQ_OK) return st;
  *bytes_out = plan.workspace_bytes;
  if (num_splits_out) *num_splits_out = plan.max_splits + plan.ring_chunks;
  return TQ_OK;
}

// Debug checks of caller data in host memory. The kernels clamp or skip bad
// device-side ids (an out-of-range slot is not written, a token of an
// out-of-range block is masked) and two tokens mapped to one slot race; these
// make such inputs visible before a call instead.
TQ_EXPORT tq_status tq_check_slot_mapping(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                          int block_size, int64_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_check_slot_mapping: need num_tokens >= 0, num_blocks >= 0, block_size > 0");
  if (num_tokens > 0 && !slot_mapping) return fail(TQ_ERR_INVALID_ARG, "tq_check_slot_mapping: slot_mapping is NULL");
  if (num_blocks > INT64_MAX / block_size)
    return fail(TQ_ERR_INVALID_ARG, "tq_check_slot_mapping: num_blocks * block_size overflows");
  const int64_t cap = num_blocks * block_size;
  std::vector<std::pair<int64_t, int64_t>> used;  // (slot, token)
  used.reserve(static_cast<size_t>(num_tokens));
  for (int64_t i = 0; i < num_tokens; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot == -1) continue;  // skipped token
    if (slot < 0 || slot >= cap) {
      if (bad_index) *bad_index = i;
      return fail(TQ_ERR_INVALID_ARG, "tq_check_slot_mapping: token " + std::to_string(i) + " maps to slot " +
                                          std::to_string(slot) + ", outside the pool's " + std::to_string(cap) +
                                          " slots");
    }
    used.emplace_back(slot, i);
  }
  std::sort(used.begin(), used.end());
  // the first token (in token order) whose slot an earlier token also takes
  int64_t worst = -1, slot_of = 0, first_of = 0;
  for (size_t j = 1; j < used.size(); ++j) {
    if (used[j].first == used[j - 1].first && (worst < 0 || used[j].second < worst)) {
      worst = used[j].second;
      slot_of = used[j].first;
      first_of = used[j - 1].second;
    }
  }
  if (worst >= 0) {
    if (bad_index) *bad_index = worst;
    return fail(TQ_ERR_INVALID_ARG, "tq_check_slot_mapping: tokens " + std::to_string(first_of) + " and " +
                                        std::to_string(worst) + " both write slot " + std::to_string(slot_of));
  }
  clear_error();
  return TQ_OK;
}

TQ_EXPORT tq_status tq_check_block_tables(const int32_t *block_tables, int batch, int max_blocks_per_seq,
                                          const int32_t *seq_lens, int64_t num_blocks, int block_size,
                                          int *bad_seq, int *bad_block) {
  if (bad_seq) *bad_seq = -1;
  if (bad_block) *bad_block = -1;
  if (batch < 0 || max_blocks_per_seq < 0 || num_blocks < 0 || block_size <= 0)
    return fail(TQ_ERR_INVALID_ARG,
                "tq_check_block_tables: need batch >= 0, max_blocks_per_seq >= 0, num_blocks >= 0, block_size > 0");
  if (batch > 0 && (!seq_lens || (max_blocks_per_seq > 0 && !block_tables)))
    return fail(TQ_ERR_INVALID_ARG, "tq_check_block_tables: NULL pointer");
  for (int b = 0; b < batch; ++b) {
    const int64_t len = seq_lens[b];
    const int64_t need = (std::max<int64_t>(len, 0) + block_size - 1) / block_size;
    if (len < 0 || need > max_blocks_per_seq) {
      if (bad_seq) *bad_seq = b;
      return fail(TQ_ERR_INVALID_ARG, "tq_check_block_tables: sequence " + std::to_string(b) + " has length " +
                                          std::to_string(len) + ", which its table row of " +
                                          std::to_string(max_blocks_per_seq) + " blocks cannot hold");
    }
    for (int64_t i = 0; i < need; ++i) {
      const int32_t id = block_tables[static_cast<int64_t>(b) * max_blocks_per_seq + i];
      if (id < 0 || id >= num_blocks) {
        if (bad_seq) *bad_seq = b;
        if (bad_block) *bad_block = static_cast<int>(i);
        return fail(TQ_ERR_INVALID_ARG, "tq_check_block_tables: sequence " + std::to_string(b) + ", logical block " +
                                            std::to_string(i) + " has id " + std::to_string(id) +
                                            ", outside the pool's " + std::to_string(num_blocks) + " blocks");
      }
    }
  }
  clear_error();
  return TQ_OK;
}

TQ_EXPORT const char *tq_last_error(void) { return g_last_error.c_str(); }

TQ_EXPORT const char *tq_version(void) { return "tq-mi355x 0.1.0 gfx950"; }
