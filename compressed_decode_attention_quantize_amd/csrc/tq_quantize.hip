// Quantize-and-append and dequant kernels.
//
// Sources: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
// TurboQuantConfig docstring (Walsh-Hadamard rotation + Lloyd-Max keys,
// uniform values, FP8 keys, norm correction at dequant) and the byte layouts
// of key_packed_size / value_packed_size / slot_size.
//
// Layout of the work: one (token, head) vector is handled by a team of D/8
// lanes holding 8 consecutive elements each (see Team<D>), so the rotation is
// in-register butterflies plus lane-xor exchanges and the norm / min / max
// are lane reductions. fp32 op order is fixed (the library is built with
// -ffp-contract=off; sqrt and divide are correctly rounded) so the bytes
// match the CPU oracle exactly.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// Write the NB (<= 4) little-endian low bytes of w at dst. Fields of an even
// size start at an even offset of an even-sized slot (slot_size_aligned is
// even, the pool 16-byte aligned), so they go out as 16-bit stores; a field
// of 3 bytes can start at an odd offset and goes out byte by byte.
template <int NB>
__device__ __forceinline__ void store_field(uint8_t *dst, uint32_t w) {
  static_assert(NB >= 1 && NB <= 4, "field bytes");
  if constexpr (NB % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NB; i += 2) *reinterpret_cast<uint16_t *>(dst + i) = static_cast<uint16_t>(w >> (8 * i));
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) dst[i] = static_cast<uint8_t>(w >> (8 * i));
  }
}

// The 8 consecutive elements of a lane, read as raw bits (16-byte aligned
// source): one 16-byte load for bf16/f16 (a), two for f32 (a, b).
template <int DT>  // 0 = f32, 1 = bf16, 2 = f16 (tq_dtype values)
__device__ __forceinline__ void load_raw8(const void *base, int64_t elem, uint4 &a, uint4 &b) {
  if constexpr (DT == 0) {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + elem);
    a = q[0];
    b = q[1];
  } else {
    a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
  }
}

// Raw bits of load_raw8 as fp32 (exact for every input format).
template <int DT>
__device__ __forceinline__ void widen8(const uint4 &a, const uint4 &b, float x[8]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if constexpr (DT == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 1) {
        x[2 * i] = bf16_bits_to_float(w[i] & 0xffffu);
        x[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
      } else {
        x[2 * i] = f16_bits_to_float(w[i] & 0xffffu);
        x[2 * i + 1] = f16_bits_to_float(w[i] >> 16);
      }
    }
  }
}

// The 8 sign bits of lane r (bit i: element 8r + i is negated) from the four
// mask words held as values, so no lane reads a word from a selected address.
__device__ __forceinline__ uint32_t lane_signs(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int r) {
  const uint32_t word = r < 8 ? (r < 4 ? w0 : w1) : (r < 12 ? w2 : w3);
  return (word >> (8 * (r & 3))) & 0xffu;
}

// Minimum (or maximum) over a 16- or 8-lane row block of values that are
// already canonical (outputs of arithmetic: no signalling NaN), with the DPP
// lane moves folded into v_min/v_max. The compiler's fminf/fmaxf re-quiet a
// DPP-moved operand first, as it cannot tell it is canonical; for canonical
// operands IEEE-mode v_min/v_max give exactly fminf/fmaxf (a quiet NaN loses
// to a number). Each step opens with two wait states: a DPP source must not
// be read right after a VALU op writes it.
template <int LANES, bool MAX>
__device__ __forceinline__ float row_reduce_canonical(float v) {
  static_assert(LANES == 8 || LANES == 16, "row block");
  float t, u;
  if constexpr (MAX) {
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(t) : "v"(v));
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(u) : "v"(t));
    asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(t) : "v"(u));
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %2 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(v) : "v"(t), "v"(u));
    if constexpr (LANES == 16)
      asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                   : "=&v"(t) : "v"(v));
    else
      t = v;
  } else {
    asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(t) : "v"(v));
    asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(u) : "v"(t));
    asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(t) : "v"(u));
    asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %1, %2 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "=&v"(v) : "v"(t), "v"(u));
    if constexpr (LANES == 16)
      asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                   : "=&v"(t) : "v"(v));
    else
      t = v;
  }
  return t;
}

template <int BITS>
__device__ __forceinline__ uint32_t pack8(const uint32_t c[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= c[i] << (BITS * i);
  return w;
}

template <int BITS>
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t c[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = (w >> (BITS * i)) & ((1u << BITS) - 1u);
}

// Reads the BITS*8-bit group of lane r from a packed field (byte aligned).
template <int BITS>
__device__ __forceinline__ uint32_t load_group(const uint8_t *field, int r) {
  const uint8_t *p = field + BITS * r;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) w |= static_cast<uint32_t>(p[i]) << (8 * i);
  return w;
}

// Lloyd-Max index of u: the number of midpoints strictly below u, from the
// bin table the host built (QuantParams::lm_table). bin(u) is the host's bin
// function step for step (fma, clamp with NaN -> 0, truncation); the table
// entry holds the bin's midpoint (+inf if none) and the count of midpoints in
// lower bins, so one compare finishes the count. NaN gets 0.
__device__ __forceinline__ uint32_t lm_index(float u, float scale, float offset, const uint2 *lut) {
  const float t = fminf(fmaxf(fmaf(u, scale, offset), 0.0f), static_cast<float>(kLmBins - 1));
  const uint2 e = lut[static_cast<int>(t)];
  return e.y + (u > __uint_as_float(e.x) ? 1u : 0u);
}

template <int D, int KB, int VB, int DT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  using T = Team<D>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int team = lane / T::kLanes;
  const int r = lane - team * T::kLanes;           // lane within the team
  const int team_base = team * T::kLanes;
  const int lane_in_block = r % T::kBlockLanes;
  // grid (token groups, KV heads): the teams of a wave take consecutive
  // tokens of one head, whose slots are neighbours in a pool block
  const int64_t tok = (static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave) * T::kPerWave + team;
  const bool active = team < T::kPerWave && tok < p.num_tokens;
  const int64_t t = active ? tok : 0;
  const int h = static_cast<int>(blockIdx.y);

  // the row bits of this (token, head), and its slot; zeros where nothing is
  // read (the team then computes on zeros and writes nothing)
  int64_t slot = -1;
  uint4 xa = make_uint4(0, 0, 0, 0), xb = xa, va = xa, vb = xa;
  if (p.ring_lens) {
    // ring flush: token t is position pos of sequence seq; a ring that is not
    // full is not read. A team shares its token, so this is uniform per team.
    const int64_t seq = t / p.ring_cap;
    const int pos = static_cast<int>(t - seq * p.ring_cap);
    if (active && p.ring_lens[seq] >= p.ring_cap) {
      const int64_t at = static_cast<int64_t>(max(p.seq_lens[seq], 0)) + pos;
      const int64_t lblk = at / p.block_size;
      if (lblk < p.max_blocks_per_seq) {
        const int64_t phys = p.block_tables[seq * p.max_blocks_per_seq + lblk];
        if (phys >= 0) slot = phys * p.block_size + (at - lblk * p.block_size);
      }
    }
    if (slot >= 0) {
      const int64_t off = ((seq * p.num_kv_heads + h) * p.ring_cap + pos) * D + 8 * r;
      load_raw8<DT>(p.k, off, xa, xb);
      load_raw8<DT>(p.v, off, va, vb);
    }
  } else if (active) {
    // the slot id and both rows are independent reads, issued together
    slot = p.slot_mapping[t];
    load_raw8<DT>(p.k, t * p.k_stride + static_cast<int64_t>(h) * D + 8 * r, xa, xb);
    load_raw8<DT>(p.v, t * p.v_stride + static_cast<int64_t>(h) * D + 8 * r, va, vb);
  }
  // Lloyd-Max bin table (MSE keys) into LDS, behind the row reads; read after
  // the barrier in the key path
  __shared__ uint2 lut[KB == 8 ? 1 : kLmBins];
  if constexpr (KB != 8) {
    if (threadIdx.x < kLmBins) lut[threadIdx.x] = make_uint2(p.lm_table[2 * threadIdx.x], p.lm_table[2 * threadIdx.x + 1]);
  }
  float x[8], v[8];
  widen8<DT>(xa, xb, x);
  widen8<DT>(va, vb, v);
  const bool write = active && slot >= 0 && slot < p.total_slots;
  if (!write) slot = 0;
  int64_t blk, off;
  if ((p.block_size & (p.block_size - 1)) == 0) {
    // power-of-two block: shift and mask instead of a 64-bit division
    blk = slot >> __builtin_ctz(static_cast<uint32_t>(p.block_size));
    off = slot & (p.block_size - 1);
  } else {
    blk = slot / p.block_size;
    off = slot - blk * p.block_size;
  }
  uint8_t *dst = p.pool + ((blk * p.num_kv_heads + h) * p.block_size + off) * p.slot_bytes;

  // ---- keys
  if constexpr (KB == 8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= float_to_e4m3fn(x[i]) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= float_to_e4m3fn(x[4 + i]) << (8 * i);
    if (write) {
      store_field<4>(dst + 8 * r, lo);
      store_field<4>(dst + 8 * r + 4, hi);
    }
  } else {
    const float n2 = team_sumsq<D>(x, team_base);
    const float n = sqrtf(n2);
    const uint32_t sbits = lane_signs(p.sign_words[0], p.sign_words[1], p.sign_words[2], p.sign_words[3], r);
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = flip_sign(x[i], (sbits >> i) & 1u);
    team_wht<D>(z, lane_in_block);
    const float pn = n * p.sqrt_block;
    // divide unconditionally and select (no branch between the WHT's lane
    // moves and their adds)
    const float inv_pn = 1.0f / pn;
    const float rcp = (n == 0.0f) ? 0.0f : inv_pn;
    static_assert(KB == 3 || KB == 4, "MSE key widths");
    __syncthreads();  // the bin table is in LDS (no thread has left the kernel)
    uint32_t idx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) idx[i] = lm_index(z[i] * rcp, p.lm_scale, p.lm_offset, lut);
    uint32_t w = pack8<KB>(idx);
    // computed before the store branch, so the WHT's last lane moves stay in
    // one block with their adds (and fold into them)
    asm volatile("" : "+v"(w));
    if (write) {
      store_field<KB>(dst + KB * r, w);
      if (r == 0) store_field<2>(dst + (D * KB) / 8, float_to_f16_bits(n));
    }
  }

  // ---- values
  // quieted first: a signalling NaN is then skipped by min and max like any
  // NaN (v_min3/v_max3 would return it), and the lane reductions below see
  // canonical values only
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_canonicalizef(v[i]);
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  if constexpr (T::kBlocks == 1) {
    // one row block per vector (D = 64, 128); in-lane results are canonical
    mn = row_reduce_canonical<T::kBlockLanes, false>(mn);
    mx = row_reduce_canonical<T::kBlockLanes, true>(mx);
  } else {
    mn = team_min<D>(mn, team_base);
    mx = team_max<D>(mx, team_base);
  }
  constexpr float kLevels = static_cast<float>((1 << VB) - 1);
  const float scale32 = (mx - mn) / kLevels;
  const uint32_t s16 = float_to_f16_bits(scale32);
  const uint32_t z16 = float_to_f16_bits(mn);
  const float s1 = f16_bits_to_float(s16);
  const float z1 = f16_bits_to_float(z16);
  const float inv = (s1 == 0.0f) ? 0.0f : 1.0f / s1;
  uint32_t code[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float qv = rintf((v[i] - z1) * inv);
    code[i] = static_cast<uint32_t>(fminf(fmaxf(qv, 0.0f), kLevels));
  }
  const uint32_t wv = pack8<VB>(code);
  if (write) {
    uint8_t *vf = dst + p.key_bytes;
    store_field<VB>(vf + VB * r, wv);
    if (r == 0) {
      store_field<2>(vf + (D * VB) / 8, s16);
      store_field<2>(vf + (D * VB) / 8 + 2, z16);
      if (p.slot_bytes > p.key_bytes + (D * VB) / 8 + 4) dst[p.slot_bytes - 1] = 0;
    }
  }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantParams p) {
  using T = Team<D>;
  __shared__ float cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = p.centroids[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int team = lane / T::kLanes;
  const int r = lane - team * T::kLanes;
  const int team_base = team * T::kLanes;
  const int lane_in_block = r % T::kBlockLanes;
  const int64_t vec = (static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave) * T::kPerWave + team;
  const int64_t nvec = p.n * p.num_kv_heads;
  const bool active = team < T::kPerWave && vec < nvec;
  const int64_t i = active ? vec / p.num_kv_heads : 0;
  const int h = active ? static_cast<int>(vec - i * p.num_kv_heads) : 0;
  int64_t slot = active ? p.slot_ids[i] : -1;
  const bool valid = active && slot >= 0 && slot < p.total_slots;
  if (!valid) slot = 0;
  const int64_t blk = slot / p.block_size;
  const int64_t off = slot - blk * p.block_size;
  const uint8_t *src = p.pool + ((blk * p.num_kv_heads + h) * p.block_size + off) * p.slot_bytes;

  float k[8], v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) k[e] = v[e] = 0.0f;
  // validity is uniform over a team, so the team's lane exchanges stay paired
  if (valid) {
  if constexpr (KB == 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = e4m3fn_to_float(src[8 * r + e]);
  } else {
    uint32_t idx[8];
    unpack8<KB>(load_group<KB>(src, r), idx);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = cent[idx[e]];
    if (p.norm_correction) {
      const float cn = sqrtf(team_sumsq<D>(y, team_base));
      const float inv = 1.0f / cn;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = y[e] * inv;
    }
    team_wht<D>(y, lane_in_block);
    const uint32_t nb = static_cast<uint32_t>(src[(D * KB) / 8]) | (static_cast<uint32_t>(src[(D * KB) / 8 + 1]) << 8);
    const float fac = f16_bits_to_float(nb) * p.inv_sqrt_block;
    const uint32_t sbits = lane_sign_bits(p.sign_words, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = flip_sign(y[e] * fac, (sbits >> e) & 1u);
  }
  {
    const uint8_t *vf = src + p.key_bytes;
    uint32_t code[8];
    unpack8<VB>(load_group<VB>(vf, r), code);
    const uint32_t sb = static_cast<uint32_t>(vf[(D * VB) / 8]) | (static_cast<uint32_t>(vf[(D * VB) / 8 + 1]) << 8);
    const uint32_t zb = static_cast<uint32_t>(vf[(D * VB) / 8 + 2]) | (static_cast<uint32_t>(vf[(D * VB) / 8 + 3]) << 8);
    const float s1 = f16_bits_to_float(sb), z1 = f16_bits_to_float(zb);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (s1 * static_cast<float>(code[e])) + z1;
  }
  }  // valid
  if (!active) return;
  float4 *ko = reinterpret_cast<float4 *>(p.k_out + (i * p.num_kv_heads + h) * D + 8 * r);
  float4 *vo = reinterpret_cast<float4 *>(p.v_out + (i * p.num_kv_heads + h) * D + 8 * r);
  ko[0] = make_float4(k[0], k[1], k[2], k[3]);
  ko[1] = make_float4(k[4], k[5], k[6], k[7]);
  vo[0] = make_float4(v[0], v[1], v[2], v[3]);
  vo[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// After a ring flush: every full ring's tokens are now compressed positions,
// so its sequence grows by ring_cap and the ring empties.
__global__ void ring_commit_kernel(int32_t *ring_lens, int32_t *seq_lens, int batch, int ring_cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && ring_lens[b] >= ring_cap) {
    seq_lens[b] = max(seq_lens[b], 0) + ring_cap;
    ring_lens[b] = 0;
  }
}

// One workgroup per sequence: its new token's K and V rows (bf16, 8 elements
// per thread and step) go to ring position ring_lens[b], which then grows by
// one. A full ring is left as it is.
__global__ __launch_bounds__(kThreads) void ring_append_kernel(const uint16_t *k_new, const uint16_t *v_new,
                                                                 uint16_t *ring_k, uint16_t *ring_v,
                                                                 int32_t *ring_lens, int num_kv_heads,
                                                                 int head_dim, int ring_cap) {
  const int b = blockIdx.x;
  const int r = ring_lens[b];
  const bool room = r >= 0 && r < ring_cap;
  if (room) {
    const int vecs = num_kv_heads * head_dim / 8;
    for (int i = threadIdx.x; i < vecs; i += blockDim.x) {
      const int h = (i * 8) / head_dim, j = i * 8 - h * head_dim;
      const int64_t src = (static_cast<int64_t>(b) * num_kv_heads + h) * head_dim + j;
      const int64_t dst = ((static_cast<int64_t>(b) * num_kv_heads + h) * ring_cap + r) * head_dim + j;
      *reinterpret_cast<uint4 *>(ring_k + dst) = *reinterpret_cast<const uint4 *>(k_new + src);
      *reinterpret_cast<uint4 *>(ring_v + dst) = *reinterpret_cast<const uint4 *>(v_new + src);
    }
  }
  __syncthreads();  // every thread has read ring_lens[b]
  if (threadIdx.x == 0 && room) ring_lens[b] = r + 1;
}

template <int D, int KB, int VB>
int launch_quantize_t(tq_dtype dt, const QuantParams &p, hipStream_t s) {
  using T = Team<D>;
  const int64_t per_block = (kThreads / 64) * T::kPerWave;  // tokens per workgroup
  const int64_t blocks = (p.num_tokens + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff || p.num_kv_heads > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(p.num_kv_heads));
  switch (dt) {
    case TQ_F32: hipLaunchKernelGGL((quantize_kernel<D, KB, VB, 0>), grid, dim3(kThreads), 0, s, p); break;
    case TQ_BF16: hipLaunchKernelGGL((quantize_kernel<D, KB, VB, 1>), grid, dim3(kThreads), 0, s, p); break;
    case TQ_F16: hipLaunchKernelGGL((quantize_kernel<D, KB, VB, 2>), grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

template <int D, int KB, int VB>
int launch_dequant_t(const DequantParams &p, hipStream_t s) {
  using T = Team<D>;
  const int64_t nvec = p.n * p.num_kv_heads;
  const int64_t per_block = (kThreads / 64) * T::kPerWave;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dequant_kernel<D, KB, VB>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
int dispatch_quantize_bits(const tq_config &c, tq_dtype dt, const QuantParams &p, hipStream_t s) {
  const int kb = c.key_quant_bits, vb = c.value_quant_bits;
  if (kb == 3 && vb == 2) return launch_quantize_t<D, 3, 2>(dt, p, s);
  if (kb == 4 && vb == 2) return launch_quantize_t<D, 4, 2>(dt, p, s);
  if (kb == 8 && vb == 2) return launch_quantize_t<D, 8, 2>(dt, p, s);
  if (kb == 3 && vb == 3) return launch_quantize_t<D, 3, 3>(dt, p, s);
  if (kb == 3 && vb == 4) return launch_quantize_t<D, 3, 4>(dt, p, s);
  if (kb == 4 && vb == 3) return launch_quantize_t<D, 4, 3>(dt, p, s);
  if (kb == 4 && vb == 4) return launch_quantize_t<D, 4, 4>(dt, p, s);
  if (kb == 8 && vb == 3) return launch_quantize_t<D, 8, 3>(dt, p, s);
  if (kb == 8 && vb == 4) return launch_quantize_t<D, 8, 4>(dt, p, s);
  return hipErrorInvalidValue;
}

template <int D>
int dispatch_dequant_bits(const tq_config &c, const DequantParams &p, hipStream_t s) {
  const int kb = c.key_quant_bits, vb = c.value_quant_bits;
  if (kb == 3 && vb == 2) return launch_dequant_t<D, 3, 2>(p, s);
  if (kb == 4 && vb == 2) return launch_dequant_t<D, 4, 2>(p, s);
  if (kb == 8 && vb == 2) return launch_dequant_t<D, 8, 2>(p, s);
  if (kb == 3 && vb == 3) return launch_dequant_t<D, 3, 3>(p, s);
  if (kb == 3 && vb == 4) return launch_dequant_t<D, 3, 4>(p, s);
  if (kb == 4 && vb == 3) return launch_dequant_t<D, 4, 3>(p, s);
  if (kb == 4 && vb == 4) return launch_dequant_t<D, 4, 4>(p, s);
  if (kb == 8 && vb == 3) return launch_dequant_t<D, 8, 3>(p, s);
  if (kb == 8 && vb == 4) return launch_dequant_t<D, 8, 4>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

int launch_quantize(const tq_config &c, tq_dtype dt, const QuantParams &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (c.head_dim) {
    case 64: return dispatch_quantize_bits<64>(c, dt, p, s);
    case 96: return dispatch_quantize_bits<96>(c, dt, p, s);
    case 128: return dispatch_quantize_bits<128>(c, dt, p, s);
  }
  return hipErrorInvalidValue;
}

int launch_ring_commit(int32_t *ring_lens, int32_t *seq_lens, int batch, int ring_cap, void *stream) {
  hipLaunchKernelGGL(ring_commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     ring_lens, seq_lens, batch, ring_cap);
  return hipGetLastError();
}

int launch_ring_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *ring_k, uint16_t *ring_v,
                       int32_t *ring_lens, int batch, int num_kv_heads, int head_dim, int ring_cap, void *stream) {
  hipLaunchKernelGGL(ring_append_kernel, dim3(batch), dim3(kThreads), 0, static_cast<hipStream_t>(stream), k_new, v_new,
                     ring_k, ring_v, ring_lens, num_kv_heads, head_dim, ring_cap);
  return hipGetLastError();
}

int launch_dequant(const tq_config &c, const DequantParams &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (c.head_dim) {
    case 64: return dispatch_dequant_bits<64>(c, p, s);
    case 96: return dispatch_dequant_bits<96>(c, p, s);
    case 128: return dispatch_dequant_bits<128>(c, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
