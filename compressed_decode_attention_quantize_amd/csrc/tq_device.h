// Device helpers shared by the kernel translation units (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

namespace tq {

// ---------------------------------------------------------------------------
// scalar formats

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  return static_cast<float>(__ushort_as_half(static_cast<unsigned short>(b)));
}

// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default
// rounding mode).
__device__ __forceinline__ uint32_t float_to_f16_bits(float x) {
  return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(x)));
}

// fp32 -> OCP E4M3FN byte: round to nearest even, |x| saturated to 448, the
// sign of zero kept, NaN -> 0x7f with its sign.
__device__ __forceinline__ uint32_t float_to_e4m3fn(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if ((bits & 0x7fffffffu) > 0x7f800000u) return sign | 0x7fu;
  const float a = fminf(__uint_as_float(bits & 0x7fffffffu), 448.0f);
  const uint32_t ab = __float_as_uint(a);
  const int e = static_cast<int>(ab >> 23) - 127;
  if (e < -6) {
    // below the smallest normal: multiples of 2^-9, rounded to nearest even
    return sign | static_cast<uint32_t>(rintf(a * 512.0f));
  }
  const uint32_t mant = ab & 0x7fffffu;
  const uint32_t keep = mant >> 20;
  const uint32_t rest = mant & 0xfffffu;
  uint32_t q = (static_cast<uint32_t>(e + 7) << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) q += 1;
  return sign | q;
}

// E4M3FN byte -> fp32 (exact).
__device__ __forceinline__ float e4m3fn_to_float(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 7u;
  float mag;
  if (e == 0) {
    mag = static_cast<float>(m) * (1.0f / 512.0f);
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  if ((c & 0x7fu) == 0x7fu) mag = __uint_as_float(0x7fc00000u);
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// element loads as fp32

__device__ __forceinline__ float load_as_float(const void *base, int dtype, int64_t i) {
  if (dtype == 0) return static_cast<const float *>(base)[i];
  const uint32_t b = static_cast<const uint16_t *>(base)[i];
  return dtype == 1 ? bf16_bits_to_float(b) : f16_bits_to_float(b);
}

// ---------------------------------------------------------------------------
// cross-lane (wave64)

// v of lane (this lane xor mask). The masks a team uses (1, 2, 4, 8: inside a
// 16-lane row) are DPP moves, lane c reading lane f(c) of its row: quad_perm
// [1,0,3,2] and [2,3,0,1] for 1 and 2, row_half_mirror (c xor 7) then
// quad_perm [3,2,1,0] (xor 3) for 4, row_ror:8 for 8. Other masks go through
// the LDS permute unit.
template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor(float v, int mask) {
  switch (mask) {
    case 1: return dpp_mov<0xB1>(v);
    case 2: return dpp_mov<0x4E>(v);
    case 4: return dpp_mov<0x1B>(dpp_mov<0x141>(v));
    case 8: return dpp_mov<0x128>(v);
    default: return __shfl_xor(v, mask, 64);
  }
}
__device__ __forceinline__ float lane_read(float v, int src) { return __shfl(v, src, 64); }

// ---------------------------------------------------------------------------
// Vector "teams": one (token, head) vector of D elements is held by D/8
// consecutive lanes, 8 consecutive elements per lane (lane r of a team holds
// elements 8r..8r+7). A Walsh-Hadamard block of B elements spans B/8 lanes.

template <int D>
struct Team {
  static constexpr int kLanes = D / 8;                 // lanes per vector
  static constexpr int kPerWave = 64 / kLanes;         // vectors per wave
  static constexpr int kBlock = D & (-D);              // Hadamard block length
  static constexpr int kBlockLanes = kBlock / 8;       // lanes per block
  static constexpr int kBlocks = D / kBlock;           // 1 or 3
};

// Sum of squares of a team's vector in the fixed order: adjacent-pair tree
// inside each lane, then an xor butterfly across the block's lanes (the same
// pairing tree), then block totals added left to right. Every lane of the
// team receives the total.
template <int D>
__device__ __forceinline__ float team_sumsq(const float x[8], int team_base) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[i] * x[i];
  float s = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
#pragma unroll
  for (int m = 1; m < Team<D>::kBlockLanes; m <<= 1) s = s + lane_xor(s, m);
  if constexpr (Team<D>::kBlocks > 1) {
    float acc = lane_read(s, team_base);
#pragma unroll
    for (int blk = 1; blk < Team<D>::kBlocks; ++blk) acc = acc + lane_read(s, team_base + blk * Team<D>::kBlockLanes);
    s = acc;
  }
  return s;
}

// Unnormalised Sylvester Walsh-Hadamard transform of each block, strides
// ascending: stride 1, 2, 4 inside the lane, then lane xor 1, 2, ... ; the
// lower element of a pair becomes a + b, the upper one a - b.
template <int D>
__device__ __forceinline__ void team_wht(float z[8], int lane_in_block) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = z[i], b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < Team<D>::kBlockLanes; m <<= 1) {
    const bool upper = (lane_in_block & m) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = lane_xor(z[i], m);
      z[i] = upper ? (p - z[i]) : (z[i] + p);
    }
  }
}

template <int D>
__device__ __forceinline__ float team_min(float v, int team_base) {
#pragma unroll
  for (int m = 1; m < Team<D>::kBlockLanes; m <<= 1) v = fminf(v, lane_xor(v, m));
  if constexpr (Team<D>::kBlocks > 1) {
    float acc = lane_read(v, team_base);
#pragma unroll
    for (int blk = 1; blk < Team<D>::kBlocks; ++blk) acc = fminf(acc, lane_read(v, team_base + blk * Team<D>::kBlockLanes));
    v = acc;
  }
  return v;
}

template <int D>
__device__ __forceinline__ float team_max(float v, int team_base) {
#pragma unroll
  for (int m = 1; m < Team<D>::kBlockLanes; m <<= 1) v = fmaxf(v, lane_xor(v, m));
  if constexpr (Team<D>::kBlocks > 1) {
    float acc = lane_read(v, team_base);
#pragma unroll
    for (int blk = 1; blk < Team<D>::kBlocks; ++blk) acc = fmaxf(acc, lane_read(v, team_base + blk * Team<D>::kBlockLanes));
    v = acc;
  }
  return v;
}

// The 8 sign bits of lane r (elements 8r..8r+7) from the 4-word layer mask.
__device__ __forceinline__ uint32_t lane_sign_bits(const uint32_t w[4], int r) {
  const uint32_t word = r < 4 ? w[0] : r < 8 ? w[1] : r < 12 ? w[2] : w[3];
  return (word >> (8 * (r & 3))) & 0xffu;
}

__device__ __forceinline__ float flip_sign(float x, uint32_t bit) {
  return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

}  // namespace tq
