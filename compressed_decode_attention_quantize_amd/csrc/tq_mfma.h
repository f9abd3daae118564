// Device helpers shared by the attention kernels over compressed slots: the
// slot geometry of a (head_dim, key bits, value bits) variant, direct
// HBM -> LDS tile loads, LDS field reads, the code -> f16 operand expansion
// of keys (centroid pair table / FP8 conversion) and values (exponent trick),
// lane-mask selects and the MFMA column reductions.
//
// MFMA operand layouts used (gfx950, wave64), checked on hardware:
//  16x16x32 f16 / bf16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16],
//  e<8; result lane l register r = D[4(l/16)+r][l%16].
#pragma once

#include <cstdint>

#include "tq_device.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;

// Compile-time geometry of one (head_dim, key bits, value bits) variant.
template <int D, int KB, int VB>
struct Geo {
  static constexpr bool kMse = KB != 8;
  static constexpr int kKeyCodeBytes = kMse ? D * KB / 8 : D;
  static constexpr int kKeyBytes = kMse ? kKeyCodeBytes + 2 : D;
  static constexpr int kValCodeBytes = D * VB / 8;
  static constexpr int kSlot = kKeyBytes + kValCodeBytes + 4;   // even for D % 32 == 0
  static constexpr int kKM = D / 32;                // score MFMAs per tile
  static constexpr int kLaneKeyBytes = kKeyCodeBytes / 4;       // key bytes per lane
  static constexpr int kGroups = D / 8;             // 8-element value groups
  static constexpr int kTileBytes = kTile * kSlot;
  static constexpr int kTileChunks = kTileBytes / 16;           // 16-byte chunks
  static constexpr int kChunksPerLane = (kTileChunks + 63) / 64;
  static constexpr int kQBytes = 16 * D * 2;        // one f16 plane of rotated queries [16][D]
  // a tile buffer: the tile plus slack for the funnel-shifted reads that run
  // up to 7 bytes past a field, rounded to 16 bytes
  static constexpr int kTileBuf = ((kTileBytes + 16) + 15) / 16 * 16;
  // one wave's LDS: `bufs` tile buffers, or the queries
  static constexpr int stage_bytes(int bufs) { return bufs * kTileBuf > kQBytes ? bufs * kTileBuf : kQBytes; }
  static constexpr int kLut = KB == 4 ? 256 : (KB == 3 ? 64 : 1);
  // every lane's key bytes, and every value code group, start on a word
  static constexpr bool kKeyAligned = kSlot % 4 == 0 && kLaneKeyBytes % 4 == 0;
  static constexpr bool kValAligned = kSlot % 4 == 0 && kKeyBytes % 4 == 0 && VB % 4 == 0;
  static_assert(kSlot % 2 == 0, "slot size must be even");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Byte offset of an LDS object (the value an LDS-address-space pointer holds).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void *)(p)));
}

// Direct HBM -> LDS load of 16 bytes per lane from a wave-uniform base in
// SGPRs: lane l's 16 bytes at sbase + voff (voff a per-lane VGPR offset,
// no per-lane 64-bit address arithmetic) land at LDS offset lds_base + 16 l
// (lds_base wave-uniform). Issued as inline asm so the compiler does not
// hold later LDS reads of other buffers behind it; callers wait for it with
// wait_vmcnt before reading the destination.
__device__ __forceinline__ void load_lds_16s(const void *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(sbase)
      : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N); the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until this wave's LDS reads have returned (s_waitcnt lgkmcnt(0)).
// A direct HBM -> LDS load writes LDS through the memory path, unordered with
// the wave's earlier ds_read instructions; without this wait a load into a
// buffer can land before earlier reads of that buffer have executed.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int N>
struct Words {
  uint32_t w[N];
};

// NB bytes at byte offset `off` (any alignment) of an LDS word array, as
// NB/4 (rounded up) little-endian words: aligned dword reads and a byte
// funnel shift. Offsets, not pointer casts, keep the accesses in the LDS
// address space.
template <int NB, bool kAligned = false>
__device__ __forceinline__ Words<(NB + 3) / 4> lds_bytes(const uint32_t *words, uint32_t off) {
  constexpr int NW = (NB + 3) / 4;
  const uint32_t w0 = off >> 2;
  if constexpr (kAligned) {
    // off is a multiple of 4: whole words, no funnel shift
    Words<NW> out;
#pragma unroll
    for (int i = 0; i < NW; ++i) out.w[i] = words[w0 + i];
    return out;
  }
  const uint32_t sh = off & 3u;
  uint32_t raw[NW + 1];
#pragma unroll
  for (int i = 0; i <= NW; ++i) raw[i] = words[w0 + i];
  Words<NW> out;
#pragma unroll
  for (int i = 0; i < NW; ++i) out.w[i] = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], sh);
  return out;
}

// The NB-byte field (NB <= 4) at byte offset `off` of an LDS word array, in
// the low bytes of a word, from 16-bit reads: NB = 2 and 4 need an even
// offset, NB = 3 takes any (two 16-bit reads from the even byte at or below
// off, then a shift). One register per field, no funnel shift of word
// pairs, so a tile's fields can all be in flight at once.
template <int NB>
__device__ __forceinline__ uint32_t lds_field16(const uint32_t *words, uint32_t off) {
  static_assert(NB >= 2 && NB <= 4, "field bytes");
  const uint16_t *h = reinterpret_cast<const uint16_t *>(words);
  const uint32_t e = off >> 1;
  if constexpr (NB == 2) {
    return h[e];
  } else {
    const uint32_t y = static_cast<uint32_t>(h[e]) | (static_cast<uint32_t>(h[e + 1]) << 16);
    return NB == 4 ? y : (y >> (8u * (off & 1u)));
  }
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 x = __builtin_bit_cast(h2, a), y = __builtin_bit_cast(h2, b);
  return __builtin_bit_cast(uint32_t, x + y);
}

__device__ __forceinline__ uint32_t f16_pair_bits(float lo, float hi) {
  return float_to_f16_bits(lo) | (float_to_f16_bits(hi) << 16);
}

// Exponent-trick expansion of value codes of one element for a pair of
// tokens: `x` holds the two tokens' code bits in its low and high halves,
// `mask` selects the element's field in place (bits <= 9), so
// (x & mask) | 0x6400 is the f16 1024 + code * 2^pos in each half; adding
// -(1024 + 2^pos * c0) leaves 2^pos * (code - c0), exact in f16.
//
// The mask and the exponent constant reach the compiler as register values it
// cannot see into (empty asm with a register constraint), so it selects one
// v_and_or_b32 with register operands: gfx950 VOP3 encodings take no literal,
// and with literals it would split the expression into v_and + v_or.
__device__ __forceinline__ uint32_t sgpr_value(uint32_t v) {
  asm("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t code_pair(uint32_t x, uint32_t mask, uint32_t neg_off) {
  uint32_t magic = 0x64006400u;
  asm("" : "+v"(magic));
  return pk_add_f16((x & mask) | magic, neg_off);
}

// Value codes of element group i (8 elements) for tokens 4kq..4kq+3 as the
// A operands of the eight value MFMAs (element 8i+c in MFMA c), with the
// per-element power-of-two scales the expansion leaves (inv_scale[c]).
// prep() gathers the tokens' code bytes into 16-bit halves (token pairs
// (0, 1) and (2, 3) in the two words of each selection); get(c) expands
// element c from them.
template <int VB>
struct ValueExpand;

template <>
struct ValueExpand<4> {
  static constexpr int kC0 = 8;
  struct Prep {
    uint32_t x[4][2];  // byte k of tokens (0, 1) and (2, 3): elements 2k, 2k + 1
  };
  __device__ static void prep(const uint32_t d[4], Prep &pr) {
    // d[r]: 8 nibbles (elements 8i..8i+7) of token 4kq + r
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t sel = static_cast<uint32_t>(k) | (0x0Cu << 8) | ((4u + k) << 16) | (0x0Cu << 24);
      pr.x[k][0] = perm(d[1], d[0], sel);
      pr.x[k][1] = perm(d[3], d[2], sel);
    }
  }
  __device__ static half4_t get(const Prep &pr, int c) {
    const bool odd = c & 1;
    const float off = -(1024.0f + (odd ? 16.0f : 1.0f) * kC0);
    const uint32_t neg = f16_pair_bits(off, off);
    const uint32_t mask = sgpr_value(odd ? 0x00F000F0u : 0x000F000Fu);
    u32x2_t v;
    v[0] = code_pair(pr.x[c >> 1][0], mask, neg);
    v[1] = code_pair(pr.x[c >> 1][1], mask, neg);
    return __builtin_bit_cast(half4_t, v);
  }
  __device__ static float inv_scale(int c) { return (c & 1) ? (1.0f / 16.0f) : 1.0f; }
};

template <>
struct ValueExpand<3> {
  static constexpr int kC0 = 4;
  // element c sits at bits 3c..3c+2; after the byte selection below its
  // field starts at bit pos(c) of a 16-bit half.
  __device__ static constexpr int pos(int c) {
    return c == 0 ? 0 : c == 1 ? 3 : c == 2 ? 6 : c == 3 ? 1 : c == 4 ? 4 : c == 5 ? 7 : c == 6 ? 2 : 5;
  }
  struct Prep {
    uint32_t x[3][2];  // bits 0..15, 8..23 and 16..23 of tokens (0, 1) and (2, 3)
  };
  __device__ static void prep(const uint32_t d[4], Prep &pr) {
    // d[r]: 24 bits (elements 8i..8i+7) of token 4kq + r
    constexpr uint32_t selX = 0u | (1u << 8) | (4u << 16) | (5u << 24);     // bits 0..15
    constexpr uint32_t selY = 1u | (2u << 8) | (5u << 16) | (6u << 24);     // bits 8..23
    constexpr uint32_t selZ = 2u | (0x0Cu << 8) | (6u << 16) | (0x0Cu << 24);  // bits 16..23
    pr.x[0][0] = perm(d[1], d[0], selX);
    pr.x[0][1] = perm(d[3], d[2], selX);
    pr.x[1][0] = perm(d[1], d[0], selY);
    pr.x[1][1] = perm(d[3], d[2], selY);
    pr.x[2][0] = perm(d[1], d[0], selZ);
    pr.x[2][1] = perm(d[3], d[2], selZ);
  }
  __device__ static half4_t get(const Prep &pr, int c) {
    const int src = c < 3 ? 0 : (c < 6 ? 1 : 2);
    const uint32_t m16 = 7u << pos(c);
    const uint32_t mask = sgpr_value(m16 | (m16 << 16));
    const float off = -(1024.0f + static_cast<float>(1 << pos(c)) * kC0);
    const uint32_t neg = f16_pair_bits(off, off);
    u32x2_t v;
    v[0] = code_pair(pr.x[src][0], mask, neg);
    v[1] = code_pair(pr.x[src][1], mask, neg);
    return __builtin_bit_cast(half4_t, v);
  }
  __device__ static float inv_scale(int c) { return 1.0f / static_cast<float>(1 << pos(c)); }
};

template <>
struct ValueExpand<2> {
  static constexpr int kC0 = 2;
  // element c sits at bits 2c..2c+1; byte c / 4 holds it, at bit 2 (c % 4)
  __device__ static constexpr int pos(int c) { return 2 * (c & 3); }
  struct Prep {
    uint32_t x[2][2];  // byte k of tokens (0, 1) and (2, 3): elements 4k..4k+3
  };
  __device__ static void prep(const uint32_t d[4], Prep &pr) {
    // d[r]: 16 bits (elements 8i..8i+7) of token 4kq + r
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t sel = static_cast<uint32_t>(k) | (0x0Cu << 8) | ((4u + k) << 16) | (0x0Cu << 24);
      pr.x[k][0] = perm(d[1], d[0], sel);
      pr.x[k][1] = perm(d[3], d[2], sel);
    }
  }
  __device__ static half4_t get(const Prep &pr, int c) {
    const uint32_t m16 = 3u << pos(c);
    const uint32_t mask = sgpr_value(m16 | (m16 << 16));
    const float off = -(1024.0f + static_cast<float>(1 << pos(c)) * kC0);
    const uint32_t neg = f16_pair_bits(off, off);
    u32x2_t v;
    v[0] = code_pair(pr.x[c >> 2][0], mask, neg);
    v[1] = code_pair(pr.x[c >> 2][1], mask, neg);
    return __builtin_bit_cast(half4_t, v);
  }
  __device__ static float inv_scale(int c) { return 1.0f / static_cast<float>(1 << pos(c)); }
};

// Key operand of one lane: token t = lane % 16, elements kq*D/4 .. +D/4-1 as
// f16 centroid values (MSE, via the pair table) or FP8-decoded values.
template <int D, int KB, int VB>
__device__ __forceinline__ void key_operand(const uint32_t *words, uint32_t off, const uint32_t *lut,
                                            half8_t kf[D / 32]) {
  using G = Geo<D, KB, VB>;
  constexpr int LB = G::kLaneKeyBytes;
  const auto kw = lds_bytes<LB, G::kKeyAligned>(words, off);
  if constexpr (KB == 4) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const uint32_t w = kw.w[m];
      u32x4_t v;
      v[0] = lut[w & 0xffu];
      v[1] = lut[(w >> 8) & 0xffu];
      v[2] = lut[(w >> 16) & 0xffu];
      v[3] = lut[w >> 24];
      kf[m] = __builtin_bit_cast(half8_t, v);
    }
  } else if constexpr (KB == 3) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      // 24 bits of elements 8m..8m+7 start at bit 24m of the lane's bytes
      const int bit = 24 * m;
      const int wi = bit >> 5, sh = bit & 31;
      uint32_t g = kw.w[wi] >> sh;
      if (sh > 8) g |= kw.w[wi + 1] << (32 - sh);
      u32x4_t v;
      v[0] = lut[g & 63u];
      v[1] = lut[(g >> 6) & 63u];
      v[2] = lut[(g >> 12) & 63u];
      v[3] = lut[(g >> 18) & 63u];
      kf[m] = __builtin_bit_cast(half8_t, v);
    }
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const uint32_t a = kw.w[2 * m], b = kw.w[2 * m + 1];
      u32x4_t v;
      v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false));
      v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true));
      v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false));
      v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true));
      kf[m] = __builtin_bit_cast(half8_t, v);
    }
  }
}

// Lane l takes a if bit l of the lane mask m is set, else b (one
// v_cndmask_b32 with the mask bit as the lane's condition; the arms are
// values already in registers, so the compiler has no reason to branch).
// Masks of loop-invariant conditions are computed once, outside the loops.
__device__ __forceinline__ bool mask_bit(uint64_t m) {
  return (m >> __lane_id()) & 1ull;
}
__device__ __forceinline__ float mask_select(uint64_t m, float a, float b) { return mask_bit(m) ? a : b; }
__device__ __forceinline__ uint32_t mask_select(uint64_t m, uint32_t a, uint32_t b) { return mask_bit(m) ? a : b; }
__device__ __forceinline__ uint64_t lane_mask(bool c) { return __builtin_amdgcn_ballot_w64(c); }
// Lanes whose column (lane % 16) is below n, for 0 <= n <= 16.
__device__ __forceinline__ uint64_t column_mask(int n) {
  return ((1ull << n) - 1ull) * 0x0001000100010001ull;
}

// Hand-off of LDS data between lanes of one wave: lanes write, other lanes
// of the same wave read. The hardware keeps one wave's LDS operations in
// order; the fence tells the compiler that other lanes' stores are visible
// here, so it neither forwards a lane's own earlier values to the reads nor
// moves memory accesses across this point.
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Reductions over the 4 lane rows of an MFMA column (lanes c, c + 16,
// c + 32, c + 48) with the gfx950 row-swap permutes: swapping a register
// with itself gives both halves of each row pair.
__device__ __forceinline__ float column_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float column_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Value of the lane N columns away in the lane's 16-lane row (DPP row_ror:N:
// lane c reads lane (c - N) mod 16 of its row; for N = 8 that is the partner
// half of the row either way).
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  static_assert(N > 0 && N < 16, "row rotation");
  // every lane has a source lane, so no old value is needed
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x120 + N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __uint_as_float(row_ror<N>(__float_as_uint(v)));
}

// 16-bit field at an even byte offset of an LDS word array.
__device__ __forceinline__ uint32_t lds_u16(const uint32_t *words, uint32_t off) {
  const uint32_t w = words[off >> 2];
  return (off & 2u) ? (w >> 16) : (w & 0xffffu);
}


// Slack of the online softmax's lazy reference maximum (log2 units): the
// running reference moves only when a column's maximum passes it by more
// than this, so weights stay below 2^kLazy and rescales are rare.
constexpr float kLazy = 4.0f;

// Plain v_max / v_min: the compiler puts a canonicalising max around
// operands it cannot prove canonical (cross-lane moves, LDS reads); the
// values here are finite or -inf. column_max_raw: maximum over the 4 lane
// rows of an MFMA column (lanes c, c + 16, c + 32, c + 48) by the gfx950
// row-swap permutes.
__device__ __forceinline__ float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float fmin_raw(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float column_max_raw(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_raw(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// f16 hi + lo parts of the products w0 = p0 s0, w1 = p1 s1 as packed pairs:
// hi = RNE(p s), lo = RNE(fma(p, s, -hi)), so |w - hi - lo| <= 2^-22 |w|.
// Mixed-precision multiply-adds form both halves from the f32 factors (the
// product is never rounded to f32), reading hi's f16 halves in place; the
// inputs are ordinary VALU results.
__device__ __forceinline__ void split_prod_f16(float p0, float s0, float p1, float s1, uint32_t &hi, uint32_t &lo) {
  asm("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
      "v_fma_mixhi_f16 %0, %4, %5, 0\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(hi), "=&v"(lo)
      : "v"(p0), "v"(s0), "v"(p1), "v"(s1));
}
}  // namespace
}  // namespace tq
