// Fused decode attention over compressed slots.
//
// Source: hnwysp.cn article on the stand-alone turboquant project,
// next-directions section, direction 1 (one pass over the compressed data,
// flash-attention style online softmax block by block, the query rotated
// forward so D-dim keys are never rotated back, no materialised FP16 KV);
// its write-path section (128-token bf16 exact ring buffer) for the ring
// chunk; vLLM API page TurboQuantConfig docstring for norm correction.
//
// Three kernels on one stream:
//
//  split kernel  (compressed tokens; one wave per (sequence, KV head, split),
//                four waves per workgroup sharing a code->f16 pair table)
//     per 16-token tile, staged HBM -> LDS with 16-byte loads one tile ahead:
//       K~ = centroid values (MSE: pair-table lookup, FP8: hardware cvt), f16
//       S^T[t][g] = K~ . (Pi q)^T           MFMA 16x16x32 f16, D/32 of them
//       |c_t|^2   = diag(K~ K~^T)            (norm correction only)
//       s = S^T * n16_t * scale*log2(e) (/|c_t|), online softmax in exp2,
//       the running max only ever grows, acc is rescaled when it does
//       Out^T[j][g] += (code_tj - c0)^T . (p_t s'_t)   MFMA 16x16x32 f16
//                      over tile pairs (K = 2 x 16 tokens),
//                      codes expanded by the 0x6400 exponent trick in place,
//                      the weights p_t s'_t as f16 hi + lo parts
//       zero terms  += p_t (z'_t + c0 s'_t)   fp32
//     writes an unnormalised partial (m, l, acc[D]) per (sequence, q head).
//  ring kernel   (exact bf16 ring tokens, fp32 VALU; one workgroup per
//                (sequence, KV head)), same partial format.
//  reduce kernel (log-sum-exp merge of a (sequence, q head)'s partials).
//
// MFMA operand layouts used (gfx950, wave64), checked on hardware:
//  16x16x32 f16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], e<8;
//  result lane l register r = D[4(l/16)+r][l%16].

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_mfma.h"

namespace tq {
namespace {

constexpr int kWaves = 4;               // waves (= splits) per workgroup
constexpr int kPartStride_pad = 4;      // partial = [m, l, -, -, acc[D]]

__device__ __forceinline__ int partial_stride(int d) { return d + kPartStride_pad; }

// Active waves of the decode: all W launched waves, but no wave with fewer
// than min_tiles tiles (min_tokens / 16; 256 tokens when the caller passes 0).
constexpr int kDefaultMinTokens = 256;
__host__ __device__ __forceinline__ int work_waves(long long total_tiles, int launched, int min_tokens) {
  const long long min_tiles = (min_tokens > 0 ? min_tokens : kDefaultMinTokens) / kTile;
  long long w = total_tiles / min_tiles;
  if (w < 1) w = 1;
  return static_cast<int>(w < launched ? w : launched);
}

// The wave whose range [w T / W, (w+1) T / W) holds flattened tile f.
__host__ __device__ __forceinline__ int first_wave(long long f, long long total, int active) {
  return static_cast<int>(((f + 1) * active - 1) / total);
}


// NB = column groups: the 16 MFMA columns hold NB tile slots of GP = 16 / NB
// query heads each (NB = 4 for G <= 4, 2 for G <= 8, 1 else). A macro tile is
// NT = NB * TL tiles: with one column group (G > 8) every lane holds the
// scores of TL = 2 tiles, so that the value contraction still takes two
// tiles per 16x16x32 MFMA.
//
// With NB > 1 the f16 hi and lo parts of an operand share one MFMA: group j
// and its partner j +- NB/2 (the lanes 8 columns away, same row) carry the
// two parts of the same query heads, and one DPP row rotation adds them.
//  scores: tile i (kept by group i) multiplies the plane with the hi parts
//          in group i and the lo parts in its partner;
//  values: the weights of tile i go to group i as hi parts and to the
//          partner group as lo parts, so every group accumulates a mix of
//          tiles. All groups of a query head therefore share one running
//          maximum, and the final merge of the groups is a plain sum.
template <int D, int KB, int VB, int NB, bool NC>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3))) void decode_split_kernel(DecodeParams p, int q_dtype) {
  using GE = Geo<D, KB, VB>;
  using VX = ValueExpand<VB>;
  constexpr int S = GE::kSlot;
  constexpr int KM = GE::kKM;
  constexpr int GP = 16 / NB;
  constexpr int TL = NB == 1 ? 2 : 1;  // tiles whose scores one lane holds
  constexpr int NT = NB * TL;          // tiles per macro tile
  constexpr bool kFold = NB > 1;       // hi and lo parts in partner column groups
  // Tile buffers per wave. MSE keys keep all NT tiles of a macro tile in LDS
  // until the value phase re-reads their codes there (NT + 1 buffers: the
  // next tile loads into the spare one); FP8 keys use two buffers, the value
  // code words held in registers across the softmax.
  constexpr bool kValLds = GE::kMse;
  constexpr int kBufs = kValLds ? NT + 1 : 2;

  __shared__ uint32_t lut[GE::kLut];
  __shared__ __align__(16) uint32_t stage[kWaves][GE::stage_bytes(kBufs) / 4];
  // per-token scalars of the macro tile: norm * scale (< 0: masked), s', z' + c0 s', ||c||^2;
  // plane 4 takes the writes of lanes that hold nothing for a plane
  __shared__ __align__(16) float tokf[kWaves][5][NT][16];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int kq = lane >> 4;

  if constexpr (GE::kMse) {
    for (int e = threadIdx.x; e < GE::kLut; e += 64 * kWaves) {
      const int lo = e & ((1 << KB) - 1), hi = e >> KB;
      lut[e] = f16_pair_bits(p.centroids[lo] * p.centroid_scale, p.centroids[hi] * p.centroid_scale);
    }
  }
  // ---- work division, computed by every workgroup from the device-side
  // lengths. The (sequence, KV head, 16-token tile) triples are flattened in
  // that order; wave w of the W active waves takes the contiguous range
  // [w T / W, (w+1) T / W) of the T tiles (at least min_tiles each), so every
  // wave streams the same number of tiles whatever the length mix. A wave
  // writes one partial per (sequence, KV head) segment it covers, at row
  // w + s of the partials (s = b Hkv + h): the waves' ranges follow each
  // other, so a wave's segments and the next wave's start at or after its
  // last one, and the rows are distinct.
  extern __shared__ int32_t seq_prefix[];  // [batch + 1]: tiles of sequences < b
  __shared__ int32_t scan_s[64 * kWaves];
  const int tid = threadIdx.x;
  const int B = p.batch;
  const int Hkv = p.num_kv_heads;
  const int seq_cap = min(p.max_seq_len, p.max_blocks_per_seq * p.block_size);
  const int per = (B + 64 * kWaves - 1) / (64 * kWaves);
  const int b_lo = min(B, tid * per), b_hi = min(B, b_lo + per);
  int local = 0;
  for (int bb = b_lo; bb < b_hi; ++bb) local += (min(max(p.seq_lens[bb], 0), seq_cap) + kTile - 1) / kTile;
  scan_s[tid] = local;
  __syncthreads();  // also publishes the code-pair table
  for (int off = 1; off < 64 * kWaves; off <<= 1) {
    const int v = tid >= off ? scan_s[tid - off] : 0;
    __syncthreads();
    scan_s[tid] += v;
    __syncthreads();
  }
  {
    int run = scan_s[tid] - local;
    for (int bb = b_lo; bb < b_hi; ++bb) {
      seq_prefix[bb] = run;
      run += (min(max(p.seq_lens[bb], 0), seq_cap) + kTile - 1) / kTile;
    }
    if (tid == 64 * kWaves - 1) seq_prefix[B] = scan_s[tid];
  }
  __syncthreads();  // the last workgroup barrier; waves are independent below
  const long long total = static_cast<long long>(seq_prefix[B]) * Hkv;  // T
  const int active = work_waves(total, gridDim.x * kWaves, p.split_tokens);
  if (blockIdx.x == 0) {
    // header for the reduce kernel: T, W and the per-sequence tile prefix
    for (int bb = tid; bb <= B; bb += 64 * kWaves) p.plan[4 + bb] = seq_prefix[bb];
    if (tid == 0) {
      reinterpret_cast<long long *>(p.plan)[0] = total;
      p.plan[2] = active;
    }
  }
  const int G = p.num_q_heads / Hkv;
  const int pstride = partial_stride(D);
  // the wave index is uniform across the wave: say so, so that the range
  // bookkeeping, block-table reads and tile addresses stay in scalar registers
  const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(wave);
  if (w >= active) return;
  long long f = static_cast<long long>(w) * total / active;
  const long long f_end = static_cast<long long>(w + 1) * total / active;
  while (f < f_end) {
  int lo = 0, hi = B - 1;  // largest b with seq_prefix[b] * Hkv <= f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<long long>(__builtin_amdgcn_readfirstlane(seq_prefix[mid])) * Hkv <= f) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int pb = __builtin_amdgcn_readfirstlane(seq_prefix[b]);
  const int nb = __builtin_amdgcn_readfirstlane(seq_prefix[b + 1]) - pb;  // tiles of the sequence
  const long long seg0 = static_cast<long long>(pb) * Hkv;
  const int h = static_cast<int>((f - seg0) / nb);
  const long long seg_start = seg0 + static_cast<long long>(h) * nb;   // first tile of (b, h)
  const long long seg_stop = seg_start + nb;
  const long long run_end = seg_stop < f_end ? seg_stop : f_end;
  const int begin = static_cast<int>(f - seg_start) * kTile;
  // The range's first loads go out together: its length, the block ids of
  // its first 64 blocks (lane i: logical block blk_base + i) and, below, the
  // query rows.
  const int len_raw = p.seq_lens[b];
  const int32_t *bt_row = p.block_tables + static_cast<int64_t>(b) * p.max_blocks_per_seq;
  // the next tile to load: logical block and first token in it, advanced by
  // one tile per load (tiles of a range are loaded in order)
  int nx_blk = begin / p.block_size;
  int nx_off = begin - nx_blk * p.block_size;
  int blk_base = nx_blk;
  int blk_lane = blk_base + lane < p.max_blocks_per_seq ? bt_row[blk_base + lane] : 0;
  // this wave's partial row of segment (b, h): row w + s, s = b Hkv + h
  float *part_base = p.partials + (static_cast<int64_t>(w) + static_cast<int64_t>(b) * Hkv + h) * G * pstride;

  uint32_t *scr = stage[wave];  // this wave's LDS: queries, then the staged tile

  // ---- rotated queries as f16 hi + lo parts, in the MFMA B-operand layout.
  // Column n of the score MFMA is query head n % GP of tile slot n / GP:
  // every tile slot sees the same GP query heads (heads >= G are zero).
  half8_t qf[KM], ql[KM];
  {
    using T = Team<D>;
    const int team = lane / T::kLanes;
    const int r = lane - team * T::kLanes;
    constexpr int rows_per_pass = T::kPerWave;
    constexpr int kPasses = (GP + rows_per_pass - 1) / rows_per_pass;
    u32x4_t qhi[kPasses], qlo[kPasses];
    // raw query rows first (16 or 32 bytes per lane; lanes without a live
    // head read head 0 and discard it), so all loads are in flight at once
    u32x4_t qraw[kPasses][2];
#pragma unroll
    for (int k = 0; k < kPasses; ++k) {
      const int g = k * rows_per_pass + team;
      const bool live = team < rows_per_pass && g < G;
      const int64_t e0 = (static_cast<int64_t>(b) * p.num_q_heads + h * G + (live ? g : 0)) * D + 8 * r;
      if (q_dtype == TQ_F32) {
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(p.q) + e0);
        qraw[k][0] = src[0];
        qraw[k][1] = src[1];
      } else {
        qraw[k][0] = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p.q) + e0);
        qraw[k][1] = qraw[k][0];
      }
    }
#pragma unroll
    for (int k = 0; k < kPasses; ++k) {
      const int g = k * rows_per_pass + team;
      float x[8];
      const bool live = team < rows_per_pass && g < G;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = qraw[k][0][e];
        if (q_dtype == TQ_F32) {
          x[e] = __uint_as_float(w0);
          x[4 + e] = __uint_as_float(qraw[k][1][e]);
        } else if (q_dtype == TQ_BF16) {
          x[2 * e] = bf16_bits_to_float(w0 & 0xffffu);
          x[2 * e + 1] = bf16_bits_to_float(w0 >> 16);
        } else {
          x[2 * e] = f16_bits_to_float(w0 & 0xffffu);
          x[2 * e + 1] = f16_bits_to_float(w0 >> 16);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = live ? x[e] : 0.0f;
      if constexpr (GE::kMse) {
        const uint32_t sb = lane_sign_bits(p.sign_words, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = flip_sign(x[e], (sb >> e) & 1u);
        team_wht<D>(x, r % T::kBlockLanes);
        const float rb = rsqrtf(static_cast<float>(T::kBlock));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rb;
      }
      u32x4_t hv, lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[e] = f16_pair_bits(x[2 * e], x[2 * e + 1]);
        const float h0 = f16_bits_to_float(hv[e] & 0xffffu), h1 = f16_bits_to_float(hv[e] >> 16);
        lv[e] = f16_pair_bits(x[2 * e] - h0, x[2 * e + 1] - h1);
      }
      qhi[k] = hv;
      qlo[k] = lv;
    }
    // hi parts through LDS into the MFMA operand layout, then the lo parts.
    // With partner groups (kFold) the first plane (qf) has the hi parts in
    // groups < NB/2 and the lo parts in the others, the second (ql) the
    // opposite.
    _Float16 *qs = reinterpret_cast<_Float16 *>(scr);
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
      wave_lds_sync();  // earlier reads of this plane (other lanes) are done
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int g = k * rows_per_pass + team;
        if (team < rows_per_pass && g < GP) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const bool hi_part = kFold ? ((phase == 0) == (j < NB / 2)) : (phase == 0);
            *reinterpret_cast<u32x4_t *>(qs + (j * GP + g) * D + 8 * r) = hi_part ? qhi[k] : qlo[k];
          }
        }
      }
      wave_lds_sync();  // the rows other lanes wrote are visible
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const half8_t v = *reinterpret_cast<const half8_t *>(qs + col * D + kq * (D / 4) + 8 * m);
        if (phase == 0) qf[m] = v;
        else ql[m] = v;
      }
    }
  }

  const int len = min(max(len_raw, 0), seq_cap);
  const int end = min(len, static_cast<int>(run_end - seg_start) * kTile);
  f = run_end;

  // ---- macro-tile loop: NT tiles of 16 tokens, tile i in column group i % NB
  float4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_lane = 0.0f, z_lane = 0.0f;
  const int my_tile = col / GP;  // column group of this lane's column
  // lane masks of loop-invariant conditions
  uint64_t m_grp[NB];  // lanes of column group j
#pragma unroll
  for (int j = 0; j < NB; ++j) m_grp[j] = lane_mask(my_tile == j);
  const uint64_t m_kq0 = lane_mask(kq == 0), m_kq1 = lane_mask(kq == 1);
  // the Gram diagonal of token col sits in register col - 4 kq of lane row
  // kq: one-hot weights pick it with exact multiply-adds (the Gram entries
  // are finite). Ordinary arithmetic on purpose: an inline-asm select that
  // reads an MFMA result is invisible to the compiler's MFMA hazard checks
  // and could read the registers before the MFMA has written them.
  const int diag_r = col - 4 * kq;
  const float dsel0 = diag_r == 0 ? 1.0f : 0.0f, dsel1 = diag_r == 1 ? 1.0f : 0.0f;
  const float dsel2 = diag_r == 2 ? 1.0f : 0.0f, dsel3 = diag_r == 3 ? 1.0f : 0.0f;
  // LDS planes this lane writes per token: its lane-row scalar, and under
  // norm correction the score factor if it holds the token's Gram diagonal
  constexpr bool kNcPlanes = GE::kMse && NC;
  const int plane_v = ((kNcPlanes && kq == 0) || kq == 3) ? 4 : kq;
  const int plane_g = static_cast<uint32_t>(diag_r) < 4u ? 0 : 4;

  // Tiles go HBM -> LDS by direct loads (global_load_lds_dwordx4: lane l of
  // a load instruction fills bytes [16 l, 16 l + 16) of a 1 KiB LDS window),
  // double buffered: the next tile is in flight while this one is used.
  constexpr int kLoads = GE::kChunksPerLane;     // load instructions per tile
  // Block ids of the range, 64 at a time (blk_base, blk_lane above); tiles
  // pick theirs with readlane.
  bool ok_next = false;
  // bytes of one pool block (all heads; the host keeps it below 2^31) and
  // this head's run inside a block
  const uint32_t blk_stride = static_cast<uint32_t>(p.num_kv_heads * p.block_size * S);
  const uint8_t *head_base = p.pool + static_cast<int64_t>(h) * p.block_size * S;
  const uint32_t nblk = static_cast<uint32_t>(p.num_blocks < 0x7fffffff ? p.num_blocks : 0x7fffffff);
  // this wave's staging area in LDS (wave-uniform)
  const uint32_t stage_base = lds_offset(stage[0]) + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) *
                                                         (GE::stage_bytes(kBufs) / 4 * 4);
  // refill the window of block ids so that it covers the next `ahead`
  // logical blocks from nx_blk
  auto cover = [&](int ahead) __attribute__((always_inline)) {
    if (nx_blk - blk_base + ahead > 64) {
      blk_base = nx_blk;
      blk_lane = blk_base + lane < p.max_blocks_per_seq ? bt_row[blk_base + lane] : 0;
      // the wait for this load stays on this (rare) path: after the branch
      // the compiler would otherwise wait for every load in flight
      wait_vmcnt<0>();
    }
  };
  // kCovered: the window is known to hold the block (full macro tiles check
  // once for all their tiles)
  auto issue = [&](int bsel, auto covered) __attribute__((always_inline)) {
    constexpr bool kCovered = decltype(covered)::value;
    if constexpr (!kCovered) cover(1);
    const int phys = __builtin_amdgcn_readlane(blk_lane, nx_blk - blk_base);
    ok_next = static_cast<uint32_t>(phys) < nblk;
    // an invalid block reads the pool's first block instead (its tokens are masked)
    const uint8_t *src = head_base + static_cast<uint64_t>(ok_next ? static_cast<uint32_t>(phys) : 0u) * blk_stride +
                         static_cast<uint32_t>(nx_off * S);
    nx_off += kTile;
    if (nx_off == p.block_size) {
      nx_off = 0;
      ++nx_blk;
    }
    const uint32_t dst = stage_base + bsel * GE::kTileBuf;
    wait_lds_reads();  // earlier reads of this buffer (or the query plane) have executed
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = lane + 64 * k;
      if (c < GE::kTileChunks) load_lds_16s(src, static_cast<uint32_t>(16 * c), dst + 1024 * k);
    }
  };
  issue(0, std::false_type{});  // waits for the query plane reads before overwriting it

  const float c0 = static_cast<float>(VX::kC0);
  const float inv_sigma = 1.0f / p.centroid_scale;
  constexpr bool nc = GE::kMse && NC;  // norm correction (compile-time: its MFMAs join the tile's schedule)
  int bsel = 0;
  // LDS byte offset of element group col's value codes in token 4kq's slot
  const uint32_t val_off = static_cast<uint32_t>(4 * kq * S + GE::kKeyBytes + VB * col);
  const uint32_t val_off_rd = static_cast<uint32_t>(4 * kq * S + GE::kKeyBytes + VB * min(col, GE::kGroups - 1));
  // One macro tile. kFull: all NT tiles are inside the range and a tile
  // follows them, so no tile needs a bounds check and every tile issues the
  // next load; one branch-free basic block the compiler can schedule as a
  // whole. The range's last macro tile takes the checked form.
  auto macro_tile = [&](const int mt0, auto full) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full)::value;
    if constexpr (kFull) cover(NT);
    uint32_t vraw[kValLds ? 1 : NT][4];
    int tbuf[NT];  // buffer of tile i (wave-uniform)
    float4_t sraw[TL];
#pragma unroll
    for (int u = 0; u < TL; ++u) sraw[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // ---- phase A, per tile: scores into the tile's column group, value
    // code words kept in registers, per-token scalars to LDS
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int tile0 = mt0 + i * kTile;
      if (kFull || tile0 < end) {
        const int ntok = kFull ? kTile : min(kTile, end - tile0);
        const bool tile_ok = ok_next;
        const int nsel = bsel + 1 == kBufs ? 0 : bsel + 1;
        if (kFull || tile0 + kTile < end) {
          issue(nsel, std::integral_constant<bool, kFull>{});
          wait_vmcnt<kLoads>();  // this tile's loads are done, the next tile's may run
        } else {
          wait_vmcnt<0>();
        }
        const uint32_t *tw = scr + bsel * (GE::kTileBuf / 4);  // this tile's bytes as words
        tbuf[i] = bsel;
        bsel = nsel;

        // this tile's LDS reads go out together: the per-token scalar window
        // (the norm for lane row 0, the scale and the zero after it for the
        // others; the same instructions in every lane) and the key bytes
        constexpr uint32_t kScaleOff = GE::kKeyBytes + GE::kValCodeBytes;
        uint32_t x;
        {
          // two 16-bit reads into the halves of one register (the fields
          // are at even offsets of even-sized slots)
          const uint16_t *h = reinterpret_cast<const uint16_t *>(tw);
          const uint32_t off = static_cast<uint32_t>(col * S) + (kq == 0 ? GE::kKeyCodeBytes : kScaleOff);
          x = static_cast<uint32_t>(h[off >> 1]) | (static_cast<uint32_t>(h[(off >> 1) + 1]) << 16);
        }
        half8_t kf[KM];
        key_operand<D, KB, VB>(tw, static_cast<uint32_t>(col * S + kq * GE::kLaneKeyBytes), lut, kf);

        // per-token scalars of token col, plane kq: the score factor (-inf:
        // masked), s', z' + c0 s'. The factor is norm * scale / sigma (the
        // centroids carry the table scale sigma), the constant scale for FP8
        // keys; under norm correction the lane holding the token's Gram
        // diagonal writes it below instead (plane 4 takes unused writes).
        const uint64_t ok = tile_ok ? column_mask(ntok) : 0ull;  // live tokens
        {
          const float a = f16_bits_to_float(x & 0xffffu);
          const float z1 = f16_bits_to_float(x >> 16);
          const float fb = GE::kMse ? p.scale_log2 * inv_sigma * a : p.scale_log2;
          const float val_k = mask_select(ok, fb, -INFINITY);
          const float val_v = mask_select(ok, mask_select(m_kq1, a, fmaf(c0, a, z1)), 0.0f);
          tokf[wave][plane_v][i][col] = mask_select(m_kq0, val_k, val_v);
        }

        // keys -> scores S^T[4kq + r][col]; this lane keeps them if col is in
        // the tile's column group
        float4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (kFold) {
          // hi parts in group i, lo parts in its partner: one MFMA per K
          // step, then the partner's column is added
#pragma unroll
          for (int m = 0; m < KM; ++m)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], i < NB / 2 ? qf[m] : ql[m], sc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] += row_ror<8>(sc[r]);
        } else {
#pragma unroll
          for (int m = 0; m < KM; ++m) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], qf[m], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], ql[m], sc, 0, 0, 0);
          }
        }
        if constexpr (TL == 1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sraw[0][r] = mask_select(m_grp[i], sc[r], sraw[0][r]);
        } else {
          sraw[i] = sc;
        }
        if constexpr (GE::kMse) {
          if constexpr (nc) {
            // ||c_t||^2 of token t = 4kq + r sits on the Gram diagonal, at
            // lane (kq, col = t), register r
            float4_t gram = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < KM; ++m) gram = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], kf[m], gram, 0, 0, 0);
            const float dg = fmaf(gram[3], dsel3, fmaf(gram[2], dsel2, fmaf(gram[1], dsel1, gram[0] * dsel0)));
            // the factor norm * scale / ||c||: sigma cancels; one reciprocal
            // square root per token
            const uint16_t *hh = reinterpret_cast<const uint16_t *>(tw);
            const float nrm = f16_bits_to_float(hh[(static_cast<uint32_t>(col * S) + GE::kKeyCodeBytes) >> 1]);
            const float fnc = p.scale_log2 * nrm * __builtin_amdgcn_rsqf(dg);
            tokf[wave][plane_g][i][col] = mask_select(ok, fnc, -INFINITY);
          }
        }

        // value codes of element group col for tokens 4kq..4kq+3
        if constexpr (!kValLds) {
          if (col < GE::kGroups) {
#pragma unroll
            for (int r = 0; r < 4; ++r) vraw[i][r] = lds_bytes<VB, GE::kValAligned>(tw, val_off + r * S).w[0];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) vraw[i][r] = 0u;
          }
        }
      } else {
        // tile slot past the end of the segment: all its tokens masked. The
        // softmax still multiplies the slot's scale / zero by its zero
        // weights, so they must be finite: LDS holds whatever an earlier
        // workgroup left there (packed slot bytes can read as Inf or NaN)
        tokf[wave][kq][i][col] = kq == 0 ? -INFINITY : 0.0f;
        tbuf[i] = 0;
        if constexpr (!kValLds) {
#pragma unroll
          for (int r = 0; r < 4; ++r) vraw[i][r] = 0u;
        }
      }
    }

    // ---- phase B, once per macro tile: lane (kq, col) holds tokens
    // 4kq..4kq+3 of tile my_tile (TL = 1) or of both tiles (TL = 2) for query
    // head col % GP
    wave_lds_sync();  // per-token scalars written by other lanes
    float s[TL][4];
#pragma unroll
    for (int u = 0; u < TL; ++u) {
      const int ti = TL == 1 ? my_tile : u;
      const float4_t fb4 = *reinterpret_cast<const float4_t *>(&tokf[wave][0][ti][4 * kq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // live tokens: factor >= 0, bias 0; masked ones (-inf): factor 0,
        // bias -inf. MSE scores are finite; FP8 codes of a masked tile may
        // decode to NaN: select instead.
        const float f = fb4[r];
        if constexpr (GE::kMse) s[u][r] = fmaf(sraw[u][r], fmax_raw(f, 0.0f), fmin_raw(f, 0.0f));
        else s[u][r] = f >= 0.0f ? sraw[u][r] * f : -INFINITY;
      }
    }
    // running max of the column: the lane's registers, then the 4 lane rows
    float mloc = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int u = 1; u < TL; ++u) mloc = fmaxf(mloc, fmaxf(fmaxf(s[u][0], s[u][1]), fmaxf(s[u][2], s[u][3])));
    float mt = column_max_raw(mloc);
    if constexpr (kFold) {
      // one maximum per query head over all column groups
      if constexpr (NB == 4) mt = fmax_raw(mt, row_ror<4>(mt));
      mt = fmax_raw(mt, row_ror<8>(mt));
    }
    // lazy reference maximum: weights are exp2(s - m_run), m_run moves only
    // when a column's maximum passes it by more than kLazy (weights up to
    // 2^kLazy; the normalisation by l cancels the reference), so the
    // rescale of the accumulators is rare
    if (mt > m_run + kLazy) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - mn);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] *= alpha;
      l_lane *= alpha;
      z_lane *= alpha;
      m_run = mn;
    }
    const float mr = (m_run == -INFINITY) ? 0.0f : m_run;
    // weights p * s' as f16 hi + lo parts: the value contraction then sees
    // them to ~22 bits (f16 alone leaves a 2^-12 error that cancellation in
    // the weighted sum can amplify)
    u32x2_t hw[TL], lw[TL];
#pragma unroll
    for (int u = 0; u < TL; ++u) {
      const int ti = TL == 1 ? my_tile : u;
      const float4_t s14 = *reinterpret_cast<const float4_t *>(&tokf[wave][1][ti][4 * kq]);
      const float4_t zc4 = *reinterpret_cast<const float4_t *>(&tokf[wave][2][ti][4 * kq]);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(s[u][r] - mr);
        l_lane += pr[r];
        z_lane = fmaf(pr[r], zc4[r], z_lane);
      }
      uint32_t h0, l0, h1, l1;
      split_prod_f16(pr[0], s14[0], pr[1], s14[1], h0, l0);
      split_prod_f16(pr[2], s14[2], pr[3], s14[3], h1, l1);
      hw[u] = u32x2_t{h0, h1};
      lw[u] = u32x2_t{l0, l1};
    }
    wave_lds_sync();  // scalar reads done before the next macro tile rewrites them

    // ---- phase C: value MFMAs, the weights of each tile in its own column
    // group only (zero elsewhere)
    // value code bytes of tile i for this lane's element group, gathered
    auto prep_tile = [&](int i, typename VX::Prep &pr) {
      if constexpr (kValLds) {
        // the tile is still in its buffer: the next load went to the spare one
        const uint32_t *tw = scr + tbuf[i] * (GE::kTileBuf / 4);
        uint32_t vr[4];
        // every lane reads: lanes past the last element group (col >=
        // kGroups, at D < 128) read group kGroups - 1, inside the tile. Those
        // codes are finite, and they only reach output rows 8 col + c >= D of
        // the value MFMAs, which are padding and never written out.
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[r] = lds_field16<VB>(tw, val_off_rd + r * S);
        VX::prep(vr, pr);
      } else {
        VX::prep(vraw[i], pr);
      }
    };
    // Tiles in pairs: one 16x16x32 MFMA takes tokens 4kq..4kq+3 of tile i in
    // K slots 8kq..8kq+3 and those of tile i+1 in 8kq+4..8kq+7, each tile's
    // weights masked to its own column group (TL = 1) or both unmasked
    // (TL = 2: every column is in both tiles' group).
    // A wave in its value phase takes issue priority over the others of its
    // SIMD until the macro tile ends: it feeds the matrix pipe with a burst of
    // MFMAs while they do the VALU-heavy key decode (+1-4 % measured).
    __builtin_amdgcn_s_setprio(1);
    // With partner groups the lo weights of tile t reach group t's partner
    // (the lanes 8 columns away, which hold another tile's scores).
    uint32_t lx[2] = {0u, 0u};
    if constexpr (kFold) {
      lx[0] = row_ror<8>(lw[0][0]);
      lx[1] = row_ror<8>(lw[0][1]);
    }
#pragma unroll
    for (int i = 0; i < NT; i += 2) {
      if (kFull || mt0 + i * kTile < end) {
        if constexpr (kFold) {
          // K rows of tile t: hi weights in group t, lo weights in group
          // (t + NB/2) mod NB, zero elsewhere
          auto pick = [&](int t, int e) -> uint32_t {
            return mask_select(m_grp[t], hw[0][e], mask_select(m_grp[(t + NB / 2) % NB], lx[e], 0u));
          };
          u32x4_t bw;
          bw[0] = pick(i, 0);
          bw[1] = pick(i, 1);
          bw[2] = pick(i + 1, 0);
          bw[3] = pick(i + 1, 1);
          const half8_t pv = __builtin_bit_cast(half8_t, bw);
          // both tiles' fields in flight together; past the end of the range
          // the second tile's weights are zero (masked tokens) and its buffer
          // holds finite codes of some tile
          typename VX::Prep p0, p1;
          prep_tile(i, p0);
          prep_tile(i + 1, p1);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const half8_t av = __builtin_shufflevector(VX::get(p0, c), VX::get(p1, c), 0, 1, 2, 3, 4, 5, 6, 7);
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pv, acc[c], 0, 0, 0);
          }
          continue;
        }
        u32x4_t bh, bl;
        if constexpr (TL == 1) {
          const uint64_t m0 = m_grp[i], m1 = m_grp[i + 1];
          bh[0] = mask_select(m0, hw[0][0], 0u);
          bh[1] = mask_select(m0, hw[0][1], 0u);
          bh[2] = mask_select(m1, hw[0][0], 0u);
          bh[3] = mask_select(m1, hw[0][1], 0u);
          bl[0] = mask_select(m0, lw[0][0], 0u);
          bl[1] = mask_select(m0, lw[0][1], 0u);
          bl[2] = mask_select(m1, lw[0][0], 0u);
          bl[3] = mask_select(m1, lw[0][1], 0u);
        } else {
          bh[0] = hw[0][0];
          bh[1] = hw[0][1];
          bh[2] = hw[1][0];
          bh[3] = hw[1][1];
          bl[0] = lw[0][0];
          bl[1] = lw[0][1];
          bl[2] = lw[1][0];
          bl[3] = lw[1][1];
        }
        const half8_t pvh = __builtin_bit_cast(half8_t, bh);
        const half8_t pvl = __builtin_bit_cast(half8_t, bl);
        typename VX::Prep p0, p1;
        prep_tile(i, p0);
        // past the end of the range the second half's weights are zero
        // (masked tokens) and its buffer holds finite codes of some tile
        prep_tile(i + 1, p1);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const half8_t av = __builtin_shufflevector(VX::get(p0, c), VX::get(p1, c), 0, 1, 2, 3, 4, 5, 6, 7);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pvh, acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pvl, acc[c], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  int mt0 = begin;
  for (; mt0 + NT * kTile < end; mt0 += NT * kTile) macro_tile(mt0, std::true_type{});
  if (mt0 < end) macro_tile(mt0, std::false_type{});

  // ---- partial (m, l, acc + zero terms) of query head col
  l_lane = column_sum(l_lane);
  z_lane = column_sum(z_lane);
  if constexpr (NB > 1) {
    // merge the NB tile slots of each query head: lanes col, col + GP, ...
    // of the same 16-lane row
    float mm = m_run;
#pragma unroll
    for (int o = GP; o < 16; o <<= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
    const float a = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - mm);
    l_lane *= a;
    z_lane *= a;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= a;
#pragma unroll
    for (int o = GP; o < 16; o <<= 1) {
      l_lane += __shfl_xor(l_lane, o, 64);
      z_lane += __shfl_xor(z_lane, o, 64);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[c][r] += __shfl_xor(acc[c][r], o, 64);
    }
    m_run = mm;
  }
  if (col < G) {
    float *dst = part_base + static_cast<int64_t>(col) * pstride;
    if (kq == 0) {
      dst[0] = m_run;
      dst[1] = l_lane;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int grp = 4 * kq + r;
      if (grp < GE::kGroups) {
        float4_t lo, hi;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          lo[c] = fmaf(acc[c][r], VX::inv_scale(c), z_lane);
          hi[c] = fmaf(acc[c + 4][r], VX::inv_scale(c + 4), z_lane);
        }
        *reinterpret_cast<float4_t *>(dst + 4 + 8 * grp) = lo;
        *reinterpret_cast<float4_t *>(dst + 4 + 8 * grp + 4) = hi;
      }
    }
  }
  }  // segment loop
}

// Exact bf16 ring tokens: fp32 VALU, one workgroup per (sequence, KV head,
// kRingChunk-token chunk of the ring), writing partial slot max_splits + chunk
// of the sequence's query heads. The query rows and the chunk's K/V rows are
// all loaded before any of them is stored (one round trip to memory); K rows
// and V transposed go through LDS; scores (thread = token x head group),
// softmax of the chunk (wave = head, lane = token), then P.V (thread = output
// column x head group).
constexpr int kRingThreads = 256;
constexpr int kMaxG = 16;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int D>
__global__ __launch_bounds__(kRingThreads) void decode_ring_kernel(DecodeParams p, int q_dtype) {
  static_assert(kRingChunk <= 64 && kRingChunk % 8 == 0, "a chunk's softmax runs on one wave");
  constexpr int kRow = D + 8;                       // bf16 per K row in LDS (16 bytes of padding)
  constexpr int kTRow = kRingChunk + 8;             // bf16 per transposed V row
  constexpr int kVec = D / 8;                       // 16-byte vectors per K/V row
  constexpr int kHeadGroups = kRingThreads / D;     // P.V: threads per output column
  constexpr int kAcc = (kMaxG + kHeadGroups - 1) / kHeadGroups;
  constexpr int kScoreGroups = kRingThreads / kRingChunk;
  constexpr int kScoreHeads = (kMaxG + kScoreGroups - 1) / kScoreGroups;
  constexpr int kKvLoads = (kRingChunk * kVec + kRingThreads - 1) / kRingThreads;
  constexpr int kQLoads = (kMaxG * D + kRingThreads - 1) / kRingThreads;
  __shared__ float q_s[kMaxG][D];
  __shared__ __align__(16) uint16_t k_s[kRingChunk][kRow];
  __shared__ __align__(16) uint16_t vt_s[D][kTRow];
  __shared__ __align__(16) float p_s[kMaxG][kRingChunk];

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int chunk = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int c0 = chunk * kRingChunk;
  const int n = min(max(min(max(p.ring_lens[b], 0), p.ring_cap) - c0, 0), kRingChunk);
  const int pstride = partial_stride(D);
  const int64_t part0 = static_cast<int64_t>(b) * p.num_q_heads + h * G;
  // this chunk's partial row (G query heads)
  float *prow = p.ring_partials + ((static_cast<int64_t>(b) * p.num_kv_heads + h) * p.ring_chunks + chunk) * G * pstride;

  // A chunk past the ring's length gets the empty partial (m = -inf, l = 0,
  // acc = 0) without loading anything.
  if (n == 0) {
    for (int e = tid; e < G * pstride; e += kRingThreads) {
      const int g = e / pstride, j = e - g * pstride;
      prow[static_cast<int64_t>(g) * pstride + j] = j == 0 ? -INFINITY : 0.0f;
    }
    return;
  }

  const int64_t ring0 = ((static_cast<int64_t>(b) * p.num_kv_heads + h) * p.ring_cap + c0) * D;
  float qv[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int e = tid + i * kRingThreads;
    qv[i] = e < G * D ? load_as_float(p.q, q_dtype, part0 * D + e) : 0.0f;
  }
  u32x4_t kv[kKvLoads], vv[kKvLoads];
#pragma unroll
  for (int i = 0; i < kKvLoads; ++i) {
    const int e = tid + i * kRingThreads;
    const int t = e % kRingChunk, c = e / kRingChunk;
    kv[i] = u32x4_t{0u, 0u, 0u, 0u};
    vv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (c < kVec && t < n) {
      kv[i] = *reinterpret_cast<const u32x4_t *>(p.ring_k + ring0 + t * D + 8 * c);
      vv[i] = *reinterpret_cast<const u32x4_t *>(p.ring_v + ring0 + t * D + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int e = tid + i * kRingThreads;
    if (e < G * D) q_s[e / D][e % D] = qv[i];
  }
#pragma unroll
  for (int i = 0; i < kKvLoads; ++i) {
    const int e = tid + i * kRingThreads;
    const int t = e % kRingChunk, c = e / kRingChunk;
    if (c < kVec) {
      *reinterpret_cast<u32x4_t *>(&k_s[t][8 * c]) = kv[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vt_s[8 * c + 2 * j][t] = static_cast<uint16_t>(vv[i][j] & 0xffffu);
        vt_s[8 * c + 2 * j + 1][t] = static_cast<uint16_t>(vv[i][j] >> 16);
      }
    }
  }
  __syncthreads();
  {
    // scores of token t for heads sg + kScoreGroups i
    const int t = tid % kRingChunk;
    const int sg = tid / kRingChunk;
    float dot[kScoreHeads];
#pragma unroll
    for (int i = 0; i < kScoreHeads; ++i) dot[i] = 0.0f;
    for (int c = 0; c < kVec; ++c) {
      const u32x4_t kw = *reinterpret_cast<const u32x4_t *>(&k_s[t][8 * c]);
      float kx[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kx[2 * e] = bf16_bits_to_float(kw[e] & 0xffffu);
        kx[2 * e + 1] = bf16_bits_to_float(kw[e] >> 16);
      }
#pragma unroll
      for (int i = 0; i < kScoreHeads; ++i) {
        const int g = sg + kScoreGroups * i;
        if (g < G) {
          const float4_t qa = *reinterpret_cast<const float4_t *>(&q_s[g][8 * c]);
          const float4_t qb = *reinterpret_cast<const float4_t *>(&q_s[g][8 * c + 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot[i] = fmaf(qa[e], kx[e], dot[i]);
            dot[i] = fmaf(qb[e], kx[4 + e], dot[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kScoreHeads; ++i) {
      const int g = sg + kScoreGroups * i;
      if (g < G) p_s[g][t] = t < n ? dot[i] * p.scale_log2 : -INFINITY;
    }
  }
  __syncthreads();
  for (int g = wave; g < G; g += kRingThreads / 64) {
    // one wave per head, lane = token (lanes past the chunk hold nothing)
    const float sc = lane < kRingChunk ? p_s[g][lane] : -INFINITY;
    const float m = wave_max(sc);
    const float pt = (sc == -INFINITY) ? 0.0f : exp2f(sc - m);
    if (lane < kRingChunk) p_s[g][lane] = pt;
    const float l = wave_sum(pt);
    if (lane == 0) {
      float *dst = prow + static_cast<int64_t>(g) * pstride;
      dst[0] = m;
      dst[1] = l;
    }
  }
  __syncthreads();
  const int col = tid % D;
  const int grp = tid / D;
  if (grp < kHeadGroups) {
    float acc[kAcc];
#pragma unroll
    for (int a = 0; a < kAcc; ++a) acc[a] = 0.0f;
    for (int t = 0; t < n; t += 8) {
      const u32x4_t vw = *reinterpret_cast<const u32x4_t *>(&vt_s[col][t]);
      float vx[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vx[2 * e] = bf16_bits_to_float(vw[e] & 0xffffu);
        vx[2 * e + 1] = bf16_bits_to_float(vw[e] >> 16);
      }
#pragma unroll
      for (int a = 0; a < kAcc; ++a) {
        const int g = grp + a * kHeadGroups;
        if (g < G) {
          // tokens >= n have p = 0 and zero-filled values
          const float4_t pa = *reinterpret_cast<const float4_t *>(&p_s[g][t]);
          const float4_t pb = *reinterpret_cast<const float4_t *>(&p_s[g][t + 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[a] = fmaf(pa[e], vx[e], acc[a]);
            acc[a] = fmaf(pb[e], vx[4 + e], acc[a]);
          }
        }
      }
    }
#pragma unroll
    for (int a = 0; a < kAcc; ++a) {
      const int g = grp + a * kHeadGroups;
      if (g < G) prow[static_cast<int64_t>(g) * pstride + 4 + col] = acc[a];
    }
  }
}

constexpr int kReduceThreads = 256;
constexpr int kReduceBatch = 6;

// Merge of the split partials of one (sequence, query head): nslots
// compressed-token partials (+ the ring's). Thread (c, r) owns float4 column
// c and merges slots r, r + R, ... with a running log-sum-exp (base 2),
// kReduceBatch slots per step so their loads overlap: a segment of up to
// R kReduceBatch slots (60 at D = 96, 48 at D = 128) is read in one round
// of loads. Six keep the kernel within 64 VGPRs, so 8 waves per SIMD fit
// and a 2048-workgroup grid runs in one generation. The phases are then put
// on their common maximum and summed through LDS.
template <int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeParams p) {
  constexpr int kCols = D / 4;                   // float4 columns
  constexpr int R = kReduceThreads / kCols;      // slot phases
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int col = tid % kCols;
  const int r = tid / kCols;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int h = hq / G;
  const int g = hq - h * G;
  const int ps = partial_stride(D);
  const int64_t seg = static_cast<int64_t>(b) * p.num_kv_heads + h;
  int nslots = 0;
  int64_t row0 = 0;
  if (p.max_seq_len > 0) {
    // the split kernel's work division (header written before this launch):
    // waves w0..w1 covered segment (b, h) and wrote rows w0 + seg .. w1 + seg
    const long long total = reinterpret_cast<const long long *>(p.plan)[0];
    const int active = p.plan[2];
    const int pb = p.plan[4 + b];
    const int nb = p.plan[4 + b + 1] - pb;
    if (nb > 0) {
      const long long s0 = static_cast<long long>(pb) * p.num_kv_heads + static_cast<long long>(h) * nb;
      const int w0 = first_wave(s0, total, active);
      nslots = first_wave(s0 + nb - 1, total, active) - w0 + 1;
      row0 = w0 + seg;
    }
  }
  const int n = nslots + p.ring_chunks;
  const float *part = p.partials + (row0 * G + g) * ps;                       // row stride G ps
  const float *ring_part = p.ring_partials + (seg * p.ring_chunks * G + g) * ps;
  float m = -INFINITY, l = 0.0f;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (r < R) {
    for (int s0 = r; s0 < n; s0 += R * kReduceBatch) {
      float ms[kReduceBatch], ls[kReduceBatch];
      float4_t as[kReduceBatch];
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        const int s = s0 + i * R;
        ms[i] = -INFINITY;
        ls[i] = 0.0f;
        as[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (s < n) {
          const float *e = s < nslots ? part + static_cast<int64_t>(s) * G * ps
                                      : ring_part + static_cast<int64_t>(s - nslots) * G * ps;
          ms[i] = e[0];
          ls[i] = e[1];
          as[i] = reinterpret_cast<const float4_t *>(e + kPartStride_pad)[col];
        }
      }
      float mb = m;
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) mb = fmaxf(mb, ms[i]);
      if (mb > -INFINITY) {
        const float a = exp2f(m - mb);
        acc = acc * a;
        l = l * a;
#pragma unroll
        for (int i = 0; i < kReduceBatch; ++i) {
          const float w = ms[i] > -INFINITY ? exp2f(ms[i] - mb) : 0.0f;
          acc = acc + as[i] * w;
          l = fmaf(ls[i], w, l);
        }
        m = mb;
      }
    }
  }
  // phases -> their common maximum -> sum. Phases without a slot keep
  // m = -inf and add nothing; with no slot at all the output is 0.
  __shared__ float red_m[R], red_l[R];
  __shared__ float4_t red_acc[R][kCols];
  if (r < R && col == 0) red_m[r] = m;
  __syncthreads();
  if (r < R) {
    float mm = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < R; ++i) mm = fmaxf(mm, red_m[i]);
    const float a = m > -INFINITY ? exp2f(m - mm) : 0.0f;
    red_acc[r][col] = acc * a;
    if (col == 0) red_l[r] = l * a;
  }
  __syncthreads();
  if (r == 0) {
    float4_t sum = red_acc[0][col];
    float lsum = red_l[0];
#pragma unroll 8
    for (int i = 1; i < R; ++i) {
      sum = sum + red_acc[i][col];
      lsum += red_l[i];
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    reinterpret_cast<float4_t *>(p.out + (static_cast<int64_t>(b) * p.num_q_heads + hq) * D)[col] = sum * inv;
  }
}

// Workgroups of the split kernel that fit on the device at once
// (occupancy x compute units), cached per (kernel, device, LDS size).
int resident_workgroups(const void *kernel, size_t dyn_lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void *, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const auto key = std::make_tuple(kernel, dev, dyn_lds);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWaves, dyn_lds) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const int n = std::max(1, per_cu) * std::max(1, cus);
  std::lock_guard<std::mutex> g(mu);
  cache[key] = n;
  return n;
}

// Workgroups of one split launch: enough waves for the largest possible
// context, capped at what fits on the device at once. 0 when no split
// kernel runs (no compressed tokens); < 0 on a HIP error.
template <int D, int KB, int VB, int NB, bool NC>
int split_grid(const DecodeParams &p) {
  if (p.batch == 0 || p.max_seq_len <= 0) return 0;
  const size_t dyn = static_cast<size_t>(p.batch + 1) * sizeof(int32_t);
  const void *kern = reinterpret_cast<const void *>(&decode_split_kernel<D, KB, VB, NB, NC>);
  const int resident = resident_workgroups(kern, dyn);
  if (resident < 0) return -1;
  const long long worst_tiles = static_cast<long long>(p.batch) * p.num_kv_heads * ((p.max_seq_len + kTile - 1) / kTile);
  const long long need = (work_waves(worst_tiles, 1 << 30, p.split_tokens) + kWaves - 1) / kWaves;
  return static_cast<int>(std::max(1LL, std::min<long long>(need, resident)));
}

// launch = false: only the split grid, as waves (for sizing the partials).
template <int D, int KB, int VB, int NB, bool NC>
long long launch_decode_t(tq_dtype q_dtype, const DecodeParams &p, hipStream_t s, bool launch) {
  const int grid = split_grid<D, KB, VB, NB, NC>(p);
  if (grid < 0) return -1;
  if (!launch) return static_cast<long long>(grid) * kWaves;
  if (p.batch == 0) return hipSuccess;
  const int qd = static_cast<int>(q_dtype);
  if (grid > 0) {
    const size_t dyn = static_cast<size_t>(p.batch + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, NB, NC>), dim3(grid), dim3(64 * kWaves), dyn, s, p, qd);
    const int err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.ring_cap > 0) {
    hipLaunchKernelGGL((decode_ring_kernel<D>), dim3(p.num_kv_heads, p.batch, p.ring_chunks), dim3(kRingThreads), 0, s,
                       p, qd);
    const int err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(p.num_q_heads, p.batch), dim3(kReduceThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, int KB, int VB, bool NC>
long long dispatch_decode_group(tq_dtype qd, const DecodeParams &p, hipStream_t s, bool launch) {
  const int G = p.num_q_heads / p.num_kv_heads;
  if (G <= 4) return launch_decode_t<D, KB, VB, 4, NC>(qd, p, s, launch);
  if (G <= 8) return launch_decode_t<D, KB, VB, 2, NC>(qd, p, s, launch);
  return launch_decode_t<D, KB, VB, 1, NC>(qd, p, s, launch);
}

// norm correction applies to MSE keys only
template <int D, int KB, int VB>
long long dispatch_decode_nc(tq_dtype qd, const DecodeParams &p, hipStream_t s, bool launch) {
  if (KB != 8 && p.norm_correction) return dispatch_decode_group<D, KB, VB, KB != 8>(qd, p, s, launch);
  return dispatch_decode_group<D, KB, VB, false>(qd, p, s, launch);
}

template <int D>
long long dispatch_decode_bits(const tq_config &c, tq_dtype qd, const DecodeParams &p, hipStream_t s, bool launch) {
  const int kb = c.key_quant_bits, vb = c.value_quant_bits;
  if (kb == 3 && vb == 2) return dispatch_decode_nc<D, 3, 2>(qd, p, s, launch);
  if (kb == 4 && vb == 2) return dispatch_decode_nc<D, 4, 2>(qd, p, s, launch);
  if (kb == 8 && vb == 2) return dispatch_decode_nc<D, 8, 2>(qd, p, s, launch);
  if (kb == 3 && vb == 3) return dispatch_decode_nc<D, 3, 3>(qd, p, s, launch);
  if (kb == 3 && vb == 4) return dispatch_decode_nc<D, 3, 4>(qd, p, s, launch);
  if (kb == 4 && vb == 3) return dispatch_decode_nc<D, 4, 3>(qd, p, s, launch);
  if (kb == 4 && vb == 4) return dispatch_decode_nc<D, 4, 4>(qd, p, s, launch);
  if (kb == 8 && vb == 3) return dispatch_decode_nc<D, 8, 3>(qd, p, s, launch);
  if (kb == 8 && vb == 4) return dispatch_decode_nc<D, 8, 4>(qd, p, s, launch);
  return launch ? hipErrorInvalidValue : -1;
}

long long dispatch_decode(const tq_config &c, tq_dtype q_dtype, const DecodeParams &p, hipStream_t s, bool launch) {
  switch (c.head_dim) {
    case 64: return dispatch_decode_bits<64>(c, q_dtype, p, s, launch);
    case 96: return dispatch_decode_bits<96>(c, q_dtype, p, s, launch);
    case 128: return dispatch_decode_bits<128>(c, q_dtype, p, s, launch);
  }
  return launch ? hipErrorInvalidValue : -1;
}

}  // namespace

// Scratch of the no-allocation decode entry point: the work-division header
// and the partials live here instead of in caller memory. Each device that
// loads the library holds one copy until the process ends; every call on a
// device shares it, so calls that overlap on one device race.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

int static_scratch(void **ptr, size_t *bytes) {
  // The array's name in host code is a host-side stand-in, not a device
  // address: the device address is looked up once per device, with that
  // device current, and kept.
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = 0;
  int err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> g(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

long long decode_launch_waves(const tq_config &c, const DecodeParams &p) {
  return dispatch_decode(c, TQ_BF16, p, nullptr, false);
}

int launch_decode(const tq_config &c, tq_dtype q_dtype, const DecodeParams &p, void *stream) {
  return static_cast<int>(dispatch_decode(c, q_dtype, p, static_cast<hipStream_t>(stream), true));
}

}  // namespace tq
