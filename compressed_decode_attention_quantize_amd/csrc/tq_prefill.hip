// Continuation prefill over the compressed cache.
//
// Source: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
// TurboQuantConfig.mse_bits docstring (the centroid table is kept for
// continuation-prefill dequant); attention of a chunk's tokens to the
// history, as in direction 1 of the hnwysp.cn article on the stand-alone
// turboquant project (query rotated forward, online softmax over blocks,
// no materialised FP16 KV); norm correction after the TurboQuantConfig
// docstring.
//
// Token t of sequence b's chunk attends to the sequence's compressed history
// and, causally, to the chunk's exact bf16 tokens 0..t. The query rows of one
// KV head are ordered token-major (row r = t * G + g for query head h G + g)
// and cut into row blocks of R = 16 NG rows, one wave each, eight consecutive
// blocks to a workgroup: a history tile is decoded once per workgroup and
// multiplied with all of its 8 R rows.
//
//  attention kernel (one workgroup of eight waves per (sequence, KV head,
//                history split, eight consecutive 32-row blocks); each wave
//                owns one row block, the decoded history is shared)
//     per pair of 16-token history tiles, staged HBM -> LDS two pairs ahead
//     by the waves, then decoded once into LDS operand planes: waves 0 and
//     1 each one tile's key operand, per-token scalars and Gram diagonal,
//     waves 2 and 3 the pair's value operands (element groups 0-3 / 4-7),
//     waves 4-7 nothing:
//       K~ = centroid values (MSE: pair table, FP8: hardware cvt), f16
//       |c_t|^2 = diag(K~ K~^T)             (norm correction only)
//     and every wave, for its own rows:
//       S^T[t][row] = K~ . (Pi q)^T        MFMA 16x16x32 f16 per row group,
//                                          q as f16 hi + lo parts
//       online softmax in exp2 per row group
//       Out^T[j][row] += (code_tj - c0)^T . (p_t s'_t)   MFMA 16x16x32 f16
//                      over the tile pair, codes expanded by the 0x6400
//                      exponent trick, weights as f16 hi + lo parts
//       zero terms += p_t (z'_t + c0 s'_t)
//     the last history split of a row block then takes the chunk's exact
//     tokens 0..t (bf16 MFMA 16x16x32, raw q and the weights as bf16 hi + lo
//     parts, causal mask per row) into the same softmax state;
//     writes an unnormalised partial (m, l, acc[D]) per (row, split).
//  reduce kernel (log-sum-exp merge of a row's split partials, written to
//                out[token][query head]).

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_mfma.h"

namespace tq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = kPrefillWaves;  // waves per workgroup
constexpr int kPad = 4;         // partial = [m, l, -, -, acc[D]]
constexpr int kThreads = 256;   // reduce kernel

__device__ __forceinline__ int pstride(int d) { return d + kPad; }

// bf16 hi + lo parts of 8 floats (hi = RNE(x), lo = RNE(x - hi): 16
// significant bits together).
__device__ __forceinline__ void split_bf16(const float x[8], bf16x8_t &hi, bf16x8_t &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<__bf16>(x[e]);
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hi[e]));
  }
}

// 8 query elements (f32, bf16 or f16) as floats.
__device__ __forceinline__ void load_q8(const void *q, int q_dtype, int64_t e0, bool live, float x[8]) {
  if (q_dtype == TQ_F32) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(q) + e0);
    const u32x4_t a = live ? src[0] : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t b = live ? src[1] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(a[e]);
      x[4 + e] = __uint_as_float(b[e]);
    }
  } else {
    const u32x4_t a = live ? *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(q) + e0)
                           : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q_dtype == TQ_BF16) {
        x[2 * e] = bf16_bits_to_float(a[e] & 0xffffu);
        x[2 * e + 1] = bf16_bits_to_float(a[e] >> 16);
      } else {
        x[2 * e] = f16_bits_to_float(a[e] & 0xffffu);
        x[2 * e + 1] = f16_bits_to_float(a[e] >> 16);
      }
    }
  }
}

template <int D, int KB, int VB, int NG, bool NC>
__global__ __launch_bounds__(64 * kWaves) void prefill_attn_kernel(PrefillParams p, int q_dtype) {
  using GE = Geo<D, KB, VB>;
  using VX = ValueExpand<VB>;
  constexpr int S = GE::kSlot;
  constexpr int KM = GE::kKM;
  constexpr int R = 16 * NG;        // query rows of a wave
  constexpr int kSets = 3;          // staged tile pairs: decoding, loading, spare
  constexpr bool nc = GE::kMse && NC;
  static_assert(GE::kTileChunks <= 64 * kWaves, "a tile is one load instruction per wave");

  // The kWaves waves of a workgroup take consecutive row blocks of one
  // (sequence, KV head, history split) and share the history: each tile pair
  // is staged once for the workgroup and decoded once, split over the first
  // four waves (waves 0 and 1: key operand, Gram diagonal and per-token
  // scalars of tile 0 and 1; waves 2 and 3: value operands of elements 0..3
  // and 4..7 of every 8-element group), into double-buffered operand arrays
  // that every wave then multiplies with its own rows. Waves 4 and up only
  // multiply: two waves share a SIMD, so per pair a SIMD runs one decode
  // share next to two waves' products. One barrier per pair.
  __shared__ uint32_t lut[GE::kLut];
  __shared__ __align__(16) uint32_t stage[kSets][2][GE::kTileBuf / 4];
  __shared__ __align__(16) half8_t kop[2][2][KM][64];  // [parity][tile][k step][lane]
  __shared__ __align__(16) half8_t vop[2][8][64];      // [parity][element c][lane]
  // per-token scalars of a pair: score factor (-inf: masked), s', z' + c0 s';
  // plane 3 takes the writes of lanes that hold nothing for a plane
  __shared__ __align__(16) float tokf[2][4][2][16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int kq = lane >> 4;

  if constexpr (GE::kMse) {
    for (int e = threadIdx.x; e < GE::kLut; e += 64 * kWaves) {
      const int lo = e & ((1 << KB) - 1), hi = e >> KB;
      lut[e] = f16_pair_bits(p.centroids[lo] * p.centroid_scale, p.centroids[hi] * p.centroid_scale);
    }
  }

  // ---- work item of the workgroup. Logical workgroups follow each other on
  // one XCD (the hardware deals workgroups to the 8 XCDs in turn), so the
  // row blocks that stream the same history share that XCD's L2.
  int wg = blockIdx.x;
  if ((gridDim.x & 7u) == 0) wg = (wg & 7) * static_cast<int>(gridDim.x >> 3) + (wg >> 3);
  const int rset = wg % p.row_sets;  // which kWaves consecutive row blocks
  int rest = wg / p.row_sets;
  const int s = rest % p.splits;
  rest /= p.splits;
  const int h = rest % p.num_kv_heads;
  const int b = rest / p.num_kv_heads;
  const int G = p.group;
  const int Hq = p.num_q_heads;
  const int c0 = p.cu_chunk[b];
  const int clen = min(max(p.cu_chunk[b + 1] - c0, 0), p.max_chunk);
  const int nrows = clen * G;
  // no live row in the workgroup: the reduce reads nothing of it
  if (rset * kWaves * R >= nrows) return;
  const int row0 = (rset * kWaves + wave) * R;  // this wave's rows (none: it still decodes its share)
  const int seq_cap = min(p.max_hist, p.max_blocks_per_seq * p.block_size);
  const int hist = min(max(p.hist_lens[b], 0), seq_cap);
  const int t_begin = min(hist, s * p.split_tokens);
  const int t_end = s == p.splits - 1 ? hist : min(hist, t_begin + p.split_tokens);

  // ---- rotated query rows as f16 hi + lo parts in the MFMA B-operand
  // layout, one plane pass per row group through a quarter of the key-operand
  // array (waves 0-3) or of the value-operand array (waves 4-7), both free
  // until the first pair is decoded, after a barrier: column n of group i is
  // row row0 + 16 i + n (zero past the chunk).
  half8_t qf[NG][KM], ql[NG][KM];
  {
    using T = Team<D>;
    const int team = lane / T::kLanes;
    const int r = lane - team * T::kLanes;
    constexpr int rows_per_pass = T::kPerWave;
    constexpr int kPasses = (16 + rows_per_pass - 1) / rows_per_pass;
    static_assert(kWaves == 8, "query planes: four in kop, four in vop");
    static_assert(16 * D * 2 <= static_cast<int>(sizeof(kop)) / 4, "query plane fits a quarter of kop");
    static_assert(16 * D * 2 <= static_cast<int>(sizeof(vop)) / 4, "query plane fits a quarter of vop");
    _Float16 *qs = wave < 4 ? reinterpret_cast<_Float16 *>(&kop[0][0][0][0]) + wave * (static_cast<int>(sizeof(kop)) / 8)
                            : reinterpret_cast<_Float16 *>(&vop[0][0][0]) + (wave - 4) * (static_cast<int>(sizeof(vop)) / 8);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      u32x4_t qhi[kPasses], qlo[kPasses];
      float xs[kPasses][8];
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int g = k * rows_per_pass + team;
        const int row = row0 + 16 * gi + g;
        const bool live = team < rows_per_pass && g < 16 && row < nrows;
        const int t = row / G;
        const int64_t e0 = (static_cast<int64_t>(c0 + (live ? t : 0)) * Hq + h * G + (live ? row - t * G : 0)) * D + 8 * r;
        load_q8(p.q, q_dtype, e0, live, xs[k]);
      }
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        float *x = xs[k];
        if constexpr (GE::kMse) {
          const uint32_t sb = lane_sign_bits(p.sign_words, r);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = flip_sign(x[e], (sb >> e) & 1u);
          team_wht<D>(x, r % T::kBlockLanes);
          const float rb_scale = rsqrtf(static_cast<float>(T::kBlock));
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= rb_scale;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qhi[k][e] = f16_pair_bits(x[2 * e], x[2 * e + 1]);
          qlo[k][e] = f16_pair_bits(x[2 * e] - f16_bits_to_float(qhi[k][e] & 0xffffu),
                                    x[2 * e + 1] - f16_bits_to_float(qhi[k][e] >> 16));
        }
      }
#pragma unroll
      for (int phase = 0; phase < 2; ++phase) {
        wave_lds_sync();  // earlier reads of the plane (other lanes) are done
#pragma unroll
        for (int k = 0; k < kPasses; ++k) {
          const int g = k * rows_per_pass + team;
          if (team < rows_per_pass && g < 16)
            *reinterpret_cast<u32x4_t *>(qs + g * D + 8 * r) = phase == 0 ? qhi[k] : qlo[k];
        }
        wave_lds_sync();  // the rows other lanes wrote are visible
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          const half8_t v = *reinterpret_cast<const half8_t *>(qs + col * D + kq * (D / 4) + 8 * m);
          if (phase == 0) qf[gi][m] = v;
          else ql[gi][m] = v;
        }
      }
    }
  }

  float4_t acc[NG][8];
  float m_run[NG], l_lane[NG], z_lane[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[gi][c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[gi] = -INFINITY;
    l_lane[gi] = 0.0f;
    z_lane[gi] = 0.0f;
  }
  // Online softmax with a lazy reference maximum: weights are exp2(s - m_run)
  // with m_run moved only when a column's maximum exceeds it by more than
  // kLazy (weights up to 2^kLazy; the normalisation by l cancels the
  // reference), so the rescale of the accumulators is a rare branch.
  auto rescale = [&](int gi, float mt) __attribute__((always_inline)) {
    const float mn = fmaxf(m_run[gi], mt);
    const float alpha = mn == -INFINITY ? 1.0f : exp2f(m_run[gi] - mn);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[gi][c] *= alpha;
    l_lane[gi] *= alpha;
    z_lane[gi] *= alpha;
    m_run[gi] = mn;
  };

  // ---- history: tile pairs HBM -> LDS by direct loads (lane l of a load
  // instruction fills bytes [16 l, 16 l + 16) of a 1 KiB LDS window; wave w
  // loads chunks 64 w .. 64 w + 63 of each tile), three staged pairs. In
  // iteration j: pair j + 2 loads, pair j + 1 is decoded (each wave its
  // share), pair j is multiplied from the operands decoded the iteration
  // before.
  if (t_begin < t_end) {
    const int32_t *bt_row = p.block_tables + static_cast<int64_t>(b) * p.max_blocks_per_seq;
    int nx_blk = t_begin / p.block_size;
    int nx_off = t_begin - nx_blk * p.block_size;
    int nx_tok = t_begin;  // first token of the next tile to load
    // block ids of the range, 64 at a time (lane i: logical block blk_base + i)
    int blk_base = nx_blk;
    int blk_lane = blk_base + lane < p.max_blocks_per_seq ? bt_row[blk_base + lane] : 0;
    const uint32_t blk_stride = static_cast<uint32_t>(p.num_kv_heads * p.block_size * S);
    const uint8_t *head_base = p.pool + static_cast<int64_t>(h) * p.block_size * S;
    const uint32_t nblk = static_cast<uint32_t>(p.num_blocks < 0x7fffffff ? p.num_blocks : 0x7fffffff);
    const uint32_t stage_base = lds_offset(&stage[0][0][0]) + 1024u * static_cast<uint32_t>(wave);
    const uint8_t *src = head_base;  // the last tile's source
    uint32_t tile_ok = 0;            // bit 2 set + u: tile u of staged pair `set` is of a valid block
    // the block-id window covers the blocks of the next two tiles
    auto cover = [&]() __attribute__((always_inline)) {
      if (nx_blk - blk_base + 2 > 64) {
        blk_base = nx_blk;
        blk_lane = blk_base + lane < p.max_blocks_per_seq ? bt_row[blk_base + lane] : 0;
        wait_vmcnt<0>();
      }
    };
    // This wave's share of the next tile into tile slot bsel (= 2 set + u).
    // A tile past the range reloads the last source and is masked.
    auto issue = [&](int bsel) __attribute__((always_inline)) {
      const bool live = nx_tok < t_end;
      const int phys = __builtin_amdgcn_readlane(blk_lane, min(nx_blk - blk_base, 63));
      const bool ok = live && static_cast<uint32_t>(phys) < nblk;
      // an invalid block reads the pool's first block instead (its tokens are masked)
      const uint8_t *fresh = head_base + static_cast<uint64_t>(ok ? static_cast<uint32_t>(phys) : 0u) * blk_stride +
                             static_cast<uint32_t>(nx_off * S);
      src = live ? fresh : src;
      tile_ok = (tile_ok & ~(1u << bsel)) | ((ok ? 1u : 0u) << bsel);
      const int adv = live ? kTile : 0;
      nx_tok += adv;
      nx_off += adv;
      const bool wrap = nx_off == p.block_size;
      nx_blk += wrap ? 1 : 0;
      nx_off = wrap ? 0 : nx_off;
      const int c = 64 * wave + lane;
      if (c < GE::kTileChunks)
        load_lds_16s(src, static_cast<uint32_t>(16 * c), stage_base + static_cast<uint32_t>(bsel) * GE::kTileBuf);
    };

    const float c0f = static_cast<float>(VX::kC0);
    const float inv_sigma = 1.0f / p.centroid_scale;
    const uint64_t m_kq0 = lane_mask(kq == 0), m_kq1 = lane_mask(kq == 1);
    const int diag_r = col - 4 * kq;
    const float dsel0 = diag_r == 0 ? 1.0f : 0.0f, dsel1 = diag_r == 1 ? 1.0f : 0.0f;
    const float dsel2 = diag_r == 2 ? 1.0f : 0.0f, dsel3 = diag_r == 3 ? 1.0f : 0.0f;
    const uint32_t val_off_rd = static_cast<uint32_t>(4 * kq * S + GE::kKeyBytes + VB * min(col, GE::kGroups - 1));
    // LDS planes this lane writes per token (loop-invariant): its lane-row
    // scalar, and under norm correction the factor if it holds the diagonal
    const int plane_v = ((nc && kq == 0) || kq == 3) ? 3 : kq;
    const int plane_g = static_cast<uint32_t>(diag_r) < 4u ? 0 : 3;

    // This wave's share of the decode of the staged pair `set` (first token
    // tok0) into operand buffer `par`.
    auto decode_share = [&](int set, int tok0, int par) __attribute__((always_inline)) {
      if (wave < 2) {
        // key operand, per-token scalars and Gram diagonal of tile u = wave
        const int u = wave;
        const int bsel = 2 * set + u;
        const uint32_t *tw = &stage[set][u][0];
        const int ntok = min(max(t_end - (tok0 + u * kTile), 0), kTile);
        const bool tile_valid = (tile_ok >> bsel) & 1u;
        constexpr uint32_t kScaleOff = GE::kKeyBytes + GE::kValCodeBytes;
        uint32_t x;
        {
          const uint16_t *hh = reinterpret_cast<const uint16_t *>(tw);
          const uint32_t off = static_cast<uint32_t>(col * S) + (kq == 0 ? GE::kKeyCodeBytes : kScaleOff);
          x = static_cast<uint32_t>(hh[off >> 1]) | (static_cast<uint32_t>(hh[(off >> 1) + 1]) << 16);
        }
        half8_t kf[KM];
        key_operand<D, KB, VB>(tw, static_cast<uint32_t>(col * S + kq * GE::kLaneKeyBytes), lut, kf);
#pragma unroll
        for (int m = 0; m < KM; ++m) kop[par][u][m][lane] = kf[m];
        const uint64_t ok = tile_valid ? column_mask(ntok) : 0ull;  // live tokens
        {
          // plane kq of token col: the score factor (-inf: masked), s',
          // z' + c0 s'. The factor is norm * scale / sigma (the centroids
          // carry the table scale sigma), the constant scale for FP8 keys;
          // under norm correction the lane holding the token's Gram diagonal
          // writes it below instead.
          const float a = f16_bits_to_float(x & 0xffffu);
          const float z1 = f16_bits_to_float(x >> 16);
          const float fb = GE::kMse ? p.scale_log2 * inv_sigma * a : p.scale_log2;
          const float val_k = mask_select(ok, fb, -INFINITY);
          const float val_v = mask_select(ok, mask_select(m_kq1, a, fmaf(c0f, a, z1)), 0.0f);
          tokf[par][plane_v][u][col] = mask_select(m_kq0, val_k, val_v);
        }
        if constexpr (nc) {
          // ||c_t||^2 of token t = 4kq + r on the Gram diagonal: lane (kq,
          // col = t), register r, picked with exact one-hot multiply-adds
          float4_t gram = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int m = 0; m < KM; ++m) gram = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], kf[m], gram, 0, 0, 0);
          const float dg = fmaf(gram[3], dsel3, fmaf(gram[2], dsel2, fmaf(gram[1], dsel1, gram[0] * dsel0)));
          // the factor norm * scale / ||c||: sigma cancels; one reciprocal
          // square root per token
          const uint16_t *hh = reinterpret_cast<const uint16_t *>(tw);
          const float nrm = f16_bits_to_float(hh[(static_cast<uint32_t>(col * S) + GE::kKeyCodeBytes) >> 1]);
          const float fnc = p.scale_log2 * nrm * __builtin_amdgcn_rsqf(dg);
          tokf[par][plane_g][u][col] = mask_select(ok, fnc, -INFINITY);
        }
      } else if (wave < 4) {
        // value operands of elements c = 4 (wave - 2) .. + 3 of every group:
        // tokens 4kq..4kq+3 of tile 0 in K slots 8kq..8kq+3, of tile 1 in
        // 8kq+4..8kq+7
        typename VX::Prep p0, p1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t *tw = &stage[set][u][0];
          uint32_t vr[4];
          // lanes past the last element group (D < 128) read group kGroups - 1:
          // finite codes that only reach the padding rows 8 col + c >= D
#pragma unroll
          for (int r = 0; r < 4; ++r) vr[r] = lds_field16<VB>(tw, val_off_rd + r * S);
          VX::prep(vr, u == 0 ? p0 : p1);
        }
        // elements at compile time keep the expansion's masks and offsets
        // constant: one branch per wave half
        auto emit = [&](auto half) __attribute__((always_inline)) {
          constexpr int cb = 4 * decltype(half)::value;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            vop[par][cb + k][lane] =
                __builtin_shufflevector(VX::get(p0, cb + k), VX::get(p1, cb + k), 0, 1, 2, 3, 4, 5, 6, 7);
        };
        if (wave == 2) emit(std::integral_constant<int, 0>{});
        else emit(std::integral_constant<int, 1>{});
      }
    };

    // Scores, softmax weights and value MFMAs of the pair decoded into
    // operand buffer `par` (first token tok0, staged pair `set`).
    auto compute_pair = [&](int set, int tok0, int par) __attribute__((always_inline)) {
      float4_t sraw[NG][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        half8_t kf[KM];
#pragma unroll
        for (int m = 0; m < KM; ++m) kf[m] = kop[par][u][m][lane];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          float4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int m = 0; m < KM; ++m) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], qf[gi][m], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[m], ql[gi][m], sc, 0, 0, 0);
          }
          sraw[gi][u] = sc;
        }
      }
      float4_t fb4[2], s1v[2], zcv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        fb4[u] = *reinterpret_cast<const float4_t *>(&tokf[par][0][u][4 * kq]);
        s1v[u] = *reinterpret_cast<const float4_t *>(&tokf[par][1][u][4 * kq]);
        zcv[u] = *reinterpret_cast<const float4_t *>(&tokf[par][2][u][4 * kq]);
      }
      // the exponent arguments s - m of every row group. Full pairs (both
      // tiles inside the range, valid blocks): one fma per score with the
      // reference maximum folded in, and a check that no column passes it by
      // more than kLazy. Otherwise (a masked pair, or a column past the
      // reference) the exact path: masked tokens at -inf, the rescale of the
      // groups whose maximum grew.
      float sv[NG][2][4];
      const bool full = tok0 + 2 * kTile <= t_end && ((tile_ok >> (2 * set)) & 3u) == 3u;
      bool grow = !full;
      if (full) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[gi][u][r] = fmaf(sraw[gi][u][r], fb4[u][r], -m_run[gi]);
          const float mloc = fmaxf(fmaxf(fmaxf(sv[gi][0][0], sv[gi][0][1]), fmaxf(sv[gi][0][2], sv[gi][0][3])),
                                   fmaxf(fmaxf(sv[gi][1][0], sv[gi][1][1]), fmaxf(sv[gi][1][2], sv[gi][1][3])));
          grow = grow || column_max_raw(mloc) > kLazy;
        }
      }
      if (lane_mask(grow) != 0ull) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // live tokens: factor >= 0, bias 0; masked ones (-inf): factor
              // 0, bias -inf. MSE scores are finite; FP8 codes of a masked
              // tile may decode to NaN: select instead.
              const float f = fb4[u][r];
              if constexpr (GE::kMse) sv[gi][u][r] = fmaf(sraw[gi][u][r], fmax_raw(f, 0.0f), fmin_raw(f, 0.0f));
              else sv[gi][u][r] = f >= 0.0f ? sraw[gi][u][r] * f : -INFINITY;
            }
          const float mloc = fmaxf(fmaxf(fmaxf(sv[gi][0][0], sv[gi][0][1]), fmaxf(sv[gi][0][2], sv[gi][0][3])),
                                   fmaxf(fmaxf(sv[gi][1][0], sv[gi][1][1]), fmaxf(sv[gi][1][2], sv[gi][1][3])));
          const float mt = column_max_raw(mloc);
          if (mt > m_run[gi] + kLazy || m_run[gi] == -INFINITY) rescale(gi, mt);
          const float mr = (m_run[gi] == -INFINITY) ? 0.0f : m_run[gi];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[gi][u][r] -= mr;
        }
      }
      // the weights p = exp2(s - m) of every row group, p s' as f16 hi + lo
      // parts, then the value MFMAs of every row group
      u32x4_t bh[NG], bl[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        uint32_t hw[2][2], lw[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float pr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pr[r] = __builtin_amdgcn_exp2f(sv[gi][u][r]);
            l_lane[gi] += pr[r];
            z_lane[gi] = fmaf(pr[r], zcv[u][r], z_lane[gi]);
          }
          split_prod_f16(pr[0], s1v[u][0], pr[1], s1v[u][1], hw[u][0], lw[u][0]);
          split_prod_f16(pr[2], s1v[u][2], pr[3], s1v[u][3], hw[u][1], lw[u][1]);
        }
        bh[gi] = u32x4_t{hw[0][0], hw[0][1], hw[1][0], hw[1][1]};
        bl[gi] = u32x4_t{lw[0][0], lw[0][1], lw[1][0], lw[1][1]};
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const half8_t av = vop[par][c][lane];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          acc[gi][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, bh[gi]), acc[gi][c], 0, 0, 0);
          acc[gi][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, bl[gi]), acc[gi][c], 0, 0, 0);
        }
      }
    };

    // prologue: pairs 0 and 1 loading, pair 0 decoded
    cover();
    issue(0);
    issue(1);
    issue(2);
    issue(3);
    wait_vmcnt<0>();
    __syncthreads();  // pair 0 staged; every wave's query plane reads done
    decode_share(0, t_begin, 0);
    int set_cur = 0, set_n1 = 1, set_n2 = 2, par = 0;
    for (int pt = t_begin; pt < t_end; pt += 2 * kTile) {
      wait_vmcnt<0>();  // this wave's loads of pair j + 1
      // every wave's share of pair j + 1 has landed and its decode of pair j
      // is in the operand buffers; the buffers the iteration rewrites were
      // last read before this point
      __syncthreads();
      cover();
      issue(2 * set_n2);
      issue(2 * set_n2 + 1);
      decode_share(set_n1, pt + 2 * kTile, par ^ 1);  // pair j + 1
      compute_pair(set_cur, pt, par);                 // pair j
      const int t = set_cur;
      set_cur = set_n1;
      set_n1 = set_n2;
      set_n2 = t;
      par ^= 1;
    }
  }

  // accumulators from expanded-code units (2^pos(c) per element c) to plain
  // units: exact power-of-two scales
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[gi][c] *= VX::inv_scale(c);

  // ---- the chunk's exact tokens, causally: the last split of a row block,
  // one row group at a time (the chunk is short next to the history)
  if (s == p.splits - 1) {
    // chunk tokens any row of this block sees: 0 .. t_hi - 1
    const int t_hi = min(clen, (min(row0 + R, nrows) - 1) / G + 1);
    const int64_t kv_row = static_cast<int64_t>(p.num_kv_heads) * D;  // elements per chunk token
    const uint16_t *kbase = p.k_chunk + (static_cast<int64_t>(c0) * p.num_kv_heads + h) * D;
    const uint16_t *vbase = p.v_chunk + (static_cast<int64_t>(c0) * p.num_kv_heads + h) * D;
    const bool vcol = col < GE::kGroups;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int row = row0 + 16 * gi + col;
      const bool live_row = row < nrows;
      const int trow = live_row ? row / G : -1;  // chunk token of this lane's row (-1: no row)
      // chunk tokens this group's rows see
      const int g_hi = min(t_hi, (min(row0 + 16 * gi + 16, nrows) - 1) / G + 1);
      if (row0 + 16 * gi >= nrows) continue;
      // raw query rows as bf16 hi + lo B operands, loaded in place
      bf16x8_t qh[KM], qo[KM];
      {
        const int t = live_row ? row / G : 0;
        const int64_t e0 = (static_cast<int64_t>(c0 + t) * Hq + h * G + (live_row ? row - t * G : 0)) * D + kq * (D / 4);
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          float x[8];
          load_q8(p.q, q_dtype, e0 + 8 * m, live_row, x);
          split_bf16(x, qh[m], qo[m]);
        }
      }
      for (int ct = 0; ct < g_hi; ct += 2 * kTile) {
          float sv[2][4];
          u32x4_t vv[8];
          {
            // keys of this lane's token (col) of both tiles, and the value
            // vectors (element group col) of its 8 tokens: all loads in
            // flight together
            u32x4_t kraw[2][KM];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int tok = ct + u * kTile + col;
              const bool live = tok < g_hi;
              const u32x4_t *src = reinterpret_cast<const u32x4_t *>(kbase + (live ? tok : 0) * kv_row + kq * (D / 4));
#pragma unroll
              for (int m = 0; m < KM; ++m) kraw[u][m] = live ? src[m] : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int tok = ct + (e < 4 ? 4 * kq + e : kTile + 4 * kq + e - 4);
              const bool live = vcol && tok < g_hi;
              vv[e] = live ? *reinterpret_cast<const u32x4_t *>(vbase + tok * kv_row + 8 * col) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              float4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int m = 0; m < KM; ++m) {
                const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kraw[u][m]);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qh[m], a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qo[m], a, 0, 0, 0);
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int tok = ct + u * kTile + 4 * kq + r;
                sv[u][r] = tok <= trow ? a[r] * p.scale_log2 : -INFINITY;
              }
            }
            const float mloc = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
            const float mtc = column_max_raw(mloc);
            if (lane_mask(mtc > m_run[gi] + kLazy) != 0ull) rescale(gi, mtc);
          }
          const float mr = (m_run[gi] == -INFINITY) ? 0.0f : m_run[gi];
          float pw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pw[e] = __builtin_amdgcn_exp2f(sv[e >> 2][e & 3] - mr);
            l_lane[gi] += pw[e];
          }
          bf16x8_t ph, pl;
          split_bf16(pw, ph, pl);
          // element c of the lane's 8 tokens, token pairs packed in 16-bit halves
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t a;
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] = perm(vv[2 * k + 1][c >> 1], vv[2 * k][c >> 1], sel);
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
            acc[gi][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph, acc[gi][c], 0, 0, 0);
            acc[gi][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl, acc[gi][c], 0, 0, 0);
          }
      }
    }
  }

  // ---- partials (m, l, acc + zero terms) of the live rows
  const int64_t bh_rows = (static_cast<int64_t>(b) * p.num_kv_heads + h) * p.rows_pad;
  const int ps = pstride(D);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l = column_sum(l_lane[gi]);
    const float z = column_sum(z_lane[gi]);
    const int row = row0 + 16 * gi + col;
    if (row < nrows) {
      float *dst = p.partials + ((bh_rows + row) * p.splits + s) * ps;
      if (kq == 0) {
        dst[0] = m_run[gi];
        dst[1] = l;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int grp = 4 * kq + r;
        if (grp < GE::kGroups) {
          float4_t lo, hi;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            lo[c] = acc[gi][c][r] + z;
            hi[c] = acc[gi][c + 4][r] + z;
          }
          *reinterpret_cast<float4_t *>(dst + kPad + 8 * grp) = lo;
          *reinterpret_cast<float4_t *>(dst + kPad + 8 * grp + 4) = hi;
        }
      }
    }
  }
}

// Log-sum-exp merge (base 2) of a row's split partials, normalised, to
// out[cu[b] + t][h G + g]: D/4 threads per row, one float4 column each.
template <int D>
__global__ __launch_bounds__(kThreads) void prefill_reduce_kernel(PrefillParams p) {
  constexpr int kCols = D / 4;
  constexpr int kRows = kThreads / kCols;
  const int tid = threadIdx.x;
  const int lr = tid / kCols;
  const int c = tid - lr * kCols;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int row = blockIdx.x * kRows + lr;
  const int G = p.group;
  const int c0 = p.cu_chunk[b];
  const int clen = min(max(p.cu_chunk[b + 1] - c0, 0), p.max_chunk);
  if (lr >= kRows || row >= clen * G) return;
  const int ps = pstride(D);
  const float *part = p.partials + ((static_cast<int64_t>(b) * p.num_kv_heads + h) * p.rows_pad + row) * p.splits * ps;
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, part[static_cast<int64_t>(s) * ps]);
  float l = 0.0f;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < p.splits; ++s) {
    const float *e = part + static_cast<int64_t>(s) * ps;
    const float ms = e[0];
    if (ms > -INFINITY) {
      const float wgt = exp2f(ms - m);
      l = fmaf(e[1], wgt, l);
      acc = acc + reinterpret_cast<const float4_t *>(e + kPad)[c] * wgt;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const int t = row / G;
  const int g = row - t * G;
  reinterpret_cast<float4_t *>(p.out + (static_cast<int64_t>(c0 + t) * p.num_q_heads + h * G + g) * D)[c] = acc * inv;
}

template <int D, int KB, int VB, bool NC>
int launch_t(tq_dtype q_dtype, const PrefillParams &p, hipStream_t st) {
  const int qd = static_cast<int>(q_dtype);
  const long long wgs = p.workgroups;
  if (wgs > 0) {
    hipLaunchKernelGGL((prefill_attn_kernel<D, KB, VB, kPrefillRowGroups, NC>), dim3(static_cast<unsigned>(wgs)),
                       dim3(64 * kWaves), 0, st, p, qd);
    const int err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  constexpr int kRows = kThreads / (D / 4);
  const unsigned gx = static_cast<unsigned>((p.rows_pad + kRows - 1) / kRows);
  hipLaunchKernelGGL((prefill_reduce_kernel<D>), dim3(gx, p.num_kv_heads, p.batch), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D, int KB, int VB>
int launch_nc(tq_dtype qd, const PrefillParams &p, hipStream_t st, bool nc) {
  if (KB != 8 && nc) return launch_t<D, KB, VB, KB != 8>(qd, p, st);
  return launch_t<D, KB, VB, false>(qd, p, st);
}

template <int D>
int launch_bits(const tq_config &c, tq_dtype qd, const PrefillParams &p, hipStream_t st) {
  const int kb = c.key_quant_bits, vb = c.value_quant_bits;
  const bool nc = c.norm_correction != 0;
  if (kb == 3 && vb == 2) return launch_nc<D, 3, 2>(qd, p, st, nc);
  if (kb == 4 && vb == 2) return launch_nc<D, 4, 2>(qd, p, st, nc);
  if (kb == 8 && vb == 2) return launch_nc<D, 8, 2>(qd, p, st, nc);
  if (kb == 3 && vb == 3) return launch_nc<D, 3, 3>(qd, p, st, nc);
  if (kb == 3 && vb == 4) return launch_nc<D, 3, 4>(qd, p, st, nc);
  if (kb == 4 && vb == 3) return launch_nc<D, 4, 3>(qd, p, st, nc);
  if (kb == 4 && vb == 4) return launch_nc<D, 4, 4>(qd, p, st, nc);
  if (kb == 8 && vb == 3) return launch_nc<D, 8, 3>(qd, p, st, nc);
  if (kb == 8 && vb == 4) return launch_nc<D, 8, 4>(qd, p, st, nc);
  return hipErrorInvalidValue;
}

}  // namespace

int launch_prefill(const tq_config &cfg, tq_dtype q_dtype, const PrefillParams &p, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (cfg.head_dim) {
    case 64: return launch_bits<64>(cfg, q_dtype, p, st);
    case 96: return launch_bits<96>(cfg, q_dtype, p, st);
    case 128: return launch_bits<128>(cfg, q_dtype, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
