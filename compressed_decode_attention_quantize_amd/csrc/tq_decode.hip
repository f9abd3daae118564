// Fused decode attention over compressed slots: split kernel + reduce kernel.
//
// Source: hnwysp.cn article on the stand-alone turboquant project,
// next-directions section, direction 1 (one pass over the compressed data,
// flash-attention style online softmax block by block, query rotated forward
// so the D-dim keys are never rotated back, no materialised FP16 KV); the
// write-path section (128-token bf16 exact ring buffer) for the ring chunk;
// vLLM API page TurboQuantConfig docstring for norm correction.
//
// Work split (flash-decoding): one workgroup per (split, kv head, sequence).
// A split is a range of split_tokens compressed positions, or the ring. It
// walks 16-token tiles; since block_size is a multiple of 16 each tile's 16
// slots are contiguous in the pool ([blk][h][bs][S]). It writes an
// unnormalised partial (m, l, acc[D]) in the exp2 domain; the reduce kernel
// merges the partials of a (sequence, query head) by log-sum-exp.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kDecThreads = 256;
constexpr int kTile = 16;
constexpr int kMaxG = 16;
constexpr int kMaxSlot = 196;

template <int D, int KB, int VB>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeParams p, int q_dtype) {
  constexpr int kGroups = kDecThreads / D;         // thread groups over query heads
  constexpr int kAccPerThread = (kMaxG + kGroups - 1) / kGroups;
  constexpr bool kMse = KB != 8;
  constexpr int kKeyIdxBytes = kMse ? (D * KB) / 8 : D;
  constexpr int kValCodeBytes = (D * VB) / 8;

  __shared__ float q_s[kMaxG][D];
  __shared__ float k_s[kTile][D + 1];
  __shared__ float v_s[kTile][D + 1];
  __shared__ float f_s[kTile];
  __shared__ float p_s[kMaxG][kTile];
  __shared__ float alpha_s[kMaxG];
  __shared__ float cent_s[16];
  __shared__ __align__(16) uint8_t run_s[kTile * kMaxSlot];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const bool ring_split = split >= p.num_splits;

  // ---- token range of this split
  int begin = 0, end = 0;
  if (!ring_split) {
    int len = p.seq_lens[b];
    len = min(max(len, 0), min(p.max_seq_len, p.max_blocks_per_seq * p.block_size));
    begin = split * p.split_tokens;
    end = min(len, begin + p.split_tokens);
  } else if (p.ring_k != nullptr) {
    end = min(max(p.ring_lens[b], 0), p.ring_cap);
  }

  if (tid < 16) cent_s[tid] = p.centroids[tid];

  // ---- queries (rotated forward for MSE keys on compressed splits)
  const bool rotate = kMse && !ring_split;
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int g = e / D, j = e % D;
    float qv = load_as_float(p.q, q_dtype, (static_cast<int64_t>(b) * p.num_q_heads + h * G + g) * D + j);
    if (rotate && ((p.sign_words[j >> 5] >> (j & 31)) & 1u)) qv = -qv;
    q_s[g][j] = qv;
  }
  __syncthreads();
  if (rotate) {
    constexpr int B = D & (-D);
    for (int hh = 1; hh < B; hh <<= 1) {
      for (int e = tid; e < G * (D / 2); e += kDecThreads) {
        const int g = e / (D / 2), pr = e % (D / 2);
        const int j = (pr / hh) * (2 * hh) + (pr % hh);
        const float a = q_s[g][j], c = q_s[g][j + hh];
        q_s[g][j] = a + c;
        q_s[g][j + hh] = a - c;
      }
      __syncthreads();
    }
    const float rb = rsqrtf(static_cast<float>(B));
    for (int e = tid; e < G * D; e += kDecThreads) q_s[e / D][e % D] *= rb;
    __syncthreads();
  }

  // running max / sum of query head tid (threads tid < G)
  float m_run = -INFINITY, l_run = 0.0f;
  float acc[kAccPerThread];
#pragma unroll
  for (int a = 0; a < kAccPerThread; ++a) acc[a] = 0.0f;
  const int jj = tid % D;
  const int grp = tid / D;

  for (int tile = begin; tile < end; tile += kTile) {
    const int ntok = min(kTile, end - tile);
    bool tile_ok = true;
    if (!ring_split) {
      // stage the tile's 16 contiguous slots
      const int lblk = tile / p.block_size;
      const int off = tile % p.block_size;
      const int phys = p.block_tables[static_cast<int64_t>(b) * p.max_blocks_per_seq + lblk];
      tile_ok = phys >= 0 && phys < p.num_blocks;
      if (tile_ok) {
        const uint8_t *src = p.pool + ((static_cast<int64_t>(phys) * p.num_kv_heads + h) * p.block_size + off) *
                                          static_cast<int64_t>(p.slot_bytes);
        const int nvec = (kTile * p.slot_bytes) / 16;
        for (int e = tid; e < nvec; e += kDecThreads)
          reinterpret_cast<uint4 *>(run_s)[e] = reinterpret_cast<const uint4 *>(src)[e];
      }
    }
    __syncthreads();
    // decode the tile to fp32 (keys in the rotated basis for MSE)
    for (int e = tid; e < kTile * D; e += kDecThreads) {
      const int t = e / D, j = e % D;
      float kv = 0.0f, vv = 0.0f;
      if (t < ntok) {
        if (ring_split) {
          const int64_t ro = ((static_cast<int64_t>(b) * p.num_kv_heads + h) * p.ring_cap + tile + t) * D + j;
          kv = bf16_bits_to_float(p.ring_k[ro]);
          vv = bf16_bits_to_float(p.ring_v[ro]);
        } else if (tile_ok) {
          const uint8_t *slot = run_s + t * p.slot_bytes;
          if constexpr (kMse) {
            const int bit = j * KB;
            const uint32_t w = static_cast<uint32_t>(slot[bit >> 3]) | (static_cast<uint32_t>(slot[(bit >> 3) + 1]) << 8);
            kv = cent_s[(w >> (bit & 7)) & ((1u << KB) - 1u)];
          } else {
            kv = e4m3fn_to_float(slot[j]);
          }
          const uint8_t *vf = slot + p.key_bytes;
          const int vbit = j * VB;
          const uint32_t w = static_cast<uint32_t>(vf[vbit >> 3]) | (static_cast<uint32_t>(vf[(vbit >> 3) + 1]) << 8);
          const uint32_t code = (w >> (vbit & 7)) & ((1u << VB) - 1u);
          const uint32_t sb = vf[kValCodeBytes] | (static_cast<uint32_t>(vf[kValCodeBytes + 1]) << 8);
          const uint32_t zb = vf[kValCodeBytes + 2] | (static_cast<uint32_t>(vf[kValCodeBytes + 3]) << 8);
          vv = fmaf(f16_bits_to_float(sb), static_cast<float>(code), f16_bits_to_float(zb));
        }
      }
      k_s[t][j] = kv;
      v_s[t][j] = vv;
    }
    __syncthreads();
    // per-token score factor
    if (tid < kTile) {
      float f = 1.0f;
      if (kMse && !ring_split && tid < ntok && tile_ok) {
        const uint8_t *slot = run_s + tid * p.slot_bytes;
        f = f16_bits_to_float(slot[kKeyIdxBytes] | (static_cast<uint32_t>(slot[kKeyIdxBytes + 1]) << 8));
        if (p.norm_correction) {
          float ss = 0.0f;
          for (int j = 0; j < D; ++j) ss = fmaf(k_s[tid][j], k_s[tid][j], ss);
          f = f / sqrtf(ss);
        }
      }
      f_s[tid] = f;
    }
    __syncthreads();
    // scores (log2 domain)
    for (int e = tid; e < G * kTile; e += kDecThreads) {
      const int g = e / kTile, t = e % kTile;
      float s = -INFINITY;
      if (t < ntok && (ring_split || tile_ok)) {
        float d = 0.0f;
        for (int j = 0; j < D; ++j) d = fmaf(q_s[g][j], k_s[t][j], d);
        s = d * f_s[t] * p.scale_log2;
      }
      p_s[g][t] = s;
    }
    __syncthreads();
    // online softmax bookkeeping, one thread per query head
    if (tid < G) {
      const int g = tid;
      float mt = -INFINITY;
      for (int t = 0; t < kTile; ++t) mt = fmaxf(mt, p_s[g][t]);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
      float lsum = 0.0f;
      for (int t = 0; t < kTile; ++t) {
        const float pt = (p_s[g][t] == -INFINITY) ? 0.0f : exp2f(p_s[g][t] - m_new);
        p_s[g][t] = pt;
        lsum += pt;
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      alpha_s[g] = alpha;
    }
    __syncthreads();
    // value accumulation
    if (grp < kGroups) {
#pragma unroll
      for (int a = 0; a < kAccPerThread; ++a) {
        const int g = grp + a * kGroups;
        if (g < G) {
          float s = acc[a] * alpha_s[g];
          for (int t = 0; t < kTile; ++t) s = fmaf(p_s[g][t], v_s[t][jj], s);
          acc[a] = s;
        }
      }
    }
    __syncthreads();
  }

  // ---- partials
  const int64_t stride = D + 2;
  if (grp < kGroups) {
#pragma unroll
    for (int a = 0; a < kAccPerThread; ++a) {
      const int g = grp + a * kGroups;
      if (g < G) {
        float *dst = p.partials + ((static_cast<int64_t>(b) * p.num_q_heads + h * G + g) * p.splits_total + split) * stride;
        dst[2 + jj] = acc[a];
      }
    }
  }
  if (tid < G) {
    float *dst = p.partials + ((static_cast<int64_t>(b) * p.num_q_heads + h * G + tid) * p.splits_total + split) * stride;
    dst[0] = m_run;
    dst[1] = l_run;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeParams p) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int j = threadIdx.x;
  const float *part = p.partials + (static_cast<int64_t>(b) * p.num_q_heads + hq) * p.splits_total * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < p.splits_total; ++s) m = fmaxf(m, part[s * (D + 2)]);
  float l = 0.0f, o = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < p.splits_total; ++s) {
      const float ms = part[s * (D + 2)];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - m);
      l = fmaf(part[s * (D + 2) + 1], w, l);
      o = fmaf(part[s * (D + 2) + 2 + j], w, o);
    }
  }
  p.out[(static_cast<int64_t>(b) * p.num_q_heads + hq) * D + j] = (l > 0.0f) ? o / l : 0.0f;
}

template <int D, int KB, int VB>
int launch_decode_t(tq_dtype q_dtype, const DecodeParams &p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const dim3 grid(p.splits_total, p.num_kv_heads, p.batch);
  hipLaunchKernelGGL((decode_split_kernel<D, KB, VB>), grid, dim3(kDecThreads), 0, s, p, static_cast<int>(q_dtype));
  int err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(p.num_q_heads, p.batch), dim3(D), 0, s, p);
  return hipGetLastError();
}

template <int D>
int dispatch_decode_bits(const tq_config &c, tq_dtype qd, const DecodeParams &p, hipStream_t s) {
  const int kb = c.key_quant_bits, vb = c.value_quant_bits;
  if (kb == 3 && vb == 3) return launch_decode_t<D, 3, 3>(qd, p, s);
  if (kb == 3 && vb == 4) return launch_decode_t<D, 3, 4>(qd, p, s);
  if (kb == 4 && vb == 3) return launch_decode_t<D, 4, 3>(qd, p, s);
  if (kb == 4 && vb == 4) return launch_decode_t<D, 4, 4>(qd, p, s);
  if (kb == 8 && vb == 3) return launch_decode_t<D, 8, 3>(qd, p, s);
  if (kb == 8 && vb == 4) return launch_decode_t<D, 8, 4>(qd, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

int launch_decode(const tq_config &c, tq_dtype q_dtype, const DecodeParams &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (c.head_dim) {
    case 64: return dispatch_decode_bits<64>(c, q_dtype, p, s);
    case 96: return dispatch_decode_bits<96>(c, q_dtype, p, s);
    case 128: return dispatch_decode_bits<128>(c, q_dtype, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
