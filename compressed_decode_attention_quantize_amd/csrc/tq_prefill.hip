// Continuation prefill over the compressed cache: layout kernels around the
// decode kernels.
//
// Source: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
// TurboQuantConfig.mse_bits docstring (the centroid table is kept for
// continuation-prefill dequant); attention of a chunk's tokens to the
// history, as in direction 1 of the hnwysp.cn article on the stand-alone
// turboquant project (query rotated forward, online softmax over blocks).
//
// Token t of sequence b's chunk attends to the sequence's compressed history
// and, causally, to the chunk's exact tokens 0..t. The query rows of one KV
// head (chunk token x query head of that KV head, token-major) are cut into
// groups of 16; each group is one "virtual sequence" of the decode kernels,
// which fill all 16 MFMA columns with its rows:
//   - the split kernel streams the history once per row group (its block
//     table row and length are the sequence's),
//   - the ring kernel attends to the chunk, stored once per sequence in the
//     ring layout and shared by the sequence's row groups, each row cut at
//     its own causal limit,
//   - the reduce merges both into one fp32 row per virtual query head,
// and a scatter puts the rows back in [token][head] order.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// q' [vb][h * 16 + c][D] <- q [cu[b] + t][h * G + g] with vb = b * rg + j,
// row r = 16 j + c = t * G + g; rows past the chunk are zero. 16 bytes per
// thread step (elem_bytes 2 or 4).
__global__ __launch_bounds__(kThreads) void prefill_gather_q(PrefillParams p) {
  const int64_t vec_per_row = static_cast<int64_t>(p.head_dim) * p.q_elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(p.vbatch) * p.num_kv_heads * 16 * vec_per_row;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = e / vec_per_row;  // vb * (Hkv * 16) + h * 16 + c
    const int64_t x = e - row * vec_per_row;
    const int vb = static_cast<int>(row / (p.num_kv_heads * 16));
    const int hc = static_cast<int>(row - static_cast<int64_t>(vb) * p.num_kv_heads * 16);
    const int h = hc / 16, c = hc % 16;
    const int b = vb / p.row_groups;
    const int r = (vb - b * p.row_groups) * 16 + c;
    const int t = r / p.group, g = r % p.group;
    const int c0 = p.cu_chunk[b], clen = p.cu_chunk[b + 1] - c0;
    uint4 v = {0u, 0u, 0u, 0u};
    if (t < clen) {
      const int64_t src = (static_cast<int64_t>(c0 + t) * p.num_q_heads + h * p.group + g) * vec_per_row + x;
      v = reinterpret_cast<const uint4 *>(p.q)[src];
    }
    reinterpret_cast<uint4 *>(p.vq)[e] = v;
  }
}

// ring' [b][h][t][D] <- chunk [cu[b] + t][h][D] (bf16), zero past the chunk.
__global__ __launch_bounds__(kThreads) void prefill_gather_chunk(PrefillParams p) {
  const int64_t vec_per_row = p.head_dim / 8;
  const int64_t total = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.max_chunk * vec_per_row;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = e / vec_per_row;  // (b * Hkv + h) * max_chunk + t
    const int64_t x = e - row * vec_per_row;
    const int t = static_cast<int>(row % p.max_chunk);
    const int64_t bh = row / p.max_chunk;
    const int h = static_cast<int>(bh % p.num_kv_heads);
    const int b = static_cast<int>(bh / p.num_kv_heads);
    const int c0 = p.cu_chunk[b], clen = p.cu_chunk[b + 1] - c0;
    uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (t < clen) {
      const int64_t src = (static_cast<int64_t>(c0 + t) * p.num_kv_heads + h) * vec_per_row + x;
      kv = reinterpret_cast<const uint4 *>(p.k_chunk)[src];
      vv = reinterpret_cast<const uint4 *>(p.v_chunk)[src];
    }
    reinterpret_cast<uint4 *>(p.ring_k)[e] = kv;
    reinterpret_cast<uint4 *>(p.ring_v)[e] = vv;
  }
}

// Per virtual sequence: its block-table row, history length and chunk length
// (0 for a row group past the chunk), and each row's causal limit.
__global__ __launch_bounds__(kThreads) void prefill_tables(PrefillParams p) {
  const int vb = blockIdx.x;
  const int b = vb / p.row_groups;
  const int j = vb - b * p.row_groups;
  const int c0 = p.cu_chunk[b], clen = p.cu_chunk[b + 1] - c0;
  const bool live = 16 * j < clen * p.group;
  for (int i = threadIdx.x; i < p.max_blocks_per_seq; i += blockDim.x)
    p.vtables[static_cast<int64_t>(vb) * p.max_blocks_per_seq + i] =
        p.block_tables[static_cast<int64_t>(b) * p.max_blocks_per_seq + i];
  for (int hc = threadIdx.x; hc < p.num_kv_heads * 16; hc += blockDim.x) {
    const int r = 16 * j + hc % 16;
    const int t = r / p.group;
    p.row_lens[static_cast<int64_t>(vb) * p.num_kv_heads * 16 + hc] = t < clen ? t + 1 : 0;
  }
  if (threadIdx.x == 0) {
    p.vseq_lens[vb] = live ? max(p.hist_lens[b], 0) : 0;
    p.vring_lens[vb] = live ? clen : 0;
  }
}

// out [cu[b] + t][h * G + g][D] <- out' [vb][h * 16 + c][D].
__global__ __launch_bounds__(kThreads) void prefill_scatter(PrefillParams p) {
  const int64_t vec_per_row = p.head_dim / 4;
  const int64_t total = static_cast<int64_t>(p.vbatch) * p.num_kv_heads * 16 * vec_per_row;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = e / vec_per_row;
    const int64_t x = e - row * vec_per_row;
    const int vb = static_cast<int>(row / (p.num_kv_heads * 16));
    const int hc = static_cast<int>(row - static_cast<int64_t>(vb) * p.num_kv_heads * 16);
    const int h = hc / 16, c = hc % 16;
    const int b = vb / p.row_groups;
    const int r = (vb - b * p.row_groups) * 16 + c;
    const int t = r / p.group, g = r % p.group;
    const int c0 = p.cu_chunk[b], clen = p.cu_chunk[b + 1] - c0;
    if (t < clen) {
      const int64_t dst = (static_cast<int64_t>(c0 + t) * p.num_q_heads + h * p.group + g) * vec_per_row + x;
      reinterpret_cast<float4 *>(p.out)[dst] = reinterpret_cast<const float4 *>(p.vout)[e];
    }
  }
}

unsigned grid_for(int64_t items) {
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
}

}  // namespace

int launch_prefill_prep(const PrefillParams &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t qv = static_cast<int64_t>(p.vbatch) * p.num_kv_heads * 16 * p.head_dim * p.q_elem_bytes / 16;
  hipLaunchKernelGGL(prefill_gather_q, dim3(grid_for(qv)), dim3(kThreads), 0, s, p);
  const int64_t cv = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.max_chunk * (p.head_dim / 8);
  hipLaunchKernelGGL(prefill_gather_chunk, dim3(grid_for(cv)), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(prefill_tables, dim3(p.vbatch), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

int launch_prefill_scatter(const PrefillParams &p, void *stream) {
  const int64_t ov = static_cast<int64_t>(p.vbatch) * p.num_kv_heads * 16 * (p.head_dim / 4);
  hipLaunchKernelGGL(prefill_scatter, dim3(grid_for(ov)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return hipGetLastError();
}

}  // namespace tq
