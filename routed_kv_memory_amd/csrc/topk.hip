// topk.hip -- A3: Top-k documents per (layer, query), ordered by (score
// descending, id ascending).
//
// Method: the k best-scoring documents are kept per routed layer (yunpan.plus
// "MSA端到端可训练记忆模型完整开源…", 整体设计 -> 架构; xuqi2024.github.io
// "【MSA】突破100M Token 上下文…", 3.3.2 doc_top_k = 16; xiaohongrsx.github.io
// "MSA paper reading", 方法拆解).
//
// Each (score, id) becomes one 64-bit key (order-preserving score code << 32 |
// ~id) so a single unsigned comparison realises the total order.  Pass 1: every
// workgroup bitonic-sorts 2048 keys in LDS and keeps its k best; further passes
// merge the candidates the same way until one workgroup per row remains, which
// writes ids and scores.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kChunk = 2048;
constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)ordered_code(s) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

template <bool FROM_SCORES, bool FINAL>
__global__ void __launch_bounds__(kThreads)
topk_pass_kernel(const float* __restrict__ scores, const uint64_t* __restrict__ keys_in, int64_t n_in,
                 int32_t k, int32_t n_chunks, uint64_t* __restrict__ keys_out, int32_t* __restrict__ ids,
                 float* __restrict__ out_scores) {
  __shared__ uint64_t keys[kChunk];
  const int64_t row = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  const int tid = threadIdx.x;
  for (int i = tid; i < kChunk; i += kThreads) {
    const int64_t idx = base + i;
    uint64_t key = 0;  // below every real key
    if (idx < n_in) {
      if (FROM_SCORES) key = make_key(scores[row * n_in + idx], (uint32_t)idx);
      else key = keys_in[row * n_in + idx];
    }
    keys[i] = key;
  }
  // bitonic sort, descending
  for (int size = 2; size <= kChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < kChunk / 2; i += kThreads) {
        const int a = 2 * i - (i & (stride - 1));
        const int c = a + stride;
        const bool desc = (a & size) == 0;
        const uint64_t x = keys[a], y = keys[c];
        if ((x < y) == desc) { keys[a] = y; keys[c] = x; }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += kThreads) {
    const uint64_t key = keys[i];
    if (FINAL) {
      ids[row * k + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      if (out_scores) out_scores[row * k + i] = from_ordered_code((uint32_t)(key >> 32));
    } else {
      keys_out[(row * n_chunks + blockIdx.x) * k + i] = key;
    }
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int32_t n_docs, int32_t k) {
  const int64_t c1 = cdiv(n_docs, kChunk);
  if (c1 <= 1) return 0;
  const int64_t per = rows * c1 * k * (int64_t)sizeof(uint64_t);
  return (size_t)(2 * ((per + 255) / 256) * 256);
}

hipError_t launch_topk(int64_t rows, const float* scores, int32_t n_docs, int32_t k, int32_t* ids,
                       float* out_scores, void* ws, hipStream_t s) {
  int64_t n_in = n_docs;
  int64_t chunks = cdiv(n_in, kChunk);
  if (chunks <= 1) {
    hipLaunchKernelGGL((topk_pass_kernel<true, true>), dim3(1, (unsigned)rows), dim3(kThreads), 0, s, scores,
                       nullptr, n_in, k, 1, nullptr, ids, out_scores);
    return hipGetLastError();
  }
  const int64_t c1 = chunks;
  const int64_t per = rows * c1 * k * (int64_t)sizeof(uint64_t);
  uint64_t* buf[2] = {reinterpret_cast<uint64_t*>(ws),
                      reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + ((per + 255) / 256) * 256)};
  hipLaunchKernelGGL((topk_pass_kernel<true, false>), dim3((unsigned)chunks, (unsigned)rows), dim3(kThreads), 0, s,
                     scores, nullptr, n_in, k, (int32_t)chunks, buf[0], nullptr, nullptr);
  int cur = 0;
  n_in = chunks * k;
  for (;;) {
    chunks = cdiv(n_in, kChunk);
    if (chunks <= 1) {
      hipLaunchKernelGGL((topk_pass_kernel<false, true>), dim3(1, (unsigned)rows), dim3(kThreads), 0, s, nullptr,
                         buf[cur], n_in, k, 1, nullptr, ids, out_scores);
      break;
    }
    hipLaunchKernelGGL((topk_pass_kernel<false, false>), dim3((unsigned)chunks, (unsigned)rows), dim3(kThreads), 0,
                       s, nullptr, buf[cur], n_in, k, (int32_t)chunks, buf[cur ^ 1], nullptr, nullptr);
    cur ^= 1;
    n_in = chunks * k;
  }
  return hipGetLastError();
}

}  // namespace msa
