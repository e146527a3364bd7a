// gather.hip -- A4: assemble each query's memory context from the selected
// documents' compressed K-bar / V-bar blocks (documents in top-k order, blocks
// ascending), a bit-exact copy.
//
// Method: the Top-k documents' compressed K/V are concatenated with the query's
// local K/V for decoding (yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 ->
// 架构; xuqi2024.github.io "【MSA】突破100M Token 上下文…", 5.2; xiaohongrsx.github.io
// "MSA paper reading", 推理全流程).  The local part is read in place by the decode
// kernel, so only the memory part is copied.
//
// One workgroup per (selected document, layer, query); block counts of the k
// selected documents are loaded in parallel and prefix-summed in LDS, then the
// rows are copied with 16-byte coalesced loads and nontemporal stores.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kCopyBatch = 8;   // 16-byte pieces of K and of V in flight per thread

__global__ void __launch_bounds__(kThreads)
gather_kernel(int32_t B, const int32_t* __restrict__ ids, int32_t k, const int64_t* __restrict__ off,
              int32_t n_docs, const uint4* __restrict__ kbar, const uint4* __restrict__ vbar, int64_t n_blk,
              int32_t max_ctx, uint4* __restrict__ ctx_k, uint4* __restrict__ ctx_v, int32_t* __restrict__ ctx_len) {
  __shared__ int64_t s_nb[kMaxTopk];
  __shared__ int64_t s_b0[kMaxTopk];
  const int j = blockIdx.x;
  const int64_t lb = blockIdx.y;
  const int64_t layer = lb / B;
  const int tid = threadIdx.x;
  for (int i = tid; i < k; i += kThreads) {
    const int32_t d = ids[lb * k + i];
    int64_t b0 = 0, nb = 0;
    if (d >= 0 && d < n_docs) {
      b0 = off[d];
      int64_t b1 = off[d + 1];
      if (b0 < 0) b0 = 0;
      if (b1 > n_blk) b1 = n_blk;
      nb = b1 > b0 ? b1 - b0 : 0;
    }
    s_nb[i] = nb;
    s_b0[i] = b0;
  }
  __syncthreads();
  int64_t start = 0;
  for (int i = 0; i < j; ++i) start += s_nb[i];
  if (j == 0 && tid == 0) {
    int64_t total = 0;
    for (int i = 0; i < k; ++i) total += s_nb[i];
    __builtin_nontemporal_store((int32_t)(total < max_ctx ? total : max_ctx), ctx_len + lb);
  }
  int64_t rows = s_nb[j];
  if (start >= max_ctx) rows = 0;
  else if (start + rows > max_ctx) rows = max_ctx - start;
  const int64_t b0 = s_b0[j];
  constexpr int kRowU4 = kRow / 8;  // 128
  const uint4* ks = kbar + (layer * n_blk + b0) * kRowU4;
  const uint4* vs = vbar + (layer * n_blk + b0) * kRowU4;
  uint4* kd = ctx_k + (lb * max_ctx + start) * kRowU4;
  uint4* vd = ctx_v + (lb * max_ctx + start) * kRowU4;
  const int64_t n = rows * kRowU4;
  // kCopyBatch 16-byte pieces of K and of V per thread in flight at once (a document's rows are a
  // few tens of KiB: one or two rounds of loads instead of one round per 4 KiB); nontemporal
  // stores: the rows go out to memory instead of staying dirty in the caches, where the decode
  // that reads them next would find them expensive to fetch
  for (int64_t u0 = tid; u0 < n; u0 += (int64_t)kCopyBatch * kThreads) {
    u32x4 a[kCopyBatch], b[kCopyBatch];
#pragma unroll
    for (int e = 0; e < kCopyBatch; ++e) {
      const int64_t u = u0 + (int64_t)e * kThreads;
      if (u < n) {
        a[e] = *reinterpret_cast<const u32x4*>(ks + u);
        b[e] = *reinterpret_cast<const u32x4*>(vs + u);
      }
    }
#pragma unroll
    for (int e = 0; e < kCopyBatch; ++e) {
      const int64_t u = u0 + (int64_t)e * kThreads;
      if (u < n) {
        __builtin_nontemporal_store(a[e], reinterpret_cast<u32x4*>(kd + u));
        __builtin_nontemporal_store(b[e], reinterpret_cast<u32x4*>(vd + u));
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(int32_t L, int32_t B, const int32_t* ids, int32_t k, const int64_t* doc_blk_off,
                         int32_t n_docs, const uint16_t* kbar, const uint16_t* vbar, int64_t n_blk,
                         int32_t max_ctx, uint16_t* ctx_k, uint16_t* ctx_v, int32_t* ctx_len, hipStream_t s) {
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)k, (unsigned)(L * B)), dim3(kThreads), 0, s, B, ids, k,
                     doc_blk_off, n_docs, reinterpret_cast<const uint4*>(kbar), reinterpret_cast<const uint4*>(vbar),
                     n_blk, max_ctx, reinterpret_cast<uint4*>(ctx_k), reinterpret_cast<uint4*>(ctx_v), ctx_len);
  return hipGetLastError();
}

}  // namespace msa
