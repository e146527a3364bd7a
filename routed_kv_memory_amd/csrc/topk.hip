// topk.hip -- A3: Top-k documents per (layer, query), ordered by (score
// descending, id ascending).
//
// Method: the k best-scoring documents are kept per routed layer (yunpan.plus
// "MSA端到端可训练记忆模型完整开源…", 整体设计 -> 架构; xuqi2024.github.io
// "【MSA】突破100M Token 上下文…", 3.3.2 doc_top_k = 16; xiaohongrsx.github.io
// "MSA paper reading", 方法拆解).
//
// Each (score, id) becomes one 64-bit key (order-preserving score code << 32 |
// ~id) so a single unsigned comparison realises the total order.  Every pass
// splits each row into chunks, one workgroup per chunk keeps the chunk's k best
// keys, and the next pass merges the candidates until one workgroup per row
// remains, which writes ids and scores.
//
// For k <= 64 a chunk is 2048 keys held in registers (8 per lane): each wave finds
// its k best by ranks among the few keys that can qualify (or, when many keys share a
// score, by repeated wave-wide maxima), and one wave merges the four waves' lists the
// same way.  Larger k bitonic-sorts the chunk in LDS.
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

// ------------------------------------------------------------ register selection (k <= 64)

constexpr int kSelE = 8;                        // keys per lane
constexpr int kSelChunk = 4 * 64 * kSelE;       // keys per workgroup
constexpr int kSelMaxK = 64;

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  return ((uint64_t)h2 << 32) | l2;
}

// Max over the 64 lanes; every lane gets it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp64<0xB1>(v));    // quad_perm [1,0,3,2]
  v = umax64(v, dpp64<0x4E>(v));    // quad_perm [2,3,0,1]
  v = umax64(v, dpp64<0x141>(v));   // row_half_mirror
  v = umax64(v, dpp64<0x140>(v));   // row_mirror: max of the 16-lane row
  {
    // each swap hands a lane its own value and the one of lane l ^ 16 (then l ^ 32)
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = umax64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
  }
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = umax64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
  }
  return v;
}

// The k (<= 64) largest of the wave's E x 64 keys, in descending order: lane r
// returns the r-th (0 for r >= k).  Keys are distinct except the padding key 0.
template <int E>
__device__ __forceinline__ uint64_t wave_topk(uint64_t (&x)[E], int k, int lane) {
  uint64_t m = x[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = umax64(m, x[e]);
  uint64_t res = 0;
  for (int r = 0; r < k; ++r) {
    const uint64_t w = wave_max_u64(m);
    if (lane == r) res = w;
    if (m == w) {                        // the owner drops it and finds its next best
      bool hit = false;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool t = !hit && x[e] == w;
        x[e] = t ? 0 : x[e];
        hit = hit || t;
      }
      m = x[0];
#pragma unroll
      for (int e = 1; e < E; ++e) m = umax64(m, x[e]);
    }
  }
  return res;
}

constexpr int kMaxSurvivors = 128;            // survivors the ranking path takes (else the loop above)
constexpr int kRankLds = 64 + kMaxSurvivors + 64;   // per wave: lane maxima, survivors, results

// The same selection by ranks, with no chain of k dependent wave-wide maxima.  The k-th
// largest of the 64 lane maxima is a lower bound T of the k-th largest key (the lanes holding
// the k largest maxima hold k keys >= T), so only keys >= T can be among the k best; those
// few survivors are compacted in the wave's LDS area, each survivor's rank is the number of
// survivors above it (keys are distinct), and the survivor of rank r is the r-th result.  A
// chunk whose survivors do not fit (many keys of one score) takes wave_topk.  `sm` is the
// wave's own kRankLds-entry LDS area; one wave's LDS operations complete in order.
template <int E>
__device__ __forceinline__ uint64_t wave_topk_rank(uint64_t (&x)[E], int k, int lane, uint64_t* sm) {
  uint64_t m = x[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = umax64(m, x[e]);
  sm[lane] = m;
  int above = 0;
  for (int l = 0; l < 64; ++l) above += sm[l] > m ? 1 : 0;   // same address in every lane
  const uint64_t nz = __ballot(m != 0);
  uint64_t t = 0;                                            // keep every key when < k lanes hold one
  if (__popcll(nz) >= k) {
    const uint64_t hit = __ballot(m != 0 && above == k - 1);   // exactly one lane
    const int src = __ffsll((long long)hit) - 1;
    t = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(m >> 32), src) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, src);
  }
  uint64_t* surv = sm + 64;
  int n_surv = 0;                                            // uniform
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool keep = x[e] != 0 && x[e] >= t;
    const uint64_t mask = __ballot(keep);
    const int pos = n_surv + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (keep && pos < kMaxSurvivors) surv[pos] = x[e];
    n_surv += __popcll(mask);
  }
  if (n_surv > kMaxSurvivors) return wave_topk(x, k, lane);   // uniform
  uint64_t* res = sm + 64 + kMaxSurvivors;
  for (int i = lane; i < n_surv; i += 64) {
    const uint64_t v = surv[i];
    int r = 0;
    for (int q = 0; q < n_surv; ++q) r += surv[q] > v ? 1 : 0;
    if (r < k) res[r] = v;
  }
  return lane < k && lane < n_surv ? res[lane] : 0;
}

template <bool FROM_SCORES, bool FINAL>
__global__ void __launch_bounds__(kThreads)
topk_select_kernel(const float* __restrict__ scores, const uint64_t* __restrict__ keys_in, int64_t n_in,
                   int32_t k, int32_t n_chunks, uint64_t* __restrict__ keys_out, int32_t* __restrict__ ids,
                   float* __restrict__ out_scores) {
  __shared__ uint64_t cand[kThreads / 64][64];
  __shared__ uint64_t rank_lds[kThreads / 64][kRankLds];
  const int64_t row = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * kSelChunk + (int64_t)wave * 64 * kSelE + lane;
  uint64_t x[kSelE];
#pragma unroll
  for (int e = 0; e < kSelE; ++e) {
    const int64_t idx = base + e * 64;
    uint64_t key = 0;  // below every real key
    if (idx < n_in) {
      if (FROM_SCORES) key = make_key(scores[row * n_in + idx], (uint32_t)idx);
      else key = keys_in[row * n_in + idx];
    }
    x[e] = key;
  }
  cand[wave][lane] = wave_topk_rank(x, k, lane, rank_lds[wave]);
  __syncthreads();
  if (wave != 0) return;
  uint64_t y[kThreads / 64];
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) y[w] = cand[w][lane];
  const uint64_t key = wave_topk_rank(y, k, lane, rank_lds[0]);
  if (lane < k) {
    if (FINAL) {
      ids[row * k + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      if (out_scores) out_scores[row * k + lane] = from_ordered_code((uint32_t)(key >> 32));
    } else {
      keys_out[(row * n_chunks + blockIdx.x) * k + lane] = key;
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int32_t n_docs, int32_t k) {
  const int64_t c1 = cdiv(n_docs, kChunk);
  if (c1 <= 1) return 0;
  const int64_t per = rows * c1 * k * (int64_t)sizeof(uint64_t);
  return (size_t)(2 * ((per + 255) / 256) * 256);
}

namespace {

hipError_t launch_topk_select(int64_t rows, const float* scores, int32_t n_docs, int32_t k, int32_t* ids,
                              float* out_scores, void* ws, hipStream_t s) {
  int64_t n_in = n_docs;
  int64_t chunks = cdiv(n_in, kSelChunk);
  if (chunks <= 1) {
    hipLaunchKernelGGL((topk_select_kernel<true, true>), dim3(1, (unsigned)rows), dim3(kThreads), 0, s, scores,
                       nullptr, n_in, k, 1, nullptr, ids, out_scores);
    return hipGetLastError();
  }
  // candidates of pass 1 fit in the bitonic path's workspace (its chunks are smaller)
  const int64_t per = rows * cdiv(n_docs, kChunk) * k * (int64_t)sizeof(uint64_t);
  uint64_t* buf[2] = {reinterpret_cast<uint64_t*>(ws),
                      reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + ((per + 255) / 256) * 256)};
  hipLaunchKernelGGL((topk_select_kernel<true, false>), dim3((unsigned)chunks, (unsigned)rows), dim3(kThreads), 0,
                     s, scores, nullptr, n_in, k, (int32_t)chunks, buf[0], nullptr, nullptr);
  int cur = 0;
  n_in = chunks * k;
  for (;;) {
    chunks = cdiv(n_in, kSelChunk);
    if (chunks <= 1) {
      hipLaunchKernelGGL((topk_select_kernel<false, true>), dim3(1, (unsigned)rows), dim3(kThreads), 0, s,
                         nullptr, buf[cur], n_in, k, 1, nullptr, ids, out_scores);
      break;
    }
    hipLaunchKernelGGL((topk_select_kernel<false, false>), dim3((unsigned)chunks, (unsigned)rows), dim3(kThreads),
                       0, s, nullptr, buf[cur], n_in, k, (int32_t)chunks, buf[cur ^ 1], nullptr, nullptr);
    cur ^= 1;
    n_in = chunks * k;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(int64_t rows, const float* scores, int32_t n_docs, int32_t k, int32_t* ids,
                       float* out_scores, void* ws, hipStream_t s) {
  if (k <= kSelMaxK) return launch_topk_select(rows, scores, n_docs, k, ids, out_scores, ws, s);
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
