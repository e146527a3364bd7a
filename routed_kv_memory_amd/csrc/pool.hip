// pool.hip -- A1: segmented 64-token block mean pooling of K, V and Kr, with the
// pooled routing keys written in the route-key tile layout plus their norms.
//
// Method: each document is cut into 64-token blocks on its own grid and every
// block (a final partial one included) is replaced by the mean of its tokens
// (yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 -> 架构; xuqi2024.github.io
// "【MSA】突破100M Token 上下文…", 3.3.2; xiaohongrsx.github.io "MSA paper reading",
// 方法拆解).
//
// One 512-thread workgroup pools one 16-block tile of one layer; wave w pools
// blocks w and w + 8.  Lane l owns 16-byte chunks l and 64 + l of each 2 KiB token
// row, so every row is two contiguous 1 KiB wave loads (nontemporal: each input
// byte is read once), four tokens in flight per step, summed in fp32 in registers.
// The tile's outputs (K-bar and V-bar rows, routing keys in the route layout) are
// staged in LDS and written as three contiguous 32 KiB runs at the end: writes
// interleaved finely with the read stream, and the route layout's scattered
// 16-byte pieces, cost far more HBM time than their size.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

// Largest d with off[d] <= x, searching d in [0, n) (off non-decreasing, off[0] = 0).
__device__ __forceinline__ int32_t find_doc(const int64_t* __restrict__ off, int32_t n, int64_t x) {
  int32_t lo = 0, hi = n;  // invariant: off[lo] <= x < off[hi] (off[n] treated as +inf)
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Token rows are read exactly once: nontemporal loads keep them from displacing
// useful lines in the caches.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void add8(float* acc, uint4 w) {
  acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
  acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
  acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
  acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
}

// Rounds acc/n to bf16, returns the packed 8 values and adds their squares to *ss.
__device__ __forceinline__ uint4 mean8(const float* acc, float n, float* ss) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = f32_to_bf16_rne(acc[2 * i] / n);
    uint32_t hi = f32_to_bf16_rne(acc[2 * i + 1] / n);
    if (ss) {
      float a = __uint_as_float(lo << 16), b = __uint_as_float(hi << 16);
      *ss += a * a + b * b;
    }
    p[i] = lo | (hi << 16);
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

constexpr int kU = 4;   // tokens per unrolled step

__global__ void __launch_bounds__(512) pool_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                   const uint4* __restrict__ kr, int64_t n_tok,
                                                   const int64_t* __restrict__ tok_off,
                                                   const int64_t* __restrict__ blk_off, int32_t n_docs,
                                                   int64_t n_blk, int64_t tiles, uint4* __restrict__ kbar,
                                                   uint4* __restrict__ vbar, uint4* __restrict__ krt,
                                                   float* __restrict__ krn) {
  __shared__ int64_t s_t0[kTile];
  __shared__ int32_t s_n[kTile];
  __shared__ uint4 s_out[3][kTileElems / 8];   // the tile's K-bar, V-bar rows and route-layout keys
  const int64_t tile = blockIdx.x;
  const int64_t layer = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < kTile) {
    int64_t blk = tile * kTile + tid;
    int64_t t0 = 0;
    int32_t n = 0;
    if (blk < n_blk) {
      int32_t d = find_doc(blk_off, n_docs, blk);
      int64_t j = blk - blk_off[d];
      int64_t s = tok_off[d], e = tok_off[d + 1];
      t0 = s + (int64_t)kBlockTokens * j;
      int64_t t1 = t0 + kBlockTokens < e ? t0 + kBlockTokens : e;
      if (t0 < 0) t0 = 0;
      if (t1 > n_tok) t1 = n_tok;
      n = t1 > t0 ? (int32_t)(t1 - t0) : 0;
    }
    s_t0[tid] = t0;
    s_n[tid] = n;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const uint4* kl = k + layer * n_tok * (kRow / 8);
  const uint4* vl = v + layer * n_tok * (kRow / 8);
  const uint4* rl = kr + layer * n_tok * (kRow / 8);
  for (int b = wave; b < kTile; b += 8) {
    const int64_t blk = tile * kTile + b;
    const int64_t t0 = s_t0[b];
    const int32_t n = s_n[b];
    float ak[2][8] = {}, av[2][8] = {}, ar[2][8] = {};
    int32_t t = 0;
    for (; t + kU <= n; t += kU) {
      uint4 wk[kU][2], wv[kU][2], wr[kU][2];
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t row = (t0 + t + u) * (kRow / 8) + hh * 64 + lane;
          wk[u][hh] = ld_nt(kl + row); wv[u][hh] = ld_nt(vl + row); wr[u][hh] = ld_nt(rl + row);
        }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) { add8(ak[hh], wk[u][hh]); add8(av[hh], wv[u][hh]); add8(ar[hh], wr[u][hh]); }
    }
    for (; t < n; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int64_t row = (t0 + t) * (kRow / 8) + hh * 64 + lane;
        add8(ak[hh], ld_nt(kl + row)); add8(av[hh], ld_nt(vl + row)); add8(ar[hh], ld_nt(rl + row));
      }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c16 = hh * 64 + lane;   // chunk of the row: head c16 / 16, dims (c16 % 16) * 8
      const int h = c16 >> 4, c = c16 & 15;
      float ss = 0.f;
      uint4 ok = make_uint4(0, 0, 0, 0), ov = ok, orr = ok;
      if (n > 0) {
        const float fn = (float)n;
        ok = mean8(ak[hh], fn, nullptr);
        ov = mean8(av[hh], fn, nullptr);
        orr = mean8(ar[hh], fn, &ss);
      }
      s_out[0][b * (kRow / 8) + c16] = ok;
      s_out[1][b * (kRow / 8) + c16] = ov;
      // route layout: [layer][tile][h][c][b][8]
      s_out[2][h * (kTile * 16) + c * kTile + b] = orr;
      ss = row16_sum(ss);   // the 16 lanes of a DPP row hold the 16 chunks of head h
      if (krn && c == 0) krn[((layer * tiles + tile) * kHeads + h) * kTile + b] = sqrtf(ss);
    }
  }
  __syncthreads();
  const int64_t nb = n_blk - tile * kTile < kTile ? n_blk - tile * kTile : kTile;   // real blocks in the tile
  uint4* dk = kbar + (layer * n_blk + tile * kTile) * (kRow / 8);
  uint4* dv = vbar + (layer * n_blk + tile * kTile) * (kRow / 8);
  uint4* dr = krt + (layer * tiles + tile) * (kTileElems / 8);
  for (int i = tid; i < kTileElems / 8; i += 512) {
    if (i < nb * (kRow / 8)) {
      dk[i] = s_out[0][i];
      dv[i] = s_out[1][i];
    }
    dr[i] = s_out[2][i];
  }
}

__global__ void __launch_bounds__(256) pack_kernel(const uint4* __restrict__ rows, int64_t n_blk, int64_t tiles,
                                                   uint4* __restrict__ krt, float* __restrict__ krn) {
  const int64_t tile = blockIdx.x;
  const int64_t layer = blockIdx.y;
  const int tid = threadIdx.x;
  const int half = tid >> 7, c16 = tid & 127, h = c16 >> 4, c = c16 & 15;
  for (int b = half; b < kTile; b += 2) {
    const int64_t blk = tile * kTile + b;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (blk < n_blk) w = rows[(layer * n_blk + blk) * (kRow / 8) + c16];
    float ss = 0.f;
    const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = bf16_lo(p[i]), bb = bf16_hi(p[i]);
      ss += a * a + bb * bb;
    }
    krt[((layer * tiles + tile) * kHeads + h) * (kTile * 16) + c * kTile + b] = w;
    ss = row16_sum(ss);
    if (krn && c == 0) krn[((layer * tiles + tile) * kHeads + h) * kTile + b] = sqrtf(ss);
  }
}

}  // namespace

hipError_t launch_pool(int32_t L, const uint16_t* k, const uint16_t* v, const uint16_t* kr, int64_t n_tok,
                       const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                       uint16_t* kbar, uint16_t* vbar, uint16_t* krt, float* krn, hipStream_t s) {
  const int64_t tiles = route_tiles(n_blk);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)tiles, (unsigned)L), dim3(512), 0, s,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     reinterpret_cast<const uint4*>(kr), n_tok, doc_tok_off, doc_blk_off, n_docs, n_blk, tiles,
                     reinterpret_cast<uint4*>(kbar), reinterpret_cast<uint4*>(vbar), reinterpret_cast<uint4*>(krt),
                     krn);
  return hipGetLastError();
}

hipError_t launch_pack(int32_t L, const uint16_t* rows, int64_t n_blk, uint16_t* krt, float* krn, hipStream_t s) {
  const int64_t tiles = route_tiles(n_blk);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)tiles, (unsigned)L), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(rows), n_blk, tiles, reinterpret_cast<uint4*>(krt), krn);
  return hipGetLastError();
}

}  // namespace msa
