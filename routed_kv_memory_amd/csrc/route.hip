// route.hip -- A2: the routing scan.  Scores every pooled routing key against the
// query's routing projection by cosine similarity, averages over the 8 heads,
// takes the max over query tokens, and folds the per-block results into
// per-document maxima.
//
// Method: yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 -> 架构 (cosine,
// mean over heads first, then max over tokens, Top-k documents); xiaohongrsx.github.io
// "MSA paper reading", 方法拆解 (Qr against every document's Kr-bar by cosine).
//
// Design (gfx950):
//  * Queries of >= 16 tokens: per head the scan is a [blocks x 128] . [128 x tokens]
//    bf16 contraction, run on v_mfma_f32_16x16x32_bf16 with blocks as the A operand
//    (read straight from HBM: the route-key tile layout makes every wave load one
//    contiguous 1 KiB fragment) and the query as the B operand (staged once per
//    workgroup in LDS in fragment order, 128 KiB for 64 tokens).  The per-head
//    cosine scaling 1/(|q| |k|) is applied to the fp32 accumulators before the head
//    sum, so the bf16 inputs enter the matrix cores exactly as stored.
//  * The max over tokens is a DPP row reduction (tokens are the 16 lanes of a row
//    of the accumulator layout); the per-document max is a segmented shuffle scan
//    keyed by a block->document map, ending in one atomic max per document run.
//  * Persistent grid: one 512-thread workgroup per CU; each owns a contiguous range
//    of (layer, 32-block wave tile) items for one 64-token query chunk, so the
//    128 KiB K-bar_r stream is read once with two waves per SIMD in flight.
//  * Queries of < 16 tokens use a vector-ALU kernel over the same layout.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kWaves = 8;
constexpr int kWG = kWaves * 64;
constexpr int kTokChunk = 64;
constexpr int kTileU4 = kTileElems / 8;   // 2048 uint4 per tile
constexpr int kHeadU4 = kTileU4 / kHeads; // 256 uint4 per (tile, head)

__device__ __forceinline__ int32_t find_doc(const int64_t* __restrict__ off, int32_t n, int64_t x) {
  int32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// blk_doc[i] = document of block i, -1 for padding blocks (i >= n_blk) or if the
// offsets do not cover i.
__global__ void blk_doc_kernel(const int64_t* __restrict__ off, int32_t n_docs, int64_t n_blk, int64_t n_pad,
                               int32_t* __restrict__ blk_doc) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pad; i += stride) {
    int32_t d = -1;
    if (i < n_blk) {
      int32_t c = find_doc(off, n_docs, i);
      if (off[c] <= i && i < off[c + 1]) d = c;
    }
    blk_doc[i] = d;
  }
}

__global__ void codes_init_kernel(uint32_t* __restrict__ codes, int64_t n, int accumulate) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint32_t c = 0u;
    if (accumulate) {
      float f = __uint_as_float(codes[i]);
      c = (f == -__builtin_huge_valf()) ? 0u : ordered_code(f);
    }
    codes[i] = c;
  }
}

__global__ void codes_final_kernel(uint32_t* __restrict__ codes, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    codes[i] = __float_as_uint(from_ordered_code(codes[i]));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ---------------------------------------------------------------- MFMA scan
//
// Work item = one 32-block wave tile (route tiles 2w, 2w+1) of one layer.
// Accumulator layout of v_mfma_f32_16x16x32_bf16 (A = 16 blocks x 32 dims,
// B = 32 dims x 16 tokens): lane l holds token (l & 15) and blocks 4*(l >> 4) + r.
template <int NT>
__global__ void __launch_bounds__(kWG)
route_mfma_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, int32_t n_tc,
                  const uint4* __restrict__ krt, const float4* __restrict__ krn, int64_t n_blk, int64_t tiles,
                  const int32_t* __restrict__ blk_doc, int32_t n_docs, int32_t L, int32_t R,
                  uint32_t* __restrict__ codes) {
  __shared__ uint4 q_lds[kHeads * 4 * 4 * 64];   // [h][s][nt][lane] fragments, 128 KiB
  __shared__ float rq_lds[kHeads * kTokChunk];   // [h][token] 1/max(|q|, eps)

  // XCD-aware placement: workgroups are dispatched round-robin over 8 XCDs; when the
  // ranges divide evenly, keep the chunks that share a range on one XCD (shared L2).
  const int C = (int)(gridDim.x / (unsigned)R);
  int r, cidx;
  {
    const int i = (int)blockIdx.x;
    if ((R & 7) == 0) {
      const int xcd = i & 7, slot = i >> 3;
      r = xcd + 8 * (slot / C);
      cidx = slot % C;
    } else {
      r = i / C;
      cidx = i % C;
    }
  }
  const int b = cidx / n_tc;
  const int tc = cidx % n_tc;
  const int t_base = tc * kTokChunk;

  const int64_t n_wt = (tiles + 1) >> 1;
  const int64_t W = (int64_t)L * n_wt;
  const int64_t it_begin = W * r / R;
  const int64_t it_end = W * (r + 1) / R;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int j = lane & 15;

  for (int64_t seg = it_begin; seg < it_end;) {
    const int layer = (int)(seg / n_wt);
    const int64_t lay_end = (int64_t)(layer + 1) * n_wt;
    const int64_t seg_end = it_end < lay_end ? it_end : lay_end;

    // ---- stage this layer's query chunk in fragment order, then its inverse norms
    __syncthreads();
    const uint16_t* qbase = qr + (((int64_t)layer * B + b) * T) * kRow;
    for (int f = tid; f < kHeads * 4 * 4 * 64; f += kWG) {
      const int fl = f & 63, nt = (f >> 6) & 3, s = (f >> 8) & 3, h = f >> 10;
      const int tok = t_base + nt * 16 + (fl & 15);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (nt < NT && tok < T)
        v = *reinterpret_cast<const uint4*>(qbase + (int64_t)tok * kRow + h * kDim + s * 32 + (fl >> 4) * 8);
      q_lds[f] = v;
    }
    __syncthreads();
    {
      const int h = tid >> 6, tt = tid & 63;   // 512 threads = 8 heads x 64 tokens
      const int nt = tt >> 4;
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          uint4 w = q_lds[((h * 4 + s) * 4 + nt) * 64 + gg * 16 + (tt & 15)];
          const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float a = bf16_lo(p[e]), c = bf16_hi(p[e]);
            ss += a * a + c * c;
          }
        }
      rq_lds[h * kTokChunk + tt] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
    }
    __syncthreads();

    const uint4* kt = krt + (int64_t)layer * tiles * kTileU4;
    const float4* kn = krn + (int64_t)layer * tiles * (kHeads * 4);
    uint32_t* lcodes = codes + ((int64_t)layer * B + b) * n_docs;

    for (int64_t it = seg + wave; it < seg_end; it += kWaves) {
      const int64_t wt = it - (int64_t)layer * n_wt;
      const int64_t tau0 = 2 * wt;
      const bool has1 = (tau0 + 1) < tiles;
      const int64_t blk_lane = tau0 * kTile + lane;
      const int32_t doc = (lane < 32 && blk_lane < tiles * kTile) ? blk_doc[blk_lane] : -1;

      f32x4 tot[2][NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) tot[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

      uint4 a_cur[2][4];
      float4 n_cur[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bool ok = mt == 0 || has1;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          a_cur[mt][s] = ok ? kt[(tau0 + mt) * kTileU4 + 0 * kHeadU4 + s * 64 + lane] : make_uint4(0, 0, 0, 0);
        n_cur[mt] = ok ? kn[((tau0 + mt) * kHeads + 0) * 4 + g] : make_float4(1.f, 1.f, 1.f, 1.f);
      }

#pragma unroll 1
      for (int h = 0; h < kHeads; ++h) {
        uint4 a_nxt[2][4];
        float4 n_nxt[2];
        if (h + 1 < kHeads) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bool ok = mt == 0 || has1;
#pragma unroll
            for (int s = 0; s < 4; ++s)
              a_nxt[mt][s] = ok ? kt[(tau0 + mt) * kTileU4 + (h + 1) * kHeadU4 + s * 64 + lane]
                                : make_uint4(0, 0, 0, 0);
            n_nxt[mt] = ok ? kn[((tau0 + mt) * kHeads + h + 1) * 4 + g] : make_float4(1.f, 1.f, 1.f, 1.f);
          }
        }

        f32x4 acc[2][NT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const bf16x8 bq = as_bf16x8(q_lds[((h * 4 + s) * 4 + nt) * 64 + lane]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_cur[mt][s]), bq, acc[mt][nt],
                                                                     0, 0, 0);
          }
        }
        float rq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) rq[nt] = rq_lds[h * kTokChunk + nt * 16 + j];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const float rk[4] = {__builtin_amdgcn_rcpf(fmaxf(n_cur[mt].x, kNormEps)),
                               __builtin_amdgcn_rcpf(fmaxf(n_cur[mt].y, kNormEps)),
                               __builtin_amdgcn_rcpf(fmaxf(n_cur[mt].z, kNormEps)),
                               __builtin_amdgcn_rcpf(fmaxf(n_cur[mt].w, kNormEps))};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) tot[mt][nt][q] += acc[mt][nt][q] * (rq[nt] * rk[q]);
        }
        if (h + 1 < kHeads) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int s = 0; s < 4; ++s) a_cur[mt][s] = a_nxt[mt][s];
            n_cur[mt] = n_nxt[mt];
          }
        }
      }

      // max over this chunk's valid tokens, then over the 16 token lanes of each row
      float m[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = -__builtin_huge_valf();
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if (t_base + nt * 16 + j < T) v = fmaxf(v, tot[mt][nt][q]);
          m[mt][q] = row16_max(v) * 0.125f;   // head mean
        }
      // lane i < 32 takes block i of the wave tile: rows mt*16 + 4*g' + q live in lane 16*g'
      float mine = -__builtin_huge_valf();
      const int src = 16 * ((lane >> 2) & 3);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = __shfl(m[mt][q], src, 64);
          if ((lane >> 4) == mt && (lane & 3) == q) mine = v;
        }
      flush_doc_max(mine, doc, 32, n_docs, lcodes);
    }
    seg = seg_end;
  }
}

// ---------------------------------------------------------------- VALU scan
//
// One wave per 16-block tile: lane l holds block (l & 15) and, per head, the 8-dim
// chunks 4s + (l >> 4); partial dots are summed over the 4 lane groups.
template <int TMAX>
__global__ void __launch_bounds__(256)
route_valu_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, const uint4* __restrict__ krt,
                  const float* __restrict__ krn, int64_t n_blk, int64_t tiles,
                  const int32_t* __restrict__ blk_doc, int32_t n_docs, uint32_t* __restrict__ codes) {
  __shared__ float q_s[TMAX * kRow];
  __shared__ float rq_s[TMAX * kHeads];
  const int layer = blockIdx.z, b = blockIdx.y;
  const int tid = threadIdx.x;
  const uint16_t* qbase = qr + (((int64_t)layer * B + b) * T) * kRow;
  for (int i = tid; i < TMAX * kRow; i += 256) {
    const int t = i / kRow;
    q_s[i] = t < T ? __uint_as_float((uint32_t)qbase[i] << 16) : 0.f;
  }
  __syncthreads();
  if (tid < TMAX * kHeads) {
    const int t = tid / kHeads, h = tid % kHeads;
    float ss = 0.f;
    for (int d = 0; d < kDim; ++d) {
      float a = q_s[t * kRow + h * kDim + d];
      ss += a * a;
    }
    rq_s[tid] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile >= tiles) return;
  const uint4* kt = krt + ((int64_t)layer * tiles + tile) * kTileU4;
  const float* kn = krn + ((int64_t)layer * tiles + tile) * (kHeads * kTile);
  float sc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sc[t] = 0.f;
  for (int h = 0; h < kHeads; ++h) {
    float x[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 w = kt[h * kHeadU4 + s * 64 + lane];
      const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[s * 8 + 2 * e] = bf16_lo(p[e]); x[s * 8 + 2 * e + 1] = bf16_hi(p[e]); }
    }
    const float rk = 1.0f / fmaxf(kn[h * kTile + j], kNormEps);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const float* qv = q_s + t * kRow + h * kDim;
        float d = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) d += x[s * 8 + e] * qv[s * 32 + g * 8 + e];
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        sc[t] += d * (rq_s[t * kHeads + h] * rk);
      }
    }
  }
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int t = 0; t < TMAX; ++t)
    if (t < T) m = fmaxf(m, sc[t]);
  m *= 0.125f;
  const int64_t blk = tile * kTile + lane;
  const int32_t doc = (lane < kTile) ? blk_doc[blk] : -1;
  flush_doc_max(m, doc, kTile, n_docs, codes + ((int64_t)layer * B + b) * n_docs);
}

int choose_ranges(int C, int cus) {
  // R ranges per chunk so that R*C workgroups fill whole waves of one workgroup per CU
  if (C >= cus) return 1;
  int best = 1;
  double best_eff = 0.0;
  for (int R = 1; R <= 64; ++R) {
    const long total = (long)R * C;
    const long waves = (total + cus - 1) / cus;
    const double eff = (double)total / (double)(waves * cus);
    if (eff > best_eff + 1e-9) { best_eff = eff; best = R; }
    if (eff >= 0.999) break;
  }
  return best;
}

}  // namespace

hipError_t launch_blk_doc(const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk, int32_t* blk_doc,
                          hipStream_t s) {
  const int64_t n_pad = route_tiles(n_blk) * kTile;
  if (n_pad == 0) return hipSuccess;
  const int grid = (int)((n_pad + 255) / 256 < 65536 ? (n_pad + 255) / 256 : 65536);
  hipLaunchKernelGGL(blk_doc_kernel, dim3(grid), dim3(256), 0, s, doc_blk_off, n_docs, n_blk, n_pad, blk_doc);
  return hipGetLastError();
}

hipError_t launch_route_scores(int32_t L, const uint16_t* qr, int32_t B, int32_t T, const uint16_t* krt,
                               const float* krn, int64_t n_blk, const int32_t* blk_doc, int32_t n_docs,
                               int32_t accumulate, float* doc_scores, hipStream_t s) {
  const int64_t tiles = route_tiles(n_blk);
  const int64_t n_codes = (int64_t)L * B * n_docs;
  uint32_t* codes = reinterpret_cast<uint32_t*>(doc_scores);
  const DeviceInfo di = device_info();
  const int fill_grid = (int)((n_codes + 255) / 256 < di.cus * 4 ? (n_codes + 255) / 256 : di.cus * 4);

  hipLaunchKernelGGL(codes_init_kernel, dim3(fill_grid), dim3(256), 0, s, codes, n_codes, accumulate);
  if (tiles > 0) {
    if (T >= 16) {
      const int n_tc = (T + kTokChunk - 1) / kTokChunk;
      const int C = B * n_tc;
      const int R = choose_ranges(C, di.cus);
      const int NT = T >= kTokChunk ? 4 : (T + 15) / 16;
      const dim3 grid((unsigned)(R * C));
      const uint4* kt = reinterpret_cast<const uint4*>(krt);
      const float4* kn = reinterpret_cast<const float4*>(krn);
      switch (NT) {
        case 1: hipLaunchKernelGGL(route_mfma_kernel<1>, grid, dim3(kWG), 0, s, qr, B, T, n_tc, kt, kn, n_blk,
                                   tiles, blk_doc, n_docs, L, R, codes); break;
        case 2: hipLaunchKernelGGL(route_mfma_kernel<2>, grid, dim3(kWG), 0, s, qr, B, T, n_tc, kt, kn, n_blk,
                                   tiles, blk_doc, n_docs, L, R, codes); break;
        case 3: hipLaunchKernelGGL(route_mfma_kernel<3>, grid, dim3(kWG), 0, s, qr, B, T, n_tc, kt, kn, n_blk,
                                   tiles, blk_doc, n_docs, L, R, codes); break;
        default: hipLaunchKernelGGL(route_mfma_kernel<4>, grid, dim3(kWG), 0, s, qr, B, T, n_tc, kt, kn, n_blk,
                                    tiles, blk_doc, n_docs, L, R, codes); break;
      }
    } else {
      const dim3 grid((unsigned)((tiles + 3) / 4), (unsigned)B, (unsigned)L);
      hipLaunchKernelGGL(route_valu_kernel<16>, grid, dim3(256), 0, s, qr, B, T,
                         reinterpret_cast<const uint4*>(krt), krn, n_blk, tiles, blk_doc, n_docs, codes);
    }
  }
  hipLaunchKernelGGL(codes_final_kernel, dim3(fill_grid), dim3(256), 0, s, codes, n_codes);
  return hipGetLastError();
}

}  // namespace msa
