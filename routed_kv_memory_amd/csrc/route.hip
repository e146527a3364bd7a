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
// One workgroup per CU, 8 waves: wave h owns KV head h.  It keeps the query
// chunk's head-h fragments (64 tokens x 128 dims, the B operand of
// v_mfma_f32_16x16x32_bf16) and their inverse norms in registers for the whole
// layer, and streams only its own head's 4 KiB of each 16-block route tile (four
// contiguous 1 KiB A-operand fragments), prefetched three tiles ahead in
// registers.  Per tile it scales its 16 blocks x 64 tokens of dot products by
// 1/(|q| |k|) and writes them to LDS; after a barrier, wave n sums the 8 heads for
// token group n, takes the max over its 16 tokens with a DPP row reduction, and
// wave 0 folds the four token groups into per-document maxima.
//
// Accumulator layout (A = 16 blocks x 32 dims, B = 32 dims x 16 tokens): lane l
// holds token (l & 15) and blocks 4*(l >> 4) + r, r = 0..3.
constexpr int kScanWaves = kHeads;              // one wave per KV head
constexpr int kScanWG = kScanWaves * 64;
constexpr int kPrefetch = 3;                     // tiles in flight per wave beyond the current one

__device__ __forceinline__ void lds_barrier() {
  // orders LDS only: in-flight global prefetches stay in flight across the barrier
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NT>
__global__ void __launch_bounds__(kScanWG)
route_mfma_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, int32_t n_tc,
                  const uint4* __restrict__ krt, const float4* __restrict__ krn, int64_t tiles,
                  const int32_t* __restrict__ blk_doc, int32_t n_docs, int32_t L, int32_t R,
                  uint32_t* __restrict__ codes) {
  __shared__ float4 P[2][kScanWaves][NT][64];   // per-head scaled partial scores of one tile
  __shared__ float M[2][4][kTile];               // per token-group block maxima

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
  const int t_base = (cidx % n_tc) * kTokChunk;

  const int64_t W = (int64_t)L * tiles;          // items = (layer, tile)
  const int64_t it_begin = W * r / R;
  const int64_t it_end = W * (r + 1) / R;

  const int wave = threadIdx.x >> 6;             // = head
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int j = lane & 15;

  bf16x8 q[4][NT];       // [s][nt]
  float rq[NT];
  int cur_layer = -1;

  if (it_begin >= it_end) return;   // uniform across the workgroup

  // Prefetch cursor.  Items are consecutive, so the head's fragments and norms of
  // item i sit at a linear offset; loads are unconditional (past the range end the
  // last item is simply fetched again) so that every wait is an exact count.
  const uint4* isrc = krt + it_begin * kTileU4 + wave * kHeadU4 + lane;
  const float4* insrc = krn + (it_begin * kHeads + wave) * 4 + g;
  int64_t itau = it_begin % tiles;
  int64_t inext = it_begin;

  u32x4 kb[kPrefetch + 1][4];
  f32x4 nb[kPrefetch + 1];
  int32_t db[kPrefetch + 1];

  // The route keys and norms are read exactly once: non-temporal loads keep them
  // from displacing useful lines in the caches.
  auto issue = [&](u32x4 (&kbuf)[4], f32x4& nbuf, int32_t& dbuf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kbuf[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(isrc + s * 64));
    nbuf = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(insrc));
    dbuf = blk_doc[itau * kTile + j];
    if (inext + 1 < it_end) {
      ++inext;
      isrc += kTileU4;
      insrc += kHeads * 4;
      itau = (itau + 1 == tiles) ? 0 : itau + 1;
    }
  };

#pragma unroll
  for (int x = 0; x < kPrefetch; ++x) issue(kb[x], nb[x], db[x]);

  // compute cursor
  int layer = (int)(it_begin / tiles);
  int64_t ctau = it_begin - (int64_t)layer * tiles;

  for (int64_t base = it_begin; base < it_end; base += kPrefetch + 1) {
#pragma unroll
    for (int x = 0; x <= kPrefetch; ++x) {
      const int64_t it = base + x;
      constexpr int kNB = kPrefetch + 1;
      issue(kb[(x + kPrefetch) % kNB], nb[(x + kPrefetch) % kNB], db[(x + kPrefetch) % kNB]);
      if (it >= it_end) break;   // uniform across the workgroup

      if (layer != cur_layer) {
        // this layer's query chunk, head `wave`, as B fragments; inverse norms per token
        const uint16_t* qb = qr + (((int64_t)layer * B + b) * T) * kRow + wave * kDim + g * 8;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int tok = t_base + nt * 16 + j;
          float ss = 0.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tok < T) v = *reinterpret_cast<const uint4*>(qb + (int64_t)tok * kRow + s * 32);
            q[s][nt] = as_bf16x8(v);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a = bf16_lo(p[e]), c = bf16_hi(p[e]);
              ss += a * a + c * c;
            }
          }
          ss += __shfl_xor(ss, 16, 64);
          ss += __shfl_xor(ss, 32, 64);
          rq[nt] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
        }
        cur_layer = layer;
      }

      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[x][s]), q[s][nt], acc[nt],
                                                                  0, 0, 0);

      const f32x4 kn4 = nb[x];
      const float rk[4] = {__builtin_amdgcn_rcpf(fmaxf(kn4[0], kNormEps)), __builtin_amdgcn_rcpf(fmaxf(kn4[1], kNormEps)),
                           __builtin_amdgcn_rcpf(fmaxf(kn4[2], kNormEps)), __builtin_amdgcn_rcpf(fmaxf(kn4[3], kNormEps))};
      const int pb = x & 1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float w = rq[nt];
        P[pb][wave][nt][lane] = make_float4(acc[nt][0] * (w * rk[0]), acc[nt][1] * (w * rk[1]),
                                            acc[nt][2] * (w * rk[2]), acc[nt][3] * (w * rk[3]));
      }
      lds_barrier();
      if (wave < NT) {
        float4 tot = P[pb][0][wave][lane];
#pragma unroll
        for (int h = 1; h < kHeads; ++h) {
          const float4 v = P[pb][h][wave][lane];
          tot.x += v.x; tot.y += v.y; tot.z += v.z; tot.w += v.w;
        }
        const bool valid = t_base + wave * 16 + j < T;
        const float ninf = -__builtin_huge_valf();
        const float m0 = row16_max(valid ? tot.x : ninf), m1 = row16_max(valid ? tot.y : ninf);
        const float m2 = row16_max(valid ? tot.z : ninf), m3 = row16_max(valid ? tot.w : ninf);
        if (j == 0) {
          M[pb][wave][4 * g + 0] = m0 * 0.125f;   // head mean
          M[pb][wave][4 * g + 1] = m1 * 0.125f;
          M[pb][wave][4 * g + 2] = m2 * 0.125f;
          M[pb][wave][4 * g + 3] = m3 * 0.125f;
        }
      }
      lds_barrier();
      if (wave == 0) {
        float v = -__builtin_huge_valf();
        if (lane < kTile) {
#pragma unroll
          for (int n = 0; n < NT; ++n) v = fmaxf(v, M[pb][n][lane]);
        }
        flush_doc_max(v, db[x], kTile, n_docs, codes + ((int64_t)layer * B + b) * n_docs);
      }
      if (++ctau == tiles) { ctau = 0; ++layer; }
    }
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
  // R ranges per query chunk; the persistent grid of R*C workgroups (one per CU at a
  // time) should fill whole waves of the device: pick R in [ceil(cus/C), 4*ceil(cus/C)]
  // with the best filled fraction, the smallest R on ties.
  if (C >= cus) return 1;
  const int r0 = (cus + C - 1) / C;
  int best = r0;
  double best_eff = 0.0;
  for (int R = r0; R <= 4 * r0; ++R) {
    const long total = (long)R * C;
    const long waves = (total + cus - 1) / cus;
    const double eff = (double)total / (double)(waves * cus);
    if (eff > best_eff + 1e-9) { best_eff = eff; best = R; }
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
        case 1: hipLaunchKernelGGL(route_mfma_kernel<1>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, kn, tiles,
                                   blk_doc, n_docs, L, R, codes); break;
        case 2: hipLaunchKernelGGL(route_mfma_kernel<2>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, kn, tiles,
                                   blk_doc, n_docs, L, R, codes); break;
        case 3: hipLaunchKernelGGL(route_mfma_kernel<3>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, kn, tiles,
                                   blk_doc, n_docs, L, R, codes); break;
        default: hipLaunchKernelGGL(route_mfma_kernel<4>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, kn, tiles,
                                    blk_doc, n_docs, L, R, codes); break;
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
