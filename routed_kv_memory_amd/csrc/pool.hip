// pool.hip -- A1: segmented 64-token block mean pooling of K, V and Kr, with the
// pooled routing keys written in the route-key tile layout plus their norms.
//
// Method: each document is cut into 64-token blocks on its own grid and every
// block (a final partial one included) is replaced by the mean of its tokens
// (yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 -> 架构; xuqi2024.github.io
// "【MSA】突破100M Token 上下文…", 3.3.2; xiaohongrsx.github.io "MSA paper reading",
// 方法拆解).
//
// One 1024-thread workgroup (16 waves, the whole CU) pools one of the three tensors (K, V or
// Kr) over four consecutive 16-block tiles of one layer; wave w pools blocks w, w + 16, w + 32
// and w + 48 in turn (a launch too small to fill the device takes one tile per workgroup, one
// block per wave).  Lane l owns 16-byte chunks l and 64 + l of each 2 KiB token row, so a row
// is two contiguous 1 KiB wave loads (nontemporal: every input byte is read once), eight tokens
// in flight per step.  Sums are accumulated in fp64: a sum of at most 64 bf16 values is exact
// there unless their magnitudes span more than 2^39, so the mean is the exactly rounded fp64
// quotient, rounded once more to bf16 (nearest-even) straight from fp64.  The tiles' 64 output
// rows (row-major for K-bar and V-bar, the route layout for the routing keys) are staged in LDS
// (128 KiB) and written at the end as one contiguous 128 KiB run with nontemporal stores.
//
// Writes are 1.6% of the bytes but set the pace, and the size of the runs they arrive in
// decides their cost in HBM: on 4 layers of the 1M-token set (22.9 GB per launch) the same
// pooling ran at 0.750 of peak HBM bandwidth with 32 KiB runs (one tile per 256-thread
// workgroup, four per CU), 0.779 with 64 KiB runs (two tiles, 8 waves), 0.823 with 128 KiB runs
// (this layout), and 0.861 with the stores absorbed by the caches (every workgroup writing the
// same 32 KiB, a timing copy).  Ordinary stores issued block by block ran at 0.697.
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

__device__ __forceinline__ void add8(double* acc, uint4 w) {
  acc[0] += (double)bf16_lo(w.x); acc[1] += (double)bf16_hi(w.x);
  acc[2] += (double)bf16_lo(w.y); acc[3] += (double)bf16_hi(w.y);
  acc[4] += (double)bf16_lo(w.z); acc[5] += (double)bf16_hi(w.z);
  acc[6] += (double)bf16_lo(w.w); acc[7] += (double)bf16_hi(w.w);
}

// fp64 -> bf16 bits, round to nearest even, straight from the double (no intermediate
// fp32 rounding).  Finite inputs; beyond the largest finite bf16 gives infinity.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  uint32_t r;
  if (a >= ((uint64_t)(1023 - 126) << 52)) {
    // normal range: keep 7 of the 52 fraction bits, nearest-even on the 45 dropped ones
    // (a carry moves into the exponent), then rebias the exponent from 1023 to 127
    const uint64_t q = (a + ((1ull << 44) - 1) + ((a >> 45) & 1ull)) >> 45;
    r = (uint32_t)(q - ((uint64_t)(1023 - 127) << 7));
    if (r > 0x7F80u) r = 0x7F80u;
  } else {
    // below 2^-126: multiples of 2^-133; the scaling is exact and rint rounds to even
    r = (uint32_t)__builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
  }
  return sign | r;
}

// Rounds acc / n to bf16 and packs 8 values; adds the squares of the rounded values to *ss.
__device__ __forceinline__ uint4 mean8(const double* acc, int32_t n, float* ss) {
  double m[8];
  if (n == kBlockTokens) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = acc[i] * (1.0 / kBlockTokens);   // exact: a power of two
  } else {
    const double dn = (double)n;
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = acc[i] / dn;                     // correctly rounded
  }
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = f64_to_bf16_rne(m[2 * i]);
    const uint32_t hi = f64_to_bf16_rne(m[2 * i + 1]);
    const float a = __uint_as_float(lo << 16), b = __uint_as_float(hi << 16);
    *ss += a * a + b * b;
    p[i] = lo | (hi << 16);
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

constexpr int kU = 8;                      // tokens in flight per wave step

// W waves per workgroup over TPW consecutive 16-block tiles of one tensor and layer, each wave
// pooling blocks wave, wave + W, ...: <16, 4> for large sets (one workgroup per CU, its 128 KiB of
// outputs written as one run), <16, 1> when the launch has too few workgroups to fill the device
// (one block per wave: the time is each wave's chain of loads, not bandwidth).
template <int W, int TPW>
__global__ void __launch_bounds__(64 * W) pool_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                       const uint4* __restrict__ kr, int64_t n_tok,
                                                       const int64_t* __restrict__ tok_off,
                                                       const int64_t* __restrict__ blk_off, int32_t n_docs,
                                                       int64_t n_blk, int64_t tiles, uint4* __restrict__ kbar,
                                                       uint4* __restrict__ vbar, uint4* __restrict__ krt,
                                                       float* __restrict__ krn) {
  constexpr int NB = kTile * TPW;             // blocks of the workgroup
  __shared__ int64_t s_t0[NB];
  __shared__ int32_t s_n[NB];
  __shared__ uint4 s_out[TPW * (kTileElems / 8)];   // the tiles' pooled rows (route layout for Kr)
  const int tensor = (int)(blockIdx.x % 3u);  // 0: K, 1: V, 2: Kr (uniform per workgroup)
  const int64_t tile0 = (int64_t)(blockIdx.x / 3u) * TPW;
  const int64_t layer = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < NB) {
    int64_t blk = tile0 * kTile + tid;
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
  const uint4* src = (tensor == 0 ? k : tensor == 1 ? v : kr) + layer * n_tok * (kRow / 8);
  for (int b = wave; b < NB; b += W) {
    const int64_t t0 = s_t0[b];
    const int32_t n = s_n[b];
    double acc[2][8] = {};
    int32_t t = 0;
    for (; t + kU <= n; t += kU) {
      uint4 w[kU][2];
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) w[u][hh] = ld_nt(src + (t0 + t + u) * (kRow / 8) + hh * 64 + lane);
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) add8(acc[hh], w[u][hh]);
    }
    for (; t < n; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) add8(acc[hh], ld_nt(src + (t0 + t) * (kRow / 8) + hh * 64 + lane));
    const int tl = b / kTile, bl = b % kTile;   // tile of the workgroup, block of the tile
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c16 = hh * 64 + lane;   // chunk of the row: head c16 / 16, dims (c16 % 16) * 8
      float ss = 0.f;
      uint4 o = make_uint4(0, 0, 0, 0);
      if (n > 0) o = mean8(acc[hh], n, &ss);
      if (tensor < 2) {
        s_out[b * (kRow / 8) + c16] = o;
      } else {
        const int h = c16 >> 4, c = c16 & 15;
        s_out[tl * (kTileElems / 8) + h * (kTile * 16) + c * kTile + bl] = o;   // route layout: [h][c][b][8]
        ss = row16_sum(ss);   // the 16 lanes of a DPP row hold the 16 chunks of head h
        if (krn && c == 0 && tile0 + tl < tiles) krn[((layer * tiles + tile0 + tl) * kHeads + h) * kTile + bl] = sqrtf(ss);
      }
    }
  }
  __syncthreads();
  // one contiguous run: the real blocks' rows of K-bar / V-bar, the whole route tiles
  const int64_t nt = tiles - tile0 < TPW ? tiles - tile0 : TPW;
  const int64_t nb = n_blk - tile0 * kTile < NB ? n_blk - tile0 * kTile : NB;
  uint4* out = tensor == 2 ? krt + (layer * tiles + tile0) * (kTileElems / 8)
                           : (tensor == 0 ? kbar : vbar) + (layer * n_blk + tile0 * kTile) * (kRow / 8);
  const int n_out = tensor == 2 ? (int)nt * (kTileElems / 8) : (int)nb * (kRow / 8);
  for (int i = tid; i < n_out; i += 64 * W)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&s_out[i]), reinterpret_cast<u32x4*>(out + i));
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
  if (3 * tiles * (int64_t)L < 4 * (int64_t)stream_cus(s)) {
    hipLaunchKernelGGL((pool_kernel<16, 1>), dim3((unsigned)(3 * tiles), (unsigned)L), dim3(64 * 16), 0, s,
                       reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                       reinterpret_cast<const uint4*>(kr), n_tok, doc_tok_off, doc_blk_off, n_docs, n_blk, tiles,
                       reinterpret_cast<uint4*>(kbar), reinterpret_cast<uint4*>(vbar), reinterpret_cast<uint4*>(krt),
                       krn);
  } else {
    hipLaunchKernelGGL((pool_kernel<16, 4>), dim3((unsigned)(3 * ((tiles + 3) / 4)), (unsigned)L), dim3(64 * 16), 0,
                       s, reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                       reinterpret_cast<const uint4*>(kr), n_tok, doc_tok_off, doc_blk_off, n_docs, n_blk, tiles,
                       reinterpret_cast<uint4*>(kbar), reinterpret_cast<uint4*>(vbar), reinterpret_cast<uint4*>(krt),
                       krn);
  }
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
