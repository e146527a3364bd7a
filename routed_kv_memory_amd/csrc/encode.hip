// encode.hip -- the offline encode front-end: projections of the memory documents'
// hidden rows to K, V and the routing key Kr, the per-head key normalisation and the
// document-wise rotary position, fused with the 64-token block mean pooling.
//
// Method: the layer projects its hidden states with k_proj (then k_norm), v_proj and
// the bias-free router_k_proj to 8 heads x 128 dims (xuqi2024.github.io "【MSA】突破
// 100M Token 上下文…", 5.1 and 5.2 Step 1); keys are rotated with positions that restart
// at 0 in every document (the same page, 3.3.1; yunpan.plus "MSA端到端可训练记忆模型完整
// 开源…", 整体设计 -> 架构); the memory keeps the 64-token block means (3.3.2).
//
// The projections are one GEMM per layer, C = X . W^T with X [tokens][H] and W
// [3 x 8 x 128][H] (both K-contiguous, W as a linear layer stores it), so every MFMA
// operand fragment of v_mfma_f32_16x16x32_bf16 -- 16 rows x 32 k, lane 16 g + j holding
// row j, k 8 g .. 8 g + 7 -- is 16 contiguous bytes per lane in either operand.
//
// Work: one 512-thread workgroup per (4 consecutive blocks = 256 token rows, pair of
// output heads = 256 columns of K, V or Kr).  The hidden dimension is walked in 64-wide
// chunks (two MFMA k steps).  A chunk of the 256 hidden rows and of the 256 weight rows
// (32 KiB each, 128 bytes of every row) reaches LDS by direct global->LDS loads
// (global_load_lds_dwordx4: one wave instruction writes 64 lanes x 16 B contiguously),
// each instruction covering 8 rows x one whole 128-byte line, with no staging registers.
// Within a row the eight 16-byte segments are XOR-permuted by the row's index in its
// group of 8, so that fragment reads (16 rows, one segment each) spread over all banks.
// Two stages of 64 KiB alternate: the next chunk's loads go out right after the barrier
// that publishes the current one, and each wave waits for its own loads of a chunk
// before that barrier.  Wave (wr, wc) accumulates block wr (64 rows) x head wc of the
// pair (128 columns): 4 x 8 accumulator tiles, kept in VGPRs (the library is built with
// MFMA's VGPR form).  The epilogue stays in registers: a row's 128 columns sit in the 16
// lanes of a DPP row (per-row mean square by a row reduction), columns e and e + 64 of a
// head are in the same lane (the rotation needs no exchange), and a block mean is an
// in-lane sum over 16 rows plus a sum over the 4 lane groups.  Workgroups are placed so
// that those an XCD runs together share 4 head pairs' weights and 8 row groups' hidden
// rows through its L2.  Rows past a block's end (or the last token) are loaded from a
// clamped, in-bounds row and never enter a mean.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kEncBlocks = 4;                  // blocks per workgroup (= 256 token rows)
constexpr int kPairs = 3 * kHeads / 2;         // head pairs: K 0-3, V 4-7, Kr 8-11
constexpr int kRunPairs = 4;                   // head pairs in a run of 32 workgroups on one XCD
constexpr int kRunGroups = 32 / kRunPairs;        // row groups in a run
constexpr int kKC = 64;                        // hidden columns per staged chunk (128 B of a row)
constexpr int kRegionKB = 32;                  // per chunk: 256 rows (or columns) x 128 B = 32 KiB
constexpr int kLoadsPerChunk = 8;              // direct-to-LDS loads per wave per chunk
// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// everything retired
constexpr int kWaitAll = 0;
constexpr double kInv2Pi = 0.15915494309189533577;

__device__ __forceinline__ int32_t find_doc(const int64_t* __restrict__ off, int32_t n, int64_t x) {
  int32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(512)
encode_kernel(int32_t H, const uint16_t* __restrict__ x, int64_t n_tok, const uint16_t* __restrict__ w_k,
              const uint16_t* __restrict__ w_v, const uint16_t* __restrict__ w_kr,
              const uint16_t* __restrict__ w_norm, float eps, double log2_theta,
              const int64_t* __restrict__ tok_off, const int64_t* __restrict__ blk_off, int32_t n_docs,
              int64_t n_blk, int64_t tiles, int64_t n_groups, uint16_t* __restrict__ kbar,
              uint16_t* __restrict__ vbar, uint16_t* __restrict__ krt, float* __restrict__ krn) {
  // two stages of one chunk each: rows region (32 KiB) then columns region (32 KiB).  Inside a
  // region, load d (d = 0..31) holds rows 8 d .. 8 d + 7: lane l of the load holds 16-byte
  // segment (l & 7) ^ (l >> 3) of row 8 d + (l >> 3), i.e. row r' = l >> 3 keeps its eight
  // segments XOR-permuted by r', so the loads read whole 128-byte lines and the fragment reads
  // (16 rows, one segment each) spread over all banks.  Two arrays, so that the compiler
  // sees which stage each access touches.
  __shared__ u32x4 stage0[2 * kRegionKB * 64], stage1[2 * kRegionKB * 64];
  __shared__ int64_t s_t0[kEncBlocks], s_pos[kEncBlocks];
  __shared__ int32_t s_n[kEncBlocks];

  // XCD-aware placement (workgroup i runs on XCD i % 8).  An XCD takes the row groups
  // grp = 8 r + xcd; its workgroups come in runs of 32 (about what its 32 CUs hold at once)
  // covering 8 of its row groups x 4 head pairs of one output, so that while they run
  // together each pair's weights are read by 8 workgroups and each row group's hidden rows
  // by 4, from the XCD's L2.  The three outputs' runs over the same 8 row groups follow
  // each other.
  const int64_t i = blockIdx.x;
  const int xcd = (int)(i & 7);
  const int64_t slot = i >> 3;
  const int64_t run = slot / 32, within = slot % 32;
  const int64_t grp = ((run / (kPairs / kRunPairs)) * kRunGroups + within / kRunPairs) * 8 + xcd;
  const int pair = (int)((run % (kPairs / kRunPairs)) * kRunPairs + within % kRunPairs);
  if (grp >= n_groups) return;                 // uniform
  const int out = pair / 4;                    // 0 K, 1 V, 2 Kr
  const int head0 = 2 * (pair % 4);
  const int64_t layer = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;

  if (tid < kEncBlocks) {
    const int64_t blk = grp * kEncBlocks + tid;
    int64_t t0 = 0, pos = 0;
    int32_t n = 0;
    if (blk < n_blk) {
      const int32_t d = find_doc(blk_off, n_docs, blk);
      const int64_t jb = blk - blk_off[d];
      const int64_t s = tok_off[d], e = tok_off[d + 1];
      t0 = s + (int64_t)kBlockTokens * jb;
      int64_t t1 = t0 + kBlockTokens < e ? t0 + kBlockTokens : e;
      if (t0 < 0) t0 = 0;
      if (t1 > n_tok) t1 = n_tok;
      n = t1 > t0 ? (int32_t)(t1 - t0) : 0;
      if (t0 > n_tok - 1) t0 = n_tok - 1;
      pos = (int64_t)kBlockTokens * jb;         // position of the block's first token in its document
    }
    s_t0[tid] = t0;
    s_n[tid] = n;
    s_pos[tid] = pos;
  }
  __syncthreads();

  // this wave's loads: d = wave + 8 q (q = 0..3) of the rows region (token rows 8 d + (lane >> 3))
  // and of the columns region (output columns 8 d + (lane >> 3) of the pair)
  const int seg = (lane & 7) ^ ((lane >> 3) & 7);
  const uint16_t* xrow[4];
  const uint16_t* wrow[4];
  {
    const uint16_t* xl = x + layer * n_tok * (int64_t)H;
    const uint16_t* wsel = out == 0 ? w_k : (out == 1 ? w_v : w_kr);
    const uint16_t* wl = wsel + layer * (int64_t)kRow * H;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * (wave + 8 * q) + (lane >> 3);      // 0..255
      int64_t t = s_t0[r >> 6] + (r & 63);
      if (t > n_tok - 1) t = n_tok - 1;
      xrow[q] = xl + t * (int64_t)H + 8 * seg;
      const int col = (head0 + (r >> 7)) * kDim + (r & 127);
      wrow[q] = wl + (int64_t)col * H + 8 * seg;
    }
  }
  typedef __attribute__((address_space(1))) const void* gptr_t;
  typedef __attribute__((address_space(3))) void* lptr_t;
  auto stage_of = [&](int st) -> u32x4* { return st == 0 ? stage0 : stage1; };   // st constant after unrolling
  auto issue = [&](int c, int st) {          // chunk c -> stage st = c % 2
    u32x4* sp = stage_of(st);
    const int kc = c * kKC;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_global_load_lds((gptr_t)(xrow[q] + kc), (lptr_t)(sp + (wave + 8 * q) * 64), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(wrow[q] + kc), (lptr_t)(sp + (kRegionKB + wave + 8 * q) * 64),
                                       16, 0, 0);
    }
  };
  // fragment (16 rows from row0, k segment s of 8) of a region, as this lane's 16 bytes:
  // lane (g, j) takes row row0 + j, which sits in load (row0 + j) >> 3 at lane 8 (j & 7) + (s ^ (j & 7))
  auto frag = [&](const u32x4* region, int row0, int s) {
    const int r = row0 + j;
    return __builtin_bit_cast(bf16x8, region[(r >> 3) * 64 + 8 * (j & 7) + (s ^ (j & 7))]);
  };

  const int wr = wave & 3, wc = wave >> 2;
  f32x4 acc[4][8];   // rows 16 m + 4 g + r of block wr, columns 16 n + j of head head0 + wc
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_chunks = H / kKC;                // even (H % 128 == 0)
  // one chunk: wait for this wave's loads of it (and lgkmcnt(0): this wave's reads of the other
  // stage are retired), barrier (chunk c is in its stage for every wave, and every wave is done
  // reading chunk c - 1), load chunk c + 1 into chunk c - 1's stage, multiply chunk c.  No
  // branch: past the end the loads repeat the last chunk (never read), so every wait is exact.
  auto step = [&](int c, int st) {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    asm volatile("s_barrier" ::: "memory");  // the clobber keeps every LDS access on its side
    issue(min(c + 1, n_chunks - 1), st ^ 1);
    __builtin_amdgcn_sched_barrier(0);       // keep the loads ahead of the products (no sinking)
    const u32x4* sp = stage_of(st);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 af[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) af[m] = frag(sp, 64 * wr + 16 * m, 4 * h + g);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const bf16x8 bf = frag(sp + kRegionKB * 64, 128 * wc + 16 * n, 4 * h + g);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bf, acc[m][n], 0, 0, 0);
      }
    }
  };
  issue(0, 0);
  for (int c = 0; c < n_chunks; c += 2) {
    step(c, 0);
    step(c + 1, 1);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);        // the repeated loads land before the LDS is released

  // epilogue, row by row: the key's per-row RMS normalisation (the 16 lanes of a DPP row
  // hold the row's 128 columns, 8 per lane), norm weight and rotation of pairs (c, c + 64),
  // then the block sum over valid rows, in-lane over the lane's 16 rows and over the 4 lane
  // groups; the rotation angle p * theta^(-e/64) is formed and reduced to a fraction of a
  // turn in fp64 (the positions of long documents would otherwise lose it to fp32 rounding)
  const int head = head0 + wc;
  const int64_t blk = grp * kEncBlocks + wr;
  const int32_t nv = s_n[wr];
  float wn[8];
  double fturn[4];
  if (out == 0) {
#pragma unroll
    for (int n = 0; n < 8; ++n) wn[n] = bf16_lo(w_norm[layer * kDim + 16 * n + j]);
#pragma unroll
    for (int n = 0; n < 4; ++n) fturn[n] = exp2(-(double)(16 * n + j) * (1.0 / 64.0) * log2_theta) * kInv2Pi;
  }
  float sum[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) sum[n] = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * m + 4 * g + r;        // within the block
      float v[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) v[n] = acc[m][n][r];
      if (out == 0) {
        float ss = 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) ss += v[n] * v[n];
        ss = row16_sum(ss);
        const float inv = 1.0f / sqrtf(ss * (1.0f / kDim) + eps);
        const double p = (double)s_pos[wr] + (double)row;
#pragma unroll
        for (int n = 0; n < 4; ++n) {        // pair (16 n + j, 16 n + j + 64)
          const double turns = p * fturn[n];
          const float half_turns = (float)(2.0 * (turns - rint(turns)));   // angle / pi in [-1, 1]
          float sn, cs;
          sincospif(half_turns, &sn, &cs);
          const float a = v[n] * inv * wn[n], c = v[n + 4] * inv * wn[n + 4];
          v[n] = a * cs - c * sn;
          v[n + 4] = c * cs + a * sn;
        }
      }
      const bool valid = row < nv;
#pragma unroll
      for (int n = 0; n < 8; ++n) sum[n] += valid ? v[n] : 0.f;
    }
  const float inv_n = nv > 0 ? 1.0f / (float)nv : 0.f;
  float mean[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) mean[n] = rows4_sum(sum[n]) * inv_n;
  // lane group g writes the columns of n = 2 g, 2 g + 1
  if (out < 2) {
    if (blk < n_blk) {
      uint16_t* dst = (out == 0 ? kbar : vbar) + ((layer * n_blk + blk) * kHeads + head) * kDim;
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int n = 2 * g + e2;
        dst[16 * n + j] = (uint16_t)f32_to_bf16_rne(mean[n]);
      }
    }
  } else {
    // route layout: [layer][tile][h][c][b][8]; padding blocks of the last tile get zeros
    const int64_t tile = blk / kTile;
    const int b = (int)(blk % kTile);
    float ssr = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int n = 2 * g + e2;
      const int col = 16 * n + j;
      const uint32_t bits = blk < n_blk ? f32_to_bf16_rne(mean[n]) : 0u;
      if (tile < tiles)
        krt[(((layer * tiles + tile) * kHeads + head) * (kTile * 16) + (col >> 3) * kTile + b) * 8 + (col & 7)] =
            (uint16_t)bits;
      const float vr = __uint_as_float(bits << 16);
      ssr += vr * vr;
    }
    if (krn && tile < tiles) {
      ssr = row16_sum(ssr);                      // the lane group's 32 columns
      ssr = rows4_sum(ssr);                      // all 128
      if (lane == 0) krn[((layer * tiles + tile) * kHeads + head) * kTile + b] = sqrtf(ssr);
    }
  }
}

}  // namespace

hipError_t launch_encode(int32_t L, int32_t H, const uint16_t* x, int64_t n_tok, const uint16_t* w_k,
                         const uint16_t* w_v, const uint16_t* w_kr, const uint16_t* w_norm, float eps, float theta,
                         const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                         uint16_t* kbar, uint16_t* vbar, uint16_t* krt, float* krn, hipStream_t s) {
  const int64_t tiles = route_tiles(n_blk);
  if (tiles == 0) return hipSuccess;
  // every block of every tile (padding blocks included, so the route layout is complete)
  const int64_t n_groups = tiles * kTile / kEncBlocks;
  const int64_t groups_per_xcd = ((n_groups + 7) / 8 + kRunGroups - 1) / kRunGroups * kRunGroups;   // whole runs
  const dim3 grid((unsigned)(8 * groups_per_xcd * kPairs), (unsigned)L);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(512), 0, s, H, x, n_tok, w_k, w_v, w_kr, w_norm, eps,
                     log2((double)theta), doc_tok_off, doc_blk_off, n_docs, n_blk, tiles, n_groups, kbar, vbar,
                     krt, krn);
  return hipGetLastError();
}

}  // namespace msa
