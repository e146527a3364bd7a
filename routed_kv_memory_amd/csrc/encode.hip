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
// Layout of the work: one 256-thread workgroup per (4 consecutive blocks, output
// head) where an output head is 128 columns of K, V or Kr; wave w owns block w
// (64 token rows, zero-padded past the block's end) and all 128 columns, as 4 x 8
// accumulator tiles of v_mfma_f32_16x16x32_bf16.  The hidden dimension is walked in
// 32-wide chunks: the 4 blocks' rows and the weight slice are staged in LDS (double
// buffered, the next chunk's loads issued before the current one is used).  Hidden
// rows are the A operand (16-byte LDS reads); the weights, stored input-major, reach
// the B operand through LDS transposed reads (ds_read_b64_tr_b16).  The epilogue
// stays in registers: the key's per-row mean square is a cross-lane sum over the 16
// lanes of a DPP row, columns e and e + 64 of a head sit in the same lane so the
// rotation needs no exchange, and the block mean is an in-lane sum over 16 rows plus
// a row-swap sum over the four lane groups.  The 24 workgroups of a block group run on
// one XCD, so its L2 serves their common hidden rows.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kEncBlocks = 4;                  // blocks (= waves) per workgroup
constexpr int kEncRows = kEncBlocks * kBlockTokens;
constexpr int kKC = 32;                        // hidden columns per chunk (one MFMA k step)
constexpr int kAStride = kKC + 8;              // bf16 per staged hidden row
constexpr int kBStride = kDim + 8;             // bf16 per staged weight row (128 output columns)
constexpr int kHeadOutputs = 3 * kHeads;       // K, V and Kr heads
constexpr double kInv2Pi = 0.15915494309189533577;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the
// 8-byte chunks addressed by lanes 4 e + i / 4 (e = 0..3).
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ int32_t find_doc(const int64_t* __restrict__ off, int32_t n, int64_t x) {
  int32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(256)
encode_kernel(int32_t H, const uint16_t* __restrict__ x, int64_t n_tok, const uint16_t* __restrict__ w_k,
              const uint16_t* __restrict__ w_v, const uint16_t* __restrict__ w_kr,
              const uint16_t* __restrict__ w_norm, float eps, double log2_theta,
              const int64_t* __restrict__ tok_off, const int64_t* __restrict__ blk_off, int32_t n_docs,
              int64_t n_blk, int64_t tiles, int64_t n_groups, uint16_t* __restrict__ kbar,
              uint16_t* __restrict__ vbar, uint16_t* __restrict__ krt, float* __restrict__ krn) {
  __shared__ uint16_t a_s[2][kEncRows * kAStride];
  __shared__ uint16_t b_s[2][kKC * kBStride];
  __shared__ int64_t s_t0[kEncBlocks], s_pos[kEncBlocks];
  __shared__ int32_t s_n[kEncBlocks];

  // XCD-aware placement: the 24 output heads of a block group share the XCD of the group
  const int64_t i = blockIdx.x;
  const int xcd = (int)(i & 7);
  const int64_t slot = i >> 3;
  const int64_t grp = (slot / kHeadOutputs) * 8 + xcd;
  const int ho = (int)(slot % kHeadOutputs);
  if (grp >= n_groups) return;                 // uniform
  const int out = ho / kHeads, head = ho % kHeads;
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
      pos = (int64_t)kBlockTokens * jb;         // position of the block's first token in its document
    }
    s_t0[tid] = t0;
    s_n[tid] = n;
    s_pos[tid] = pos;
  }
  __syncthreads();

  const uint16_t* xl = x + layer * n_tok * (int64_t)H;
  const uint16_t* wsel = out == 0 ? w_k : (out == 1 ? w_v : w_kr);
  const uint16_t* wl = wsel + layer * (int64_t)H * kRow + head * kDim;

  // chunk loader: A = 256 rows x 4 x 16 B, B = 32 k-rows x 16 x 16 B
  uint4 pa[4], pb[2];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + q * 256;
      const int r = u >> 2, c = u & 3;
      const int w = r >> 6, rr = r & 63;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < s_n[w]) v = *reinterpret_cast<const uint4*>(xl + (s_t0[w] + rr) * (int64_t)H + kc + 8 * c);
      pa[q] = v;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + q * 256;
      const int kk = u >> 4, c = u & 15;
      pb[q] = *reinterpret_cast<const uint4*>(wl + (int64_t)(kc + kk) * kRow + 8 * c);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + q * 256;
      const int r = u >> 2, c = u & 3;
      *reinterpret_cast<uint4*>(a_s[buf] + r * kAStride + 8 * c) = pa[q];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + q * 256;
      const int kk = u >> 4, c = u & 15;
      *reinterpret_cast<uint4*>(b_s[buf] + kk * kBStride + 8 * c) = pb[q];
    }
  };

  f32x4 acc[4][8];   // rows 16 mt + 4 g + r of block `wave`, columns 16 nt + j of the head
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_chunk(0);
  store_chunk(0);
  int buf = 0;
  // B operand source: lane j of lane group g points at columns 16 nt + 4 (j & 3) .. +3 of
  // k-row 8 g + (j >> 2) (first four k) and of k-row 8 g + 4 + (j >> 2) (last four k)
  const int bsrc = (8 * g + (j >> 2)) * kBStride + 4 * (j & 3);
  for (int kc = 0; kc < H; kc += kKC, buf ^= 1) {
    __syncthreads();   // chunk kc is in buf; every reader of buf ^ 1 is done
    if (kc + kKC < H) load_chunk(kc + kKC);
    bf16x8 af[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      af[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              a_s[buf] + (wave * kBlockTokens + 16 * mt + j) * kAStride + 8 * g));
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint2 b0 = lds_read_tr16(b_s[buf] + bsrc + 16 * nt);
      const uint2 b1 = lds_read_tr16(b_s[buf] + bsrc + 4 * kBStride + 16 * nt);
      const bf16x8 bf = __builtin_bit_cast(bf16x8, (u32x4{b0.x, b0.y, b1.x, b1.y}));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf, acc[mt][nt], 0, 0, 0);
    }
    if (kc + kKC < H) store_chunk(buf ^ 1);
  }

  const int64_t blk = grp * kEncBlocks + wave;
  const int32_t n = s_n[wave];
  if (out == 0) {
    // key: per-row RMS normalisation (the 16 lanes of a DPP row hold the row's 128
    // columns, 8 per lane), norm weight, then the rotation of pairs (c, c + 64)
    float wn[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) wn[nt] = bf16_lo(w_norm[layer * kDim + 16 * nt + j]);
    // angle p * theta^(-e/64) formed and reduced to a fraction of a turn in fp64 (the
    // positions of long documents would otherwise lose the angle to fp32 rounding)
    double fturn[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) fturn[nt] = exp2(-(double)(16 * nt + j) * (1.0 / 64.0) * log2_theta) * kInv2Pi;
    const double pos0 = (double)s_pos[wave];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) ss += acc[mt][nt][r] * acc[mt][nt][r];
        ss = row16_sum(ss);
        const float inv = 1.0f / sqrtf(ss * (1.0f / kDim) + eps);
        const double p = pos0 + (double)(16 * mt + 4 * g + r);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {       // pair (16 nt + j, 16 nt + j + 64)
          const double turns = p * fturn[nt];
          const float half_turns = (float)(2.0 * (turns - rint(turns)));   // angle / pi in [-1, 1]
          float sn, cs;
          sincospif(half_turns, &sn, &cs);
          const float a = acc[mt][nt][r] * inv * wn[nt], c = acc[mt][nt + 4][r] * inv * wn[nt + 4];
          acc[mt][nt][r] = a * cs - c * sn;
          acc[mt][nt + 4][r] = c * cs + a * sn;
        }
      }
  }
  // block mean: in-lane over the lane's 16 rows (valid ones), then over the 4 lane groups
  float mean[8];
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.f;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * mt + 4 * g + r < n) sum += acc[mt][nt][r];
    mean[nt] = rows4_sum(sum) * inv_n;
  }
  // every lane now holds the 8 column means of its j; lane group g writes nt = 2 g, 2 g + 1
  if (blk < n_blk) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = 2 * g + q;
      const int col = 16 * nt + j;
      const uint16_t bits = (uint16_t)f32_to_bf16_rne(mean[nt]);
      if (out == 0) kbar[((layer * n_blk + blk) * kHeads + head) * kDim + col] = bits;
      else if (out == 1) vbar[((layer * n_blk + blk) * kHeads + head) * kDim + col] = bits;
    }
  }
  if (out == 2) {
    // route layout: [layer][tile][h][c][b][8]; padding blocks of the last tile get zeros
    const int64_t tile = blk / kTile;
    const int b = (int)(blk % kTile);
    float ssr = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = 2 * g + q;
      const int col = 16 * nt + j;
      const uint32_t bits = blk < n_blk ? f32_to_bf16_rne(mean[nt]) : 0u;
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
  const int64_t groups8 = (n_groups + 7) / 8 * 8;
  const dim3 grid((unsigned)(groups8 * kHeadOutputs), (unsigned)L);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(256), 0, s, H, x, n_tok, w_k, w_v, w_kr, w_norm, eps,
                     log2((double)theta), doc_tok_off, doc_blk_off, n_docs, n_blk, tiles, n_groups, kbar, vbar, krt, krn);
  return hipGetLastError();
}

}  // namespace msa
