// decode.hip -- A5: one decode token of grouped-query attention over
// [memory context ; local KV], split over rows with an online softmax, then merged.
//
// Method: the decode token attends to the Top-k documents' compressed K/V
// followed by the query's local K/V, with no mask; the memory part is fixed and
// only the local part grows (yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 ->
// 架构; xuqi2024.github.io "【MSA】突破100M Token 上下文…", 5.2; xiaohongrsx.github.io
// "MSA paper reading", 推理全流程).
//
// Layout of the work: one workgroup per (row split, KV head, layer x query) with
// one wave per query head of the KV head's group.  Each 64-row tile of the KV
// head's K and V slices is staged in LDS with coalesced 16-byte loads, and the
// next tile's loads are issued before the current tile is used.  Scores: lane =
// row, a wave-wide online-softmax update per tile (DPP and row-swap reductions).
// P.V: lane (g, j) sums rows 16 g .. 16 g + 15 into dims 8 j .. 8 j + 7 with
// 16-byte LDS reads; the four row groups are summed once at the end.  Partial
// (max, sum, acc) per split go to the workspace and a second kernel merges the
// splits in one pass.  All accumulation is fp32.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kRowsPerSplit = 256;
constexpr int kTileRows = 64;
constexpr int kKStride = kDim + 8;   // bf16 per staged K row (16-byte pad against bank conflicts)

template <int G>
__global__ void __launch_bounds__(64 * G)
decode_split_kernel(int32_t Hq, const uint16_t* __restrict__ q, const uint16_t* __restrict__ ctx_k,
                    const uint16_t* __restrict__ ctx_v, const int32_t* __restrict__ ctx_len, int32_t max_ctx,
                    const uint16_t* __restrict__ loc_k, const uint16_t* __restrict__ loc_v,
                    const int32_t* __restrict__ loc_len, int32_t max_loc, float scale, int32_t n_splits,
                    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  __shared__ uint16_t k_s[kTileRows * kKStride];
  __shared__ uint16_t v_s[kTileRows * kDim];
  __shared__ float q_s[G * kDim];
  __shared__ float p_s[G * kTileRows];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int64_t lb = blockIdx.z;
  const int tid = threadIdx.x;
  const int hh = tid >> 6;       // query head within the group (= wave)
  const int lane = tid & 63;
  constexpr int NT = 64 * G;

  int32_t clen = ctx_len[lb];
  clen = clen < 0 ? 0 : (clen > max_ctx ? max_ctx : clen);
  int32_t llen = 0;
  if (max_loc > 0) {
    llen = loc_len[lb];
    llen = llen < 0 ? 0 : (llen > max_loc ? max_loc : llen);
  }
  const int32_t n_rows = clen + llen;
  const int32_t r_begin = split * kRowsPerSplit;
  const int32_t r_end = min(n_rows, r_begin + kRowsPerSplit);

  for (int i = tid; i < G * kDim; i += NT) {
    const int h = i / kDim, d = i % kDim;
    q_s[i] = __uint_as_float((uint32_t)q[(lb * Hq + kvh * G + h) * kDim + d] << 16);
  }

  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  // P.V ownership: lane (g, j) = (lane >> 4, lane & 15) sums rows 16 g .. 16 g + 15 of
  // each tile into dims 8 j .. 8 j + 7; the four row groups are summed at the end.
  const int pg = lane >> 4, pj = lane & 15;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* ck = ctx_k + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* cv = ctx_v + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* lk = loc_k + (lb * (int64_t)max_loc) * kRow + kvh * kDim;
  const uint16_t* lv = loc_v + (lb * (int64_t)max_loc) * kRow + kvh * kDim;

  // Tile loader: 64 rows x 16 chunks of 16 B for K and for V, kPer chunks per thread.
  constexpr int kPer = kTileRows * 16 / NT;
  uint4 pk[kPer], pv[kPer];
  auto load_tile = [&](int32_t t0) {
    const int32_t nr = min(kTileRows, r_end - t0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * NT;
      const int rr = u >> 4, c = u & 15;
      uint4 kw = make_uint4(0, 0, 0, 0), vw = kw;
      if (rr < nr) {
        const int32_t row = t0 + rr;
        const uint16_t* ks = row < clen ? ck + (int64_t)row * kRow : lk + (int64_t)(row - clen) * kRow;
        const uint16_t* vs = row < clen ? cv + (int64_t)row * kRow : lv + (int64_t)(row - clen) * kRow;
        kw = *reinterpret_cast<const uint4*>(ks + c * 8);
        vw = *reinterpret_cast<const uint4*>(vs + c * 8);
      }
      pk[i] = kw;
      pv[i] = vw;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * NT;
      const int rr = u >> 4, c = u & 15;
      *reinterpret_cast<uint4*>(k_s + rr * kKStride + c * 8) = pk[i];
      *reinterpret_cast<uint4*>(v_s + rr * kDim + c * 8) = pv[i];
    }
  };

  if (r_begin < r_end) load_tile(r_begin);
  for (int32_t t0 = r_begin; t0 < r_end; t0 += kTileRows) {
    const int32_t nr = min(kTileRows, r_end - t0);
    __syncthreads();   // the previous tile's readers are done
    store_tile();
    __syncthreads();
    // the next tile's loads stay in flight while this one is scored
    if (t0 + kTileRows < r_end) load_tile(t0 + kTileRows);
    // scores: lane = row
    float s = -__builtin_huge_valf();
    if (lane < nr) {
      const uint4* kr = reinterpret_cast<const uint4*>(k_s + lane * kKStride);
      const float4* qv = reinterpret_cast<const float4*>(q_s + hh * kDim);
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 w = kr[c];
        const float4 qa = qv[2 * c], qb = qv[2 * c + 1];
        d += bf16_lo(w.x) * qa.x + bf16_hi(w.x) * qa.y + bf16_lo(w.y) * qa.z + bf16_hi(w.y) * qa.w;
        d += bf16_lo(w.z) * qb.x + bf16_hi(w.z) * qb.y + bf16_lo(w.w) * qb.z + bf16_hi(w.w) * qb.w;
      }
      s = d * scale;
    }
    const float m_tile = rows4_max(row16_max(s));
    const float m_new = fmaxf(m_run, m_tile);          // finite: the tile has >= 1 row
    const float alpha = __expf(m_run - m_new);          // 0 when m_run = -inf
    const float p = lane < nr ? __expf(s - m_new) : 0.f;   // rows past the tile's end weigh 0
    l_run = l_run * alpha + rows4_sum(row16_sum(p));
    m_run = m_new;
    p_s[hh * kTileRows + lane] = p;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    const float4* pp = reinterpret_cast<const float4*>(p_s + hh * kTileRows + 16 * pg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 pr4 = pp[i];
      const float prs[4] = {pr4.x, pr4.y, pr4.z, pr4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // rows past the tile's end were staged as zeros and carry p = 0
        const uint4 w = *reinterpret_cast<const uint4*>(v_s + (16 * pg + 4 * i + r) * kDim + 8 * pj);
        const float pr = prs[r];
        acc[0] += pr * bf16_lo(w.x); acc[1] += pr * bf16_hi(w.x);
        acc[2] += pr * bf16_lo(w.y); acc[3] += pr * bf16_hi(w.y);
        acc[4] += pr * bf16_lo(w.z); acc[5] += pr * bf16_hi(w.z);
        acc[6] += pr * bf16_lo(w.w); acc[7] += pr * bf16_hi(w.w);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = rows4_sum(acc[e]);
  const int64_t part = ((lb * kHeads + kvh) * n_splits + split) * G + hh;
  if (lane == 0) {
    ws_ml[2 * part] = m_run;
    ws_ml[2 * part + 1] = l_run;
  }
  if (pg == 0) {
    float4* dst = reinterpret_cast<float4*>(ws_acc + part * kDim + 8 * pj);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

__global__ void __launch_bounds__(256)
decode_merge_kernel(int32_t Hq, int32_t G, int32_t n_splits, const float* __restrict__ ws_ml,
                    const float* __restrict__ ws_acc, float* __restrict__ out) {
  const int64_t lb = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;   // (hq, d)
  if (i >= Hq * kDim) return;
  const int hq = i / kDim, d = i % kDim;
  const int kvh = hq / G, hh = hq % G;
  // one pass with a running maximum over batches of 8 splits (their loads are
  // independent); empty splits carry (max = -inf, sum = 0)
  const float ninf = -__builtin_huge_valf();
  float M = ninf, num = 0.f, den = 0.f;
  const int64_t part0 = (lb * kHeads + kvh) * n_splits * G + hh;
  for (int s0 = 0; s0 < n_splits; s0 += 8) {
    float m[8], l[8], a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t part = part0 + (int64_t)(s0 + u) * G;
      const bool ok = s0 + u < n_splits;
      m[u] = ok ? ws_ml[2 * part] : ninf;
      l[u] = ok ? ws_ml[2 * part + 1] : 0.f;
      a[u] = ok ? ws_acc[part * kDim + d] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, m[u]);
    if (Mn == ninf) continue;
    const float c = __expf(M - Mn);   // 0 while M = -inf
    num *= c;
    den *= c;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = __expf(m[u] - Mn);   // 0 for empty splits
      num += w * a[u];
      den += w * l[u];
    }
    M = Mn;
  }
  out[(lb * Hq + hq) * kDim + d] = den > 0.f ? num / den : 0.f;
}

}  // namespace

int decode_rows_per_split() { return kRowsPerSplit; }

hipError_t launch_decode(int32_t L, int32_t B, int32_t Hq, const uint16_t* q, const uint16_t* ctx_k,
                         const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx, const uint16_t* loc_k,
                         const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc, float scale, float* out,
                         void* ws, hipStream_t s) {
  const int G = Hq / kHeads;
  const int32_t n_splits = (max_ctx + max_loc + kRowsPerSplit - 1) / kRowsPerSplit;
  const int64_t parts = (int64_t)L * B * kHeads * n_splits * G;
  float* ws_ml = reinterpret_cast<float*>(ws);
  float* ws_acc = ws_ml + ((2 * parts + 63) / 64) * 64;
  const dim3 grid((unsigned)n_splits, kHeads, (unsigned)(L * B));
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(64), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(128), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(256), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, dim3(512), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((Hq * kDim + 255) / 256), (unsigned)(L * B)), dim3(256), 0,
                     s, Hq, G, n_splits, ws_ml, ws_acc, out);
  return hipGetLastError();
}

}  // namespace msa
