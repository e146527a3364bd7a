// decode.hip -- A5: one decode token of grouped-query attention over
// [memory context ; local KV], split over rows, then merged.
//
// Method: the decode token attends to the Top-k documents' compressed K/V
// followed by the query's local K/V, with no mask; the memory part is fixed and
// only the local part grows (yunpan.plus "MSA端到端可训练记忆模型完整开源…", 整体设计 ->
// 架构; xuqi2024.github.io "【MSA】突破100M Token 上下文…", 5.2; xiaohongrsx.github.io
// "MSA paper reading", 推理全流程).
//
// Layout of the work: one workgroup per (256-row split, KV head, layer x query); each of
// its 8 waves takes 32 of the split's rows for all G query heads of the KV head, so the
// heads share every K and V read.  On the matrix cores (v_mfma_f32_16x16x32_bf16) the
// G heads are the 16-wide column side: S^T = K . Q^T takes the keys as the A operand,
// loaded from global memory straight into fragment layout (lane 16 g + j: key j, dims
// 8 g .. 8 g + 7 of each 32-dim step); O^T = V^T . P^T takes V^T from the wave's own
// row-major V tile in LDS through transposed reads (ds_read_b64_tr_b16), and P as a
// bf16 high part plus a bf16 residual (~16 significant bits).  Every load of a split is
// issued at once (one memory latency per split).  The 8 waves' (max, sum, output) are
// combined in LDS into one partial per split and head; a second kernel merges the
// splits in one pass.  All accumulation is fp32.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kSplitWaves = 8;
constexpr int kWaveRows = 32;                          // per wave
constexpr int kRowsPerSplit = kWaveRows * kSplitWaves;  // per workgroup
constexpr int kVStride = kDim + 8;        // bf16 per staged V row


template <int G>
__global__ void __launch_bounds__(64 * kSplitWaves)
decode_split_kernel(int32_t Hq, const uint16_t* __restrict__ q, const uint16_t* __restrict__ ctx_k,
                    const uint16_t* __restrict__ ctx_v, const int32_t* __restrict__ ctx_len, int32_t max_ctx,
                    const uint16_t* __restrict__ loc_k, const uint16_t* __restrict__ loc_v,
                    const int32_t* __restrict__ loc_len, int32_t max_loc, float scale, int32_t n_splits,
                    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  // per wave: its K tile, then its V tile (row-major), then its output columns
  __shared__ uint16_t v_s[kSplitWaves][kWaveRows * kVStride];
  __shared__ float c_m[kSplitWaves][G], c_l[kSplitWaves][G];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int64_t lb = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;   // lane group; column j = query head j of the group
  const float ninf = -__builtin_huge_valf();

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
  const int64_t part0 = ((lb * kHeads + kvh) * n_splits + split) * G;
  if (r_begin >= r_end) return;            // uniform: the merge reads only splits with rows

  const uint16_t* ck = ctx_k + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* cv = ctx_v + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* lk = loc_k + (lb * (int64_t)max_loc) * kRow + kvh * kDim;
  const uint16_t* lv = loc_v + (lb * (int64_t)max_loc) * kRow + kvh * kDim;
  // rows past the split's end are loaded from its last row (in bounds, finite), masked
  // out of the scores, and carry probability 0; the loads need no branch
  const int32_t w0 = r_begin + kWaveRows * wave;
  const bool active = w0 < r_end;           // uniform per wave
  auto row_ptr = [&](const uint16_t* c, const uint16_t* l, int32_t r) {
    r = min(r, r_end - 1);
    return r < clen ? c + (int64_t)r * kRow : l + (int64_t)(r - clen) * kRow;
  };

  // K and V rows, whole rows per 16 lanes: load i brings keys w0 + 4 i + g, dims 8 j .. 8 j + 7
  u32x4 kr[8], vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t r = active ? w0 + 4 * i + g : r_begin;
    kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row_ptr(ck, lk, r) + 8 * j));
    vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row_ptr(cv, lv, r) + 8 * j));
  }
  // Q^T as the B operand: column j = head j of the group (zero past G), dims 32 s + 8 g .. +7
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < G) v = *reinterpret_cast<const u32x4*>(q + (lb * Hq + kvh * G + j) * kDim + 32 * s + 8 * g);
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }

  uint16_t* vt = v_s[wave];
  float m = ninf, l = 0.f;
  f32x4 o[8];   // O^T: dims 16 dt + 4 g + r, head j
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    // stage this wave's V rows (wave-private: the wave's own LDS ordering suffices)
    // K through the wave's own LDS tile (the wave's LDS operations complete in order, so
    // no barrier): fragments of key block kb are keys 16 kb + j, dims 32 s + 8 g .. +7
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(vt + (4 * i + g) * kVStride + 8 * j) = kr[i];
    u32x4 kf[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[kb][s] = *reinterpret_cast<const u32x4*>(vt + (16 * kb + j) * kVStride + 32 * s + 8 * g);
    // then the V rows into the same tile, once the K fragments are in registers
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(vt + (4 * i + g) * kVStride + 8 * j) = vr[i];
    // S^T for keys w0 + 16 kb + 4 g + r, head j (log2 units: scale folded with log2 e)
    const float scale2 = scale * 1.4426950408889634f;
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kb][s]), qf[s], sc[kb], 0,
                                                        0, 0);
    }
    float mt = ninf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = w0 + 16 * kb + 4 * g + r < r_end;
        const float v = ok ? sc[kb][r] * scale2 : ninf;
        sc[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    m = rows4_max(mt);                      // over the wave's 32 keys (finite: key w0 is valid)
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[kb][r] - m);
        sc[kb][r] = p;
        ps += p;
      }
    l = rows4_sum(ps);
    // P^T as the B operand: k slot 8 g + e holds key 4 g + e (e < 4) or 16 + 4 g + e - 4
    u32x4 pwh, pwl;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float p0 = sc[e2 >> 1][2 * (e2 & 1)], p1 = sc[e2 >> 1][2 * (e2 & 1) + 1];
      const uint32_t hw = pack2_bf16(p0, p1);
      pwh[e2] = hw;
      pwl[e2] = pack2_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u));
    }
    const bf16x8 pfh = __builtin_bit_cast(bf16x8, pwh), pfl = __builtin_bit_cast(bf16x8, pwl);
    // V^T fragments by transposed reads: lane (g, j) of the A operand needs dim 16 dt + j of
    // keys 4 g + e and 16 + 4 g + e, so source lane j points at dims 16 dt + 4 (j & 3) .. +3
    // of key 4 g + (j >> 2)
    const uint16_t* vsrc = vt + (4 * g + (j >> 2)) * kVStride + 4 * (j & 3);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint2 a0 = lds_read_tr16(vsrc + 16 * dt);
      const uint2 a1 = lds_read_tr16(vsrc + 16 * kVStride + 16 * dt);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, (u32x4{a0.x, a0.y, a1.x, a1.y}));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl, o[dt], 0, 0, 0);
    }
  }
  // combine the waves: each wave's output columns go to its own V tile's space (its
  // reads of it are done: one wave's LDS operations complete in order)
  float* co = reinterpret_cast<float*>(vt);   // [G][kDim]
  if (j < G) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(co + j * kDim + 16 * dt + 4 * g) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
      c_m[wave][j] = m;                     // -inf for an inactive wave
      c_l[wave][j] = l;
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kDim; i += 64 * kSplitWaves) {
    const int h = i / kDim;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) M = fmaxf(M, c_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float c = __builtin_amdgcn_exp2f(c_m[w][h] - M);   // 0 for an inactive wave
      num += c * reinterpret_cast<const float*>(v_s[w])[i];
      den += c * c_l[w][h];
    }
    ws_acc[part0 * kDim + i] = num;
    if ((i & (kDim - 1)) == 0) {
      ws_ml[2 * (part0 + h)] = M * 0.6931471805599453f;   // natural-log units for the merge
      ws_ml[2 * (part0 + h) + 1] = den;
    }
  }
}

__global__ void __launch_bounds__(256)
decode_merge_kernel(int32_t Hq, int32_t G, int32_t n_splits, const int32_t* __restrict__ ctx_len, int32_t max_ctx,
                    const int32_t* __restrict__ loc_len, int32_t max_loc, const float* __restrict__ ws_ml,
                    const float* __restrict__ ws_acc, float* __restrict__ out) {
  const int64_t lb = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;   // (hq, d)
  if (i >= Hq * kDim) return;
  const int hq = i / kDim, d = i % kDim;
  const int kvh = hq / G, hh = hq % G;
  // the splits that hold rows (the same clamping as the split kernel)
  int32_t clen = ctx_len[lb];
  clen = clen < 0 ? 0 : (clen > max_ctx ? max_ctx : clen);
  int32_t llen = 0;
  if (max_loc > 0) {
    llen = loc_len[lb];
    llen = llen < 0 ? 0 : (llen > max_loc ? max_loc : llen);
  }
  const int32_t n_act = min(n_splits, (clen + llen + kRowsPerSplit - 1) / kRowsPerSplit);
  // one pass with a running maximum over batches of 8 splits (their loads are
  // independent); splits past the last row are never read (their kernel wrote nothing)
  const float ninf = -__builtin_huge_valf();
  float M = ninf, num = 0.f, den = 0.f;
  const int64_t part0 = (lb * kHeads + kvh) * n_splits * G + hh;
  for (int s0 = 0; s0 < n_act; s0 += 8) {
    float m[8], l[8], a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t part = part0 + (int64_t)(s0 + u) * G;
      const bool ok = s0 + u < n_act;
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
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(64 * kSplitWaves), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(64 * kSplitWaves), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(64 * kSplitWaves), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, dim3(64 * kSplitWaves), 0, s, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx,
                               loc_k, loc_v, loc_len, max_loc, scale, n_splits, ws_ml, ws_acc); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((Hq * kDim + 255) / 256), (unsigned)(L * B)), dim3(256), 0,
                     s, Hq, G, n_splits, ctx_len, max_ctx, loc_len, max_loc, ws_ml, ws_acc, out);
  return hipGetLastError();
}

}  // namespace msa
