// prefill.hip -- multi-token sparse prefill: T query tokens of grouped-query
// attention over [memory context ; local KV], causal in the local part.
//
// Method: after routing, the layer's attention runs over the query states and the
// concatenation of the selected documents' compressed K/V with the local K/V
// (xuqi2024.github.io "【MSA】突破100M Token 上下文…", 5.2; yunpan.plus
// "MSA端到端可训练记忆模型完整开源…", 推理流水线, Stage 2).  Query token t is the
// (n_loc - T + t)-th local row: it sees every memory-context row and local rows
// 0 .. n_loc - T + t.
//
// Layout of the work: one workgroup per (16-token query block, KV head, layer x
// query), one wave per query head of the KV head's group, so the waves share the
// K/V tiles and the causal mask.  Per 32-key tile (K and V row-major, staged in
// LDS; the next tile's loads are issued before the current tile is
// used) a wave computes S^T = K . Q^T with v_mfma_f32_16x16x32_bf16 (keys as the A
// operand, the query block as the B operand held in registers): lane l owns query
// token l & 15 and keys 4 (l >> 4) + r of each 16-key half.  The online softmax
// runs on those fp32 scores (cross-lane max over the four lane groups, per-lane
// partial sums).  For O^T += V^T . P^T the MFMA's 32-long k axis is taken in the
// order (first half: keys 4g..4g+3, second half: keys 16+4g..16+4g+3) for lane
// group g, which is exactly how the score accumulators already sit in the lanes,
// so P enters as the B operand without any shuffle; V^T comes from the row-major
// V tile in the same key order through LDS transposed reads (ds_read_b64_tr_b16).  P goes in as a bf16 high part plus a bf16
// residual (two products), so the probabilities keep ~16 significant bits.
// Accumulation is fp32 throughout.
#include "msa_device.hpp"
#include "msa_kernels.hpp"

namespace msa {
namespace {

constexpr int kQBlock = 16;            // query tokens per workgroup
constexpr int kKeyTile = 32;           // keys per step
constexpr int kKStride = kDim + 8;     // bf16 per staged K row
constexpr int kVStride = kDim + 8;     // bf16 per staged V row

// G query heads per KV head; HPW of them per wave; TB 16-token query blocks per workgroup.
// Waves: (G / HPW) x TB; wave w takes token block w / (G / HPW) and heads
// HPW * (w % (G / HPW)) .. +HPW-1 of the group.  The heads of a wave share every K
// fragment and every V^T fragment read from LDS, and the tokens' mask.
template <int G, int HPW, int TB>
__global__ void __launch_bounds__(64 * (G / HPW) * TB)
prefill_kernel(int32_t T, int32_t Hq, const uint16_t* __restrict__ q, const uint16_t* __restrict__ ctx_k,
               const uint16_t* __restrict__ ctx_v, const int32_t* __restrict__ ctx_len, int32_t max_ctx,
               const uint16_t* __restrict__ loc_k, const uint16_t* __restrict__ loc_v,
               const int32_t* __restrict__ loc_len, int32_t max_loc, float scale, float* __restrict__ out) {
  __shared__ uint16_t k_s[2][kKeyTile * kKStride];   // double buffered: one barrier per tile
  __shared__ uint16_t v_s[2][kKeyTile * kVStride];

  constexpr int WPB = G / HPW;             // waves per token block
  constexpr int NT = 64 * WPB * TB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;  // lane group, query token t0 + j
  const int t0 = (blockIdx.x * TB + wave / WPB) * kQBlock;
  const int hq0 = blockIdx.y * G + HPW * (wave % WPB);
  const int kvh = blockIdx.y;
  const int64_t lb = blockIdx.z;
  const float ninf = -__builtin_huge_valf();

  int32_t clen = ctx_len[lb];
  clen = clen < 0 ? 0 : (clen > max_ctx ? max_ctx : clen);
  int32_t llen = loc_len[lb];
  llen = llen < 0 ? 0 : (llen > max_loc ? max_loc : llen);
  // local rows visible to token t: 0 .. llen - T + t (clamped to [0, llen])
  auto visible = [&](int t) {
    int v = llen - T + t + 1;
    return v < 0 ? 0 : (v > llen ? llen : v);
  };
  // keys of the workgroup (its last token's limit) and of this wave's block
  const int tw_last = (int)blockIdx.x * TB * kQBlock + TB * kQBlock - 1;
  const int32_t n_keys = clen + visible(tw_last < T - 1 ? tw_last : T - 1);
  const int tb_last = t0 + kQBlock - 1 < T - 1 ? t0 + kQBlock - 1 : T - 1;
  const int32_t n_keys_w = t0 < T ? clen + visible(tb_last) : 0;
  const int tok = t0 + j;
  const int vis_tok = tok < T ? visible(tok) : 0;

  // query blocks as B fragments: token t0 + j, dims 32 s + 8 g .. +7, per head
  bf16x8 qf[HPW][4];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tok < T)
        v = *reinterpret_cast<const u32x4*>(q + (((lb * T + tok) * Hq + hq0 + hh) * kDim) + 32 * s + 8 * g);
      qf[hh][s] = __builtin_bit_cast(bf16x8, v);
    }

  const uint16_t* ck = ctx_k + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* cv = ctx_v + (lb * max_ctx) * (int64_t)kRow + kvh * kDim;
  const uint16_t* lk = loc_k + (lb * (int64_t)max_loc) * kRow + kvh * kDim;
  const uint16_t* lv = loc_v + (lb * (int64_t)max_loc) * kRow + kvh * kDim;

  // tile loader: 32 keys x 16 chunks of 16 B for K and for V.  Rows past the last key
  // are loaded from the last key (in bounds, finite) and masked out of the scores, so the
  // loads carry no branch and no zero fill.
  constexpr int kPer = (kKeyTile * 16 + NT - 1) / NT;
  static_assert(kPer * NT == kKeyTile * 16, "the tile's chunks split evenly over the threads");
  u32x4 pk[kPer], pv[kPer];
  auto load_tile = [&](int32_t k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * NT;
      const int kk = u >> 4, c = u & 15;
      const int32_t row = k0 + kk < n_keys ? k0 + kk : n_keys - 1;
      const int64_t off = (row < clen ? (int64_t)row : (int64_t)(row - clen)) * kRow + c * 8;
      pk[i] = *reinterpret_cast<const u32x4*>((row < clen ? ck : lk) + off);
      pv[i] = *reinterpret_cast<const u32x4*>((row < clen ? cv : lv) + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * NT;
      const int kk = u >> 4, c = u & 15;
      *reinterpret_cast<u32x4*>(k_s[buf] + kk * kKStride + c * 8) = pk[i];
      *reinterpret_cast<u32x4*>(v_s[buf] + kk * kVStride + c * 8) = pv[i];
    }
  };

  // The running maximum is kept in log2 units (scale folded with log2 e): each raw score s
  // enters exp2 as one fma(s, scale2, -m), and the tile maximum is taken over raw scores
  // (scale2 > 0 keeps the order).  The maximum is raised only when a tile exceeds it by more
  // than kSlack, so unnormalised probabilities stay below 2^kSlack and the accumulators are
  // rescaled rarely.
  constexpr float kSlack = 8.f;
  const float scale2 = scale * 1.4426950408889634f;
  float m_run[HPW], l_lane[HPW];
  f32x4 o[HPW][8];   // O^T: dims 16 dt + 4 g + r, token t0 + j
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m_run[hh] = ninf;
    l_lane[hh] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[hh][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // keys every token of the wave's block may see: its first token's limit
  const int32_t all_visible = clen + (t0 < T ? visible(t0) : 0);
  if (n_keys > 0) {
    load_tile(0);
    store_tile(0);
  }
  // every load issued so far (the query fragments, the first tile) completes here, so the
  // loop's wait bookkeeping starts clean and waits only for each tile's own loads
  __builtin_amdgcn_s_waitcnt(0);
  int buf = 0;
  for (int32_t k0 = 0; k0 < n_keys; k0 += kKeyTile, buf ^= 1) {
    __syncthreads();   // tile k0 is in buf; every reader of buf ^ 1 (the tile before) is done
    if (k0 + kKeyTile < n_keys) load_tile(k0 + kKeyTile);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the tile's products
    if (k0 < n_keys_w) {                       // uniform per wave: the block sees part of the tile
      const uint16_t* kt = k_s[buf];
      // S^T for keys k0 + 16 h2 + 4 g + r (h2 = 0, 1), token t0 + j, per head
      f32x4 sc[HPW][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) sc[hh][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 kw = *reinterpret_cast<const u32x4*>(kt + (16 * h2 + j) * kKStride + 32 * s + 8 * g);
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh)
            sc[hh][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[hh][s],
                                                                 sc[hh][h2], 0, 0, 0);
        }
      }
      const bool whole = k0 + kKeyTile <= all_visible;   // no mask needed
      bf16x8 pfh[HPW], pfl[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        // mask (tiles every token of the block sees whole need none), raw maximum
        float mt = ninf;
        if (whole) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sc[hh][h2][r]);
        } else {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int32_t key = k0 + 16 * h2 + 4 * g + r;
              const bool ok = key < n_keys && (key < clen || key - clen < vis_tok);
              const float v = ok ? sc[hh][h2][r] : ninf;
              sc[hh][h2][r] = v;
              mt = fmaxf(mt, v);
            }
        }
        mt = rows4_max(mt) * scale2;           // over the tile's 32 keys of token t0 + j, log2 units
        // raise the reference maximum only past the slack (ballot: most tiles skip the rescale)
        const bool raise = mt > m_run[hh] + kSlack;
        if (__ballot(raise)) {
          const float m_new = raise ? mt : m_run[hh];
          const float alpha = m_run[hh] == ninf ? 0.f : __builtin_amdgcn_exp2f(m_run[hh] - m_new);
          m_run[hh] = m_new;
          l_lane[hh] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[hh][dt] *= alpha;
        }
        const float neg_m = m_run[hh] == ninf ? 0.f : -m_run[hh];   // a token with no visible key yet
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hh][h2][r], scale2, neg_m));
            sc[hh][h2][r] = p;
            l_lane[hh] += p;
          }
        // P^T as the B operand: k slot 8 g + e holds key 4 g + e (e < 4) or 16 + 4 g + e - 4.
        // P = P_hi + P_lo with both parts in bf16 (two products), so the probabilities
        // enter the matrix cores with ~16 significant bits rather than 8.
        u32x4 pwh, pwl;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = sc[hh][e2 >> 1][2 * (e2 & 1)], p1 = sc[hh][e2 >> 1][2 * (e2 & 1) + 1];
          const uint32_t hw = pack2_bf16(p0, p1);
          pwh[e2] = hw;
          pwl[e2] = pack2_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u));
        }
        pfh[hh] = __builtin_bit_cast(bf16x8, pwh);
        pfl[hh] = __builtin_bit_cast(bf16x8, pwl);
      }
      // V^T fragments by transposed reads of the row-major V tile: lane (g, j) of the
      // A operand needs dim 16 dt + j of keys 4 g + e and 16 + 4 g + e (e = 0..3), so
      // source lane j points at dims 16 dt + 4 (j & 3) .. +3 of key 4 g + (j >> 2).
      const uint16_t* vsrc = v_s[buf] + (4 * g + (j >> 2)) * kVStride + 4 * (j & 3);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint2 a0 = lds_read_tr16(vsrc + 16 * dt);
        const uint2 a1 = lds_read_tr16(vsrc + 16 * kVStride + 16 * dt);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, (u32x4{a0.x, a0.y, a1.x, a1.y}));
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          o[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh[hh], o[hh][dt], 0, 0, 0);
          o[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl[hh], o[hh][dt], 0, 0, 0);
        }
      }
    }
    if (k0 + kKeyTile < n_keys) store_tile(buf ^ 1);
  }

#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float l_tok = rows4_sum(l_lane[hh]);
    if (tok < T) {
      const float inv = l_tok > 0.f ? 1.0f / l_tok : 0.f;
      float* dst = out + ((lb * T + tok) * Hq + hq0 + hh) * kDim + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(dst + 16 * dt) =
            make_float4(o[hh][dt][0] * inv, o[hh][dt][1] * inv, o[hh][dt][2] * inv, o[hh][dt][3] * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefill(int32_t L, int32_t B, int32_t T, int32_t Hq, const uint16_t* q, const uint16_t* ctx_k,
                          const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx, const uint16_t* loc_k,
                          const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc, float scale, float* out,
                          hipStream_t s) {
  const int G = Hq / kHeads;
#define MSA_PREFILL_LAUNCH(GV, HPWV, TBV)                                                                       \
  hipLaunchKernelGGL((prefill_kernel<GV, HPWV, TBV>),                                                          \
                     dim3((unsigned)((T + kQBlock * (TBV) - 1) / (kQBlock * (TBV))), kHeads, (unsigned)(L * B)), \
                     dim3(64 * ((GV) / (HPWV)) * (TBV)), 0, s, T, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx, loc_k,   \
                     loc_v, loc_len, max_loc, scale, out)
  switch (G) {
    case 1: MSA_PREFILL_LAUNCH(1, 1, 4); break;
    case 2: MSA_PREFILL_LAUNCH(2, 2, 2); break;
    case 4: MSA_PREFILL_LAUNCH(4, 2, 2); break;
    case 8: MSA_PREFILL_LAUNCH(8, 2, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef MSA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace msa
