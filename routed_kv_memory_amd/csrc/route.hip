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
//  * Queries of >= 16 tokens: per KV head the scan is a [tokens x 128] . [128 x
//    blocks] bf16 contraction on v_mfma_f32_16x16x32_bf16.  The route-key tile
//    layout makes each head's slice of a 16-block tile four contiguous 1 KiB MFMA
//    fragments, so keys go from HBM straight into registers; the query chunk stays
//    in registers for the whole layer.  The per-head cosine scaling 1/(|q| |k|) is
//    applied to the fp32 accumulators, so the bf16 inputs enter the matrix cores
//    exactly as stored; key norms are summed from the fragments already held, so
//    the scan reads nothing but the keys and the block -> document map.
//  * Persistent grid over all CUs: each 512-thread workgroup owns a contiguous
//    range of (layer, tile) items for one 64-token query chunk; ranges sharing a
//    chunk are placed XCD by XCD.
//  * Heads meet in LDS once per two tiles; the max over tokens is a cross-lane
//    reduction; the per-document max is a segmented scan keyed by a block ->
//    document map, with each document emitted once per range.
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
// chunk's head-h fragments (64 tokens x 128 dims) in registers for the whole
// layer, and streams only its own head's 4 KiB of each 16-block route tile (four
// contiguous 1 KiB fragments) through a register ring, four tiles ahead, with
// nontemporal loads.  The same fragment bytes serve as the A operand (query:
// rows = tokens) and the B operand (keys: columns = blocks) of
// v_mfma_f32_16x16x32_bf16, so lane l ends up owning block (l & 15) and tokens
// 4*(l >> 4) + r: the key norm is summed from the fragment the lane already holds,
// and the per-head cosine scaling 1/(|q| |k|) is applied to the fp32 accumulators
// before the head sum.  The 8 heads' scaled partials of two consecutive tiles
// meet in LDS behind one barrier (double buffered, so the next two tiles' matrix
// work overlaps the reduction); waves 4..7 sum them for one token group each and
// take the max over its 16 tokens; wave 0 folds the token groups and keeps each
// document's running maximum across tiles, emitting it once when the document
// ends (a plain store when no other workgroup can touch that document, an atomic
// max otherwise).
constexpr int kScanWaves = kHeads;              // one wave per KV head
constexpr int kScanWG = kScanWaves * 64;
constexpr int kGroup = 2;                        // tiles per barrier
constexpr int kStages = 6;                       // prefetch ring (a multiple of kGroup)
constexpr int kAhead = 4;                        // tiles in flight per wave beyond the current one

__device__ __forceinline__ void lds_barrier() {
  // orders LDS only: in-flight global prefetches stay in flight across the barrier
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float sumsq8(u32x4 w) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf16_lo(w[e]), c = bf16_hi(w[e]);
    s += a * a + c * c;
  }
  return s;
}

// Document score emission: `exclusive` means this workgroup is the only writer of
// the codes row and the codes started from zero, so a document seen whole here can
// be stored; documents that may continue in another workgroup use atomic max.
__device__ __forceinline__ void emit_doc(uint32_t* __restrict__ codes, int32_t doc, float v, bool atomic) {
  if (atomic) atomicMax(codes + doc, ordered_code(v));
  else codes[doc] = ordered_code(v);
}

template <int NT>
__global__ void __launch_bounds__(kScanWG)
route_mfma_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, int32_t n_tc,
                  const uint4* __restrict__ krt, int64_t tiles, const int32_t* __restrict__ blk_doc,
                  int32_t n_docs, int32_t L, int32_t R, int32_t exclusive, uint32_t* __restrict__ codes) {
  // per-head scaled partial scores of one group of tiles, double buffered
  __shared__ float4 P[2][kGroup][kScanWaves][NT][64];
  __shared__ float M[2][kGroup][4][kTile];       // block maxima per token group
  __shared__ float RQ[kHeads][kTokChunk];        // 1/max(|q|, eps) per head and token of the chunk

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
  if (it_begin >= it_end) return;                // uniform across the workgroup

  const int wave = threadIdx.x >> 6;             // = head
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int j = lane & 15;
  const float ninf = -__builtin_huge_valf();

  bf16x8 q[4][NT];       // A fragments [s][nt]: token 16 nt + j, dims 32 s + 8 g .. +7
  int cur_layer = -1;

  // Prefetch cursor.  Items are consecutive, so the head's fragments of item i sit
  // at a linear offset; loads are unconditional (past the range end the last item
  // is fetched again) so that every wait is an exact count.
  const uint4* isrc = krt + it_begin * kTileU4 + wave * kHeadU4 + lane;
  int64_t itau = it_begin % tiles;
  int64_t inext = it_begin;

  u32x4 kb[kStages][4];
  int32_t db[kStages];

  // The route keys are read exactly once: nontemporal loads keep them from
  // displacing useful lines in the caches.
  auto issue = [&](u32x4 (&kbuf)[4], int32_t& dbuf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kbuf[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(isrc + s * 64));
    dbuf = blk_doc[itau * kTile + j];
    if (inext + 1 < it_end) {
      ++inext;
      isrc += kTileU4;
      itau = (itau + 1 == tiles) ? 0 : itau + 1;
    }
  };

#pragma unroll
  for (int x = 0; x < kAhead; ++x) issue(kb[x], db[x]);

  // compute cursor and wave 0's open document (the last run of the previous tile)
  int layer = (int)(it_begin / tiles);
  int64_t ctau = it_begin - (int64_t)layer * tiles;
  int32_t cdoc = -1;
  float cmax = ninf;
  bool cshared = true;          // the open document may have blocks outside this range
  bool seg_first = true;        // first tile of this layer inside the range
  int pb = 0;                   // LDS buffer parity, alternates every group
  // the tiles of the current group (c_*) and of the group wave 0 folds next (p_*)
  bool c_valid[kGroup], c_first[kGroup], c_last[kGroup];
  int c_layer[kGroup];
  int32_t c_doc[kGroup];
  bool p_valid[kGroup], p_first[kGroup], p_last[kGroup];
  int p_layer[kGroup];
  int32_t p_doc[kGroup];
#pragma unroll
  for (int u = 0; u < kGroup; ++u) p_valid[u] = false;

  // Wave 0: fold the block maxima of one tile (written before the last barrier)
  // into document scores.  Blocks of a document are contiguous, so a segmented
  // suffix max within each run of equal documents gives the run maxima; the last
  // run stays open because the document may continue in the next tile.
  auto flush_tile = [&](const float (&Mt)[4][kTile], bool t_first, bool t_last, int t_layer, int32_t t_doc) {
    float v = ninf;
    int32_t d = -1;
    if (lane < kTile) {
#pragma unroll
      for (int n = 0; n < NT; ++n) v = fmaxf(v, Mt[n][lane]);
      d = t_doc;
      if (d >= n_docs) d = -1;   // map entries are trusted only inside [0, n_docs)
    }
    uint32_t* lcodes = codes + ((int64_t)t_layer * B + b) * n_docs;
    const int32_t d0 = __builtin_amdgcn_readlane(d, 0);
    if (cdoc >= 0 && cdoc != d0) {          // this tile does not continue the open document
      if (lane == 0) emit_doc(lcodes, cdoc, cmax, cshared || !exclusive);
      cdoc = -1;
    }
    bool run0_shared = t_first;
    if (cdoc >= 0) {                        // lane 0's run continues the open document
      if (lane == 0) v = fmaxf(v, cmax);
      run0_shared = cshared;
    }
    {
      const int ninf_bits = __float_as_int(ninf);
      float vo = __int_as_float(row_shl<1>(__float_as_int(v), ninf_bits));
      int32_t dn = row_shl<1>(d, -2);
      if (dn == d) v = fmaxf(v, vo);
      vo = __int_as_float(row_shl<2>(__float_as_int(v), ninf_bits));
      dn = row_shl<2>(d, -2);
      if (dn == d) v = fmaxf(v, vo);
      vo = __int_as_float(row_shl<4>(__float_as_int(v), ninf_bits));
      dn = row_shl<4>(d, -2);
      if (dn == d) v = fmaxf(v, vo);
      vo = __int_as_float(row_shl<8>(__float_as_int(v), ninf_bits));
      dn = row_shl<8>(d, -2);
      if (dn == d) v = fmaxf(v, vo);
    }
    const int32_t dprev = row_shr<1>(d, -2);
    const bool head = lane < kTile && (lane == 0 || dprev != d);
    const uint64_t heads = __ballot(head);
    const int hl = 63 - __builtin_clzll(heads);          // head lane of the last run
    const int32_t dl = __builtin_amdgcn_readlane(d, hl);
    const float vl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), hl));
    if (head && lane != hl && d >= 0) emit_doc(lcodes, d, v, (lane == 0 ? run0_shared : false) || !exclusive);
    cdoc = dl;
    cmax = vl;
    cshared = hl == 0 ? run0_shared : false;
    if (t_last) {                           // the range or the layer ends here
      if (cdoc >= 0 && lane == 0) emit_doc(lcodes, cdoc, cmax, true);
      cdoc = -1;
    }
  };

  for (int64_t base = it_begin; base < it_end; base += kStages) {
#pragma unroll
    for (int x = 0; x < kStages; ++x) {
      const int64_t it = base + x;
      const int u = x % kGroup;               // position in the group
      issue(kb[(x + kAhead) % kStages], db[(x + kAhead) % kStages]);
      c_valid[u] = it < it_end;               // uniform across the workgroup
      if (c_valid[u]) {
        if (layer != cur_layer) {
          // this layer's query chunk, head `wave`, as fragments; inverse norms per token
          const uint16_t* qb = qr + (((int64_t)layer * B + b) * T) * kRow + wave * kDim + g * 8;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int tok = t_base + nt * 16 + j;
            float ss = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              u32x4 v = {0u, 0u, 0u, 0u};
              if (tok < T) v = *reinterpret_cast<const u32x4*>(qb + (int64_t)tok * kRow + s * 32);
              q[s][nt] = __builtin_bit_cast(bf16x8, v);
              ss += sumsq8(v);
            }
            ss = rows4_sum(ss);
            if (g == 0) RQ[wave][nt * 16 + j] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
          }
          cur_layer = layer;
        }

        // C[token][block] = Q . K^T for this head; lane: block j, tokens 4 g + r
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float ssk = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, kb[x % kStages][s]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[s][nt], kf, acc[nt], 0, 0, 0);
          ssk += sumsq8(kb[x % kStages][s]);
        }
        ssk = rows4_sum(ssk);
        const float rk = __builtin_amdgcn_rcpf(fmaxf(sqrtf(ssk), kNormEps));   // block j, head `wave`
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 rq = *reinterpret_cast<const float4*>(&RQ[wave][nt * 16 + 4 * g]);   // tokens 4 g + r
          P[pb][u][wave][nt][lane] = make_float4(acc[nt][0] * (rq.x * rk), acc[nt][1] * (rq.y * rk),
                                                 acc[nt][2] * (rq.z * rk), acc[nt][3] * (rq.w * rk));
        }
        const bool seg_last = (ctau + 1 == tiles) || (it + 1 == it_end);
        c_first[u] = seg_first;
        c_last[u] = seg_last;
        c_layer[u] = layer;
        c_doc[u] = db[x % kStages];
        seg_first = seg_last;
        if (++ctau == tiles) { ctau = 0; ++layer; }
      }

      if (u == kGroup - 1) {
        lds_barrier();   // the only barrier per group: P[pb] complete, M[pb ^ 1] complete
        if (wave >= kScanWaves - 4 && wave - (kScanWaves - 4) < NT) {
          // token group n = wave - 4: sum the 8 heads, max over the group's 16 valid tokens
          const int n = wave - (kScanWaves - 4);
          const int tok0 = t_base + n * 16 + 4 * g;
#pragma unroll
          for (int v = 0; v < kGroup; ++v) {
            if (!c_valid[v]) break;
            float4 tot = P[pb][v][0][n][lane];
#pragma unroll
            for (int h = 1; h < kHeads; ++h) {
              const float4 w = P[pb][v][h][n][lane];
              tot.x += w.x; tot.y += w.y; tot.z += w.z; tot.w += w.w;
            }
            float m = tok0 < T ? tot.x : ninf;
            m = fmaxf(m, tok0 + 1 < T ? tot.y : ninf);
            m = fmaxf(m, tok0 + 2 < T ? tot.z : ninf);
            m = fmaxf(m, tok0 + 3 < T ? tot.w : ninf);
            m = rows4_max(m);
            if (g == 0) M[pb][v][n][j] = m * 0.125f;   // head mean
          }
        }
        if (wave == 0) {
#pragma unroll
          for (int v = 0; v < kGroup; ++v)
            if (p_valid[v]) flush_tile(M[pb ^ 1][v], p_first[v], p_last[v], p_layer[v], p_doc[v]);
        }
#pragma unroll
        for (int v = 0; v < kGroup; ++v) {
          p_valid[v] = c_valid[v];
          p_first[v] = c_first[v];
          p_last[v] = c_last[v];
          p_layer[v] = c_layer[v];
          p_doc[v] = c_doc[v];
        }
        pb ^= 1;
        if (it + 1 >= it_end) break;   // uniform across the workgroup
      }
    }
  }
  lds_barrier();        // M of the last group complete
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < kGroup; ++v)
      if (p_valid[v]) flush_tile(M[pb ^ 1][v], p_first[v], p_last[v], p_layer[v], p_doc[v]);
  }
}

// ---------------------------------------------------------------- VALU scan
//
// One wave per 16-block tile: lane l holds block (l & 15) and, per head, the 8-dim
// chunks 4s + (l >> 4); partial dots are summed over the 4 lane groups.
template <int TMAX>
__global__ void __launch_bounds__(256)
route_valu_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, const uint4* __restrict__ krt,
                  int64_t n_blk, int64_t tiles,
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
    float ssk = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ssk += x[i] * x[i];
    ssk += __shfl_xor(ssk, 16, 64);
    ssk += __shfl_xor(ssk, 32, 64);
    const float rk = 1.0f / fmaxf(sqrtf(ssk), kNormEps);
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
                               int64_t n_blk, const int32_t* blk_doc, int32_t n_docs,
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
      const int excl = (n_tc == 1 && !accumulate) ? 1 : 0;
      switch (NT) {
        case 1: hipLaunchKernelGGL(route_mfma_kernel<1>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,
                                   blk_doc, n_docs, L, R, excl, codes); break;
        case 2: hipLaunchKernelGGL(route_mfma_kernel<2>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,
                                   blk_doc, n_docs, L, R, excl, codes); break;
        case 3: hipLaunchKernelGGL(route_mfma_kernel<3>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,
                                   blk_doc, n_docs, L, R, excl, codes); break;
        default: hipLaunchKernelGGL(route_mfma_kernel<4>, grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,
                                    blk_doc, n_docs, L, R, excl, codes); break;
      }
    } else {
      const dim3 grid((unsigned)((tiles + 3) / 4), (unsigned)B, (unsigned)L);
      hipLaunchKernelGGL(route_valu_kernel<16>, grid, dim3(256), 0, s, qr, B, T,
                         reinterpret_cast<const uint4*>(krt), n_blk, tiles, blk_doc, n_docs, codes);
    }
  }
  hipLaunchKernelGGL(codes_final_kernel, dim3(fill_grid), dim3(256), 0, s, codes, n_codes);
  return hipGetLastError();
}

}  // namespace msa
