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
//    fragments, so keys go from HBM straight into registers; the query chunk is
//    staged in LDS once per layer.  The per-head cosine scaling 1/(|q| |k|) is
//    applied to the fp32 accumulators, so the bf16 inputs enter the matrix cores
//    exactly as stored; key norms come from the same fragments (the diagonal of
//    K K^T on the matrix cores), so the scan reads nothing but the keys and the
//    block -> document map.
//  * A grid of (range, query chunk) workgroups, one per CU at a time, run in whole
//    rounds: each 512-thread workgroup owns a contiguous range of (layer, tile)
//    items for one 64-token query chunk (the chunks that share a range are placed
//    on one XCD, and shared ranges are kept short so that those workgroups stay
//    together); per layer it stages the chunk's query in LDS and each wave then
//    scans its own share of the range.
//  * A wave walks the 8 heads of a tile itself, so the head sum, the max over
//    tokens and the per-document max (a segmented scan keyed by a block ->
//    document map, each document emitted once) all stay in registers.
//  * When several query chunks share the key ranges, route_heads_kernel takes two chunks
//    per workgroup with one head per wave (the query in registers, the head sum through
//    LDS), halving the key bytes each CU reads per product.
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
// One workgroup per CU at a time, 8 waves.  The workgroup owns a contiguous range of
// (layer, tile) items for one 64-token query chunk and walks it layer by layer:
// per layer the 8 waves stage the chunk's query fragments (64 tokens x 8 heads x
// 128 dims, 128 KiB) and inverse norms in LDS, then each wave scans its own
// contiguous eighth of the layer's items with no further synchronisation.
//
// Per tile a wave streams the 8 heads' 4 KiB key slices (four contiguous 1 KiB
// fragments each) through a register ring, three slices ahead (nontemporal loads
// when no other workgroup re-reads the keys).  The same fragment bytes serve as the A operand (query: rows = tokens,
// read from LDS) and the B operand (keys: columns = blocks) of
// v_mfma_f32_16x16x32_bf16, so lane l ends up owning block (l & 15) and tokens
// 4*(l >> 4) + r of each 16-token group.  Per head four more MFMAs of the key
// fragments with themselves give K K^T, whose diagonal is the blocks' squared
// norms (when the caller passes the keys' norms the scan reads those instead and
// skips these products: worth it when several query chunks make the scan bound by
// the matrix cores); the fp32 accumulators are scaled by 1/(|q| |k|) and added
// into the lane's running head sum, all in registers.  The key addresses are wave-uniform (scalar
// registers) plus each lane's 16 bytes, so the ring's bookkeeping is scalar work.
// After the 8th head the lane takes the max over its tokens, a cross-lane max
// completes it over the 64 tokens, and the block maxima are folded into
// per-document maxima: a segmented scan over the 16 blocks, with each document's
// running maximum carried across the wave's consecutive tiles and emitted once
// when the document ends (a plain store when no other wave or workgroup can touch
// that document, an atomic max otherwise).
constexpr int kScanWaves = 8;
constexpr int kScanWG = kScanWaves * 64;
constexpr int kRing = 4;          // key slices (one head of one tile) held in registers; divides kHeads
constexpr int kAhead = 3;         // slices in flight beyond the current one

__device__ __forceinline__ void lds_barrier() {
  // orders LDS only: in-flight global loads stay in flight across the barrier
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

// Document score emission: a document that only this wave can see, in a codes row
// that started from zero, is stored; any other goes through an atomic max.
__device__ __forceinline__ void emit_doc(uint32_t* __restrict__ codes, int32_t doc, float v, bool atomic) {
  if (atomic) atomicMax(codes + doc, ordered_code(v));
  else codes[doc] = ordered_code(v);
}

// A wave-uniform 64-bit value moved to scalar registers (the compiler cannot always prove it).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// STREAM: the keys are read once (one query chunk per range), so nontemporal loads
// keep them from displacing other lines; with several query chunks the workgroups
// sharing a range re-read each tile, and ordinary loads let L2 serve the repeats.
// NORMS: the key norms come from knorm ([layer][tile][head][16] fp32) instead of the
// K K^T products.
template <int NT, bool STREAM, bool NORMS>
__global__ void __launch_bounds__(kScanWG)
route_mfma_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, int32_t n_tc,
                  const uint4* __restrict__ krt, int64_t tiles, const int32_t* __restrict__ blk_doc,
                  int32_t n_docs, int32_t L, int32_t R, int32_t exclusive, uint32_t* __restrict__ codes,
                  const float* __restrict__ knorm) {
  __shared__ u32x4 QS[kHeads][4][NT][64];      // query fragments [head][k step][token group][lane]
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

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int j = lane & 15;
  const float ninf = -__builtin_huge_valf();

  // accumulator row (nt, r) of this lane is token t_base + 16 nt + 4 g + r
  const bool full_chunk = t_base + NT * 16 <= T;   // uniform: every row is a valid token
  uint32_t tmask = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (t_base + nt * 16 + 4 * g + rr < T) tmask |= 1u << (nt * 4 + rr);

  for (int64_t seg = it_begin; seg < it_end;) {
    const int layer = (int)(seg / tiles);
    const int64_t layer0 = (int64_t)layer * tiles;
    const int64_t seg_end = it_end < layer0 + tiles ? it_end : layer0 + tiles;

    lds_barrier();   // every wave is done with the previous layer's query
    {
      // wave h stages head h of this layer's query chunk and its inverse norms
      const uint16_t* qb = qr + (((int64_t)layer * B + b) * T) * kRow + wave * kDim + g * 8;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = t_base + nt * 16 + j;
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (tok < T) v = *reinterpret_cast<const u32x4*>(qb + (int64_t)tok * kRow + s * 32);
          QS[wave][s][nt][lane] = v;
          ss += sumsq8(v);
        }
        ss = rows4_sum(ss);
        if (g == 0) RQ[wave][nt * 16 + j] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
      }
    }
    lds_barrier();

    // This wave's share of the layer's items: a contiguous eighth when the keys are
    // streamed once; every eighth tile when several query chunks re-read the range,
    // so that all waves of all those workgroups walk one front through L2.
    const int64_t n_items = seg_end - seg;
    const int64_t w0 = STREAM ? seg + n_items * wave / kScanWaves : seg + wave;
    const int64_t w1 = STREAM ? seg + n_items * (wave + 1) / kScanWaves : seg_end;
    constexpr int64_t tstep = STREAM ? 1 : kScanWaves;
    const int64_t n_tw = w0 < w1 ? (w1 - w0 + tstep - 1) / tstep : 0;   // tiles of this wave
    if (n_tw > 0) {
      uint32_t* lcodes = codes + ((int64_t)layer * B + b) * n_docs;
      const int64_t n_units = uniform64(n_tw * kHeads);   // key slices of the wave's tiles
      // the slice address is wave-uniform; each lane adds its own 16 bytes.  NORMS: the
      // norms of heads 4q .. 4q + 3 of a tile (64 floats, lane l: head 4q + (l >> 4), block
      // l & 15) are loaded with the tile's slice 4q into hn[q], which the next load into it
      // (four slices later) replaces only after those heads are done.
      const u32x4* src = reinterpret_cast<const u32x4*>(krt + w0 * kTileU4);
      const float* nsrc = NORMS ? knorm + w0 * (kHeads * kTile) : nullptr;   // this slice's 16 norms
      int64_t unext = 0;
      u32x4 kb[kRing][4];
      float hn[2];
      // Loads are unconditional (past the run's end the last slice is fetched again)
      // so that every wait is an exact count.
      auto issue = [&](u32x4 (&kbuf)[4], int slice) {   // slice: head of the issued slice (static)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kbuf[s] = STREAM ? __builtin_nontemporal_load(src + lane + s * 64) : src[lane + s * 64];
        if (NORMS && (slice & 3) == 0)   // from the tile's start: in bounds when the ring is clamped
          hn[slice >> 2] = nsrc[(slice - (int)(unext & (kHeads - 1))) * kTile + lane];
        if (unext + 1 < n_units) {
          ++unext;
          const int64_t step = (unext & (kHeads - 1)) == 0 ? (tstep - 1) * kTileU4 + kHeadU4 : kHeadU4;
          src += step;
          if (NORMS) nsrc += step / (kHeadU4 / kTile);   // 16 norms per 256-uint4 slice
        }
      };
#pragma unroll
      for (int x = 0; x < kAhead; ++x) {
        issue(kb[x], x);
        __builtin_amdgcn_sched_barrier(0);   // keep the ring's issue order (exact wait counts)
      }

      // open document: the last run of the previous tile
      int32_t cdoc = -1;
      float cmax = ninf;
      bool cshared = true;
      int64_t tau = w0 - layer0;                  // tile index within the layer
      int32_t dcur = -1;
      f32x4 tot[NT];

      for (int64_t ti = 0; ti < n_tw; ++ti) {
#pragma unroll
        for (int h = 0; h < kHeads; ++h) {
          // keeps each head's query-fragment reads from being hoisted into earlier heads
          __builtin_amdgcn_sched_barrier(0);
          issue(kb[(h + kAhead) % kRing], (h + kAhead) % kHeads);
          if (h == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) tot[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dcur = blk_doc[tau * kTile + j];     // consumed after the 8th head
          }

          // C[token][block] = Q . K^T for head h; lane: block j, tokens 4 g + r
          f32x4 acc[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 kk = {0.f, 0.f, 0.f, 0.f};   // K . K^T of the tile's 16 blocks for head h
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, kb[h % kRing][s]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, QS[h][s][nt][lane]), kf,
                                                                acc[nt], 0, 0, 0);
            if (!NORMS) kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, kf, kk, 0, 0, 0);
          }
          float rk;   // 1/max(|k|, eps) of block j, head h
          if (NORMS) {
            // head h, block j: lane 16 (h & 3) + j of hn[h >> 2]
            const float nh = __int_as_float(
                __builtin_amdgcn_ds_bpermute((16 * (h & 3) + j) * 4, __float_as_int(hn[h >> 2])));
            rk = __builtin_amdgcn_rcpf(fmaxf(nh, kNormEps));
          } else {
            // |k_j|^2 is the diagonal entry (j, j): row j = 4 g + r sits in lane group
            // g = j >> 2, register r = j & 3; the sum over the 4 lane groups hands it
            // to every lane of block j.
            const int jr = j & 3;
            const float k01 = (jr & 1) ? kk[1] : kk[0];
            const float k23 = (jr & 1) ? kk[3] : kk[2];
            float ssk = (jr & 2) ? k23 : k01;
            ssk = rows4_sum(g == (j >> 2) ? ssk : 0.f);
            rk = __builtin_amdgcn_rsqf(fmaxf(ssk, kNormEps * kNormEps));   // = 1/max(|k|, eps)
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float4 rq = *reinterpret_cast<const float4*>(&RQ[h][nt * 16 + 4 * g]);   // tokens 4 g + r
            tot[nt][0] += acc[nt][0] * (rq.x * rk);
            tot[nt][1] += acc[nt][1] * (rq.y * rk);
            tot[nt][2] += acc[nt][2] * (rq.z * rk);
            tot[nt][3] += acc[nt][3] * (rq.w * rk);
          }

          if (h == kHeads - 1) {
            // block j's max over the chunk's valid tokens, as a head mean
            float v = ninf;
            if (full_chunk) {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v = fmaxf(v, tot[nt][rr]);
            } else {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                  if (tmask & (1u << (nt * 4 + rr))) v = fmaxf(v, tot[nt][rr]);
            }
            v = rows4_max(v) * 0.125f;

            // Fold the tile's 16 block maxima into document maxima.  Blocks of a
            // document are contiguous, so a segmented suffix max within each run
            // of equal documents gives the run maxima; the last run stays open
            // because the document may continue in the next tile.
            // with interleaved tiles every tile's edge runs may continue elsewhere
            const bool t_first = !STREAM || ti == 0;
            const bool t_last = !STREAM || ti + 1 == n_tw;
            int32_t d = -1;
            if (lane < kTile) {
              d = dcur;
              if (d >= n_docs) d = -1;   // map entries are trusted only inside [0, n_docs)
            } else {
              v = ninf;
            }
            const int32_t d0 = __builtin_amdgcn_readlane(d, 0);
            if (cdoc >= 0 && cdoc != d0) {      // this tile does not continue the open document
              if (lane == 0) emit_doc(lcodes, cdoc, cmax, cshared || !exclusive);
              cdoc = -1;
            }
            bool run0_shared = t_first;
            if (cdoc >= 0) {                    // lane 0's run continues the open document
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
            const int hl = 63 - __builtin_clzll(heads);      // head lane of the last run
            const int32_t dl = __builtin_amdgcn_readlane(d, hl);
            const float vl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), hl));
            if (head && lane != hl && d >= 0)
              emit_doc(lcodes, d, v, (lane == 0 ? run0_shared : false) || !exclusive);
            cdoc = dl;
            cmax = vl;
            cshared = hl == 0 ? run0_shared : false;
            if (t_last) {                       // the run ends here
              if (cdoc >= 0 && lane == 0) emit_doc(lcodes, cdoc, cmax, true);
              cdoc = -1;
            }
            tau += tstep;
          }
        }
      }
    }
    seg = seg_end;
  }
}

// ------------------------------------------------------ many query chunks
//
// When several query chunks re-read every key range (B > 1, or more than 64 tokens), the
// kernel above is bound by how fast a CU's loads come back from L2: every chunk's
// workgroup reads every key tile, about 64 bytes per clock and CU at full matrix rate,
// and a CU's L1 sustains about half of that at the L2's latency.  Here a workgroup takes
// CP = 2 chunks, so each key byte serves 128 tokens.  Each of its 8 waves owns one head:
// it keeps that head's fragments of both chunks in registers (128 VGPRs) and takes the
// head's 4 KiB slice of every tile of the range, so the workgroup reads each key byte once
// per tile and no product touches LDS.  The products are K . Q^T (keys as the A operand),
// so a lane owns one token column and four blocks: the token's inverse norm is one value
// per lane, the blocks' norms a 16-byte load.
//
// LDS carries only the sum over heads.  Each wave adds its scaled cosines, as fixed-point
// integers, into one of kSlots tile slots (integer addition, so the sum does not depend on
// the order in which the waves arrive) and counts itself in the slot's counter one tile
// later (by then its adds are long complete).  Tile t is folded by wave t mod 8, kFoldLag
// tiles later: it waits for the count to reach 8, takes the max over tokens, folds the
// tile's blocks into document maxima, clears the slot and bumps its generation, which the
// adds of tile t + kSlots wait for.  There is no barrier, and no wait that a slower wave
// depends on: the slowest wave's slot was folded by a wave ahead of it, and every wave's
// count of a tile precedes its own next wait.
//
// Fixed point: a cosine c in [-1, 1] is held as round(c * 2^21).  fma(x, s, 1.5 * 2^23)
// with x s = c 2^21 leaves round(c 2^21) in the low mantissa bits of the result (exactly,
// for |c 2^21| < 2^22), so the bit patterns of the 8 heads' results add, as 32-bit
// integers, to 8 (1.5 * 2^23 bits) + the sum of the rounded terms.  Each term is off by at
// most 2^-22, the head mean by at most 2^-22 as well.  Two sums travel as one 64-bit add:
// the low word's eight biased terms carry exactly 2 into the high word.
constexpr int kSlots = 8;                         // tile slots of the head sum in LDS
constexpr int kHRing = 4;                         // tiles of key slices held in registers (one chunk)
constexpr int kHAhead = 3;                        // tiles in flight beyond the current one
constexpr int kFoldLag = 3;                       // tiles between a tile's adds and its fold
constexpr float kFixScale = 2097152.0f;           // 2^21 units per unit of cosine
constexpr float kFixMagic = 12582912.0f;          // 1.5 * 2^23
constexpr uint32_t kFixMagicBits = 0x4B400000u;   // its bit pattern
constexpr float kFixToMean = 1.0f / 16777216.0f;  // 2^-21 per unit, over 8 heads

template <int NT, bool NORMS, int CP>
__global__ void __launch_bounds__(kScanWG)
route_heads_kernel(const uint16_t* __restrict__ qr, int32_t B, int32_t T, int32_t n_tc,
                   const uint4* __restrict__ krt, int64_t tiles, const int32_t* __restrict__ blk_doc,
                   int32_t n_docs, int32_t L, int32_t R, int32_t exclusive, uint32_t* __restrict__ codes,
                   const float* __restrict__ knorm) {
  static_assert(kFoldLag < kHeads && kFoldLag + 2 < kSlots, "a wave folds each tile it owns before its next one");
  // two chunks' query fragments take 128 VGPRs: then the key ring holds two tiles
  constexpr int kRingT = CP == 2 ? 2 : kHRing;
  constexpr int kAheadT = kRingT - 1;
  __shared__ uint64_t s_sum[kSlots][CP][NT * 2][64];   // head sums of row pairs: [slot][chunk][pair][lane]
  __shared__ int32_t s_cnt[kSlots];                    // heads added to the slot's tile
  __shared__ int32_t s_gen[kSlots];                    // tiles of the slot folded so far

  // placement as in route_mfma_kernel: the chunk groups sharing a range sit on one XCD
  const int C = (n_tc * B);                      // query chunks
  const int G = (int)(gridDim.x / (unsigned)R);  // groups of CP chunks
  int r, gidx;
  {
    const int i = (int)blockIdx.x;
    if ((R & 7) == 0) {
      const int xcd = i & 7, slot = i >> 3;
      r = xcd + 8 * (slot / G);
      gidx = slot % G;
    } else {
      r = i / G;
      gidx = i % G;
    }
  }
  // chunk cp of the group; a missing last chunk repeats the group's first and is never folded
  int cb[CP], ct[CP];
  bool cvalid[CP];
#pragma unroll
  for (int cp = 0; cp < CP; ++cp) {
    int c = gidx * CP + cp;
    cvalid[cp] = c < C;
    if (!cvalid[cp]) c = gidx * CP;
    cb[cp] = c / n_tc;
    ct[cp] = (c % n_tc) * kTokChunk;
  }
  const int64_t W = (int64_t)L * tiles;
  const int64_t it_begin = W * r / R;
  const int64_t it_end = W * (r + 1) / R;
  if (it_begin >= it_end) return;                // uniform across the workgroup

  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // this wave's head
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int j = lane & 15;
  const float ninf = -__builtin_huge_valf();

  for (int i = threadIdx.x; i < kSlots * CP * NT * 2 * 64; i += kScanWG) (&s_sum[0][0][0][0])[i] = 0ull;
  if (threadIdx.x < kSlots) {
    s_cnt[threadIdx.x] = 0;
    s_gen[threadIdx.x] = 0;
  }
  __syncthreads();

  // accumulator column of this lane: token 16 nt + j of its chunk
  bool full_chunk[CP];
  uint32_t tmask[CP];
#pragma unroll
  for (int cp = 0; cp < CP; ++cp) {
    full_chunk[cp] = ct[cp] + NT * 16 <= T;
    tmask[cp] = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (ct[cp] + nt * 16 + j < T) tmask[cp] |= 1u << nt;
  }
  const uint32_t sum_bias = (uint32_t)kHeads * kFixMagicBits;   // modulo 2^32

  int64_t k = 0;   // tiles walked by the workgroup (every wave walks the same sequence)
  for (int64_t seg = it_begin; seg < it_end;) {
    const int layer = (int)(seg / tiles);
    const int64_t layer0 = (int64_t)layer * tiles;
    const int64_t seg_end = it_end < layer0 + tiles ? it_end : layer0 + tiles;
    const int n_t = (int)uniform64(seg_end - seg);   // tiles of the segment (< 2^31)

    // head h of each chunk's query as A-operand fragments (rows: tokens 16 nt + j; k: dims
    // 32 s + 8 g .. + 7) and its inverse norms in fixed-point units, in accumulator order.
    // s_rq[h] is this wave's own row, and one wave's LDS accesses complete in order.
    u32x4 qf[CP][4][NT];
    float rqs[CP][NT];   // token 16 nt + j of chunk cp (the accumulators' column)
#pragma unroll
    for (int cp = 0; cp < CP; ++cp) {
      const uint16_t* qb = qr + (((int64_t)layer * B + cb[cp]) * T) * kRow + h * kDim + g * 8;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = ct[cp] + nt * 16 + j;
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (tok < T) v = *reinterpret_cast<const u32x4*>(qb + (int64_t)tok * kRow + s * 32);
          qf[cp][s][nt] = v;
          ss += sumsq8(v);
        }
        rqs[cp][nt] = kFixScale / fmaxf(sqrtf(rows4_sum(ss)), kNormEps);
      }
    }

    // the ring: per tile this head's four 1 KiB key fragments, the blocks' norms (NORMS)
    // and their documents; loads are unconditional (past the segment's end the last tile
    // is fetched again) so that every wait is an exact count.  Wave-uniform addresses
    // (scalar registers); each lane adds its own offset.
    const u32x4* src = reinterpret_cast<const u32x4*>(krt + seg * kTileU4 + h * kHeadU4);
    const float* nsrc = NORMS ? knorm + (seg * kHeads + h) * kTile : nullptr;
    const int32_t* dsrc = blk_doc + (seg - layer0) * kTile;
    int issued = 0;
    u32x4 kb[kRingT][4];
    float4 nb[kRingT];
    int32_t db[kRingT];
    int cnt_slot = -1;      // slot of the tile added but not yet counted
    bool pend = false;      // a tile this wave is to fold
    int64_t pend_k = 0;
    int32_t pend_d = -1;
    auto issue = [&](int q) {
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[q][s] = src[lane + s * 64];
      if (NORMS) nb[q] = *reinterpret_cast<const float4*>(nsrc + 4 * g);
      db[q] = dsrc[j];
      if (issued + 1 < n_t) {
        ++issued;
        src += kTileU4;
        if (NORMS) nsrc += kHeads * kTile;
        dsrc += kTile;
      }
    };
#pragma unroll
    for (int q = 0; q < kAheadT; ++q) {
      issue(q);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Fold of a tile whose head sums are complete, per chunk: the max over the chunk's valid
    // tokens per block, then the blocks' runs of equal documents into document maxima.
    // Tiles are folded independently, so a run at either edge of the tile may continue in a
    // neighbouring tile and is emitted with an atomic max; runs inside are stored directly
    // when no other workgroup writes this row.
    auto fold = [&]() {
      const int slot = (int)(pend_k & (kSlots - 1));
      while (__builtin_amdgcn_readfirstlane(
                 __hip_atomic_load(&s_cnt[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != kHeads)
        __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      // The slot holds, at [cp][2 nt + rp][16 g' + j'], the pair of sums for blocks
      // 4 g' + 2 rp (low word) and 4 g' + 2 rp + 1 (high word) of token 16 nt + j'.  Lane
      // (g, jb) takes block jb over tokens 16 nt + 4 g + i (i < 4), reading only its word;
      // the biased sums stay inside [bias - 2^24, bias + 2^24], so their unsigned max is the
      // max of the sums (the high word carries 2 more, from the low word).
      const int jb = lane & 15;
      const int widx = (((jb >> 1) & 1) * 64 + 16 * (jb >> 2) + 4 * g) * 2 + (jb & 1);   // 32-bit word
      const uint32_t wbias = sum_bias + (uint32_t)(2 * (jb & 1));
      uint32_t mxu[CP];
#pragma unroll
      for (int cp = 0; cp < CP; ++cp) {
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(&s_sum[slot][cp][0][0]) + widx;
        mxu[cp] = 0u;
        if (full_chunk[cp]) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mxu[cp] = max(mxu[cp], sw[(nt * 2 * 64 + i) * 2]);
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = sw[(nt * 2 * 64 + i) * 2];
              if (ct[cp] + nt * 16 + 4 * g + i < T) mxu[cp] = max(mxu[cp], w);
            }
        }
      }
      // clear the slot: each lane its own entries (after this wave's reads of them, in order)
#pragma unroll
      for (int cp = 0; cp < CP; ++cp)
#pragma unroll
        for (int pr = 0; pr < NT * 2; ++pr) s_sum[slot][cp][pr][lane] = 0ull;
      if (lane == 0) s_cnt[slot] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0)
        __hip_atomic_store(&s_gen[slot], (int32_t)(pend_k / kSlots) + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
      int32_t d = -1;
      if (lane < kTile) {
        d = pend_d;
        if (d >= n_docs) d = -1;   // map entries are trusted only inside [0, n_docs)
      }
      const int32_t dprev = row_shr<1>(d, -2);
      const bool head = lane < kTile && (lane == 0 || dprev != d);
      const uint64_t heads = __ballot(head);
      const int hl = 63 - __builtin_clzll(heads);      // head lane of the last run
#pragma unroll
      for (int cp = 0; cp < CP; ++cp) {
        if (!cvalid[cp]) continue;                     // uniform
        // block jb's max over the chunk's valid tokens (0: none in this lane), as a head mean
        float v = mxu[cp] != 0u ? (float)(int32_t)(mxu[cp] - wbias) * kFixToMean : ninf;
        v = rows4_max(v);
        if (lane >= kTile) v = ninf;
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
        uint32_t* lcodes = codes + ((int64_t)layer * B + cb[cp]) * n_docs;
        if (head && d >= 0) emit_doc(lcodes, d, v, lane == 0 || lane == hl || !exclusive);
      }
    };

    for (int i0 = 0; i0 < n_t; i0 += kRingT) {
#pragma unroll
      for (int u = 0; u < kRingT; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        issue((u + kAheadT) % kRingT);
        __builtin_amdgcn_sched_barrier(0);
        const int i = i0 + u;
        if (i < n_t) {
          // the slot's generation, read before the products so that its latency hides behind them
          const int slot = (int)(k & (kSlots - 1));
          const int32_t gen = (int32_t)(k / kSlots);
          int32_t gv = __hip_atomic_load(&s_gen[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          // C[block][token] = K . Q^T for head h; lane: token 16 nt + j, blocks 4 g + rr
          f32x4 acc[CP][NT];
#pragma unroll
          for (int cp = 0; cp < CP; ++cp)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[cp][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, kb[u][s]);
#pragma unroll
            for (int cp = 0; cp < CP; ++cp)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                acc[cp][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, __builtin_bit_cast(bf16x8, qf[cp][s][nt]),
                                                                      acc[cp][nt], 0, 0, 0);
            if (!NORMS) kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, kf, kk, 0, 0, 0);
          }
          float rk[4];   // 1/max(|k|, eps) of blocks 4 g + rr, head h
          if (NORMS) {
            rk[0] = __builtin_amdgcn_rcpf(fmaxf(nb[u].x, kNormEps));
            rk[1] = __builtin_amdgcn_rcpf(fmaxf(nb[u].y, kNormEps));
            rk[2] = __builtin_amdgcn_rcpf(fmaxf(nb[u].z, kNormEps));
            rk[3] = __builtin_amdgcn_rcpf(fmaxf(nb[u].w, kNormEps));
          } else {
            // |k_b|^2 is the diagonal entry (b, b) of K K^T: row b = 4 g' + rr' sits in lane
            // group g' = b >> 2, register rr' = b & 3, column lane j = b
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int src_lane = 16 * g + 4 * g + rr;
              const float d2 = __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane * 4, __float_as_int(kk[rr])));
              rk[rr] = __builtin_amdgcn_rsqf(fmaxf(d2, kNormEps * kNormEps));
            }
          }
          // the slot is free once its previous tile (kSlots tiles back) is folded
          while (__builtin_amdgcn_readfirstlane(gv) != gen) {
            __builtin_amdgcn_s_sleep(1);
            gv = __hip_atomic_load(&s_gen[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
          for (int cp = 0; cp < CP; ++cp)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int rp = 0; rp < 2; ++rp) {
                const uint32_t y0 = __float_as_uint(
                    __builtin_fmaf(acc[cp][nt][2 * rp], rqs[cp][nt] * rk[2 * rp], kFixMagic));
                const uint32_t y1 = __float_as_uint(
                    __builtin_fmaf(acc[cp][nt][2 * rp + 1], rqs[cp][nt] * rk[2 * rp + 1], kFixMagic));
                __hip_atomic_fetch_add(&s_sum[slot][cp][nt * 2 + rp][lane], (uint64_t)y0 | ((uint64_t)y1 << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              }
          // count the previous tile in its slot now: its adds have long completed, so the
          // release finds nothing to wait for (this tile is counted one tile later)
          if (cnt_slot >= 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0)
              __hip_atomic_fetch_add(&s_cnt[cnt_slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          cnt_slot = slot;
          if ((int)(k & (kHeads - 1)) == h) {   // this wave folds the tile, kFoldLag tiles from now
            pend = true;
            pend_k = k;
            pend_d = db[u];
          }
          ++k;
          if (pend && k - pend_k > kFoldLag) {
            fold();
            pend = false;
          }
        }
      }
    }
    if (cnt_slot >= 0) {   // the segment's last tile
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) __hip_atomic_fetch_add(&s_cnt[cnt_slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      cnt_slot = -1;
    }
    if (pend) {     // the segment's last tiles
      fold();
      pend = false;
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
                  int64_t n_blk, int64_t tiles,
                  const int32_t* __restrict__ blk_doc, int32_t n_docs, uint32_t* __restrict__ codes) {
  static_assert(TMAX * kRow / 8 == 8 * 256, "eight 16-byte query chunks per thread");
  __shared__ float q_s[TMAX * kRow];
  __shared__ float rq_s[TMAX * kHeads];
  const int layer = blockIdx.z, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  // this wave's tile: all 8 heads' key fragments requested first (the loads are independent
  // of the query), clamped to the last tile for waves past the end (never used)
  const uint4* kt = krt + ((int64_t)layer * tiles + (tile < tiles ? tile : tiles - 1)) * kTileU4;
  uint4 kw[kHeads][4];
#pragma unroll
  for (int h = 0; h < kHeads; ++h)
#pragma unroll
    for (int s = 0; s < 4; ++s) kw[h][s] = kt[h * kHeadU4 + s * 64 + lane];
  // the query, 16 bytes per load (chunk i: token i / 128, dims 8 (i % 128) .. + 7), to fp32 in LDS;
  // the 16 chunks of one (token, head) sit in the 16 lanes of a DPP row, whose sum of squares
  // gives the head's inverse norm
  const uint4* qbase = reinterpret_cast<const uint4*>(qr + (((int64_t)layer * B + b) * T) * kRow);
  uint4 qw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = tid + 256 * u;
    qw[u] = i / 128 < T ? qbase[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = tid + 256 * u;
    const uint32_t p[4] = {qw[u].x, qw[u].y, qw[u].z, qw[u].w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(p[e]), c = bf16_hi(p[e]);
      q_s[8 * i + 2 * e] = a;
      q_s[8 * i + 2 * e + 1] = c;
      ss += a * a + c * c;
    }
    ss = row16_sum(ss);
    if ((tid & 15) == 0) rq_s[i / 16] = 1.0f / fmaxf(sqrtf(ss), kNormEps);   // (token, head) = i / 16
  }
  __syncthreads();
  if (tile >= tiles) return;

  float sc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) sc[t] = 0.f;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {   // unrolled: kw stays in registers
    float x[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 w = kw[h][s];
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

constexpr int64_t kMaxRangeTiles = 1024;   // per range when several query chunks share it
constexpr int64_t kMinStreamTiles = 512;   // per range when one query chunk streams the keys

int choose_ranges(int C, int cus, int64_t W) {
  // C: the workgroups that share each range (one per query chunk, or per pair of chunks).
  // R ranges per query chunk; the persistent grid of R*C workgroups (one per CU at a
  // time) should fill whole waves of the device: pick R in [ceil(cus/C), 4*ceil(cus/C)]
  // with the best filled fraction.  When several query chunks share each range, a
  // multiple of 8 wins ties, so that each range's workgroups sit on one XCD (one L2);
  // otherwise the smallest R wins.
  int best = 1;
  if (C < cus) {
    const int r0 = (cus + C - 1) / C;
    best = r0;
    double best_eff = 0.0;
    bool best_x8 = false;
    for (int R = r0; R <= 4 * r0; ++R) {
      const long total = (long)R * C;
      const long waves = (total + cus - 1) / cus;
      const double eff = (double)total / (double)(waves * cus);
      const bool x8 = C > 1 && (R & 7) == 0;
      if (eff > best_eff + 1e-9 || (eff > best_eff - 1e-9 && x8 && !best_x8)) {
        best_eff = eff;
        best = R;
        best_x8 = x8;
      }
    }
  }
  if (C == 1) {
    // One query chunk: each range is read once, with no sharing to protect; still, several
    // rounds of ranges (up to 8, each range at least kMinStreamTiles) measured faster and
    // steadier than one range per CU: 100M-token memory, 8.26-8.40 ms over nine processes
    // with 8 to 32 rounds, 8.41-8.92 ms with one.
    int64_t rounds = W / ((int64_t)cus * kMinStreamTiles);
    rounds = rounds < 1 ? 1 : (rounds > 8 ? 8 : rounds);
    return best == cus ? (int)(rounds * cus) : best;
  }
  // Shared ranges are kept short: the workgroups reading one range drift apart over a long
  // run until the tiles one of them fetched are gone from L2 before the others read them.
  // Ranges of at most kMaxRangeTiles tiles (32 MiB) keep the repeats in L2; R stays a
  // multiple of 8 and, where one is near, R*C a whole number of waves.
  // (The grid, R*C workgroups, stays below 2^31.)
  const int64_t rcap = (int64_t)0x7FFFFFFF / C;
  int64_t rmin = (W + kMaxRangeTiles - 1) / kMaxRangeTiles;
  if (rmin <= best || best >= rcap) return best;
  rmin = (rmin + 7) / 8 * 8;
  for (int64_t R = rmin; R <= rmin + 8 * 64 && R <= rcap; R += 8)
    if ((R * C) % cus == 0) return (int)R;
  return (int)(rmin < rcap ? rmin : rcap);
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
                               const float* knorm, int64_t n_blk, const int32_t* blk_doc, int32_t n_docs,
                               int32_t accumulate, float* doc_scores, hipStream_t s) {
  const int64_t tiles = route_tiles(n_blk);
  const int64_t n_codes = (int64_t)L * B * n_docs;
  uint32_t* codes = reinterpret_cast<uint32_t*>(doc_scores);
  const int cus = stream_cus(s);                 // the persistent grid fills the stream's CUs
  const int fill_grid = (int)((n_codes + 255) / 256 < cus * 4 ? (n_codes + 255) / 256 : cus * 4);

  hipLaunchKernelGGL(codes_init_kernel, dim3(fill_grid), dim3(256), 0, s, codes, n_codes, accumulate);
  if (tiles > 0) {
    if (T >= 16) {
      const int n_tc = (T + kTokChunk - 1) / kTokChunk;
      const int C = B * n_tc;
      // one chunk: route_mfma_kernel streams the keys once; several: route_heads_kernel, two
      // chunks per workgroup (R ranges x G workgroups sharing each range)
      const bool stream = C == 1;
      const int G = stream ? 1 : (C + 1) / 2;
      const int R = choose_ranges(G, cus, (int64_t)L * tiles);
      const int NT = T >= kTokChunk ? 4 : (T + 15) / 16;
      const dim3 grid((unsigned)(R * G));
      const uint4* kt = reinterpret_cast<const uint4*>(krt);
      const int excl = (n_tc == 1 && !accumulate) ? 1 : 0;
#define MSA_ROUTE_LAUNCH(NTV, ST, NM)                                                                       \
  hipLaunchKernelGGL((route_mfma_kernel<NTV, ST, NM>), grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,   \
                     blk_doc, n_docs, L, R, excl, codes, knorm)
#define MSA_ROUTE_HEADS(NTV, NM)                                                                       \
  hipLaunchKernelGGL((route_heads_kernel<NTV, NM, 2>), grid, dim3(kScanWG), 0, s, qr, B, T, n_tc, kt, tiles,  \
                     blk_doc, n_docs, L, R, excl, codes, knorm)
#define MSA_ROUTE_NT(NTV)                                          \
  if (stream) {                                                    \
    if (knorm) MSA_ROUTE_LAUNCH(NTV, true, true);                  \
    else MSA_ROUTE_LAUNCH(NTV, true, false);                       \
  } else {                                                         \
    if (knorm) MSA_ROUTE_HEADS(NTV, true);                         \
    else MSA_ROUTE_HEADS(NTV, false);                              \
  }
      switch (NT) {
        case 1: MSA_ROUTE_NT(1); break;
        case 2: MSA_ROUTE_NT(2); break;
        case 3: MSA_ROUTE_NT(3); break;
        default: MSA_ROUTE_NT(4); break;
      }
#undef MSA_ROUTE_NT
#undef MSA_ROUTE_HEADS
#undef MSA_ROUTE_LAUNCH
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
