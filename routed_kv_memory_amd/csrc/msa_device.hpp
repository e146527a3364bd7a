// msa_device.hpp -- device-side helpers shared by the libmsa kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kHeads = 8;
constexpr int kDim = 128;
constexpr int kRow = kHeads * kDim;        // 1024 bf16 per block/token row
constexpr int kBlockTokens = 64;
constexpr int kTile = 16;                  // blocks per route-key tile
constexpr int kTileElems = kTile * kRow;   // 16384 bf16 = 32 KiB
constexpr float kNormEps = 1e-8f;
constexpr int kMaxTopk = 256;           // MSA_MAX_TOPK

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the
// 8-byte chunks addressed by lanes 4 e + i / 4 (e = 0..3) -- a 16 x 4 transpose of
// 16-bit elements.  `p` points into LDS.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Order-preserving map fp32 -> uint32 (larger float <=> larger code).  Code 0 is
// below every float's code and stands for "no score yet" (-inf on decode).
__device__ __forceinline__ uint32_t ordered_code(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_code(uint32_t c) {
  if (c == 0u) return -__builtin_huge_valf();
  uint32_t u = (c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c;
  return __uint_as_float(u);
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane gets it.
__device__ __forceinline__ float row16_max(float v) {
  int x = __float_as_int(v);
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false)));
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false)));
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false)));
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false)));
  return v;
}

// Sum over the 16 lanes of a DPP row; every lane gets it.
__device__ __forceinline__ float row16_sum(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return v;
}

// Sum / max over the four 16-lane rows at the same row position (lanes l, l^16,
// l^32, l^48) with the gfx950 row-swap instructions: VALU only, no LDS crossbar.
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// DPP row shifts: lane i of each 16-lane row receives lane i + N (shl) or i - N (shr)
// of the same row; lanes whose source falls outside the row receive `fill`.
template <int N>
__device__ __forceinline__ int row_shl(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x100 + N, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ int row_shr(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x110 + N, 0xF, 0xF, false);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Per-document max of block scores held one per lane in lanes [0, n) of a wave
// (lanes >= n pass doc = -1).  Blocks of a document are contiguous, so a
// segmented suffix max inside each run leaves the run's max in its first lane,
// which folds it into the document score with one atomic max on its code.
__device__ __forceinline__ void flush_doc_max(float v, int32_t doc, int n, int32_t n_docs,
                                              uint32_t* __restrict__ codes) {
  const int lane = __lane_id();
  if (lane >= n || doc >= n_docs) doc = -1;   // map entries are trusted only inside [0, n_docs)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float vo = __shfl_down(v, off, 64);
    int32_t dn = __shfl_down(doc, off, 64);
    if (lane + off < 64 && dn == doc) v = fmaxf(v, vo);
  }
  int32_t dprev = __shfl_up(doc, 1, 64);
  bool head = (lane == 0) || (dprev != doc);
  if (head && doc >= 0) atomicMax(codes + doc, ordered_code(v));
}

}  // namespace msa
