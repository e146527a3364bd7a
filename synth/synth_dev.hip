// synth_dev.hip -- device side of the seeded synthetic-input generator.
//
// This module only makes inputs; it holds none of the routing/pooling/decode
// arithmetic.  The host side (synth.py) implements the same definitions in
// numpy, so any element can be regenerated on the CPU by its index:
//
//   word(seed, stream, j) = SplitMix64 output j of the state
//                           base = mix64(seed ^ (stream << 32)), i.e.
//                           mix64(base + (j + 1) * 0x9E3779B97F4A7C15)
//   (mix64 = the SplitMix64 finaliser of Steele, Lea & Flood, OOPSLA 2014).
//   element e of a stream  = table[(word(seed, stream, e >> 2) >> (16 * (e & 3))) & 0xFFFF],
//   where table (uploaded by the caller) holds bf16 N(0,1) quantiles.
//
//   needle value           = bf16_rne(q + 0.3f * z) in fp32, two separately
//                            rounded operations (no fused multiply-add), with
//                            q a bf16 query value and z a table value.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_API extern "C" __attribute__((visibility("default")))

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word_at(uint64_t base, uint64_t j) {
  return mix64(base + (j + 1ull) * 0x9E3779B97F4A7C15ull);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Fill out[i] = element (e0 + i) of (seed, stream), i < n.  The table is first
// copied into LDS (128 KiB) by each workgroup.
__global__ void __launch_bounds__(1024) fill_kernel(uint16_t* __restrict__ out, int64_t n, uint64_t base,
                                                    int64_t e0, const uint16_t* __restrict__ table) {
  extern __shared__ uint16_t tab[];
  for (int i = threadIdx.x; i < 65536 / 8; i += blockDim.x)
    reinterpret_cast<uint4*>(tab)[i] = reinterpret_cast<const uint4*>(table)[i];
  __syncthreads();
  // Work in 4-element groups aligned to the stream's word grid.
  const int64_t g0 = e0 >> 2;                    // first word
  const int64_t g1 = (e0 + n + 3) >> 2;          // one past the last word
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool aligned = ((e0 & 3) == 0) && ((reinterpret_cast<uintptr_t>(out) & 7) == 0);
  for (int64_t g = g0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < g1; g += stride) {
    uint64_t w = word_at(base, (uint64_t)g);
    int64_t i0 = (g << 2) - e0;
    if (aligned && i0 + 4 <= n) {
      uint64_t v = (uint64_t)tab[w & 0xFFFFu] | ((uint64_t)tab[(w >> 16) & 0xFFFFu] << 16) |
                   ((uint64_t)tab[(w >> 32) & 0xFFFFu] << 32) | ((uint64_t)tab[(w >> 48) & 0xFFFFu] << 48);
      *reinterpret_cast<uint64_t*>(out + i0) = v;
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        int64_t i = i0 + s;
        if (i >= 0 && i < n) out[i] = tab[(w >> (16 * s)) & 0xFFFFu];
      }
    }
  }
}

// Needle planting.  For needle row j (0 <= j < n_rows):
//   dst row  = rows + (row_idx[j] - row_base) * 1024
//   q row    = qr + q_row[j] * 1024          (bf16 [*][8][128])
//   z        = element (row_idx[j] + n_rows_total * layer) * 1024 + c of the needle stream
//   value[c] = bf16_rne(q[c] + 0.3f * z[c])
__global__ void __launch_bounds__(256) plant_kernel(uint16_t* __restrict__ rows, int64_t row_base,
                                                    int64_t n_rows_total, int32_t layer,
                                                    const int64_t* __restrict__ row_idx,
                                                    const int64_t* __restrict__ q_row,
                                                    int32_t n_rows, const uint16_t* __restrict__ qr,
                                                    uint64_t base, const uint16_t* __restrict__ table) {
#pragma clang fp contract(off)
  int j = blockIdx.x;
  if (j >= n_rows) return;
  const int64_t r = row_idx[j];
  const uint16_t* q = qr + q_row[j] * 1024;
  uint16_t* dst = rows + (r - row_base) * 1024;
  const int64_t ebase = ((int64_t)layer * n_rows_total + r) * 1024;
  for (int c = threadIdx.x; c < 1024; c += blockDim.x) {
    int64_t e = ebase + c;
    uint64_t w = word_at(base, (uint64_t)(e >> 2));
    uint16_t zb = table[(w >> (16 * (e & 3))) & 0xFFFFu];
    float z = __uint_as_float((uint32_t)zb << 16);
    float qv = __uint_as_float((uint32_t)q[c] << 16);
    float prod = 0.3f * z;   // rounded on its own (contraction is off here)
    float v = qv + prod;
    dst[c] = f32_to_bf16_rne(v);
  }
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

// Returns 0 on success, else the hipError_t value.
SYNTH_API int synth_fill(uint16_t* out, int64_t n, uint64_t seed, uint32_t stream, int64_t e0,
                         const uint16_t* table, void* hip_stream) {
  if (n <= 0) return 0;
  uint64_t base = host_mix64(seed ^ ((uint64_t)stream << 32));
  int dev = 0;
  (void)hipGetDevice(&dev);
  int cus = 256;
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  int64_t groups = (n + 7) / 4 + 1;
  int64_t want = (groups + 1023) / 1024;
  int grid = (int)(want < (int64_t)cus * 4 ? want : (int64_t)cus * 4);
  if (grid < 1) grid = 1;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fill_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 65536 * (int)sizeof(uint16_t));
    attr_set = true;
  }
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(1024), 65536 * sizeof(uint16_t),
                     (hipStream_t)hip_stream, out, n, base, e0, table);
  return (int)hipGetLastError();
}

SYNTH_API int synth_plant(uint16_t* rows, int64_t row_base, int64_t n_rows_total, int32_t layer,
                          const int64_t* row_idx, const int64_t* q_row, int32_t n_rows,
                          const uint16_t* qr, uint64_t seed, uint32_t stream, const uint16_t* table,
                          void* hip_stream) {
  if (n_rows <= 0) return 0;
  uint64_t base = host_mix64(seed ^ ((uint64_t)stream << 32));
  hipLaunchKernelGGL(plant_kernel, dim3(n_rows), dim3(256), 0, (hipStream_t)hip_stream, rows, row_base,
                     n_rows_total, layer, row_idx, q_row, n_rows, qr, base, table);
  return (int)hipGetLastError();
}
