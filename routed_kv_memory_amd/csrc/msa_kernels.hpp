// msa_kernels.hpp -- host-side launchers of the libmsa kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct DeviceInfo {
  int cus;       // compute units
};
DeviceInfo device_info();
// CUs a stream may run on: the popcount of its CU mask (all of the device's CUs for an
// unmasked stream).  Persistent grids are sized by it, so a scan on a CU-masked stream fills
// exactly the CUs it was given and leaves the others to work on other streams.
int stream_cus(hipStream_t s);

inline int64_t route_tiles(int64_t n_blk) { return (n_blk + 15) / 16; }

// pool.hip
hipError_t launch_pool(int32_t L, const uint16_t* k, const uint16_t* v, const uint16_t* kr, int64_t n_tok,
                       const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                       uint16_t* kbar, uint16_t* vbar, uint16_t* krt, float* krn, hipStream_t s);
hipError_t launch_pack(int32_t L, const uint16_t* rows, int64_t n_blk, uint16_t* krt, float* krn,
                       hipStream_t s);

// route.hip
hipError_t launch_blk_doc(const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk, int32_t* blk_doc, hipStream_t s);
hipError_t launch_route_scores(int32_t L, const uint16_t* qr, int32_t B, int32_t T, const uint16_t* krt,
                               const float* knorm, int64_t n_blk, const int32_t* blk_doc, int32_t n_docs,
                               int32_t accumulate, float* doc_scores, hipStream_t s);

// topk.hip
size_t topk_workspace_bytes(int64_t rows, int32_t n_docs, int32_t k);
hipError_t launch_topk(int64_t rows, const float* scores, int32_t n_docs, int32_t k, int32_t* ids,
                       float* out_scores, void* ws, hipStream_t s);

// gather.hip
hipError_t launch_gather(int32_t L, int32_t B, const int32_t* ids, int32_t k, const int64_t* doc_blk_off,
                         int32_t n_docs, const uint16_t* kbar, const uint16_t* vbar, int64_t n_blk,
                         int32_t max_ctx, uint16_t* ctx_k, uint16_t* ctx_v, int32_t* ctx_len, hipStream_t s);

// decode.hip
int decode_rows_per_split();
hipError_t launch_decode(int32_t L, int32_t B, int32_t Hq, const uint16_t* q, const uint16_t* ctx_k,
                         const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx, const uint16_t* loc_k,
                         const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc, float scale, float* out,
                         void* ws, hipStream_t s);
hipError_t launch_encode(int32_t L, int32_t H, const uint16_t* x, int64_t n_tok, const uint16_t* w_k,
                         const uint16_t* w_v, const uint16_t* w_kr, const uint16_t* w_norm, float eps, float theta,
                         const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                         uint16_t* kbar, uint16_t* vbar, uint16_t* krt, float* krn, hipStream_t s);
hipError_t launch_prefill(int32_t L, int32_t B, int32_t T, int32_t Hq, const uint16_t* q, const uint16_t* ctx_k,
                          const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx, const uint16_t* loc_k,
                          const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc, float scale, float* out,
                          hipStream_t s);

}  // namespace msa
