// abi.cpp -- the C ABI of libmsa: argument validation, workspace carving and
// kernel launches (declared and documented in include/msa.h).
#include "msa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "msa_kernels.hpp"

#define MSA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The kernels move bf16 rows (and a few fp32 arrays) in 16-byte vectors: such pointers must be
// 16-byte aligned.  NULL entries (optional arguments) pass.
bool all_aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return false;
  return true;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace msa {

DeviceInfo device_info() {
  static int cached_cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{256};
  if (cached_cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached_cus[dev] = cus;
  }
  return DeviceInfo{cached_cus[dev]};
}

int stream_cus(hipStream_t s) {
  const int dev_cus = device_info().cus;
  uint32_t mask[32] = {0};                       // up to 1,024 CUs
  const uint32_t words = (uint32_t)((dev_cus + 31) / 32);
  if (words > 32) return dev_cus;
  if (hipExtStreamGetCUMask(s, words, mask) != hipSuccess) {
    (void)hipGetLastError();                     // not a launch error: leave no sticky status behind
    return dev_cus;
  }
  int n = 0;
  for (uint32_t w = 0; w < words; ++w) n += __builtin_popcount(mask[w]);
  return n > 0 && n < dev_cus ? n : dev_cus;
}

}  // namespace msa

MSA_API int msa_abi_version(void) { return MSA_ABI_VERSION; }

MSA_API const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "null pointer";
    case MSA_ERR_SHAPE: return "invalid shape or size";
    case MSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

MSA_API const char* msa_last_error(void) { return g_err; }

// ------------------------------------------------------------------ host helpers

MSA_API int msa_group_offsets_host(const int64_t* doc_ids_host, int64_t n_tok, int64_t* doc_tok_off_host,
                                   int32_t* n_docs_host) {
  if (!doc_tok_off_host || !n_docs_host || (n_tok > 0 && !doc_ids_host))
    return fail(MSA_ERR_NULL, "msa_group_offsets_host: null pointer");
  if (n_tok < 0) return fail(MSA_ERR_SHAPE, "msa_group_offsets_host: n_tok < 0");
  int64_t n = 0;
  for (int64_t i = 0; i < n_tok; ++i) {
    if (i == 0 || doc_ids_host[i] != doc_ids_host[i - 1]) {
      if (n >= INT32_MAX) return fail(MSA_ERR_SHAPE, "msa_group_offsets_host: too many documents");
      doc_tok_off_host[n++] = i;
    }
  }
  doc_tok_off_host[n] = n_tok;
  *n_docs_host = (int32_t)n;
  return MSA_OK;
}

MSA_API int msa_block_offsets_host(const int64_t* doc_tok_off_host, int32_t n_docs, int64_t* doc_blk_off_host,
                                   int64_t* n_blk_host, int32_t* max_doc_blocks_host) {
  if (!doc_tok_off_host || !doc_blk_off_host) return fail(MSA_ERR_NULL, "msa_block_offsets_host: null pointer");
  if (n_docs < 0) return fail(MSA_ERR_SHAPE, "msa_block_offsets_host: n_docs < 0");
  if (doc_tok_off_host[0] != 0) return fail(MSA_ERR_SHAPE, "msa_block_offsets_host: doc_tok_off[0] != 0");
  int64_t acc = 0;
  int64_t mx = 0;
  doc_blk_off_host[0] = 0;
  for (int32_t d = 0; d < n_docs; ++d) {
    const int64_t len = doc_tok_off_host[d + 1] - doc_tok_off_host[d];
    if (len < 0) return fail(MSA_ERR_SHAPE, "msa_block_offsets_host: doc_tok_off decreases at %d", d);
    const int64_t nb = (len + MSA_BLOCK_TOKENS - 1) / MSA_BLOCK_TOKENS;
    acc += nb;
    if (nb > mx) mx = nb;
    doc_blk_off_host[d + 1] = acc;
  }
  if (mx > INT32_MAX) return fail(MSA_ERR_SHAPE, "msa_block_offsets_host: document too long");
  if (n_blk_host) *n_blk_host = acc;
  if (max_doc_blocks_host) *max_doc_blocks_host = (int32_t)mx;
  return MSA_OK;
}

MSA_API int64_t msa_route_tiles(int64_t n_blk) { return n_blk <= 0 ? 0 : msa::route_tiles(n_blk); }

// ------------------------------------------------------------------------ A1

MSA_API int msa_pool_blocks(int32_t n_layers, const uint16_t* k, const uint16_t* v, const uint16_t* kr,
                            int64_t n_tok, const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
                            int64_t n_blk, uint16_t* kbar, uint16_t* vbar, uint16_t* krbar_route,
                            float* krbar_norm, void* stream) {
  // token rows may be NULL when there are no tokens, outputs when there are no blocks
  if ((n_tok > 0 && (!k || !v || !kr)) || !doc_tok_off || !doc_blk_off ||
      (n_blk > 0 && (!kbar || !vbar || !krbar_route)))
    return fail(MSA_ERR_NULL, "msa_pool_blocks: null pointer");
  if (!all_aligned16({k, v, kr, kbar, vbar, krbar_route}))
    return fail(MSA_ERR_SHAPE, "msa_pool_blocks: bf16 arrays must be 16-byte aligned");
  if (n_layers < 1 || n_docs < 1 || n_tok < 0 || n_blk < 0)
    return fail(MSA_ERR_SHAPE, "msa_pool_blocks: n_layers=%d n_docs=%d n_tok=%lld n_blk=%lld", n_layers, n_docs,
                (long long)n_tok, (long long)n_blk);
  if (msa::route_tiles(n_blk) > INT32_MAX / 3) return fail(MSA_ERR_UNSUPPORTED, "msa_pool_blocks: n_blk too large");
  return hip_status(msa::launch_pool(n_layers, k, v, kr, n_tok, doc_tok_off, doc_blk_off, n_docs, n_blk, kbar, vbar,
                                     krbar_route, krbar_norm, as_stream(stream)),
                    "msa_pool_blocks");
}

MSA_API int msa_pack_route_keys(int32_t n_layers, const uint16_t* krbar_rows, int64_t n_blk, uint16_t* krbar_route,
                                float* krbar_norm, void* stream) {
  if (n_blk > 0 && (!krbar_rows || !krbar_route)) return fail(MSA_ERR_NULL, "msa_pack_route_keys: null pointer");
  if (!all_aligned16({krbar_rows, krbar_route}))
    return fail(MSA_ERR_SHAPE, "msa_pack_route_keys: bf16 arrays must be 16-byte aligned");
  if (n_layers < 1 || n_blk < 0) return fail(MSA_ERR_SHAPE, "msa_pack_route_keys: n_layers=%d n_blk=%lld", n_layers,
                                             (long long)n_blk);
  if (msa::route_tiles(n_blk) > INT32_MAX) return fail(MSA_ERR_UNSUPPORTED, "msa_pack_route_keys: n_blk too large");
  return hip_status(msa::launch_pack(n_layers, krbar_rows, n_blk, krbar_route, krbar_norm, as_stream(stream)),
                    "msa_pack_route_keys");
}

// ------------------------------------------------------------------------ A2

MSA_API int msa_block_doc_map(const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk, int32_t* blk_doc,
                              void* stream) {
  if (!doc_blk_off || (n_blk > 0 && !blk_doc)) return fail(MSA_ERR_NULL, "msa_block_doc_map: null pointer");
  if (n_docs < 1 || n_blk < 0)
    return fail(MSA_ERR_SHAPE, "msa_block_doc_map: n_docs=%d n_blk=%lld", n_docs, (long long)n_blk);
  if (n_blk >= (int64_t)INT32_MAX - 32) return fail(MSA_ERR_UNSUPPORTED, "msa_block_doc_map: n_blk too large");
  return hip_status(msa::launch_blk_doc(doc_blk_off, n_docs, n_blk, blk_doc, as_stream(stream)),
                    "msa_block_doc_map");
}

static int check_route_args(const char* fn, int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T,
                            const uint16_t* krbar_route, const float* krbar_norm, int64_t n_blk,
                            const int32_t* blk_doc, int32_t n_docs) {
  if (!qr || (n_blk > 0 && (!krbar_route || !blk_doc))) return fail(MSA_ERR_NULL, "%s: null pointer", fn);
  if (!all_aligned16({qr, krbar_route, krbar_norm}))
    return fail(MSA_ERR_SHAPE, "%s: qr, the route keys and their norms must be 16-byte aligned", fn);
  if (n_layers < 1 || B < 1 || T < 1 || n_docs < 1 || n_blk < 0)
    return fail(MSA_ERR_SHAPE, "%s: n_layers=%d B=%d T=%d n_docs=%d n_blk=%lld", fn, n_layers, B, T, n_docs,
                (long long)n_blk);
  if (n_blk >= (int64_t)INT32_MAX - 32) return fail(MSA_ERR_UNSUPPORTED, "%s: n_blk too large", fn);
  if ((int64_t)B * ((T + 63) / 64) > INT32_MAX / 64) return fail(MSA_ERR_UNSUPPORTED, "%s: B*T too large", fn);
  if (T < 16 && ((int64_t)n_layers > 65535 || B > 65535))
    return fail(MSA_ERR_UNSUPPORTED, "%s: n_layers or B > 65535", fn);
  return MSA_OK;
}

MSA_API int msa_route_scores(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T, const uint16_t* krbar_route,
                             const float* krbar_norm, int64_t n_blk, const int32_t* blk_doc, int32_t n_docs, int32_t accumulate,
                             float* doc_scores, void* stream) {
  int st = check_route_args("msa_route_scores", n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc, n_docs);
  if (st) return st;
  if (!doc_scores) return fail(MSA_ERR_NULL, "msa_route_scores: null pointer");
  return hip_status(msa::launch_route_scores(n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc, n_docs,
                                             accumulate ? 1 : 0, doc_scores, as_stream(stream)),
                    "msa_route_scores");
}

// ------------------------------------------------------------------------ A3

MSA_API size_t msa_topk_docs_workspace_size(int32_t n_layers, int32_t B, int32_t n_docs, int32_t k) {
  if (n_layers < 1 || B < 1 || n_docs < 1 || k < 1) return 0;
  return msa::topk_workspace_bytes((int64_t)n_layers * B, n_docs, k) + 256;
}

MSA_API int msa_topk_docs(int32_t n_layers, int32_t B, const float* doc_scores, int32_t n_docs, int32_t k,
                          int32_t* topk_ids, float* topk_scores, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!doc_scores || !topk_ids || !workspace) return fail(MSA_ERR_NULL, "msa_topk_docs: null pointer");
  if (n_layers < 1 || B < 1 || n_docs < 1 || k < 1 || k > n_docs)
    return fail(MSA_ERR_SHAPE, "msa_topk_docs: n_layers=%d B=%d n_docs=%d k=%d", n_layers, B, n_docs, k);
  if (k > MSA_MAX_TOPK) return fail(MSA_ERR_UNSUPPORTED, "msa_topk_docs: k=%d > %d", k, MSA_MAX_TOPK);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_topk_docs: n_layers*B > 65535");
  const size_t need = msa_topk_docs_workspace_size(n_layers, B, n_docs, k);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "msa_topk_docs: workspace %zu < %zu bytes", workspace_bytes, need);
  return hip_status(msa::launch_topk((int64_t)n_layers * B, doc_scores, n_docs, k, topk_ids, topk_scores, workspace,
                                     as_stream(stream)),
                    "msa_topk_docs");
}

// ------------------------------------------------------------------ A2 + A3

MSA_API size_t msa_route_topk_workspace_size(int32_t n_layers, int32_t B, int32_t n_docs, int32_t k) {
  if (n_layers < 1 || B < 1 || n_docs < 1 || k < 1) return 0;
  const size_t scores = align256((size_t)n_layers * B * n_docs * sizeof(float));
  return scores + msa_topk_docs_workspace_size(n_layers, B, n_docs, k);
}

MSA_API int msa_route_topk(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T, const uint16_t* krbar_route,
                           const float* krbar_norm, int64_t n_blk, const int32_t* blk_doc, int32_t n_docs, int32_t k, int32_t* topk_ids,
                           float* topk_scores, float* doc_scores, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_route_args("msa_route_topk", n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc, n_docs);
  if (st) return st;
  if (!topk_ids || !workspace) return fail(MSA_ERR_NULL, "msa_route_topk: null pointer");
  if (k < 1 || k > n_docs) return fail(MSA_ERR_SHAPE, "msa_route_topk: k=%d n_docs=%d", k, n_docs);
  if (k > MSA_MAX_TOPK) return fail(MSA_ERR_UNSUPPORTED, "msa_route_topk: k=%d > %d", k, MSA_MAX_TOPK);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_route_topk: n_layers*B > 65535");
  const size_t need = msa_route_topk_workspace_size(n_layers, B, n_docs, k);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "msa_route_topk: workspace %zu < %zu bytes", workspace_bytes, need);
  char* ws = reinterpret_cast<char*>(workspace);
  float* scores = doc_scores ? doc_scores : reinterpret_cast<float*>(ws);
  char* rest = ws + align256((size_t)n_layers * B * n_docs * sizeof(float));
  hipStream_t s = as_stream(stream);
  hipError_t e =
      msa::launch_route_scores(n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc, n_docs, 0, scores, s);
  if (e != hipSuccess) return hip_status(e, "msa_route_topk (scores)");
  e = msa::launch_topk((int64_t)n_layers * B, scores, n_docs, k, topk_ids, topk_scores, rest, s);
  if (e != hipSuccess) return hip_status(e, "msa_route_topk (top-k)");
  return MSA_OK;
}

// ------------------------------------------------- A2 + A3 without allocation
//
// Scratch of msa_route_topk_noalloc: one fixed array per GPU, in the library's code
// object, so the call needs no workspace argument and allocates nothing.  In host code
// the array's name is only a stand-in: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that pointer is what the kernels
// receive.  Every call on a device shares the array; calls that overlap on one device
// (two streams, two threads) race on it.

static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up on first use.
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "msa_route_topk_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "msa_route_topk_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                  "msa_route_topk_noalloc (hipGetSymbolAddress)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

MSA_API size_t msa_route_topk_noalloc_max_scratch(void) { return MSA_NOALLOC_SCRATCH_BYTES; }

MSA_API int msa_route_topk_noalloc(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T,
                                   const uint16_t* krbar_route, const float* krbar_norm, int64_t n_blk,
                                   const int32_t* blk_doc, int32_t n_docs, int32_t k, int32_t* topk_ids,
                                   float* topk_scores, float* doc_scores, void* stream) {
  int st = check_route_args("msa_route_topk_noalloc", n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc,
                            n_docs);
  if (st) return st;
  if (!topk_ids) return fail(MSA_ERR_NULL, "msa_route_topk_noalloc: null pointer");
  if (k < 1 || k > n_docs) return fail(MSA_ERR_SHAPE, "msa_route_topk_noalloc: k=%d n_docs=%d", k, n_docs);
  if (k > MSA_MAX_TOPK) return fail(MSA_ERR_UNSUPPORTED, "msa_route_topk_noalloc: k=%d > %d", k, MSA_MAX_TOPK);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_route_topk_noalloc: n_layers*B > 65535");
  // the same carving as msa_route_topk: scores (unless the caller keeps them), then top-k
  const size_t need = msa_route_topk_workspace_size(n_layers, B, n_docs, k);
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE,
                "msa_route_topk_noalloc: needs %zu bytes of scratch, the fixed maximum is %zu "
                "(use msa_route_topk with a workspace)", need, (size_t)MSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st) return st;
  char* base = reinterpret_cast<char*>(ws);
  float* scores = doc_scores ? doc_scores : reinterpret_cast<float*>(base);
  char* rest = base + align256((size_t)n_layers * B * n_docs * sizeof(float));
  hipStream_t s = as_stream(stream);
  hipError_t e =
      msa::launch_route_scores(n_layers, qr, B, T, krbar_route, krbar_norm, n_blk, blk_doc, n_docs, 0, scores, s);
  if (e != hipSuccess) return hip_status(e, "msa_route_topk_noalloc (scores)");
  e = msa::launch_topk((int64_t)n_layers * B, scores, n_docs, k, topk_ids, topk_scores, rest, s);
  if (e != hipSuccess) return hip_status(e, "msa_route_topk_noalloc (top-k)");
  return MSA_OK;
}

// ------------------------------------------------------------------------ A4

MSA_API int msa_gather_ctx(int32_t n_layers, int32_t B, const int32_t* topk_ids, int32_t k,
                           const int64_t* doc_blk_off, int32_t n_docs, int32_t max_doc_blocks, const uint16_t* kbar,
                           const uint16_t* vbar, int64_t n_blk, int32_t max_ctx, uint16_t* ctx_k, uint16_t* ctx_v,
                           int32_t* ctx_len, void* stream) {
  if (!topk_ids || !doc_blk_off || (n_blk > 0 && (!kbar || !vbar)) || !ctx_k || !ctx_v || !ctx_len)
    return fail(MSA_ERR_NULL, "msa_gather_ctx: null pointer");
  if (!all_aligned16({kbar, vbar, ctx_k, ctx_v}))
    return fail(MSA_ERR_SHAPE, "msa_gather_ctx: bf16 arrays must be 16-byte aligned");
  if (n_layers < 1 || B < 1 || k < 1 || n_docs < 1 || max_doc_blocks < 0 || n_blk < 0 || max_ctx < 1)
    return fail(MSA_ERR_SHAPE, "msa_gather_ctx: n_layers=%d B=%d k=%d n_docs=%d max_doc_blocks=%d max_ctx=%d",
                n_layers, B, k, n_docs, max_doc_blocks, max_ctx);
  if (k > MSA_MAX_TOPK) return fail(MSA_ERR_UNSUPPORTED, "msa_gather_ctx: k=%d > %d", k, MSA_MAX_TOPK);
  if ((int64_t)max_ctx < (int64_t)k * max_doc_blocks)
    return fail(MSA_ERR_SHAPE, "msa_gather_ctx: max_ctx=%d < k*max_doc_blocks=%lld", max_ctx,
                (long long)k * max_doc_blocks);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_gather_ctx: n_layers*B > 65535");
  return hip_status(msa::launch_gather(n_layers, B, topk_ids, k, doc_blk_off, n_docs, kbar, vbar, n_blk, max_ctx,
                                       ctx_k, ctx_v, ctx_len, as_stream(stream)),
                    "msa_gather_ctx");
}

// ------------------------------------------------------------------------ A5

MSA_API size_t msa_sparse_decode_workspace_size(int32_t n_layers, int32_t B, int32_t Hq, int32_t max_ctx,
                                                int32_t max_loc) {
  if (n_layers < 1 || B < 1 || Hq < 8 || max_ctx < 0 || max_loc < 0) return 0;
  const int64_t rps = msa::decode_rows_per_split();
  const int64_t n_splits = ((int64_t)max_ctx + max_loc + rps - 1) / rps;
  const int64_t parts = (int64_t)n_layers * B * MSA_HEADS * n_splits * (Hq / MSA_HEADS);
  const int64_t ml = ((2 * parts + 63) / 64) * 64;
  return (size_t)(ml + parts * MSA_HEAD_DIM) * sizeof(float) + 256;
}

MSA_API int msa_sparse_decode(int32_t n_layers, int32_t B, int32_t Hq, const uint16_t* q, const uint16_t* ctx_k,
                              const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx, const uint16_t* loc_k,
                              const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc, float scale, float* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !ctx_k || !ctx_v || !ctx_len || !out || !workspace) return fail(MSA_ERR_NULL, "msa_sparse_decode: null pointer");
  if (max_loc > 0 && (!loc_k || !loc_v || !loc_len)) return fail(MSA_ERR_NULL, "msa_sparse_decode: null local KV");
  if (!all_aligned16({q, ctx_k, ctx_v, max_loc > 0 ? loc_k : nullptr, max_loc > 0 ? loc_v : nullptr}))
    return fail(MSA_ERR_SHAPE, "msa_sparse_decode: bf16 arrays must be 16-byte aligned");
  if (n_layers < 1 || B < 1 || Hq < 1 || max_ctx < 1 || max_loc < 0 || Hq % MSA_HEADS != 0)
    return fail(MSA_ERR_SHAPE, "msa_sparse_decode: n_layers=%d B=%d Hq=%d max_ctx=%d max_loc=%d", n_layers, B, Hq,
                max_ctx, max_loc);
  const int G = Hq / MSA_HEADS;
  if (!(G == 1 || G == 2 || G == 4 || G == 8))
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_decode: Hq=%d (supported: 8, 16, 32, 64)", Hq);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_decode: n_layers*B > 65535");
  const size_t need = msa_sparse_decode_workspace_size(n_layers, B, Hq, max_ctx, max_loc);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "msa_sparse_decode: workspace %zu < %zu bytes", workspace_bytes, need);
  return hip_status(msa::launch_decode(n_layers, B, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx, loc_k, loc_v, loc_len,
                                       max_loc, scale, out, workspace, as_stream(stream)),
                    "msa_sparse_decode");
}

MSA_API int msa_encode_blocks(int32_t n_layers, int32_t H, const uint16_t* x, int64_t n_tok, const uint16_t* w_k,
                              const uint16_t* w_v, const uint16_t* w_kr, const uint16_t* w_norm, float eps, float theta,
                              const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                              uint16_t* kbar, uint16_t* vbar, uint16_t* krbar_route, float* krbar_norm, void* stream) {
  if (!x || !w_k || !w_v || !w_kr || !w_norm || !doc_tok_off || !doc_blk_off || !kbar || !vbar || !krbar_route)
    return fail(MSA_ERR_NULL, "msa_encode_blocks: null pointer");
  if (!all_aligned16({x, w_k, w_v, w_kr}))
    return fail(MSA_ERR_SHAPE, "msa_encode_blocks: hidden rows and weights must be 16-byte aligned");
  if (n_layers < 1 || H < 128 || H % 128 != 0 || n_tok < 1 || n_docs < 1 || n_blk < 0 || !(eps >= 0.f) ||
      !(theta > 0.f))
    return fail(MSA_ERR_SHAPE, "msa_encode_blocks: n_layers=%d H=%d n_tok=%lld n_docs=%d n_blk=%lld", n_layers, H,
                (long long)n_tok, n_docs, (long long)n_blk);
  if (n_layers > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_encode_blocks: n_layers > 65535");
  return hip_status(msa::launch_encode(n_layers, H, x, n_tok, w_k, w_v, w_kr, w_norm, eps, theta, doc_tok_off,
                                       doc_blk_off, n_docs, n_blk, kbar, vbar, krbar_route, krbar_norm,
                                       as_stream(stream)),
                    "msa_encode_blocks");
}

MSA_API int msa_sparse_prefill(int32_t n_layers, int32_t B, int32_t T, int32_t Hq, const uint16_t* q,
                               const uint16_t* ctx_k, const uint16_t* ctx_v, const int32_t* ctx_len, int32_t max_ctx,
                               const uint16_t* loc_k, const uint16_t* loc_v, const int32_t* loc_len, int32_t max_loc,
                               float scale, float* out, void* stream) {
  if (!q || !ctx_k || !ctx_v || !ctx_len || !loc_k || !loc_v || !loc_len || !out)
    return fail(MSA_ERR_NULL, "msa_sparse_prefill: null pointer");
  if (!all_aligned16({q, ctx_k, ctx_v, loc_k, loc_v, out}))
    return fail(MSA_ERR_SHAPE, "msa_sparse_prefill: q, K/V and out must be 16-byte aligned");
  if (n_layers < 1 || B < 1 || T < 1 || Hq < 1 || max_ctx < 1 || max_loc < T || Hq % MSA_HEADS != 0)
    return fail(MSA_ERR_SHAPE, "msa_sparse_prefill: n_layers=%d B=%d T=%d Hq=%d max_ctx=%d max_loc=%d", n_layers,
                B, T, Hq, max_ctx, max_loc);
  const int G = Hq / MSA_HEADS;
  if (!(G == 1 || G == 2 || G == 4 || G == 8))
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_prefill: Hq=%d (supported: 8, 16, 32, 64)", Hq);
  if ((int64_t)n_layers * B > 65535) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_prefill: n_layers*B > 65535");
  return hip_status(msa::launch_prefill(n_layers, B, T, Hq, q, ctx_k, ctx_v, ctx_len, max_ctx, loc_k, loc_v, loc_len,
                                        max_loc, scale, out, as_stream(stream)),
                    "msa_sparse_prefill");
}
