/*
 * msa.h -- C ABI of libmsa, the Memory Sparse Attention (MSA) hot path on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages about MSA, cited by title and section):
 *  [P1] yunpan.plus, "MSA端到端可训练记忆模型完整开源，支持亿级Token上下文", 整体设计 -> 架构
 *       and 推理流水线: document K, V and routing key Kr are compressed by block mean
 *       pooling; a routing projection Qr is compared with every pooled routing key by
 *       cosine similarity, averaged over heads and maxed over tokens; the Top-k
 *       documents' compressed K/V are concatenated with the query's local K/V for
 *       autoregressive decoding.
 *  [P2] xuqi2024.github.io, "【MSA】突破100M Token 上下文：记忆稀疏注意力架构深度解析",
 *       3.3.2 (64-token blocks, Top-16), 5.2 (concatenation, varlen attention),
 *       5.3 (map_tensor_to_group_ids).
 *  [P3] bi-chao.com, "把一亿 token 装进模型的“记忆”里：EverMind 开源 MSA 能干什么、不能干什么…",
 *       3.3 (routing keys on the GPU, content K/V in host memory).
 *  [P5] xiaohongrsx.github.io, "MSA paper reading", 方法拆解 (8 KV heads x 128 dims,
 *       18 routed layers, fixed 64-token blocks per document, Top-16 by cosine) and
 *       推理全流程 (context = [Top-16 compressed KV ; local KV]; memory KV is fixed
 *       while the local KV grows token by token).
 *
 * Conventions for every entry point:
 *  - Shapes are fixed at H = 8 KV heads, D = 128, 64-token blocks.  bf16 values
 *    travel as uint16_t bit patterns.  Layouts are layer-major and row-major; a
 *    "row" is [8 heads][128 dims] = 1024 bf16.
 *  - Pointers without a _host suffix are DEVICE pointers owned by the caller (the
 *    one exception, content K/V in pinned host memory, is noted at msa_gather_ctx); the
 *    library never allocates, frees or keeps them.  Workspaces are caller-owned
 *    device memory of at least the size the matching *_workspace_size returns.
 *  - bf16 arrays (and the scan's optional key norms, the prefill's output) are moved in
 *    16-byte vectors: their pointers must be 16-byte aligned, else MSA_ERR_SHAPE.
 *  - An array with no elements may be NULL: the token rows of a memory with no tokens
 *    (n_tok == 0), and every per-block array (pooled K/V, route keys, norms, block map)
 *    of a memory with no blocks (n_blk == 0, e.g. every document empty).  Such a memory
 *    scores -inf for every document.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    validate on the host, enqueue kernels on `stream` and return; results are
 *    valid once the stream has been synchronised.  No call synchronises.
 *  - Return value: MSA_OK, or an MSA_ERR_* code; host-checkable errors are
 *    reported before anything is enqueued.  msa_last_error() gives a message for
 *    the last failing call on the calling thread.  The library never aborts or
 *    prints.  Device-side inconsistencies (offsets out of range, invalid ids) are
 *    clamped, never read or written out of bounds.
 *  - Calls on different streams that share an output or workspace race.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 2
#define MSA_HEADS 8          /* KV heads per routed layer                        [P5 方法拆解] */
#define MSA_HEAD_DIM 128     /* head dimension                                   [P5 方法拆解] */
#define MSA_BLOCK_TOKENS 64  /* pooling_kernel_size: tokens per compressed block [P2 3.3.2] */
#define MSA_TILE_BLOCKS 16   /* blocks per tile of the route-key layout (below) */
#define MSA_MAX_TOPK 256     /* largest k accepted by the top-k entry points */

enum {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,        /* a required pointer is NULL */
    MSA_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or inconsistent */
    MSA_ERR_UNSUPPORTED = 3, /* a valid request outside what this build implements */
    MSA_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_size figure */
    MSA_ERR_HIP = 5          /* the HIP runtime reported an error while enqueueing */
};

int msa_abi_version(void);
/* Static, never-NULL description of a status code. */
const char* msa_status_string(int status);
/* Message of the last non-OK return on the calling thread ("" if none). */
const char* msa_last_error(void);

/* ------------------------------------------------------------------ host helpers */

/* [P2 5.3] Document offsets from per-token document ids.  A new document starts
 * wherever consecutive ids differ (the ids need not be sorted or distinct).
 * doc_ids_host[n_tok]; doc_tok_off_host must hold n_tok + 1 entries; on return
 * doc_tok_off_host[0..*n_docs_host] are the first token of each document followed
 * by n_tok.  Host memory only. */
int msa_group_offsets_host(const int64_t* doc_ids_host, int64_t n_tok,
                           int64_t* doc_tok_off_host, int32_t* n_docs_host);

/* [P1 架构; P5 方法拆解] Block offsets of documents split into 64-token blocks,
 * each document on its own grid (blocks never span documents; a final partial
 * block still counts): doc_blk_off[d+1] - doc_blk_off[d] = ceil(len_d / 64).
 * doc_tok_off_host[n_docs + 1] must be non-decreasing from 0.  Writes
 * doc_blk_off_host[n_docs + 1], the total block count and the largest per-doc
 * count.  Host memory only. */
int msa_block_offsets_host(const int64_t* doc_tok_off_host, int32_t n_docs,
                           int64_t* doc_blk_off_host, int64_t* n_blk_host,
                           int32_t* max_doc_blocks_host);

/* -------------------------------------------------------------- route-key layout
 *
 * Pooled routing keys are stored for the routing scan, not row-major.  Blocks are
 * grouped in tiles of 16 (the last tile padded with zero rows); within a tile the
 * 16 blocks' 8-dim chunks are interleaved:
 *
 *   krbar_route[l][tile][h][c][b][e]  = Kr-bar of block (tile*16 + b), head h,
 *                                       dims c*8 + e          (c < 16, b < 16, e < 8)
 *   krbar_norm [l][tile][h][b]        = || Kr-bar[tile*16 + b][h] ||_2 (fp32; 0 for padding)
 *
 * so each 1 KiB of a tile is one matrix-core operand fragment for 16 blocks.
 * Sizes per layer: msa_route_tiles(n_blk) * 16384 bf16 and * 128 floats.  The norms
 * are an optional output of the pooling/packing calls and an optional input of the
 * routing scan (which otherwise recomputes them from the keys it streams). */
int64_t msa_route_tiles(int64_t n_blk);

/* ------------------------------------------------------------- A1: block pooling
 *
 * [P1 架构, 推理流水线 stage 1; P2 3.3.2; P5 方法拆解] For every layer l, document d
 * (tokens [doc_tok_off[d], doc_tok_off[d+1])) and block j of d, the block covers
 * tokens [s_d + 64 j, min(s_d + 64 j + 64, e_d)) and its value is the mean over
 * those real tokens (a final partial block is averaged over its own tokens),
 * accumulated in fp64 (exact for sums of up to 64 bf16 values whose magnitudes span
 * less than 2^39), divided in fp64 and rounded once to bf16 (nearest-even).  Applied
 * to K, V and Kr.
 *
 *   k, v, kr       [n_layers][n_tok][8][128] bf16, per-token inputs
 *   doc_tok_off    [n_docs + 1] int64, device
 *   doc_blk_off    [n_docs + 1] int64, device (as msa_block_offsets_host computes)
 *   kbar, vbar     [n_layers][n_blk][8][128] bf16, row-major outputs
 *   krbar_route    route-key layout (above), output; krbar_norm its norms, output (may be NULL)
 *
 * Norms are of the rounded bf16 Kr-bar.  Errors: NULL pointers, n_layers/n_docs < 1,
 * n_tok < 0, n_blk < 0. */
int msa_pool_blocks(int32_t n_layers, const uint16_t* k, const uint16_t* v, const uint16_t* kr,
                    int64_t n_tok, const int64_t* doc_tok_off, const int64_t* doc_blk_off,
                    int32_t n_docs, int64_t n_blk,
                    uint16_t* kbar, uint16_t* vbar, uint16_t* krbar_route, float* krbar_norm,
                    void* stream);

/* Routing keys that already exist row-major ([n_layers][n_blk][8][128] bf16, e.g. a
 * memory bank built elsewhere) -> route-key layout + norms (krbar_norm may be NULL),
 * as msa_pool_blocks writes them.  Errors: NULL pointers, n_layers < 1, n_blk < 0. */
int msa_pack_route_keys(int32_t n_layers, const uint16_t* krbar_rows, int64_t n_blk,
                        uint16_t* krbar_route, float* krbar_norm, void* stream);

/* Block -> document map of a memory: blk_doc[n] = the document whose block range
 * [doc_blk_off[d], doc_blk_off[d+1]) holds block n, -1 for the padding blocks of
 * the last route tile (or for blocks no document covers).  Built once per memory
 * bank next to the route keys; it keys the per-document max of the routing scan.
 *   doc_blk_off  [n_docs + 1] int64, device;  blk_doc [msa_route_tiles(n_blk) * 16] int32, output
 * Errors: NULL pointers, n_docs < 1, n_blk < 0. */
int msa_block_doc_map(const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk, int32_t* blk_doc,
                      void* stream);

/* --------------------------------------------------------------- A2: routing scan
 *
 * [P1 架构; P2 3.3.3, 5.2; P5 方法拆解] For each layer l, query b, query token t and
 * block n:  s(t, n) = (1/8) sum_h <Qr[t,h], Kr-bar[n,h]> / (max(|Qr[t,h]|, 1e-8) *
 * max(|Kr-bar[n,h]|, 1e-8)); the document score is the max of s over t < T and the
 * document's blocks:
 *
 *   doc_scores[l][b][d] = max_{t < T, n in d} s(t, n)      (-inf for a 0-block doc)
 *
 *   qr           [n_layers][B][T][8][128] bf16
 *   krbar_route  route-key layout of n_blk blocks per layer
 *   krbar_norm   the keys' norms as msa_pool_blocks / msa_pack_route_keys wrote them, or
 *                NULL.  When given, the matrix-core scan (T >= 16) reads them (32 more bytes
 *                per block and layer) instead of recomputing them from the keys: worth it
 *                when B * ceil(T / 64) > 1 makes the scan bound by the matrix cores, not
 *                for one query chunk, which is bound by HBM.  Both are norms of the same
 *                bf16 keys; results with and without may differ in the last fp32 bits,
 *                so calls whose scores are max-merged (accumulate) should agree on it.
 *   blk_doc      block -> document map (msa_block_doc_map) of the same memory
 *   doc_scores   [n_layers][B][n_docs] fp32, output (accumulate = 0) or in/out
 *                (accumulate = 1: the result is max(previous value, new scores),
 *                i.e. the scores of the query rows seen so far plus these T rows;
 *                this is how a query grown by appended rows is re-routed exactly)
 *
 * Queries with T >= 16 use bf16 matrix cores (fp32 accumulate); shorter ones use
 * vector dot products.  Errors: NULL pointers, n_layers/B/T/n_docs < 1, n_blk < 0. */
int msa_route_scores(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T,
                     const uint16_t* krbar_route, const float* krbar_norm, int64_t n_blk,
                     const int32_t* blk_doc, int32_t n_docs, int32_t accumulate,
                     float* doc_scores, void* stream);

/* ---------------------------------------------------------------- A3: top-k docs
 *
 * [P1 架构; P2 3.3.2 (doc_top_k = 16), 5.2; P5 方法拆解] For each (layer, query): the
 * k documents with the largest score, ordered by (score descending, id ascending).
 *
 *   doc_scores   [n_layers][B][n_docs] fp32 (NaN is not supported)
 *   topk_ids     [n_layers][B][k] int32, output
 *   topk_scores  [n_layers][B][k] fp32, output (may be NULL)
 *
 * Errors: NULL pointers, k < 1, k > n_docs (MSA_ERR_SHAPE), k > MSA_MAX_TOPK
 * (MSA_ERR_UNSUPPORTED), small workspace. */
size_t msa_topk_docs_workspace_size(int32_t n_layers, int32_t B, int32_t n_docs, int32_t k);
int msa_topk_docs(int32_t n_layers, int32_t B, const float* doc_scores, int32_t n_docs, int32_t k,
                  int32_t* topk_ids, float* topk_scores,
                  void* workspace, size_t workspace_bytes, void* stream);

/* A2 then A3 with the document scores kept in the workspace (doc_scores may be
 * NULL; if given it receives a copy of them). */
size_t msa_route_topk_workspace_size(int32_t n_layers, int32_t B, int32_t n_docs, int32_t k);
int msa_route_topk(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T,
                   const uint16_t* krbar_route, const float* krbar_norm, int64_t n_blk,
                   const int32_t* blk_doc, int32_t n_docs, int32_t k,
                   int32_t* topk_ids, float* topk_scores, float* doc_scores,
                   void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): msa_route_topk with no workspace
 * argument.  Its scratch (the scores when doc_scores is NULL, and the top-k candidate
 * buffers) is a fixed array of MSA_NOALLOC_SCRATCH_BYTES in the library's device code
 * object, one per GPU, held until the process ends; the call itself allocates nothing.
 * Arguments, layouts and results are those of msa_route_topk.  The caller still owns
 * the inputs and outputs.
 * Limit: msa_route_topk_workspace_size(n_layers, B, n_docs, k) must not exceed
 * MSA_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. 18 layers x 8 queries x 100,000 documents),
 * else MSA_ERR_WORKSPACE and nothing is launched.  The array is shared by every call on
 * the same GPU and keeps the last call's contents: calls that overlap on one GPU (on
 * different streams or threads) race and must be serialised by the caller. */
#define MSA_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t msa_route_topk_noalloc_max_scratch(void);
int msa_route_topk_noalloc(int32_t n_layers, const uint16_t* qr, int32_t B, int32_t T,
                           const uint16_t* krbar_route, const float* krbar_norm, int64_t n_blk,
                           const int32_t* blk_doc, int32_t n_docs, int32_t k,
                           int32_t* topk_ids, float* topk_scores, float* doc_scores, void* stream);

/* ------------------------------------------------------------ A4: context gather
 *
 * [P1 架构 (selected compressed K/V concatenated with the local K/V); P2 5.2;
 * P5 推理全流程] For each (layer, query): all blocks of the selected documents,
 * documents in top-k order, blocks ascending, copied bit-exactly into a contiguous
 * memory context.
 *
 *   topk_ids     [n_layers][B][k] int32 (ids outside [0, n_docs) contribute no rows)
 *   doc_blk_off  [n_docs + 1] int64, device
 *   kbar, vbar   [n_layers][n_blk][8][128] bf16
 *   ctx_k, ctx_v [n_layers][B][max_ctx][8][128] bf16, output (rows >= ctx_len untouched)
 *   ctx_len      [n_layers][B] int32, output
 *
 * max_doc_blocks is the caller's bound on blocks per document (from
 * msa_block_offsets_host); max_ctx < k * max_doc_blocks is MSA_ERR_SHAPE.  Rows that
 * would pass max_ctx (only if the bound was wrong) are dropped.
 *
 * Host tier [P1 推理流水线; P3 3.3; P5 KV 缓存压缩 + Memory Parallel: the compressed
 * content K/V may stay in host DRAM and only the selected documents' blocks cross to
 * the GPU]: kbar and vbar may point to pinned host memory that the device can address
 * (hipHostMalloc); the kernel then reads the selected rows over the host link while
 * ctx_k/ctx_v stay in device memory. */
int msa_gather_ctx(int32_t n_layers, int32_t B, const int32_t* topk_ids, int32_t k,
                   const int64_t* doc_blk_off, int32_t n_docs, int32_t max_doc_blocks,
                   const uint16_t* kbar, const uint16_t* vbar, int64_t n_blk,
                   int32_t max_ctx, uint16_t* ctx_k, uint16_t* ctx_v, int32_t* ctx_len,
                   void* stream);

/* -------------------------------------------------------------- A5: sparse decode
 *
 * [P1 架构; P2 5.2 (attention over the concatenated K/V); P5 推理全流程] One decode
 * token of grouped-query attention per (layer, query): query head hq reads KV head
 * hq / (Hq / 8); its output is sum_j softmax_j(scale * <q_hq, k_j>) v_j over the rows
 * [memory context rows 0..ctx_len) ; [local rows 0..loc_len), with no mask.  Split
 * over rows, online softmax in fp32, then merged.
 *
 *   q            [n_layers][B][Hq][128] bf16, Hq a multiple of 8, Hq <= 64
 *   ctx_k, ctx_v [n_layers][B][max_ctx][8][128] bf16;  ctx_len [n_layers][B] int32
 *   loc_k, loc_v [n_layers][B][max_loc][8][128] bf16;  loc_len [n_layers][B] int32
 *   out          [n_layers][B][Hq][128] fp32 (zero where a query has no rows)
 *
 * Lengths are clamped to [0, max_ctx] / [0, max_loc].  loc_k/loc_v/loc_len may be
 * NULL when max_loc == 0.  Errors: NULL pointers, sizes < 1, Hq % 8 != 0 (SHAPE),
 * Hq > 64 (UNSUPPORTED), small workspace. */
size_t msa_sparse_decode_workspace_size(int32_t n_layers, int32_t B, int32_t Hq, int32_t max_ctx,
                                        int32_t max_loc);
int msa_sparse_decode(int32_t n_layers, int32_t B, int32_t Hq, const uint16_t* q,
                      const uint16_t* ctx_k, const uint16_t* ctx_v, const int32_t* ctx_len,
                      int32_t max_ctx,
                      const uint16_t* loc_k, const uint16_t* loc_v, const int32_t* loc_len,
                      int32_t max_loc, float scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ offline encode front-end
 *
 * [P2 5.1 (router_k_proj: bias-free linear map to 8 x 128), 5.2 Step 1 (k_proj then
 * k_norm, v_proj, rotary positions), 3.3.1 (document-wise positions restarting at 0);
 * P1 整体设计 -> 架构]  For every memory token t at position p (its offset in its
 * document) with hidden row x_t:  k = W_k x_t, scaled per head by 1/sqrt(mean(k^2) +
 * eps) and by w_norm, then rotated (pairs (e, e + 64) of each head by the angle
 * p * theta^(-e/64));  v = W_v x_t;  kr = W_kr x_t.  The three are mean-pooled over
 * the document's 64-token blocks as msa_pool_blocks does (fp32 accumulation, one
 * rounding to bf16) without ever being stored per token.  All pointers are device
 * memory owned by the caller; only rows [0, n_tok) of x are read; the launch is
 * asynchronous on `stream`.
 *
 *   x            [n_layers][n_tok][H] bf16, H a multiple of 128
 *   w_k, w_v, w_kr [n_layers][8 * 128][H] bf16, output-major as a linear layer stores its
 *                weight (row o maps the hidden vector to output o = head * 128 + dim)
 *   w_norm       [n_layers][128] bf16
 *   doc_tok_off, doc_blk_off, n_docs, n_blk: as for msa_pool_blocks
 *   kbar, vbar   [n_layers][n_blk][8][128] bf16 outputs
 *   krbar_route  [n_layers][tiles * 16][8][128] bf16 output (route-key tile layout)
 *   krbar_norm   [n_layers][tiles][8][16] fp32 output or NULL
 *
 * Errors: NULL pointers, sizes < 1, H % 128 != 0 (SHAPE); n_layers > 65535
 * (UNSUPPORTED). */
int msa_encode_blocks(int32_t n_layers, int32_t H, const uint16_t* x, int64_t n_tok,
                      const uint16_t* w_k, const uint16_t* w_v, const uint16_t* w_kr,
                      const uint16_t* w_norm, float eps, float theta,
                      const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
                      int64_t n_blk, uint16_t* kbar, uint16_t* vbar, uint16_t* krbar_route,
                      float* krbar_norm, void* stream);

/* ------------------------------------------------------------ multi-token prefill
 *
 * [P2 5.2 (varlen attention over the query states and the concatenation of local and
 * selected K/V); P1 推理流水线 (Stage 2 prefills the assembled sparse context)]  T query
 * tokens of grouped-query attention per (layer, query).  The query tokens are the last
 * T of the local rows: token t sees every memory-context row and the local rows
 * 0 .. loc_len - T + t (causal, aligned to the end of the local part; with T = 1 this is
 * msa_sparse_decode).  Query head hq reads KV head hq / (Hq / 8); softmax scale as
 * given; online softmax in fp32; the probabilities enter the P.V product as a bf16
 * high part plus a bf16 residual (~16 significant bits).
 *
 *   q            [n_layers][B][T][Hq][128] bf16, Hq in {8, 16, 32, 64}
 *   ctx_k, ctx_v [n_layers][B][max_ctx][8][128] bf16;  ctx_len [n_layers][B] int32
 *   loc_k, loc_v [n_layers][B][max_loc][8][128] bf16;  loc_len [n_layers][B] int32
 *   out          [n_layers][B][T][Hq][128] fp32 (zero for a token that sees no row)
 *
 * Lengths are clamped to [0, max_ctx] / [0, max_loc].  No workspace.  Errors: NULL
 * pointers, sizes < 1, max_loc < T, Hq % 8 != 0 (SHAPE), Hq > 64 or n_layers * B >
 * 65535 (UNSUPPORTED). */
int msa_sparse_prefill(int32_t n_layers, int32_t B, int32_t T, int32_t Hq, const uint16_t* q,
                       const uint16_t* ctx_k, const uint16_t* ctx_v, const int32_t* ctx_len,
                       int32_t max_ctx,
                       const uint16_t* loc_k, const uint16_t* loc_v, const int32_t* loc_len,
                       int32_t max_loc, float scale, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
