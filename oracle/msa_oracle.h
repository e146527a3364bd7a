/*
 * msa_oracle.h -- plain CPU reference ("oracle") of the Memory Sparse Attention
 * hot path, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may link or call this code.  It shares no code,
 * header, table or helper with the GPU library; neither side includes the other.
 *
 * Every function is a direct, unblocked, single-threaded transcription of the
 * definition it cites.  The two *_mt functions are drivers with no arithmetic of
 * their own: they run the single-threaded function on contiguous document ranges
 * in parallel threads, so their outputs are those of one single-threaded call.  Floating point is fp64 over the exact values of the
 * bf16 inputs; the only roundings are the ones the definition itself contains
 * (the pooled means are stored as bf16, round-to-nearest-even).
 *
 * Sources (web pages about MSA, cited by title and section):
 *  [P1] yunpan.plus, "MSA端到端可训练记忆模型完整开源，支持亿级Token上下文",
 *       section 整体设计 -> 架构 / 推理流水线.
 *  [P2] xuqi2024.github.io, "【MSA】突破100M Token 上下文：记忆稀疏注意力架构深度解析",
 *       sections 3.3.2 (分块均值池化), 3.3.3, 5.2, 5.3.
 *  [P5] xiaohongrsx.github.io, "MSA paper reading" notes, sections 方法拆解
 *       (路由投影器 + Top-k 稀疏注意力; KV 缓存压缩 + Memory Parallel; 推理全流程).
 *
 * Fixed shapes: 8 KV heads x head_dim 128 per routed layer [P5 方法拆解], blocks
 * of 64 tokens [P2 3.3.2 table; P5 方法拆解].  bf16 values travel as uint16_t.
 * Row layout everywhere: [row][head 8][dim 128].
 *
 * Parity status per function (see also the test files):
 *   orc_bf16_from_double / orc_bf16_to_double   pinned (RNE cases, float32 library conversion)
 *   orc_group_ids, orc_doc_tok_offsets          pinned (hand-worked example of the 5.3 mapping)
 *   orc_block_offsets                           pinned (closed-form counts, hand-worked 65/64 case)
 *   orc_pool                                    pinned (constant block, 1-token tail, {a,-a}, hand case)
 *   orc_head_norms                              pinned (library norm on exact inputs)
 *   orc_block_score / orc_doc_scores            pinned (scale invariance, +-1, orthogonal, library cosine, superset)
 *   orc_doc_scores_mt, orc_pool_mt              pinned (bit-identical to the single-threaded calls)
 *   orc_topk                                    pinned (brute-force sort, ties, permutation)
 *   orc_gather                                  pinned (library concatenation)
 *   orc_decode                                  pinned (single key, equal keys, q=0, library softmax, permutation)
 *   orc_prefill                                 pinned (library masked attention, T = 1 is decode, causality,
 *                                               single visible row)
 *   orc_encode                                  pinned (identity projection = orc_pool, library matmul, unit
 *                                               RMS, RoPE angle and pair norm per position, document order)
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_H 8       /* KV heads per routed layer                 [P5 方法拆解] */
#define ORC_D 128     /* head dim                                  [P5 方法拆解] */
#define ORC_ROW (ORC_H * ORC_D)
#define ORC_BLOCK 64  /* pooling_kernel_size                       [P2 3.3.2] */

/* Exact value of a bf16 bit pattern. */
double orc_bf16_to_double(uint16_t b);
/* Nearest bf16 to x, ties to even (no intermediate float rounding). */
uint16_t orc_bf16_from_double(double x);

/* [P2 5.3, the document-id to group-id mapping] Per-token document ids, whose
 * tokens are consecutive per document, -> 1-based group ids: each maximal run of
 * equal ids is one group, numbered in order of appearance.  Writes n values. */
void orc_group_ids(const int64_t* doc_ids, int64_t n, int64_t* group_ids);

/* Token offsets of the groups found by orc_group_ids: doc_tok_off[g] is the
 * first token of group g (0-based), doc_tok_off[n_groups] = n.  Returns
 * n_groups; doc_tok_off must hold n+1 entries. */
int64_t orc_doc_tok_offsets(const int64_t* doc_ids, int64_t n, int64_t* doc_tok_off);

/* Blocks per document: ceil(len/64) (a final partial block is still a block).
 * doc_blk_off[0] = 0, doc_blk_off[d+1] = doc_blk_off[d] + ceil(len_d / 64).
 * Returns the total block count; *max_doc_blocks gets the largest per-doc count. */
int64_t orc_block_offsets(const int64_t* doc_tok_off, int32_t n_docs,
                          int64_t* doc_blk_off, int32_t* max_doc_blocks);

/* [P1 架构; P2 3.3.2; P5 方法拆解] Block mean pooling of one per-token tensor.
 * x: [n_layers][n_tok][8][128] bf16.  For layer l, document d and block j the
 * block covers tokens [s_d + 64 j, min(s_d + 64 j + 64, e_d)); its value is the
 * fp64 mean over those (real) tokens, rounded to bf16 (RNE).
 * xbar: [n_layers][n_blk][8][128] bf16. */
void orc_pool(int32_t n_layers, const uint16_t* x, int64_t n_tok,
              const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
              int64_t n_blk, uint16_t* xbar);

/* L2 norm of each (row, head) 128-vector: norms[r*8 + h]. */
void orc_head_norms(const uint16_t* rows, int64_t n_rows, double* norms);

/* [P1 架构; P5 方法拆解] Routing score of one query token against one block:
 * the mean over the 8 heads of cos(q_h, k_h), where
 * cos(a, b) = <a,b> / (max(|a|, 1e-8) * max(|b|, 1e-8)). */
double orc_block_score(const uint16_t* q_row, const uint16_t* k_row);

/* Document scores of one query: S[d] = max over query tokens t < T and blocks
 * of d of orc_block_score.  A document with no blocks scores -inf.
 * qr: [T][8][128]; krbar: [n_blk][8][128]; S: [n_docs]. */
void orc_doc_scores(int32_t T, const uint16_t* qr, const uint16_t* krbar,
                    const int64_t* doc_blk_off, int32_t n_docs, double* S);

/* orc_doc_scores over n_threads threads (each runs orc_doc_scores on a contiguous
 * range of documents of about equal block count); S is identical to one
 * orc_doc_scores call.  A thread that cannot be started runs in the caller. */
void orc_doc_scores_mt(int32_t T, const uint16_t* qr, const uint16_t* krbar,
                       const int64_t* doc_blk_off, int32_t n_docs, double* S, int32_t n_threads);

/* orc_pool over n_threads threads (contiguous document ranges of about equal token
 * count); xbar is identical to one orc_pool call. */
void orc_pool_mt(int32_t n_layers, const uint16_t* x, int64_t n_tok,
                 const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
                 int64_t n_blk, uint16_t* xbar, int32_t n_threads);

/* [P1 架构; P2 3.3.2 doc_top_k; P5 方法拆解] Top-k documents: the k largest S,
 * ordered by (S descending, id ascending).  ids[k], scores[k]. */
void orc_topk(const double* S, int32_t n_docs, int32_t k, int32_t* ids, double* scores);

/* [P1 架构; P2 5.2; P5 推理全流程] Memory context of one query: all blocks of
 * the selected documents, documents in the order given, blocks ascending.
 * kbar/vbar: [n_blk][8][128]; ctx_k/ctx_v: [>= total][8][128].
 * Returns the number of rows written. */
int64_t orc_gather(const int32_t* ids, int32_t k, const int64_t* doc_blk_off,
                   const uint16_t* kbar, const uint16_t* vbar,
                   uint16_t* ctx_k, uint16_t* ctx_v);

/* [P1 架构; P5 推理全流程] One decode token of GQA attention over the rows
 * [memory context ; local KV]: for query head hq with KV head g = hq / (Hq/8),
 * out[hq] = sum_j softmax_j(scale * <q_hq, k_j,g>) v_j,g, two-pass softmax in fp64.
 * q: [Hq][128]; ctx_*: [n_ctx][8][128]; loc_*: [n_loc][8][128]; out: [Hq][128].
 * With no rows at all the output is zero. */
void orc_decode(int32_t Hq, const uint16_t* q,
                const uint16_t* ctx_k, const uint16_t* ctx_v, int64_t n_ctx,
                const uint16_t* loc_k, const uint16_t* loc_v, int64_t n_loc,
                double scale, double* out);

/* [P2 5.2 (the layer's attention runs varlen flash attention over the query states
 * and the concatenation of local and selected K/V); P1 推理流水线 (Stage 2 prefills
 * the assembled sparse context)] Multi-token sparse prefill: T query tokens, the
 * last T of the n_loc local rows, each attend to every memory-context row and,
 * causally, to local rows 0 .. n_loc - T + t (the pages name no mask; this is the
 * causal reading aligned to the end of the local part, so T = 1 is orc_decode).
 * Token t is computed exactly as orc_decode over [ctx ; local rows visible to t].
 * q: [T][Hq][128]; ctx_*: [n_ctx][8][128]; loc_*: [n_loc][8][128], n_loc >= T;
 * out: [T][Hq][128]. */
void orc_prefill(int32_t T, int32_t Hq, const uint16_t* q,
                 const uint16_t* ctx_k, const uint16_t* ctx_v, int64_t n_ctx,
                 const uint16_t* loc_k, const uint16_t* loc_v, int64_t n_loc,
                 double scale, double* out);

/* [P2 5.2 Step 1 (k_proj, k_norm, v_proj); P2 5.1 (router_k_proj, a bias-free
 * linear map to 8 x 128); P2 3.3.1 and P1 整体设计 -> 架构 (parallel, document-wise
 * RoPE: positions restart at 0 in every document); then the block pooling of
 * orc_pool]  The offline encode of one layer's memory documents.  For token t at
 * position p (its offset inside its document), with hidden row x_t of length H:
 *   k = x_t W_k, normalised per head by its root mean square (+ eps) and scaled by
 *   w_norm, then rotated: for e < 64, angle = p * theta^(-e/64),
 *   k'[e] = k[e] cos - k[e+64] sin,  k'[e+64] = k[e+64] cos + k[e] sin  (per head);
 *   v = x_t W_v;  kr = x_t W_kr  (no norm, no rotation).
 * Each is then mean-pooled over the document's 64-token blocks as in orc_pool and
 * rounded once to bf16.  fp64 throughout.
 * x: [n_tok][H]; W_*: [H][8 * 128] (input-major); w_norm: [128];
 * kbar, vbar, krbar: [n_blk][8][128]. */
void orc_encode(int32_t H, const uint16_t* x, int64_t n_tok,
                const uint16_t* w_k, const uint16_t* w_v, const uint16_t* w_kr, const uint16_t* w_norm,
                double eps, double theta,
                const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                uint16_t* kbar, uint16_t* vbar, uint16_t* krbar);

#ifdef __cplusplus
}
#endif
#endif
