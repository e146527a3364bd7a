"""Thin Python binding of libmsa (include/msa.h) over ctypes.

Argument marshalling only: every function takes torch tensors that already live
on the GPU, checks dtype/contiguity/device, passes raw pointers and the current
HIP stream to the C entry point of the same name, and raises MsaError on a
non-OK status.  All computation happens in the library's HIP kernels.  bf16
tensors may be torch.bfloat16 or torch.int16/uint16 views of the bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MSA_SANITIZED=1 loads the build whose host code carries AddressSanitizer and UBSan checks
LIB_PATH = os.path.join(_PKG, "libmsa_san.so" if os.environ.get("MSA_SANITIZED") == "1" else "libmsa.so")

MSA_OK, MSA_ERR_NULL, MSA_ERR_SHAPE, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(6)
HEADS, HEAD_DIM, BLOCK_TOKENS, TILE_BLOCKS, MAX_TOPK = 8, 128, 64, 16, 256


class MsaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__("%s failed: status %d (%s): %s" % (fn, status, _status_string(status), message))
        self.status = status


_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "msa_abi_version": ([], ctypes.c_int),
    "msa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "msa_last_error": ([], ctypes.c_char_p),
    "msa_group_offsets_host": ([_P, _I64, _P, _P], ctypes.c_int),
    "msa_block_offsets_host": ([_P, _I32, _P, _P, _P], ctypes.c_int),
    "msa_route_tiles": ([_I64], _I64),
    "msa_pool_blocks": ([_I32, _P, _P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "msa_pack_route_keys": ([_I32, _P, _I64, _P, _P, _P], ctypes.c_int),
    "msa_block_doc_map": ([_P, _I32, _I64, _P, _P], ctypes.c_int),
    "msa_route_scores": ([_I32, _P, _I32, _I32, _P, _P, _I64, _P, _I32, _I32, _P, _P], ctypes.c_int),
    "msa_topk_docs_workspace_size": ([_I32, _I32, _I32, _I32], _SZ),
    "msa_topk_docs": ([_I32, _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "msa_route_topk_workspace_size": ([_I32, _I32, _I32, _I32], _SZ),
    "msa_route_topk": ([_I32, _P, _I32, _I32, _P, _P, _I64, _P, _I32, _I32, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "msa_route_topk_noalloc_max_scratch": ([], _SZ),
    "msa_route_topk_noalloc": ([_I32, _P, _I32, _I32, _P, _P, _I64, _P, _I32, _I32, _P, _P, _P, _P], ctypes.c_int),
    "msa_gather_ctx": ([_I32, _I32, _P, _I32, _P, _I32, _I32, _P, _P, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "msa_sparse_decode_workspace_size": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_decode": ([_I32, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _F32, _P, _P, _SZ, _P],
                          ctypes.c_int),
    "msa_encode_blocks": ([_I32, _I32, _P, _I64, _P, _P, _P, _P, _F32, _F32, _P, _P, _I32, _I64, _P, _P, _P, _P, _P],
                          ctypes.c_int),
    "msa_sparse_prefill": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _F32, _P, _P],
                           ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmsa.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmsa.so is missing at %s: build it with __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().msa_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(fn: str, status: int):
    if status != MSA_OK:
        raise MsaError(fn, status, lib().msa_last_error().decode(errors="replace"))


def _ptr(t, dtypes, name, allow_none=False, allow_pinned=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if not t.is_cuda and not (allow_pinned and t.is_pinned()):
        raise ValueError("%s must be a GPU tensor%s" % (name, " or pinned host memory" if allow_pinned else ""))
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I64T = (torch.int64,)
_I32T = (torch.int32,)
_F32T = (torch.float32,)
_ANY = (torch.uint8, torch.int8, torch.int16, torch.int32, torch.int64, torch.float32, torch.bfloat16)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ host helpers

def msa_abi_version() -> int:
    return lib().msa_abi_version()


def msa_group_offsets_host(doc_ids):
    """CPU int64 per-token doc ids -> CPU int64 doc_tok_off [n_docs + 1]."""
    ids = torch.as_tensor(doc_ids, dtype=torch.int64).contiguous()
    out = torch.empty(ids.numel() + 1, dtype=torch.int64)
    n = ctypes.c_int32(0)
    _check("msa_group_offsets_host",
           lib().msa_group_offsets_host(ctypes.c_void_p(ids.data_ptr()), ids.numel(),
                                        ctypes.c_void_p(out.data_ptr()), ctypes.byref(n)))
    return out[: n.value + 1].clone()


def msa_block_offsets_host(doc_tok_off):
    """CPU int64 doc_tok_off -> (CPU int64 doc_blk_off, n_blk, max_doc_blocks)."""
    tok = torch.as_tensor(doc_tok_off, dtype=torch.int64).contiguous()
    n_docs = tok.numel() - 1
    out = torch.empty(n_docs + 1, dtype=torch.int64)
    n_blk, mx = ctypes.c_int64(0), ctypes.c_int32(0)
    _check("msa_block_offsets_host",
           lib().msa_block_offsets_host(ctypes.c_void_p(tok.data_ptr()), n_docs, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.byref(n_blk), ctypes.byref(mx)))
    return out, int(n_blk.value), int(mx.value)


def msa_route_tiles(n_blk: int) -> int:
    return int(lib().msa_route_tiles(n_blk))


# ----------------------------------------------------------------------- entry points

def msa_pool_blocks(k, v, kr, doc_tok_off, doc_blk_off, n_blk, kbar, vbar, krbar_route, krbar_norm=None,
                    stream=None):
    L, n_tok = k.shape[0], k.shape[1]
    n_docs = doc_tok_off.numel() - 1
    _check("msa_pool_blocks", lib().msa_pool_blocks(
        L, _ptr(k, _BF16, "k"), _ptr(v, _BF16, "v"), _ptr(kr, _BF16, "kr"), n_tok,
        _ptr(doc_tok_off, _I64T, "doc_tok_off"), _ptr(doc_blk_off, _I64T, "doc_blk_off"), n_docs, n_blk,
        _ptr(kbar, _BF16, "kbar"), _ptr(vbar, _BF16, "vbar"), _ptr(krbar_route, _BF16, "krbar_route"),
        _ptr(krbar_norm, _F32T, "krbar_norm", allow_none=True), _stream(stream)))


def msa_pack_route_keys(krbar_rows, n_blk, krbar_route, krbar_norm=None, stream=None):
    L = krbar_rows.shape[0]
    _check("msa_pack_route_keys", lib().msa_pack_route_keys(
        L, _ptr(krbar_rows, _BF16, "krbar_rows"), n_blk, _ptr(krbar_route, _BF16, "krbar_route"),
        _ptr(krbar_norm, _F32T, "krbar_norm", allow_none=True), _stream(stream)))


def msa_block_doc_map(doc_blk_off, n_blk, blk_doc, stream=None):
    n_docs = doc_blk_off.numel() - 1
    _check("msa_block_doc_map", lib().msa_block_doc_map(
        _ptr(doc_blk_off, _I64T, "doc_blk_off"), n_docs, n_blk, _ptr(blk_doc, _I32T, "blk_doc"), _stream(stream)))


def _norms(krbar_norm, n_layers, n_blk):
    """The optional key norms of the scan: None, or at least [n_layers][tiles][8][16] fp32."""
    if krbar_norm is None:
        return None
    need = n_layers * msa_route_tiles(n_blk) * 128
    if krbar_norm.numel() < need:
        raise ValueError("krbar_norm has %d elements, the scan needs %d" % (krbar_norm.numel(), need))
    return _ptr(krbar_norm, _F32T, "krbar_norm")


def msa_route_scores(qr, krbar_route, n_blk, blk_doc, n_docs, doc_scores, accumulate=False, stream=None,
                     krbar_norm=None):
    L, B, T = qr.shape[0], qr.shape[1], qr.shape[2]
    _check("msa_route_scores", lib().msa_route_scores(
        L, _ptr(qr, _BF16, "qr"), B, T, _ptr(krbar_route, _BF16, "krbar_route"),
        _norms(krbar_norm, L, n_blk), n_blk, _ptr(blk_doc, _I32T, "blk_doc"), n_docs,
        1 if accumulate else 0, _ptr(doc_scores, _F32T, "doc_scores"), _stream(stream)))


def msa_topk_docs_workspace_size(n_layers, B, n_docs, k) -> int:
    return int(lib().msa_topk_docs_workspace_size(n_layers, B, n_docs, k))


def msa_topk_docs(doc_scores, k, topk_ids, topk_scores, workspace, stream=None):
    L, B, n_docs = doc_scores.shape
    _check("msa_topk_docs", lib().msa_topk_docs(
        L, B, _ptr(doc_scores, _F32T, "doc_scores"), n_docs, k, _ptr(topk_ids, _I32T, "topk_ids"),
        _ptr(topk_scores, _F32T, "topk_scores", allow_none=True), _ptr(workspace, _ANY, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_route_topk_workspace_size(n_layers, B, n_docs, k) -> int:
    return int(lib().msa_route_topk_workspace_size(n_layers, B, n_docs, k))


def msa_route_topk(qr, krbar_route, n_blk, blk_doc, n_docs, k, topk_ids, topk_scores, workspace, doc_scores=None,
                   stream=None, krbar_norm=None):
    L, B, T = qr.shape[0], qr.shape[1], qr.shape[2]
    _check("msa_route_topk", lib().msa_route_topk(
        L, _ptr(qr, _BF16, "qr"), B, T, _ptr(krbar_route, _BF16, "krbar_route"),
        _norms(krbar_norm, L, n_blk), n_blk, _ptr(blk_doc, _I32T, "blk_doc"), n_docs, k,
        _ptr(topk_ids, _I32T, "topk_ids"), _ptr(topk_scores, _F32T, "topk_scores", allow_none=True),
        _ptr(doc_scores, _F32T, "doc_scores", allow_none=True), _ptr(workspace, _ANY, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_route_topk_noalloc_max_scratch() -> int:
    return int(lib().msa_route_topk_noalloc_max_scratch())


def msa_route_topk_noalloc(qr, krbar_route, n_blk, blk_doc, n_docs, k, topk_ids, topk_scores, doc_scores=None,
                           stream=None, krbar_norm=None):
    """msa_route_topk without a workspace: the library's fixed per-GPU scratch is used."""
    L, B, T = qr.shape[0], qr.shape[1], qr.shape[2]
    _check("msa_route_topk_noalloc", lib().msa_route_topk_noalloc(
        L, _ptr(qr, _BF16, "qr"), B, T, _ptr(krbar_route, _BF16, "krbar_route"),
        _norms(krbar_norm, L, n_blk), n_blk, _ptr(blk_doc, _I32T, "blk_doc"), n_docs, k,
        _ptr(topk_ids, _I32T, "topk_ids"), _ptr(topk_scores, _F32T, "topk_scores", allow_none=True),
        _ptr(doc_scores, _F32T, "doc_scores", allow_none=True), _stream(stream)))


def msa_gather_ctx(topk_ids, doc_blk_off, max_doc_blocks, kbar, vbar, ctx_k, ctx_v, ctx_len, stream=None):
    """kbar/vbar may live in HBM or in pinned host memory (read over the host link)."""
    L, B, k = topk_ids.shape
    n_docs = doc_blk_off.numel() - 1
    n_blk = kbar.shape[1]
    max_ctx = ctx_k.shape[2]
    _check("msa_gather_ctx", lib().msa_gather_ctx(
        L, B, _ptr(topk_ids, _I32T, "topk_ids"), k, _ptr(doc_blk_off, _I64T, "doc_blk_off"), n_docs,
        max_doc_blocks, _ptr(kbar, _BF16, "kbar", allow_pinned=True), _ptr(vbar, _BF16, "vbar", allow_pinned=True),
        n_blk, max_ctx,
        _ptr(ctx_k, _BF16, "ctx_k"), _ptr(ctx_v, _BF16, "ctx_v"), _ptr(ctx_len, _I32T, "ctx_len"),
        _stream(stream)))


def msa_sparse_decode_workspace_size(n_layers, B, Hq, max_ctx, max_loc) -> int:
    return int(lib().msa_sparse_decode_workspace_size(n_layers, B, Hq, max_ctx, max_loc))


def msa_sparse_decode(q, ctx_k, ctx_v, ctx_len, loc_k, loc_v, loc_len, scale, out, workspace, stream=None):
    L, B, Hq = q.shape[0], q.shape[1], q.shape[2]
    max_ctx = ctx_k.shape[2]
    max_loc = 0 if loc_k is None else loc_k.shape[2]
    _check("msa_sparse_decode", lib().msa_sparse_decode(
        L, B, Hq, _ptr(q, _BF16, "q"), _ptr(ctx_k, _BF16, "ctx_k"), _ptr(ctx_v, _BF16, "ctx_v"),
        _ptr(ctx_len, _I32T, "ctx_len"), max_ctx,
        _ptr(loc_k, _BF16, "loc_k", allow_none=True), _ptr(loc_v, _BF16, "loc_v", allow_none=True),
        _ptr(loc_len, _I32T, "loc_len", allow_none=True), max_loc, float(scale),
        _ptr(out, _F32T, "out"), _ptr(workspace, _ANY, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_sparse_prefill(q, ctx_k, ctx_v, ctx_len, loc_k, loc_v, loc_len, scale, out, stream=None):
    """q [L][B][T][Hq][128] bf16; contexts as for msa_sparse_decode; out [L][B][T][Hq][128] fp32."""
    L, B, T, Hq = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    _check("msa_sparse_prefill", lib().msa_sparse_prefill(
        L, B, T, Hq, _ptr(q, _BF16, "q"), _ptr(ctx_k, _BF16, "ctx_k"), _ptr(ctx_v, _BF16, "ctx_v"),
        _ptr(ctx_len, _I32T, "ctx_len"), ctx_k.shape[2], _ptr(loc_k, _BF16, "loc_k"), _ptr(loc_v, _BF16, "loc_v"),
        _ptr(loc_len, _I32T, "loc_len"), loc_k.shape[2], float(scale), _ptr(out, _F32T, "out"), _stream(stream)))


def msa_encode_blocks(x, w_k, w_v, w_kr, w_norm, eps, theta, doc_tok_off, doc_blk_off, n_blk, kbar, vbar,
                      krbar_route, krbar_norm=None, stream=None):
    """x [L][n_tok][H]; W_* [L][1024][H] (output-major); w_norm [L][128]; outputs as msa_pool_blocks."""
    L, n_tok, H = x.shape
    n_docs = doc_tok_off.numel() - 1
    _check("msa_encode_blocks", lib().msa_encode_blocks(
        L, H, _ptr(x, _BF16, "x"), n_tok, _ptr(w_k, _BF16, "w_k"), _ptr(w_v, _BF16, "w_v"),
        _ptr(w_kr, _BF16, "w_kr"), _ptr(w_norm, _BF16, "w_norm"), float(eps), float(theta),
        _ptr(doc_tok_off, _I64T, "doc_tok_off"), _ptr(doc_blk_off, _I64T, "doc_blk_off"), n_docs, n_blk,
        _ptr(kbar, _BF16, "kbar"), _ptr(vbar, _BF16, "vbar"), _ptr(krbar_route, _BF16, "krbar_route"),
        _ptr(krbar_norm, _F32T, "krbar_norm", allow_none=True), _stream(stream)))

