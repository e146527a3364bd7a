"""ctypes binding of the fp64 C oracle (msa_oracle.c).

TEST INFRASTRUCTURE ONLY.  All arrays are numpy; bf16 travels as uint16.
Row layout: [row][8 heads][128 dims].  Definitions and citations are in
msa_oracle.h; this module only marshals arguments and loops over
(layer, query) pairs where the C functions work on one pair.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PLAIN = os.path.join(_HERE, "liboracle.so")
# MSA_SANITIZED=1 selects the AddressSanitizer + UndefinedBehaviorSanitizer build (clang, so that one
# ASan runtime serves the whole process; run Python with that runtime preloaded)
_SAN = os.environ.get("MSA_SANITIZED") == "1"
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
_LIB = _LIB_SAN if _SAN else _LIB_PLAIN

H, D, BLOCK = 8, 128, 64
ROW = H * D


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, fp64, no FMA contraction); with sanitize=True a
    second library, liboracle_san.so, built by clang with -fsanitize=address,undefined."""
    lib_path = _LIB_SAN if sanitize else _LIB_PLAIN
    if force or not os.path.exists(lib_path) or os.path.getmtime(lib_path) < os.path.getmtime(_SRC):
        tmp = lib_path + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-ffp-contract=off",
                   "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"]
        else:
            cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC,
                   "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, lib_path)
    return lib_path


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True, sanitize=_SAN)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = f64
        L.orc_bf16_from_double.argtypes = [f64]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_group_ids.argtypes = [P, i64, P]
        L.orc_doc_tok_offsets.argtypes = [P, i64, P]
        L.orc_doc_tok_offsets.restype = i64
        L.orc_block_offsets.argtypes = [P, i32, P, P]
        L.orc_block_offsets.restype = i64
        L.orc_pool.argtypes = [i32, P, i64, P, P, i32, i64, P]
        L.orc_head_norms.argtypes = [P, i64, P]
        L.orc_block_score.argtypes = [P, P]
        L.orc_block_score.restype = f64
        L.orc_doc_scores.argtypes = [i32, P, P, P, i32, P]
        L.orc_doc_scores_mt.argtypes = [i32, P, P, P, i32, P, i32]
        L.orc_pool_mt.argtypes = [i32, P, i64, P, P, i32, i64, P, i32]
        L.orc_topk.argtypes = [P, i32, i32, P, P]
        L.orc_gather.argtypes = [P, i32, P, P, P, P, P]
        L.orc_gather.restype = i64
        L.orc_decode.argtypes = [i32, P, P, P, i64, P, P, i64, f64, P]
        L.orc_prefill.argtypes = [i32, i32, P, P, P, i64, P, P, i64, f64, P]
        L.orc_encode.argtypes = [i32, P, i64, P, P, P, P, f64, f64, P, P, i32, i64, P, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


# ------------------------------------------------------------------ bf16 ---

def bf16_to_f64(a) -> np.ndarray:
    """Exact values of bf16 bit patterns (vectorised through the C routine's rule)."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_from_f64_scalar(x: float) -> int:
    return int(lib().orc_bf16_from_double(float(x)))


def bf16_from_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    f = lib().orc_bf16_from_double
    out = np.fromiter((f(float(v)) for v in x.ravel()), dtype=np.uint16, count=x.size)
    return out.reshape(x.shape)


# --------------------------------------------------------- offset tables ---

def group_ids(doc_ids) -> np.ndarray:
    a = _i64(doc_ids)
    out = np.empty_like(a)
    lib().orc_group_ids(_p(a), a.size, _p(out))
    return out


def doc_tok_offsets(doc_ids) -> np.ndarray:
    a = _i64(doc_ids)
    out = np.empty(a.size + 1, np.int64)
    n = lib().orc_doc_tok_offsets(_p(a), a.size, _p(out))
    return out[: n + 1].copy()


def block_offsets(doc_tok_off):
    t = _i64(doc_tok_off)
    n_docs = t.size - 1
    out = np.empty(n_docs + 1, np.int64)
    mx = ctypes.c_int32(0)
    n_blk = lib().orc_block_offsets(_p(t), n_docs, _p(out), ctypes.byref(mx))
    return out, int(n_blk), int(mx.value)


# -------------------------------------------------------------- pooling ---

def pool(x, doc_tok_off, doc_blk_off) -> np.ndarray:
    """x: [L][N_tok][8][128] uint16 -> [L][N_blk][8][128] uint16."""
    x = _u16(x)
    L, n_tok = x.shape[0], x.shape[1]
    t, b = _i64(doc_tok_off), _i64(doc_blk_off)
    n_docs, n_blk = t.size - 1, int(b[-1])
    out = np.zeros((L, n_blk, H, D), np.uint16)
    lib().orc_pool(L, _p(x), n_tok, _p(t), _p(b), n_docs, n_blk, _p(out))
    return out


def host_threads() -> int:
    """Worker threads for the threaded drivers: the CPUs this process may run on, at most 16
    (the host share of one GPU on the machines this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool_mt(x, doc_tok_off, doc_blk_off, threads: int = None) -> np.ndarray:
    """pool() with the documents split over threads (identical output)."""
    x = _u16(x)
    L, n_tok = x.shape[0], x.shape[1]
    t, b = _i64(doc_tok_off), _i64(doc_blk_off)
    n_docs, n_blk = t.size - 1, int(b[-1])
    out = np.zeros((L, n_blk, H, D), np.uint16)
    lib().orc_pool_mt(L, _p(x), n_tok, _p(t), _p(b), n_docs, n_blk, _p(out), threads or host_threads())
    return out


def head_norms(rows) -> np.ndarray:
    """rows: [..., 8, 128] uint16 -> [..., 8] float64."""
    rows = _u16(rows)
    n = rows.size // ROW
    out = np.empty(n * H, np.float64)
    lib().orc_head_norms(_p(rows), n, _p(out))
    return out.reshape(rows.shape[:-1])


# -------------------------------------------------------------- routing ---

def block_score(q_row, k_row) -> float:
    q, k = _u16(q_row), _u16(k_row)
    assert q.size == ROW and k.size == ROW
    return float(lib().orc_block_score(_p(q), _p(k)))


def doc_scores(qr, krbar, doc_blk_off) -> np.ndarray:
    """qr: [T][8][128]; krbar: [n_blk][8][128] -> S[n_docs] (float64, -inf if empty)."""
    q, k, b = _u16(qr), _u16(krbar), _i64(doc_blk_off)
    T, n_docs = q.shape[0], b.size - 1
    S = np.empty(n_docs, np.float64)
    lib().orc_doc_scores(T, _p(q), _p(k), _p(b), n_docs, _p(S))
    return S


def doc_scores_mt(qr, krbar, doc_blk_off, threads: int = None, chunks: int = 1, progress=None) -> np.ndarray:
    """doc_scores() with the documents split over threads (identical output).  With chunks > 1
    the documents are processed in that many consecutive pieces of about equal block count and
    progress(i, chunks) is called after piece i."""
    q, k, b = _u16(qr), _u16(krbar), _i64(doc_blk_off)
    T, n_docs = q.shape[0], b.size - 1
    assert k.shape[0] >= int(b[-1]), "krbar holds fewer rows than the offsets name"
    S = np.empty(n_docs, np.float64)
    threads = threads or host_threads()
    chunks = max(1, min(chunks, max(n_docs, 1)))
    total = int(b[-1] - b[0])
    starts = [int(np.searchsorted(b[:-1], b[0] + total * i // chunks, side="left")) for i in range(chunks)] + [n_docs]
    for i in range(chunks):
        d0, d1 = starts[i], max(starts[i], starts[i + 1])
        if d1 > d0:
            lib().orc_doc_scores_mt(T, _p(q), _p(k), _p(b[d0:]), d1 - d0, _p(S[d0:]), threads)
        if progress is not None:
            progress(i + 1, chunks)
    return S


def doc_scores_all(qr, krbar, doc_blk_off) -> np.ndarray:
    """qr: [L][B][T][8][128]; krbar: [L][n_blk][8][128] -> S[L][B][n_docs]."""
    L, B = qr.shape[0], qr.shape[1]
    n_docs = len(doc_blk_off) - 1
    S = np.empty((L, B, n_docs), np.float64)
    for l in range(L):
        for b in range(B):
            S[l, b] = doc_scores(qr[l, b], krbar[l], doc_blk_off)
    return S


def topk(S, k: int):
    s = np.ascontiguousarray(S, dtype=np.float64)
    ids = np.empty(k, np.int32)
    sc = np.empty(k, np.float64)
    lib().orc_topk(_p(s), s.size, k, _p(ids), _p(sc))
    return ids, sc


# --------------------------------------------------------------- gather ---

def gather(ids, doc_blk_off, kbar, vbar):
    """One (layer, query): kbar/vbar [n_blk][8][128] -> (ctx_k, ctx_v) [rows][8][128]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    b = _i64(doc_blk_off)
    kb, vb = _u16(kbar), _u16(vbar)
    total = int(sum(b[i + 1] - b[i] for i in ids))
    ck = np.zeros((max(total, 1), H, D), np.uint16)
    cv = np.zeros((max(total, 1), H, D), np.uint16)
    n = lib().orc_gather(_p(ids), ids.size, _p(b), _p(kb), _p(vb), _p(ck), _p(cv))
    assert n == total
    return ck[:total], cv[:total]


# --------------------------------------------------------------- decode ---

def decode(q, ctx_k, ctx_v, loc_k, loc_v, scale: float) -> np.ndarray:
    """One (layer, query): q [Hq][128]; rows [n][8][128] -> out [Hq][128] float64."""
    q = _u16(q)
    Hq = q.shape[0]

    def rows(a):
        a = _u16(a) if a is not None and len(a) else np.zeros((1, H, D), np.uint16)
        return a

    ck, cv = _u16(ctx_k), _u16(ctx_v)
    lk, lv = _u16(loc_k), _u16(loc_v)
    n_ctx, n_loc = ck.shape[0], lk.shape[0]
    ck_, cv_ = (ck, cv) if n_ctx else (rows(None), rows(None))
    lk_, lv_ = (lk, lv) if n_loc else (rows(None), rows(None))
    out = np.empty((Hq, D), np.float64)
    lib().orc_decode(Hq, _p(q), _p(ck_), _p(cv_), n_ctx, _p(lk_), _p(lv_), n_loc, float(scale), _p(out))
    return out


def prefill(q, ctx_k, ctx_v, loc_k, loc_v, scale: float) -> np.ndarray:
    """One (layer, query): q [T][Hq][128]; ctx rows [n_ctx][8][128]; local rows [n_loc][8][128]
    (the query tokens are the last T of them) -> out [T][Hq][128] float64."""
    q = _u16(q)
    T, Hq = q.shape[0], q.shape[1]
    ck, cv, lk, lv = _u16(ctx_k), _u16(ctx_v), _u16(loc_k), _u16(loc_v)
    n_ctx, n_loc = ck.shape[0], lk.shape[0]
    assert n_loc >= T
    one = np.zeros((1, H, D), np.uint16)
    ck_, cv_ = (ck, cv) if n_ctx else (one, one)
    out = np.empty((T, Hq, D), np.float64)
    lib().orc_prefill(T, Hq, _p(q), _p(ck_), _p(cv_), n_ctx, _p(lk), _p(lv), n_loc, float(scale), _p(out))
    return out


def encode(x, w_k, w_v, w_kr, w_norm, eps: float, theta: float, doc_tok_off, doc_blk_off):
    """One layer: x [n_tok][H]; W_* [H][8*128]; w_norm [128] -> pooled (kbar, vbar, krbar) [n_blk][8][128]."""
    x = _u16(x)
    n_tok, Hd = x.shape
    wk, wv, wr, wn = _u16(w_k), _u16(w_v), _u16(w_kr), _u16(w_norm)
    assert wk.shape == (Hd, ROW) and wv.shape == (Hd, ROW) and wr.shape == (Hd, ROW) and wn.size == D
    t, b = _i64(doc_tok_off), _i64(doc_blk_off)
    n_docs, n_blk = t.size - 1, int(b[-1])
    outs = [np.zeros((max(n_blk, 1), H, D), np.uint16) for _ in range(3)]
    lib().orc_encode(Hd, _p(x), n_tok, _p(wk), _p(wv), _p(wr), _p(wn), float(eps), float(theta), _p(t), _p(b),
                     n_docs, n_blk, _p(outs[0]), _p(outs[1]), _p(outs[2]))
    return tuple(o[:n_blk] for o in outs)


__all__ = ["build", "lib", "bf16_to_f64", "bf16_from_f64", "bf16_from_f64_scalar", "group_ids",
           "doc_tok_offsets", "block_offsets", "pool", "pool_mt", "head_norms", "block_score", "doc_scores",
           "doc_scores_mt", "host_threads",
           "doc_scores_all", "topk", "gather", "decode", "prefill", "encode", "H", "D", "BLOCK", "ROW"]
