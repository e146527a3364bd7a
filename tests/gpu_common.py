"""Helpers shared by the GPU parity tests (test infrastructure)."""
import math

import numpy as np
import torch

import oracle as O
from routed_kv_memory_amd import msa

SCALE = 1.0 / math.sqrt(128.0)
SCORE_TOL = 1e-4          # document scores, absolute
DECODE_TOL = 2e-3         # decode output, relative to the row's max |value|


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_dev_bf16(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def untile_keys(krt: torch.Tensor, n_blk: int) -> np.ndarray:
    """Route-key layout [L][tile][h][c][b][e] -> row-major [L][n_blk][8][128] (uint16)."""
    a = u16(krt)
    L = a.shape[0]
    tiles = a.size // (L * 16 * 1024)
    a = a.reshape(L, tiles, 8, 16, 16, 8).transpose(0, 1, 4, 2, 3, 5).reshape(L, tiles * 16, 8, 128)
    return a[:, :n_blk]


def untile_norms(krn: torch.Tensor, n_blk: int) -> np.ndarray:
    a = krn.detach().cpu().numpy()
    L = a.shape[0]
    tiles = a.size // (L * 128)
    return a.reshape(L, tiles, 8, 16).transpose(0, 1, 3, 2).reshape(L, tiles * 16, 8)[:, :n_blk]


def alloc_route_keys(L, n_blk, dev="cuda"):
    tiles = msa.msa_route_tiles(n_blk)
    krt = torch.empty((L, max(tiles, 1) * 16, 8, 128), dtype=torch.bfloat16, device=dev)
    krn = torch.empty((L, max(tiles, 1) * 16, 8), dtype=torch.float32, device=dev)
    return krt, krn


def pack_rows(rows: torch.Tensor, n_blk: int):
    krt, krn = alloc_route_keys(rows.shape[0], n_blk, rows.device)
    msa.msa_pack_route_keys(rows, n_blk, krt, krn)
    return krt, krn


def doc_map(blk_off_d: torch.Tensor, n_blk: int) -> torch.Tensor:
    tiles = msa.msa_route_tiles(n_blk)
    m = torch.empty(max(tiles, 1) * 16, dtype=torch.int32, device=blk_off_d.device)
    msa.msa_block_doc_map(blk_off_d, n_blk, m)
    return m


def route(qr, krt, krn, n_blk, blk_off_d, k, dev="cuda", blk_doc=None, norms=None):
    """Scores + top-k through msa_route_topk.  norms: pass the key norms to the scan (True), let
    it recompute them (False), or None: pass them when the scan has more than one query chunk."""
    L, B = qr.shape[0], qr.shape[1]
    n_docs = blk_off_d.numel() - 1
    if blk_doc is None:
        blk_doc = doc_map(blk_off_d, n_blk)
    ws = torch.empty(msa.msa_route_topk_workspace_size(L, B, n_docs, k), dtype=torch.uint8, device=dev)
    ids = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    sc = torch.empty((L, B, k), dtype=torch.float32, device=dev)
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=dev)
    if norms is None:
        norms = B * ((qr.shape[2] + 63) // 64) > 1
    msa.msa_route_topk(qr, krt, n_blk, blk_doc, n_docs, k, ids, sc, ws, doc_scores=dsc,
                       krbar_norm=krn if norms else None)
    return ids, sc, dsc


def exact_topk_of(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of given float32 scores by (score desc, id asc) -- for checking the selection kernel."""
    order = np.lexsort((np.arange(scores.size), -scores.astype(np.float64)))
    return order[:k]


def assert_topk(ids_gpu: np.ndarray, sc_gpu: np.ndarray, dsc_gpu: np.ndarray, S_oracle: np.ndarray, k: int):
    """ids_gpu: the GPU's top-k for one (layer, query).  Selection must be exact on the GPU's own
    scores; against the oracle the id sets must match except across near-ties (< SCORE_TOL)."""
    assert ids_gpu.tolist() == exact_topk_of(dsc_gpu, k).tolist()
    assert np.array_equal(sc_gpu, dsc_gpu[ids_gpu])
    ids_o, _ = O.topk(S_oracle, k)
    a, b = set(ids_gpu.tolist()), set(ids_o.tolist())
    if a != b:
        kth = S_oracle[ids_o[k - 1]]
        for d in a ^ b:
            assert abs(S_oracle[d] - kth) < SCORE_TOL, (d, S_oracle[d], kth)


def assert_decode(out_gpu: np.ndarray, out_oracle: np.ndarray):
    err = np.max(np.abs(out_gpu - out_oracle), axis=-1)
    ref = np.max(np.abs(out_oracle), axis=-1)
    bad = err > DECODE_TOL * np.maximum(ref, 1e-30)
    assert not bad.any(), (err / np.maximum(ref, 1e-30)).max()


def decode_all(q, ck, cv, cl, lk, lv, ll, dev="cuda"):
    L, B, Hq = q.shape[0], q.shape[1], q.shape[2]
    max_ctx = ck.shape[2]
    max_loc = 0 if lk is None else lk.shape[2]
    out = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, max_loc), dtype=torch.uint8,
                     device=dev)
    msa.msa_sparse_decode(q, ck, cv, cl, lk, lv, ll, SCALE, out, ws)
    return out


def gather_all(ids, blk_off_d, max_db, kbar, vbar, max_ctx=None, dev="cuda"):
    L, B, k = ids.shape
    max_ctx = max_ctx or k * max_db
    ck = torch.zeros((L, B, max_ctx, 8, 128), dtype=torch.bfloat16, device=dev)
    cv = torch.zeros_like(ck)
    cl = torch.empty((L, B), dtype=torch.int32, device=dev)
    msa.msa_gather_ctx(ids, blk_off_d, max_db, kbar, vbar, ck, cv, cl)
    return ck, cv, cl
