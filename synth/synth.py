"""Seeded synthetic inputs for the MSA hot path (host side + device wrappers).

This module makes inputs only: it holds none of the pooling, routing, top-k,
gather or decode arithmetic.  Both the GPU library's tests/bench and the CPU
oracle take their inputs from here.

Definitions (the device side, synth_dev.hip, implements the same ones):

* ``word(seed, stream, j)``: SplitMix64 (Steele, Lea & Flood 2014) output j of
  the state ``base = mix64(seed ^ (stream << 32))``, i.e.
  ``mix64(base + (j + 1) * 0x9E3779B97F4A7C15)`` modulo 2**64.
* element e of a stream: ``TABLE[(word(seed, stream, e >> 2) >> 16*(e & 3)) & 0xFFFF]``,
  where ``TABLE[i]`` is the bf16 (round-to-nearest-even of the float32) of the
  standard normal quantile at (i + 0.5) / 65536.  Integer hashing plus a shared
  table makes host and device values bit-identical.
* tensor [L][R][8][128]: element (l, r, c) is stream element (l*R + r)*1024 + c.
* needle row: ``bf16(q + float32(0.3) * z)`` in float32 with two separate
  roundings, q the query's Qr row and z the needle stream's element at
  (l*N + r)*1024 + c, N the row count of the tensor the row lives in.
* host-only draws (lengths, needle choice) use ``u = ((word >> 11) + 0.5) / 2**53``
  from the TABLES stream.

Workload recipes (shapes, sizes, length mix, needles) are in ``CONFIGS``.
"""
from __future__ import annotations

import ctypes
import math
import os
import statistics
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_dev.hip")
_LIB = os.path.join(_HERE, "libsynth.so")

H, D, ROW = 8, 128, 1024
M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

# stream ids
S_K, S_V, S_KR = 1, 2, 3            # per-token K, V, routing keys
S_KBAR, S_VBAR, S_KRBAR = 4, 5, 6   # pre-pooled K-bar, V-bar, routing keys
S_QR, S_NEEDLE = 7, 8
S_DEC_Q, S_LOC_K, S_LOC_V = 9, 10, 11
S_TABLES = 12
S_PF_Q, S_PF_CTX_K, S_PF_CTX_V, S_PF_DOCS = 13, 14, 15, 16   # multi-token prefill inputs
S_ENC_X, S_ENC_WK, S_ENC_WV, S_ENC_WKR, S_ENC_WN = 17, 18, 19, 20, 21   # encode front-end inputs
ENC_HIDDEN = 2560          # hidden size of the encode workload (the pages' 4B backbone)

SEED0 = 0x4D534100


# --------------------------------------------------------------------------- hash

def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def stream_base(seed: int, stream: int) -> int:
    return _mix64_int((seed ^ (stream << 32)) & M64)


def words(seed: int, stream: int, j: np.ndarray) -> np.ndarray:
    base = np.uint64(stream_base(seed, stream))
    j = np.asarray(j, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(base + (j + np.uint64(1)) * np.uint64(GAMMA))


_TABLE = None


def table() -> np.ndarray:
    """bf16 bit patterns of N(0,1) quantiles at (i + 0.5)/65536, i < 65536."""
    global _TABLE
    if _TABLE is None:
        nd = statistics.NormalDist()
        f = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        _TABLE = u.astype(np.uint16)
    return _TABLE


def elements(seed: int, stream: int, e: np.ndarray) -> np.ndarray:
    """Stream elements at (int64) indices e -> uint16 bf16 patterns."""
    e = np.asarray(e, dtype=np.int64)
    w = words(seed, stream, (e >> 2).astype(np.uint64))
    sh = ((e & 3) * 16).astype(np.uint64)
    return table()[((w >> sh) & np.uint64(0xFFFF)).astype(np.int64)]


def fill_host(n: int, seed: int, stream: int, e0: int = 0) -> np.ndarray:
    """Elements e0 .. e0+n-1 of a stream (uint16 bf16 patterns)."""
    if n <= 0:
        return np.zeros(0, np.uint16)
    g0, g1 = e0 >> 2, (e0 + n + 3) >> 2
    w = words(seed, stream, np.arange(g0, g1, dtype=np.uint64))
    t = table()
    four = np.empty((g1 - g0, 4), np.uint16)
    for s in range(4):
        four[:, s] = t[((w >> np.uint64(16 * s)) & np.uint64(0xFFFF)).astype(np.int64)]
    flat = four.reshape(-1)
    off = e0 - (g0 << 2)
    return flat[off:off + n].copy()


def rows_host(seed: int, stream: int, layer: int, n_rows_total: int, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of layer `layer` of a [L][n_rows_total][8][128] tensor -> [r1-r0][8][128]."""
    e0 = (layer * n_rows_total + r0) * ROW
    return fill_host((r1 - r0) * ROW, seed, stream, e0).reshape(r1 - r0, H, D)


def uniforms(seed: int, j: np.ndarray) -> np.ndarray:
    w = words(seed, S_TABLES, j)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def needle_rows_host(seed: int, layer: int, n_rows_total: int, rows: np.ndarray,
                     q_rows: np.ndarray) -> np.ndarray:
    """Needle values for global rows `rows` (int64) given their query rows [n][8][128] (uint16)."""
    rows = np.asarray(rows, np.int64)
    e = ((layer * n_rows_total + rows)[:, None] * ROW + np.arange(ROW)[None, :]).reshape(-1)
    z = bf16_to_f32(elements(seed, S_NEEDLE, e)).reshape(len(rows), ROW)
    q = bf16_to_f32(q_rows).reshape(len(rows), ROW)
    prod = (np.float32(0.3) * z).astype(np.float32)
    v = (q + prod).astype(np.float32)
    return f32_to_bf16(v).reshape(len(rows), H, D)


# ------------------------------------------------------------------------- recipes

@dataclass
class Config:
    name: str
    index: int
    n_layers: int
    n_docs: int
    per_token: bool             # True: per-token K/V/Kr pooled by the library
    B: int
    T: int                      # query tokens (first round)
    needles: int                # planted needle docs per query (0 for none)
    needle_queries: int         # how many queries carry needles
    k: int
    Hq: int
    L_loc: int
    lengths: str                # "uniform64_512" | "lognormal"
    n_blk: int = 0              # pre-pooled configs: exact block total
    T_rounds: tuple = ()        # interleaved re-routing: query length per round
    memory_of: str = ""         # reuse another config's memory
    description: str = ""
    seed: int = field(init=False)

    def __post_init__(self):
        self.seed = SEED0 + self.index


CONFIGS = {
    "tiny": Config("tiny", 0, 1, 64, True, 1, 8, 2, 1, 4, 32, 16, "uniform64_512",
                   description="1 routed layer, 64 docs U[64,512] tokens, T=8, 2 needles, top-4, local 16"),
    "1m": Config("1m", 1, 18, 1000, True, 1, 64, 16, 1, 16, 32, 512, "lognormal",
                 description="18 layers, 1,000 lognormal docs (~1M tokens), T=64, 16 needles, top-16, local 512"),
    "10m": Config("10m", 2, 18, 10000, False, 32, 64, 16, 32, 16, 32, 1024, "lognormal", n_blk=156250,
                  description="18 layers x 156,250 pre-pooled blocks, 10,000 docs, 32 queries x 64 tokens, "
                              "16 needles each, top-16, local 1,024"),
    "100m": Config("100m", 3, 18, 100000, False, 1, 64, 16, 1, 16, 32, 4096, "lognormal", n_blk=1562500,
                   description="18 layers x 1,562,500 pre-pooled blocks (100M tokens), 100,000 docs, "
                               "1 query x 64 tokens, 16 needles, top-16, local 4,096"),
    "interleaved": Config("interleaved", 4, 18, 100000, False, 8, 64, 16, 1, 16, 32, 1088, "lognormal",
                          n_blk=1562500, T_rounds=(64, 576, 1088), memory_of="100m",
                          description="100M-token memory; 8 queries re-routed over 3 rounds, "
                                      "T = 64 -> 576 -> 1,088; top-16 per round; local 1,088"),
}


def doc_lengths(cfg: Config) -> np.ndarray:
    """Token lengths of the documents (int64)."""
    u = uniforms(cfg.seed if not cfg.memory_of else CONFIGS[cfg.memory_of].seed,
                 np.arange(cfg.n_docs, dtype=np.uint64))
    if cfg.lengths == "uniform64_512":
        return (64 + np.floor(u * 449.0)).astype(np.int64)
    nd = statistics.NormalDist()
    mu, sigma = math.log(1000.0) - 0.5, 1.0
    z = np.array([nd.inv_cdf(x) for x in u])
    return np.clip(np.rint(np.exp(mu + sigma * z)), 64, 8192).astype(np.int64)


def doc_tok_offsets(cfg: Config) -> np.ndarray:
    lens = doc_lengths(cfg)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def prepooled_block_counts(cfg: Config) -> np.ndarray:
    """Pre-pooled memories: per-doc block counts proportional to len/64, rescaled by
    largest remainder to sum to exactly cfg.n_blk, at least 1 per doc."""
    raw = doc_lengths(cfg).astype(np.float64) / 64.0
    quota = raw * (cfg.n_blk / raw.sum())
    n = np.maximum(1, np.floor(quota)).astype(np.int64)
    rem = int(cfg.n_blk - n.sum())
    if rem > 0:
        frac = quota - np.floor(quota)
        order = np.lexsort((np.arange(len(n)), -frac))
        n[order[:rem]] += 1
    while rem < 0:
        order = np.lexsort((np.arange(len(n)), -n))
        take = min(-rem, int((n[order] > 1).sum()))
        n[order[:take]] -= 1
        rem += take
    assert n.sum() == cfg.n_blk and n.min() >= 1
    return n


def prepooled_doc_blk_offsets(cfg: Config) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(prepooled_block_counts(cfg))]).astype(np.int64)


def memory_config(cfg: Config) -> Config:
    return CONFIGS[cfg.memory_of] if cfg.memory_of else cfg


def needle_docs(cfg: Config) -> np.ndarray:
    """[needle_queries][needles] distinct document ids (a seeded permutation).  A config
    that reuses another's memory gets that memory's needles (carried by its query 0)."""
    mem = memory_config(cfg)
    if mem is not cfg:
        return needle_docs(mem)
    if cfg.needles == 0:
        return np.zeros((0, 0), np.int64)
    pri = words(cfg.seed, S_TABLES, np.arange(cfg.n_docs, dtype=np.uint64) + np.uint64(1 << 40))
    order = np.lexsort((np.arange(cfg.n_docs), pri))
    need = cfg.needle_queries * cfg.needles
    return order[:need].reshape(cfg.needle_queries, cfg.needles).astype(np.int64)


def needle_token(i: int, T: int) -> int:
    """Query token a needle doc is aligned to."""
    return i % T


def needle_row_table(mem: Config, offsets: np.ndarray):
    """Needle rows of a memory config: (global rows [n] int64, Qr rows [n] int64 into that
    config's [B][T] query grid).  `offsets` are token offsets (per-token memories) or
    block offsets (pre-pooled memories)."""
    assert not mem.memory_of
    nd = needle_docs(mem)
    rows, qrows = [], []
    for b in range(nd.shape[0]):
        for i in range(nd.shape[1]):
            d = int(nd[b, i])
            r = np.arange(offsets[d], offsets[d + 1], dtype=np.int64)
            rows.append(r)
            qrows.append(np.full(r.size, b * mem.T + needle_token(i, mem.T), np.int64))
    if not rows:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(rows), np.concatenate(qrows)


def qr_host(cfg: Config, layer: int) -> np.ndarray:
    """Qr of one layer: [B][T][8][128] (T = longest round for interleaved)."""
    T = max(cfg.T_rounds) if cfg.T_rounds else cfg.T
    base = layer * cfg.B * T
    q = fill_host(cfg.B * T * ROW, cfg.seed, S_QR, base * ROW).reshape(cfg.B, T, H, D)
    if cfg.memory_of:
        mem = CONFIGS[cfg.memory_of]
        q[0, :mem.T] = qr_host(mem, layer)[0]
    return q


# ------------------------------------------------------------------------- device

_dlib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-o", tmp, _SRC], stderr=subprocess.DEVNULL)
        os.replace(tmp, _LIB)
    return _LIB


def dlib():
    global _dlib
    if _dlib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError("synth/libsynth.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        P, i32, i64, u32, u64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                 ctypes.c_uint64)
        L.synth_fill.argtypes = [P, i64, u64, u32, i64, P, P]
        L.synth_fill.restype = ctypes.c_int
        L.synth_plant.argtypes = [P, i64, i64, i32, P, P, i32, P, u64, u32, P, P]
        L.synth_plant.restype = ctypes.c_int
        _dlib = L
    return _dlib


class DeviceGen:
    """Device-side generation into torch tensors (bf16 storage)."""

    def __init__(self, device="cuda"):
        import torch
        self.torch = torch
        self.table = torch.from_numpy(table().view(np.int16).copy()).to(device)

    def _stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def fill(self, t, seed: int, stream: int, e0: int = 0):
        rc = dlib().synth_fill(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, stream, e0,
                               ctypes.c_void_p(self.table.data_ptr()), self._stream())
        if rc:
            raise RuntimeError("synth_fill failed: hip error %d" % rc)
        return t

    def plant(self, rows_t, row_base: int, n_rows_total: int, layer: int, row_idx, q_row, qr_layer_t,
              seed: int):
        """Overwrite needle rows of rows_t (a [*][8][128] slice whose first row is global row
        row_base) with bf16(q + 0.3 z); row_idx/q_row are int64 device tensors."""
        n = int(row_idx.numel())
        rc = dlib().synth_plant(ctypes.c_void_p(rows_t.data_ptr()), row_base, n_rows_total, layer,
                                ctypes.c_void_p(row_idx.data_ptr()), ctypes.c_void_p(q_row.data_ptr()), n,
                                ctypes.c_void_p(qr_layer_t.data_ptr()), seed, S_NEEDLE,
                                ctypes.c_void_p(self.table.data_ptr()), self._stream())
        if rc:
            raise RuntimeError("synth_plant failed: hip error %d" % rc)
        return rows_t


# --------------------------------------------------------------------------- encode inputs

def enc_weight_scale(hidden: int) -> float:
    """Power of two nearest 1/sqrt(hidden): scaling N(0,1) bf16 weights by it is exact and
    gives projections of about unit variance."""
    return float(2.0 ** -round(math.log2(math.sqrt(hidden))))


def enc_weights_host(seed: int, stream: int, layer: int, hidden: int) -> np.ndarray:
    """Layer `layer` of a [L][1024][hidden] projection weight, stored as a linear layer
    stores it (output-major), as uint16 bf16 [1024][hidden]."""
    raw = fill_host(ROW * hidden, seed, stream, layer * ROW * hidden).reshape(ROW, hidden)
    return f32_to_bf16(bf16_to_f32(raw) * np.float32(enc_weight_scale(hidden)))


def enc_norm_weight_host(seed: int, n_layers: int) -> np.ndarray:
    """[L][128] key-norm weights near 1 (uint16 bf16)."""
    z = bf16_to_f32(fill_host(n_layers * D, seed, S_ENC_WN))
    return f32_to_bf16(np.float32(1.0) + np.float32(0.25) * z).reshape(n_layers, D)


def enc_x_host(seed: int, layer: int, n_tok: int, hidden: int, t0: int, t1: int) -> np.ndarray:
    """Hidden rows [t0, t1) of layer `layer` of x [L][n_tok][hidden] (uint16 bf16)."""
    return fill_host((t1 - t0) * hidden, seed, S_ENC_X, (layer * n_tok + t0) * hidden).reshape(t1 - t0, hidden)

