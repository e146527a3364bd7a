"""CPU-side checks of the C ABI: the library loads and exports every declared
symbol, the host helpers match the oracle and the pages' worked mapping, and
invalid arguments are rejected before anything touches a GPU."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
LIB = os.path.join(ROOT, "routed_kv_memory_amd",
                   "libmsa_san.so" if os.environ.get("MSA_SANITIZED") == "1" else "libmsa.so")


@pytest.fixture(scope="module")
def msa():
    if not os.path.exists(LIB):
        pytest.fail("libmsa.so not built (run __graft_entry__.build())")
    from routed_kv_memory_amd import msa as m
    m.lib()
    return m


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(msa):
    syms = declared_symbols()
    assert len(syms) >= 15
    L = ctypes.CDLL(LIB)
    missing = [s for s in syms if not hasattr(L, s)]
    assert not missing, missing
    assert msa.msa_abi_version() == 2


def test_only_msa_symbols_are_exported():
    out = os.popen("nm -D --defined-only %s" % LIB).read()
    names = [ln.split()[-1] for ln in out.splitlines() if " T " in ln]
    assert names and all(n.startswith("msa_") for n in names), [n for n in names if not n.startswith("msa_")]


def test_group_offsets_golden(msa):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "group_ids.json")))
    for case in g["cases"]:
        assert msa.msa_group_offsets_host(case["doc_ids"]).tolist() == case["doc_tok_off"]


def test_block_offsets_match_oracle(msa, orc):
    rng = np.random.default_rng(0)
    lens = rng.integers(0, 700, 300)
    tok = np.concatenate([[0], np.cumsum(lens)])
    off, n_blk, mx = msa.msa_block_offsets_host(tok)
    off_o, n_o, mx_o = orc.block_offsets(tok)
    assert off.numpy().tolist() == off_o.tolist() and n_blk == n_o and mx == mx_o
    with pytest.raises(msa.MsaError) as e:
        msa.msa_block_offsets_host([0, 5, 3])
    assert e.value.status == msa.MSA_ERR_SHAPE


def test_route_tiles(msa):
    assert [msa.msa_route_tiles(n) for n in (0, 1, 16, 17, 1562500)] == [0, 1, 1, 2, 97657]


def _call(msa, name, *args):
    return getattr(msa.lib(), name)(*args)


def test_invalid_arguments_are_rejected_on_the_host(msa):
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    lib = msa.lib()
    # null pointers
    assert lib.msa_pool_blocks(1, None, fake, fake, 10, fake, fake, 1, 1, fake, fake, fake, fake, None) == 1
    assert lib.msa_route_scores(1, None, 1, 8, fake, None, 16, fake, 1, 0, fake, None) == 1
    assert lib.msa_block_doc_map(None, 4, 16, fake, None) == 1
    # shapes
    assert lib.msa_route_scores(0, fake, 1, 8, fake, None, 16, fake, 1, 0, fake, None) == 2
    assert lib.msa_route_scores(1, fake, 1, 0, fake, fake, 16, fake, 1, 0, fake, None) == 2
    assert lib.msa_route_topk(1, fake, 1, 8, fake, None, 16, fake, 4, 5, fake, None, None, fake, 1 << 20, None) == 2
    assert lib.msa_topk_docs(1, 1, fake, 10, 11, fake, None, fake, 1 << 20, None) == 2       # k > n_docs
    assert lib.msa_topk_docs(1, 1, fake, 1000, 300, fake, None, fake, 1 << 20, None) == 3    # k > MAX_TOPK
    assert lib.msa_gather_ctx(1, 1, fake, 4, fake, 10, 8, fake, fake, 100, 31, fake, fake, fake, None) == 2
    assert lib.msa_sparse_decode(1, 1, 12, fake, fake, fake, fake, 16, fake, fake, fake, 4, ctypes.c_float(0.1),
                                 fake, fake, 1 << 20, None) == 2                              # Hq % 8
    assert lib.msa_sparse_decode(1, 1, 24, fake, fake, fake, fake, 16, fake, fake, fake, 4, ctypes.c_float(0.1),
                                 fake, fake, 1 << 20, None) == 3                              # group of 3
    assert lib.msa_sparse_decode(1, 1, 32, fake, fake, fake, fake, 16, None, None, None, 4, ctypes.c_float(0.1),
                                 fake, fake, 1 << 20, None) == 1                              # local KV missing
    # prefill: null, fewer local rows than tokens, unsupported head group
    assert lib.msa_sparse_prefill(1, 1, 4, 32, None, fake, fake, fake, 8, fake, fake, fake, 4, ctypes.c_float(0.1),
                                  fake, None) == 1
    assert lib.msa_sparse_prefill(1, 1, 4, 32, fake, fake, fake, fake, 8, fake, fake, fake, 3, ctypes.c_float(0.1),
                                  fake, None) == 2
    assert lib.msa_sparse_prefill(1, 1, 4, 24, fake, fake, fake, fake, 8, fake, fake, fake, 4, ctypes.c_float(0.1),
                                  fake, None) == 3
    # encode: null, hidden size not a multiple of 128, zero layers, theta 0
    F = ctypes.c_float
    assert lib.msa_encode_blocks(1, 128, None, 10, fake, fake, fake, fake, F(1e-6), F(1e6), fake, fake, 1, 1, fake,
                                 fake, fake, None, None) == 1
    assert lib.msa_encode_blocks(1, 192, fake, 10, fake, fake, fake, fake, F(1e-6), F(1e6), fake, fake, 1, 1, fake,
                                 fake, fake, None, None) == 2
    assert lib.msa_encode_blocks(0, 128, fake, 10, fake, fake, fake, fake, F(1e-6), F(1e6), fake, fake, 1, 1, fake,
                                 fake, fake, None, None) == 2
    assert lib.msa_encode_blocks(1, 128, fake, 10, fake, fake, fake, fake, F(1e-6), F(0.0), fake, fake, 1, 1, fake,
                                 fake, fake, None, None) == 2
    # bf16 arrays not 16-byte aligned (each otherwise valid call)
    odd = P(0x1002)
    assert lib.msa_pool_blocks(1, fake, odd, fake, 10, fake, fake, 1, 1, fake, fake, fake, fake, None) == 2
    assert b"aligned" in lib.msa_last_error()
    assert lib.msa_pack_route_keys(1, odd, 16, fake, None, None) == 2
    assert lib.msa_route_scores(1, odd, 1, 8, fake, None, 16, fake, 1, 0, fake, None) == 2
    assert lib.msa_route_scores(1, fake, 1, 64, fake, P(0x1004), 16, fake, 1, 0, fake, None) == 2   # key norms
    assert lib.msa_route_topk(1, fake, 1, 8, odd, None, 16, fake, 4, 2, fake, None, None, fake, 1 << 20, None) == 2
    assert lib.msa_gather_ctx(1, 1, fake, 4, fake, 10, 8, fake, fake, 100, 32, odd, fake, fake, None) == 2
    assert lib.msa_sparse_decode(1, 1, 32, fake, fake, fake, fake, 16, fake, odd, fake, 4, ctypes.c_float(0.1),
                                 fake, fake, 1 << 20, None) == 2
    assert lib.msa_sparse_prefill(1, 1, 4, 32, fake, fake, fake, fake, 8, fake, fake, fake, 4, ctypes.c_float(0.1),
                                  P(0x1008), None) == 2
    F = ctypes.c_float
    assert lib.msa_encode_blocks(1, 128, fake, 10, fake, odd, fake, fake, F(1e-6), F(1e6), fake, fake, 1, 1, fake,
                                 fake, fake, None, None) == 2
    # workspace too small
    need = lib.msa_route_topk_workspace_size(2, 1, 100000, 16)
    assert lib.msa_route_topk(2, fake, 1, 8, fake, None, 1000, fake, 100000, 16, fake, None, None, fake, need - 1,
                              None) == 4
    need = lib.msa_sparse_decode_workspace_size(2, 3, 32, 100, 50)
    assert lib.msa_sparse_decode(2, 3, 32, fake, fake, fake, fake, 100, fake, fake, fake, 50, ctypes.c_float(0.1),
                                 fake, fake, need - 1, None) == 4
    assert b"workspace" in lib.msa_last_error()
    assert lib.msa_status_string(4) == b"workspace too small"


def test_noalloc_route_topk_rejects_oversized_scratch_on_the_host(msa):
    """The no-allocation entry point refuses work whose scratch exceeds its fixed array, and
    checks its arguments, before any device call."""
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    lib = msa.lib()
    cap = lib.msa_route_topk_noalloc_max_scratch()
    assert cap == 64 << 20
    # 18 layers x 8 queries x 100,000 documents fit; 20M documents of one query do not
    assert lib.msa_route_topk_workspace_size(18, 8, 100000, 16) <= cap
    assert lib.msa_route_topk_workspace_size(1, 1, 20000000, 16) > cap
    assert lib.msa_route_topk_noalloc(1, fake, 1, 64, fake, None, 1000, fake, 20000000, 16, fake, None, None,
                                      None) == 4
    assert b"64" in lib.msa_last_error() or b"maximum" in lib.msa_last_error()
    assert lib.msa_route_topk_noalloc(1, None, 1, 64, fake, None, 1000, fake, 100, 16, fake, None, None, None) == 1
    assert lib.msa_route_topk_noalloc(1, fake, 1, 64, fake, None, 1000, fake, 10, 16, fake, None, None, None) == 2
    assert lib.msa_route_topk_noalloc(1, fake, 1, 64, fake, None, 1000, fake, 1000, 300, fake, None, None, None) == 3


def test_empty_arrays_may_be_null(msa):
    """A memory with no tokens and no blocks (every document empty) passes NULL for its empty
    arrays; pooling, packing and the block map then have nothing to do and return before any
    device call.  A NULL array that does have elements is still refused."""
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced
    lib = msa.lib()
    # n_tok = 0, n_blk = 0: token rows and every per-block output NULL
    assert lib.msa_pool_blocks(2, None, None, None, 0, fake, fake, 5, 0, None, None, None, None, None) == 0
    assert lib.msa_pack_route_keys(2, None, 0, None, None, None) == 0
    assert lib.msa_block_doc_map(fake, 5, 0, None, None) == 0
    # the same NULLs with elements present
    assert lib.msa_pool_blocks(2, None, fake, fake, 10, fake, fake, 5, 1, fake, fake, fake, None, None) == 1
    assert lib.msa_pool_blocks(2, fake, fake, fake, 10, fake, fake, 5, 1, None, fake, fake, None, None) == 1
    assert lib.msa_pack_route_keys(2, None, 3, fake, None, None) == 1
    assert lib.msa_block_doc_map(fake, 5, 3, None, None) == 1
    assert lib.msa_route_scores(1, fake, 1, 8, None, None, 16, fake, 1, 0, fake, None) == 1
    assert lib.msa_gather_ctx(1, 1, fake, 4, fake, 10, 8, None, fake, 100, 32, fake, fake, fake, None) == 1

