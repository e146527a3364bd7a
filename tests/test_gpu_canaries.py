"""Canary guards around every output and workspace buffer of every entry point.

Each output (and each workspace, passed at exactly the size its size query returns) is a view into
a larger device buffer whose 64 KiB before and after it hold a sentinel byte pattern.  After the
call the sentinels must be intact: no kernel writes outside the extent its header documents.  The
shapes are small and ragged (empty documents, partial tiles, partial query chunks, all three scan
kernels) so that every edge path runs; the values themselves are checked by the parity tests."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
GUARD = 65536
SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routed_kv_memory_amd import msa
    msa.lib()
    yield
    torch.cuda.synchronize()


from routed_kv_memory_amd import msa  # noqa: E402
from synth import synth as S  # noqa: E402

from gpu_common import SCALE, to_dev_bf16  # noqa: E402


class Guarded:
    """A device tensor of `shape` and `dtype` with sentinel bytes on both sides."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, name):
        torch.cuda.synchronize()
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.n:]
        bad_h = int((head != SENTINEL).sum().item())
        bad_t = int((tail != SENTINEL).sum().item())
        assert bad_h == 0 and bad_t == 0, "%s: %d bytes before and %d bytes after the buffer changed" % (
            name, bad_h, bad_t)


def guarded_ws(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8)


def rand_bf16(rng, shape):
    return S.f32_to_bf16(rng.standard_normal(shape).astype(np.float32))


def memory(rng, L, lens_tok):
    """Per-token K/V/Kr of documents with the given token counts (zeros allowed)."""
    tok = np.zeros(len(lens_tok) + 1, np.int64)
    tok[1:] = np.cumsum(lens_tok)
    blk_h, n_blk, max_db = msa.msa_block_offsets_host(torch.from_numpy(tok))
    n_tok = int(tok[-1])
    x = [to_dev_bf16(rand_bf16(rng, (L, n_tok, 8, 128))) for _ in range(3)]
    return torch.from_numpy(tok), blk_h, n_blk, max_db, x


def test_canaries_pool_pack_map_route_topk_gather_decode():
    print("case: canaries around pool, pack, block map, scan (3 kernels), top-k, gather, decode", flush=True)
    rng = np.random.default_rng(31)
    L = 2
    lens = rng.integers(1, 400, 37)
    lens[[0, 9, 36]] = 0                                   # empty documents, first and last included
    tok, blk, n_blk, max_db, (k, v, kr) = memory(rng, L, lens)
    tok_d, blk_d = tok.to(DEV), blk.to(DEV)
    n_docs = len(lens)
    tiles = msa.msa_route_tiles(n_blk)
    print("  %d blocks in %d tiles (last tile %d blocks)" % (n_blk, tiles, n_blk - 16 * (tiles - 1)), flush=True)

    kbar = Guarded((L, n_blk, 8, 128), torch.bfloat16)
    vbar = Guarded((L, n_blk, 8, 128), torch.bfloat16)
    krt = Guarded((L, tiles * 16, 8, 128), torch.bfloat16)
    krn = Guarded((L, tiles * 16, 8), torch.float32)
    msa.msa_pool_blocks(k, v, kr, tok_d, blk_d, n_blk, kbar.t, vbar.t, krt.t, krn.t)
    for g, name in ((kbar, "pool kbar"), (vbar, "pool vbar"), (krt, "pool krbar_route"), (krn, "pool krbar_norm")):
        g.check(name)

    krt2 = Guarded((L, tiles * 16, 8, 128), torch.bfloat16)
    krn2 = Guarded((L, tiles * 16, 8), torch.float32)
    msa.msa_pack_route_keys(kbar.t, n_blk, krt2.t, krn2.t)
    krt2.check("pack krbar_route")
    krn2.check("pack krbar_norm")

    bmap = Guarded((tiles * 16,), torch.int32)
    msa.msa_block_doc_map(blk_d, n_blk, bmap.t)
    bmap.check("block_doc_map")

    # the three scan kernels: vector ALU (T < 16), one query chunk, several chunks (odd count)
    for (B, T, norms) in ((2, 9, False), (1, 64, False), (1, 64, True), (3, 70, True), (3, 70, False)):
        qr = to_dev_bf16(rand_bf16(rng, (L, B, T, 8, 128)))
        dsc = Guarded((L, B, n_docs), torch.float32)
        msa.msa_route_scores(qr, krt.t, n_blk, bmap.t, n_docs, dsc.t, krbar_norm=krn.t if norms else None)
        dsc.check("route_scores B=%d T=%d norms=%d" % (B, T, norms))
        msa.msa_route_scores(qr, krt.t, n_blk, bmap.t, n_docs, dsc.t, accumulate=True,
                             krbar_norm=krn.t if norms else None)
        dsc.check("route_scores accumulate B=%d T=%d" % (B, T))

        kk = 5
        ids = Guarded((L, B, kk), torch.int32)
        sc = Guarded((L, B, kk), torch.float32)
        ws = guarded_ws(msa.msa_topk_docs_workspace_size(L, B, n_docs, kk))
        msa.msa_topk_docs(dsc.t, kk, ids.t, sc.t, ws.t)
        for g, name in ((ids, "topk ids"), (sc, "topk scores"), (ws, "topk workspace")):
            g.check(name + " B=%d T=%d" % (B, T))

        ids2 = Guarded((L, B, kk), torch.int32)
        sc2 = Guarded((L, B, kk), torch.float32)
        dsc2 = Guarded((L, B, n_docs), torch.float32)
        ws2 = guarded_ws(msa.msa_route_topk_workspace_size(L, B, n_docs, kk))
        msa.msa_route_topk(qr, krt.t, n_blk, bmap.t, n_docs, kk, ids2.t, sc2.t, ws2.t, doc_scores=dsc2.t,
                           krbar_norm=krn.t if norms else None)
        for g, name in ((ids2, "route_topk ids"), (sc2, "route_topk scores"), (dsc2, "route_topk doc_scores"),
                        (ws2, "route_topk workspace")):
            g.check(name + " B=%d T=%d" % (B, T))

        ids3 = Guarded((L, B, kk), torch.int32)
        sc3 = Guarded((L, B, kk), torch.float32)
        dsc3 = Guarded((L, B, n_docs), torch.float32)
        msa.msa_route_topk_noalloc(qr, krt.t, n_blk, bmap.t, n_docs, kk, ids3.t, sc3.t, doc_scores=dsc3.t,
                                   krbar_norm=krn.t if norms else None)
        for g, name in ((ids3, "noalloc ids"), (sc3, "noalloc scores"), (dsc3, "noalloc doc_scores")):
            g.check(name + " B=%d T=%d" % (B, T))

    # gather of the last scan's selection, then decode over it and a ragged local KV
    B, kk = ids2.t.shape[1], ids2.t.shape[2]
    max_ctx = kk * max_db
    ck = Guarded((L, B, max_ctx, 8, 128), torch.bfloat16)
    cv = Guarded((L, B, max_ctx, 8, 128), torch.bfloat16)
    cl = Guarded((L, B), torch.int32)
    msa.msa_gather_ctx(ids2.t, blk_d, max_db, kbar.t, vbar.t, ck.t, cv.t, cl.t)
    for g, name in ((ck, "gather ctx_k"), (cv, "gather ctx_v"), (cl, "gather ctx_len")):
        g.check(name)

    for Hq in (8, 32):
        max_loc = 300
        q = to_dev_bf16(rand_bf16(rng, (L, B, Hq, 128)))
        lk = to_dev_bf16(rand_bf16(rng, (L, B, max_loc, 8, 128)))
        lv = to_dev_bf16(rand_bf16(rng, (L, B, max_loc, 8, 128)))
        ll = torch.tensor(rng.integers(0, max_loc + 1, (L, B)), dtype=torch.int32, device=DEV)
        out = Guarded((L, B, Hq, 128), torch.float32)
        ws = guarded_ws(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, max_loc))
        msa.msa_sparse_decode(q, ck.t, cv.t, cl.t, lk, lv, ll, SCALE, out.t, ws.t)
        out.check("decode out Hq=%d" % Hq)
        ws.check("decode workspace Hq=%d" % Hq)


def test_canaries_prefill_and_encode():
    print("case: canaries around prefill and encode", flush=True)
    rng = np.random.default_rng(32)
    L, B, T, Hq = 2, 2, 37, 32
    max_ctx, max_loc = 70, 50
    q = to_dev_bf16(rand_bf16(rng, (L, B, T, Hq, 128)))
    ck = to_dev_bf16(rand_bf16(rng, (L, B, max_ctx, 8, 128)))
    cv = to_dev_bf16(rand_bf16(rng, (L, B, max_ctx, 8, 128)))
    lk = to_dev_bf16(rand_bf16(rng, (L, B, max_loc, 8, 128)))
    lv = to_dev_bf16(rand_bf16(rng, (L, B, max_loc, 8, 128)))
    cl = torch.tensor([[0, 70], [33, 1]], dtype=torch.int32, device=DEV)
    ll = torch.tensor([[50, 40], [37, 50]], dtype=torch.int32, device=DEV)
    out = Guarded((L, B, T, Hq, 128), torch.float32)
    msa.msa_sparse_prefill(q, ck, cv, cl, lk, lv, ll, SCALE, out.t)
    out.check("prefill out")

    H = 256
    lens = np.array([1, 63, 64, 65, 0, 130, 7], np.int64)
    tok = np.zeros(len(lens) + 1, np.int64)
    tok[1:] = np.cumsum(lens)
    blk, n_blk, _ = msa.msa_block_offsets_host(torch.from_numpy(tok))
    n_tok = int(tok[-1])
    tiles = msa.msa_route_tiles(n_blk)
    x = to_dev_bf16(rand_bf16(rng, (L, n_tok, H)))
    w = [to_dev_bf16(S.f32_to_bf16((rng.standard_normal((L, 1024, H)) / math.sqrt(H)).astype(np.float32)))
         for _ in range(3)]
    wn = to_dev_bf16(rand_bf16(rng, (L, 128)))
    kbar = Guarded((L, n_blk, 8, 128), torch.bfloat16)
    vbar = Guarded((L, n_blk, 8, 128), torch.bfloat16)
    krt = Guarded((L, tiles * 16, 8, 128), torch.bfloat16)
    krn = Guarded((L, tiles * 16, 8), torch.float32)
    msa.msa_encode_blocks(x, w[0], w[1], w[2], wn, 1e-6, 1e4, torch.from_numpy(tok).to(DEV), blk.to(DEV), n_blk,
                          kbar.t, vbar.t, krt.t, krn.t)
    for g, name in ((kbar, "encode kbar"), (vbar, "encode vbar"), (krt, "encode krbar_route"),
                    (krn, "encode krbar_norm")):
        g.check(name)
