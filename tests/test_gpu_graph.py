"""The path captured in a HIP graph: pooling, the routing scan with top-k (with a workspace and
without one), the gather, the decode and the prefill are recorded once and replayed; every
replay must give exactly the eager results, with the program's own eager work (which
overwrites the outputs and reuses the scratch) between replays, and a replay after the
inputs change must follow the new inputs.  The entry points allocate nothing and issue no
memory-set nodes, so a capture holds only their kernels."""
import numpy as np
import pytest
import torch

from synth import synth as S
from synth.device import DeviceInputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routed_kv_memory_amd import msa
    msa.lib()
    yield
    torch.cuda.synchronize()


from gpu_common import SCALE, alloc_route_keys, doc_map, to_dev_bf16  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def test_captured_path_replays_match_eager():
    print("case: graph capture of pool, route (workspace and scratch), gather, decode, prefill", flush=True)
    cfg = S.CONFIGS["tiny"]
    di = DeviceInputs(cfg, DEV)
    tok, k, v, kr = di.per_token()
    blk, n_blk, max_db = msa.msa_block_offsets_host(tok)
    L = cfg.n_layers
    n_docs = blk.numel() - 1
    tok_d, blk_d = tok.to(DEV), blk.to(DEV)
    B, T, kk, Hq, n_loc, Tp = 3, 130, 4, 32, 40, 24      # several query chunks: the shared-range scan
    max_ctx = kk * max_db
    rng = np.random.default_rng(77)

    def rand_bf16(shape):
        return to_dev_bf16(S.f32_to_bf16(rng.standard_normal(shape).astype(np.float32)))

    # inputs (static addresses: a replay reads whatever they hold then)
    qr = rand_bf16((L, B, T, 8, 128))
    q = rand_bf16((L, B, Hq, 128))
    lk = rand_bf16((L, B, n_loc, 8, 128))
    lv = rand_bf16((L, B, n_loc, 8, 128))
    ll = torch.full((L, B), n_loc, dtype=torch.int32, device=DEV)
    qp = rand_bf16((L, B, Tp, Hq, 128))
    # outputs and workspaces, all allocated before the capture
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    krt, krn = alloc_route_keys(L, n_blk)
    blk_doc = doc_map(blk_d, n_blk)
    ws_r = torch.empty(msa.msa_route_topk_workspace_size(L, B, n_docs, kk), dtype=torch.uint8, device=DEV)
    ids = torch.empty((L, B, kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((L, B, kk), dtype=torch.float32, device=DEV)
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=DEV)
    ids_n = torch.empty_like(ids)
    sc_n = torch.empty_like(sc)
    ck = torch.zeros((L, B, max_ctx, 8, 128), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros_like(ck)
    cl = torch.empty((L, B), dtype=torch.int32, device=DEV)
    ws_d = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, n_loc), dtype=torch.uint8,
                       device=DEV)
    out = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=DEV)
    outp = torch.empty((L, B, Tp, Hq, 128), dtype=torch.float32, device=DEV)
    outs = [kbar, vbar, krt, krn, ids, sc, dsc, ids_n, sc_n, ck, cv, cl, out, outp]

    def step():
        msa.msa_pool_blocks(k, v, kr, tok_d, blk_d, n_blk, kbar, vbar, krt, krn)
        msa.msa_route_topk(qr, krt, n_blk, blk_doc, n_docs, kk, ids, sc, ws_r, doc_scores=dsc, krbar_norm=krn)
        msa.msa_route_topk_noalloc(qr, krt, n_blk, blk_doc, n_docs, kk, ids_n, sc_n, krbar_norm=krn)
        msa.msa_gather_ctx(ids, blk_d, max_db, kbar, vbar, ck, cv, cl)
        msa.msa_sparse_decode(q, ck, cv, cl, lk, lv, ll, SCALE, out, ws_d)
        msa.msa_sparse_prefill(qp, ck, cv, cl, lk, lv, ll, SCALE, outp)

    def snapshot():
        torch.cuda.synchronize()
        return [x.clone() for x in outs]

    def clobber():
        # eager work between replays: other scores through the shared scratch, outputs overwritten
        other = torch.empty_like(dsc)
        msa.msa_route_topk_noalloc(rand_bf16((L, B, T, 8, 128)), krt, n_blk, blk_doc, n_docs, kk,
                                   torch.empty_like(ids), torch.empty_like(sc), doc_scores=other, krbar_norm=krn)
        for x in outs:
            x.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()

    def at(t):
        return next(i for i, x in enumerate(outs) if x is t)

    ctx_ix = (at(ck), at(cv))

    def check(ref, tag):
        torch.cuda.synchronize()
        n_rows = ref[at(cl)].cpu()
        for i, (x, y) in enumerate(zip(outs, ref)):
            if i in ctx_ix:          # the gather defines a context's first ctx_len rows only
                for l in range(L):
                    for b in range(B):
                        n = int(n_rows[l, b])
                        ok = torch.equal(_bits(x[l, b, :n]), _bits(y[l, b, :n]))
                        assert ok, "%s: output %d differs (layer %d, query %d)" % (tag, i, l, b)
            else:
                assert torch.equal(_bits(x), _bits(y)), "%s: output %d differs" % (tag, i)

    step()                      # eager reference (and the scratch's one-time lookup)
    ref = snapshot()
    assert bool((ids == ids_n).all()) and bool((sc == sc_n).all())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        clobber()
        g.replay()
        check(ref, "replay %d" % rep)

    # new inputs at the same addresses: the replay follows them
    qr.copy_(rand_bf16((L, B, T, 8, 128)))
    q.copy_(rand_bf16((L, B, Hq, 128)))
    step()
    ref2 = snapshot()
    assert not torch.equal(ref2[at(dsc)], ref[at(dsc)])
    clobber()
    g.replay()
    check(ref2, "new inputs")
