"""msa_route_topk_noalloc (the entry point for callers that cannot allocate: its scratch is
the library's fixed per-GPU array) against msa_route_topk with a caller workspace, through
the C ABI: two calls in a row, the second smaller than the first, so leftovers of the first
call in the shared scratch would show up in the second."""
import numpy as np
import pytest
import torch

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


from gpu_common import assert_topk, doc_map, pack_rows, route, to_dev_bf16, u16, untile_keys  # noqa: E402

import oracle as O  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402
from synth import synth as S  # noqa: E402


def rand_bf16(rng, shape):
    return S.f32_to_bf16(rng.standard_normal(shape).astype(np.float32))


def memory(rng, L, counts):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    n_blk = int(off[-1])
    rows = to_dev_bf16(rand_bf16(rng, (L, n_blk, 8, 128)))
    krt, krn = pack_rows(rows, n_blk)
    off_d = torch.from_numpy(off).to(DEV)
    return off, off_d, n_blk, krt, krn, doc_map(off_d, n_blk)


def noalloc(qr, krt, krn, n_blk, blk_doc, n_docs, k, keep_scores, norms):
    L, B = qr.shape[0], qr.shape[1]
    ids = torch.full((L, B, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((L, B, k), 9.0, dtype=torch.float32, device=DEV)
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=DEV) if keep_scores else None
    msa.msa_route_topk_noalloc(qr, krt, n_blk, blk_doc, n_docs, k, ids, sc, doc_scores=dsc,
                               krbar_norm=krn if norms else None)
    return ids, sc, dsc


@pytest.mark.parametrize("keep_scores", [False, True])
def test_noalloc_matches_workspace_entry_point_twice(keep_scores):
    rng = np.random.default_rng(31 + keep_scores)
    print("case: no-alloc route+top-k, call 1 (3 layers, 2 queries x 70 tokens, 700 docs, k=16)", flush=True)
    counts = rng.integers(0, 30, 700)
    counts[:3] = 0                                     # empty documents score -inf
    off, off_d, n_blk, krt, krn, blk_doc = memory(rng, 3, counts)
    qr = to_dev_bf16(rand_bf16(rng, (3, 2, 70, 8, 128)))
    n_docs = len(counts)
    ids_w, sc_w, dsc_w = route(qr, krt, krn, n_blk, off_d, 16, blk_doc=blk_doc, norms=True)
    ids_n, sc_n, dsc_n = noalloc(qr, krt, krn, n_blk, blk_doc, n_docs, 16, keep_scores, True)
    torch.cuda.synchronize()
    assert torch.equal(ids_w, ids_n) and torch.equal(sc_w, sc_n)
    if keep_scores:
        assert torch.equal(dsc_w, dsc_n)

    print("case: no-alloc route+top-k, call 2 (1 layer, 1 query x 8 tokens, 90 docs, k=5)", flush=True)
    counts2 = rng.integers(1, 12, 90)
    off2, off2_d, n_blk2, krt2, krn2, blk_doc2 = memory(rng, 1, counts2)
    qr2 = to_dev_bf16(rand_bf16(rng, (1, 1, 8, 8, 128)))
    ids_w2, sc_w2, dsc_w2 = route(qr2, krt2, krn2, n_blk2, off2_d, 5, blk_doc=blk_doc2, norms=False)
    ids_n2, sc_n2, dsc_n2 = noalloc(qr2, krt2, krn2, n_blk2, blk_doc2, len(counts2), 5, keep_scores, False)
    torch.cuda.synchronize()
    assert torch.equal(ids_w2, ids_n2) and torch.equal(sc_w2, sc_n2)
    if keep_scores:
        assert torch.equal(dsc_w2, dsc_n2)
    # and the second call's selection is the oracle's
    S_o = O.doc_scores(u16(qr2[0, 0]), untile_keys(krt2, n_blk2)[0], off2)
    assert_topk(ids_n2[0, 0].cpu().numpy(), sc_n2[0, 0].cpu().numpy(), dsc_w2[0, 0].cpu().numpy(), S_o, 5)


def test_noalloc_rejects_scratch_beyond_its_maximum():
    rng = np.random.default_rng(33)
    counts = np.ones(64, np.int64)
    off, off_d, n_blk, krt, krn, blk_doc = memory(rng, 1, counts)
    qr = to_dev_bf16(rand_bf16(rng, (1, 1, 16, 8, 128)))
    ids = torch.empty((1, 1, 16), dtype=torch.int32, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_route_topk_noalloc(qr, krt, n_blk, blk_doc, 20_000_000, 16, ids, None)
    assert e.value.status == msa.MSA_ERR_WORKSPACE
