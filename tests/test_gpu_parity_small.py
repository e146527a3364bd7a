"""GPU parity against the fp64 oracle at sizes the oracle finishes in seconds:
the tiny workload end to end, plus ragged/edge shapes of every entry point.
Each oracle step consumes the GPU's previous-step output (step-isolated)."""
import numpy as np
import pytest
import torch

import oracle as O
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


from gpu_common import (SCORE_TOL, SCALE, alloc_route_keys, assert_decode, assert_topk, decode_all,  # noqa: E402
                        doc_map, gather_all, pack_rows, route, to_dev_bf16, u16, untile_keys, untile_norms)
from routed_kv_memory_amd import msa  # noqa: E402


def rand_bf16(rng, shape):
    return S.f32_to_bf16(rng.standard_normal(shape).astype(np.float32))


# ------------------------------------------------------------------ the tiny workload, end to end

def test_tiny_workload_end_to_end():
    cfg = S.CONFIGS["tiny"]
    print("case: tiny workload end to end", flush=True)
    di = DeviceInputs(cfg, DEV)
    tok, k, v, kr = di.per_token()
    blk, n_blk, max_db = msa.msa_block_offsets_host(tok)
    L = cfg.n_layers
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    krt, krn = alloc_route_keys(L, n_blk)
    tok_d, blk_d = tok.to(DEV), blk.to(DEV)
    msa.msa_pool_blocks(k, v, kr, tok_d, blk_d, n_blk, kbar, vbar, krt, krn)
    torch.cuda.synchronize()
    tok_n, blk_n = tok.numpy(), blk.numpy()
    # inputs regenerate on the host bit-identically
    assert np.array_equal(u16(k)[0, :100], S.rows_host(cfg.seed, S.S_K, 0, int(tok_n[-1]), 0, 100))
    # A1: pooled K, V, Kr bit-exact (fp64 sums of bf16 values are exact here, and both sides
    # round the fp64 mean once to bf16); norms of the stored Kr-bar within 1e-6 relative
    for name, x, got in (("K", k, u16(kbar)), ("V", v, u16(vbar)), ("Kr", kr, untile_keys(krt, n_blk))):
        ref = O.pool(u16(x), tok_n, blk_n)
        assert np.array_equal(ref, got), name
    krbar = untile_keys(krt, n_blk)
    nref = O.head_norms(krbar)
    assert np.allclose(untile_norms(krn, n_blk), nref, rtol=1e-6, atol=0)
    # A2 + A3
    qr = di.qr()
    ids, sc, dsc = route(qr, krt, krn, n_blk, blk_d, cfg.k)
    torch.cuda.synchronize()
    S_o = O.doc_scores(u16(qr)[0, 0], krbar[0], blk_n)
    dsc_h = dsc.cpu().numpy()[0, 0]
    assert np.max(np.abs(S_o - dsc_h)) < SCORE_TOL
    assert_topk(ids.cpu().numpy()[0, 0], sc.cpu().numpy()[0, 0], dsc_h, S_o, cfg.k)
    needles = set(S.needle_docs(cfg)[0].tolist())
    assert set(ids.cpu().numpy()[0, 0, :2].tolist()) == needles
    # A4: bit-exact gather of the GPU's selection
    ck, cv, cl = gather_all(ids, blk_d, max_db, kbar, vbar)
    torch.cuda.synchronize()
    ref_k, ref_v = O.gather(ids.cpu().numpy()[0, 0], blk_n, u16(kbar)[0], u16(vbar)[0])
    n_ctx = int(cl.cpu()[0, 0])
    assert n_ctx == ref_k.shape[0]
    assert np.array_equal(u16(ck)[0, 0, :n_ctx], ref_k) and np.array_equal(u16(cv)[0, 0, :n_ctx], ref_v)
    # A5
    q, lk, lv, ll = di.decode_inputs()
    out = decode_all(q, ck, cv, cl, lk, lv, ll)
    torch.cuda.synchronize()
    ref = O.decode(u16(q)[0, 0], ref_k, ref_v, u16(lk)[0, 0], u16(lv)[0, 0], SCALE)
    assert_decode(out.cpu().numpy()[0, 0], ref)


# ----------------------------------------------------------------------- routing shapes

def _memory(rng, L, lens_blocks):
    off = np.concatenate([[0], np.cumsum(lens_blocks)]).astype(np.int64)
    n_blk = int(off[-1])
    rows = rand_bf16(rng, (L, max(n_blk, 1), 8, 128))[:, :n_blk]
    return off, n_blk, rows


@pytest.mark.parametrize("norms", [False, True])
@pytest.mark.parametrize("T,B", [(1, 1), (5, 2), (15, 1), (16, 1), (17, 2), (40, 1), (64, 1), (65, 2), (130, 1)])
def test_route_scores_and_topk_shapes(T, B, norms):
    print("case: route T=%d B=%d norms=%d" % (T, B, norms), flush=True)
    rng = np.random.default_rng(1000 + T * 7 + B)
    L = 2
    lens = rng.integers(1, 9, 45)
    lens[[3, 17, 44]] = 0                    # empty documents
    off, n_blk, rows = _memory(rng, L, lens)  # ragged: n_blk is not a multiple of 16 or 32
    qr = rand_bf16(rng, (L, B, T, 8, 128))
    # one block equal to a query token -> score 1 for that document (per layer)
    rows[0, off[5]] = qr[0, 0, T - 1]
    rows[1, off[31] - 1] = qr[1, B - 1, 0]   # last block of doc 30
    krt, krn = pack_rows(to_dev_bf16(rows), n_blk)
    blk_d = torch.from_numpy(off).to(DEV)
    k = 7
    ids, sc, dsc = route(to_dev_bf16(qr), krt, krn, n_blk, blk_d, k, norms=norms)
    torch.cuda.synchronize()
    assert np.array_equal(untile_keys(krt, n_blk), rows)
    assert np.allclose(untile_norms(krn, n_blk), O.head_norms(rows), rtol=1e-6, atol=0)
    dsc_h, ids_h, sc_h = dsc.cpu().numpy(), ids.cpu().numpy(), sc.cpu().numpy()
    for l in range(L):
        for b in range(B):
            S_o = O.doc_scores(qr[l, b], rows[l], off)
            fin = np.isfinite(S_o)
            assert np.array_equal(fin, np.isfinite(dsc_h[l, b]))
            assert np.max(np.abs(S_o[fin] - dsc_h[l, b][fin])) < SCORE_TOL
            assert np.all(dsc_h[l, b][~fin] == -np.inf)
            assert_topk(ids_h[l, b], sc_h[l, b], dsc_h[l, b], S_o, k)
    assert abs(dsc_h[0, 0, 5] - 1.0) < SCORE_TOL and abs(dsc_h[1, B - 1, 30] - 1.0) < SCORE_TOL


@pytest.mark.parametrize("norms", [False, True])
def test_route_accumulate_equals_full_query(norms):
    """Re-routing a grown query by max-merging the appended rows' scores is exact (every call
    either reads the key norms or recomputes them)."""
    print("case: route accumulate norms=%d" % norms, flush=True)
    rng = np.random.default_rng(7)
    L, B = 2, 2
    off, n_blk, rows = _memory(rng, L, rng.integers(1, 20, 60))
    krt, krn = pack_rows(to_dev_bf16(rows), n_blk)
    blk_d = torch.from_numpy(off).to(DEV)
    qr = rand_bf16(rng, (L, B, 64 + 128, 8, 128))
    n_docs = len(off) - 1
    m = doc_map(blk_d, n_blk)
    nrm = krn if norms else None
    full = torch.empty((L, B, n_docs), dtype=torch.float32, device=DEV)
    msa.msa_route_scores(to_dev_bf16(qr), krt, n_blk, m, n_docs, full, krbar_norm=nrm)
    inc = torch.empty_like(full)
    msa.msa_route_scores(to_dev_bf16(qr[:, :, :64]), krt, n_blk, m, n_docs, inc, krbar_norm=nrm)
    first = inc.clone()
    msa.msa_route_scores(to_dev_bf16(qr[:, :, 64:]), krt, n_blk, m, n_docs, inc, accumulate=True, krbar_norm=nrm)
    torch.cuda.synchronize()
    assert torch.equal(inc, full)
    assert bool((inc >= first).all())


def test_topk_multi_pass_and_ties():
    """More documents than one selection workgroup holds, with ties, -inf and k up to 256."""
    print("case: top-k multi pass", flush=True)
    rng = np.random.default_rng(9)
    L, B, n_docs = 2, 3, 70001
    sc = np.round(rng.standard_normal((L, B, n_docs)), 2).astype(np.float32)
    sc[0, 0, ::7] = -np.inf
    for k in (1, 2, 16, 63, 64, 65, 256):
        ws = torch.empty(msa.msa_topk_docs_workspace_size(L, B, n_docs, k), dtype=torch.uint8, device=DEV)
        ids = torch.empty((L, B, k), dtype=torch.int32, device=DEV)
        out = torch.empty((L, B, k), dtype=torch.float32, device=DEV)
        msa.msa_topk_docs(torch.from_numpy(sc).to(DEV), k, ids, out, ws)
        torch.cuda.synchronize()
        for l in range(L):
            for b in range(B):
                ref_ids, ref_sc = O.topk(sc[l, b].astype(np.float64), k)
                assert ids.cpu().numpy()[l, b].tolist() == ref_ids.tolist()
                assert np.array_equal(out.cpu().numpy()[l, b], ref_sc.astype(np.float32))


@pytest.mark.gpu
@pytest.mark.parametrize("n_docs,k", [(5, 5), (64, 64), (2048, 1), (2048, 64), (2049, 64), (2049, 3),
                                      (4097, 16), (6144, 64), (131072, 16), (256, 256), (1000, 256), (70000, 256)])
def test_topk_chunk_edges(n_docs, k):
    """Row lengths at and around the selection chunk, k equal to the row length, k at the
    register path's limit; every score equal in one row (order by id alone)."""
    print("case: top-k edges n_docs=%d k=%d" % (n_docs, k), flush=True)
    rng = np.random.default_rng(n_docs * 131 + k)
    L, B = 2, 2
    sc = rng.standard_normal((L, B, n_docs)).astype(np.float32)
    sc[1, 1, :] = 0.25
    ws = torch.empty(max(1, msa.msa_topk_docs_workspace_size(L, B, n_docs, k)), dtype=torch.uint8, device=DEV)
    ids = torch.empty((L, B, k), dtype=torch.int32, device=DEV)
    out = torch.empty((L, B, k), dtype=torch.float32, device=DEV)
    msa.msa_topk_docs(torch.from_numpy(sc).to(DEV), k, ids, out, ws)
    torch.cuda.synchronize()
    ids_h, out_h = ids.cpu().numpy(), out.cpu().numpy()
    for l in range(L):
        for b in range(B):
            ref_ids, ref_sc = O.topk(sc[l, b].astype(np.float64), k)
            assert ids_h[l, b].tolist() == ref_ids.tolist(), (l, b)
            assert np.array_equal(out_h[l, b], ref_sc.astype(np.float32))


def test_topk_rank_selection_random_rows():
    """Rows built so that the k-th best key sits near the lower bound the register path takes
    from its lanes' maxima (few distinct scores, -inf runs, rows a little longer or shorter than
    a chunk, k from 1 to 64), and rows with one score repeated so many times that the path keeps
    its fallback: ids and scores must equal the oracle's full sort exactly."""
    print("case: top-k rank selection, random rows", flush=True)
    rng = np.random.default_rng(41)
    for case in range(12):
        n_docs = int(rng.choice([33, 511, 2047, 2048, 2049, 4100, 9000]))
        k = int(rng.integers(1, 65))
        k = min(k, n_docs)
        L, B = 1, 3
        distinct = int(rng.choice([3, 17, 1000]))
        sc = (rng.integers(0, distinct, (L, B, n_docs)) / distinct).astype(np.float32)
        sc[0, 1, rng.random(n_docs) < 0.3] = -np.inf
        sc[0, 2, :] = 0.5
        sc[0, 2, rng.integers(0, n_docs, 5)] = 0.75
        ws = torch.empty(max(1, msa.msa_topk_docs_workspace_size(L, B, n_docs, k)), dtype=torch.uint8, device=DEV)
        ids = torch.empty((L, B, k), dtype=torch.int32, device=DEV)
        out = torch.empty((L, B, k), dtype=torch.float32, device=DEV)
        msa.msa_topk_docs(torch.from_numpy(sc).to(DEV), k, ids, out, ws)
        torch.cuda.synchronize()
        ids_h, out_h = ids.cpu().numpy(), out.cpu().numpy()
        for b in range(B):
            ref_ids, ref_sc = O.topk(sc[0, b].astype(np.float64), k)
            assert ids_h[0, b].tolist() == ref_ids.tolist(), (case, n_docs, k, b)
            assert np.array_equal(out_h[0, b], ref_sc.astype(np.float32)), (case, n_docs, k, b)


# ----------------------------------------------------------------------- pooling edges

def test_pool_cancellation_tiny_and_huge_values():
    """Means that nearly cancel, land in the bf16 subnormal range, or sit near the largest finite
    bf16: the device's fp64 sums and single rounding must give the oracle's bits exactly."""
    print("case: pool cancellation / subnormal / large", flush=True)
    rng = np.random.default_rng(12)
    def bits(vals):
        return S.f32_to_bf16(np.asarray(vals, np.float32))
    lens = np.array([3, 3, 2, 64, 5, 7, 1])
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    n_tok = int(tok[-1])
    x = rand_bf16(rng, (1, n_tok, 8, 128))
    t = 0
    x[0, t:t + 3, :, :] = bits([1.0, 2.0 ** -20, -1.0])[:, None, None]            # cancels to 2^-20 / 3
    t += 3
    x[0, t:t + 3, :, :] = bits([2.0 ** -126, 2.0 ** -130, -(2.0 ** -126)])[:, None, None]   # subnormal mean
    t += 3
    x[0, t:t + 2, :, :] = bits([3.0e38, 3.3e38])[:, None, None]                   # near the largest finite
    t += 2
    big = rand_bf16(rng, (64, 8, 128))                                            # a full block whose sum cancels
    big[32:] = big[:32] ^ np.uint16(0x8000)
    big[31] = bits([2.0 ** -10])[0]
    big[63] = bits([2.0 ** -12])[0]                                               # sum (2^-10 + 2^-12) / 64
    x[0, t:t + 64] = big
    t += 64
    x[0, t:t + 5, 0, :3] = bits([2.0 ** -133, 3 * 2.0 ** -133, 2.0 ** -130])      # smallest subnormals
    xs = [x, x[:, ::-1].copy(), S.f32_to_bf16((rng.standard_normal((1, n_tok, 8, 128)) * 1e-30).astype(np.float32))]
    kbar = torch.empty((1, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    krt, krn = alloc_route_keys(1, n_blk)
    msa.msa_pool_blocks(*[to_dev_bf16(a) for a in xs], torch.from_numpy(tok).to(DEV), blk.to(DEV), n_blk,
                        kbar, vbar, krt, krn)
    torch.cuda.synchronize()
    for name, a, got in zip("KVR", xs, (u16(kbar), u16(vbar), untile_keys(krt, n_blk))):
        ref = O.pool(a, tok, blk.numpy())
        assert np.array_equal(ref, got), (name, np.argwhere(ref != got)[:5])



def test_pool_ragged_documents():
    print("case: pool ragged", flush=True)
    rng = np.random.default_rng(11)
    lens = np.array([1, 63, 64, 65, 0, 127, 128, 129, 3, 0, 700, 2])
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    L, n_tok = 3, int(tok[-1])
    xs = [rand_bf16(rng, (L, n_tok, 8, 128)) for _ in range(3)]
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    krt, krn = alloc_route_keys(L, n_blk)
    msa.msa_pool_blocks(*[to_dev_bf16(x) for x in xs], torch.from_numpy(tok).to(DEV), blk.to(DEV), n_blk,
                        kbar, vbar, krt, krn)
    torch.cuda.synchronize()
    for x, got in zip(xs, (u16(kbar), u16(vbar), untile_keys(krt, n_blk))):
        ref = O.pool(x, tok, blk.numpy())
        assert np.array_equal(ref, got)
    # padding rows of the last tile are zero with zero norm
    tiles = msa.msa_route_tiles(n_blk)
    full = untile_keys(krt, tiles * 16)
    assert np.all(full[:, n_blk:] == 0)
    assert np.all(untile_norms(krn, tiles * 16)[:, n_blk:] == 0)


@pytest.mark.parametrize("T,B", [(8, 2), (64, 1), (130, 2)])
def test_degenerate_memories(T, B):
    """The memory's degenerate cases through the whole path: every document empty (no tokens, no
    blocks: empty arrays passed as NULL, every score -inf, the top-k the first k ids, empty
    contexts, decode and prefill over the local rows alone), and a single document with k = 1."""
    print("case: degenerate memories T=%d B=%d" % (T, B), flush=True)
    rng = np.random.default_rng(71 + T + B)
    L, Hq, n_loc = 2, 32, 24
    for lens, k in (([0, 0, 0, 0, 0], 3), ([100], 1)):
        tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        n_tok = int(tok[-1])
        blk, n_blk, max_db = msa.msa_block_offsets_host(torch.from_numpy(tok))
        off = blk.numpy()
        n_docs = len(lens)
        kt, vt, rt = (rand_bf16(rng, (L, n_tok, 8, 128)) for _ in range(3))
        tiles = msa.msa_route_tiles(n_blk)
        kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
        vbar = torch.empty_like(kbar)
        krt = torch.empty((L, tiles * 16, 8, 128), dtype=torch.bfloat16, device=DEV)
        krn = torch.empty((L, tiles * 16, 8), dtype=torch.float32, device=DEV)
        blk_d = blk.to(DEV)
        msa.msa_pool_blocks(to_dev_bf16(kt), to_dev_bf16(vt), to_dev_bf16(rt), torch.from_numpy(tok).to(DEV), blk_d,
                            n_blk, kbar, vbar, krt, krn)
        blk_doc = torch.empty(tiles * 16, dtype=torch.int32, device=DEV)
        msa.msa_block_doc_map(blk_d, n_blk, blk_doc)
        qr = rand_bf16(rng, (L, B, T, 8, 128))
        ids, sc, dsc = route(to_dev_bf16(qr), krt, krn, n_blk, blk_d, k, blk_doc=blk_doc)
        max_ctx = max(1, k * max_db)
        ck, cv, cl = gather_all(ids, blk_d, max_db, kbar, vbar, max_ctx=max_ctx)
        q = rand_bf16(rng, (L, B, Hq, 128))
        lk, lv = rand_bf16(rng, (L, B, n_loc, 8, 128)), rand_bf16(rng, (L, B, n_loc, 8, 128))
        ll = torch.full((L, B), n_loc, dtype=torch.int32, device=DEV)
        out = decode_all(to_dev_bf16(q), ck, cv, cl, to_dev_bf16(lk), to_dev_bf16(lv), ll)
        torch.cuda.synchronize()
        if n_blk:
            kb_o, vb_o, kr_o = (O.pool(x, tok, off) for x in (kt, vt, rt))
            assert np.array_equal(u16(kbar), kb_o) and np.array_equal(u16(vbar), vb_o)
            assert np.array_equal(untile_keys(krt, n_blk), kr_o)
        else:
            kb_o = vb_o = kr_o = np.zeros((L, 0, 8, 128), np.uint16)
        for l in range(L):
            kr_rows = kr_o[l]
            for b in range(B):
                S_o = O.doc_scores(qr[l, b], kr_rows, off)
                d = dsc.cpu().numpy()[l, b]
                fin = np.isfinite(S_o)
                assert np.array_equal(fin, np.isfinite(d)) and np.all(d[~fin] == -np.inf)
                assert np.max(np.abs(S_o[fin] - d[fin]), initial=0.0) < SCORE_TOL
                assert_topk(ids.cpu().numpy()[l, b], sc.cpu().numpy()[l, b], d, S_o, k)
                rk, rv = O.gather(ids.cpu().numpy()[l, b], off, kb_o[l], vb_o[l])
                assert int(cl.cpu()[l, b]) == rk.shape[0] == (0 if not n_blk else n_blk)
                ref = O.decode(q[l, b], rk, rv, lk[l, b], lv[l, b], SCALE)
                assert_decode(out.cpu().numpy()[l, b], ref)


# ------------------------------------------------------------------ gather / decode edges

@pytest.mark.parametrize("Hq", [8, 16, 32, 64])
def test_gather_decode_edges(Hq):
    print("case: gather/decode Hq=%d" % Hq, flush=True)
    rng = np.random.default_rng(13 + Hq)
    L, B, k = 2, 3, 4
    off = np.array([0, 3, 3, 10, 11, 30, 31], np.int64)      # doc 1 empty, doc 4 has 19 blocks
    n_blk, max_db = int(off[-1]), 19
    kb, vb = rand_bf16(rng, (L, n_blk, 8, 128)), rand_bf16(rng, (L, n_blk, 8, 128))
    ids = np.array([[[4, 0, 2, 5], [1, 1, 3, 0], [-1, 99, 1, 1]],
                    [[5, 4, 3, 2], [0, 5, 1, 2], [2, 2, 2, 2]]], np.int32)   # invalid ids give no rows
    ck, cv, cl = gather_all(torch.from_numpy(ids).to(DEV), torch.from_numpy(off).to(DEV), max_db,
                            to_dev_bf16(kb), to_dev_bf16(vb))
    max_loc = 37
    lk, lv = rand_bf16(rng, (L, B, max_loc, 8, 128)), rand_bf16(rng, (L, B, max_loc, 8, 128))
    ll = np.array([[37, 0, 5], [1, 37, 0]], np.int32)        # query (0,2): no memory rows and 5 local
    q = rand_bf16(rng, (L, B, Hq, 128))
    out = decode_all(to_dev_bf16(q), ck, cv, cl, to_dev_bf16(lk), to_dev_bf16(lv), torch.from_numpy(ll).to(DEV))
    out0 = decode_all(to_dev_bf16(q), ck, cv, cl, None, None, None)          # no local part
    torch.cuda.synchronize()
    for l in range(L):
        for b in range(B):
            valid = ids[l, b][(ids[l, b] >= 0) & (ids[l, b] < len(off) - 1)]
            rk, rv = O.gather(valid, off, kb[l], vb[l])
            n_ctx = int(cl.cpu()[l, b])
            assert n_ctx == rk.shape[0]
            assert np.array_equal(u16(ck)[l, b, :n_ctx], rk) and np.array_equal(u16(cv)[l, b, :n_ctx], rv)
            ref = O.decode(q[l, b], rk, rv, lk[l, b, :ll[l, b]], lv[l, b, :ll[l, b]], SCALE)
            assert_decode(out.cpu().numpy()[l, b], ref)
            ref0 = O.decode(q[l, b], rk, rv, lk[l, b, :0], lv[l, b, :0], SCALE)
            assert_decode(out0.cpu().numpy()[l, b], ref0)
    # a query with neither memory nor local rows decodes to zero
    empty_ids = torch.full((1, 1, 1), -1, dtype=torch.int32, device=DEV)
    ck1, cv1, cl1 = gather_all(empty_ids, torch.from_numpy(off).to(DEV), max_db, to_dev_bf16(kb[:1]),
                               to_dev_bf16(vb[:1]))
    z = decode_all(to_dev_bf16(q[:1, :1]), ck1, cv1, cl1, None, None, None)
    torch.cuda.synchronize()
    assert int(cl1.cpu()[0, 0]) == 0 and bool((z == 0).all())


@pytest.mark.parametrize("Hq", [8, 64])
def test_decode_row_count_boundaries(Hq):
    """Total row counts around the 32-row wave and the 256-row split boundaries (and 128), with
    the memory / local seam inside a wave's rows."""
    print("case: decode boundaries Hq=%d" % Hq, flush=True)
    rng = np.random.default_rng(29 + Hq)
    totals = [1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512, 513]
    L, B = 1, len(totals)
    max_ctx, max_loc = 300, 300
    ck, cv = rand_bf16(rng, (L, B, max_ctx, 8, 128)), rand_bf16(rng, (L, B, max_ctx, 8, 128))
    lk, lv = rand_bf16(rng, (L, B, max_loc, 8, 128)), rand_bf16(rng, (L, B, max_loc, 8, 128))
    q = rand_bf16(rng, (L, B, Hq, 128))
    cl = np.array([[min(t // 2 + 3, t, max_ctx) for t in totals]], np.int32)
    ll = np.array([[t - c for t, c in zip(totals, cl[0])]], np.int32)
    assert (ll <= max_loc).all()
    out = decode_all(to_dev_bf16(q), to_dev_bf16(ck), to_dev_bf16(cv), torch.from_numpy(cl).to(DEV),
                     to_dev_bf16(lk), to_dev_bf16(lv), torch.from_numpy(ll).to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        ref = O.decode(q[0, b], ck[0, b, :cl[0, b]], cv[0, b, :cl[0, b]], lk[0, b, :ll[0, b]], lv[0, b, :ll[0, b]],
                       SCALE)
        assert_decode(out.cpu().numpy()[0, b], ref)


def test_decode_long_context_many_splits():
    print("case: decode long context", flush=True)
    rng = np.random.default_rng(17)
    L, B, Hq, n_ctx, n_loc = 1, 2, 32, 700, 1500
    ck = rand_bf16(rng, (L, B, n_ctx, 8, 128))
    cv = rand_bf16(rng, (L, B, n_ctx, 8, 128))
    lk = rand_bf16(rng, (L, B, n_loc, 8, 128))
    lv = rand_bf16(rng, (L, B, n_loc, 8, 128))
    q = rand_bf16(rng, (L, B, Hq, 128))
    q[0, 1] = S.f32_to_bf16(S.bf16_to_f32(q[0, 1]) * 8)       # peaked softmax
    cl = np.array([[n_ctx, 513]], np.int32)
    ll = np.array([[n_loc, 1]], np.int32)
    out = decode_all(to_dev_bf16(q), to_dev_bf16(ck), to_dev_bf16(cv), torch.from_numpy(cl).to(DEV),
                     to_dev_bf16(lk), to_dev_bf16(lv), torch.from_numpy(ll).to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        ref = O.decode(q[0, b], ck[0, b, :cl[0, b]], cv[0, b, :cl[0, b]], lk[0, b, :ll[0, b]], lv[0, b, :ll[0, b]],
                       SCALE)
        assert_decode(out.cpu().numpy()[0, b], ref)
