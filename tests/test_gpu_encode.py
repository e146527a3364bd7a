"""Offline encode front-end (projections, per-head key normalisation, document-wise
rotary positions, 64-token block pooling) against the oracle's fp64 definition.

Tolerance, derived from the arithmetic: the device accumulates each projection (a dot
product of length H) in fp32 and the oracle in fp64, so before the single rounding to
bf16 the two differ by a few fp32 roundings of the row's scale; after it they agree
within one bf16 ulp of the oracle's value, except where cancellation leaves a pooled
value far below its row's scale, whose ulp is smaller than that fp32 difference: there
the bound is 2^-16 of the row's largest magnitude."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import synth as S

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


from gpu_common import alloc_route_keys, to_dev_bf16, u16, untile_keys, untile_norms  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402


def assert_pooled_close(got, ref, what):
    g = S.bf16_to_f32(got).astype(np.float64)
    r = S.bf16_to_f32(ref).astype(np.float64)
    mag = np.abs(r)
    ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    floor = np.exp2(-16) * mag.max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bad = err > np.maximum(ulp, floor)
    assert not bad.any(), (what, np.argwhere(bad)[:5], g[bad][:5], r[bad][:5])
    assert (err > 0).mean() < 0.02, (what, (err > 0).mean())


def make_weights(rng, L, Hd):
    sc = 2.0 ** -np.round(np.log2(np.sqrt(Hd)))        # exact in bf16: projections ~ N(0, 1)
    w = [S.f32_to_bf16((rng.standard_normal((L, Hd, 1024)) * sc).astype(np.float32)) for _ in range(3)]
    wn = S.f32_to_bf16((1.0 + 0.25 * rng.standard_normal((L, 128))).astype(np.float32))
    return w, wn


def run_encode(x, w, wn, eps, theta, tok, with_norms=True):
    L = x.shape[0]
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    kbar = torch.full((L, max(n_blk, 1), 8, 128), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vbar = torch.full_like(kbar, -1)
    krt, krn = alloc_route_keys(L, n_blk)
    krt.view(torch.int16).fill_(-1)
    krn.fill_(-1.0)
    # the library takes the weights output-major ([L][1024][H]), the oracle input-major
    msa.msa_encode_blocks(to_dev_bf16(x), *[to_dev_bf16(a.transpose(0, 2, 1)) for a in w], to_dev_bf16(wn), eps, theta,
                          torch.from_numpy(tok).to(DEV), blk.to(DEV), n_blk, kbar, vbar, krt,
                          krn if with_norms else None)
    torch.cuda.synchronize()
    return blk.numpy(), n_blk, kbar, vbar, krt, krn


def check_layerwise(x, w, wn, eps, theta, tok, with_norms=True):
    blk, n_blk, kbar, vbar, krt, krn = run_encode(x, w, wn, eps, theta, tok, with_norms)
    L = x.shape[0]
    got_k, got_v, got_r = u16(kbar)[:, :n_blk], u16(vbar)[:, :n_blk], untile_keys(krt, n_blk)
    for l in range(L):
        rk, rv, rr = O.encode(x[l], w[0][l], w[1][l], w[2][l], wn[l], eps, theta, tok, blk)
        assert_pooled_close(got_k[l], rk, "K layer %d" % l)
        assert_pooled_close(got_v[l], rv, "V layer %d" % l)
        assert_pooled_close(got_r[l], rr, "Kr layer %d" % l)
    tiles = msa.msa_route_tiles(n_blk)
    full = untile_keys(krt, tiles * 16)
    assert np.all(full[:, n_blk:] == 0)                     # padding rows of the last tile
    if with_norms:
        assert np.allclose(untile_norms(krn, n_blk), O.head_norms(got_r), rtol=1e-6, atol=0)
        assert np.all(untile_norms(krn, tiles * 16)[:, n_blk:] == 0)
    else:
        assert np.all(krn.cpu().numpy() == -1.0)           # not written


def test_ragged_documents_all_outputs():
    """Documents of 1, 63, 64, 65 tokens, an empty one, and longer ones; two layers."""
    print("case: encode ragged H=384", flush=True)
    rng = np.random.default_rng(301)
    lens = np.array([1, 63, 64, 65, 0, 130, 200, 7, 640, 129])
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    L, Hd = 2, 384
    x = S.f32_to_bf16(rng.standard_normal((L, int(tok[-1]), Hd)).astype(np.float32))
    w, wn = make_weights(rng, L, Hd)
    check_layerwise(x, w, wn, 1e-6, 1e6, tok)


def test_many_tiles_wide_hidden_no_norms():
    print("case: encode H=256 many tiles", flush=True)
    rng = np.random.default_rng(302)
    lens = rng.integers(1, 400, 30)
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    L, Hd = 1, 256
    x = S.f32_to_bf16(rng.standard_normal((L, int(tok[-1]), Hd)).astype(np.float32))
    w, wn = make_weights(rng, L, Hd)
    check_layerwise(x, w, wn, 1e-6, 1e6, tok, with_norms=False)


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_long_document_positions(theta):
    """One 12,000-token document: rotation angles up to 12,000 radians."""
    print("case: encode long document theta=%g" % theta, flush=True)
    rng = np.random.default_rng(303)
    tok = np.array([0, 5, 12005], np.int64)
    L, Hd = 1, 128
    x = S.f32_to_bf16(rng.standard_normal((L, 12005, Hd)).astype(np.float32))
    w, wn = make_weights(rng, L, Hd)
    check_layerwise(x, w, wn, 1e-6, theta, tok)


def test_zero_rows_use_eps():
    """All-zero hidden rows give a zero key whatever eps (no division by zero)."""
    print("case: encode zero rows", flush=True)
    rng = np.random.default_rng(304)
    tok = np.array([0, 70, 140], np.int64)
    L, Hd = 1, 128
    x = S.f32_to_bf16(rng.standard_normal((L, 140, Hd)).astype(np.float32))
    x[0, :70] = 0
    w, wn = make_weights(rng, L, Hd)
    blk, n_blk, kbar, vbar, krt, krn = run_encode(x, w, wn, 1e-6, 1e6, tok)
    assert np.all(u16(kbar)[0, :2] == 0) and np.all(u16(vbar)[0, :2] == 0)
    check_layerwise(x, w, wn, 1e-6, 1e6, tok)


def test_full_size_encode_sampled():
    """The encode workload at its full size and in bench.py's launch configuration (18 layers x
    947,395 tokens x hidden 2,560, one launch): sampled blocks against the oracle -- the key of
    documents' first blocks (positions 0..63), value and routing key of blocks anywhere (they do
    not depend on position) -- plus the stored routing-key norms of whole tiles."""
    print("case: encode full size (18 x 947,395 x 2,560)", flush=True)
    from synth.device import DeviceInputs
    torch.cuda.empty_cache()
    cfg = S.CONFIGS["1m"]
    Hd, eps, theta = S.ENC_HIDDEN, 1e-6, 1e6
    tok, x, wk, wv, wr, wn = DeviceInputs(cfg, DEV).encode_inputs(Hd)
    L, n_tok = x.shape[0], x.shape[1]
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    krt, krn = alloc_route_keys(L, n_blk)
    msa.msa_encode_blocks(x, wk, wv, wr, wn, eps, theta, tok.to(DEV), blk.to(DEV), n_blk, kbar, vbar, krt, krn)
    torch.cuda.synchronize()
    del x
    seed = S.memory_config(cfg).seed
    tok_n, blk_n = tok.numpy(), blk.numpy()
    rng = np.random.default_rng(71)
    wn_h = u16(wn)
    for l in (0, 9, L - 1):
        w_h = [np.ascontiguousarray(S.enc_weights_host(seed, st, l, Hd).T)
               for st in (S.S_ENC_WK, S.S_ENC_WV, S.S_ENC_WKR)]
        d = int(rng.integers(0, tok_n.size - 1))
        nb = int(blk_n[d + 1] - blk_n[d])
        for jb, keys in ((0, "KVR"), (int(rng.integers(0, nb)), "VR"), (nb - 1, "VR")):
            t0 = int(tok_n[d]) + 64 * jb
            t1 = min(t0 + 64, int(tok_n[d + 1]))
            xh = S.enc_x_host(seed, l, n_tok, Hd, t0, t1)
            ref = O.encode(xh, *w_h, wn_h[l], eps, theta, np.array([0, t1 - t0], np.int64),
                           np.array([0, 1], np.int64))
            b = int(blk_n[d]) + jb
            got = {"K": u16(kbar[l, b]), "V": u16(vbar[l, b]),
                   "R": untile_keys(krt[l:l + 1, 16 * (b // 16):16 * (b // 16) + 16], 16)[0, b % 16]}
            for key, r in zip("KVR", ref):
                if key in keys:
                    assert_pooled_close(got[key][None], r, "%s layer %d doc %d block %d" % (key, l, d, jb))
    # stored norms of the routing keys, two whole layers
    for l in (0, L - 1):
        rows = untile_keys(krt[l:l + 1], n_blk)
        assert np.allclose(untile_norms(krn[l:l + 1], n_blk), O.head_norms(rows), rtol=1e-6, atol=0)
