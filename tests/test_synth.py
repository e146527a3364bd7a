"""Host-side checks of the seeded input generator and of the workload recipes,
plus the needle pin of the oracle: planted needle documents rank first."""
import math

import numpy as np
import pytest

from synth import synth as S


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567 (reference implementation's first outputs)
    state = 1234567
    out = []
    for _ in range(5):
        state = (state + S.GAMMA) & S.M64
        out.append(S._mix64_int(state))
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]
    # the vectorised form agrees with the scalar one
    base = S.stream_base(7, 3)
    j = np.arange(10, dtype=np.uint64)
    ref = [S._mix64_int(base + (int(i) + 1) * S.GAMMA) for i in j]
    assert S.words(7, 3, j).tolist() == ref


def test_table_is_a_symmetric_normal_quantile_table():
    t = S.table()
    f = S.bf16_to_f32(t).astype(np.float64)
    assert np.all(np.diff(f) >= 0)                          # monotone
    assert np.array_equal(t, t[::-1] ^ np.uint16(0x8000))  # q(1-p) = -q(p)
    assert abs(f.mean()) < 1e-12 and abs(f.std() - 1.0) < 2e-3
    assert abs(f[32768] - 1.9e-5) < 1e-4


def test_fill_is_indexable():
    a = S.fill_host(1000, 11, 5, 0)
    b = S.fill_host(301, 11, 5, 333)
    assert np.array_equal(a[333:634], b)
    assert np.array_equal(S.elements(11, 5, np.arange(333, 634)), b)
    v = S.bf16_to_f32(S.fill_host(200000, 3, 1)).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_recipes():
    c0 = S.CONFIGS["tiny"]
    lens = S.doc_lengths(c0)
    assert lens.size == 64 and lens.min() >= 64 and lens.max() <= 512
    c1 = S.CONFIGS["1m"]
    l1 = S.doc_lengths(c1)
    assert l1.size == 1000 and l1.min() >= 64 and l1.max() <= 8192
    assert 0.85e6 < l1.sum() < 1.15e6
    for name, n_blk in [("10m", 156250), ("100m", 1562500)]:
        c = S.CONFIGS[name]
        off = S.prepooled_doc_blk_offsets(c)
        assert off[-1] == n_blk and np.all(np.diff(off) >= 1)
    nd = S.needle_docs(S.CONFIGS["10m"])
    assert nd.shape == (32, 16) and np.unique(nd).size == 512
    assert np.array_equal(S.needle_docs(S.CONFIGS["interleaved"]), S.needle_docs(S.CONFIGS["100m"]))
    # interleaved query 0 starts with the 100M config's query
    q4 = S.qr_host(S.CONFIGS["interleaved"], 5)
    q3 = S.qr_host(S.CONFIGS["100m"], 5)
    assert q4.shape == (8, 1088, 8, 128) and np.array_equal(q4[0, :64], q3[0])


def test_needle_values_follow_the_definition():
    q = S.fill_host(2 * 1024, 1, S.S_QR).reshape(2, 8, 128)
    rows = np.array([5, 9])
    got = S.needle_rows_host(77, 2, 100, rows, q)
    z = S.bf16_to_f32(S.elements(77, S.S_NEEDLE, ((2 * 100 + rows)[:, None] * 1024 + np.arange(1024)).ravel()))
    ref = S.f32_to_bf16((S.bf16_to_f32(q).ravel() + (np.float32(0.3) * z).astype(np.float32)).astype(np.float32))
    assert np.array_equal(got.ravel(), ref)


def tiny_memory_host(cfg):
    """Per-token K, V, Kr of a per-token config on the host, needles planted."""
    tok = S.doc_tok_offsets(cfg)
    n_tok = int(tok[-1])
    L = cfg.n_layers
    k = S.fill_host(L * n_tok * 1024, cfg.seed, S.S_K).reshape(L, n_tok, 8, 128)
    v = S.fill_host(L * n_tok * 1024, cfg.seed, S.S_V).reshape(L, n_tok, 8, 128)
    kr = S.fill_host(L * n_tok * 1024, cfg.seed, S.S_KR).reshape(L, n_tok, 8, 128)
    rows, qrows = S.needle_row_table(cfg, tok)
    for l in range(L):
        q = S.qr_host(cfg, l).reshape(-1, 8, 128)
        kr[l, rows] = S.needle_rows_host(cfg.seed, l, n_tok, rows, q[qrows])
    return tok, k, v, kr


def test_oracle_ranks_planted_needles_first(orc):
    cfg = S.CONFIGS["tiny"]
    tok, k, v, kr = tiny_memory_host(cfg)
    blk, n_blk, _ = orc.block_offsets(tok)
    krbar = orc.pool(kr, tok, blk)
    q = S.qr_host(cfg, 0)[0]
    Sd = orc.doc_scores(q, krbar[0], blk)
    ids, sc = orc.topk(Sd, cfg.k)
    needles = set(S.needle_docs(cfg)[0].tolist())
    assert set(ids[:2].tolist()) == needles
    assert sc[1] > 0.9 and sc[2] < 0.5                 # needles ~1, noise maxima well below
    assert np.all(np.abs(Sd) <= 1.0)
