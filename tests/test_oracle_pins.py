"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values worked
by hand from the definitions, closed forms, invariants, special cases that
reduce to a library routine, or brute force written differently.  A plausible
mistake (wrong divisor, dropped head, sum instead of mean, wrong GQA index,
double rounding, transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

H, D, ROW = 8, 128, 1024
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    """bf16 bits of float32-representable values (exact, truncation is exact here)."""
    a = np.asarray(x, np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ------------------------------------------------------------------ bf16 RNE

@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),      # just above a tie: no double rounding via float
    (-(1.0 + 2.0 ** -8 + 2.0 ** -30), 0xBF81),
    (2.0 ** -133, 0x0001),                       # smallest subnormal
    (2.0 ** -134, 0x0000),                       # tie with zero -> even
    (3 * 2.0 ** -134, 0x0002),                   # tie -> even (up)
    (3.4e38, 0x7F80),                            # beyond the largest finite bf16
    (131.5, 0x4304),                             # 131.5 -> 132 (tie, even)
    (0.0, 0x0000),
])
def test_bf16_rne_cases(orc, x, bits):
    assert orc.bf16_from_f64_scalar(x) == bits


def test_bf16_rne_matches_library_on_float32_values(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_from_f64(f.astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------------- offset tables (5.3)

def test_group_ids_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "group_ids.json")))
    for case in g["cases"]:
        assert orc.group_ids(case["doc_ids"]).tolist() == case["group_ids"]
        assert orc.doc_tok_offsets(case["doc_ids"]).tolist() == case["doc_tok_off"]


def test_block_offsets_closed_form(orc):
    lens = [64, 65, 128, 1, 0, 129, 8192]
    tok = np.concatenate([[0], np.cumsum(lens)])
    off, n_blk, mx = orc.block_offsets(tok)
    counts = [1, 2, 2, 1, 0, 3, 128]
    assert (off[1:] - off[:-1]).tolist() == counts
    assert n_blk == sum(counts) and mx == 128


def test_page_size_figures(orc):
    """The pages' capacity figures follow from 64:1 blocks x 18 layers x 8 heads x 128 x 2 B."""
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))["figures"]
    # one 100M-token memory at 64:1 (the pages divide the token count by 64)
    _, n_blk, _ = orc.block_offsets([0, 100_000_000])
    row_bytes = 18 * 8 * 128 * 2
    got = {
        "blocks for 100M tokens at 64:1": n_blk,
        "routing keys bytes": n_blk * row_bytes,
        "content K/V bytes": 2 * n_blk * row_bytes,
        "whole compressed cache bytes": 3 * n_blk * row_bytes,
    }
    # Top-16 of ~1000-token documents: ceil(1000/64) blocks each, K and V, all layers
    _, blk16, _ = orc.block_offsets(np.arange(17) * 1000)
    got["content loaded for a Top-16 of ~1000-token documents, all routed layers"] = blk16 * 2 * row_bytes
    for f in g:
        assert abs(got[f["what"]] - f["value"]) <= f["rel_tol"] * f["value"], f


# ------------------------------------------------------------------ pooling

def _pool_one(orc, x_tok, lens):
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    blk, _, _ = orc.block_offsets(tok)
    return orc.pool(x_tok, tok, blk), blk


def test_pool_constant_blocks_return_the_constant(orc):
    lens = [100, 64, 3]                 # full + partial, full, partial
    n = sum(lens)
    x = np.broadcast_to(bf([1.4375]), (1, n, H, D)).copy()   # bf16-exact constant
    out, blk = _pool_one(orc, x, lens)
    assert out.shape == (1, 4, H, D)
    assert np.all(out == bf([1.4375])[0])


def test_pool_one_token_tail_equals_that_token(orc):
    rng = np.random.default_rng(2)
    x = rand_bf16(rng, (1, 65, H, D))
    out, _ = _pool_one(orc, x, [65])
    assert np.array_equal(out[0, 1], x[0, 64])


def test_pool_opposite_pair_is_zero(orc):
    rng = np.random.default_rng(3)
    a = rand_bf16(rng, (1, 1, H, D))
    x = np.concatenate([a, a ^ np.uint16(0x8000)], axis=1)   # {a, -a}
    out, _ = _pool_one(orc, x, [2])
    assert np.all(val(out) == 0.0)


def test_pool_hand_worked_two_docs(orc):
    """Docs of 65 and 64 tokens -> 2 + 1 blocks.  Token value = (position in the
    doc, +100 for doc 1) * sign, sign = +1 on even channels and -1 on odd ones;
    layer 1 holds half of layer 0.  All inputs are bf16-exact integers/halves."""
    lens = [65, 64]
    pos = np.concatenate([np.arange(65), 100 + np.arange(64)]).astype(np.float32)
    sign = np.where(np.arange(ROW) % 2 == 0, 1.0, -1.0).astype(np.float32)
    x = np.stack([bf(pos[:, None] * sign[None, :]), bf(0.5 * pos[:, None] * sign[None, :])])
    out, blk = _pool_one(orc, x.reshape(2, 129, H, D), lens)
    assert blk.tolist() == [0, 2, 3]
    o = val(out).reshape(2, 3, ROW)
    # layer 0: mean(0..63) = 31.5, token 64 alone = 64, mean(100..163) = 131.5 -> bf16 132 (tie, even)
    assert np.array_equal(o[0], np.stack([31.5 * sign, 64.0 * sign, 132.0 * sign]))
    # layer 1: 15.75, 32, 65.75 -> bf16 66 (tie between 65.5 and 66, even)
    assert np.array_equal(o[1], np.stack([15.75 * sign, 32.0 * sign, 66.0 * sign]))


def test_pool_random_matches_library_mean(orc):
    rng = np.random.default_rng(4)
    lens = [1, 63, 64, 65, 200]
    x = rand_bf16(rng, (2, sum(lens), H, D))
    out, blk = _pool_one(orc, x, lens)
    tok = np.concatenate([[0], np.cumsum(lens)])
    xv = val(x)
    for l in range(2):
        bi = 0
        for d in range(len(lens)):
            for s in range(tok[d], tok[d + 1], 64):
                e = min(s + 64, tok[d + 1])
                ref = np.mean(xv[l, s:e], axis=0)
                got = val(out[l, bi])
                # one bf16 rounding of the exact mean: within half an ulp (2^-8 relative)
                assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
                bi += 1
        assert bi == blk[-1]


# ------------------------------------------------------------------- norms

def test_head_norms(orc):
    rows = np.zeros((2, H, D), np.uint16)
    rows[0, 3, 0], rows[0, 3, 5] = bf([3.0])[0], bf([4.0])[0]
    rows[1, 7, 127] = bf([-2.0])[0]
    n = orc.head_norms(rows)
    assert n[0, 3] == 5.0 and n[1, 7] == 2.0 and n[0, 0] == 0.0
    rng = np.random.default_rng(5)
    r = rand_bf16(rng, (50, H, D))
    ref = np.linalg.norm(val(r).reshape(50, H, D), axis=-1)
    assert np.allclose(orc.head_norms(r), ref, rtol=1e-14, atol=0)


# ----------------------------------------------------------------- scoring

def test_score_power_of_two_rescaling_is_exact(orc):
    rng = np.random.default_rng(6)
    T, nb = 3, 7
    q = rand_bf16(rng, (T, H, D))
    k = rand_bf16(rng, (nb, H, D))
    off = np.array([0, 3, 7])
    s0 = orc.doc_scores(q, k, off)
    q2 = bf(val(q).astype(np.float32) * np.float32(2.0))          # exact in bf16
    k2 = bf(val(k).astype(np.float32) * np.float32(0.25))
    assert np.array_equal(orc.doc_scores(q2, k, off), s0)
    assert np.array_equal(orc.doc_scores(q, k2, off), s0)
    # one head of one token rescaled only
    q3 = q.copy()
    q3[1, 4] = bf(val(q[1, 4]).astype(np.float32) * np.float32(8.0))
    for t in range(T):
        for b in range(nb):
            a = orc.block_score(q3[t], k[b])
            c = orc.block_score(q[t], k[b])
            assert a == c


def test_score_equal_opposite_orthogonal(orc):
    rng = np.random.default_rng(7)
    q = rand_bf16(rng, (1, H, D))
    assert abs(orc.block_score(q[0], q[0]) - 1.0) < 1e-15
    assert abs(orc.block_score(q[0], q[0] ^ np.uint16(0x8000)) + 1.0) < 1e-15
    e = np.zeros((2, H, D), np.uint16)
    e[0, :, 0] = bf([1.0])[0]
    e[1, :, 1] = bf([1.0])[0]
    assert orc.block_score(e[0], e[1]) == 0.0


def test_score_is_mean_over_heads(orc):
    rng = np.random.default_rng(8)
    q = rand_bf16(rng, (H, D))
    k = q.copy()
    k[3:] ^= np.uint16(0x8000)            # heads 0-2 aligned (+1), heads 3-7 opposite (-1)
    assert abs(orc.block_score(q, k) - (3 - 5) / 8) < 1e-15


def test_score_zero_vector_scores_zero(orc):
    rng = np.random.default_rng(9)
    k = rand_bf16(rng, (H, D))
    assert orc.block_score(np.zeros((H, D), np.uint16), k) == 0.0


def test_single_head_single_token_is_textbook_cosine(orc):
    scipy_dist = pytest.importorskip("scipy.spatial.distance")
    rng = np.random.default_rng(10)
    for _ in range(20):
        q = np.zeros((1, H, D), np.uint16)
        k = np.zeros((1, H, D), np.uint16)
        q[0, 0] = rand_bf16(rng, D)
        k[0, 0] = rand_bf16(rng, D)
        s = orc.doc_scores(q, k, np.array([0, 1]))[0]
        ref = 1.0 - scipy_dist.cosine(val(q[0, 0]), val(k[0, 0]))
        assert abs(8.0 * s - ref) < 1e-13          # other heads are zero vectors -> cos 0


def test_doc_score_is_max_over_tokens_and_blocks(orc):
    rng = np.random.default_rng(11)
    T = 4
    q = rand_bf16(rng, (T, H, D))
    k = rand_bf16(rng, (5, H, D))
    k[3] = q[2]                                     # doc 1 block 1 equals token 2 -> 1.0
    off = np.array([0, 2, 5])
    S = orc.doc_scores(q, k, off)
    assert abs(S[1] - 1.0) < 1e-15
    brute0 = max(orc.block_score(q[t], k[b]) for t in range(T) for b in range(0, 2))
    assert S[0] == brute0
    assert np.all(np.abs(S) <= 1.0 + 1e-15)


def test_appending_query_rows_never_lowers_scores(orc):
    rng = np.random.default_rng(12)
    q = rand_bf16(rng, (6, H, D))
    k = rand_bf16(rng, (30, H, D))
    off = np.array([0, 4, 4, 11, 30])               # doc 1 is empty
    s_small = orc.doc_scores(q[:2], k, off)
    s_big = orc.doc_scores(q, k, off)
    assert np.all(s_big[[0, 2, 3]] >= s_small[[0, 2, 3]])
    assert s_big[1] == -math.inf and s_small[1] == -math.inf
    # exact max-merge: S over all rows = max(S over first rows, S over the rest)
    assert np.array_equal(s_big[[0, 2, 3]],
                          np.maximum(s_small, orc.doc_scores(q[2:], k, off))[[0, 2, 3]])


@pytest.mark.parametrize("threads", [1, 2, 3, 7, 64])
def test_threaded_doc_scores_equal_single_threaded(orc, threads):
    # ragged documents, empty ones at both ends and in the middle, more threads than documents
    rng = np.random.default_rng(13)
    counts = np.array([0, 3, 1, 0, 0, 17, 2, 9, 1, 1, 0, 40, 5, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    q = rand_bf16(rng, (5, H, D))
    k = rand_bf16(rng, (int(off[-1]), H, D))
    ref = orc.doc_scores(q, k, off)
    got = orc.doc_scores_mt(q, k, off, threads=threads)
    assert np.array_equal(got, ref)                 # bit-identical, -inf for empty documents
    got = orc.doc_scores_mt(q, k, off, threads=threads, chunks=4, progress=lambda i, n: None)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("threads", [1, 4, 9])
def test_threaded_pool_equals_single_threaded(orc, threads):
    rng = np.random.default_rng(14)
    lens = np.array([65, 0, 1, 130, 64, 7, 200])
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    blk, _, _ = orc.block_offsets(tok)
    x = rand_bf16(rng, (2, int(tok[-1]), H, D))
    assert np.array_equal(orc.pool_mt(x, tok, blk, threads=threads), orc.pool(x, tok, blk))


# -------------------------------------------------------------------- top-k

def _selection_topk(S, k):
    """Different formulation: repeated selection of the best remaining (score, then id)."""
    left = list(range(len(S)))
    out = []
    for _ in range(k):
        best = left[0]
        for d in left[1:]:
            if S[d] > S[best]:
                best = d
        out.append(best)
        left.remove(best)
    return out


def test_topk_brute_force_ties_and_empty(orc):
    rng = np.random.default_rng(13)
    for n, k in [(10, 3), (50, 16), (17, 17)]:
        S = np.round(rng.standard_normal(n), 1)    # many ties
        S[rng.integers(0, n, 2)] = -math.inf
        ids, sc = orc.topk(S, k)
        assert ids.tolist() == _selection_topk(S, k)
        assert np.array_equal(sc, S[ids])
    ids, _ = orc.topk(np.array([1.0, 2.0, 2.0, 0.0]), 2)
    assert ids.tolist() == [1, 2]
    ids, _ = orc.topk(np.array([-math.inf, 0.5, -math.inf]), 3)
    assert ids.tolist() == [1, 0, 2]


def test_topk_permutation_equivariance(orc):
    rng = np.random.default_rng(14)
    S = rng.standard_normal(40)
    perm = rng.permutation(40)
    ids, _ = orc.topk(S, 8)
    ids_p, _ = orc.topk(S[perm], 8)
    assert perm[ids_p].tolist() == ids.tolist()


# ------------------------------------------------------------------- gather

def test_gather_is_concatenation(orc):
    rng = np.random.default_rng(15)
    off = np.array([0, 3, 3, 7, 8, 12])
    kb = rand_bf16(rng, (12, H, D))
    vb = rand_bf16(rng, (12, H, D))
    ids = np.array([3, 0, 1, 4])
    ck, cv = orc.gather(ids, off, kb, vb)
    ref_k = np.concatenate([kb[off[i]:off[i + 1]] for i in ids])
    ref_v = np.concatenate([vb[off[i]:off[i + 1]] for i in ids])
    assert np.array_equal(ck, ref_k) and np.array_equal(cv, ref_v)
    assert ck.shape[0] == 1 + 3 + 0 + 4


# ------------------------------------------------------------------- decode

def test_decode_single_key_returns_its_value(orc):
    rng = np.random.default_rng(16)
    q = rand_bf16(rng, (32, D))
    k = rand_bf16(rng, (1, H, D))
    v = rand_bf16(rng, (1, H, D))
    out = orc.decode(q, k, v, np.zeros((0, H, D), np.uint16), np.zeros((0, H, D), np.uint16),
                     1 / math.sqrt(128))
    for hq in range(32):
        assert np.array_equal(out[hq], val(v[0, hq // 4]))


def test_decode_equal_keys_or_zero_query_give_mean_value(orc):
    rng = np.random.default_rng(17)
    n = 5
    k = np.broadcast_to(rand_bf16(rng, (1, H, D)), (n, H, D)).copy()
    v = rand_bf16(rng, (n, H, D))
    q = rand_bf16(rng, (32, D))
    mean_v = val(v).mean(axis=0)
    out = orc.decode(q, k[:2], v[:2], k[2:], v[2:], 0.088)
    for hq in range(32):
        assert np.allclose(out[hq], mean_v[hq // 4], rtol=0, atol=1e-14)
    k2 = rand_bf16(rng, (n, H, D))
    out0 = orc.decode(np.zeros((32, D), np.uint16), k2, v, k2[:0], v[:0], 0.088)
    for hq in range(32):
        assert np.allclose(out0[hq], mean_v[hq // 4], rtol=0, atol=1e-14)


def test_decode_matches_library_softmax_and_gqa_mapping(orc):
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(18)
    n_ctx, n_loc = 9, 4
    q = rand_bf16(rng, (32, D))
    ck, cv = rand_bf16(rng, (n_ctx, H, D)), rand_bf16(rng, (n_ctx, H, D))
    lk, lv = rand_bf16(rng, (n_loc, H, D)), rand_bf16(rng, (n_loc, H, D))
    scale = 1 / math.sqrt(128)
    out = orc.decode(q, ck, cv, lk, lv, scale)
    K = np.concatenate([val(ck), val(lk)])
    V = np.concatenate([val(cv), val(lv)])
    for hq in range(32):
        g = hq // 4
        w = special.softmax(scale * (K[:, g, :] @ val(q[hq])))
        assert np.allclose(out[hq], w @ V[:, g, :], rtol=1e-12, atol=1e-13)
    # rows are a set: permutation and a different ctx/local split leave the output unchanged
    perm = rng.permutation(n_ctx + n_loc)
    Kb = np.concatenate([ck, lk])[perm]
    Vb = np.concatenate([cv, lv])[perm]
    out2 = orc.decode(q, Kb[:3], Vb[:3], Kb[3:], Vb[3:], scale)
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-13)


def test_decode_gqa_groups_are_contiguous(orc):
    """Query head hq reads KV head hq // 4: make only KV head 1 carry a value."""
    rng = np.random.default_rng(19)
    k = rand_bf16(rng, (3, H, D))
    v = np.zeros((3, H, D), np.uint16)
    v[:, 1, :] = bf([7.0])[0]
    out = orc.decode(rand_bf16(rng, (32, D)), k, v, k[:0], v[:0], 0.1)
    assert np.allclose(out[4:8], 7.0, rtol=1e-14, atol=0)
    assert np.all(out[:4] == 0.0) and np.all(out[8:] == 0.0)


def test_decode_no_rows_is_zero(orc):
    e = np.zeros((0, H, D), np.uint16)
    out = orc.decode(np.ones((32, D), np.uint16), e, e, e, e, 0.1)
    assert np.all(out == 0.0)


# ------------------------------------------------------------------- prefill

def _prefill_inputs(rng, T, n_ctx, n_loc, Hq=32):
    q = rand_bf16(rng, (T, Hq, D))
    ck, cv = rand_bf16(rng, (n_ctx, H, D)), rand_bf16(rng, (n_ctx, H, D))
    lk, lv = rand_bf16(rng, (n_loc, H, D)), rand_bf16(rng, (n_loc, H, D))
    return q, ck, cv, lk, lv


def test_prefill_matches_library_masked_attention(orc):
    """torch's scaled_dot_product_attention in float64 with an explicit boolean mask: memory rows
    always visible, local row j visible to token t iff j <= n_loc - T + t; GQA by repeating KV heads."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40)
    T, n_ctx, n_loc, Hq = 6, 7, 9, 16
    q, ck, cv, lk, lv = _prefill_inputs(rng, T, n_ctx, n_loc, Hq)
    scale = 1 / math.sqrt(128)
    out = orc.prefill(q, ck, cv, lk, lv, scale)
    K = torch.from_numpy(np.concatenate([val(ck), val(lk)]))          # [n, 8, 128]
    V = torch.from_numpy(np.concatenate([val(cv), val(lv)]))
    G = Hq // H
    Kq = K.permute(1, 0, 2).repeat_interleave(G, dim=0)                # [Hq, n, 128]
    Vq = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
    Q = torch.from_numpy(val(q)).permute(1, 0, 2)                      # [Hq, T, 128]
    j = torch.arange(n_ctx + n_loc)
    t = torch.arange(T)[:, None]
    mask = (j[None, :] < n_ctx) | (j[None, :] - n_ctx <= n_loc - T + t)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kq, Vq, attn_mask=mask, scale=scale)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_with_one_token_is_decode_and_last_token_sees_everything(orc):
    rng = np.random.default_rng(41)
    q, ck, cv, lk, lv = _prefill_inputs(rng, 5, 4, 8)
    scale = 0.09
    out = orc.prefill(q, ck, cv, lk, lv, scale)
    assert np.array_equal(out[4], orc.decode(q[4], ck, cv, lk, lv, scale))
    assert np.array_equal(orc.prefill(q[:1], ck, cv, lk, lv, scale)[0], orc.decode(q[0], ck, cv, lk, lv, scale))


def test_prefill_is_causal_in_the_local_rows(orc):
    """Changing local row r changes exactly the tokens that may see it."""
    rng = np.random.default_rng(42)
    T, n_ctx, n_loc = 6, 3, 10
    q, ck, cv, lk, lv = _prefill_inputs(rng, T, n_ctx, n_loc)
    base = orc.prefill(q, ck, cv, lk, lv, 0.1)
    for r in (0, 4, 5, 9):
        lk2, lv2 = lk.copy(), lv.copy()
        lk2[r] = rand_bf16(rng, (H, D))
        lv2[r] = rand_bf16(rng, (H, D))
        out = orc.prefill(q, ck, cv, lk2, lv2, 0.1)
        for t in range(T):
            sees = r <= n_loc - T + t
            assert np.array_equal(out[t], base[t]) != sees, (r, t)


def test_prefill_first_token_of_a_bare_query_sees_one_row(orc):
    """No memory rows and local = the query itself: token 0 attends to local row 0 alone."""
    rng = np.random.default_rng(43)
    T = 4
    q, ck, cv, lk, lv = _prefill_inputs(rng, T, 0, T)
    out = orc.prefill(q, ck, cv, lk, lv, 0.1)
    for hq in range(32):
        assert np.array_equal(out[0, hq], val(lv[0, hq // 4]))


# -------------------------------------------------------------------- encode

def _eye_bf16(n):
    w = np.zeros((n, ROW), np.uint16)
    w[np.arange(n), np.arange(n)] = bf([1.0])[0]
    return w


def _offsets(lens):
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    blk = np.concatenate([[0], np.cumsum((np.asarray(lens) + 63) // 64)]).astype(np.int64)
    return tok, blk


def test_encode_identity_projection_is_the_block_pooling(orc):
    """With W_v = W_kr = I (H = 1024) the encode pools the hidden rows themselves."""
    rng = np.random.default_rng(50)
    lens = [1, 64, 65, 130, 7]
    tok, blk = _offsets(lens)
    x = rand_bf16(rng, (int(tok[-1]), ROW))
    eye = _eye_bf16(ROW)
    _, vbar, krbar = orc.encode(x, eye, eye, eye, np.full(D, bf([1.0])[0], np.uint16), 1e-6, 1e6, tok, blk)
    ref = orc.pool(x.reshape(1, -1, H, D), tok, blk)[0]
    assert np.array_equal(vbar, ref) and np.array_equal(krbar, ref)


def test_encode_projection_matches_library_matmul(orc):
    """Single-token documents: each pooled V / Kr row is bf16(x W) of numpy's fp64 matmul."""
    rng = np.random.default_rng(51)
    Hd, n = 96, 12
    x = rand_bf16(rng, (n, Hd))
    wk, wv, wr = (rand_bf16(rng, (Hd, ROW), 0.1) for _ in range(3))
    tok, blk = _offsets([1] * n)
    _, vbar, krbar = orc.encode(x, wk, wv, wr, np.full(D, bf([1.0])[0], np.uint16), 1e-6, 1e6, tok, blk)
    for w, got in ((wv, vbar), (wr, krbar)):
        ref = orc.bf16_from_f64(val(x) @ val(w)).reshape(n, H, D)
        d = np.abs(ref.astype(np.int32) - got.astype(np.int32))
        assert d.max() <= 1 and (d > 0).mean() < 0.01       # fp64 summation order only


def test_encode_key_is_rms_normalised_per_head(orc):
    """Position 0 (no rotation) and unit norm weight: every head of every key has RMS 1."""
    rng = np.random.default_rng(52)
    Hd, n = 64, 10
    x = rand_bf16(rng, (n, Hd))
    wk = rand_bf16(rng, (Hd, ROW), 0.3)
    tok, blk = _offsets([1] * n)
    kbar, _, _ = orc.encode(x, wk, wk, wk, np.full(D, bf([1.0])[0], np.uint16), 1e-12, 1e6, tok, blk)
    rms = np.sqrt((val(kbar) ** 2).mean(axis=-1))
    assert np.allclose(rms, 1.0, atol=2.0 ** -8)
    raw = (val(x) @ val(wk)).reshape(n, H, D)
    ref = orc.bf16_from_f64(raw / np.sqrt((raw ** 2).mean(axis=-1, keepdims=True) + 1e-12))
    assert np.abs(ref.astype(np.int32) - kbar.astype(np.int32)).max() <= 1


def test_encode_rotation_angle_and_pair_norm_at_position_64(orc):
    """The same hidden row at position 64 (the lone token of a 65-token document's second
    block) and at position 0 (a 1-token document): every pair (e, e + 64) of every head keeps
    its length and turns by 64 * theta^(-e/64)."""
    rng = np.random.default_rng(53)
    Hd, theta = 64, 10000.0
    xr = rand_bf16(rng, (1, Hd))
    x = np.concatenate([rand_bf16(rng, (64, Hd)), xr, xr])
    wk = rand_bf16(rng, (Hd, ROW), 0.3)
    tok, blk = _offsets([65, 1])
    kbar, _, _ = orc.encode(x, wk, wk, wk, np.full(D, bf([1.0])[0], np.uint16), 1e-6, theta, tok, blk)
    a, b = val(kbar[1]), val(kbar[2])          # position 64 / position 0
    for h in range(H):
        for e in range(D // 2):
            ra, rb = np.hypot(a[h, e], a[h, e + 64]), np.hypot(b[h, e], b[h, e + 64])
            assert abs(ra - rb) <= 2.0 ** -7 * max(rb, 1e-3) + 2.0 ** -10
            if rb > 0.2:
                turn = math.atan2(a[h, e + 64], a[h, e]) - math.atan2(b[h, e + 64], b[h, e])
                want = 64.0 * theta ** (-e / 64.0)
                err = (turn - want + math.pi) % (2 * math.pi) - math.pi
                assert abs(err) < 0.03, (h, e, err)


def test_encode_documents_are_position_independent_and_norm_weight_scales_keys(orc):
    """Positions restart in every document: swapping two documents swaps their pooled rows
    exactly; a norm weight of 2 doubles the keys exactly and leaves V and Kr alone."""
    rng = np.random.default_rng(54)
    Hd = 64
    la, lb = 70, 130
    xa, xb = rand_bf16(rng, (la, Hd)), rand_bf16(rng, (lb, Hd))
    wk, wv, wr = (rand_bf16(rng, (Hd, ROW), 0.2) for _ in range(3))
    one = np.full(D, bf([1.0])[0], np.uint16)
    tok, blk = _offsets([la, lb])
    ab = orc.encode(np.concatenate([xa, xb]), wk, wv, wr, one, 1e-6, 1e6, tok, blk)
    tok2, blk2 = _offsets([lb, la])
    ba = orc.encode(np.concatenate([xb, xa]), wk, wv, wr, one, 1e-6, 1e6, tok2, blk2)
    na = (la + 63) // 64
    for u, w in zip(ab, ba):
        assert np.array_equal(u[:na], w[-na:]) and np.array_equal(u[na:], w[:-na])
    two = orc.encode(np.concatenate([xa, xb]), wk, wv, wr, np.full(D, bf([2.0])[0], np.uint16), 1e-6, 1e6,
                     tok, blk)
    assert np.array_equal(val(two[0]), 2.0 * val(ab[0]))
    assert np.array_equal(two[1], ab[1]) and np.array_equal(two[2], ab[2])
