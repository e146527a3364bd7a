"""GPU parity of the multi-token sparse prefill against the fp64 oracle: ragged memory
and local lengths, every supported query-head group, tokens that see no row, the
one-token case against the decode, and sampled tokens at the 1,088-token shape of the
interleaved workload's last round."""
import math

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


from gpu_common import DECODE_TOL, SCALE, assert_decode, to_dev_bf16  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402


def rand_bf16(rng, shape):
    return S.f32_to_bf16(rng.standard_normal(shape).astype(np.float32))


def make(rng, L, B, T, Hq, max_ctx, max_loc, ctx_len, loc_len):
    h = {"q": rand_bf16(rng, (L, B, T, Hq, 128)),
         "ck": rand_bf16(rng, (L, B, max_ctx, 8, 128)), "cv": rand_bf16(rng, (L, B, max_ctx, 8, 128)),
         "lk": rand_bf16(rng, (L, B, max_loc, 8, 128)), "lv": rand_bf16(rng, (L, B, max_loc, 8, 128)),
         "cl": np.asarray(ctx_len, np.int32).reshape(L, B), "ll": np.asarray(loc_len, np.int32).reshape(L, B)}
    d = {k: to_dev_bf16(v) for k, v in h.items() if k not in ("cl", "ll")}
    d["cl"] = torch.from_numpy(h["cl"]).to(DEV)
    d["ll"] = torch.from_numpy(h["ll"]).to(DEV)
    return h, d


def run(d, scale=SCALE):
    L, B, T, Hq = d["q"].shape[:4]
    out = torch.full((L, B, T, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    msa.msa_sparse_prefill(d["q"], d["ck"], d["cv"], d["cl"], d["lk"], d["lv"], d["ll"], scale, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_all(h, out, scale=SCALE):
    L, B = h["q"].shape[:2]
    for l in range(L):
        for b in range(B):
            n_ctx, n_loc = int(h["cl"][l, b]), int(h["ll"][l, b])
            ref = O.prefill(h["q"][l, b], h["ck"][l, b, :n_ctx], h["cv"][l, b, :n_ctx],
                            h["lk"][l, b, :n_loc], h["lv"][l, b, :n_loc], scale) if n_loc >= h["q"].shape[2] else None
            if ref is None:   # fewer local rows than tokens: tokens see local rows 0 .. n_loc - T + t
                T = h["q"].shape[2]
                ref = np.stack([O.decode(h["q"][l, b, t], h["ck"][l, b, :n_ctx], h["cv"][l, b, :n_ctx],
                                         h["lk"][l, b, :max(0, n_loc - T + t + 1)],
                                         h["lv"][l, b, :max(0, n_loc - T + t + 1)], scale) for t in range(T)])
            assert np.isfinite(out[l, b]).all()
            assert_decode(out[l, b], ref)


@pytest.mark.parametrize("T,Hq", [(1, 32), (5, 32), (16, 32), (17, 32), (40, 8), (33, 16), (20, 64)])
def test_prefill_ragged(T, Hq):
    """Memory and local lengths differ per (layer, query); T spans partial and several query blocks."""
    print("case: prefill ragged T=%d Hq=%d" % (T, Hq), flush=True)
    rng = np.random.default_rng(1000 + 7 * T + Hq)
    L, B, max_ctx, max_loc = 2, 2, 70, T + 45
    ctx_len = [0, 33, 70, 1]
    loc_len = [T, T + 45, T + 3, T + 31]
    h, d = make(rng, L, B, T, Hq, max_ctx, max_loc, ctx_len, loc_len)
    check_all(h, run(d))


def test_prefill_tokens_without_rows_are_zero():
    """No memory rows and fewer local rows than tokens: the first tokens see nothing."""
    print("case: prefill empty rows", flush=True)
    rng = np.random.default_rng(77)
    T = 8
    h, d = make(rng, 1, 1, T, 32, 4, T, [0], [5])
    out = run(d)
    assert np.all(out[0, 0, :3] == 0.0)
    check_all(h, out)


def test_prefill_one_token_matches_decode():
    print("case: prefill T=1 vs decode", flush=True)
    rng = np.random.default_rng(78)
    L, B, Hq, max_ctx, max_loc = 2, 3, 32, 50, 40
    h, d = make(rng, L, B, 1, Hq, max_ctx, max_loc, [50, 0, 17, 3, 49, 20], [40, 1, 39, 2, 30, 11])
    pre = run(d)[:, :, 0]
    ws = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, max_loc), dtype=torch.uint8, device=DEV)
    dec = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=DEV)
    msa.msa_sparse_decode(d["q"][:, :, 0].contiguous(), d["ck"], d["cv"], d["cl"], d["lk"], d["lv"], d["ll"], SCALE,
                          dec, ws)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    err = np.abs(pre - dec).max(axis=-1)
    assert (err <= DECODE_TOL * np.abs(dec).max(axis=-1)).all()


def test_prefill_interleaved_round_shape_sampled():
    """1,088 query tokens over ~250 memory rows and 1,088 local rows (the interleaved workload's
    last round), checked on sampled tokens, each against the oracle's one-token attention."""
    print("case: prefill 1088 tokens sampled", flush=True)
    rng = np.random.default_rng(79)
    L, B, T, Hq = 2, 2, 1088, 32
    max_ctx, max_loc = 300, 1088
    h, d = make(rng, L, B, T, Hq, max_ctx, max_loc, [250, 300, 0, 197], [1088, 1088, 1088, 1088])
    out = run(d)
    assert np.isfinite(out).all()
    for l in range(L):
        for b in range(B):
            n_ctx = int(h["cl"][l, b])
            for t in (0, 1, 15, 16, 500, 1023, 1087):
                ref = O.decode(h["q"][l, b, t], h["ck"][l, b, :n_ctx], h["cv"][l, b, :n_ctx],
                               h["lk"][l, b, :t + 1], h["lv"][l, b, :t + 1], SCALE)
                assert_decode(out[l, b, t], ref)


def test_prefill_rejects_bad_shapes():
    rng = np.random.default_rng(80)
    h, d = make(rng, 1, 1, 4, 32, 8, 4, [8], [4])
    out = torch.empty((1, 1, 4, 32, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_prefill(d["q"], d["ck"], d["cv"], d["cl"], d["lk"][:, :, :3].contiguous(),
                               d["lv"][:, :, :3].contiguous(), d["ll"], SCALE, out)
    assert e.value.status == msa.MSA_ERR_SHAPE
    assert math.isfinite(SCALE)
