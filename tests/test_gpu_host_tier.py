"""Host tier: the content K-bar/V-bar kept in pinned host memory and gathered over the
host link must give exactly the device-memory gather (and the oracle's)."""
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


from gpu_common import to_dev_bf16, u16  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402


def test_gather_from_pinned_host_memory_matches_device():
    print("case: host-tier gather", flush=True)
    rng = np.random.default_rng(90)
    L, B, k, n_docs = 3, 2, 5, 40
    counts = rng.integers(0, 9, n_docs)
    counts[7] = 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    n_blk, max_db = int(off[-1]), int(counts.max())
    kb = S.f32_to_bf16(rng.standard_normal((L, n_blk, 8, 128)).astype(np.float32))
    vb = S.f32_to_bf16(rng.standard_normal((L, n_blk, 8, 128)).astype(np.float32))
    ids = rng.integers(0, n_docs, (L, B, k)).astype(np.int32)
    ids[0, 0, 1] = 7         # an empty document
    ids[1, 1, 0] = -1        # an invalid id contributes nothing
    kd, vd = to_dev_bf16(kb), to_dev_bf16(vb)
    kh = torch.from_numpy(kb.view(np.int16)).pin_memory()
    vh = torch.from_numpy(vb.view(np.int16)).pin_memory()
    assert kh.is_pinned() and vh.is_pinned()
    ids_d, off_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(off).to(DEV)
    max_ctx = k * max_db
    outs = []
    for kk, vv in ((kd, vd), (kh, vh)):
        ck = torch.full((L, B, max_ctx, 8, 128), -1, dtype=torch.int16, device=DEV)
        cv = torch.full_like(ck, -1)
        cl = torch.empty((L, B), dtype=torch.int32, device=DEV)
        msa.msa_gather_ctx(ids_d, off_d, max_db, kk, vv, ck, cv, cl)
        torch.cuda.synchronize()
        outs.append((ck.cpu(), cv.cpu(), cl.cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    # and the oracle, on every (layer, query)
    ck, cv, cl = outs[1]
    for l in range(L):
        for b in range(B):
            sel = ids[l, b][(ids[l, b] >= 0) & (ids[l, b] < n_docs)]
            rk, rv = O.gather(sel, off, kb[l], vb[l])
            n = int(cl[l, b])
            assert n == rk.shape[0]
            assert np.array_equal(u16(ck[l, b, :n]), rk) and np.array_equal(u16(cv[l, b, :n]), rv)
