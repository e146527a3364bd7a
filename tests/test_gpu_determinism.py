"""Generator agreement and run-to-run determinism.

The device generator must produce exactly the host generator's values (every input of
every workload is regenerated on the host by the oracle side), and every entry point
must give bitwise-identical results when run twice on the same inputs: the document
maxima are integer atomic maxima, the other reductions have a fixed order, so any
difference would mean a race."""
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


from gpu_common import SCALE, alloc_route_keys, route, to_dev_bf16, u16  # noqa: E402
from routed_kv_memory_amd import msa  # noqa: E402


@pytest.mark.parametrize("stream", [S.S_K, S.S_KRBAR, S.S_QR, S.S_LOC_V, S.S_PF_Q])
def test_device_generator_matches_host(stream):
    """Slices at scattered offsets of a long stream, including unaligned starts."""
    print("case: generator stream %d" % stream, flush=True)
    gen = S.DeviceGen(DEV)
    seed = S.CONFIGS["10m"].seed
    rng = np.random.default_rng(stream)
    for e0 in [0, 1, 3, 4095, 1 << 20, int(rng.integers(0, 1 << 40))]:
        n = 5000 + int(rng.integers(0, 64))
        t = torch.empty(n, dtype=torch.bfloat16, device=DEV)
        gen.fill(t, seed, stream, e0)
        torch.cuda.synchronize()
        assert np.array_equal(u16(t), S.fill_host(n, seed, stream, e0)), e0


def test_every_entry_point_is_deterministic():
    print("case: determinism", flush=True)
    rng = np.random.default_rng(5)
    cfg = S.CONFIGS["tiny"]
    di = DeviceInputs(cfg, DEV)
    tok, k, v, kr = di.per_token()
    blk, n_blk, max_db = msa.msa_block_offsets_host(tok)
    L = cfg.n_layers
    tok_d, blk_d = tok.to(DEV), blk.to(DEV)
    B, T, kk = 5, 130, 4                      # several query chunks: the shared-range scan path
    qr = to_dev_bf16(S.f32_to_bf16(rng.standard_normal((L, B, T, 8, 128)).astype(np.float32)))

    def run_all():
        kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
        vbar = torch.empty_like(kbar)
        krt, krn = alloc_route_keys(L, n_blk)
        msa.msa_pool_blocks(k, v, kr, tok_d, blk_d, n_blk, kbar, vbar, krt, krn)
        ids1, sc1, dsc1 = route(qr[:, :1, :64].contiguous(), krt, krn, n_blk, blk_d, kk)   # streamed path
        ids, sc, dsc = route(qr, krt, krn, n_blk, blk_d, kk)                                 # shared-range path
        max_ctx = kk * max_db
        ck = torch.zeros((L, B, max_ctx, 8, 128), dtype=torch.bfloat16, device=DEV)
        cv = torch.zeros_like(ck)
        cl = torch.empty((L, B), dtype=torch.int32, device=DEV)
        msa.msa_gather_ctx(ids, blk_d, max_db, kbar, vbar, ck, cv, cl)
        Hq, n_loc = 32, 40
        q = to_dev_bf16(S.f32_to_bf16(np.random.default_rng(6).standard_normal((L, B, Hq, 128)).astype(np.float32)))
        lk = to_dev_bf16(S.f32_to_bf16(np.random.default_rng(7).standard_normal((L, B, n_loc, 8, 128))
                                       .astype(np.float32)))
        lv = to_dev_bf16(S.f32_to_bf16(np.random.default_rng(8).standard_normal((L, B, n_loc, 8, 128))
                                       .astype(np.float32)))
        ll = torch.full((L, B), n_loc, dtype=torch.int32, device=DEV)
        ws = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, n_loc), dtype=torch.uint8,
                         device=DEV)
        out = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=DEV)
        msa.msa_sparse_decode(q, ck, cv, cl, lk, lv, ll, SCALE, out, ws)
        qp = torch.cat([lk[:, :, n_loc - 24:]] * (Hq // 8), dim=3).contiguous()
        outp = torch.empty((L, B, 24, Hq, 128), dtype=torch.float32, device=DEV)
        msa.msa_sparse_prefill(qp, ck, cv, cl, lk, lv, ll, SCALE, outp)
        torch.cuda.synchronize()
        return [kbar, vbar, krt, krn, ids1, sc1, dsc1, ids, sc, dsc, ck, cv, cl, out, outp]

    a = run_all()
    b = run_all()
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), i


def test_scan_on_a_cu_masked_stream_matches():
    """A scan launched on a CU-masked stream sizes its persistent grid to that stream's CUs and
    gives exactly the scores of an unmasked launch (single query and shared-range cases)."""
    print("case: scan on a CU-masked stream", flush=True)
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    words = (cus + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for b in range(cus):
        if b % 32 >= 4:                                   # drop 4 of every 32 CUs
            mask[b // 32] |= 1 << (b % 32)
    handle = ctypes.c_void_p()
    assert hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), mask) == 0
    masked = torch.cuda.ExternalStream(handle.value)
    rng = np.random.default_rng(41)
    cfg = S.CONFIGS["tiny"]
    di = DeviceInputs(cfg, DEV)
    tok, k, v, kr = di.per_token()
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    L = cfg.n_layers
    krt, krn = alloc_route_keys(L, n_blk)
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=DEV)
    vbar = torch.empty_like(kbar)
    blk_d = blk.to(DEV)
    msa.msa_pool_blocks(k, v, kr, tok.to(DEV), blk_d, n_blk, kbar, vbar, krt, krn)
    torch.cuda.synchronize()
    for B, T in ((1, 64), (5, 130)):
        qr = to_dev_bf16(S.f32_to_bf16(rng.standard_normal((L, B, T, 8, 128)).astype(np.float32)))
        _, _, d_ref = route(qr, krt, krn, n_blk, blk_d, 4)
        torch.cuda.synchronize()
        with torch.cuda.stream(masked):
            _, _, d_msk = route(qr, krt, krn, n_blk, blk_d, 4)
        torch.cuda.synchronize()
        assert torch.equal(d_ref, d_msk), (B, T)
