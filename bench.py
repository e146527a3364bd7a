#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

Default workload: the 100M-token memory (18 routed layers x 1,562,500 pooled
blocks x 8 heads x 128 dims, 100,000 documents, K-bar/V-bar and routing keys all
HBM-resident), one 64-token query, Top-16 per layer, then gather and a GQA
32/8 decode token over [memory context ; 4,096 local rows].

One step = one pass of the whole path over that input: routing scan (all 18
layers, one launch) -> top-k -> context gather -> sparse decode.  Memories that
arrive per token (--workload tiny / 1m) also pool inside the step.  Inputs are
generated on the GPU before timing.  Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routing scan GB/s (% HBM peak) + ms/query, 18 layers, 100M-token memory"
# What each per-workload line reports (the 100M-token line carries the headline metric).
WORKLOAD_METRICS = {
    "100m": (METRIC, "GB/s", True),
    "10m": ("routing scan TFLOP/s (% of bf16 MFMA peak) over whole steps, 18 layers, 10M-token memory, "
            "32 queries x 64 tokens", "TFLOP/s", True),
    "1m": ("tokens/s through the whole path (pool, route, top-k, gather, decode), 18 layers, "
           "1M-token memory", "tokens/s", True),
    "tiny": ("ms per step of the whole path (pool, route, top-k, gather, decode), tiny workload: 1 layer, "
             "64 documents", "ms", False),
}
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0             # dense bf16 matrix-core peak
SCAN_BYTES_PER_BLOCK_LAYER = 2048         # bf16 Kr-bar row (8 x 128): key norms are computed in-kernel
SCAN_BYTES_PER_BLOCK = 4                   # int32 block -> document map entry, needed once per launch
SCAN_BYTES_PER_DOC_LAYER = 4               # fp32 document score written per (layer, query)
DECODE_BYTES_PER_ROW = 2 * 8 * 128 * 2    # K and V row of all 8 KV heads
POOL_BYTES_PER_TOKEN = 3 * 1024 * 2       # K, V, Kr rows read

# HBM traffic of one route-scan launch at the 100M-token workload, from the FETCH_SIZE and
# WRITE_SIZE rocprofv3 passes (scaled by a 1 GiB calibration kernel) recorded in
# profiles/route_scan_100m.md.  It describes the kernel source it was measured on only: if the
# sources' digest differs, the figure is stale and bench.py reports null.
SCAN_TRAFFIC_BYTES = 57.794e9
SCAN_TRAFFIC_SOURCE_DIGEST = "e330cd7932c352eeecce0daa7e8edeced52e593ed5a80d76be5414330cc46d7c"


# HBM traffic of one pooling launch over the 1M-token set (18 layers x 947,395 tokens), FETCH_SIZE
# + WRITE_SIZE passes scaled by the 1 GiB calibration copy, recorded in profiles/pool_1m_tokens.md;
# valid for the kernel source it was measured on only (null otherwise).
POOL_TRAFFIC_BYTES = 106.53e9
POOL_TRAFFIC_SOURCE_DIGEST = "42db7ac2fdcbc30c564bb556aac3d7e8f15abe76b428b5049b39791270a20d0c"


# HBM traffic of one encode launch (18 layers, 1M-token document set), FETCH_SIZE + WRITE_SIZE
# passes scaled by the 1 GiB calibration copy, recorded in profiles/encode_1m_tokens.md; valid for
# the kernel source it was measured on only.
ENCODE_TRAFFIC_BYTES = 543.1e9
ENCODE_TRAFFIC_SOURCE_DIGEST = "79853e71207fa062f195069d8f42ae3fea6aea386678cc1d009d7578b15fa291"


def source_digest(files=("route.hip", "msa_device.hpp")):
    import hashlib
    csrc = os.path.join(ROOT, "routed_kv_memory_amd", "csrc")
    parts = [hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest() for f in files]
    return hashlib.sha256("".join(parts).encode()).hexdigest()


def scan_source_digest():
    return source_digest()


def calibration_copy(dev="cuda"):
    """Kernels of known traffic for scaling hardware byte counters: a 1 GiB fill, then a
    1 GiB elementwise copy (reads 1 GiB, writes 1 GiB)."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(7)
    torch.cuda.synchronize()
    torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    del src, dst
    return 1 << 30


_CONTIGUOUS = []     # (pointer, bytes) of the key memory allocated by route_key_memory


def route_key_memory(shape, dtype):
    """Device memory for a resident memory bank's routing keys (or their norms): one physically
    contiguous allocation (hipExtMallocWithFlags, hipDeviceMallocContiguous), wrapped as a tensor
    and kept until the process ends.  The scan over the 100M-token memory ran ~4% faster from such
    an allocation than from the caching allocator's, with the same steady rate in every process.
    Falls back to torch.empty (returned with False) if the runtime refuses."""
    import ctypes

    import torch
    itemsize = torch.empty((), dtype=dtype).element_size()
    nbytes = itemsize
    for d in shape:
        nbytes *= d
    hip = ctypes.CDLL("libamdhip64.so")
    ptr = ctypes.c_void_p()
    if nbytes == 0 or hip.hipExtMallocWithFlags(ctypes.byref(ptr), ctypes.c_size_t(nbytes), ctypes.c_uint(0x4)) != 0:
        hip.hipGetLastError()
        return torch.empty(shape, dtype=dtype, device="cuda"), False
    _CONTIGUOUS.append((ptr.value, nbytes))
    typestr = {1: "|u1", 2: "<i2", 4: "<i4", 8: "<i8"}[itemsize]

    class _Mem:
        __cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (ptr.value, False),
                                    "version": 2, "strides": None}
    return torch.as_tensor(_Mem(), device="cuda").view(dtype), True


def warm_up(step, args):
    """Untimed warm-up: exactly --warmup steps if given, else at least 3 steps and at least
    --warmup-seconds of them.  Sets args.warmup to the count run (reported in the JSON line)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        if args.warmup is not None and n >= args.warmup:
            break
        if args.warmup is None and n >= 3:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= args.warmup_seconds:
                break
        step()
        n += 1
    torch.cuda.synchronize()
    args.warmup = n
    return n


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3 and at least --warmup-seconds of them)")
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="with no --warmup: keep warming up this long; the scan ran up to 7%% slower in a "
                         "process's first second of sustained load than afterwards")
    ap.add_argument("--workload", default="100m", choices=["tiny", "1m", "10m", "100m", "prefill", "interleaved", "host-tier", "encode"],
                    help="prefill: the multi-token sparse prefill alone at the interleaved workload's last "
                         "round (18 layers x 8 queries x 1,088 tokens); encode: the offline encode front-end "
                         "over the 1M-token document set (18 layers, hidden 2,560); both reported against the "
                         "bf16 MFMA peak")
    ap.add_argument("--host-groups", type=int, default=6,
                    help="host-tier: layer groups whose top-k and host gather overlap the next group's scan")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the second timing of the step as one replayed HIP graph (path workloads)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a 1 GiB fill and a 1 GiB elementwise copy (kernels of known traffic, "
                         "used to scale hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X here; "
              "sharding over several GPUs is a design note, not built (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from routed_kv_memory_amd import msa
    from synth import synth as S
    from synth.device import DeviceInputs

    msa.lib()
    torch.cuda.set_device(int(os.environ.get("LOCAL_RANK", "0")))
    dev = "cuda"
    if args.workload == "prefill":
        return prefill_bench(args)
    if args.workload == "interleaved":
        return interleaved_bench(args)
    if args.workload == "host-tier":
        return host_tier_bench(args)
    if args.workload == "encode":
        return encode_bench(args)
    cfg = S.CONFIGS[args.workload]
    L, B, T, k, Hq = cfg.n_layers, cfg.B, cfg.T, cfg.k, cfg.Hq
    t_setup = time.time()
    di = DeviceInputs(cfg, dev)

    # ---------------------------------------------------------------- memory (outside timing)
    pool_args = None
    if cfg.per_token:
        tok, kt_, vt_, krt_ = di.per_token()
        blk, n_blk, max_db = msa.msa_block_offsets_host(tok)
        tok_d = tok.to(dev)
        n_tok = int(tok[-1])
    else:
        blk = di.prepooled_offsets()
        n_blk = int(blk[-1])
        max_db = int((blk[1:] - blk[:-1]).max())
    n_docs = blk.numel() - 1
    blk_d = blk.to(dev)
    tiles = msa.msa_route_tiles(n_blk)
    krt, contiguous = route_key_memory((L, tiles * 16, 8, 128), torch.bfloat16)
    krn, _ = route_key_memory((L, tiles * 16, 8), torch.float32)
    if cfg.per_token:
        kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device=dev)
        vbar = torch.empty_like(kbar)
        pool_args = (kt_, vt_, krt_, tok_d, blk_d, n_blk, kbar, vbar, krt, krn)
    else:
        kbar, vbar = di.prepooled_content()
        for l, rows in di.prepooled_route_rows():
            msa.msa_pack_route_keys(rows.view(1, n_blk, 8, 128), n_blk, krt[l:l + 1], krn[l:l + 1])
    blk_doc = torch.empty(tiles * 16, dtype=torch.int32, device=dev)
    msa.msa_block_doc_map(blk_d, n_blk, blk_doc)
    qr = di.qr()
    q, lk, lv, ll = di.decode_inputs()
    max_ctx = k * max_db
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=dev)
    ids = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    tsc = torch.empty((L, B, k), dtype=torch.float32, device=dev)
    ws_topk = torch.empty(max(msa.msa_topk_docs_workspace_size(L, B, n_docs, k), 256), dtype=torch.uint8, device=dev)
    ck = torch.empty((L, B, max_ctx, 8, 128), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    cl = torch.empty((L, B), dtype=torch.int32, device=dev)
    out = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=dev)
    ws_dec = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, cfg.L_loc), dtype=torch.uint8,
                         device=dev)
    scale = 1.0 / math.sqrt(128.0)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    print("bench: %s memory ready in %.1f s (%d blocks x %d layers, %d docs, %.1f GB on device)"
          % (cfg.name, t_setup, n_blk, L, n_docs, torch.cuda.memory_allocated() / 1e9), file=sys.stderr, flush=True)

    # The scan reads the key norms when several query chunks make it bound by the matrix
    # cores; one chunk (bound by HBM) recomputes them from the keys it streams.
    scan_norms = krn if B * ((T + 63) // 64) > 1 else None
    n_ev = 6
    def step(evs=None):
        rec = (lambda i: evs[i].record()) if evs is not None else (lambda i: None)
        rec(0)
        if pool_args is not None:
            msa.msa_pool_blocks(*pool_args)
        rec(1)
        msa.msa_route_scores(qr, krt, n_blk, blk_doc, n_docs, dsc, krbar_norm=scan_norms)
        rec(2)
        msa.msa_topk_docs(dsc, k, ids, tsc, ws_topk)
        rec(3)
        msa.msa_gather_ctx(ids, blk_d, max_db, kbar, vbar, ck, cv, cl)
        rec(4)
        msa.msa_sparse_decode(q, ck, cv, cl, lk, lv, ll, scale, out, ws_dec)
        rec(5)

    warm_up(step, args)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(n_ev - 1)]
                    for i in range(args.steps)])            # ms
    seg_mean = seg.mean(axis=0)
    ms_step = wall * 1e3 / args.steps

    # The same step recorded once in a HIP graph and replayed K times: the launches' gaps are
    # what differs.  Reported beside the eager step (value is computed from the eager step).
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # sanity of the result (cheap, outside the timed region): planted needles are the top-k
    nd = S.needle_docs(cfg)
    ids_h = ids.cpu().numpy()
    needle_ok = all(set(ids_h[l, b].tolist()) == set(nd[b].tolist())
                    for l in range(L) for b in range(nd.shape[0])) if cfg.needles == k else None

    scan_bytes = (L * n_blk * SCAN_BYTES_PER_BLOCK_LAYER + n_blk * SCAN_BYTES_PER_BLOCK
                  + L * B * n_docs * SCAN_BYTES_PER_DOC_LAYER)
    value = scan_bytes * args.steps / wall / 1e9                       # GB/s over whole steps
    scan_ms = float(seg_mean[1])
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    # The scan does 2*B*T*1024 flop per 2,048-byte key row: below the ridge (peak flop/s over
    # peak B/s, ~312 flop/B) it is bound by HBM, above it by the matrix cores.
    scan_flop = 2.0 * B * T * 1024 * L * n_blk
    n_chunks = B * ((T + 63) // 64)
    nt = min(4, (T + 15) // 16)
    norms_s = "true" if scan_norms is not None else "false"
    if T < 16:
        scan_kernel = "route_valu_kernel (msa_route_scores)"
    elif n_chunks == 1:
        scan_kernel = "route_mfma_kernel<%d, true, %s> (msa_route_scores)" % (nt, norms_s)
    else:   # several query chunks: two per workgroup, one head per wave
        scan_kernel = "route_heads_kernel<%d, %s, 2> (msa_route_scores)" % (nt, norms_s)
    if scan_flop / scan_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        tflops = scan_flop / (scan_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": scan_kernel,
                    "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "algorithmic_flop_per_launch": scan_flop, "hbm_GBps": round(achieved, 2)}
    else:
        roofline = {"bound": "hbm", "kernel": scan_kernel,
                    "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": (round(SCAN_TRAFFIC_BYTES / 1e9, 3)
                                if cfg.name == "100m" and scan_source_digest() == SCAN_TRAFFIC_SOURCE_DIGEST
                                else None),
                    "traffic_unit": "GB per launch", "algorithmic_GB_per_launch": round(scan_bytes / 1e9, 3)}
    ctx_rows = int(cl.sum().item())
    dec_rows = ctx_rows + int(ll.sum().item())
    metric, unit, higher = WORKLOAD_METRICS[cfg.name]
    if cfg.name == "10m":
        value = scan_flop * args.steps / wall / 1e12                 # TFLOP/s over whole steps
    elif cfg.name == "1m":
        value = L * n_tok * args.steps / wall                       # tokens/s through the path
    elif cfg.name == "tiny":
        value = ms_step
    result = {
        "metric": metric,
        "value": round(value, 4 if unit == "ms" else 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms is not None else None,
        "higher_is_better": higher,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "layers": L, "blocks_per_layer": n_blk, "docs": n_docs, "queries": B, "query_tokens": T,
            "top_k": k, "kv_heads": 8, "head_dim": 128, "q_heads": Hq, "local_rows": cfg.L_loc,
            "route_key_bytes": L * tiles * 16 * 2048, "content_kv_bytes": 2 * L * n_blk * 2048,
            "route_key_alloc": "one contiguous device allocation" if contiguous else "caching allocator",
            "scan_key_norms": "read" if scan_norms is not None else "recomputed from the keys",
        },
        "scan_GBps_over_whole_steps": round(scan_bytes * args.steps / wall / 1e9, 2),
        "hbm_frac_of_peak": round(scan_bytes * args.steps / wall / 1e9 / HBM_PEAK_GBPS, 4),
        "ms_per_query_18_layers": round(ms_step / B, 4),
        "ms_per_query_per_layer": round(ms_step / B / L, 5),
        "scan_ms": round(scan_ms, 4),
        "scan_ms_median_min_max": [round(float(np.median(seg[:, 1])), 4), round(float(seg[:, 1].min()), 4),
                                   round(float(seg[:, 1].max()), 4)],
        "scan_ms_per_layer": round(scan_ms / L, 5),
        "blocks_scanned_per_s": round(L * n_blk * B / (scan_ms * 1e-3), 1),
        "breakdown_ms": {"pool": round(float(seg_mean[0]), 4), "route_scan": round(scan_ms, 4),
                         "topk": round(float(seg_mean[2]), 4), "gather": round(float(seg_mean[3]), 4),
                         "decode": round(float(seg_mean[4]), 4)},
        "decode_us_per_token": round(float(seg_mean[4]) * 1e3, 2),
        "decode_rows": dec_rows,
        "needles_are_topk": needle_ok,
        "roofline": roofline,
    }
    if cfg.per_token:
        pool_ms = float(seg_mean[0])
        result["pooled_tokens_per_s"] = round(L * n_tok / (pool_ms * 1e-3), 1)
        result["pool_GBps"] = round(L * n_tok * POOL_BYTES_PER_TOKEN / (pool_ms * 1e-3) / 1e9, 2)
        # the pooling dominates a per-token step: it is the line's roofline kernel
        pool_bytes = L * n_tok * POOL_BYTES_PER_TOKEN + 3 * L * n_blk * 2048 + L * tiles * 16 * 8 * 4
        pool_gbps = pool_bytes / (pool_ms * 1e-3) / 1e9
        pool_traffic = (round(POOL_TRAFFIC_BYTES / 1e9, 3)
                        if (POOL_TRAFFIC_BYTES and cfg.name == "1m"
                            and source_digest(("pool.hip", "msa_device.hpp")) == POOL_TRAFFIC_SOURCE_DIGEST)
                        else None)
        # the library takes one tile per workgroup when the launch would have fewer than 4 per CU
        small = 3 * tiles * L < 4 * torch.cuda.get_device_properties(0).multi_processor_count
        result["roofline"] = {"bound": "hbm", "kernel": "pool_kernel<16, %d> (msa_pool_blocks)" % (1 if small else 4),
                              "achieved": round(pool_gbps, 2),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(pool_gbps / HBM_PEAK_GBPS, 4),
                              "traffic": pool_traffic, "traffic_unit": "GB per launch",
                              "algorithmic_GB_per_launch": round(pool_bytes / 1e9, 3)}

    # Every step of the path against its own bound (mean over the timed steps).
    def hbm_row(ms, nbytes, note):
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "algorithmic_GB": round(nbytes / 1e9, 4), "GBps": round(gbps, 1),
                "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": note}
    rows = {}
    if cfg.per_token:
        rows["A1_pool"] = hbm_row(float(seg_mean[0]), L * n_tok * POOL_BYTES_PER_TOKEN + 3 * L * n_blk * 2048
                                  + L * tiles * 16 * 8 * 4,
                                  "K, V, Kr token rows read + K-bar, V-bar, Kr-bar rows and Kr-bar norms written")
    LLC_BYTES = 256e6                     # MI355X last-level (Infinity) cache
    scan_bytes = L * n_blk * SCAN_BYTES_PER_BLOCK_LAYER
    if cfg.per_token:
        scan_cache = ("keys written by the pooling earlier in the step (%.2f GB): the part still in the "
                      "%d MB last-level cache is served from it" % (scan_bytes / 1e9, LLC_BYTES / 1e6))
    else:
        scan_cache = ("cold: %.1f GB of keys stream through the %d MB last-level cache"
                      % (scan_bytes / 1e9, LLC_BYTES / 1e6))
    rows["A2_route_scan"] = dict(roofline, ms=round(scan_ms, 4), cache=scan_cache)
    rows["A3_topk"] = dict(hbm_row(float(seg_mean[2]), L * B * n_docs * 4 + L * B * k * 8, "scores read + ids/scores written"),
                           bound="latency (%d rows of %d scores)" % (L * B, n_docs))
    rows["A4_gather"] = dict(hbm_row(float(seg_mean[3]), ctx_rows * 4 * 2048, "K-bar and V-bar rows read + written"),
                             bound="latency (dependent id -> offset -> row loads)")
    loc_bytes = L * B * cfg.L_loc * DECODE_BYTES_PER_ROW
    other = scan_bytes + (L * n_tok * POOL_BYTES_PER_TOKEN if cfg.per_token else 0)
    rows["A5_decode"] = dict(hbm_row(float(seg_mean[4]), dec_rows * DECODE_BYTES_PER_ROW, "K and V rows of 8 heads read"),
                             bound="hbm",
                             cache="memory context (%.1f MB) written by the gather just before: warm; local rows "
                                   "(%.0f MB) last touched a step earlier, behind %.2f GB of other traffic: %s"
                                   % (ctx_rows * 2048 * 2 / 1e6, loc_bytes / 1e6, other / 1e9,
                                      "cold" if other + loc_bytes > LLC_BYTES else "cache-resident"))
    result["rows"] = rows
    if not args.no_cpu_baseline:
        result["cpu_rows"] = cpu_rows(cfg, L, B, k, n_docs, blk.numpy(), dsc, ids, kbar, vbar, q, ck, cv, cl, lk,
                                      lv, ll, scale, pool_args)

    if args.calibrate_copy:
        del ck, cv
        result["calibration_copy_bytes"] = calibration_copy(dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, di, blk.numpy(), args.cpu_seconds, unit, pool_args, scale)
    print(json.dumps(result), flush=True)


def host_tier_bench(args):
    """The step with the content K-bar/V-bar in pinned host DRAM (the pages' own deployment):
    routing keys stay in HBM, and each layer group's Top-16 documents are gathered over the host
    link on a second stream while the next group's layers are scanned.  Pinned host memory on
    this machine is capped near 64 GiB, so the 100M-token memory's 115 GB of content cannot be
    pinned; the 10M-token memory (11.5 GB of content, the same document-length mix, 32 queries)
    is used, and the link traffic is reported per query (it depends only on the selected
    documents' lengths)."""
    import numpy as np
    import torch

    from routed_kv_memory_amd import msa
    from synth import synth as S
    from synth.device import DeviceInputs

    cfg = S.CONFIGS["10m"]
    dev = "cuda"
    L, B, k, Hq = cfg.n_layers, cfg.B, cfg.k, cfg.Hq
    t_setup = time.time()
    di = DeviceInputs(cfg, dev)
    blk = di.prepooled_offsets()
    n_blk = int(blk[-1])
    max_db = int((blk[1:] - blk[:-1]).max())
    n_docs = blk.numel() - 1
    blk_d = blk.to(dev)
    tiles = msa.msa_route_tiles(n_blk)
    krt, contiguous = route_key_memory((L, tiles * 16, 8, 128), torch.bfloat16)
    krn, _ = route_key_memory((L, tiles * 16, 8), torch.float32)
    for l, rows in di.prepooled_route_rows():
        msa.msa_pack_route_keys(rows.view(1, n_blk, 8, 128), n_blk, krt[l:l + 1], krn[l:l + 1])
    blk_doc = torch.empty(tiles * 16, dtype=torch.int32, device=dev)
    msa.msa_block_doc_map(blk_d, n_blk, blk_doc)
    kh, vh = di.prepooled_content_host()
    qr = di.qr()
    q, lk, lv, ll = di.decode_inputs()
    max_ctx = k * max_db
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=dev)
    ids = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    tsc = torch.empty((L, B, k), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msa.msa_topk_docs_workspace_size(L, B, n_docs, k), 256), dtype=torch.uint8, device=dev)
    ck = torch.empty((L, B, max_ctx, 8, 128), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    cl = torch.empty((L, B), dtype=torch.int32, device=dev)
    out = torch.empty((L, B, Hq, 128), dtype=torch.float32, device=dev)
    ws_dec = torch.empty(msa.msa_sparse_decode_workspace_size(L, B, Hq, max_ctx, cfg.L_loc), dtype=torch.uint8,
                         device=dev)
    scale = 1.0 / math.sqrt(128.0)
    torch.cuda.synchronize()
    print("bench: host-tier memory ready in %.1f s (%.1f GB pinned host content)"
          % (time.time() - t_setup, 2 * sum(t.numel() for t in kh) * 2 / 1e9), file=sys.stderr, flush=True)

    def gather_layers(l0, l1, stream=None):
        # the content is one pinned allocation per layer
        for l in range(l0, l1):
            msa.msa_gather_ctx(ids[l:l + 1], blk_d, max_db, kh[l], vh[l], ck[l:l + 1], cv[l:l + 1], cl[l:l + 1],
                               stream=stream)

    G = max(1, min(args.host_groups, L))
    bounds = [L * g // G for g in range(G + 1)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()            # default priority
    evs = [torch.cuda.Event() for _ in range(G)]

    def step(overlap=True):
        for g in range(G):
            l0, l1 = bounds[g], bounds[g + 1]
            msa.msa_route_scores(qr[l0:l1], krt[l0:l1], n_blk, blk_doc, n_docs, dsc[l0:l1], krbar_norm=krn[l0:l1])
            s = side if overlap else main
            if overlap:
                evs[g].record(main)
                side.wait_event(evs[g])
            msa.msa_topk_docs(dsc[l0:l1], k, ids[l0:l1], tsc[l0:l1], ws, stream=s)
            gather_layers(l0, l1, stream=s)
        if overlap:
            main.wait_stream(side)
        msa.msa_sparse_decode(q, ck, cv, cl, lk, lv, ll, scale, out, ws_dec)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

    warm_up(lambda: (step(True), step(False)), args)
    ms_overlap = timed(lambda: step(True), args.steps)
    ms_serial = timed(lambda: step(False), args.steps)
    # the gather alone, from host DRAM and (for scale) from an HBM copy of the selected rows' source
    ms_gather_host = timed(lambda: gather_layers(0, L), args.steps)
    ctx_rows = int(cl.sum().item())
    link_bytes = ctx_rows * 2 * 2048                  # K-bar and V-bar rows read over the link
    nd = S.needle_docs(cfg)
    ids_h = ids.cpu().numpy()
    needle_ok = all(set(ids_h[l, b].tolist()) == set(nd[b].tolist()) for l in range(L) for b in range(nd.shape[0]))
    result = {
        "metric": "host-tier step ms (content K/V in host DRAM), 18 layers, 10M-token memory, 32 queries",
        "value": round(ms_overlap, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_overlap, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "10M-token memory, routing keys in HBM (5.76 GB), content K-bar/V-bar in pinned "
                               "host DRAM (11.5 GB), %d queries x 64 tokens, top-16, local 1,024" % B,
                   "layer_groups": G, "route_key_alloc": "one contiguous device allocation" if contiguous else "caching allocator"},
        "ms_serial_one_stream": round(ms_serial, 4),
        "overlap_saving_ms": round(ms_serial - ms_overlap, 4),
        "host_gather_ms_18_layers": round(ms_gather_host, 4),
        "host_gather_MB": round(link_bytes / 1e6, 2),
        "host_gather_MB_per_query": round(link_bytes / 1e6 / B, 2),
        "host_gather_ms_per_query_equivalent": round(ms_gather_host / B, 4),
        "host_link_GBps": round(link_bytes / (ms_gather_host * 1e-3) / 1e9, 2),
        "needles_are_topk": needle_ok,
    }
    print(json.dumps(result), flush=True)


def interleaved_bench(args):
    """Interleaved re-routing on the 100M-token memory: 8 queries grow 64 -> 576 -> 1,088 tokens;
    each round scores only the new rows and max-merges them into the documents' scores
    (msa_route_scores accumulate=1), then selects the Top-16 again.  Reported against the bf16
    matrix-core peak (the rounds are far above the ridge)."""
    import numpy as np
    import torch

    from routed_kv_memory_amd import msa
    from synth import synth as S
    from synth.device import DeviceInputs

    cfg = S.CONFIGS["interleaved"]
    dev = "cuda"
    L, B, k = cfg.n_layers, cfg.B, cfg.k
    t_setup = time.time()
    di = DeviceInputs(cfg, dev)
    blk = di.prepooled_offsets()
    n_blk = int(blk[-1])
    n_docs = blk.numel() - 1
    blk_d = blk.to(dev)
    tiles = msa.msa_route_tiles(n_blk)
    krt, contiguous = route_key_memory((L, tiles * 16, 8, 128), torch.bfloat16)
    krn, _ = route_key_memory((L, tiles * 16, 8), torch.float32)
    for l, rows in di.prepooled_route_rows():
        msa.msa_pack_route_keys(rows.view(1, n_blk, 8, 128), n_blk, krt[l:l + 1], krn[l:l + 1])
    blk_doc = torch.empty(tiles * 16, dtype=torch.int32, device=dev)
    msa.msa_block_doc_map(blk_d, n_blk, blk_doc)
    qr = di.qr()
    bounds = [0] + list(cfg.T_rounds)
    qr_rounds = [qr[:, :, bounds[r]:bounds[r + 1]].contiguous() for r in range(len(cfg.T_rounds))]
    del qr
    dsc = torch.empty((L, B, n_docs), dtype=torch.float32, device=dev)
    ids = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    tsc = torch.empty((L, B, k), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msa.msa_topk_docs_workspace_size(L, B, n_docs, k), 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print("bench: interleaved memory ready in %.1f s" % (time.time() - t_setup), file=sys.stderr, flush=True)

    n_r = len(qr_rounds)
    def step(evs=None):
        for r in range(n_r):
            if evs is not None:
                evs[2 * r].record()
            msa.msa_route_scores(qr_rounds[r], krt, n_blk, blk_doc, n_docs, dsc, accumulate=r > 0, krbar_norm=krn)
            if evs is not None:
                evs[2 * r + 1].record()
            msa.msa_topk_docs(dsc, k, ids, tsc, ws)
        if evs is not None:
            evs[2 * n_r].record()

    warm_up(step, args)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_r + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(2 * n_r)] for i in range(args.steps)])
    seg = seg.mean(axis=0)
    rounds = []
    total_flop = 0.0
    for r in range(n_r):
        rows = B * (bounds[r + 1] - bounds[r])
        flop = 2.0 * rows * 1024 * L * n_blk
        total_flop += flop
        rounds.append({"query_tokens": bounds[r + 1], "new_rows": rows, "scan_ms": round(float(seg[2 * r]), 3),
                       "topk_ms": round(float(seg[2 * r + 1]), 4),
                       "scan_TFLOPs": round(flop / (seg[2 * r] * 1e-3) / 1e12, 1),
                       "frac_of_mfma_peak": round(flop / (seg[2 * r] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)})
    # the needles of query 0 stay selected in every layer
    nd0 = set(S.needle_docs(cfg)[0].tolist())
    ids_h = ids.cpu().numpy()
    needle_ok = all(nd0 <= set(ids_h[l, 0].tolist()) for l in range(L))
    big = max(range(n_r), key=lambda r: rounds[r]["new_rows"])
    tfl = total_flop / (wall / args.steps) / 1e12
    result = {
        "metric": "interleaved re-routing TFLOP/s (% of bf16 MFMA peak), 18 layers, 100M-token memory",
        "value": round(tfl, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.description or "interleaved re-routing", "layers": L, "queries": B,
                   "rounds_query_tokens": list(cfg.T_rounds), "blocks_per_layer": n_blk, "docs": n_docs, "top_k": k,
                   "route_key_alloc": "one contiguous device allocation" if contiguous else "caching allocator", "scan_key_norms": "read"},
        "rounds": rounds,
        "roofline": {"bound": "mfma", "kernel": "route_heads_kernel<4, true, 2> (msa_route_scores, round %d)" % (big + 1),
                     "achieved": rounds[big]["scan_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": rounds[big]["frac_of_mfma_peak"], "traffic": None},
        "needles_of_query_0_selected": needle_ok,
    }
    if not args.no_cpu_baseline:
        # the oracle's scan of layer 0 over every document for query 0's first-round rows, in TFLOP/s
        result["cpu_baseline"] = cpu_baseline(cfg, di, blk.numpy(), args.cpu_seconds, "TFLOP/s", None, None)
    print(json.dumps(result), flush=True)


def prefill_bench(args):
    """The multi-token sparse prefill at the interleaved workload's last round: every query's
    1,088 tokens over [its 16 selected documents' blocks ; its own 1,088 local rows]."""
    import numpy as np
    import torch

    import oracle as O
    from routed_kv_memory_amd import msa
    from synth import synth as S
    from synth.device import DeviceInputs

    cfg = S.CONFIGS["interleaved"]
    di = DeviceInputs(cfg, "cuda")
    q, ck, cv, cl, lk, lv, ll = di.prefill_inputs()
    L, B, T, Hq = q.shape[:4]
    scale = 1.0 / math.sqrt(128.0)
    out = torch.empty((L, B, T, Hq, 128), dtype=torch.float32, device="cuda")

    def step():
        msa.msa_sparse_prefill(q, ck, cv, cl, lk, lv, ll, scale, out)

    warm_up(step, args)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    ctx_rows = int(cl.sum().item())
    pairs = ctx_rows * T + L * B * T * (T + 1) // 2          # (token, key) pairs per query head
    flop = 4.0 * 128 * Hq * pairs                             # QK^T and P.V, 2 flop per MAC
    tflops = flop / (wall / args.steps) / 1e12
    achieved = flop / (ms * 1e-3) / 1e12

    # sampled parity against the oracle (token t sees its memory rows and local rows 0..t)
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    worst = 0.0
    for (l, b) in ((0, 0), (L - 1, B - 1)):
        n_ctx = int(cl[l, b])
        ckh, cvh, lkh, lvh = u16(ck[l, b, :n_ctx]), u16(cv[l, b, :n_ctx]), u16(lk[l, b]), u16(lv[l, b])
        for t in (0, T // 2, T - 1):
            ref = O.decode(u16(q[l, b, t]), ckh, cvh, lkh[:t + 1], lvh[:t + 1], scale)
            got = out[l, b, t].cpu().numpy()
            worst = max(worst, float((np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max()))
    result = {
        "metric": "sparse prefill TFLOP/s (% of bf16 MFMA peak), interleaved last round",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "multi-token sparse prefill: %d layers x %d queries x %d tokens, %d query heads over "
                               "8 KV heads, memory context of 16 documents' blocks (mean %.0f rows) + %d local rows, "
                               "causal in the local part" % (L, B, T, Hq, ctx_rows / (L * B), T),
                   "layers": L, "queries": B, "query_tokens": T, "q_heads": Hq, "kv_heads": 8, "head_dim": 128,
                   "memory_rows_total": ctx_rows, "local_rows": T},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<4> (msa_sparse_prefill)", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": flop,
                     "note": "the P.V product runs twice (bf16 high part + residual of the probabilities); "
                             "achieved counts the algorithmic flop once"},
        "sampled_max_rel_err": worst,
    }
    if not args.no_cpu_baseline:
        n_ctx = int(cl[0, 0])
        args_o = (u16(q[0, 0, T - 1]), u16(ck[0, 0, :n_ctx]), u16(cv[0, 0, :n_ctx]), u16(lk[0, 0]), u16(lv[0, 0]))
        tt = time.perf_counter()
        reps = 0
        while time.perf_counter() - tt < min(args.cpu_seconds, 5.0) or reps == 0:
            O.decode(*args_o, scale)
            reps += 1
        dt = (time.perf_counter() - tt) / reps
        f_tok = 4.0 * 128 * Hq * (n_ctx + T)
        result["cpu_baseline"] = {"value": round(f_tok / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "fp64 oracle, last token of (layer 0, query 0): %d query heads over %d + "
                                            "%d rows, %d repetitions, %.2f s each" % (Hq, n_ctx, T, reps, dt)}
    print(json.dumps(result), flush=True)


def encode_bench(args):
    """The offline encode front-end over the 1M-token document set: every layer projects its
    hidden rows to K, V and Kr (8 heads x 128), normalises and rotates K, and pools the three
    into 64-token block means, in one launch for all 18 layers."""
    import numpy as np
    import torch

    import oracle as O
    from routed_kv_memory_amd import msa
    from synth import synth as S
    from synth.device import DeviceInputs

    cfg = S.CONFIGS["1m"]
    Hd, eps, theta = S.ENC_HIDDEN, 1e-6, 1e6
    tok, x, wk, wv, wr, wn = DeviceInputs(cfg, "cuda").encode_inputs(Hd)
    L, n_tok = x.shape[0], x.shape[1]
    blk, n_blk, _ = msa.msa_block_offsets_host(tok)
    tok_d, blk_d = tok.to("cuda"), blk.to("cuda")
    kbar = torch.empty((L, n_blk, 8, 128), dtype=torch.bfloat16, device="cuda")
    vbar = torch.empty_like(kbar)
    tiles = msa.msa_route_tiles(n_blk)
    krt = torch.empty((L, tiles * 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    krn = torch.empty((L, tiles * 16, 8), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print("bench: encode inputs ready (%d layers x %d tokens x %d hidden, %d blocks, %.1f GB on device)"
          % (L, n_tok, Hd, n_blk, torch.cuda.memory_allocated() / 1e9), file=sys.stderr, flush=True)

    def step():
        msa.msa_encode_blocks(x, wk, wv, wr, wn, eps, theta, tok_d, blk_d, n_blk, kbar, vbar, krt, krn)

    warm_up(step, args)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flop = 2.0 * L * n_tok * Hd * 3 * 1024                    # the three projections; the epilogue is O(n_tok)
    tflops = flop / (wall / args.steps) / 1e12
    achieved = flop / (ms * 1e-3) / 1e12
    # algorithmic bytes: hidden rows and weights read once, pooled outputs written once
    nbytes = L * (n_tok * Hd * 2 + 3 * Hd * 1024 * 2 + 3 * n_blk * 1024 * 2 + tiles * 16 * 8 * 4)

    # sampled parity: V and Kr of blocks anywhere (no position dependence), K of documents'
    # first blocks, against the oracle on the host-regenerated inputs
    tok_n, blk_n = tok.numpy(), blk.numpy()
    lens = np.diff(tok_n)
    rng = np.random.default_rng(7)
    n_samples = 2 if args.no_cpu_baseline else 8      # the oracle calls double as the CPU-baseline sample
    samples = [(int(l), int(rng.integers(0, lens.size))) for l in np.linspace(0, L - 1, n_samples).round()]
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    wn_h = u16(wn)
    worst = 0.0
    cpu_dt = []
    for l, d in samples:
        w_h = [np.ascontiguousarray(S.enc_weights_host(S.memory_config(cfg).seed, st, l, Hd).T)
               for st in (S.S_ENC_WK, S.S_ENC_WV, S.S_ENC_WKR)]   # the oracle takes W as [hidden][1024]
        jb = int(rng.integers(0, blk_n[d + 1] - blk_n[d]))
        for j, what in ((0, "KVR"), (jb, "VR")):
            t0_, t1_ = int(tok_n[d]) + 64 * j, min(int(tok_n[d]) + 64 * j + 64, int(tok_n[d + 1]))
            xh = S.enc_x_host(S.memory_config(cfg).seed, l, n_tok, Hd, t0_, t1_)
            tt = time.perf_counter()
            ref = O.encode(xh, *w_h, wn_h[l], eps, theta, np.array([0, t1_ - t0_], np.int64),
                           np.array([0, 1], np.int64))
            cpu_dt.append((time.perf_counter() - tt, t1_ - t0_))
            b = int(blk_n[d]) + j
            got = {"K": u16(kbar[l, b]), "V": u16(vbar[l, b]),
                   "R": u16(krt[l, 16 * (b // 16):16 * (b // 16) + 16]).reshape(8, 16, 16, 8)[:, :, b % 16].reshape(8, 128)}
            for key, r in zip("KVR", ref):
                if key not in what:
                    continue
                g64 = S.bf16_to_f32(got[key]).astype(np.float64)
                r64 = S.bf16_to_f32(r[0]).astype(np.float64)
                mag = np.abs(r64)
                ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
                tol = np.maximum(ulp, np.exp2(-16) * mag.max(axis=-1, keepdims=True))
                worst = max(worst, float((np.abs(g64 - r64) / tol).max()))
    result = {
        "metric": "encode front-end TFLOP/s (% of bf16 MFMA peak), 1M-token document set",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "offline encode: %d layers x %d tokens (%d lognormal documents) x hidden %d -> "
                               "K, V, Kr (8 x 128 each), key RMS norm + document-wise RoPE, 64-token block "
                               "means (%d blocks)" % (L, n_tok, lens.size, Hd, n_blk),
                   "layers": L, "tokens": n_tok, "documents": int(lens.size), "hidden": Hd, "blocks": n_blk,
                   "rope_theta": theta, "norm_eps": eps},
        "tokens_per_s": round(L * n_tok / (wall / args.steps), 1),
        "roofline": {"bound": "mfma", "kernel": "encode_kernel (msa_encode_blocks)", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (ENCODE_TRAFFIC_BYTES if source_digest(("encode.hip", "msa_device.hpp"))
                                 == ENCODE_TRAFFIC_SOURCE_DIGEST else None), "traffic_unit": "bytes per launch",
                     "algorithmic_flop_per_launch": flop, "algorithmic_bytes_per_launch": nbytes,
                     "hbm_frac_at_this_rate": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "sampled_max_err_over_tol": round(worst, 4),
    }
    if args.calibrate_copy:
        del x
        result["calibration_copy_bytes"] = calibration_copy()
    if not args.no_cpu_baseline:
        dt = sum(c[0] for c in cpu_dt)
        ntk = sum(c[1] for c in cpu_dt)
        result["cpu_baseline"] = {"value": round(2.0 * Hd * 3 * 1024 * ntk / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": "fp64 oracle on the %d sampled blocks (%d tokens, %.1f s)"
                                            % (len(cpu_dt), ntk, dt)}
    print(json.dumps(result), flush=True)


def cpu_rows(cfg, L, B, k, n_docs, blk_off, dsc, ids, kbar, vbar, q, ck, cv, cl, lk, lv, ll, scale, pool_args):
    """The fp64 oracle's top-k, gather, decode (and pooling) on one (layer, query) of the same
    step's GPU data, single thread, with the whole-step equivalent (x layers x queries)."""
    import numpy as np

    import oracle as O

    import torch

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    def u16(t):   # bf16 tensor -> its uint16 bit patterns on the host
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    out = {}
    S = dsc[0, 0].double().cpu().numpy()
    dt = timed(lambda: O.topk(S, k))
    out["A3_topk"] = {"sample": "one (layer, query): top-%d of %d scores" % (k, n_docs), "s": round(dt, 6),
                      "step_equivalent_ms": round(dt * L * B * 1e3, 3)}
    sel = ids[0, 0].cpu().numpy()
    kb_parts, vb_parts, off = [], [], [0]
    for d in sel:
        b0, b1 = int(blk_off[d]), int(blk_off[d + 1])
        kb_parts.append(u16(kbar[0, b0:b1]))
        vb_parts.append(u16(vbar[0, b0:b1]))
        off.append(off[-1] + b1 - b0)
    kb_c, vb_c = np.concatenate(kb_parts), np.concatenate(vb_parts)
    off = np.array(off, np.int64)
    dt = timed(lambda: O.gather(np.arange(len(sel), dtype=np.int32), off, kb_c, vb_c))
    out["A4_gather"] = {"sample": "one (layer, query): %d selected documents, %d blocks" % (len(sel), int(off[-1])),
                        "s": round(dt, 6), "step_equivalent_ms": round(dt * L * B * 1e3, 3)}
    n_ctx, n_loc = int(cl[0, 0]), int(ll[0, 0])
    args = (u16(q[0, 0]), u16(ck[0, 0, :n_ctx]), u16(cv[0, 0, :n_ctx]), u16(lk[0, 0, :n_loc]), u16(lv[0, 0, :n_loc]))
    dt = timed(lambda: O.decode(*args, scale))
    out["A5_decode"] = {"sample": "one (layer, query): %d query heads over %d + %d rows" % (q.shape[2], n_ctx, n_loc),
                        "s": round(dt, 6), "step_equivalent_ms": round(dt * L * B * 1e3, 3)}
    if pool_args is not None:
        kt, vt, krt_, tok_d = pool_args[0], pool_args[1], pool_args[2], pool_args[3]
        tok = tok_d.cpu().numpy()
        nd = min(len(tok) - 1, 40)
        t_end = int(tok[nd])
        sub_tok = tok[: nd + 1]
        sub_blk, _, _ = O.block_offsets(sub_tok)
        xs = [u16(a[0:1, :t_end]) for a in (kt, vt, krt_)]
        dt = timed(lambda: [O.pool(x, sub_tok, sub_blk) for x in xs])
        n_tok = int(tok[-1])
        out["A1_pool"] = {"sample": "layer 0, documents 0..%d (%d tokens), K, V and Kr" % (nd - 1, t_end),
                          "s": round(dt, 6), "step_equivalent_ms": round(dt * L * n_tok / t_end * 1e3, 1)}
    out["cores"] = 1
    out["kind"] = "oracle"
    return out


def cpu_baseline(cfg, di, blk_off, seconds, unit, pool_args, scale):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload, its documents
    split over the host's cores (orc_doc_scores_mt / orc_pool_mt: threads over contiguous
    document ranges, each running the single-threaded oracle), reported in the line's unit.

    Pre-pooled memories: the routing scan of whole layers (every document) for whole queries,
    layer 0 first, until about `seconds` have passed (one full layer at least).  Per-token
    memories: the oracle's whole path for one layer at a time (pooling of K, V and Kr, scan,
    top-k, gather, decode of query 0), layers until about `seconds` have passed."""
    import numpy as np
    import torch

    import oracle as O
    from synth import synth as S

    threads = O.host_threads()
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if not cfg.per_token:
        rows = di.prepooled_route_rows_layer_host(0)
        q = S.qr_host(cfg, 0)
        n_blk = int(blk_off[-1])
        t0 = time.perf_counter()
        done = 0
        while True:
            O.doc_scores_mt(q[done, :cfg.T], rows, blk_off, threads=threads)
            done += 1
            dt = time.perf_counter() - t0
            if done >= cfg.B or dt + dt / done > seconds:
                break
        work = "routing scan of layer 0, all %d documents (%d blocks), %s (%d tokens each)" % (
            len(blk_off) - 1, n_blk, "query 0" if done == 1 else "queries 0..%d" % (done - 1), cfg.T)
        if unit == "TFLOP/s":
            v = 2.0 * cfg.T * 1024 * n_blk * done / dt / 1e12
        else:
            v = n_blk * SCAN_BYTES_PER_BLOCK_LAYER * done / dt / 1e9
        return {"value": round(v, 6), "unit": unit, "cores": threads, "kind": "oracle",
                "sample": "fp64 oracle, %s, %d threads, %.1f s" % (work, threads, dt),
                "blocks_per_s": round(n_blk * done / dt, 1)}
    # per-token memory: the oracle's own path, layer by layer
    kt, vt, krt_, tok_d = pool_args[0], pool_args[1], pool_args[2], pool_args[3]
    tok = tok_d.cpu().numpy()
    blk, n_blk, _ = O.block_offsets(tok)
    n_tok = int(tok[-1])
    q, lk, lv, ll = di.decode_inputs()
    qr = di.qr()
    t_total, layers = 0.0, 0
    while True:                 # layers in turn (again from layer 0 when a memory has few of them)
        l = layers % cfg.n_layers
        xs = [u16(a[l:l + 1]) for a in (kt, vt, krt_)]
        qr_l, q_l = u16(qr[l, 0]), u16(q[l, 0])
        nl = int(ll[l, 0])
        lk_l, lv_l = u16(lk[l, 0, :nl]), u16(lv[l, 0, :nl])
        t0 = time.perf_counter()
        kb, vb, rb = (O.pool_mt(x, tok, blk, threads=threads)[0] for x in xs)
        S_o = O.doc_scores_mt(qr_l, rb, blk, threads=threads)
        ids, _ = O.topk(S_o, cfg.k)
        ck, cv = O.gather(ids, blk, kb, vb)
        O.decode(q_l, ck, cv, lk_l, lv_l, scale)
        t_total += time.perf_counter() - t0
        layers += 1
        if t_total + t_total / layers > seconds:
            break
    if layers <= cfg.n_layers:
        span = "layer%s 0..%d" % ("" if layers == 1 else "s", layers - 1)
    else:
        span = "%d layer passes over layer%s 0..%d" % (layers, "" if cfg.n_layers == 1 else "s", cfg.n_layers - 1)
    work = ("whole path (pooling of K, V, Kr; scan; top-%d; gather; decode of query 0) of %s, "
            "%d tokens per layer" % (cfg.k, span, n_tok))
    if unit == "ms":
        v = t_total * 1e3 / layers * cfg.n_layers
    else:
        v = n_tok * layers / t_total
    return {"value": round(v, 4 if unit == "ms" else 1), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle, %s, %d threads, %.1f s" % (work, threads, t_total)}


if __name__ == "__main__":
    main()
