#!/usr/bin/env python3
"""Benchmark of the sparse NVFP4 MLA decode hot path on one MI355X.

One step = one pass of the hot path over one batch of a workload: one
sparse_mla_decode launch (gather, on-chip unpack, QK^T, online softmax, PV and the
in-launch log-sum-exp combine); the 1,024-token throughput workload also writes its
1,024 new rows with nvfp4_pack_rows first.  Inputs are resident in HBM before timing
starts.

The default run measures the 1,024-token x 128-head workload with its cache write as
the headline (the JSON line's top level), then the 1-, 35-, 128- and 264-token
workloads in the same process (under "configs").  --config k measures only workload k.

Cold caches without a flush in the timed region: every step attends a different
"layer" -- one of L copies of the pool, L chosen so the copies span >= 2 GiB --
so a step never finds its rows in the 256 MB Infinity Cache left by the steps
before it (as in serving, where the other layers run between two launches of one
layer).

The K timed steps run as one replay of a captured HIP graph (the way a serving
loop launches decode; --graph 0 launches them one by one from the host), checked
bit for bit against the eager launch.

Prints one JSON line on stdout.  `value` is decode tokens per second of the
whole step; `roofline` prices the decode kernel's algorithmic work against its
average launch duration, measured with HIP events on the launch stream around a run
of back-to-back launches queued behind a backlog (so the events bracket the kernels
and not the host): gathered KV bytes (352 per valid list entry) against 8 TB/s below
the ridge (16 heads), matrix flops (2 * H * (576 + 512) per valid entry) against
2.5 PFLOP/s above it (64 and 128 heads).  `cpu_baseline` times the CPU oracle on the
host over a token sample of the headline workload.  Untimed for `value`, side legs
report the staged two-pass variant, session-grouped decode (only with --grouped K: on
the 264-token workload it is slower than per-token decode), (`fp8_pool`) the same
decode over the pool kept as 576-byte FP8 rows, the format NVFP4 replaces,
(`indexer_topk`) the sparse indexer's top-2,048 selection that produces the lists,
and (`block_major_pool`) decode and block transfer over the block-major multi-layer
cache layout.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16 matrix, published
ROW_BYTES = 352
COLD_SPAN_BYTES = 2 << 30      # layer copies span at least this much
METRIC = "sparse NVFP4 MLA decode: µs/launch, tokens/s, achieved HBM GB/s vs peak"
CSRC = os.path.join("sparse_mla_decode_04_amd", "csrc")
# A decode kernel's sources: its own file, the shared device headers and the host code that
# sizes its launch.  A counter summary stays valid while these are unchanged.
SHARED_SOURCES = ["api.hip", "smla_combine.hpp", "smla_decode.hpp", "smla_device.hpp", "smla_launch.hpp",
                  "smla_tile.hpp"]
KERNEL_FILES = {"sparse_mla_decode_regs_kernel": "decode_regs.hip",
                "sparse_mla_decode_ws_kernel": "decode_ws.hip",
                "sparse_mla_decode_kernel": "decode.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources(kernel):
    """Source files of the decode kernel whose (possibly demangled) name contains one of
    KERNEL_FILES' keys."""
    own = [f for k, f in KERNEL_FILES.items()
           if k + "(" in kernel or k + "<" in kernel or kernel.endswith(k)]
    if len(own) != 1:
        raise ValueError(f"unknown decode kernel {kernel!r}")
    return [os.path.join(CSRC, f) for f in own + SHARED_SOURCES]


def kernel_hash(kernel):
    h = hashlib.sha256()
    for p in kernel_sources(kernel):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes per decode launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    try:
        if d.get("kernel_hash") != kernel_hash(d.get("kernel", "")):
            return None
    except ValueError:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, q, idx, src, seconds, n_tokens):
    """Time the oracle on the host over a seeded sample of the workload's tokens (repeating
    the sample until about `seconds` have passed).  The sample's rows are quantized
    beforehand by the oracle's own row writer (untimed), so the timed part is what one GPU
    launch does per token: gather, dequant, attention."""
    import oracle
    from helpers import PackedRows
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(6)
    toks = sorted(rng.choice(wl.T, size=min(wl.T, n_tokens), replace=False).tolist())
    rows = PackedRows(src, idx[toks].ravel())
    tokens_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for t in toks:
            oracle.sparse_mla_decode_ref(q, rows, idx, wl.softmax_scale, tokens=[t])
            tokens_done += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return {"value": tokens_done / dt, "unit": "tokens/s", "cores": cores, "blas_threads": int(blas),
            "kind": "oracle",
            "sample": f"{tokens_done} decode tokens of the {wl.name} workload ({len(toks)} seeded tokens of its "
                      f"{wl.T}, repeated), float64 numpy oracle, {dt:.1f} s; {cores} cores available, "
                      f"elementwise work on one thread, BLAS with {blas} threads"}


def backlog(torch, ms=20.0):
    """Queue a spin kernel of about `ms` on the current stream, so that the launches and
    events the host enqueues behind it run back to back (the side legs' Python calls take
    longer to enqueue than some of their kernels take to run)."""
    torch.cuda._sleep(int(ms * 2.0e6))


def staged_timing(binding, wl, layers, q_d, idx_d, out, lse, ws, fused_ms, steps):
    """The staged two-pass variant the pages compare against: pass 1 writes every listed
    row as FP8 E4M3 to a [T][topk][576] buffer in HBM, pass 2 attends over it.  Timed with
    events around each pass on the launch stream, over the same layer copies."""
    import torch
    staged = torch.empty((wl.T, wl.topk, 576), dtype=torch.uint8, device="cuda")
    L = len(layers)

    def run(i, ev=None):
        if ev is not None:
            ev[0].record()
        binding.nvfp4_stage_fp8(layers[i % L], idx_d, staged)
        if ev is not None:
            ev[1].record()
        binding.sparse_mla_decode_fp8rows(q_d, staged, idx_d, wl.pool_rows, wl.softmax_scale, out, lse, 0, ws)
        if ev is not None:
            ev[2].record()

    for i in range(2):
        run(i)
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    backlog(torch)
    for i in range(steps):
        run(2 + i, evs[i])
    torch.cuda.synchronize()
    p1 = float(np.mean([a.elapsed_time(b) for a, b, c in evs])) * 1e3
    p2 = float(np.mean([b.elapsed_time(c) for a, b, c in evs])) * 1e3
    log(f"staged variant: pass 1 (unpack to FP8 in HBM) {p1:.1f} us, pass 2 (attend) {p2:.1f} us, "
        f"total {p1 + p2:.1f} us vs fused {fused_ms * 1e3:.1f} us")
    del staged
    torch.cuda.empty_cache()
    return {"stage_us": p1, "attend_us": p2, "us_per_launch": p1 + p2, "fused_us": fused_ms * 1e3,
            "fused_speedup": (p1 + p2) / (fused_ms * 1e3), "steps": steps}


def grouped_timing(binding, wl, layers, q, q_d, idx, idx_d, src_full, kv_bytes, fused_ms, steps, check_tokens):
    """Session-grouped decode: the tokens of a session (64/H consecutive tokens) share
    most of their rows; smla_group_union builds each group's union list (member bits per
    row) on the GPU, sparse_mla_decode_grouped loads every union row once for all of the
    group's tokens.  Both launches are timed with events on the launch stream; the union
    capacity U is the largest union of the workload's lists rounded up to a tile."""
    import torch
    import oracle
    from helpers import OracleRows, parity_errors
    tpg = 64 // wl.H
    if tpg * wl.H != 64 or wl.T % tpg:
        return None
    sizes = []
    for g in range(wl.T // tpg):
        v = idx[g * tpg:(g + 1) * tpg].reshape(-1)
        sizes.append(len(np.unique(v[(v >= 0) & (v < wl.pool_rows)])))
    U = -(-max(sizes) // 64) * 64
    uniq_rows = int(sum(sizes))
    G = wl.T // tpg
    uni = torch.empty((G, U), dtype=torch.int32, device="cuda")
    cnt = torch.empty((G,), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.T, wl.H, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ws = binding.make_grouped_workspace(wl.T, wl.H, tpg, U, 0, "cuda")
    L = len(layers)

    def run(i, ev=None):
        if ev is not None:
            ev[0].record()
        binding.group_union(idx_d, tpg, wl.pool_rows, U, uni, cnt)
        if ev is not None:
            ev[1].record()
        binding.sparse_mla_decode_grouped(q_d, layers[i % L], uni, tpg, wl.softmax_scale, out, lse, 0, ws)
        if ev is not None:
            ev[2].record()

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    assert int(cnt.max().item()) <= U
    res = {"tokens_per_group": tpg, "union_capacity": U, "union_rows": uniq_rows,
           "unique_kv_bytes": uniq_rows * 352}
    if check_tokens > 0:
        rng = np.random.default_rng(1)
        toks = sorted(rng.choice(wl.T, size=min(wl.T, check_tokens), replace=False).tolist())
        ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src_full), idx, wl.softmax_scale, tokens=toks)
        oe, le, ok = parity_errors(out.cpu().numpy()[toks], lse.cpu().numpy()[toks], ref_o, ref_l)
        log(f"grouped parity on tokens {toks}: out err {oe:.2e}, lse err {le:.2e}, -inf ok {ok}")
        if not (oe <= 2e-3 and le <= 1e-3 and ok):
            print("bench.py: grouped decode does not match the oracle", file=sys.stderr)
            sys.exit(3)
        res["parity"] = {"tokens": toks, "out_err": oe, "lse_err": le}
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    backlog(torch)
    for i in range(steps):
        run(3 + i, evs[i])
    torch.cuda.synchronize()
    u_us = float(np.mean([a.elapsed_time(b) for a, b, c in evs])) * 1e3
    d_us = float(np.mean([b.elapsed_time(c) for a, b, c in evs])) * 1e3
    tot = u_us + d_us
    res.update({"union_us": u_us, "decode_us": d_us, "us_per_launch": tot, "steps": steps,
                "gathered_kv_GBs": kv_bytes / (tot * 1e-6) / 1e9,
                "unique_kv_GBs_decode": uniq_rows * 352 / (d_us * 1e-6) / 1e9,
                "per_token_us": fused_ms * 1e3, "speedup": fused_ms * 1e3 / tot})
    log(f"session-grouped ({tpg} tokens/group, union {uniq_rows} rows = {uniq_rows * 352 / 1e6:.1f} MB of "
        f"{kv_bytes / 1e6:.1f} MB gathered): union {u_us:.1f} us + decode {d_us:.1f} us = {tot:.1f} us "
        f"vs per-token {fused_ms * 1e3:.1f} us; {res['gathered_kv_GBs']:.0f} GB/s on gathered KV, "
        f"{res['unique_kv_GBs_decode']:.0f} GB/s on unique rows in the decode")
    del uni, out, lse, ws
    torch.cuda.empty_cache()
    return res


def fp8pool_timing(binding, wl, q, q_d, idx, idx_d, src_full, n_valid, fused_ms, steps, check_tokens):
    """Decode over the same pool kept as 576-byte FP8 rows (the format NVFP4 replaces):
    the row writer encodes the fp16 source rows, layer copies span the same cold range,
    and sparse_mla_decode_fp8pool is timed with events on the launch stream."""
    import torch
    import oracle
    from helpers import OracleFp8Rows, build_device_fp8_pool, parity_errors
    pool0 = build_device_fp8_pool(src_full, "cuda")
    L = max(2, -(-COLD_SPAN_BYTES // pool0.numel()))
    layers = [pool0] + [pool0.clone() for _ in range(L - 1)]
    out = torch.empty((wl.T, wl.H, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ws = binding.make_workspace(wl.T, wl.H, wl.topk, 0, "cuda")

    def run(i):
        binding.sparse_mla_decode_fp8pool(q_d, layers[i % L], idx_d, wl.softmax_scale, out, lse, 0, ws)

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    kv8 = n_valid * 576
    res = {"row_bytes": 576, "layer_copies": L, "gathered_kv_bytes": kv8}
    if check_tokens > 0:
        rng = np.random.default_rng(2)
        toks = sorted(rng.choice(wl.T, size=min(wl.T, check_tokens), replace=False).tolist())
        ref_o, ref_l = oracle.sparse_mla_decode_fp8pool_ref(q, OracleFp8Rows(src_full), idx, wl.softmax_scale,
                                                            tokens=toks)
        oe, le, ok = parity_errors(out.cpu().numpy()[toks], lse.cpu().numpy()[toks], ref_o, ref_l)
        log(f"fp8 pool parity on tokens {toks}: out err {oe:.2e}, lse err {le:.2e}, -inf ok {ok}")
        if not (oe <= 2e-3 and le <= 1e-3 and ok):
            print("bench.py: FP8-pool decode does not match the oracle", file=sys.stderr)
            sys.exit(3)
        res["parity"] = {"tokens": toks, "out_err": oe, "lse_err": le}
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    backlog(torch)
    for i in range(steps):
        evs[i][0].record()
        run(3 + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    res.update({"us_per_launch": us, "steps": steps, "gathered_kv_GBs": kv8 / (us * 1e-6) / 1e9,
                "nvfp4_us": fused_ms * 1e3, "nvfp4_speedup": us / (fused_ms * 1e3),
                "rows_per_byte_vs_nvfp4": 352 / 576})
    log(f"FP8 576-byte pool: {us:.1f} us per launch ({res['gathered_kv_GBs']:.0f} GB/s on {kv8 / 1e6:.1f} MB "
        f"gathered) vs NVFP4 {fused_ms * 1e3:.1f} us; NVFP4 holds {576 / 352:.2f}x the rows per byte")
    del layers, pool0, out, lse, ws
    torch.cuda.empty_cache()
    return res


def indexer_timing(binding, wl, steps, check_tokens):
    """The sparse indexer's top-k selection (the step that produces the index lists) over
    synthetic scores of each token's context, timed with events on the launch stream over
    score copies spanning >= 2 GiB (each layer has scores of its own).  Algorithmic bytes:
    the scores read once plus the lists written."""
    import torch
    import oracle
    from sparse_mla_decode_04_amd import workloads as W
    try:
        scores, lengths, off = W.indexer_inputs(wl)
    except ValueError:
        return None
    sc0 = torch.from_numpy(scores).to("cuda")
    L = max(2, -(-COLD_SPAN_BYTES // (sc0.numel() * 4)))
    copies = [sc0] + [sc0.clone() for _ in range(L - 1)]
    len_d = torch.from_numpy(lengths).to("cuda")
    off_d = torch.from_numpy(off).to("cuda")
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device="cuda")
    ws = binding.make_indexer_workspace(wl.T, scores.shape[1], wl.topk)   # None: one workgroup per token
    for i in range(3):
        binding.sparse_indexer_topk(copies[i % L], wl.topk, len_d, off_d, out, workspace=ws)
    torch.cuda.synchronize()
    res = {"scores_per_token": int(scores.shape[1]), "score_copies": L,
           "workgroups_per_token": "split" if ws is not None else 1}
    if check_tokens > 0:
        rng = np.random.default_rng(3)
        toks = sorted(rng.choice(wl.T, size=min(wl.T, check_tokens), replace=False).tolist())
        ref = oracle.topk_indices_ref(scores[toks], lengths[toks], wl.topk, off[toks])
        if not np.array_equal(out.cpu().numpy()[toks], ref):
            print("bench.py: indexer top-k does not match the oracle", file=sys.stderr)
            sys.exit(3)
        res["parity"] = {"tokens": toks, "bit_exact": True}
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    backlog(torch)
    for i in range(steps):
        evs[i][0].record()
        binding.sparse_indexer_topk(copies[(3 + i) % L], wl.topk, len_d, off_d, out, workspace=ws)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = scores.size * 4 + wl.T * wl.topk * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    res.update({"us_per_launch": us, "steps": steps, "bytes": nbytes, "GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS})
    log(f"indexer top-{wl.topk} over {scores.shape[1]} scores x {wl.T} tokens: {us:.1f} us per launch, "
        f"{gbs:.0f} GB/s on {nbytes / 1e6:.1f} MB ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    del copies, sc0, out
    torch.cuda.empty_cache()
    return res


def blhnc_timing(binding, wl, q, q_d, idx, idx_d, src_full, layers, kv_bytes, fused_ms, steps, check_tokens,
                 block_rows=16, context_rows=146000):
    """The block-major multi-layer cache (one block of every layer stored together):
      * decode: the pool's layers in one [blocks][layers][block_rows][352] allocation
        spanning >= 2 GiB, each layer written by nvfp4_pack_rows_blhnc from the fp16 source
        rows, sparse_mla_decode_blhnc of a different layer each launch, against the
        layer-major launch;
      * transfer: one request's blocks (a context of 146,000 rows as seeded scattered
        blocks) gathered into a contiguous send buffer with blhnc_copy_blocks, one segment
        per block, against the layer-major cache, one segment per block and layer (one call
        per layer tensor).  Bytes = what is read plus what is written."""
    import torch
    import oracle
    from helpers import OracleRows, parity_errors
    N, B = wl.pool_rows, block_rows
    if N % B:
        return None
    nb = N // B
    layer_bytes = N * ROW_BYTES
    L = max(2, -(-COLD_SPAN_BYTES // layer_bytes))
    if L * layer_bytes > 0xFFFFF000:
        return None
    pool = torch.empty((nb, L, B, ROW_BYTES), dtype=torch.uint8, device="cuda")
    src_d = torch.from_numpy(src_full).to("cuda")
    slots = torch.arange(N, dtype=torch.int32, device="cuda")
    for l in range(L):
        binding.nvfp4_pack_rows_blhnc(src_d, slots, pool, l)
    del src_d, slots
    out = torch.empty((wl.T, wl.H, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ws = binding.make_workspace(wl.T, wl.H, wl.topk, 0, "cuda")

    def run(i):
        binding.sparse_mla_decode_blhnc(q_d, pool, i % L, idx_d, wl.softmax_scale, out, lse, 0, ws)

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    res = {"layers": L, "block_rows": B, "allocation_bytes": int(pool.numel())}
    if check_tokens > 0:
        rng = np.random.default_rng(4)
        toks = sorted(rng.choice(wl.T, size=min(wl.T, check_tokens), replace=False).tolist())
        ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src_full), idx, wl.softmax_scale, tokens=toks)
        oe, le, ok = parity_errors(out.cpu().numpy()[toks], lse.cpu().numpy()[toks], ref_o, ref_l)
        log(f"block-major decode parity on tokens {toks}: out err {oe:.2e}, lse err {le:.2e}, -inf ok {ok}")
        if not (oe <= 2e-3 and le <= 1e-3 and ok):
            print("bench.py: block-major decode does not match the oracle", file=sys.stderr)
            sys.exit(3)
        res["parity"] = {"tokens": toks, "out_err": oe, "lse_err": le}
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    backlog(torch)
    for i in range(steps):
        evs[i][0].record()
        run(3 + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    res.update({"decode_us_per_launch": us, "steps": steps, "gathered_kv_GBs": kv_bytes / (us * 1e-6) / 1e9,
                "layer_major_us": fused_ms * 1e3})
    log(f"block-major pool ({L} layers, {B}-row blocks, {pool.numel() / 1e9:.2f} GB): decode {us:.1f} us per "
        f"launch vs layer-major {fused_ms * 1e3:.1f} us")

    # transfer of one request's blocks
    nblk = min(nb, -(-context_rows // B))
    rng = np.random.default_rng(5)
    ids_h = rng.permutation(nb)[:nblk].astype(np.int32)
    ids = torch.from_numpy(ids_h).to("cuda")
    send = torch.empty((nblk, L, B, ROW_BYTES), dtype=torch.uint8, device="cuda")
    lm = [p.view(nb, B, ROW_BYTES) for p in layers[:L]] if len(layers) >= L else None
    send_lm = torch.empty((L, nblk, B, ROW_BYTES), dtype=torch.uint8, device="cuda")

    def xfer_blocked():
        binding.blhnc_copy_blocks(pool, send, src_ids=ids)

    def xfer_layer_major():
        for l in range(L):
            binding.blhnc_copy_blocks(lm[l], send_lm[l], src_ids=ids)

    xfer_blocked()
    torch.cuda.synchronize()
    if not torch.equal(send[:, L - 1], pool[ids.long(), L - 1]):
        print("bench.py: block transfer does not match its source blocks", file=sys.stderr)
        sys.exit(3)
    moved = 2 * nblk * L * B * ROW_BYTES
    tr = {"blocks": nblk, "bytes_moved": moved, "segments_block_major": nblk, "segments_layer_major": nblk * L}
    for name, fn in (("block_major", xfer_blocked), ("layer_major", xfer_layer_major if lm else None)):
        if fn is None:
            continue
        fn()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(20)]
        backlog(torch)
        for i in range(20):
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        tr[name + "_us"] = t
        tr[name + "_GBs"] = moved / (t * 1e-6) / 1e9
    res["transfer"] = tr
    log(f"transfer of {nblk} blocks ({moved / 2e6:.1f} MB): block-major {tr['block_major_us']:.1f} us "
        f"({tr['block_major_GBs']:.0f} GB/s, {nblk} segments)" +
        (f", layer-major {tr['layer_major_us']:.1f} us ({tr['layer_major_GBs']:.0f} GB/s, {nblk * L} segments "
         f"in {L} calls)" if "layer_major_us" in tr else ""))
    del pool, send, send_lm, out, lse, ws
    torch.cuda.empty_cache()
    return res


def copy_calibration(nbytes=256 << 20, reps=5):
    """A copy of known size: rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch of this copy,
    against its 256 MiB read and 256 MiB written, give the factors that turn those counters
    into HBM bytes."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


LEG_DEFAULTS = {  # side legs and the workloads they run on in the default run
    "staged": {5}, "grouped": {4}, "fp8pool": {4, 5}, "indexer": {2, 4}, "blhnc": {4},
}


def measure(cfg, args, legs, check_tokens, steps, warmup):
    """Build workload `cfg`'s inputs on the GPU, time its step (graph replay of `steps`
    steps) and its decode launch (events around back-to-back launches), check sampled
    tokens against the oracle, run the side legs in `legs`, and free everything.  Returns
    (result dict, state for the CPU baseline)."""
    import torch
    import sparse_mla_decode_04_amd as smla
    from sparse_mla_decode_04_amd import binding, workloads as W
    from helpers import OracleRows, build_device_pool, parity_errors, pool_source_all

    dev = "cuda"
    wl = W.WORKLOADS[cfg]
    log(f"workload {wl.name}: T={wl.T} H={wl.H} pool_rows={wl.pool_rows} topk={wl.topk}")
    t_setup = time.time()
    src_full = pool_source_all(wl)            # with the workload's new rows at their slots
    new, slots = W.new_rows(wl)
    src_base = src_full
    if len(slots):                            # the step writes them; start from the base pool
        src_base = np.concatenate([c for _, c in W.pool_source_chunks(wl)], axis=0)
    pool0 = build_device_pool(src_base, dev)
    del src_base
    pool_bytes = pool0.numel()
    L = max(2, -(-COLD_SPAN_BYTES // pool_bytes))
    layers = [pool0] + [pool0.clone() for _ in range(L - 1)]
    q = W.queries(wl)
    idx = W.index_lists(wl)
    q_d = torch.from_numpy(q).to(dev)
    idx_d = torch.from_numpy(idx).to(dev)
    out = torch.empty((wl.T, wl.H, 512), dtype=torch.float16, device=dev)
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    ws = smla.make_workspace(wl.T, wl.H, wl.topk, args.num_splits, dev)
    decode = [binding.prepare_decode(q_d, p, idx_d, wl.softmax_scale, out, lse, args.num_splits, ws) for p in layers]
    pack = []
    if len(slots):
        new_d = torch.from_numpy(new).to(dev)
        slots_d = torch.from_numpy(slots).to(dev)
        pack = [binding.prepare_pack(new_d, slots_d, p) for p in layers]
    torch.cuda.synchronize()
    splits = args.num_splits or smla.choose_num_splits(wl.T, wl.H, wl.topk)
    log(f"setup {time.time() - t_setup:.1f}s; {L} layer copies of {pool_bytes / 1e6:.1f} MB; splits {splits}")

    n_valid = int(np.sum((idx >= 0) & (idx < wl.pool_rows)))
    kv_bytes = n_valid * ROW_BYTES

    def step(i, ev=None):
        l = i % L
        if pack:
            if ev is not None:
                ev[2].record()
            pack[l]()
        if ev is not None:
            ev[0].record()
        decode[l]()
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # untimed parity check of the last step's output against the oracle
    parity = None
    if check_tokens > 0:
        import oracle
        rng = np.random.default_rng(0)
        toks = sorted(rng.choice(wl.T, size=min(wl.T, check_tokens), replace=False).tolist())
        ref_o, ref_l = oracle.sparse_mla_decode_ref(q, OracleRows(src_full), idx, wl.softmax_scale, tokens=toks)
        oe, le, ok = parity_errors(out.cpu().numpy()[toks], lse.cpu().numpy()[toks], ref_o, ref_l)
        log(f"parity on tokens {toks}: out err {oe:.2e} (tol 2e-3), lse err {le:.2e} (tol 1e-3), -inf ok {ok}")
        if not (oe <= 2e-3 and le <= 1e-3 and ok):
            print(f"bench.py: {wl.name} output does not match the oracle", file=sys.stderr)
            sys.exit(3)
        parity = {"tokens": toks, "out_err": oe, "lse_err": le}

    if args.graph:
        # The timed steps as one HIP graph (captured, replayed once untimed, then timed): the
        # host enqueues one replay instead of K launches.  Every step's output is the same
        # (identical layer copies, the same rows written), so each replay must leave the
        # eager result bit for bit.
        ref_out, ref_lse = out.clone(), lse.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(warmup + i)
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
            print("bench.py: graph replay differs from the eager launch", file=sys.stderr)
            sys.exit(3)
        out.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
            print("bench.py: graph replay differs from the eager launch", file=sys.stderr)
            sys.exit(3)
        del graph
        # launch durations: a run of eager launches of one kernel queued behind a backlog, one
        # HIP event before and one after the run on the launch stream
        n_ev = min(max(steps, 50), 200)

        def bracket(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            backlog(torch)
            e0.record()
            for i in range(n_ev):
                fn(warmup + steps + i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n_ev

        k_avg = bracket(lambda i: decode[i % L]())
        pack_us = bracket(lambda i: pack[i % L]()) * 1e3 if pack else None
        ms_per_step = (t1 - t0) * 1e3 / steps
        log(f"decode launch: mean {k_avg * 1e3:.2f} us over {n_ev} back-to-back launches; "
            f"step {ms_per_step * 1e3:.2f} us (graph replay)")
    else:
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i, evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / steps
        kms = np.array([a.elapsed_time(b) for a, b, _ in evs])
        k_avg = float(np.mean(kms))
        pack_us = float(np.mean([c.elapsed_time(a) for a, b, c in evs])) * 1e3 if pack else None
        log(f"decode launch: mean {k_avg * 1e3:.2f} us, median {np.median(kms) * 1e3:.2f} us, "
            f"min {np.min(kms) * 1e3:.2f} us; step {ms_per_step * 1e3:.2f} us")
    achieved = kv_bytes / (k_avg * 1e-3) / 1e9
    log(f"gathered KV {kv_bytes / 1e6:.2f} MB -> {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    if pack:
        log(f"cache write ({len(slots)} rows): mean {pack_us:.2f} us")

    traffic = traffic_from_profiles(wl.name)
    flops = 2.0 * wl.H * (576 + 512) * n_valid        # QK^T over 576 + PV over 512, per valid entry
    tflops = flops / (k_avg * 1e-3) / 1e12
    if flops / kv_bytes > MFMA_F16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):   # above the ridge
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_F16_PEAK_TFS, "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    log(f"matrix work {flops / 1e9:.2f} GFLOP -> {tflops:.1f} TFLOP/s ({tflops / MFMA_F16_PEAK_TFS:.1%} of 2.5 PF)")
    res = {
        "workload": wl.name, "decode_tokens": wl.T, "heads": wl.H, "topk": wl.topk,
        "launch": "hip_graph" if args.graph else "eager", "pool_rows": wl.pool_rows, "valid_entries": n_valid,
        "row_bytes": ROW_BYTES, "cache_write_rows": int(len(slots)), "layer_copies": L, "num_splits": splits,
        "us_per_launch": k_avg * 1e3, "us_per_step": ms_per_step * 1e3,
        "tokens_per_s": wl.T / (ms_per_step * 1e-3), "gathered_kv_GBs": achieved,
        "hbm_frac": achieved / HBM_PEAK_GBS, "tflops": tflops, "mfma_frac": tflops / MFMA_F16_PEAK_TFS,
        "roofline": roof,
    }
    if pack:
        res["cache_write_us"] = pack_us
    if parity:
        res["parity"] = parity

    def leg_steps(name, n):
        return n if cfg in legs.get(name, ()) else 0

    n = leg_steps("staged", args.staged)
    if n:
        res["staged_variant"] = staged_timing(binding, wl, layers, q_d, idx_d, out, lse, ws, k_avg, n)
    n = leg_steps("grouped", args.grouped)
    if n:
        g = grouped_timing(binding, wl, layers, q, q_d, idx, idx_d, src_full, kv_bytes, k_avg, n, check_tokens)
        if g:
            res["session_grouped"] = g
    n = leg_steps("fp8pool", args.fp8pool)
    if n:
        res["fp8_pool"] = fp8pool_timing(binding, wl, q, q_d, idx, idx_d, src_full, n_valid, k_avg, n, check_tokens)
    n = leg_steps("indexer", args.indexer)
    if n:
        r = indexer_timing(binding, wl, n, check_tokens)
        if r:
            res["indexer_topk"] = r
    n = leg_steps("blhnc", args.blhnc)
    if n:
        r = blhnc_timing(binding, wl, q, q_d, idx, idx_d, src_full, layers, kv_bytes, k_avg, n, check_tokens)
        if r:
            res["block_major_pool"] = r
    del decode, pack, layers, pool0, out, lse, ws, q_d, idx_d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, (wl, q, idx, src_full)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=0,
                    help="run only workload 1..5 (as the headline); default 0: the 1,024-token workload as the "
                         "headline, then workloads 1-4 in the same process (under 'configs')")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing budget, 0 disables")
    ap.add_argument("--cpu-tokens", type=int, default=32, help="distinct tokens in the oracle's timed sample")
    ap.add_argument("--check-tokens", type=int, default=3, help="tokens checked against the oracle (untimed)")
    ap.add_argument("--staged", type=int, default=20,
                    help="steps of the staged two-pass variant leg (the 1,024-token workload; 0 disables)")
    ap.add_argument("--grouped", type=int, default=0,
                    help="steps of the session-grouped decode leg (union lists of groups of 64/H tokens, then "
                         "one pass over them; the 264-token workload; off by default: there it is slower than "
                         "per-token decode)")
    ap.add_argument("--fp8pool", type=int, default=50,
                    help="launches of decode over the same pool kept as 576-byte FP8 rows (the 264- and "
                         "1,024-token workloads; 0 disables)")
    ap.add_argument("--indexer", type=int, default=50,
                    help="launches of the sparse indexer's top-k selection over synthetic scores (the 35- and "
                         "264-token workloads; 0 disables)")
    ap.add_argument("--graph", type=int, default=1,
                    help="1: time the K steps as one replay of a captured HIP graph (default); 0: K eager "
                         "launches from the host")
    ap.add_argument("--blhnc", type=int, default=50,
                    help="launches of the block-major multi-layer pool decode leg, with its block transfer "
                         "(the 264-token workload; 0 disables)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus}, WORLD_SIZE {world}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mla_decode_04_amd as smla

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    smla.lib()
    head_cfg = args.config or 5
    # with --config k every leg runs on workload k; the default run places each leg on the
    # workloads listed in LEG_DEFAULTS
    legs = {k: {head_cfg} for k in LEG_DEFAULTS} if args.config else LEG_DEFAULTS
    head, cpu_state = measure(head_cfg, args, legs, args.check_tokens, args.steps, args.warmup)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(*cpu_state, args.cpu_seconds, args.cpu_tokens)
        log(f"cpu oracle: {cpu['value']:.1f} tokens/s")
    del cpu_state
    others = {}
    if not args.config:
        for cfg in (1, 2, 3, 4):
            r, _ = measure(cfg, args, legs, args.check_tokens, args.steps, min(args.warmup, 10))
            others[r["workload"]] = r
    cfg_keys = ("workload", "decode_tokens", "heads", "topk", "launch", "pool_rows", "valid_entries", "row_bytes",
                "cache_write_rows", "layer_copies", "num_splits", "us_per_launch", "cache_write_us")
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {k: head[k] for k in cfg_keys if k in head},
        "roofline": head["roofline"],
    }
    for k in ("parity", "staged_variant", "session_grouped", "fp8_pool", "indexer_topk", "block_major_pool"):
        if k in head:
            res[k] = head[k]
    if others:
        res["configs"] = others
    if cpu:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
