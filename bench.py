#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

Default workload: the full 32-layer decode step of the 8B geometry -- batch 32,
every context 4096 tokens, 32 query heads / 8 KV heads, head_dim 128,
block_size 16, F16 K/V ~ N(0, 1), a fresh random block table per layer in a
pool of twice the needed blocks.  --kv-dtype fp8 stores the same values as
E4M3 codes (per-layer key and value scales 0.02: N(0, 1) values span about
+-250 of the format's +-448) and reads half the bytes.  One step = build the schedule on the host
from the step's context lengths (pa_decode_plan), copy it to the GPU
asynchronously, then for each of the 32 layers pa_decode_run with the newest
token's K/V: it stores them into their slots and attends over the whole
context (for this batch the schedule is one piece per sequence, so each layer
is one kernel launch and nothing is merged).

Prints one JSON line: achieved KV GB/s (value), decode tokens/s, the fraction
of HBM peak, a roofline record for the dominant kernel (decode_partial), and
the fp64 CPU oracle timed on this host as a baseline.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV GB/s (% HBM peak) and decode tokens/s"
HBM_PEAK_GBPS = 8000.0
# the kernels and the header whose constants and argument layout they compile with
KERNEL_FILES = (os.path.join("paged_kv_cache_64_amd", "csrc", "pa_internal.h"),
                os.path.join("paged_kv_cache_64_amd", "csrc", "pa_kernels.hip"))
KERNEL_SOURCES = tuple(os.path.join(ROOT, f) for f in KERNEL_FILES)
COUNTERS_FILES = {"f16": os.path.join(ROOT, "profiles", "decode_partial_c3_counters.txt"),
                  "fp8": os.path.join(ROOT, "profiles", "decode_partial_fp8_c3_counters.txt")}
COUNTERS_CONFIG = 3          # the workload the counter files were taken on
FP8_SCALE = 0.02


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_code_hash(root=None):
    """sha256 of the kernel sources with comments and whitespace removed: it
    changes with the code, not with its comments.  root: another checkout's
    top directory (its files that exist are hashed), else this one."""
    paths = KERNEL_SOURCES if root is None else [os.path.join(root, f) for f in KERNEL_FILES]
    text = ""
    for path in paths:
        if root is not None and not os.path.exists(path):
            continue
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()


def launch_kernels(info, num_kv_heads=8):
    """The kernels one pa_decode_run launch of this plan runs, as the library
    picks them: ordinary and shared-prefix pieces share cascade_kernel, a plan
    with per-wave KV heads (pieces of at most 1024 tokens, KV heads a multiple
    of 4) takes decode_wave_heads_kernel, and a plan that cuts sequences adds
    the merge."""
    if info.num_items > 0 and info.num_prefix_items > 0:
        names = ["cascade_kernel"]
    else:
        wave_heads = (getattr(info, "decode_wave_heads", 0) == 1 and num_kv_heads % 4 == 0
                      and info.max_piece_tokens <= 1024)
        names = [("decode_wave_heads_kernel" if wave_heads else "decode_partial_kernel")] if info.num_items > 0 else []
        names += ["decode_prefix_kernel"] if info.num_prefix_items > 0 else []
    if info.num_merges > 0:
        names.append("decode_merge_planned_kernel")
    return " + ".join(names)


def read_counters(kv_dtype):
    """HBM traffic per decode_partial launch from the committed rocprofv3 summary,
    or None when it is missing or was taken on other kernel source."""
    return read_counter_file(COUNTERS_FILES[kv_dtype])


def read_counter_file(path):
    """fetch + write bytes per launch from a committed counter summary, or None
    when it is missing or was taken on other kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_code_sha256") != kernel_code_hash():
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def write_blocks(pool, layer, ids, k, v, dev):
    """Stores whole physical blocks (host F16 [n, B, Hkv, d]) through pa_write_kv
    with the caller-built slot list of those blocks."""
    import torch
    import workloads

    rows = lambda x: torch.from_numpy(x.reshape(-1, pool.num_kv_heads, pool.head_dim)).to(dev)
    pool.write(layer, rows(k), rows(v),
               torch.from_numpy(workloads.block_slot_mapping(ids, pool.block_size)).to(dev))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..9 (default 3); 6 and 7 are mixed steps (chunked prefill); "
                         "8 is a launch-bound 32-layer batch-1 step (see --graph); 9 is 1024 "
                         "sequences of 128 tokens")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--kv-dtype", choices=("f16", "fp8"), default="f16",
                    help="K/V storage: F16, or FP8 E4M3 codes with per-layer scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--cascade", action="store_true",
                    help="for a workload with shared prefixes, schedule with pa_cascade_plan")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB three times (to scale the FETCH_SIZE "
                         "and WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              f"supported: this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_64_amd as pa
    import workloads
    from paged_kv_cache_64_amd import roofline

    lib = pa.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        plib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_64_amd", "libpa_probe.so"))
        plib.pa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        plib.pa_probe_copy.restype = ctypes.c_int32
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for _ in range(3):
            assert plib.pa_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes,
                                      torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}), flush=True)
        return
    w = workloads.config(args.config, args.seed)
    B, HQ, HKV, D = w.block_size, w.num_q_heads, w.num_kv_heads, w.head_dim
    log(f"workload: {w.name}; pool {w.layers} layers x {w.pool_blocks} blocks")
    if w.q_lens is not None:
        if args.cascade or args.graph:
            print("mixed steps run without --cascade or --graph", file=sys.stderr)
            sys.exit(2)
        return bench_mixed(args, w, dev)

    # ---- stage the pool through pa_write_kv, layer by layer ----
    t_stage = time.time()
    fp8 = args.kv_dtype == "fp8"
    eb = 1 if fp8 else 2
    pool = pa.Pool(w.layers, w.pool_blocks, HKV, D, B, device=dev, fill=0.0,
                   dtype=pa.PA_FP8_E4M3 if fp8 else pa.PA_F16)
    q_dev, tables_dev, knew, vnew = [], [], [], []
    host0 = None
    ctx = w.ctx_lens.astype(np.int64)
    for layer in range(w.layers):
        ids, k, v = w.kv_blocks(layer)
        if fp8:
            pool.set_scales(layer, FP8_SCALE, FP8_SCALE)
        write_blocks(pool, layer, ids, k, v, dev)
        q = w.q(layer)
        tables = w.tables(layer)
        q_dev.append(torch.from_numpy(q).to(dev))
        tables_dev.append(torch.from_numpy(tables).to(dev))
        # the step's newest token (position ctx-1) is stored again with its own values,
        # so every timed step sees the same pool
        pos = np.maximum(ctx - 1, 0)
        blk = tables[np.arange(w.batch), pos // B]
        rank = np.searchsorted(ids, blk)
        rank = np.minimum(rank, len(ids) - 1) if len(ids) else rank
        kn = k[rank, pos % B] if len(ids) else np.zeros((w.batch, HKV, D), np.float16)
        vn = v[rank, pos % B] if len(ids) else np.zeros((w.batch, HKV, D), np.float16)
        knew.append(torch.from_numpy(np.ascontiguousarray(kn)).to(dev))
        vnew.append(torch.from_numpy(np.ascontiguousarray(vn)).to(dev))
        if layer == 0 and not args.no_cpu_baseline:
            host0 = (q, tables, ids, k, v)
        del ids, k, v
        if layer % 8 == 7:
            log(f"staged {layer + 1}/{w.layers} layers")
    torch.cuda.synchronize()
    log(f"staging took {time.time() - t_stage:.1f} s")

    mcl = w.max_context_len
    width = w.max_blocks
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    h = pool.handle
    scale = ctypes.c_float(w.scale)
    outs = [torch.empty_like(q) for q in q_dev]

    # the schedule: sized once, rebuilt on the host every step into one of two
    # pinned buffers and copied to the GPU without blocking the host
    lens_host = np.ascontiguousarray(w.ctx_lens, dtype=np.int32)
    info = pa.PlanInfo()
    cascade = args.cascade and w.prefix_groups is not None
    if cascade:
        n_groups, gsize, pblocks = w.prefix_groups
        group_host = np.repeat(np.arange(n_groups, dtype=np.int32), gsize)
        plen_host = np.full(n_groups, pblocks * B, dtype=np.int32)

    def make_plan(dst, nbytes):
        if cascade:
            return lib.pa_cascade_plan(h, lens_host.ctypes.data, w.batch, group_host.ctypes.data,
                                       plen_host.ctypes.data, n_groups, HQ, dst, nbytes,
                                       ctypes.byref(info))
        return lib.pa_decode_plan(h, lens_host.ctypes.data, w.batch, HQ, dst, nbytes,
                                  ctypes.byref(info))

    rc = make_plan(None, 0)
    assert rc == 0, rc
    plan_words = max(1, info.plan_bytes // 4)
    plan_pinned = [torch.zeros(plan_words, dtype=torch.int32).pin_memory() for _ in range(2)]
    plan_dev = torch.zeros(plan_words, dtype=torch.int32, device=dev)
    ws_bytes = info.workspace_bytes
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    f_run = lib.pa_decode_run
    # a cascade plan whose newest tokens lie in shared blocks cannot append them
    append = info.shared_newest == 0
    plan_dev_bytes = plan_dev.numel() * 4
    run_args = [(h, L, ctypes.byref(info), plan_dev.data_ptr(), plan_dev_bytes, q_dev[L].data_ptr(),
                 knew[L].data_ptr() if append else None, vnew[L].data_ptr() if append else None,
                 outs[L].data_ptr(),
                 tables_dev[L].data_ptr(), width, scale, ws.data_ptr(), ws_bytes, sptr)
                for L in range(w.layers)]
    nstep = [0]

    def step(events=None):
        buf = plan_pinned[nstep[0] % 2]
        nstep[0] += 1
        rc = make_plan(buf.data_ptr(), buf.numel() * 4)
        if rc != 0:
            raise RuntimeError(f"pa_decode_plan failed: {rc}")
        plan_dev.copy_(buf, non_blocking=True)
        if events is not None:
            events[0].record(stream)
        for L in range(w.layers):
            rc = f_run(*run_args[L])
            if rc != 0:
                raise RuntimeError(f"pa_decode_run failed in layer {L}: {rc}")
        if events is not None:
            events[1].record(stream)

    split = info.max_piece_tokens
    kv_bytes_step = w.kv_bytes(elem_bytes=eb)
    plib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_64_amd", "libpa_probe.so"))
    plib.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    plib.pa_probe_read.restype = ctypes.c_int32
    sink = torch.empty(plib.pa_probe_read_groups(), dtype=torch.int32, device=dev)
    # small steps would run from the 256 MB last-level cache: between timed
    # steps, read (not write, which would leave dirty lines to drain) 1 GiB
    cold_flush = kv_bytes_step < (4 << 30)
    flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev) if cold_flush else None

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); plan: {info.num_items} pieces, longest {split} "
        f"tokens, {info.num_merges} merges, workspace={ws_bytes} B; cold flush between steps: "
        f"{cold_flush}")

    # Timed region 1 (the headline): K whole steps, events only around each step.
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush_buf is not None:
            plib.pa_probe_read(flush_buf.data_ptr(), flush_buf.numel(), sink.data_ptr(), sptr)
        step_ev[i][0].record(stream)
        step()
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    ms_per_step = float(np.mean(step_ms))

    # Timed region 2 (the roofline record): the same K steps with an event pair
    # around each step's back-to-back pa_decode_run launches (after the plan
    # upload) -- one decode_partial launch per layer when the schedule merges
    # nothing -- so a launch's time is the pair's interval over the layers.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush_buf is not None:
            plib.pa_probe_read(flush_buf.data_ptr(), flush_buf.numel(), sink.data_ptr(), sptr)
        step(ev[i])
    torch.cuda.synchronize()
    part_us = [1e3 * a.elapsed_time(b) / w.layers for a, b in ev]
    log(f"timed {args.steps} steps: mean {ms_per_step:.4f} ms, min {min(step_ms):.4f} ms, "
        f"wall {1e3 * wall / args.steps:.4f} ms/step; decode_partial mean {np.mean(part_us):.2f} us")

    # optional: the same step captured once in a HIP graph and replayed, against
    # the eager step run back to back the same way (no flush between steps, the
    # host enqueueing as fast as it can: where launches dominate, this is the
    # cost a graph removes)
    graph_ms = None
    eager_b2b_ms = None
    if args.graph:
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_ev.record(stream)
        for _ in range(args.steps):
            step()
        b_ev.record(stream)
        torch.cuda.synchronize()
        eager_b2b_ms = a_ev.elapsed_time(b_ev) / args.steps
        log(f"eager steps back to back: {eager_b2b_ms:.4f} ms/step")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            sptr_saved = sptr
            run_args[:] = [a[:-1] + (side.cuda_stream,) for a in run_args]
            with torch.cuda.graph(graph, stream=side):
                step()
            run_args[:] = [a[:-1] + (sptr_saved,) for a in run_args]
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        for _ in range(args.steps):
            graph.replay()
        b_ev.record(stream)
        torch.cuda.synchronize()
        graph_ms = a_ev.elapsed_time(b_ev) / args.steps
        log(f"HIP graph replay: {graph_ms:.4f} ms/step")

    kv_gbps = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = w.batch / (ms_per_step * 1e-3)
    kb = roofline.split_kernel_bytes(w.ctx_lens, HQ, HKV, D, B, kv_elem_bytes=eb)
    part_mean_s = float(np.mean(part_us)) * 1e-6
    # shared prefix blocks: HBM need deliver each distinct slot only once, so
    # the roofline counts unique K/V bytes (the logical rate is "value")
    basis = "logical"
    launch_bytes = kb["total"]
    if w.prefix_groups is not None:
        basis = "unique"
        launch_bytes = kb["total"] - kb["kv"] + w.kv_unique_bytes(eb) // w.layers
    achieved = launch_bytes / part_mean_s / 1e9
    traffic = read_counters(args.kv_dtype) if args.config == COUNTERS_CONFIG else None

    # ---- HBM read probe: the bandwidth this GPU reaches on a plain stream ----
    probe = None
    if not args.no_probe:
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        for _ in range(2):
            plib.pa_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), sptr)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record(stream)
        for _ in range(reps):
            plib.pa_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), sptr)
        b.record(stream)
        torch.cuda.synchronize()
        probe = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        del buf
        log(f"HBM read probe: {probe:.0f} GB/s")

    # ---- gather probe: whole K tiles of the pool (the kernel's tile size) in a
    # random order, 4 GiB per launch: the rate this access pattern allows ----
    gather = None
    if not args.no_probe:
        plib.pa_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        plib.pa_probe_gather.restype = ctypes.c_int32
        tile = 16 * D * eb
        src_bytes = pool.k.numel() * pool.k.element_size()
        groups = plib.pa_probe_read_groups()
        n_tiles = min(src_bytes // tile, (4 << 30) // tile) // groups * groups
        if n_tiles > 0:
            ids = np.random.default_rng(7).choice(src_bytes // tile, size=n_tiles, replace=False).astype(np.int32)
            ids_dev = torch.from_numpy(ids).to(dev)
            go = lambda: plib.pa_probe_gather(pool.k.data_ptr(), src_bytes, tile, ids_dev.data_ptr(), n_tiles,
                                              sink.data_ptr(), sptr)
            for _ in range(2):
                assert go() == 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            a.record(stream)
            for _ in range(reps):
                go()
            b.record(stream)
            torch.cuda.synchronize()
            gather = n_tiles * tile * reps / (a.elapsed_time(b) * 1e-3) / 1e9
            del ids_dev
            log(f"HBM gather probe ({tile} B tiles, random order): {gather:.0f} GB/s")

    # ---- oracle on the host: baseline timing and a parity sample ----
    cpu = None
    parity = None
    if host0 is not None:
        import oracle

        threads = len(os.sched_getaffinity(0))
        errs, refs, diffs = [], [], []
        done_seqs, done_bytes, cpu_s = 0, 0, 0.0
        layer = 0
        while layer < w.layers and cpu_s < args.cpu_seconds:
            if layer == 0:
                q, tables, ids, k, v = host0
            else:
                ids, k, v = w.kv_blocks(layer)
                q, tables = w.q(layer), w.tables(layer)
            kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, w.ctx_lens, B)
            if fp8:   # the codes the pool holds, computed by the oracle from the F16 values
                kc = oracle.quantize_e4m3(kc, FP8_SCALE)
                vc = oracle.quantize_e4m3(vc, FP8_SCALE)
            # the GPU result of this layer (read-only decode of the staged pool)
            rc = f_run(h, layer, ctypes.byref(info), plan_dev.data_ptr(), plan_dev_bytes, q_dev[layer].data_ptr(),
                       None, None, outs[layer].data_ptr(), tables_dev[layer].data_ptr(), width,
                       scale, ws.data_ptr(), ws_bytes, sptr)
            assert rc == 0, rc
            torch.cuda.synchronize()
            gpu = outs[layer].cpu().numpy().astype(np.float64)
            for lo in range(0, w.batch, 8):
                seqs = np.arange(lo, min(w.batch, lo + 8))
                t_cpu = time.perf_counter()
                if fp8:
                    ref = oracle.decode_e4m3(q[seqs], kc, vc, t2[seqs], w.ctx_lens[seqs], w.scale,
                                             B, FP8_SCALE, FP8_SCALE, threads=threads)
                else:
                    ref = oracle.decode(q[seqs], kc, vc, t2[seqs], w.ctx_lens[seqs], w.scale, B,
                                        threads=threads)
                cpu_s += time.perf_counter() - t_cpu
                errs.append(float(np.abs(gpu[seqs] - ref).max()))
                refs.append(float((ref ** 2).sum()))
                diffs.append(float(((gpu[seqs] - ref) ** 2).sum()))
                done_seqs += len(seqs)
                done_bytes += int(w.ctx_lens[seqs].astype(np.int64).sum()) * HKV * D * 2 * eb
                if cpu_s >= args.cpu_seconds:
                    break
            layer += 1
        cpu = {"value": round(done_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "cpu_model": host_cpu_model(),
               "sample": f"{done_seqs} (sequence, layer) rows of the same step over layers "
                         f"0..{layer - 1} ({done_bytes} B of K/V), fp64, {cpu_s:.1f} s of oracle time",
               "tokens_per_s_equiv": round(done_bytes / (kv_bytes_step / w.batch) / cpu_s, 4)}
        # the same oracle on one thread, over the first sequences of layer 0
        q, tables, ids, k, v = host0
        kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, w.ctx_lens, B)
        if fp8:
            kc = oracle.quantize_e4m3(kc, FP8_SCALE)
            vc = oracle.quantize_e4m3(vc, FP8_SCALE)
        one_s, one_bytes, one_seqs = 0.0, 0, 0
        while one_seqs < w.batch and one_s < args.cpu_seconds / 4:
            seqs = np.array([one_seqs])
            t_cpu = time.perf_counter()
            if fp8:
                oracle.decode_e4m3(q[seqs], kc, vc, t2[seqs], w.ctx_lens[seqs], w.scale, B, FP8_SCALE,
                                   FP8_SCALE, threads=1)
            else:
                oracle.decode(q[seqs], kc, vc, t2[seqs], w.ctx_lens[seqs], w.scale, B, threads=1)
            one_s += time.perf_counter() - t_cpu
            one_bytes += int(w.ctx_lens[one_seqs]) * HKV * D * 2 * eb
            one_seqs += 1
        del kc, vc
        cpu["one_thread"] = {"value": round(one_bytes / one_s / 1e9, 4), "unit": "GB/s", "cores": 1,
                             "sample": f"{one_seqs} sequences of layer 0 ({one_bytes} B of K/V), fp64, "
                                       f"{one_s:.1f} s"}
        parity = {"rows": done_seqs, "max_abs_err": max(errs),
                  "rel_l2": (sum(diffs) / sum(refs)) ** 0.5}
        log(f"oracle: {cpu['value']} GB/s on {threads} threads; parity {parity}")

    line = {
        "metric": METRIC,
        "value": round(kv_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "ms_per_step_min": round(float(np.min(step_ms)), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "kv_dtype": args.kv_dtype, "layers": w.layers, "batch": w.batch,
                   "context": int(w.ctx_lens.max()), "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": D, "block_size": B, "pool_blocks_per_layer": w.pool_blocks,
                   "schedule": {"pieces": info.num_items, "longest_piece_tokens": split,
                                "merged_sequences": info.num_merges,
                                "shared_prefix_pieces": info.num_prefix_items,
                                "appends_newest_token": append},
                   "cold_flush_between_steps": cold_flush},
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_hbm_peak": round(100 * kv_gbps / HBM_PEAK_GBPS, 2),
        "kv_bytes_per_step": kv_bytes_step,
        "kv_unique_bytes_per_step": w.kv_unique_bytes(eb),
        "unique_kv_GBps": round(w.kv_unique_bytes(eb) / (ms_per_step * 1e-3) / 1e9, 2),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic if info.num_merges == 0 else None,
                     "kernel": launch_kernels(info, HKV),
                     "bytes_per_launch": launch_bytes, "kv_bytes_basis": basis,
                     "mean_launch_us": round(part_mean_s * 1e6, 3)},
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms else None,
        "eager_back_to_back_ms_per_step": round(eager_b2b_ms, 5) if eager_b2b_ms else None,
        "hbm_read_probe_GBps": round(probe, 1) if probe else None,
        "pct_of_probe": round(100 * kv_gbps / probe, 2) if probe else None,
        "hbm_gather_probe_GBps": round(gather, 1) if gather else None,
        "kernel_pct_of_gather_probe": round(100 * achieved / gather, 2) if gather else None,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "pages_context": roofline.pages_context(),
    }
    print(json.dumps(line), flush=True)
    pool.close()


MIXED_METRIC = "mixed step (chunked prefill + decode): query tokens/s"
PREFILL_COUNTERS = {6: os.path.join(ROOT, "profiles", "prefill_c6_counters.txt")}
MFMA_F16_PEAK_TFLOPS = 2500.0


def bench_mixed(args, w, dev):
    """A step of workload 6 or 7: every layer runs pa_prefill_run on the step's
    plan (decode pieces, prefill pieces, merges).  Prints one JSON line."""
    import numpy as np
    import torch

    import paged_kv_cache_64_amd as pa

    lib = pa.load_library()
    B, HQ, HKV, D = w.block_size, w.num_q_heads, w.num_kv_heads, w.head_dim
    qs = w.query_start
    total_q = int(qs[-1])
    lens_host = np.ascontiguousarray(w.ctx_lens, dtype=np.int32)
    chunk_seqs = [s for s in range(w.batch) if w.q_lens[s] > 1]
    dec_seqs = [s for s in range(w.batch) if w.q_lens[s] == 1]

    t_stage = time.time()
    fp8 = args.kv_dtype == "fp8"
    pool = pa.Pool(w.layers, w.pool_blocks, HKV, D, B, device=dev, fill=0.0,
                   dtype=pa.PA_FP8_E4M3 if fp8 else pa.PA_F16)
    q_dev, tables_dev = [], []
    host0 = None
    for layer in range(w.layers):
        ids, k, v = w.kv_blocks(layer)
        if fp8:
            pool.set_scales(layer, FP8_SCALE, FP8_SCALE)
        write_blocks(pool, layer, ids, k, v, dev)
        q = w.q_rows(total_q, layer)
        tables = w.tables(layer)
        q_dev.append(torch.from_numpy(q).to(dev))
        tables_dev.append(torch.from_numpy(tables).to(dev))
        if layer == 0 and not args.no_cpu_baseline:
            host0 = (q, tables, ids, k, v)
        del ids, k, v
    torch.cuda.synchronize()
    log(f"staging took {time.time() - t_stage:.1f} s")

    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    h = pool.handle
    width = w.max_blocks
    outs = [torch.empty_like(q) for q in q_dev]

    def make(qs_h, lens_h):
        info = pa.PlanInfo()
        rc = lib.pa_prefill_plan(h, qs_h.ctypes.data, lens_h.ctypes.data, len(lens_h), HQ, None, 0,
                                 ctypes.byref(info))
        assert rc == 0, rc
        return info

    # the whole step's plan, rebuilt on the host every step (alternating
    # pinned buffers) and uploaded without blocking the host
    info = make(qs, lens_host)
    words = max(1, info.plan_bytes // 4)
    pinned = [torch.zeros(words, dtype=torch.int32).pin_memory() for _ in range(2)]
    plan_dev = torch.zeros(words, dtype=torch.int32, device=dev)
    ws = torch.empty(max(info.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    scale = ctypes.c_float(w.scale)
    nstep = [0]

    def step():
        buf = pinned[nstep[0] % 2]
        nstep[0] += 1
        rc = lib.pa_prefill_plan(h, qs.ctypes.data, lens_host.ctypes.data, w.batch, HQ, buf.data_ptr(),
                                 buf.numel() * 4, ctypes.byref(info))
        if rc != 0:
            raise RuntimeError(f"pa_prefill_plan failed: {rc}")
        plan_dev.copy_(buf, non_blocking=True)
        for L in range(w.layers):
            rc = lib.pa_prefill_run(h, L, ctypes.byref(info), plan_dev.data_ptr(), plan_dev.numel() * 4,
                                    q_dev[L].data_ptr(),
                                    outs[L].data_ptr(), tables_dev[L].data_ptr(), width, scale,
                                    ws.data_ptr(), info.workspace_bytes, sptr)
            if rc != 0:
                raise RuntimeError(f"pa_prefill_run failed in layer {L}: {rc}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done; plan: {info.num_items} decode pieces, {info.num_prefill_items} prefill pieces, "
        f"{info.num_merges} merges, workspace {info.workspace_bytes} B")

    # Timed region 1 (the headline): K whole steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = float(np.mean(step_ms))

    # Timed regions 2 and 3: the prompt chunk alone (the prefill kernel and its
    # merge) and the decode rows alone, each as its own plan over all layers
    def part(seqs):
        sub_q = np.concatenate([[0], np.cumsum(w.q_lens[seqs])]).astype(np.int32)
        sub_l = np.ascontiguousarray(lens_host[seqs])
        inf = make(sub_q, sub_l)
        ph = np.zeros(max(1, inf.plan_bytes // 4), np.int32)
        assert lib.pa_prefill_plan(h, sub_q.ctypes.data, sub_l.ctypes.data, len(sub_l), HQ, ph.ctypes.data,
                                   ph.nbytes, ctypes.byref(inf)) == 0
        pd = torch.from_numpy(ph).to(dev)
        wsp = torch.empty(max(inf.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
        rows_t = torch.from_numpy(rows).to(dev)
        qp = [q[rows_t].contiguous() for q in q_dev]
        tp = [t[torch.tensor(seqs, device=dev)].contiguous() for t in tables_dev]
        op = [torch.empty_like(x) for x in qp]

        def go():
            for L in range(w.layers):
                rc = lib.pa_prefill_run(h, L, ctypes.byref(inf), pd.data_ptr(), pd.numel() * 4, qp[L].data_ptr(),
                                        op[L].data_ptr(),
                                        tp[L].data_ptr(), width, scale, wsp.data_ptr(), inf.workspace_bytes, sptr)
                assert rc == 0, rc
        go()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            go()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) / w.layers * 1e3, inf

    pf_us, pf_info = part(chunk_seqs)
    dec_us, _ = part(dec_seqs)
    vis = 0
    for s in chunk_seqs:
        n = int(w.q_lens[s])
        hist = int(lens_host[s]) - n
        vis += n * hist + n * (n + 1) // 2
    pf_flops = 4 * D * HQ * vis
    achieved = pf_flops / (pf_us * 1e-6) / 1e12
    dec_bytes = int(lens_host[dec_seqs].astype(np.int64).sum()) * HKV * D * 2 * (1 if fp8 else 2)
    log(f"step {ms_per_step:.4f} ms; prefill part {pf_us:.2f} us/layer ({achieved:.1f} TFLOP/s); "
        f"decode part {dec_us:.2f} us/layer ({dec_bytes / (dec_us * 1e-6) / 1e9:.0f} GB/s)")

    # the oracle on sampled rows of layer 0: baseline timing and a parity sample
    cpu = None
    parity = None
    if host0 is not None:
        import oracle

        threads = len(os.sched_getaffinity(0))
        q, tables, ids, k, v = host0
        kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, w.ctx_lens, B)
        if fp8:   # the codes the pool holds, computed by the oracle from the F16 values
            kc = oracle.quantize_e4m3(kc, FP8_SCALE)
            vc = oracle.quantize_e4m3(vc, FP8_SCALE)
        gpu = outs[0].cpu().numpy().astype(np.float64)
        owner = np.searchsorted(qs, np.arange(total_q), side="right") - 1
        rng = np.random.default_rng(0)
        order = rng.permutation(total_q)
        done, cpu_s, errs, refs, diffs = 0, 0.0, [], [], []
        while done < total_q and cpu_s < args.cpu_seconds:
            rows = np.sort(order[done:done + 16])
            own = owner[rows]
            visn = (lens_host[own] - w.q_lens[own] + (rows - qs[own]) + 1).astype(np.int32)
            t_cpu = time.perf_counter()
            one_each = np.arange(len(rows) + 1, dtype=np.int32)
            if fp8:
                ref = oracle.prefill_e4m3(q[rows], kc, vc, t2[own], one_each, visn, w.scale, B, FP8_SCALE,
                                          FP8_SCALE, threads=threads)
            else:
                ref = oracle.prefill(q[rows], kc, vc, t2[own], one_each, visn, w.scale, B, threads=threads)
            cpu_s += time.perf_counter() - t_cpu
            errs.append(float(np.abs(gpu[rows] - ref).max()))
            refs.append(float((ref ** 2).sum()))
            diffs.append(float(((gpu[rows] - ref) ** 2).sum()))
            done += len(rows)
        # a step is every row of every layer; the sample is uniform over the rows
        cpu = {"value": round(done / (cpu_s * w.layers), 4), "unit": "tokens/s", "cores": threads,
               "kind": "oracle", "cpu_model": host_cpu_model(),
               "sample": f"{done} of the {total_q} query rows of layer 0 drawn uniformly, fp64, "
                         f"{cpu_s:.1f} s of oracle time, scaled to the {w.layers}-layer step"}
        parity = {"rows": done, "max_abs_err": max(errs), "rel_l2": (sum(diffs) / sum(refs)) ** 0.5}
        log(f"oracle: {cpu['value']} tokens/s on {threads} threads; parity {parity}")

    line = {
        "metric": MIXED_METRIC,
        "value": round(total_q / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "ms_per_step_min": round(float(np.min(step_ms)), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "kv_dtype": args.kv_dtype, "layers": w.layers, "sequences": w.batch,
                   "query_tokens": total_q, "prompt_chunk_tokens": int(sum(w.q_lens[chunk_seqs])),
                   "decode_rows": len(dec_seqs), "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
                   "block_size": B,
                   "schedule": {"decode_pieces": info.num_items, "prefill_pieces": info.num_prefill_items,
                                "merges": info.num_merges}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": read_counter_file(PREFILL_COUNTERS[args.config])
                     if args.config in PREFILL_COUNTERS and pf_info.num_merges == 0 and not fp8 else None,
                     "kernel": ("prefill_kernel" if fp8 else "prefill_dma_kernel")
                     + (" + decode_merge_planned_kernel" if pf_info.num_merges else ""),
                     "flops_per_layer": pf_flops, "mean_layer_us": round(pf_us, 3)},
        "decode_rows_us_per_layer": round(dec_us, 3),
        "decode_rows_GBps": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1),
        # the whole step per layer (plan upload included) against the chunk
        # and the decode rows timed alone: how much of the two parts overlaps
        "step_us_per_layer": round(ms_per_step * 1e3 / w.layers, 3),
        "step_over_parts": round(ms_per_step * 1e3 / w.layers / (pf_us + dec_us), 4),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 5),
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)
    pool.close()


if __name__ == "__main__":
    main()
