"""Encode throughput of the byte-level BPE path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main]

One step is one bbpe_encode_segments call over the whole workload (every
step of the path: UTF-8 validation, chunk cuts, specials, split, merge,
ordered assembly), with the text, offsets, tables and workspace already
resident in device memory.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode input MB/s + tokens/s on 1 MI355X; % of HBM roofline; ids bit-exact"
HBM_PEAK_GBS = 8000.0

WORKLOAD_DESC = {
    "main": "main: one 4,200,000-byte allow_special=false segment (70% prose, 15% JSON, 10% code, "
            "5% multibyte), 100,256-rank table + 5 specials, cl100k split, tiktoken-safe",
    "tiny": "tiny: one 65,536-byte ASCII segment, 1,280-rank table, cl100k split",
    "agentic": "agentic: 300 typed segments, 4,000,000 characters, 100,256-rank table",
    "ragged": "ragged: 4,096 requests of 512-8,192 bytes, 100,256-rank table",
    "large": "large: one 67,108,864-byte segment (50% Latin prose, 40% Devanagari/CJK, 10% digit/"
             "punctuation runs), 200,000-rank table, o200k-style split, tiktoken-safe",
}


ALG_BYTES = os.path.join(ROOT, "tests", "golden", "alg_bytes.json")
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by a
# plain copy of known size), valid for the kernel sources they were taken on
TRAFFIC = os.path.join(ROOT, "profiles", "encode_%s_hbm_counters.json")
CSRC = os.path.join(ROOT, "byte_level_bpe_amd", "csrc")


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hip", ".h", ".cpp", ".inc")):
            h.update(fn.encode())
            with open(os.path.join(CSRC, fn), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """Counted HBM bytes per launch of `kernel`, or None when none were taken
    for this workload or the sources changed since."""
    path = TRAFFIC % workload
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(workload, {})
    if t.get("source_sha256_16") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return k["bytes"] if k else None


# Instances of one step under other names (grammar, units per thread, the
# word caches, the 17-32-byte units' placement, the three-phase assembly).
KERNEL_STEP = {
    "k_probe1": "k_probe", "k_probe2": "k_probe", "k_probe_wc": "k_probe", "k_probe1_wc": "k_probe",
    "k_merge_wc": "k_merge", "k_merge_elect": "k_merge", "k_merge_elect_wc": "k_merge",
    "k_merge_wide_few32": "k_merge_wide", "k_merge_wide_wc": "k_merge_wide",
    "k_split_o200k": "k_split", "k_split_agg_o200k": "k_split_agg",
    "k_assemble_based": "k_assemble",
}


def algorithmic_bytes(kernel: str, w: dict) -> int:
    """Bytes one launch of `kernel` must move by the definition of its step.

    w is the workload's entry of tests/golden/alg_bytes.json, counted once by
    the oracle (tests/golden/alg_bytes.py).  For k_probe and the merge
    kernels: the units the kernel settles, each with its bytes (once), 4 B
    per id and the merge loop's rank lookups on it (key bytes + 4 B each).
    Front-end kernels make one pass over the text: the text bytes plus
    64-bit masks in and out (1/8 byte per text byte each).
    """
    n = w["bytes"]
    kernel = KERNEL_STEP.get(kernel, kernel)
    if kernel in w["kernels"]:
        return w["kernels"][kernel]["bytes"]
    if kernel in ("k_count", "k_spans", "k_specials", "k_split_agg", "k_split"):
        return n + n // 8 * (3 if kernel != "k_count" else 1)
    if kernel == "k_pieces":
        return n // 8 + 4 * w["pieces"]
    if kernel == "k_assemble":
        return 4 * w["ids"] * 2 + 8 * w["pieces"]
    return n


def host_cpu() -> dict:
    """The host the oracle runs on: logical CPUs, the CPUs this process may
    use, and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable": len(os.sched_getaffinity(0)), "model": model}


def ids_sha256(ids) -> str:
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(ids, dtype=np.int32).tobytes()).hexdigest()


def cpu_baseline(w, budget_s: float = 10.0, max_reps: int = 200) -> dict:
    """The oracle (plain C++, -O2) on the host cores, reported beside the GPU.

    Row 1: single-threaded, pinned to one core (sched_setaffinity, as
    taskset does), over the whole workload, repeated until about budget_s
    seconds.  Row 2: the same oracle over the workload's independent units
    (segments and 400,000-character windows) on K std::threads, K = the
    usable cores (at most 16), repeated until about budget_s / 2 seconds.
    Each row gives the SHA-256 of its ids."""
    from oracle import Oracle
    from oracle.oracle import encode_parallel, window_units
    orc = Oracle(w.tokens, w.specials, w.grammar)
    cpus = sorted(os.sched_getaffinity(0))
    reps, total, ids = 0, 0.0, None
    os.sched_setaffinity(0, {cpus[-1]})
    try:
        while reps < max_reps and (total < budget_s or reps == 0):
            t0 = time.perf_counter()
            ids, _ = orc.encode_segments(w.segments, w.tiktoken_safe)
            total += time.perf_counter() - t0
            reps += 1
    finally:
        os.sched_setaffinity(0, set(cpus))
    nb = w.text_bytes
    k = min(16, len(cpus))
    pool = [Oracle(w.tokens, w.specials, w.grammar) for _ in range(k)]
    preps, ptotal, pids = 0, 0.0, None
    while preps < max_reps and (ptotal < budget_s / 2 or preps == 0):
        pids, sec = encode_parallel(pool, w.segments, w.tiktoken_safe)
        ptotal += sec
        preps += 1
    n_units = len(window_units(w.segments, w.tiktoken_safe)[0]) - 1
    host = host_cpu()
    return {"value": round(nb * reps / total / 1e6, 3), "unit": "MB/s", "cores": 1,
            "kind": "oracle",
            "tokens_per_s": round(len(ids) * reps / total, 1),
            "ids_sha256": ids_sha256(ids),
            "sample": "whole %s workload (%d bytes) encoded %d times on one pinned core, %.1f s"
                      % (w.name, nb, reps, total),
            "host": host,
            "all_cores": {"value": round(nb * preps / ptotal / 1e6, 3), "unit": "MB/s",
                          "cores": k, "units": n_units,
                          "tokens_per_s": round(len(pids) * preps / ptotal, 1),
                          "ids_sha256": ids_sha256(pids),
                          "sample": "whole workload as %d independent units on %d std::threads, "
                                    "%d times, %.1f s" % (n_units, k, preps, ptotal)}}


def decode_alg_bytes(kernel: str, n_ids: int, n_bytes: int) -> int:
    """Bytes one decode launch must move: k_dec_len reads each id and its
    8-byte table entry and writes a 4-byte length; k_dec_copy reads each id,
    its length and its bytes, writes its 8-byte offset and its bytes."""
    if kernel == "k_dec_len":
        return n_ids * (4 + 8 + 4)
    if kernel == "k_dec_copy":
        return n_ids * (4 + 4 + 8) + 2 * n_bytes
    return 0


def bench_decode(args, w):
    """Device decode of the workload's ids (encoded once on the device before
    timing) into an output sized exactly, with per-token byte offsets."""
    import torch
    import byte_level_bpe_amd as B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    ids, _ = tok.encode_segments(w.segments, w.tiktoken_safe, device=dev)
    n_ids = int(ids.numel())
    total = w.text_bytes
    out = torch.empty(max(1, total), dtype=torch.uint8, device=dev)
    tok_off = torch.empty(max(1, n_ids), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        o, _, _ = tok.decode_device(ids, out=out, tok_off=tok_off, stream=stream)
        return int(o.numel())

    for _ in range(args.warmup):
        nb = step()
    assert nb == total
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    tok.set_timing(True)
    tok.timing_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rep = tok.timing_report()
    tok.set_timing(False)
    per_kernel = {k: v[0] / max(1, v[1]) for k, v in rep.items()}
    dom = max(rep, key=lambda k: rep[k][0])
    dom_bytes = decode_alg_bytes(dom, n_ids, total)
    achieved = dom_bytes / (per_kernel[dom] * 1e-3) / 1e9
    res = {
        "metric": "decode output MB/s + tokens/s on 1 MI355X (ids to bytes with per-token offsets)",
        "value": round(total * args.steps / wall / 1e6, 2),
        "unit": "MB/s",
        "tokens_per_s": round(n_ids * args.steps / wall, 1),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC.get(w.name, w.name), "bytes": total, "ids": n_ids},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": None, "avg_ms": round(per_kernel[dom], 5),
                     "alg_bytes_per_launch": dom_bytes},
        "kernels_avg_ms": {k: round(v, 5) for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1])},
    }
    if not args.no_cpu_baseline:
        from oracle import Oracle
        orc = Oracle(w.tokens, w.specials, w.grammar)
        h = ids.cpu().numpy()
        reps, spent = 0, 0.0
        while spent < 10.0 and reps < 200:
            t0 = time.perf_counter()
            orc.decode(h)
            spent += time.perf_counter() - t0
            reps += 1
        res["cpu_baseline"] = {"value": round(total * reps / spent / 1e6, 3), "unit": "MB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "all %d ids of the %s workload decoded %d times "
                                         "single-threaded, %.1f s" % (n_ids, w.name, reps, spent)}
    print(json.dumps(res), flush=True)


def two_requests_in_flight_ms(tok, tok2, text, seg_off, allow, total, bufs, streams, steps, safe):
    """K calls alternated between two handles on two streams (the second
    handle with its own workspace and outputs), settled by one wait each."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        h, (ids, id_off), st = (tok, bufs[0], streams[0]) if k % 2 == 0 else (tok2, bufs[1], streams[1])
        h.encode_device_async(text, seg_off, allow, total, ids, id_off, tiktoken_safe=safe, stream=st)
    torch.cuda.synchronize()
    tok.encode_wait(streams[0])
    if steps > 1:
        tok2.encode_wait(streams[1])
    return (time.perf_counter() - t0) * 1e3 / steps


def two_requests_leg(tok, w, text, seg_off, allow, total, n_seg, ids, id_off, stream, steps):
    """Context, outside the timed region: the same workload as two requests
    in flight at once (two handles, two streams), the way a server overlaps
    requests; every call still runs the whole path."""
    import torch
    import byte_level_bpe_amd as B
    tok2 = B.load_ranks(w.tokens, w.specials, w.grammar)
    tok2.upload(text.device)
    tok2.workspace(total, n_seg, text.device)
    ids2 = torch.empty_like(ids)
    id_off2 = torch.empty_like(id_off)
    s2 = torch.cuda.Stream(device=text.device)
    bufs, streams = [(ids, id_off), (ids2, id_off2)], [stream, s2]
    gc.collect()
    gc.disable()
    two_requests_in_flight_ms(tok, tok2, text, seg_off, allow, total, bufs, streams, 4, w.tiktoken_safe)
    ms = two_requests_in_flight_ms(tok, tok2, text, seg_off, allow, total, bufs, streams, steps,
                                   w.tiktoken_safe)
    gc.enable()
    ok = bool(torch.equal(ids2[:int(id_off2[-1])], ids[:int(id_off[-1])]))
    del tok2
    return {"ms_per_step": round(ms, 4), "MBs": round(total / (ms * 1e-3) / 1e6, 2),
            "ids_equal": ok,
            "what": "the same calls alternated between two handles on two streams, two requests "
                    "in flight (context: every call runs the whole path; value is one request "
                    "at a time)"}


def warm_cache_leg(tok, w, text, seg_off, allow, total, ids, id_off, stream, want_sha, reps=5):
    """The word cache kept across calls (BBPE_KEEP_WORD_CACHE), outside the
    timed region of the headline number: one call's device time (events on
    the launch stream) (a) with the cache cleared, which fills it; (b) after
    the cache was filled by another text of the same mix (the ragged
    workload's requests, same table, cut to this text's length) -- a serving
    process meeting new requests; (c) re-encoding this same text, every unit
    of 2-32 bytes then found.  Each call's ids are checked against the
    oracle's SHA-256."""
    import torch
    from synth import configs
    other = b"".join(b for b, _ in configs.ragged().segments)[:total]
    while other and ((other[-1] & 0xC0) == 0x80 or other[-1] >= 0xC0):
        other = other[:-1]
    other = other + b" " * (total - len(other))
    dev = text.device
    main_bytes = text[:total].clone()
    other_t = torch.frombuffer(bytearray(other), dtype=torch.uint8).to(dev)

    def call():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n = tok.encode_device(text, seg_off, allow, total, w.tiktoken_safe, ids=ids, id_off=id_off,
                              stream=stream, keep_word_cache=True)[2]
        e1.record(stream)
        torch.cuda.synchronize()
        ok = ids_sha256(ids[:n].cpu().numpy()) == want_sha
        return e0.elapsed_time(e1), tok.word_cache_info()[1], ok

    # the graph of the keep-cache sequence is built by a first call
    tok.word_cache_clear(stream)
    call()
    rows = {"cleared": [], "after_other_text": [], "same_text": []}
    all_ok = True
    for _ in range(reps):
        tok.word_cache_clear(stream)
        ms, hits, ok = call()
        rows["cleared"].append((ms, hits))
        all_ok = all_ok and ok
        tok.word_cache_clear(stream)
        text[:total].copy_(other_t)
        tok.encode_device(text, seg_off, allow, total, w.tiktoken_safe, ids=ids, id_off=id_off,
                          stream=stream, keep_word_cache=True)
        text[:total].copy_(main_bytes)
        torch.cuda.synchronize()
        ms, hits, ok = call()
        rows["after_other_text"].append((ms, hits))
        all_ok = all_ok and ok
        ms, hits, ok = call()
        rows["same_text"].append((ms, hits))
        all_ok = all_ok and ok
    tok.word_cache_clear(stream)

    def med(v):
        v = sorted(v)
        return {"ms": round(v[len(v) // 2][0], 4), "units_from_cache": v[len(v) // 2][1]}
    return {k: med(v) for k, v in rows.items()} | {
        "calls_each": reps, "ids_match_oracle": all_ok,
        "entries": tok.word_cache_info()[0],
        "what": "one call each: cache cleared (fills it); after the cache was filled by another "
                "text of the same mix (ragged requests cut to this length); re-encoding this text"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--blocking", action="store_true",
                    help="time the entry point that waits for each call (default: calls queued "
                         "back to back and settled by one wait)")
    ap.add_argument("--no-warm-cache", action="store_true",
                    help="skip the kept-word-cache leg (main workload only)")
    ap.add_argument("--op", choices=["encode", "decode"], default="encode",
                    help="decode: device decode of the workload's ids with per-token offsets")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), "
                         "to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: every box in this setup has a single MI355X and the "
              "encode path here is single-GPU (see the multi-GPU design notes); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.randint(0, 255, (args.copy_calibration,), dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 5}), flush=True)
        return
    import byte_level_bpe_amd as B
    from synth import configs

    w = configs.ALL[args.workload]()
    if args.op == "decode":
        return bench_decode(args, w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    text, seg_off, allow, total = B.to_device_segments(w.segments, dev)
    n_seg = len(w.segments)
    ids = torch.empty(max(1, total), dtype=torch.int32, device=dev)
    id_off = torch.empty(n_seg + 1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    # first call on a fresh handle (host wall time): the table built and
    # uploaded, the workspace allocated, the call's graph built and run
    f0 = time.perf_counter()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    f1 = time.perf_counter()
    tok.upload(dev)
    tok.workspace(total, n_seg, dev)
    torch.cuda.synchronize()
    f2 = time.perf_counter()

    def step():
        return tok.encode_device(text, seg_off, allow, total, w.tiktoken_safe, ids=ids,
                                 id_off=id_off, stream=stream)[2]

    step()
    torch.cuda.synchronize()
    f3 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    f4 = time.perf_counter()
    first_call = {"load_ranks_ms": round((f1 - f0) * 1e3, 1), "upload_and_workspace_ms": round((f2 - f1) * 1e3, 1),
                  "first_encode_ms": round((f3 - f2) * 1e3, 3), "second_encode_ms": round((f4 - f3) * 1e3, 3),
                  "what": "host wall time on a fresh handle: table build, table upload + workspace "
                          "allocation, the first encode (graph built, kernels loaded) and the second"}

    def step_queued():
        tok.encode_device_async(text, seg_off, allow, total, ids, id_off,
                                tiktoken_safe=w.tiktoken_safe, stream=stream)

    for _ in range(args.warmup):
        n_ids = step()
    if not args.blocking:
        step_queued()
        n_ids = tok.encode_wait(stream)
    torch.cuda.synchronize()
    # timed region: K whole calls, one event before the first and one after
    # the last on the launch stream.  By default the calls are queued back
    # to back (bbpe_encode_segments_async, the way a serving loop issues
    # batches) and settled by one wait inside the region, which also checks
    # every call's status; --blocking times the entry point that waits for
    # each call.  (The interpreter's collector is held off meanwhile.)
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_a.record(stream)
    for k in range(args.steps):
        if args.blocking:
            n_ids = step()
        else:
            step_queued()
    ev_b.record(stream)
    torch.cuda.synchronize()
    if not args.blocking:
        n_ids = tok.encode_wait(stream)
    wall = time.perf_counter() - t0
    gc.enable()
    dev_ms = ev_a.elapsed_time(ev_b)
    # each call's device time: the same K calls again with an event between
    # calls, outside the timed region (an event between two queued calls
    # costs a few microseconds of its own)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for k in range(args.steps):
        if args.blocking:
            step()
        else:
            step_queued()
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    if not args.blocking:
        tok.encode_wait(stream)
    # the other way of calling, the same K calls, outside the timed region
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if args.blocking:
            step_queued()
        else:
            step()
    torch.cuda.synchronize()
    if args.blocking:
        tok.encode_wait(stream)
    other_wall = time.perf_counter() - t0
    gc.enable()
    two = two_requests_leg(tok, w, text, seg_off, allow, total, n_seg, ids, id_off, stream, args.steps)
    step_ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps))
    # per-kernel durations: the same K calls again with an event pair around
    # every kernel launch (same stream); kept out of the timed region above
    tok.set_timing(True)
    tok.timing_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rep = tok.timing_report()
    tok.set_timing(False)

    # ids of the last timed call, checked outside the timed region against
    # the oracle's (SHA-256 stored by tests/golden/alg_bytes.py)
    gpu_sha = ids_sha256(ids[:n_ids].cpu().numpy())

    ms_per_step = wall * 1e3 / args.steps
    mbs = total * args.steps / wall / 1e6
    tps = n_ids * args.steps / wall

    # context, outside the timed region: (1) the PCIe-inclusive rate, text
    # copied in from pinned host memory and ids copied back per call; (2) a
    # plain device-to-device copy of 256 MiB, the bandwidth one kernel can
    # actually move on this machine
    host_text = torch.empty(text.numel(), dtype=torch.uint8, pin_memory=True)
    host_text.copy_(text)
    host_ids = torch.empty(max(1, n_ids), dtype=torch.int32, pin_memory=True)
    e2e_steps = min(args.steps, 10)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(e2e_steps):
        text.copy_(host_text, non_blocking=True)
        step()
        host_ids[:n_ids].copy_(ids[:n_ids], non_blocking=True)
        torch.cuda.synchronize()
    e2e_ms = (time.perf_counter() - t0) * 1e3 / e2e_steps
    cp_src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * 5 * cp_src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cp_src, cp_dst

    # algorithmic bytes of the whole call and per kernel, counted once by the
    # oracle and stored (tests/golden/alg_bytes.py)
    with open(ALG_BYTES) as f:
        alg = json.load(f)[args.workload]
    assert alg["ids"] == n_ids and alg["bytes"] == total, "workload differs from the counted one"
    b_alg = alg["call_bytes"]
    floor_bytes = total + 4 * n_ids + 8 * (n_seg + 1) + tok.table_bytes
    per_kernel = {k: v[0] / max(1, v[1]) for k, v in rep.items()}
    # the dominant kernel: the longest one that carries at least 1% of the
    # call's algorithmic bytes (a kernel on the second stream that has
    # little to do is timed while it waits for the first stream's waves to
    # free CUs, as long as the kernel beside it)
    carrying = [k for k in rep if algorithmic_bytes(k, alg) >= 0.01 * b_alg] or list(rep)
    dom = max(carrying, key=lambda k: rep[k][0])
    dom_ms = per_kernel[dom]
    dom_bytes = algorithmic_bytes(dom, alg)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(mbs, 2),
        "unit": "MB/s",
        "tokens_per_s": round(tps, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "device_ms_per_step": round(dev_ms / args.steps, 4),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                    "max": round(step_ms[-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC.get(args.workload, args.workload),
                   "bytes": total, "segments": n_seg, "ids": n_ids, "ranks": len(w.tokens)},
        "call_roofline": {"alg_bytes": b_alg, "frac_of_8TBs": round(b_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                          "pieces": alg["pieces"], "table_bytes": alg["lookup_bytes"],
                          # compulsory bytes only: text in, ids and offsets out, the table read once
                          "floor_bytes": floor_bytes,
                          "floor_frac_of_8TBs": round(floor_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                          "copy_GBs": round(copy_gbs, 1),
                          "alg_frac_of_copy": round(b_alg / (ms_per_step * 1e-3) / 1e9 / copy_gbs, 5)},
        "calls": "blocking" if args.blocking else "queued",
        ("queued_calls" if args.blocking else "blocking_calls"): {
            "ms_per_step": round(other_wall * 1e3 / args.steps, 4),
            "MBs": round(total * args.steps / other_wall / 1e6, 2),
            "what": ("the same calls queued back to back, one wait at the end" if args.blocking else
                     "the same calls through the entry point that waits for each call's result")},
        "two_requests_in_flight": two,
        "pcie_inclusive": {"ms_per_step": round(e2e_ms, 4), "MBs": round(total / (e2e_ms * 1e-3) / 1e6, 2),
                           "steps": e2e_steps,
                           "what": "text host-to-device from pinned memory, encode, ids device-to-host"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": measured_traffic(args.workload, dom), "avg_ms": round(dom_ms, 5),
                     "alg_bytes_per_launch": dom_bytes},
        "kernels_avg_ms": {k: round(v, 5) for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1])},
        # every kernel's algorithmic rate against the same peak (the dominant
        # kernel by time above can be a latency-bound one carrying few bytes)
        "roofline_by_kernel": {k: {"alg_bytes": algorithmic_bytes(k, alg),
                                   "avg_ms": round(v, 5),
                                   "frac": round(algorithmic_bytes(k, alg) / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                                   "traffic": measured_traffic(args.workload, k)}
                               for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1])},
        "ids_sha256": gpu_sha,
        "ids_match_oracle": gpu_sha == alg.get("ids_sha256"),
    }
    out["first_call"] = first_call
    if args.workload == "main" and not args.no_warm_cache:
        out["warm_cache"] = warm_cache_leg(tok, w, text, seg_off, allow, total, ids, id_off, stream,
                                           alg.get("ids_sha256"))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
        out["ids_match_oracle"] = (out["ids_match_oracle"] and
                                   out["cpu_baseline"]["ids_sha256"] == gpu_sha)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
