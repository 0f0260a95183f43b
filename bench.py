"""Benchmark of the paged decode hot path on one MI355X.

A step is one layer's decode for 12 streams: paged_attn_decode_put (the new K/V row of each
stream written into its page slot, then the split-context part kernel and the merge) over
contexts uniform in [32768, 40960] with 8 KV / 64 query heads, head_dim 128, bf16, pages of
512 shuffled over the pool.  Inputs are resident in HBM before the timed region starts.

Before the timed region the step runs until the part kernel's time has settled (at least 150
launches, then the medians of three windows of ten launches within 2 % of each other, or a time
cap), independent of --warmup: the first tens of milliseconds of sustained load run at a lower
clock.  The settle is reported on its own.

Prints one JSON line: `value` is K/V bytes read per step over the measured step time (GB/s,
whole job), `roofline` compares the part kernel's average duration (HIP events recorded on
the kernel's stream around every launch in the timed region) with the 8 TB/s HBM peak, and
`cpu_baseline` times the float64 oracle on the same workloads; the same leg compares the
timed outputs of every workload with the oracle (`parity`).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged-attn decode µs/layer + K/V HBM GB/s (% peak), 12 streams x 40k ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "part_valu_d128_g8_batched_decode_traffic.json")
# the decode part kernel is built from these; counter figures taken on other sources are stale
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_rows_amd", "csrc", f)
                  for f in ("kernels_valu.hip", "device_common.h", "internal.h")]
PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_rows_amd", "libkvprobe.so")
FLUSH_BYTES = 1 << 30          # written before every cold call: evicts the 4 MB L2s and the 256 MB MALL
ATOL, REL_L2 = 2e-2, 1e-2      # parity bound: max-abs and relative L2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=2000.0,
                    help="cap on the settle phase before each timed region (ms of stepping)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the side measurements")
    ap.add_argument("--fixed-length", type=int, default=None, help="all 12 streams at this length")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--side-only", action="store_true",
                    help="run only the verify, wide-head, prompt and tiny workloads (for profiler runs)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="time the warm side workloads with plain launches instead of graph replays")
    ap.add_argument("--no-grid", action="store_true", help="skip the paged-vs-identity kernel grid")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("bytes_per_launch")


def stats_us(ms_list):
    """min / median / max / mean in µs of a list of ms."""
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"min": round(xs[0] * 1e3, 2), "median": round(med * 1e3, 2), "max": round(xs[-1] * 1e3, 2),
            "mean": round(sum(xs) / n * 1e3, 2), "n": n}


class DecodeSetup:
    def __init__(self, w, order_seed, torch, binding, staging, workloads, identity=False, contiguous=False):
        self.w = w
        self.torch = torch
        order = (workloads.identity_order(w.pool_pages) if identity or contiguous
                 else workloads.free_order(w.pool_pages, order_seed))
        if contiguous:
            # streams that grew side by side, a page each in turn, under the contiguous policy
            self.c = staging.make_cache(w, device="cuda", order=order, lease_policy=binding.KV_LEASE_CONTIGUOUS,
                                        grow_in_turn=1)
        else:
            self.c = staging.make_cache(w, device="cuda", order=order)
        self.ks, self.vs = workloads.kv_history(w, device="cuda")
        staging.write_history(self.c, self.ks, self.vs)
        self.q = workloads.queries(w, device="cuda")
        # the step's new rows are the last rows of each stream's history (rewritten in place)
        self.k_new = torch.stack([k[-1:] for k in self.ks]).contiguous()
        self.v_new = torch.stack([v[-1:] for v in self.vs]).contiguous()
        self.out = torch.empty_like(self.q)
        nbytes = binding.workspace_size(self.c.pool, self.c.table, self.c.seq_len, 1, w.q_heads,
                                        self.c.max_seq_len)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.binding = binding
        self.kv_bytes = sum(self.c.lengths) * w.kv_bytes_per_token

    fused = True

    def step(self):
        """One layer of the decode: the new row of each stream written into its page slot and
        attended, in one paged_attn_decode_put call (fused) or as kv_rows_put followed by
        paged_attn_decode (the same work and the same bytes)."""
        b, c = self.binding, self.c
        if self.fused:
            b.decode_put(c.pool, self.q, c.table, c.seq_len, c.max_seq_len, self.k_new, self.v_new,
                         out=self.out, workspace=self.ws)
        else:
            b.rows_put(c.pool, c.table, c.seq_len, self.k_new, self.v_new, c.max_seq_len)
            b.decode(c.pool, self.q, c.table, c.seq_len, c.max_seq_len, out=self.out, workspace=self.ws)

    def attention_only(self):
        c = self.c
        self.binding.decode(c.pool, self.q, c.table, c.seq_len, c.max_seq_len, out=self.out, workspace=self.ws)


def run_steps(setup, steps, torch, binding):
    """`steps` back-to-back steps with HIP events around every part-kernel launch: (wall ms per
    step, list of part-kernel ms)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in starts + stops:
        e.record()                      # materialise the underlying hipEvent_t
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        binding.set_part_events(starts[i].cuda_event, stops[i].cuda_event)
        setup.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    binding.set_part_events(None, None)
    return (t1 - t0) * 1e3 / steps, [starts[i].elapsed_time(stops[i]) for i in range(steps)]


def settle(setup, torch, binding, max_ms, window=10, windows=3, tol=1.02, min_steps=150):
    """Step in windows of `window` launches, at least min_steps launches (the shader clock is
    still ramping 40-80 launches into the load on some boxes, by 5-10 % per launch, in steps
    that can look flat over 30 launches), until the part kernel's median over each of the last
    `windows` windows agree within `tol` (max / min: the level has stopped moving), or until
    max_ms of stepping; returns the record of the phase."""
    times, meds = [], []
    t0 = time.perf_counter()
    reached = False
    while True:
        _, pm = run_steps(setup, window, torch, binding)
        times += pm
        meds.append(sorted(pm)[window // 2])
        last = meds[-windows:]
        if len(times) >= min_steps and len(last) == windows and max(last) <= tol * min(last):
            reached = True
            break
        if (time.perf_counter() - t0) * 1e3 > max_ms:
            break
    return {"steps": len(times), "wall_ms": round((time.perf_counter() - t0) * 1e3, 1), "reached": reached,
            "rule": f"at least {min_steps} launches, then medians of the last {windows} windows of {window} "
                    f"part-kernel launches within {round((tol - 1) * 100)} %, capped at {max_ms:.0f} ms",
            "part_us": [round(x * 1e3, 1) for x in times[:400]]}


def timed_steps(setup, steps, warmup, torch, binding, settle_ms):
    """Warmup steps, the settle phase, then exactly `steps` timed steps."""
    for _ in range(warmup):
        setup.step()
    torch.cuda.synchronize()
    st = settle(setup, torch, binding, settle_ms)
    ms_step, part = run_steps(setup, steps, torch, binding)
    return ms_step, part, st


def flush_buffer(torch):
    return torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")


def cold_calls(fn, iters, torch, flush, part=False, binding=None):
    """Event-timed calls of fn, each preceded by a FLUSH_BYTES write that evicts L2 and MALL;
    with part, also the part kernel alone (events the library records around it), in calls of
    their own that alternate with the whole-call ones: event records inside a timed call would
    add their own cost to it (about 7 µs for the two around the part kernel).  Returns (call ms
    list, part ms list or None)."""
    ms, pms = [], []
    for _ in range(iters):
        flush.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
        if part:
            flush.fill_(1)
            pa = torch.cuda.Event(enable_timing=True)
            pb = torch.cuda.Event(enable_timing=True)
            pa.record()
            pb.record()
            binding.set_part_events(pa.cuda_event, pb.cuda_event)
            fn()
            binding.set_part_events(None, None)
            torch.cuda.synchronize()
            pms.append(pa.elapsed_time(pb))
    return ms, (pms if part else None)


USE_GRAPHS = True


def graph_us(fn, torch, reps=20, iters=5, check=None):
    """Warm GPU time per fn() call in µs: `reps` calls captured into one HIP graph, replayed
    `iters` times between two events, so host-side launch cost does not show and the inputs
    stay in the caches between calls.  `check` (a tensor fn writes) is compared byte for byte
    between the eager call and the last replay.  With USE_GRAPHS off, the reps * iters calls
    are plain launches between the events."""
    if not USE_GRAPHS:
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps * iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (iters * reps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = check.clone() if check is not None else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    if check is not None and not torch.equal(eager.view(torch.int16), check.view(torch.int16)):
        raise RuntimeError("graph replay differs from the eager call")
    del g
    return a.elapsed_time(b) * 1e3 / (iters * reps)


def attn_flops(lengths, rows, q_heads, head_dim, window=0):
    """Multiply-adds of QK^T and PV, counted as 2 flops each, over the keys each row sees."""
    total = 0
    for L in lengths:
        for r in range(rows):
            p = L - rows + r
            lo = 0 if window <= 0 else max(0, p - window + 1)
            total += max(0, p + 1 - lo)
    return 4 * total * q_heads * head_dim


def visible_kv_bytes(lengths, rows, window, kv_bytes_per_token):
    """K/V bytes a call must read: every position some row of the stream sees, once."""
    total = 0
    for L in lengths:
        lo = 0 if window <= 0 else max(0, L - rows - window + 1)
        total += max(0, L - lo)
    return total * kv_bytes_per_token


def read_ceiling(torch, setup, flush, iters=10, grid=2048):
    """The HBM read rate of a plain streaming read (libkvprobe.so) over the headline's K and V
    page arrays, each call after the same flush as the cold attention calls."""
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kvprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvprobe_read.restype = ctypes.c_int
    k, v = setup.c.pool.k_pages, setup.c.pool.v_pages
    nbytes = k.numel() * 2
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def probe():
        for t in (k, v):
            rc = lib.kvprobe_read(t.data_ptr(), nbytes, grid, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"kvprobe_read failed: {rc}")
    probe()
    ms, _ = cold_calls(probe, iters, torch, flush)
    st = stats_us(ms)
    return {"GBps_median": round(2 * nbytes / (st["median"] * 1e-6) / 1e9, 1),
            "GBps_best": round(2 * nbytes / (st["min"] * 1e-6) / 1e9, 1),
            "bytes": 2 * nbytes, "us": st,
            "note": f"one streaming read of the K and V page arrays ({grid} workgroups, 16-byte nontemporal "
                    f"loads), a 1 GiB flush before each of {iters} calls"}


_READ_BUF = {}


def same_size_read(torch, nbytes, flush, iters=10, grids=(512, 1024, 2048, 4096)):
    """The cold read rate of a plain streaming read (libkvprobe.so) of `nbytes` contiguous bytes,
    timed as the cold attention calls are (a flush before each call, events around it): the
    best median over a few grid sizes.  At tens of MB the launch, the first round trips and the
    drain weigh on any kernel, so this, not the long-read ceiling, is what a workload of that
    size can approach."""
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kvprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvprobe_read.restype = ctypes.c_int
    n = nbytes // 16 * 16
    if _READ_BUF.get("t") is None or _READ_BUF["t"].numel() * 2 < n:
        _READ_BUF["t"] = None
        _READ_BUF["t"] = torch.ones((n + 1) // 2, dtype=torch.int16, device="cuda")
    buf = _READ_BUF["t"]
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for grid in grids:
        sink = torch.zeros(grid, dtype=torch.int32, device="cuda")

        def probe():
            rc = lib.kvprobe_read(buf.data_ptr(), n, grid, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"kvprobe_read failed: {rc}")
        probe()
        ms, _ = cold_calls(probe, iters, torch, flush)
        med = stats_us(ms)["median"]
        if best is None or med < best[0]:
            best = (med, grid)
    return {"us": round(best[0], 2), "GBps": round(n / (best[0] * 1e-6) / 1e9, 1), "grid": best[1]}


def cold_record(ms, kv_bytes, flops=None, part_ms=None):
    st = stats_us(ms)
    rec = {"cold_us": st, "cold_kv_GBps": round(kv_bytes / (st["median"] * 1e-6) / 1e9, 1),
           "cold_hbm_frac": round(kv_bytes / (st["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if part_ms is not None:
        ps = stats_us(part_ms)
        rec["cold_part_us"] = ps
        rec["cold_part_hbm_frac"] = round(kv_bytes / (ps["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if flops:
        rec["cold_TFLOPs"] = round(flops / (st["median"] * 1e-6) / 1e12, 2)
        rec["cold_mfma_frac"] = round(flops / (st["median"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    return rec


def other_workloads(torch, binding, staging, workloads, flush, cases):
    """The tiny decode, the verify window (causal and as draft trees), the wide-head pair, the
    head-dim-256 pair and the prompt chunks: warm GPU time per call (HIP graph replays; inputs
    stay in the caches) and cold time per call (a 1 GiB flush before each call, HIP events
    around it).  Appends to `cases` what the oracle leg needs to check each workload's output."""
    import numpy as np
    res = {}
    iters = 20

    def vs_read(rec, nbytes):
        """rec plus the same-size streaming read and the cold times' rate as a fraction of it"""
        ceil = same_size_read(torch, nbytes, flush)
        rec["same_size_read"] = ceil
        rec["cold_vs_read"] = round(ceil["us"] / rec["cold_us"]["median"], 3)
        if "cold_part_us" in rec:
            rec["cold_part_vs_read"] = round(ceil["us"] / rec["cold_part_us"]["median"], 3)
        return rec

    # tiny decode: 1 stream, 300 keys in pages of 64 (5 of an 8-page pool)
    w = workloads.tiny_decode()
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3001))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    q = workloads.queries(w, device="cuda")
    out = torch.empty_like(q)
    call = lambda: binding.decode(c.pool, q, c.table, c.seq_len, c.max_seq_len, out=out)
    warm = graph_us(call, torch, check=out)
    ms, _ = cold_calls(call, iters, torch, flush)
    by = sum(c.lengths) * w.kv_bytes_per_token
    res["tiny_decode_300"] = vs_read({"warm_us": round(warm, 2), "kv_bytes": by, **cold_record(ms, by)}, by)
    cases.append({"name": "tiny_decode_300", "q": q, "ks": ks, "vs": vs, "lengths": c.lengths, "window": 0,
                  "out": out.clone()})

    # speculative verify window: 4 streams x 8 rows x ~9k, GQA 8 (MFMA path)
    w = workloads.verify_window()
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3003))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    q = workloads.queries(w, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(binding.workspace_size(c.pool, c.table, c.seq_len, w.rows, w.q_heads, c.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    call = lambda: binding.verify(c.pool, q, c.table, c.seq_len, c.max_seq_len, out=out, workspace=ws)
    warm = graph_us(call, torch, check=out)
    ms, pms = cold_calls(call, iters, torch, flush, part=True, binding=binding)
    by = sum(c.lengths) * w.kv_bytes_per_token
    fl = attn_flops(c.lengths, w.rows, w.q_heads, w.head_dim)
    res["verify_window_4x8rows_9k"] = vs_read({"warm_us": round(warm, 2),
                                               "warm_kv_GBps": round(by / warm / 1e3, 1),
                                               "warm_TFLOPs": round(fl / warm / 1e6, 2),
                                               "kv_bytes": by, "flops": fl, **cold_record(ms, by, fl, pms)}, by)
    cases.append({"name": "verify_window_4x8rows_9k", "q": q, "ks": ks, "vs": vs, "lengths": c.lengths,
                  "window": 0, "out": out.clone()})
    # the same window as a flattened draft tree (seeded random trees, parents before children)
    rng = np.random.default_rng(3103)
    masks = np.zeros((w.streams, w.rows), dtype=np.int32)
    for s_ in range(w.streams):
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, w.rows)]
        for r in range(w.rows):
            m, i = 0, r
            while i >= 0:
                m |= 1 << i
                i = parent[i]
            masks[s_, r] = m
    tm = torch.from_numpy(masks).to("cuda")
    out_t = torch.empty_like(q)
    call = lambda: binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, tm, out=out_t, workspace=ws)
    warm = graph_us(call, torch, check=out_t)
    ms, _ = cold_calls(call, iters, torch, flush)
    res["verify_tree_4x8rows_9k"] = vs_read({"warm_us": round(warm, 2), **cold_record(ms, by)}, by)
    cases.append({"name": "verify_tree_4x8rows_9k", "q": q, "ks": ks, "vs": vs, "lengths": c.lengths,
                  "window": 0, "masks": masks, "out": out_t.clone()})

    # wide head: d 512, pages of 37; stream 0 decodes at 2048, stream 1 verifies 4 rows at 9000
    w = workloads.wide_head()
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3004))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    q0 = workloads.normal_bf16((1, 1, w.q_heads, 512), 4101, "cuda")
    q1 = workloads.normal_bf16((1, 4, w.q_heads, 512), 4102, "cuda")
    t0, l0 = c.stream_view(0)
    t1, l1 = c.stream_view(1)
    o0, o1 = torch.empty_like(q0), torch.empty_like(q1)
    call0 = lambda: binding.decode(c.pool, q0, t0, l0, c.lengths[0], out=o0)
    call1 = lambda: binding.verify(c.pool, q1, t1, l1, c.lengths[1], out=o1)
    w0 = graph_us(call0, torch, check=o0)
    w1 = graph_us(call1, torch, check=o1)
    ms0, p0 = cold_calls(call0, iters, torch, flush, part=True, binding=binding)
    ms1, p1 = cold_calls(call1, iters, torch, flush, part=True, binding=binding)
    b0, b1 = c.lengths[0] * w.kv_bytes_per_token, c.lengths[1] * w.kv_bytes_per_token
    res["wide_head_d512_p37"] = {
        "decode_2048": vs_read({"warm_us": round(w0, 2), "kv_bytes": b0, **cold_record(ms0, b0, None, p0)}, b0),
        "verify4_9000": vs_read({"warm_us": round(w1, 2), "kv_bytes": b1,
                                 **cold_record(ms1, b1, attn_flops([9000], 4, w.q_heads, 512), p1)}, b1)}
    cases.append({"name": "wide_head_decode_2048", "q": q0, "ks": ks[:1], "vs": vs[:1], "lengths": c.lengths[:1],
                  "window": 0, "out": o0.clone()})
    cases.append({"name": "wide_head_verify4_9000", "q": q1, "ks": ks[1:], "vs": vs[1:], "lengths": c.lengths[1:],
                  "window": 0, "out": o1.clone()})

    # head dim 256: 4 streams x 16,384 keys, 4 KV heads x GQA 8, pages of 512; a decode (VALU)
    # and a 4-row verify window (MFMA), 268 MB of K/V
    w = workloads.Workload("head_dim_256", streams=4, kv_heads=4, group=8, head_dim=256, page_size=512, rows=4,
                           lengths=[16384] * 4, spare_frac=0.10, seed=1006)
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3007))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    qd = workloads.normal_bf16((4, 1, w.q_heads, 256), 4104, "cuda")
    qv = workloads.normal_bf16((4, 4, w.q_heads, 256), 4105, "cuda")
    od, ov = torch.empty_like(qd), torch.empty_like(qv)
    calld = lambda: binding.decode(c.pool, qd, c.table, c.seq_len, c.max_seq_len, out=od)
    callv = lambda: binding.verify(c.pool, qv, c.table, c.seq_len, c.max_seq_len, out=ov)
    wd = graph_us(calld, torch, check=od)
    wv = graph_us(callv, torch, check=ov)
    msd, pd = cold_calls(calld, iters, torch, flush, part=True, binding=binding)
    msv, pv = cold_calls(callv, iters, torch, flush, part=True, binding=binding)
    b = sum(c.lengths) * w.kv_bytes_per_token
    res["head_dim_256"] = {
        "decode_4x16384": vs_read({"warm_us": round(wd, 2), "kv_bytes": b, **cold_record(msd, b, None, pd)}, b),
        "verify4_4x16384": vs_read({"warm_us": round(wv, 2), "kv_bytes": b,
                                    **cold_record(msv, b, attn_flops(c.lengths, 4, w.q_heads, 256), pv)}, b)}
    cases.append({"name": "head_dim_256_decode", "q": qd, "ks": ks, "vs": vs, "lengths": c.lengths, "window": 0,
                  "out": od.clone()})
    cases.append({"name": "head_dim_256_verify4", "q": qv, "ks": ks, "vs": vs, "lengths": c.lengths, "window": 0,
                  "out": ov.clone()})

    # prompt: 2048 tokens in 4 chunks of 512 rows, full layer and sliding layer (window 1024, ring)
    for window in (0, 1024):
        w = workloads.prefill_mixed(window=window)
        c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3005), lengths=[2048])
        ks, vs = workloads.kv_history(w, device="cuda")
        qa = workloads.normal_bf16((1, 2048, w.q_heads, w.head_dim), 77, "cuda")
        seqs = [torch.tensor([c0 + 512], dtype=torch.int32, device="cuda") for c0 in range(0, 2048, 512)]
        kn = [ks[0][c0:c0 + 512][None].contiguous() for c0 in range(0, 2048, 512)]
        vn = [vs[0][c0:c0 + 512][None].contiguous() for c0 in range(0, 2048, 512)]
        qs = [qa[:, c0:c0 + 512].contiguous() for c0 in range(0, 2048, 512)]
        outs = [torch.empty_like(x) for x in qs]

        def prompt():
            for i in range(4):
                binding.rows_put(c.pool, c.table, seqs[i], kn[i], vn[i], 2048, ring_pages=c.ring_pages)
                binding.prefill(c.pool, qs[i], c.table, seqs[i], 2048, window=window, ring_pages=c.ring_pages,
                                out=outs[i])
        warm = graph_us(prompt, torch, reps=5, check=outs[3])
        ms, _ = cold_calls(prompt, iters, torch, flush)
        fl = sum(attn_flops([c0 + 512], 512, w.q_heads, w.head_dim, window) for c0 in range(0, 2048, 512))
        by = sum(visible_kv_bytes([c0 + 512], 512, window, w.kv_bytes_per_token) for c0 in range(0, 2048, 512))
        name = "prefill_2048_in_512_chunks" + ("_window1024_ring" if window else "_full")
        res[name] = {"warm_us": round(warm, 2), "warm_us_per_chunk": round(warm / 4, 2),
                     "warm_TFLOPs": round(fl / warm / 1e6, 2),
                     "warm_mfma_frac": round(fl / warm / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl,
                     "kv_bytes": by, **cold_record(ms, by, fl)}
        for i, c0 in enumerate(range(0, 2048, 512)):
            cases.append({"name": f"{name}_chunk{i}", "q": qs[i], "ks": ks, "vs": vs, "lengths": [c0 + 512],
                          "window": window, "out": outs[i].clone(), "group": name})

        # the same prompt with each chunk's row write fused into its prefill (one launch per
        # chunk); the rows it writes are the ones already there, byte for byte
        outs_f = [torch.empty_like(x) for x in qs]

        def prompt_fused():
            for i in range(4):
                binding.prefill_put(c.pool, qs[i], c.table, seqs[i], 2048, kn[i], vn[i], window=window,
                                    ring_pages=c.ring_pages, out=outs_f[i])
        warm_f = graph_us(prompt_fused, torch, reps=5, check=outs_f[3])
        ms_f, _ = cold_calls(prompt_fused, iters, torch, flush)
        res[name + "_fused_row_writes"] = {
            "warm_us": round(warm_f, 2), "warm_us_per_chunk": round(warm_f / 4, 2),
            "warm_TFLOPs": round(fl / warm_f / 1e6, 2),
            "warm_mfma_frac": round(fl / warm_f / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl,
            "kv_bytes": by, **cold_record(ms_f, by, fl),
            "entry": "paged_attn_prefill_put per chunk (kv_rows_put + paged_attn_prefill in one launch)"}
        for i, c0 in enumerate(range(0, 2048, 512)):
            cases.append({"name": f"{name}_fused_chunk{i}", "q": qs[i], "ks": ks, "vs": vs, "lengths": [c0 + 512],
                          "window": window, "out": outs_f[i].clone(), "group": name + "_fused_row_writes"})
    _READ_BUF.clear()
    return res


def pages_grid(torch, binding, workloads, flush, iters=15):
    """Kernel-alone timing, paged against the identity table, cold (TensorFold PR #1620, the
    author's per-tile follow-up): 48/4 heads at d 128 over pages of 512 at 2k/9k/32k keys and
    1/4/12 rows, the paged arm's pages spread over a 20,000-page arena; and 16/1 heads at d 512
    at 9k and 32k keys with 4 rows.  One stream per call.  R = 1 runs paged_attn_decode, R = 4
    paged_attn_verify, R = 12 paged_attn_prefill (a verify window holds at most 8 rows)."""
    import numpy as np
    cells = []
    geoms = [(4, 12, 128, [2048, 9000, 32768], [1, 4, 12]), (1, 16, 512, [9000, 32768], [4])]
    for Hkv, G, D, lens, rows_list in geoms:
        P, arena = 512, 20000
        pool = binding.Pool(arena, P, Hkv, D, max_streams=1)
        dev = pool.k_pages.device
        for L in lens:
            n = -(-L // P)
            rng = np.random.default_rng(L * 7 + D)
            paged_ids = (n + rng.permutation(arena - n)[:n]).astype(np.int32)   # spread over the arena
            ident_ids = np.arange(n, dtype=np.int32)
            w = workloads.Workload(name="grid", streams=1, kv_heads=Hkv, group=G, head_dim=D, page_size=P, rows=1,
                                   lengths=[L], spare_frac=0.0, seed=1200 + L % 1000 + D)
            ks, vs = workloads.kv_history(w, device="cuda")
            tables = {}
            for arm, ids in (("paged", paged_ids), ("identity", ident_ids)):
                t = torch.tensor(ids[None], dtype=torch.int32, device=dev)
                for c0 in range(0, L, 8192):
                    c1 = min(L, c0 + 8192)
                    binding.rows_put(pool, t, torch.tensor([c1], dtype=torch.int32, device=dev),
                                     ks[0][c0:c1][None].contiguous(), vs[0][c0:c1][None].contiguous(), c1)
                tables[arm] = t
            seq = torch.tensor([L], dtype=torch.int32, device=dev)
            for R in rows_list:
                q = workloads.normal_bf16((1, R, Hkv * G, D), 1300 + R, "cuda")
                fn = binding.decode if R == 1 else (binding.verify if R <= 8 else binding.prefill)
                outs = {arm: torch.empty_like(q) for arm in tables}
                ws = torch.empty(max(256, binding.workspace_size(pool, tables["paged"], seq, R, Hkv * G, L)),
                                 dtype=torch.uint8, device=dev)
                calls = {arm: (lambda a=arm: fn(pool, q, tables[a], seq, L, out=outs[a], workspace=ws))
                         for arm in tables}
                for a in calls:
                    calls[a]()
                torch.cuda.synchronize()
                # the arms alternate, call by call
                ms = {a: [] for a in calls}
                pm = {a: [] for a in calls}
                for _ in range(iters):
                    for a in calls:
                        m, p = cold_calls(calls[a], 1, torch, flush, part=True, binding=binding)
                        ms[a] += m
                        pm[a] += p
                same = bool(torch.equal(outs["paged"].view(torch.int16), outs["identity"].view(torch.int16)))
                med = {a: stats_us(ms[a])["median"] for a in ms}
                pmed = {a: stats_us(pm[a])["median"] for a in pm}
                cells.append({"heads": f"{Hkv * G}/{Hkv}", "head_dim": D, "keys": L, "rows": R,
                              "entry": fn.__name__, "paged_us": med["paged"], "identity_us": med["identity"],
                              "paged_over_identity": round(med["paged"] / med["identity"], 4),
                              "part_paged_over_identity": round(pmed["paged"] / pmed["identity"], 4),
                              "bytes_equal": same})
                log(f"[bench] grid {Hkv * G}/{Hkv} d{D} {L} keys x {R} rows: paged {med['paged']:.1f} us, "
                    f"identity {med['identity']:.1f} us")
            del ks, vs, tables
        pool.close()
        del pool
        torch.cuda.empty_cache()
    return {"cells": cells, "arena_pages": 20000, "page_size": 512,
            "note": "one stream per call; cold (1 GiB flush before each call); arms alternate call by call; "
                    f"medians of {iters}; paged pages drawn at random from a 20,000-page arena"}


def kept_state_copy(setup, torch, binding, iters=20):
    """Keep the state of the longest stream: copy its pages onto spare pages of the pool
    (kv_pages_copy), timed with HIP events; the copy reads and writes every byte once."""
    import numpy as np
    c, w = setup.c, setup.w
    s = int(np.argmax(c.lengths))
    n = -(-c.lengths[s] // w.page_size)
    used = set(int(x) for x in c.table_host[c.table_host >= 0].ravel())
    spare = [i for i in range(w.pool_pages) if i not in used][:n]
    if len(spare) < n:
        return None
    src = torch.tensor(c.table_host[s][:n], dtype=torch.int32, device="cuda")
    dst = torch.tensor(spare, dtype=torch.int32, device="cuda")
    binding.pages_copy(c.pool, src, dst)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        binding.pages_copy(c.pool, src, dst)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / iters
    moved = 2 * n * 2 * w.kv_heads * w.page_size * w.head_dim * 2       # K and V, read and written
    return {"stream_tokens": c.lengths[s], "pages": n, "bytes_moved": moved, "us": round(us, 2),
            "GBps": round(moved / us / 1e3, 1)}


def calibration_copy(torch, nbytes=1 << 30, reps=3):
    """An elementwise kernel of known traffic (reads nbytes, writes nbytes: bitwise_not over
    int32), so that profiler byte counters can be scaled against it.  A plain copy_ may go to
    the DMA engines, which kernel counters do not see."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def oracle_leg(cases, oracle, workloads, reps=3):
    """The float64 oracle, as it stands, on every workload case: each case's streams widened
    from the generator's bf16 values and attended (causal, windowed or tree-shaped), `reps`
    times; returns per-case median seconds and the comparison with the GPU output that the
    timed run produced (max-abs and relative L2, whole output and worst stream)."""
    import numpy as np
    timing, parity = {}, {}
    for case in cases:
        qb = workloads.bf16_bits(case["q"])
        kh = [workloads.bf16_bits(k[:L]) for k, L in zip(case["ks"], case["lengths"])]
        vh = [workloads.bf16_bits(v[:L]) for v, L in zip(case["vs"], case["lengths"])]
        got = oracle.bf16_bits_to_f64(workloads.bf16_bits(case["out"]))
        secs = []
        for _ in range(reps):
            t0 = time.perf_counter()
            ref = []
            for s, L in enumerate(case["lengths"]):
                q = oracle.bf16_bits_to_f64(qb[s])
                k = oracle.bf16_bits_to_f64(kh[s])
                v = oracle.bf16_bits_to_f64(vh[s])
                if "masks" in case:
                    ref.append(oracle.attend_stream_tree(q, k, v, q.shape[0], [int(m) for m in case["masks"][s]],
                                                         case["window"], length=L))
                else:
                    ref.append(oracle.attend_stream(q, k, v, q.shape[0], case["window"], length=L))
            secs.append(time.perf_counter() - t0)
        ref = np.stack(ref)
        finite = bool(np.isfinite(got).all())
        d = got - ref
        nr = float(np.linalg.norm(ref))
        rel = float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d) > 0)
        per = [float(np.linalg.norm(d[s]) / max(float(np.linalg.norm(ref[s])), 1e-300)) for s in range(ref.shape[0])]
        mx = float(np.abs(d).max())
        group = case.get("group", case["name"])
        prev = parity.get(group)
        rec = {"max_abs": mx, "rel_l2": rel, "worst_stream_rel_l2": max(per), "finite": finite}
        if prev:      # a prompt's chunks are one record: the worst of them
            rec = {"max_abs": max(prev["max_abs"], mx), "rel_l2": max(prev["rel_l2"], rel),
                   "worst_stream_rel_l2": max(prev["worst_stream_rel_l2"], max(per)),
                   "finite": prev["finite"] and finite}
        parity[group] = rec
        timing[group] = timing.get(group, 0.0) + sorted(secs)[len(secs) // 2]
    for rec in parity.values():
        rec["ok"] = bool(rec["finite"] and rec["max_abs"] <= ATOL and rec["rel_l2"] <= REL_L2
                         and rec["worst_stream_rel_l2"] <= REL_L2)
        for k in ("max_abs", "rel_l2", "worst_stream_rel_l2"):
            rec[k] = float(f"{rec[k]:.3e}")
    return timing, parity


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the paged decode "
              "runs per GPU on its own streams); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_rows_amd import binding, staging, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    torch.cuda.set_device(0)
    global USE_GRAPHS
    USE_GRAPHS = not args.no_graphs
    flush = flush_buffer(torch)
    cases = []
    if args.side_only:
        log("[bench] side workloads only")
        res = {"side_only": True, "graphs": USE_GRAPHS,
               "other_workloads": other_workloads(torch, binding, staging, workloads, flush, cases)}
        if args.calib_copy:
            log("[bench] calibration copy")
            calibration_copy(torch)
        print(json.dumps(res), flush=True)
        return

    w = workloads.batched_decode(fixed_length=args.fixed_length)
    log(f"[bench] building {w.name}: lengths {w.lengths}, pool {w.pool_pages} pages")
    setup = DecodeSetup(w, 3002, torch, binding, staging, workloads)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps, settle, {args.steps} timed steps")
    ms_step, part_ms, settled = timed_steps(setup, args.steps, args.warmup, torch, binding, args.settle_ms)
    timed_out = setup.out.clone()
    part = stats_us(part_ms)
    value = setup.kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = setup.kv_bytes / (part["mean"] * 1e-6) / 1e9
    traffic = measured_traffic()
    log(f"[bench] settle: {settled['steps']} steps ({settled['wall_ms']} ms, reached {settled['reached']})")
    log(f"[bench] {ms_step * 1e3:.1f} us/step, part kernel mean {part['mean']:.1f} us "
        f"(median {part['median']:.1f}), {achieved:.0f} GB/s")
    cases.append({"name": "batched_decode", "q": setup.q, "ks": setup.ks, "vs": setup.vs, "lengths": setup.c.lengths,
                  "window": 0, "out": timed_out})
    # the same step as two calls (kv_rows_put, then paged_attn_decode), in interleaved rounds
    # with the fused call
    fused_ms, unfused_ms = [], []
    for _ in range(3):
        for fused, acc in ((True, fused_ms), (False, unfused_ms)):
            setup.fused = fused
            acc.append(run_steps(setup, 30, torch, binding)[0])
    setup.fused = True

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: 12 streams, contexts U[32768, 40960] (seed 2002), 8 KV / 64 query "
                        f"heads, head_dim 128, bf16 K/V, pages of 512 shuffled over a pool with 10% NaN "
                        f"spares; step = paged_attn_decode_put (the new row of each stream written into its "
                        f"page and attended, one call)"
            if args.fixed_length is None else
            f"{w.name}: 12 streams x {args.fixed_length}, otherwise as the batched decode",
            "streams": w.streams, "kv_heads": w.kv_heads, "q_heads": w.q_heads, "head_dim": w.head_dim,
            "page_size": w.page_size, "rows": 1, "lengths": w.lengths,
            "kv_bytes_per_step": setup.kv_bytes,
        },
        "us_per_layer": round(ms_step * 1e3, 2),
        "settle": settled,
        "two_call_step": {"us_per_layer": round(sorted(unfused_ms)[1] * 1e3, 2),
                          "fused_us_per_layer": round(sorted(fused_ms)[1] * 1e3, 2),
                          "note": "kv_rows_put + paged_attn_decode against paged_attn_decode_put, medians of "
                                  "3 interleaved rounds of 30 steps"},
        "roofline": {
            "bound": "hbm", "kernel": "part_valu_kernel<128,8,8>",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "part_us_mean": part["mean"], "part_us_median": part["median"], "part_us_min": part["min"],
            "part_us_max": part["max"],
            "frac_at_median": round(setup.kv_bytes / (part["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }

    if not args.quick:
        log("[bench] cold-cache calls (1 GiB flush before each)")
        ms, pms = cold_calls(setup.attention_only, 20, torch, flush, part=True, binding=binding)
        result["cold_attention"] = cold_record(ms, setup.kv_bytes, None, pms)
        log("[bench] read ceiling")
        ceiling = read_ceiling(torch, setup, flush)
        result["read_ceiling"] = ceiling
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["GBps_median"], 4)
        # the page layouts are timed in interleaved rounds, so that a drift of the clock over
        # the run falls on every arm alike
        log("[bench] page layouts: shuffled, identity table, contiguous leases (interleaved)")
        lin = DecodeSetup(w, 0, torch, binding, staging, workloads, identity=True)
        cg = DecodeSetup(w, 0, torch, binding, staging, workloads, contiguous=True)
        arms = {"shuffled": setup, "identity": lin, "contiguous": cg}
        parts = {k: [] for k in arms}
        stepms = {k: [] for k in arms}
        for _ in range(4):
            for name, st in arms.items():
                sms, pms = run_steps(st, 25, torch, binding)
                parts[name].append(stats_us(pms)["median"])
                stepms[name].append(sms * 1e3)
        med = lambda xs: sorted(xs)[len(xs) // 2]
        runs = [1 + int((np.diff(cg.c.table_host[s][:w.pages_for(L)]) != 1).sum()) for s, L in enumerate(w.lengths)]
        result["identity_table"] = {"us_per_layer": round(med(stepms["identity"]), 2),
                                    "part_us_median": round(med(parts["identity"]), 2),
                                    "shuffled_part_us_median": round(med(parts["shuffled"]), 2),
                                    "paged_over_identity": round(med(parts["shuffled"]) / med(parts["identity"]), 4),
                                    "rounds": "4 interleaved rounds of 25 steps per arm"}
        result["contiguous_leases"] = {"us_per_layer": round(med(stepms["contiguous"]), 2),
                                       "part_us_median": round(med(parts["contiguous"]), 2),
                                       "paged_over_contiguous": round(med(parts["shuffled"]) / med(parts["contiguous"]), 4),
                                       "runs_per_stream": runs,
                                       "bytes_equal": bool(torch.equal(cg.out.view(torch.int16),
                                                                       setup.out.view(torch.int16)))}
        del cg
        torch.cuda.empty_cache()
        log("[bench] kept-state page copy")
        result["kept_state_copy"] = kept_state_copy(setup, torch, binding)
        same = torch.equal(lin.out.view(torch.int16), setup.out.view(torch.int16))
        result["identity_table"]["bytes_equal"] = bool(same)
        del lin
        torch.cuda.empty_cache()
        if args.fixed_length is None:
            log("[bench] fixed 12 x 40960 variant")
            wf = workloads.batched_decode(fixed_length=40960)
            fx = DecodeSetup(wf, 3002, torch, binding, staging, workloads)
            fms, fpart, fst = timed_steps(fx, max(20, args.steps // 4), 5, torch, binding, args.settle_ms)
            fp = stats_us(fpart)
            result["fixed_12x40960"] = {"us_per_layer": round(fms * 1e3, 2), "part_us_mean": fp["mean"],
                                        "part_us_median": fp["median"],
                                        "kv_GBps": round(fx.kv_bytes / (fms * 1e-3) / 1e9, 1),
                                        "part_kv_GBps": round(fx.kv_bytes / (fp["mean"] * 1e-6) / 1e9, 1),
                                        "part_hbm_frac": round(fx.kv_bytes / (fp["mean"] * 1e-6) / 1e9 /
                                                               HBM_PEAK_GBS, 4),
                                        "settle_steps": fst["steps"], "settle_reached": fst["reached"]}
            del fx
            torch.cuda.empty_cache()
        log("[bench] tiny, verify window, wide head and prompt workloads (warm and cold)")
        result["other_workloads"] = other_workloads(torch, binding, staging, workloads, flush, cases)
        if not args.no_grid:
            log("[bench] paged-vs-identity kernel grid (cold)")
            result["pages_grid"] = pages_grid(torch, binding, workloads, flush)
    if args.calib_copy:
        log("[bench] calibration copy")
        calibration_copy(torch)

    if not args.no_cpu_baseline:
        import oracle          # the CPU reference, used by this leg only
        log("[bench] cpu baseline: the oracle on every workload, and parity of the timed outputs")
        timing, parity = oracle_leg(cases, oracle, workloads)
        cores = len(os.sched_getaffinity(0))
        secs = timing["batched_decode"]
        result["cpu_baseline"] = {
            "value": round(setup.kv_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle (widen the bf16 history + attend) on all 12 streams of the batched decode "
                      f"({setup.kv_bytes / 1e9:.3f} GB of K/V), median of 3 passes of {secs:.2f} s; numpy/BLAS "
                      f"threads: all {cores} cores; host {platform.processor() or platform.machine()}",
            "seconds_per_config": {k: round(v, 4) for k, v in timing.items()}}
        result["parity"] = {"bound": f"finite, max_abs <= {ATOL}, rel_l2 <= {REL_L2} over the output and per "
                                     f"stream (oracle: float64 from the generator's bf16 inputs)", **parity}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
