"""Benchmark of the paged decode hot path on one MI355X.

A step is one layer's decode for 12 streams: kv_rows_put of each stream's new K/V row, then
paged_attn_decode (split-context part kernel + merge) over contexts uniform in
[32768, 40960] with 8 KV / 64 query heads, head_dim 128, bf16, pages of 512 shuffled over the
pool.  Inputs are resident in HBM before the timed region starts.

Prints one JSON line: `value` is K/V bytes read per step over the measured step time (GB/s,
whole job), `roofline` compares the part kernel's average duration (HIP events recorded on
the kernel's stream around every launch in the timed region) with the 8 TB/s HBM peak, and
`cpu_baseline` times the float64 oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged-attn decode µs/layer + K/V HBM GB/s (% peak), 12 streams x 40k ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "part_valu_d128_g8_batched_decode_traffic.json")
# the decode part kernel is built from these; counter figures taken on other sources are stale
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_rows_amd", "csrc", f)
                  for f in ("kernels_valu.hip", "device_common.h", "internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 100 steps (about 30 ms): the first 10-15 ms of sustained load run through a clock transient
    # (part kernel 320-370 us against about 300 us after it)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the side measurements")
    ap.add_argument("--fixed-length", type=int, default=None, help="all 12 streams at this length")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--side-only", action="store_true",
                    help="run only the verify, wide-head and prompt workloads (for profiler runs)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="time the side workloads with plain launches instead of graph replays")
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


def timed_steps(setup, steps, warmup, torch, binding):
    """Wall time per step over `steps` back-to-back steps, and the part kernel's average
    duration from HIP events recorded around each of its launches."""
    for _ in range(warmup):
        setup.step()
    torch.cuda.synchronize()
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
    part_ms = [starts[i].elapsed_time(stops[i]) for i in range(steps)]
    return (t1 - t0) * 1e3 / steps, sum(part_ms) / steps, min(part_ms), max(part_ms)


def cold_calls(setup, iters, torch):
    """Event-timed attention calls each preceded by a 1 GiB write that evicts L2 and MALL."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ms = []
    for _ in range(iters):
        flush.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        setup.attention_only()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2]


USE_GRAPHS = True


def graph_us(fn, torch, reps=20, iters=5, check=None):
    """GPU time per fn() call in µs: `reps` calls captured into one HIP graph, replayed `iters`
    times between two events, so host-side launch cost does not show.  `check` (a tensor fn
    writes) is compared byte for byte between the eager call and the last replay.  With
    USE_GRAPHS off, the reps * iters calls are plain launches between the events."""
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
            total += (p + 1 - lo)
    return 4 * total * q_heads * head_dim


MFMA_BF16_PEAK_TFLOPS = 2500.0


def other_workloads(torch, binding, staging, workloads):
    """The verify window (causal and as a draft tree), the wide-head pair and the prompt chunks,
    timed on their own as GPU time per call (HIP graph replays, so host launch cost does not
    show)."""
    import numpy as np
    res = {}
    # speculative verify window: 4 streams x 8 rows x ~9k, GQA 8 (MFMA path)
    w = workloads.verify_window()
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3003))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    q = workloads.queries(w, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(binding.workspace_size(c.pool, c.table, c.seq_len, w.rows, w.q_heads, c.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    us = graph_us(lambda: binding.verify(c.pool, q, c.table, c.seq_len, c.max_seq_len, out=out, workspace=ws),
                  torch, check=out)
    by = sum(c.lengths) * w.kv_bytes_per_token
    fl = attn_flops(c.lengths, w.rows, w.q_heads, w.head_dim)
    res["verify_window_4x8rows_9k"] = {"us": round(us, 2), "kv_GBps": round(by / us / 1e3, 1),
                                       "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4),
                                       "TFLOPs": round(fl / us / 1e6, 2),
                                       "mfma_frac": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                                       "kv_bytes": by, "flops": fl}
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
    us_t = graph_us(lambda: binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, tm, out=out,
                                                workspace=ws), torch, check=out)
    res["verify_tree_4x8rows_9k"] = {"us": round(us_t, 2), "kv_GBps": round(by / us_t / 1e3, 1),
                                     "hbm_frac": round(by / us_t / 1e3 / HBM_PEAK_GBS, 4)}
    del c, ks, vs
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
    us0 = graph_us(lambda: binding.decode(c.pool, q0, t0, l0, c.lengths[0], out=o0), torch, check=o0)
    us1 = graph_us(lambda: binding.verify(c.pool, q1, t1, l1, c.lengths[1], out=o1), torch, check=o1)
    b0, b1 = c.lengths[0] * w.kv_bytes_per_token, c.lengths[1] * w.kv_bytes_per_token
    res["wide_head_d512_p37"] = {"decode_2048_us": round(us0, 2), "decode_kv_GBps": round(b0 / us0 / 1e3, 1),
                                 "verify4_9000_us": round(us1, 2), "verify_kv_GBps": round(b1 / us1 / 1e3, 1)}
    del c, ks, vs
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
        us = graph_us(prompt, torch, reps=5, check=outs[3])
        fl = sum(attn_flops([c0 + 512], 512, w.q_heads, w.head_dim, window) for c0 in range(0, 2048, 512))
        res["prefill_2048_in_512_chunks" + ("_window1024_ring" if window else "_full")] = {
            "us": round(us, 2), "us_per_chunk": round(us / 4, 2), "TFLOPs": round(fl / us / 1e6, 2),
            "mfma_frac": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl}
        del c, ks, vs
    torch.cuda.empty_cache()
    return res


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


def cpu_baseline(setup, oracle, workloads, budget_s=20.0):
    """The oracle, as it stands, on streams of the same workload until about budget_s of CPU
    work: gather through the table walk, widen to float64, attend.  Returns a dict in GB/s of
    K/V processed."""
    import numpy as np
    c, w = setup.c, setup.w
    kb = workloads.bf16_bits(c.pool.k_pages)
    vb = workloads.bf16_bits(c.pool.v_pages)
    qb = workloads.bf16_bits(setup.q)
    done, nbytes, secs = [], 0, 0.0
    for s in range(w.streams):
        L = c.lengths[s]
        t0 = time.perf_counter()
        kl = oracle.bf16_bits_to_f64(oracle.gather_linear(kb, c.table_host[s], L, w.page_size))
        vl = oracle.bf16_bits_to_f64(oracle.gather_linear(vb, c.table_host[s], L, w.page_size))
        out = oracle.attend_stream(oracle.bf16_bits_to_f64(qb[s]), kl, vl, 1, 0, length=L)
        secs += time.perf_counter() - t0
        assert np.isfinite(out).all()
        done.append(s)
        nbytes += L * w.kv_bytes_per_token
        if secs >= budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle (table walk + widen + attend) on streams {done[0]}..{done[-1]} "
                      f"of 12 ({nbytes / 1e9:.3f} GB of K/V) in {secs:.2f} s; numpy/BLAS may use all "
                      f"{cores} threads; host {platform.processor() or platform.machine()}"}


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
    if args.side_only:
        log("[bench] side workloads only")
        res = {"side_only": True, "graphs": USE_GRAPHS,
               "other_workloads": other_workloads(torch, binding, staging, workloads)}
        print(json.dumps(res), flush=True)
        return

    w = workloads.batched_decode(fixed_length=args.fixed_length)
    log(f"[bench] building {w.name}: lengths {w.lengths}, pool {w.pool_pages} pages")
    setup = DecodeSetup(w, 3002, torch, binding, staging, workloads)
    torch.cuda.synchronize()
    log("[bench] timing steps")
    ms_step, part_ms, part_min, part_max = timed_steps(setup, args.steps, args.warmup, torch, binding)
    value = setup.kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = setup.kv_bytes / (part_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    # the same step as two calls (kv_rows_put, then paged_attn_decode), in interleaved rounds
    # with the fused call
    fused_ms, unfused_ms = [], []
    for _ in range(3):
        for fused, acc in ((True, fused_ms), (False, unfused_ms)):
            setup.fused = fused
            acc.append(timed_steps(setup, 30, 3, torch, binding)[0])
    setup.fused = True
    log(f"[bench] {ms_step * 1e3:.1f} us/step, part kernel {part_ms * 1e3:.1f} us, {achieved:.0f} GB/s")

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
                        f"spares; step = paged_attn_decode_put (the new row of each stream written into its page and attended, one call)"
            if args.fixed_length is None else
            f"{w.name}: 12 streams x {args.fixed_length}, otherwise as the batched decode",
            "streams": w.streams, "kv_heads": w.kv_heads, "q_heads": w.q_heads, "head_dim": w.head_dim,
            "page_size": w.page_size, "rows": 1, "lengths": w.lengths,
            "kv_bytes_per_step": setup.kv_bytes,
        },
        "us_per_layer": round(ms_step * 1e3, 2),
        "two_call_step": {"us_per_layer": round(sorted(unfused_ms)[1] * 1e3, 2),
                          "fused_us_per_layer": round(sorted(fused_ms)[1] * 1e3, 2),
                          "note": "kv_rows_put + paged_attn_decode against paged_attn_decode_put, medians of "
                                  "3 interleaved rounds of 30 steps"},
        "roofline": {
            "bound": "hbm", "kernel": "part_valu_kernel<128,8,8>",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "part_us_mean": round(part_ms * 1e3, 2), "part_us_min": round(part_min * 1e3, 2),
            "part_us_max": round(part_max * 1e3, 2),
        },
    }

    if not args.quick:
        log("[bench] cold-cache calls (1 GiB flush before each)")
        result["cold_attention_us"] = round(cold_calls(setup, 20, torch) * 1e3, 2)
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
                sms, pms, _, _ = timed_steps(st, 25, 3, torch, binding)
                parts[name].append(pms)
                stepms[name].append(sms)
        med = lambda xs: sorted(xs)[len(xs) // 2]
        runs = [1 + int((np.diff(cg.c.table_host[s][:w.pages_for(L)]) != 1).sum()) for s, L in enumerate(w.lengths)]
        result["identity_table"] = {"us_per_layer": round(med(stepms["identity"]) * 1e3, 2),
                                    "part_us_median": round(med(parts["identity"]) * 1e3, 2),
                                    "shuffled_part_us_median": round(med(parts["shuffled"]) * 1e3, 2),
                                    "paged_over_identity": round(med(parts["shuffled"]) / med(parts["identity"]), 4),
                                    "rounds": "4 interleaved rounds of 25 steps per arm"}
        result["contiguous_leases"] = {"us_per_layer": round(med(stepms["contiguous"]) * 1e3, 2),
                                       "part_us_median": round(med(parts["contiguous"]) * 1e3, 2),
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
            fms, fpart, _, _ = timed_steps(fx, max(20, args.steps // 4), 5, torch, binding)
            result["fixed_12x40960"] = {"us_per_layer": round(fms * 1e3, 2), "part_us_mean": round(fpart * 1e3, 2),
                                        "kv_GBps": round(fx.kv_bytes / (fms * 1e-3) / 1e9, 1),
                                        "part_kv_GBps": round(fx.kv_bytes / (fpart * 1e-3) / 1e9, 1)}
            del fx
            torch.cuda.empty_cache()

    if not args.quick:
        log("[bench] verify window, wide head and prompt workloads")
        result["other_workloads"] = other_workloads(torch, binding, staging, workloads)
    if args.calib_copy:
        log("[bench] calibration copy")
        calibration_copy(torch)

    if not args.no_cpu_baseline:
        import oracle          # the CPU reference, used by this leg only
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(setup, oracle, workloads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
