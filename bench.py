"""Benchmark of the HiSparse decode-step swap-in on one MI355X.

One "step" is one hisparse_swap_in call (resolve + row copy) over one batch of
synthetic top-k ids. Headline workload: DeepSeek-V3.2-like decode, B=32
requests, 32,768-token contexts in a pinned-host pool of 1,048,576 x 656-byte
rows, hot_size 4096, top_k 2048, Zipf(1.1) recency ids with 85% retention.
W warm-up steps (the first is the cold step) run untimed, then K steps are
timed; inputs for every step are resident in HBM before timing starts.

Also reported in the same JSON line:
  * cold_step: the first (all-miss) call of the headline trace, timed alone;
  * roofline: the fused kernel's mean launch time from the timed calls
    replayed back to back behind a spin kernel (events on the launch stream);
  * device_pool: the same call on the device-pool workload (B=128, 16,384-token
    contexts, pool of 2,097,152 rows in HBM, 60% retention) against 8 TB/s,
    beside what this part's HBM gives a plain 1 GiB copy (hipMemcpy and the
    library's copy engine), and the steady state timed step by step from a
    restored state after a 512 MiB flush;
  * adversarial: B=64, hot_size 8192, 65,536-token contexts, ids that collide
    in the pages' low-bit multiplicative hash (1152-byte and 132-byte rows) and
    ids that collide in the kernel's own high-bit buckets (1152-byte rows):
    the cold step and the steps after it;
  * tiny: B=2, hot_size 64, top_k 16 -- GPU time and caller-visible latency
    per call;
  * kv_decode: non-MLA caches -- the headline's shape with 1024-byte K and V
    rows in two pinned pools, every miss moving both;
  * paged: vLLM-style paged addressing (64-row source and hot blocks, global
    ids as slot keys) on the device-pool and headline traces;
  * plan_replay: the headline trace with index-sharing layers (1 resolving
    layer + 3 replaying its plan): one fused replay launch for all layers
    against one copy launch per layer;
  * scatter: store_kv_scatter / store_kv_cache of one 8192-row prefill chunk
    into a 1M-row cache in HBM;
  * all_layer: the fused all-layer transfer (61 layers x 262,144 rows x 656 B,
    8192 pairs) in both directions against the host-link ceiling;
  * host_link: the measured host-link ceiling the host-pool rooflines use;
  * cpu_baseline: the CPU oracle (single thread, and on every host core the
    process may use) on the headline steps, with the host CPU's model name.
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

HBM_PEAK_GBS = 8000.0
PCIE5_X16_GBS = 64.0   # PCIe 5.0 x16, one direction, published link rate


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=63)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--device-pool-steps", type=int, default=31)
    p.add_argument("--no-device-pool", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-host-link", action="store_true")
    p.add_argument("--no-all-layer", action="store_true")
    p.add_argument("--no-adversarial", action="store_true")
    p.add_argument("--no-plan-replay", action="store_true")
    p.add_argument("--no-kv", action="store_true")
    p.add_argument("--no-paged", action="store_true")
    p.add_argument("--no-scatter", action="store_true")
    p.add_argument("--no-tiny", action="store_true")
    p.add_argument("--only", default="",
                   help="comma-separated legs to run, the rest skipped (for profiling runs): "
                        "headline, device_pool, plan_replay, kv, paged, adversarial, all_layer, "
                        "scatter, tiny, cpu_baseline, host_link")
    p.add_argument("--replay-layers", type=int, default=4,
                   help="layers per index-sharing group in the plan-replay leg (1 resolving "
                        "layer + the rest replaying its plan)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU seconds of oracle work for cpu_baseline (whole replays "
                        "of the headline's timed steps)")
    p.add_argument("--copy-row-sizes", action="store_true",
                   help="the device-pool trace with other row sizes (512, 640, 656, 672, 768 B): "
                        "copy kernel time per call, one JSON object per size")
    p.add_argument("--copy-ceilings", action="store_true",
                   help="only measure the library's row transfer on scattered rows of several "
                        "sizes (pinned host -> HBM and HBM -> HBM), one JSON line each, then exit")
    p.add_argument("--calibrate", action="store_true",
                   help="only run a plain device-to-device stream copy of known size "
                        "(256 MiB read + 256 MiB written per launch, 3 launches) so HBM byte "
                        "counters can be scaled, then exit")
    return p.parse_args()


class Trace:
    """Pre-generated inputs of one workload, uploaded to HBM."""

    def __init__(self, cfg, steps, torch):
        from workloads import gen
        self.cfg = cfg
        self.steps = steps
        self.topk_np = np.stack(list(gen.topk_trace(cfg, steps)))
        self.seq_np = np.stack([gen.seq_lens(cfg, t) for t in range(steps)])
        self.topk = torch.as_tensor(self.topk_np).cuda()
        self.seq = torch.as_tensor(self.seq_np).cuda()
        self.rows = torch.arange(cfg.B, dtype=torch.int64, device="cuda")


def run_gpu(cfg, warmup, steps, torch, hs, wdev, kv=False, lead_spin=False, b2b_pass=False):
    """Time K swap-in calls after W warm-up calls.

    Pass 1 (the timed region of the contract): W untimed calls, then K plain
    hisparse_swap_in calls bracketed by two events and the wall clock.
    Pass 2 (per-kernel times): the state is reset and the same trace replayed;
    the K timed steps run as K hisparse_resolve calls, each into its own
    workspace, back to back, then the K hisparse_gather_compact calls back to
    back -- the same work in the same order for the hot buffer, with each
    kernel's total bracketed by two events and no gaps between launches.
    The first warm-up call is the cold step (every id a miss) and is timed on
    its own with two events.
    With kv=True the workload has non-MLA caches: a V pool (its own bytes) and
    a V hot buffer, and every miss moves its K row and its V row.
    With lead_spin=True pass 1's calls also queue behind a spin kernel, so its
    events bracket the kernels alone (for traces of a few calls, where the
    host time ahead of the first launch is not amortised); the wall clock then
    includes the spin and is not meaningful.
    With b2b_pass=True a third pass replays the K timed calls from the same
    starting state queued behind a spin kernel, so the events bracket the K
    launches back to back with no host time between them: us_b2b / K is the
    mean launch time of the call's kernel (one fused kernel on a host pool).
    Returns dict(us_total, us_resolve, us_copy, us_cold, cold_rows, counts, wall, us_b2b).
    """
    log(f"[bench] {cfg.name}: building pool ({cfg.pool_nrows} x {cfg.row_bytes} B, {cfg.pool_kind})"
        + (" x 2 (K and V)" if kv else ""))
    pool = wdev.make_pool(cfg)
    st = wdev.DeviceSwapState(cfg)
    kvkw = {}
    if kv:
        kvkw = dict(pool_v=wdev.make_pool(cfg.with_(seed=cfg.seed + 777)),
                    hot_v=torch.zeros_like(st.hot))
    tr = Trace(cfg, warmup + steps, torch)
    counts = torch.empty((warmup + steps, cfg.B), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(t, fn, ws):
        fn(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t], slot_tokens=st.slot_tokens,
           lru=st.lru, pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx, workspace=ws,
           miss_counts=counts[t], stream=stream, **kvkw)

    def events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # One call with every row padding (num_real = 0) takes the library's
    # one-time costs (LDS opt-in, first launches) and changes no state. Before
    # the cold step the GPU is kept busy by a short spin kernel, so the
    # host-side time of the call is hidden and the two events bracket the
    # call's kernels only.
    pad = torch.zeros(1, dtype=torch.int32, device="cuda")
    hs.hisparse_swap_in(topk=tr.topk[0], req_rows=tr.rows, seq_lens=tr.seq[0],
                        slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                        out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws, num_real=pad,
                        stream=stream, **kvkw)
    torch.cuda.synchronize()
    c0, c1 = events()
    for t in range(warmup):
        if t == 0:
            torch.cuda._sleep(2_000_000)
            c0.record(stream)
        call(t, hs.hisparse_swap_in, st.ws)
        if t == 0:
            c1.record(stream)
    torch.cuda.synchronize()
    us_cold = c0.elapsed_time(c1) * 1000.0 if warmup else None
    # (The cold step's row count is read after the timed region: the process's
    # first tensor reduction makes the next launch's host call ~0.1 ms slower
    # once, which a short timed region would carry.)
    e0, e1 = events()
    if lead_spin:
        torch.cuda._sleep(2_000_000)
    # Python's collector stays off while the calls are issued, as timeit does:
    # a collection pause ahead of the first launches would idle the GPU.
    gc.disable()
    try:
        w0 = time.perf_counter()
        e0.record(stream)
        for k in range(steps):
            call(warmup + k, hs.hisparse_swap_in, st.ws)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    finally:
        gc.enable()
    us_total = e0.elapsed_time(e1) * 1000.0
    log(f"[bench] {cfg.name}: {steps} timed calls after {warmup} warm-up, {us_total / steps:.1f} us/call")
    cold_rows = int(counts[0].sum().item()) if warmup else 0
    c = counts.cpu().numpy()[warmup:].copy()

    # pass 2
    hs.hisparse_state_reset(slot_tokens=st.slot_tokens, lru=st.lru,
                            rows=torch.arange(st.R, dtype=torch.int64, device="cuda"))
    for t in range(warmup):
        call(t, hs.hisparse_swap_in, st.ws)
    wss = [torch.zeros_like(st.ws) for _ in range(steps)]
    torch.cuda.synchronize()
    r0, r1 = events()
    g0, g1 = events()
    # A resolve launch is shorter than the binding's host time per call: a
    # spin kernel (about 10 ms) ahead of the events lets the host enqueue both
    # batches first, so each batch runs back to back between its events.
    torch.cuda._sleep(24_000_000)
    r0.record(stream)
    for k in range(steps):
        call(warmup + k, hs.hisparse_resolve, wss[k])
    r1.record(stream)
    g0.record(stream)
    for k in range(steps):
        call(warmup + k, hs.hisparse_gather_compact, wss[k])
    g1.record(stream)
    torch.cuda.synchronize()
    us_resolve = r0.elapsed_time(r1) * 1000.0
    us_copy = g0.elapsed_time(g1) * 1000.0
    assert (counts.cpu().numpy()[warmup:] == c).all(), "replay diverged from the timed pass"
    us_b2b = None
    if b2b_pass:
        # pass 3: the timed calls again, queued behind a spin kernel
        hs.hisparse_state_reset(slot_tokens=st.slot_tokens, lru=st.lru,
                                rows=torch.arange(st.R, dtype=torch.int64, device="cuda"))
        for t in range(warmup):
            call(t, hs.hisparse_swap_in, st.ws)
        torch.cuda.synchronize()
        b0, b1 = events()
        torch.cuda._sleep(24_000_000)
        b0.record(stream)
        for k in range(steps):
            call(warmup + k, hs.hisparse_swap_in, st.ws)
        b1.record(stream)
        torch.cuda.synchronize()
        us_b2b = b0.elapsed_time(b1) * 1000.0
        assert (counts.cpu().numpy()[warmup:] == c).all(), "back-to-back pass diverged"
    del pool, st, tr, wss
    torch.cuda.empty_cache()
    return dict(us_total=us_total, us_resolve=us_resolve, us_copy=us_copy, us_cold=us_cold,
                cold_rows=cold_rows, counts=c, wall=wall, us_b2b=us_b2b)


def run_flushed(cfg, steps, replays, torch, hs, wdev):
    """The step-by-step protocol: after the cold step, each of `steps` steps
    is replayed `replays` + 1 times from a snapshot of the state taken before
    it; before every replay the state is restored and 512 MiB are written to a
    scratch buffer (evicting L2 and the MALL), both untimed, and a short spin
    kernel hides the host time of the call. Replays of a step move the same
    rows to the same slots. Returns the median over steps of each step's
    median replay time (µs), and the rows per step."""
    log(f"[bench] {cfg.name}: per-step replays with state restore and a 512 MiB flush")
    pool = wdev.make_pool(cfg)
    st = wdev.DeviceSwapState(cfg)
    tr = Trace(cfg, 1 + steps, torch)
    counts = torch.empty((1 + steps, cfg.B), dtype=torch.int32, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(t):
        hs.hisparse_swap_in(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t],
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                            miss_counts=counts[t], stream=stream)

    call(0)
    per_step = []
    for t in range(1, 1 + steps):
        snap = (st.slot_tokens.clone(), st.lru.clone())
        us = []
        for rep in range(replays + 1):
            st.slot_tokens.copy_(snap[0])
            st.lru.copy_(snap[1])
            flush.fill_(rep)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(200_000)
            e0.record(stream)
            call(t)
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                us.append(e0.elapsed_time(e1) * 1000.0)
        us.sort()
        per_step.append(us[len(us) // 2])
    rows = int(counts[1:].sum().item())
    del pool, st, tr, flush
    torch.cuda.empty_cache()
    per_step.sort()
    return per_step[len(per_step) // 2], rows / steps


def run_tiny(torch, hs, wdev):
    """The tiny workload (B=2, H=64, K=16, 656-byte rows, pinned-host pool):
    the cold step, then 7 steps, each timed four ways -- the GPU time of the
    call's kernel (the 7 calls queued behind a spin kernel, between two
    events), the latency a caller sees (host wall time of the call plus a
    synchronize, median over the 7 steps), and the same latency through a
    SwapInCall and with the call replayed from a HIP graph."""
    from workloads import gen
    cfg = gen.TINY
    r = run_gpu(cfg, 1, cfg.steps - 1, torch, hs, wdev, lead_spin=True)
    pool = wdev.make_pool(cfg)
    st = wdev.DeviceSwapState(cfg)
    tr = Trace(cfg, cfg.steps, torch)
    lat = []
    for t in range(cfg.steps):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        hs.hisparse_swap_in(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t],
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                            miss_counts=st.counts)
        torch.cuda.synchronize()
        if t:
            lat.append((time.perf_counter() - w0) * 1e6)
    lat.sort()
    # The same steps through a SwapInCall (every argument checked once; per
    # step only the step's tensors), timed the same way.
    pst = wdev.DeviceSwapState(cfg)
    pcall = hs.SwapInCall(slot_tokens=pst.slot_tokens, lru=pst.lru, pool=pool, hot=pst.hot,
                          out_rows=pst.out, ctx_stride=cfg.ctx, workspace=pst.ws,
                          miss_counts=pst.counts)
    plat = []
    for t in range(cfg.steps):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        pcall(tr.topk[t], tr.rows, tr.seq[t])
        torch.cuda.synchronize()
        if t:
            plat.append((time.perf_counter() - w0) * 1e6)
    assert torch.equal(pst.hot, st.hot) and torch.equal(pst.lru, st.lru), "prepared calls diverged"
    plat.sort()
    # The same steps with the call captured once in a HIP graph over fixed
    # input buffers: per step the inputs are written into those buffers (as an
    # indexer writing there would leave them), then the replay is timed with
    # a synchronize, like the plain calls above.
    gst = wdev.DeviceSwapState(cfg)
    topk_in = torch.zeros_like(tr.topk[0])
    seq_in = torch.zeros_like(tr.seq[0])

    def gcall(num_real=None):
        hs.hisparse_swap_in(topk=topk_in, req_rows=tr.rows, seq_lens=seq_in,
                            slot_tokens=gst.slot_tokens, lru=gst.lru, pool=pool, hot=gst.hot,
                            out_rows=gst.out, ctx_stride=cfg.ctx, workspace=gst.ws,
                            miss_counts=gst.counts, num_real=num_real)
    gcall(num_real=torch.zeros(1, dtype=torch.int32, device="cuda"))   # one-time set-up, no change
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gcall()
    glat = []
    for t in range(cfg.steps):
        topk_in.copy_(tr.topk[t])
        seq_in.copy_(tr.seq[t])
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        if t:
            glat.append((time.perf_counter() - w0) * 1e6)
    assert torch.equal(gst.hot, st.hot) and torch.equal(gst.lru, st.lru), "graph replays diverged"
    glat.sort()
    del graph
    n = cfg.steps - 1
    return {"workload": "tiny_swap_in_pinned_host_pool", "batch": cfg.B, "hot_size": cfg.H,
            "top_k": cfg.K, "context": cfg.ctx, "row_bytes": cfg.row_bytes, "steps_after_cold": n,
            "rows_per_call": round(float(r["counts"].sum()) / n, 2),
            "us_per_call_gpu": round(r["us_total"] / n, 2),
            "us_per_call_sync": round(lat[len(lat) // 2], 2),
            "us_per_call_sync_prepared": round(plat[len(plat) // 2], 2),
            "us_per_call_sync_graph": round(glat[len(glat) // 2], 2),
            "cold_step_us_gpu": round(r["us_cold"], 2),
            "bound": "latency (launch and one workgroup per request)"}


def hbm_ceiling(torch, hs):
    """What this part's HBM delivers to a plain copy: a 1 GiB device-to-device
    hipMemcpyAsync, and the library's own 16-byte-per-lane copy engine
    (transfer_rows_all_layer, HBM-sized launch) over the same 1 GiB as
    contiguous 1 MiB rows. Best of 5 each; GB/s counts bytes read + written."""
    n = 1 << 30
    src = torch.full((n,), 3, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()

    def best(fn, reps=5):
        b = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            b = max(b, 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return b

    res = {"memcpy_d2d_GBps": best(lambda: dst.copy_(src, non_blocking=True))}
    rb = 1 << 20
    idx = torch.arange(n // rb, dtype=torch.int64, device="cuda")
    sp = torch.tensor([src.data_ptr()], dtype=torch.int64, device="cuda")
    dp = torch.tensor([dst.data_ptr()], dtype=torch.int64, device="cuda")
    res["library_copy_contiguous_GBps"] = best(lambda: hs.transfer_rows_all_layer(
        src_layer_ptrs=sp, dst_layer_ptrs=dp, src_idx=idx, dst_idx=idx, row_bytes=rb,
        src_nrows=n // rb, dst_nrows=n // rb))
    del src, dst
    torch.cuda.empty_cache()
    return {k: round(v, 1) for k, v in res.items()}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_plan_replay(cfg, layers, warmup, steps, torch, hs, wdev):
    """Index-sharing layers on the headline workload: per step one resolve on
    layer 0, then the plan is copied for all `layers` layers, either as ONE
    hisparse_gather_compact_layers launch (fused) or as one
    hisparse_gather_compact launch per layer (separate). Layer 0's pool holds
    the workload's bytes; the other layers' pools are pinned buffers of the
    same shape. Each variant runs the trace from a reset state (W warm-up
    steps, then K timed steps between two events). A third pass times the K
    fused replays alone, back to back after K resolves into K workspaces."""
    log(f"[bench] plan replay: {layers} layers on {cfg.name}")
    pools = [wdev.make_pool(cfg)] + [wdev.pinned_uint8(cfg.pool_nrows, cfg.row_bytes)
                                     for _ in range(layers - 1)]
    st = wdev.DeviceSwapState(cfg)
    hots = [st.hot] + [torch.zeros_like(st.hot) for _ in range(layers - 1)]
    pptr = torch.tensor([p.data_ptr() for p in pools], dtype=torch.int64, device="cuda")
    hptr = torch.tensor([h.data_ptr() for h in hots], dtype=torch.int64, device="cuda")
    tr = Trace(cfg, warmup + steps, torch)
    counts = torch.empty((warmup + steps, cfg.B), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    allrows = torch.arange(cfg.R, dtype=torch.int64, device="cuda")

    def resolve(t, ws):
        hs.hisparse_resolve(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t],
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pools[0], hot=hots[0],
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=ws,
                            miss_counts=counts[t], stream=stream)

    def fused(ws):
        hs.hisparse_gather_compact_layers(workspace=ws, B=cfg.B, K=cfg.K, pool_layer_ptrs=pptr,
                                          pool_nrows=cfg.pool_nrows, hot_layer_ptrs=hptr,
                                          hot_nrows=hots[0].shape[0], row_bytes=cfg.row_bytes,
                                          stream=stream)

    def separate(t, ws):
        for l in range(layers):
            hs.hisparse_gather_compact(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t],
                                       slot_tokens=st.slot_tokens, lru=st.lru, pool=pools[l],
                                       hot=hots[l], out_rows=st.out, ctx_stride=cfg.ctx,
                                       workspace=ws, stream=stream)

    def timed(step_fn):
        hs.hisparse_state_reset(slot_tokens=st.slot_tokens, lru=st.lru, rows=allrows)
        for t in range(warmup):
            step_fn(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(steps):
            step_fn(warmup + k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0

    us_fused = timed(lambda t: (resolve(t, st.ws), fused(st.ws)))
    c = counts.cpu().numpy()[warmup:].copy()
    us_sep = timed(lambda t: (resolve(t, st.ws), separate(t, st.ws)))
    assert (counts.cpu().numpy()[warmup:] == c).all(), "plan replay passes diverged"
    # replay kernel alone
    hs.hisparse_state_reset(slot_tokens=st.slot_tokens, lru=st.lru, rows=allrows)
    for t in range(warmup):
        resolve(t, st.ws)
        fused(st.ws)
    wss = [torch.zeros_like(st.ws) for _ in range(steps)]
    for k in range(steps):
        resolve(warmup + k, wss[k])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(steps):
        fused(wss[k])
    e1.record(stream)
    torch.cuda.synchronize()
    us_replay = e0.elapsed_time(e1) * 1000.0
    del pools, hots, st, tr, wss
    torch.cuda.empty_cache()
    return dict(rows=int(c.sum()), us_fused=us_fused, us_separate=us_sep, us_replay=us_replay)


def run_paged(cfg, warmup, steps, torch, hs, wdev, block=64):
    """The workload's trace with vLLM-style paged addressing: every request's
    positions map through a source block table of `block`-row blocks (a
    seeded permutation of physical blocks, block 0 unused) to global pool
    rows, and its slots through a hot block table of `block`-slot blocks (a
    seeded permutation). W warm-up calls, then K hisparse_swap_in calls
    between two events, queued behind a spin kernel. Returns dict(us_total, rows)."""
    rng = np.random.default_rng(cfg.seed + 99)
    R, B, H, K, ctx = cfg.R, cfg.B, cfg.H, cfg.K, cfg.ctx
    nsb = -(-ctx // block)
    src = (rng.permutation(B * nsb) + 1).astype(np.int32).reshape(B, nsb)
    pool_nrows = (B * nsb + 1) * block
    nhb = -(-H // block)
    hot_tab = rng.permutation(R * nhb).astype(np.int32).reshape(R, nhb)
    log(f"[bench] paged {cfg.name}: building pool ({pool_nrows} x {cfg.row_bytes} B, {cfg.pool_kind})")
    pool = wdev.make_pool(cfg.with_(B=1, ctx=pool_nrows))
    keys = torch.full((R, H + 1), -1, dtype=torch.int32, device="cuda")
    lru = torch.tensor(np.tile(np.arange(H, dtype=np.int16), (R, 1)), device="cuda")
    hot = torch.zeros((R * nhb * block, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    counts = torch.empty((warmup + steps, B), dtype=torch.int32, device="cuda")
    ws = torch.empty(hs.swap_in_workspace_bytes(B, K), dtype=torch.uint8, device="cuda")
    tr = Trace(cfg, warmup + steps, torch)
    paged = {"hot_block_table": torch.as_tensor(hot_tab).cuda(), "hot_block_size": block,
             "src_block_table": torch.as_tensor(src).cuda(), "src_block_size": block}
    stream = torch.cuda.current_stream()

    def call(t):
        hs.hisparse_swap_in(topk=tr.topk[t], req_rows=tr.rows, seq_lens=None, slot_tokens=keys,
                            lru=lru, pool=pool, hot=hot, out_rows=out, ctx_stride=0, workspace=ws,
                            miss_counts=counts[t], paged=paged, stream=stream)

    for t in range(warmup):
        call(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # The paged arguments cost the Python binding more host time per call than
    # the flat ones, on some hosts more than the call's kernel. A spin kernel
    # ahead of the first event (about 10 ms) lets the host enqueue every call
    # first, so the events bracket the calls' kernels back to back.
    torch.cuda._sleep(24_000_000)
    e0.record(stream)
    for k in range(steps):
        call(warmup + k)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0
    rows = int(counts[warmup:].sum().item())
    del pool, hot, keys, lru, tr
    torch.cuda.empty_cache()
    return dict(us_total=us, rows=rows)


def run_scatter(torch, hs, n=8192, rb=656, cache_rows=1 << 20, reps=5):
    """store_kv_scatter and store_kv_cache on one prefill chunk: n rows of rb
    bytes (contiguous source in HBM) written to seeded distinct rows of a
    cache of `cache_rows` rows in HBM; the K+V form moves a second, separate
    pair. A 512 MiB write between repetitions evicts L2 and MALL. Returns
    median µs of each."""
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(0, 256, (n, rb), dtype=torch.uint8, generator=g).cuda()
    src_v = torch.randint(0, 256, (n, rb), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros((cache_rows, rb), dtype=torch.uint8, device="cuda")
    dst_v = torch.zeros((cache_rows, rb), dtype=torch.uint8, device="cuda")
    loc = torch.randperm(cache_rows, generator=g)[:n].cuda()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    res = {}
    for name, fn in (("k", lambda: hs.store_kv_scatter(src=src, dst=dst, loc=loc)),
                     ("kv", lambda: hs.store_kv_cache(k_src=src, v_src=src_v, k_dst=dst,
                                                      v_dst=dst_v, loc=loc))):
        us = []
        for rep in range(reps + 1):
            flush.fill_(rep)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            if rep:
                us.append(e0.elapsed_time(e1) * 1000.0)
        us.sort()
        res[name] = us[len(us) // 2]
    del src, src_v, dst, dst_v, flush
    torch.cuda.empty_cache()
    return res


def code_text(src):
    """C++ source with its comments removed and every run of white space
    collapsed to one blank: what the compiler sees of it, so that an edit to a
    comment does not count as a change of the kernel. Comment markers inside
    string and character literals are not comments."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_hash(files):
    """Hash of the code (comments and layout aside) of the given sources."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(code_text(open(os.path.join(ROOT, f), encoding="utf-8").read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM/fabric bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summary, if it was taken on the kernel's
    sources as they are now (each entry lists its sources and their hash)."""
    path = os.path.join(ROOT, "profiles", "swap_copy_traffic.json")
    try:
        w = json.load(open(path))["workloads"][workload]
        if w["kernel_sources_sha256_16"] != sources_hash(w["kernel_sources"]):
            return None
        return w["bytes_per_launch"]
    except (OSError, ValueError, KeyError, TypeError):
        return None


def host_link_ceiling(torch, hs):
    """Best-of-N host->device rate of (a) hipMemcpyAsync of 1 GiB pinned and
    (b) a zero-copy streaming kernel (the library's row transfer over 1 MiB
    sequential rows of pinned memory). Also device->host for reference."""
    n = 1 << 30
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = 7
    dev = torch.empty(n, dtype=torch.uint8, device="cuda")
    res = {}
    s = torch.cuda.current_stream()

    def best(fn, reps=5):
        b = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            b = max(b, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return b

    res["memcpy_h2d_gbs"] = best(lambda: dev.copy_(host, non_blocking=True))
    res["memcpy_d2h_gbs"] = best(lambda: host.copy_(dev, non_blocking=True))
    rb = 1 << 20
    rows = n // rb
    idx = torch.arange(rows, dtype=torch.int64, device="cuda")
    hp = torch.tensor([host.data_ptr()], dtype=torch.int64, device="cuda")
    dp = torch.tensor([dev.data_ptr()], dtype=torch.int64, device="cuda")
    res["zero_copy_h2d_gbs"] = best(lambda: hs.transfer_rows_all_layer(
        src_layer_ptrs=hp, dst_layer_ptrs=dp, src_idx=idx, dst_idx=idx, row_bytes=rb,
        src_nrows=rows, dst_nrows=rows, host_link=True))
    res["zero_copy_d2h_gbs"] = best(lambda: hs.transfer_rows_all_layer(
        src_layer_ptrs=dp, dst_layer_ptrs=hp, src_idx=idx, dst_idx=idx, row_bytes=rb,
        src_nrows=rows, dst_nrows=rows, host_link=True))
    res["h2d_ceiling_gbs"] = max(res["memcpy_h2d_gbs"], res["zero_copy_h2d_gbs"])
    res["d2h_ceiling_gbs"] = max(res["memcpy_d2h_gbs"], res["zero_copy_d2h_gbs"])
    del host, dev
    torch.cuda.empty_cache()
    return res


def calibrate(torch, hs):
    """Three launches of the library's row transfer over contiguous 1 MiB rows:
    exactly 256 MiB read and 256 MiB written per launch, device to device."""
    n = 256 << 20
    rb = 1 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.arange(n // rb, dtype=torch.int64, device="cuda")
    sp = torch.tensor([src.data_ptr()], dtype=torch.int64, device="cuda")
    dp = torch.tensor([dst.data_ptr()], dtype=torch.int64, device="cuda")
    for _ in range(3):
        hs.transfer_rows_all_layer(src_layer_ptrs=sp, dst_layer_ptrs=dp, src_idx=idx, dst_idx=idx,
                                   row_bytes=rb, src_nrows=n // rb, dst_nrows=n // rb)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "transfer_kernel<16, 4>", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 3}), flush=True)


def copy_row_sizes(torch, hs, wdev):
    """The device-pool trace (B=128, K=2048, H=4096, HBM pool) with rows of
    512, 640, 656, 672 and 768 bytes: the copy kernel's mean launch time over
    the 31 timed steps (pass 2: the copies back to back), to set the
    workload's 656-byte rows against rows that are whole 128-byte lines."""
    from workloads import gen
    for rb in (512, 640, 656, 672, 768):
        cfg = gen.DEVPOOL.with_(row_bytes=rb)
        r = run_gpu(cfg, 1, 31, torch, hs, wdev)
        rows = float(r["counts"].sum()) / 31
        us = r["us_copy"] / 31
        print(json.dumps({"row_bytes": rb, "rows_per_call": rows, "us_copy_kernel": round(us, 2),
                          "GBps_read_write": round(rows * rb * 2 / us / 1e3, 1),
                          "us_resolve_kernel": round(r["us_resolve"] / 31, 2)}), flush=True)


def copy_ceilings(torch, hs):
    """What the copy engine reaches on scattered rows, by row size and bytes per
    launch: transfer_rows_all_layer with one layer, rows drawn without
    replacement from a 688 MB pool (pinned host, or HBM), written to a random
    permutation of a hot buffer in HBM. Fresh rows every repetition and a
    512 MiB write between repetitions, so no row is served from L2 or MALL.
    Prints one JSON line per case with the median and best of 7 launches."""
    s = torch.cuda.current_stream()
    pool_bytes = 688 << 20
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(11)
    cases = []
    for kind in ("host", "device"):
        for rb in (132, 512, 640, 656, 1024, 1152, 2048, 4096):
            for total in (4 << 20, 64 << 20):
                cases.append((kind, rb, total))
    for kind, rb in (("device", 656),):
        cases.append((kind, rb, 85848 * 656))   # one device-pool swap-in launch
    pools = {}
    for kind, rb, total in cases:
        key = (kind, rb)
        if key not in pools:
            pools.clear()
            torch.cuda.empty_cache()
            nrows = pool_bytes // rb
            if kind == "host":
                pools[key] = torch.empty((nrows, rb), dtype=torch.uint8, pin_memory=True)
                pools[key].numpy()[:] = 3
            else:
                pools[key] = torch.full((nrows, rb), 3, dtype=torch.uint8, device="cuda")
        pool = pools[key]
        n = max(1, total // rb)
        hot = torch.zeros((max(n, 4096), rb), dtype=torch.uint8, device="cuda")
        sp = torch.tensor([pool.data_ptr()], dtype=torch.int64, device="cuda")
        dp = torch.tensor([hot.data_ptr()], dtype=torch.int64, device="cuda")
        us = []
        for rep in range(8):
            src = torch.randperm(pool.shape[0], generator=g)[:n].cuda()
            dst = torch.randperm(hot.shape[0], generator=g)[:n].cuda()
            flush.fill_(rep)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            hs.transfer_rows_all_layer(src_layer_ptrs=sp, dst_layer_ptrs=dp, src_idx=src, dst_idx=dst,
                                       row_bytes=rb, src_nrows=pool.shape[0], dst_nrows=hot.shape[0],
                                       host_link=kind == "host")
            e1.record(s)
            torch.cuda.synchronize()
            if rep:
                us.append(e0.elapsed_time(e1) * 1000.0)
        us.sort()
        moved = n * rb * (1 if kind == "host" else 2)   # host: link bytes; device: HBM read + write
        print(json.dumps({"copy_ceiling": f"{kind}_to_hbm", "row_bytes": rb, "rows": n,
                          "bytes_per_launch": moved, "us_median": round(us[len(us) // 2], 2),
                          "GBps_median": round(moved / us[len(us) // 2] / 1e3, 1),
                          "GBps_best": round(moved / us[0] / 1e3, 1)}), flush=True)
        del hot
    pools.clear()
    del flush
    torch.cuda.empty_cache()


def run_all_layer(torch, hs, reps=5):
    """The fused all-layer transfer at full size: 61 layers x 262,144 rows x
    656 B, 8192 index pairs, one call per repetition, per direction (offload =
    HBM -> pinned host, load = pinned host -> HBM), with the host-link launch
    shape (one side is host memory in both directions). A 512 MiB write between
    repetitions evicts L2 and MALL. Returns per-direction µs (median, best)."""
    from workloads import gen
    cfg = gen.ALL_LAYER
    L, rows, rb = cfg.layers, cfg.rows_per_layer, cfg.row_bytes
    log(f"[bench] all_layer: allocating 2 x {L * rows * rb / 1e9:.2f} GB")
    dev = torch.empty((L * rows, rb), dtype=torch.uint8, device="cuda")
    dev.fill_(5)
    host = torch.empty((L * rows, rb), dtype=torch.uint8, pin_memory=True)
    dptr = torch.tensor([dev[l * rows:].data_ptr() for l in range(L)], dtype=torch.int64, device="cuda")
    hptr = torch.tensor([host[l * rows:].data_ptr() for l in range(L)], dtype=torch.int64, device="cuda")
    si, di = gen.transfer_indices(cfg)
    si, di = torch.as_tensor(si).cuda(), torch.as_tensor(di).cuda()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    res = {}
    for name, sp, dp, sl, dl in (("offload", dptr, hptr, dev, host), ("load", hptr, dptr, host, dev)):
        link = hs.transfer_host_link(sl, dl)      # the launch shape from the memory kinds
        assert link, "one side is pinned host memory"
        us = []
        for rep in range(reps + 1):
            flush.fill_(rep)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            hs.transfer_rows_all_layer(src_layer_ptrs=sp, dst_layer_ptrs=dp, src_idx=si, dst_idx=di,
                                       row_bytes=rb, src_nrows=rows, dst_nrows=rows, host_link=link)
            e1.record(s)
            torch.cuda.synchronize()
            if rep:
                us.append(e0.elapsed_time(e1) * 1000.0)
        us.sort()
        res[name] = (us[len(us) // 2], us[0])
        log(f"[bench] all_layer {name}: median {us[len(us) // 2]:.1f} us")
    del dev, host, flush
    torch.cuda.empty_cache()
    return cfg, L * cfg.n_pairs * rb, res


def cpu_baseline(cfg, warmup, steps, min_seconds, threads=1):
    """The oracle on the headline trace: the warm-up steps run untimed to reach
    the timed window's starting state, then the timed steps run from that
    state, as whole passes, until at least `min_seconds` of oracle time has
    accumulated (each pass restores the slot tables; replaying a step from the
    same state repeats exactly the same work).
    threads > 1: each step's batch rows are split into `threads` contiguous
    groups and each group is one oracle call on its own thread. Rows name
    distinct state rows and hot regions, so the groups touch disjoint memory
    and the results are those of one call (the C oracle runs without the
    Python lock). A step's time is then the wall time of all its groups."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from workloads import gen
    pool = gen.fill_pool(cfg.seed, np.empty((cfg.pool_nrows, cfg.row_bytes), np.uint8))
    tok, lru = gen.initial_state(cfg)
    hot = np.zeros((cfg.R * cfg.S_r, cfg.row_bytes), np.uint8)
    rows = np.arange(cfg.B, dtype=np.int64)
    trace = list(gen.topk_trace(cfg, warmup + steps))
    for t in range(warmup):
        oracle.swap_in(topk=trace[t], req_rows=rows, seq_lens=gen.seq_lens(cfg, t), slot_tokens=tok,
                       lru=lru, pool=pool, hot=hot, ctx_stride=cfg.ctx)
    tok0, lru0 = tok.copy(), lru.copy()
    seqs = [gen.seq_lens(cfg, t) for t in range(warmup + steps)]
    groups = [g for g in np.array_split(np.arange(cfg.B), threads) if len(g)]

    def part(t, g):
        _, cnt = oracle.swap_in(topk=np.ascontiguousarray(trace[t][g]), req_rows=rows[g],
                                seq_lens=seqs[t][g], slot_tokens=tok, lru=lru, pool=pool, hot=hot,
                                ctx_stride=cfg.ctx)
        return int(cnt.sum())

    secs, rows_copied, passes = 0.0, 0, 0
    with ThreadPoolExecutor(max_workers=len(groups)) as ex:
        while passes == 0 or secs < min_seconds:
            tok[...] = tok0
            lru[...] = lru0
            for t in range(warmup, warmup + steps):
                t0 = time.perf_counter()
                if len(groups) == 1:
                    rows_copied += part(t, groups[0])
                else:
                    rows_copied += sum(ex.map(lambda g: part(t, g), groups))
                secs += time.perf_counter() - t0
            passes += 1
    return rows_copied, secs, passes


def host_threads():
    """Host cores this process may use, at most 16 (one GPU's share of a host's cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


LEGS = ("headline", "device_pool", "plan_replay", "kv", "paged", "adversarial", "all_layer",
        "scatter", "tiny", "cpu_baseline", "host_link")


def main():
    args = parse()
    if args.only:
        keep = set(args.only.split(","))
        bad = keep - set(LEGS)
        if bad:
            print(f"unknown legs: {sorted(bad)}", file=sys.stderr)
            sys.exit(2)
        for leg in LEGS[1:]:
            setattr(args, "no_" + leg, leg not in keep)
        args.skip_headline = "headline" not in keep
    else:
        args.skip_headline = False
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): requests shard across "
              f"GPUs with no exchange between them, so there is no multi-GPU leg to time.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_kv_hisparse_amd as hs
    from workloads import device as wdev
    from workloads import gen
    hs.load()
    torch.cuda.set_device(0)
    if args.calibrate:
        calibrate(torch, hs)
        return
    if args.copy_ceilings:
        copy_ceilings(torch, hs)
        return
    if args.copy_row_sizes:
        copy_row_sizes(torch, hs, wdev)
        return
    cfg = gen.DSV32

    link = None if args.no_host_link else host_link_ceiling(torch, hs)
    if link:
        log(f"[bench] host link: {json.dumps({k: round(v, 2) for k, v in link.items()})}")

    K = args.steps
    peak = link["h2d_ceiling_gbs"] if link else None
    if args.skip_headline:
        out = {"metric": "swapped-in rows/s + effective GB/s (% of HBM/host-link peak); "
                         "µs per decode-step call", "value": None, "unit": "rows/s", "n_gpus": 1,
               "steps": K, "warmup": args.warmup, "legs": args.only}
    else:
        out = headline(cfg, args, link, peak, torch, hs, wdev)
    legs(cfg, args, out, link, peak, torch, hs, wdev)
    print(json.dumps(out), flush=True)


def headline(cfg, args, link, peak, torch, hs, wdev):
    """The contract's timed region on the DeepSeek-V3.2-like decode trace."""
    r = run_gpu(cfg, args.warmup, args.steps, torch, hs, wdev, b2b_pass=True)
    K = args.steps
    rows = int(r["counts"].sum())
    bytes_link = rows * cfg.row_bytes
    value = rows / r["wall"]
    # Host pools: each call is ONE launch of the resolve kernel with the
    # request's copies fused in. Its mean launch time comes from pass 3: the
    # K launches queued back to back behind a spin kernel, between two events
    # on the launch stream. (Pass 2 reports the split API's two kernels.)
    us_kernel = r["us_b2b"]
    kernel = "resolve_kernel<false, false, 16, false> (resolution + the request's own row copies)"
    fl_us, fl_rows = run_flushed(cfg, 8, 5, torch, hs, wdev)
    achieved = bytes_link / (us_kernel * 1e-6) / 1e9
    call_gbs = bytes_link / (r["us_total"] * 1e-6) / 1e9     # whole call
    return {
        "metric": "swapped-in rows/s + effective GB/s (% of HBM/host-link peak); µs per decode-step call",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall"] / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "dsv32_decode_swap_in_pinned_host_pool", "batch": cfg.B,
                   "context": cfg.ctx, "hot_size": cfg.H, "top_k": cfg.K,
                   "row_bytes": cfg.row_bytes, "pool": "pinned_host", "retention": cfg.rho,
                   "new_ids": "zipf1.1_recency"},
        "us_per_call": round(r["us_total"] / K, 2),
        "launches_per_call": 1,
        "rows_per_call": round(rows / K, 1),
        "split_api": {"us_resolve_kernel": round(r["us_resolve"] / K, 2),
                      "us_copy_kernel": round(r["us_copy"] / K, 2),
                      "GBps_copy_kernel": round(bytes_link / r["us_copy"] / 1e3, 2)},
        "cold_step": {"us": round(r["us_cold"], 2), "rows": r["cold_rows"],
                      "GBps": round(r["cold_rows"] * cfg.row_bytes / r["us_cold"] / 1e3, 2)},
        "effective_GBps_call": round(call_gbs, 2),
        "frac_host_link_call": round(call_gbs / peak, 4) if peak else None,
        "us_per_launch_back_to_back": round(us_kernel / K, 2),
        "steady_state_protocol": {
            "back_to_back_us_per_call": round(r["us_total"] / K, 2),
            "restore_and_flush_us_per_call": round(fl_us, 2),
            "restore_and_flush_rows_per_call": round(fl_rows, 1),
            "note": "median over 8 steps of the median of 5 replays, each from a restored "
                    "state after a 512 MiB write"},
        "roofline": {"bound": "host_link", "kernel": kernel,
                     "timing": "mean launch time, launches queued back to back behind a spin "
                               "kernel, two events on the launch stream",
                     "achieved": round(achieved, 2), "peak": round(peak, 2) if peak else None,
                     "unit": "GB/s", "frac": round(achieved / peak, 4) if peak else None,
                     "peak_published": PCIE5_X16_GBS,
                     "traffic": measured_traffic("dsv32_decode")},
        "host_link": {k: round(v, 2) for k, v in link.items()} if link else None,
    }


def legs(cfg, args, out, link, peak, torch, hs, wdev):
    """Every other leg, each added to `out` under its own key."""
    from workloads import gen
    K = args.steps
    if not args.no_device_pool:
        dcfg = gen.DEVPOOL
        n = args.device_pool_steps
        d = run_gpu(dcfg, 1, n, torch, hs, wdev)
        ceil = hbm_ceiling(torch, hs)
        log(f"[bench] HBM ceiling: {json.dumps(ceil)}")
        fl_us, fl_rows = run_flushed(dcfg, 8, 5, torch, hs, wdev)
        drows = int(d["counts"].sum())
        d_copy = d["us_copy"]
        # algorithmic HBM bytes of the copy kernel: each missed row read once and
        # written once, plus its (pool row, hot row) list entry (12 B)
        dbytes = drows * (2 * dcfg.row_bytes + 12)
        dach = dbytes / (d_copy * 1e-6) / 1e9
        # whole call: rows plus the resolve's own traffic (ids, LRU read and
        # write, slot tokens read, outputs, list) per request
        meta = dcfg.B * (4 * dcfg.K + 2 * dcfg.H * 2 + 4 * dcfg.H + 4 * dcfg.K) * n
        dcall = (drows * 2 * dcfg.row_bytes + meta) / (d["us_total"] * 1e-6) / 1e9
        out["device_pool"] = {
            "workload": "device_pool_swap_in_hbm", "batch": dcfg.B, "context": dcfg.ctx,
            "hot_size": dcfg.H, "top_k": dcfg.K, "row_bytes": dcfg.row_bytes, "steps": n,
            "rows_per_s": round(drows / d["wall"], 1), "rows_per_call": round(drows / n, 1),
            "us_per_call": round(d["us_total"] / n, 2),
            "us_resolve_kernel": round(d["us_resolve"] / n, 2),
            "us_copy_kernel": round(d_copy / n, 2),
            "cold_step": {"us": round(d["us_cold"], 2), "rows": d["cold_rows"],
                          "GBps_rows_read_written": round(
                              d["cold_rows"] * 2 * dcfg.row_bytes / d["us_cold"] / 1e3, 1)},
            "effective_GBps_call": round(dcall, 1), "frac_hbm_call": round(dcall / HBM_PEAK_GBS, 4),
            "steady_state_protocol": {
                "back_to_back_us_per_call": round(d["us_total"] / n, 2),
                "restore_and_flush_us_per_call": round(fl_us, 2),
                "restore_and_flush_rows_per_call": round(fl_rows, 1),
                "note": "median over 8 steps of the median of 5 replays, each from a restored "
                        "state after a 512 MiB write"},
            "hbm_ceiling": dict(ceil, frac_of_peak_library_copy=round(
                ceil["library_copy_contiguous_GBps"] / HBM_PEAK_GBS, 4)),
            "frac_achievable_copy_kernel": round(dach / ceil["library_copy_contiguous_GBps"], 4),
            "roofline": {"bound": "hbm", "kernel": "swap_copy_kernel<16, false, 1024>", "achieved": round(dach, 1),
                         "timing": "mean launch time, copy launches queued back to back behind a "
                                   "spin kernel, two events on the launch stream",
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("device_pool")},
        }

    if not args.no_plan_replay:
        L = args.replay_layers
        pr = run_plan_replay(cfg, L, args.warmup, K, torch, hs, wdev)
        link_bytes = pr["rows"] * cfg.row_bytes * L
        out["plan_replay"] = {
            "workload": "dsv32_decode_index_sharing_layers", "layers": L,
            "rows_per_step_per_layer": round(pr["rows"] / K, 1),
            "us_per_step_fused": round(pr["us_fused"] / K, 2),
            "us_per_step_separate": round(pr["us_separate"] / K, 2),
            "us_replay_kernel": round(pr["us_replay"] / K, 2),
            "GBps_replay_kernel": round(link_bytes / pr["us_replay"] / 1e3, 2),
            "frac_host_link_replay_kernel": round(link_bytes / pr["us_replay"] / 1e3 / peak, 4)
            if peak else None,
            "GBps_step_fused": round(link_bytes / pr["us_fused"] / 1e3, 2),
            "GBps_step_separate": round(link_bytes / pr["us_separate"] / 1e3, 2),
        }

    if not args.no_kv:
        # Non-MLA caches: the headline's shape with 1024-byte K rows and V
        # rows (e.g. 4 KV heads x 128 dims x 2 bytes) in two pinned pools.
        kcfg = gen.KV_DECODE
        n = kcfg.steps - 1
        kr = run_gpu(kcfg, 1, n, torch, hs, wdev, kv=True)
        krows = int(kr["counts"].sum())
        kbytes = krows * kcfg.row_bytes * 2
        kach = kbytes / kr["us_total"] / 1e3
        out["kv_decode"] = {
            "workload": "kv_decode_swap_in_pinned_host_pools", "batch": kcfg.B,
            "context": kcfg.ctx, "hot_size": kcfg.H, "top_k": kcfg.K,
            "row_bytes_k": kcfg.row_bytes, "row_bytes_v": kcfg.row_bytes, "steps": n,
            "rows_per_call": round(krows / n, 1), "us_per_call": round(kr["us_total"] / n, 2),
            "rows_per_s": round(krows / kr["wall"], 1),
            "cold_step": {"us": round(kr["us_cold"], 2), "rows": kr["cold_rows"],
                          "GBps": round(kr["cold_rows"] * kcfg.row_bytes * 2 / kr["us_cold"] / 1e3, 2)},
            "split_api": {"us_resolve_kernel": round(kr["us_resolve"] / n, 2),
                          "us_copy_kernel": round(kr["us_copy"] / n, 2)},
            "roofline": {"bound": "host_link",
                         "kernel": "resolve_kernel<false, false, 16, false> (resolution + K and V row copies)",
                         "achieved": round(kach, 2), "peak": round(peak, 2) if peak else None,
                         "unit": "GB/s", "frac": round(kach / peak, 4) if peak else None,
                         "traffic": measured_traffic("kv_decode")},
        }

    if not args.no_paged:
        # vLLM-style paged addressing (64-row source and hot blocks) on the
        # device-pool and DeepSeek-V3.2-like traces: the same work as the
        # flat legs plus the block-table translation.
        paged_out = {}
        for pcfg, n, flat in ((gen.DEVPOOL, args.device_pool_steps, out.get("device_pool")),
                              (cfg, K, out)):
            pr = run_paged(pcfg, 1, n, torch, hs, wdev)
            us = pr["us_total"] / n
            if pcfg.pool_kind == "device":
                gbs = pr["rows"] * 2 * pcfg.row_bytes / pr["us_total"] / 1e3
                frac = gbs / HBM_PEAK_GBS
            else:
                gbs = pr["rows"] * pcfg.row_bytes / pr["us_total"] / 1e3
                frac = gbs / peak if peak else None
            paged_out[pcfg.name] = {
                "block_size": 64, "steps": n, "us_per_call": round(us, 2),
                "rows_per_call": round(pr["rows"] / n, 1),
                "GBps_call": round(gbs, 1), "frac_bound_call": round(frac, 4) if frac else None,
                "flat_us_per_call": flat.get("us_per_call") if flat else None,
            }
        out["paged"] = paged_out

    if not args.no_adversarial:
        # cold step (all misses, ids that collide in the pages' low-bit hash),
        # then the remaining steps of the 4-step trace
        adv = {}
        for acfg in (gen.ADVERSARIAL, gen.ADVERSARIAL_132, gen.ADVERSARIAL_KERNEL_HASH):
            a = run_gpu(acfg, 1, acfg.steps - 1, torch, hs, wdev, lead_spin=True)
            n = acfg.steps - 1
            arows = int(a["counts"].sum())
            cold_gbs = a["cold_rows"] * acfg.row_bytes / a["us_cold"] / 1e3
            adv[acfg.name] = {
                "batch": acfg.B, "hot_size": acfg.H, "top_k": acfg.K, "context": acfg.ctx,
                "row_bytes": acfg.row_bytes,
                "ids_collide_in": ("the kernel's own hash (top 11 bits of id * 2654435761)"
                                   if acfg.collide_high_bits else
                                   "the pages' hash (id * 2654435761 mod 2^32 mod 2*hot_size)"),
                "cold_step": {"us": round(a["us_cold"], 2), "rows": a["cold_rows"],
                              "GBps": round(cold_gbs, 2),
                              "frac_host_link": round(cold_gbs / peak, 4) if peak else None},
                "steps_after_cold": n, "us_per_call": round(a["us_total"] / n, 2),
                "split_api": {"us_resolve_kernel": round(a["us_resolve"] / n, 2),
                              "us_copy_kernel": round(a["us_copy"] / n, 2)},
                "rows_per_call": round(arows / n, 1),
                "GBps_call": round(arows * acfg.row_bytes / a["us_total"] / 1e3, 2),
            }
        out["adversarial"] = adv

    if not args.no_all_layer:
        tcfg, tbytes, tres = run_all_layer(torch, hs)
        ceil = {"offload": link["d2h_ceiling_gbs"] if link else None,
                "load": link["h2d_ceiling_gbs"] if link else None}
        out["all_layer"] = {
            "workload": "all_layer_transfer", "layers": tcfg.layers,
            "rows_per_layer": tcfg.rows_per_layer, "row_bytes": tcfg.row_bytes,
            "pairs": tcfg.n_pairs, "bytes_per_call": tbytes,
            **{name: {"us_median": round(med, 1), "us_best": round(best, 1),
                      "GBps": round(tbytes / med / 1e3, 2),
                      "frac_host_link": round(tbytes / med / 1e3 / ceil[name], 4) if ceil[name] else None}
               for name, (med, best) in tres.items()},
        }

    if not args.no_scatter:
        n, rb = 8192, 656
        sc = run_scatter(torch, hs, n=n, rb=rb)
        out["scatter"] = {
            "workload": "prefill_chunk_scatter_hbm", "rows": n, "row_bytes": rb,
            "cache_rows": 1 << 20,
            "store_kv_scatter": {"us_median": round(sc["k"], 2),
                                 "GBps": round(n * 2 * rb / sc["k"] / 1e3, 1),
                                 "frac_hbm": round(n * 2 * rb / sc["k"] / 1e3 / HBM_PEAK_GBS, 4)},
            "store_kv_cache": {"us_median": round(sc["kv"], 2),
                               "GBps": round(n * 4 * rb / sc["kv"] / 1e3, 1),
                               "frac_hbm": round(n * 4 * rb / sc["kv"] / 1e3 / HBM_PEAK_GBS, 4)},
        }

    if not args.no_tiny:
        out["tiny"] = run_tiny(torch, hs, wdev)

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the headline steps")
        crow, csec, passes = cpu_baseline(cfg, args.warmup, args.steps, args.cpu_seconds)
        out["cpu_baseline"] = {"value": round(crow / csec, 1), "unit": "rows/s", "cores": 1,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"the headline trace's {args.steps} timed steps "
                                         f"(B={cfg.B}, K={cfg.K}, H={cfg.H}) run {passes} times "
                                         f"from the same starting state, single thread, host "
                                         f"pool image in RAM; {crow} rows in {csec:.2f} s"}
        nt = host_threads()
        if nt > 1:
            log(f"[bench] cpu baseline: oracle on {nt} threads")
            trow, tsec, tpasses = cpu_baseline(cfg, args.warmup, args.steps,
                                               max(3.0, args.cpu_seconds / 2), threads=nt)
            out["cpu_baseline_all_cores"] = {
                "value": round(trow / tsec, 1), "unit": "rows/s", "cores": nt, "kind": "oracle",
                "cpu_model": cpu_model(),
                "sample": f"the same {args.steps} steps run {tpasses} times, each step's {cfg.B} "
                          f"requests split over {nt} threads (one oracle call per group); "
                          f"{trow} rows in {tsec:.2f} s of wall time"}


if __name__ == "__main__":
    main()
