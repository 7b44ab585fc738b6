"""Benchmark of the dependent-GEMM chain on one MI355X.

One step = one MLP chain X[M,12288].W1[12288,6144] -> GeLU -> .W2[6144,12288]
for each M in {256, 512, 1024, 2048} (the GPT-3 MLP slice), each with its
sync policy (TileSync for M <= 256, RowSync above, the per-batch best policy
the cuSync paper reports in its GPT-3 results).  Inputs are synthetic (seeded
normal fp16) and resident in HBM before timing.  W warm-up steps, then K timed
steps between two synchronisations; every chain call inside the timed region
is also bracketed by HIP events on the stream it is launched on, which gives
the per-launch duration of the dominant kernel (the M = 2048 chain, one
launch) for the roofline.  The line printed is the driver's JSON contract with
extra fields: per-M latency and TFLOP/s for every policy against the
stream-serialised pair, the same for the conv-pair and attention chains, the
roofline of the dominant kernel and the CPU oracle timed on host cores.

``--case`` runs one chain call repeatedly and nothing else, followed by a
plain device copy of ``--copy-mib`` MiB (a kernel of known traffic): this is
the program the hardware-counter passes profile.
"""

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("dependent-chain TFLOP/s + latency vs stream-serialised, "
          "GPT-3 MLP slice M=256–2048")
PEAK_F16_TFLOPS = 2516.6      # MI355X dense fp16 MFMA (AMD published, 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
H, F = 12288, 6144
MS = (256, 512, 1024, 2048)
CONV = dict(N=32, Hh=56, Ww=56, C=64, K=64)
ATTN = ((1, 512), (1, 1024), (4, 512), (4, 1024))
RESNET_BATCHES = (1, 8, 32)
HEADS, DHEAD = 96, 128
SA_MS = (16, 64, 256, 512, 1024, 2048)
MLP_SMALL_MS = (1, 16, 64)     # small batches of the pages' 1..2048 sweep (detail only)
SA_HEADS = 12                 # GPT-3 heads held by one of 8 model-parallel GPUs
# Spin of the head-start kernel per timed call (device cycles, about 50 us
# at 2 GHz): longer than the host needs to enqueue one call.
HEAD_START_CYCLES_PER_CALL = 100_000
DETAIL_OUT = os.path.join(ROOT, "bench_detail.json")
LINE_LIMIT = 4096            # bytes of the final contract line


def step_policy(M):
    # Measured on MI355X: TileSync is 1.5-3 % ahead of RowSync up to M = 1024,
    # RowSync ahead at M = 2048 (the 256 x 192 tile's waiting loop).
    return "tilesync" if M <= 1024 else "rowsync"


def chain_flops(M):
    return 4.0 * M * H * F


def chain_bytes(M):
    # weights once, X read, Z written and read back, Y written (fp16)
    return 2.0 * (2 * H * F + M * H + 2 * M * F + M * H)


def conv_flops(batch=CONV["N"], side=CONV["Hh"], ch=CONV["C"]):
    npix = batch * side * side
    return 2 * 2.0 * npix * ch * 9 * ch


def conv_bytes(batch=CONV["N"], side=CONV["Hh"], ch=CONV["C"]):
    npix = batch * side * side
    # X read, Z written and read, Y written, both filters
    return 2.0 * (4 * npix * ch + 18 * ch * ch)


def attn_flops(B, S):
    return 4.0 * B * HEADS * S * S * DHEAD


def attn_bytes(B, S):
    # Q, K, V read, O written, scores written and read back (fp16)
    return 2.0 * (4 * B * HEADS * S * DHEAD + 2 * B * HEADS * S * S)


def sa_flops(M, heads=SA_HEADS):
    hs = heads * DHEAD
    # QKV projection, Q.K^T and P.V per head, output projection
    return 2.0 * M * H * 3 * hs + 4.0 * M * M * hs + 2.0 * M * hs * H


def sa_bytes(M, heads=SA_HEADS):
    hs = heads * DHEAD
    # X, Wqkv, W2 read; XQKV written and read; XDot written and read; Y written (fp16)
    return 2.0 * (M * H + 3 * H * hs + hs * H + 2 * 3 * M * hs + 2 * M * hs + M * H)


# Sources that build the MLP chain (its kernels and their host side): the
# committed traffic counters describe that kernel.
MLP_SOURCES = ("chain_mlp.h", "chain_mlp.hip", "chain_mlp_f16b.hip", "chain_mlp_f16c.hip",
               "chain_mlp_bf16.hip",
               "gemm_tile.h", "device.h", "waits.h", "sched.h", "internal.h", "mlp_api.hip",
               "runtime.hip", "runtime_internal.h")


def src_digest():
    """Digest of the MLP chain's sources with their // comments and blank
    lines removed, so that only a change of its code invalidates the
    committed counters."""
    h = hashlib.sha256()
    for name in sorted(MLP_SOURCES):
        p = os.path.join(ROOT, "tile_level_sync_amd", "csrc", name)
        with open(p, "rb") as f:
            text = f.read().decode("utf-8", "replace")
        code = [re.sub(r"\s*//.*$", "", l).rstrip() for l in text.splitlines()]
        h.update(os.path.basename(p).encode())
        h.update("\n".join(l for l in code if l).encode())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel
    sources (otherwise None)."""
    p = os.path.join(ROOT, "profiles", "mlp_chain_m2048_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("src_digest") != src_digest():
        return None
    return t.get("hbm_bytes_per_launch")


# A call whose bracket exceeds this many times the median of its batch (and
# the median by more than STALL_MIN_US) held a host-side stall: the device sat
# idle between the call's first event and its launch.
STALL_FACTOR = 4.0
STALL_MIN_US = 100.0
STALL_RETAKES = 2


def time_calls(fn, reps, warmup):
    """Device time of ``reps`` back-to-back calls of ``fn`` after ``warmup``
    untimed ones.  A spin kernel is queued first so that the host enqueues
    every call before the device reaches them: the queue never runs dry and
    the figures are device time only, also for chains shorter than the host's
    cost of one call.  Every call is bracketed by events on its stream; the
    mean is the first start to the last end over ``reps`` (gaps included,
    about zero with a full queue), median and min are per call.  A host stall
    longer than the head start (tens of milliseconds, about once in a few
    thousand calls) still lands inside one call's bracket; a batch holding a
    call over STALL_FACTOR times its median is timed again, at most
    STALL_RETAKES times, and ``retaken`` counts those repeats."""
    import torch
    for _ in range(warmup):
        fn()
    for retaken in range(STALL_RETAKES + 1):
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda._sleep(HEAD_START_CYCLES_PER_CALL * reps)
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in evs]  # us
        med = statistics.median(ts)
        if max(ts) <= max(STALL_FACTOR * med, med + STALL_MIN_US):
            break
    span = evs[0][0].elapsed_time(evs[-1][1]) * 1e3
    return {"mean_us": span / reps, "median_us": med, "min_us": min(ts),
            "max_us": max(ts), "retaken": retaken, "_span": span, "_ts": ts}


def _public(r):
    return {k: v for k, v in r.items() if not k.startswith("_")}


DETAIL_ROUNDS = 4


def time_policies(fns, reps, warmup, rounds=DETAIL_ROUNDS):
    """Interleaved timing of several callables (policies, orders, tiles of one
    workload): ``rounds`` rounds, each timing every callable for
    ``reps // rounds`` calls through ``time_calls``, the order rotated by one
    per round so that each callable takes each position in a round equally
    often.  The chip's clock drifts with its power and thermal state over a
    run; timed one after the other, the callables measured last would carry
    that drift alone.  Per callable: the mean over all its calls (spans
    summed), the median, min and max of the single calls."""
    names = list(fns)
    per = max(1, reps // rounds)
    spans = {n: 0.0 for n in names}
    calls = {n: [] for n in names}
    retaken = {n: 0 for n in names}
    for r in range(rounds):
        k = r % len(names)
        for n in names[k:] + names[:k]:
            t = time_calls(fns[n], per, warmup if r == 0 else min(warmup, 2))
            spans[n] += t["_span"]
            calls[n] += t["_ts"]
            retaken[n] += t["retaken"]
    out = {}
    for n in names:
        out[n] = {"mean_us": spans[n] / len(calls[n]), "median_us": statistics.median(calls[n]),
                  "min_us": min(calls[n]), "max_us": max(calls[n]), "calls": len(calls[n])}
        if retaken[n]:
            out[n]["retaken"] = retaken[n]
    return out


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def host_cpus():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count() or 1, "affinity_cpus": aff}


def cpu_baseline(budget_s=12.0):
    """The oracle (float64 numpy, as committed) timed on the host on a bounded
    sample: whole MLP chains at M = 256, 512, 1024, 2048 in turn until about
    ``budget_s`` seconds of oracle time have been spent (the value, in the
    metric's TFLOP/s), then one call of each other configuration (the tiny
    chain, the conv pair, the smallest attention chain) for their times."""
    import oracle
    from tile_level_sync_amd import inputs
    W1, W2 = inputs.mlp_weights(H, F, seed=0)
    Xs = {M: inputs.mlp_x(M, H, seed=0) for M in MS}
    done_flops, elapsed, chains = 0.0, 0.0, 0
    per_m = {}
    while elapsed < budget_s and chains < 64:
        M = MS[chains % len(MS)]
        t0 = time.perf_counter()
        oracle.mlp_chain(Xs[M], W1, W2)
        dt = time.perf_counter() - t0
        per_m.setdefault(M, dt)
        elapsed += dt
        done_flops += chain_flops(M)
        chains += 1
    others = {}
    t0 = time.perf_counter()
    oracle.mlp_chain(*inputs.tiny_mlp_inputs(seed=0))
    others["tiny_mlp"] = time.perf_counter() - t0
    X, Wa, Wb = inputs.resnet_pair_inputs(CONV["N"], seed=0)
    t0 = time.perf_counter()
    oracle.conv_chain(X, Wa, Wb)
    others["conv_32x56x56x64"] = time.perf_counter() - t0
    Q, K, V = inputs.attn_inputs(1, HEADS, 512, DHEAD, seed=0)
    t0 = time.perf_counter()
    oracle.attn_chain(Q, K, V, scale=1.0 / DHEAD ** 0.5)
    others["attn_B1_S512"] = time.perf_counter() - t0
    out = {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()),
           "kind": "oracle",
           "sample": "%d whole float64 oracle MLP chains cycling M=256,512,1024,2048 (H=%d, "
                     "F=%d), %.1f s; value = their flops / time" % (chains, H, F, elapsed),
           "seconds": {"mlp_M%d" % M: round(t, 3) for M, t in per_m.items()}}
    out["seconds"].update({k: round(v, 3) for k, v in others.items()})
    out.update(host_cpus())
    return out


def oracle_full_times():
    """Full-size oracle time per configuration (once each), for the record;
    the default run's cpu_baseline is the bounded sample above."""
    import oracle
    from tile_level_sync_amd import inputs
    rows = []

    def timed(name, fn):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        rows.append((name, dt))
        print("[oracle] %s: %.2f s" % (name, dt), flush=True)

    timed("config 1 tiny MLP 64x256x1024", lambda: oracle.mlp_chain(*inputs.tiny_mlp_inputs(0)))
    W1, W2 = inputs.mlp_weights(H, F, seed=0)
    for M in MS:
        X = inputs.mlp_x(M, H, seed=0)
        timed("config 2 MLP M=%d (config 5 is M=512)" % M,
              lambda X=X: oracle.mlp_chain(X, W1, W2))
    X, Wa, Wb = inputs.resnet_pair_inputs(CONV["N"], seed=0)
    timed("config 4 conv pair 32x56x56x64", lambda: oracle.conv_chain(X, Wa, Wb))
    for B, S in ATTN:
        Q, K, V = inputs.attn_inputs(B, HEADS, S, DHEAD, seed=0)
        timed("config 3 attention B=%d S=%d" % (B, S),
              lambda Q=Q, K=K, V=V: oracle.attn_chain(Q, K, V, scale=1.0 / DHEAD ** 0.5))
    info = dict(host_cpus(), blas_threads=blas_threads())
    print("[oracle] host: %s" % json.dumps(info), flush=True)
    return rows, info


def with_rates(r, flops, nbytes, serial=None):
    r["tflops"] = flops / (r["mean_us"] * 1e-6) / 1e12
    r["frac_peak"] = r["tflops"] / PEAK_F16_TFLOPS
    r["alg_gbs"] = nbytes / (r["mean_us"] * 1e-6) / 1e9
    r["frac_hbm"] = r["alg_gbs"] / PEAK_HBM_GBS
    if serial is not None:
        r["speedup_vs_serial"] = serial["mean_us"] / r["mean_us"]
        r["speedup_vs_serial_median"] = serial["median_us"] / r["median_us"]
    return r


class Workloads:
    """Device-resident synthetic inputs of every chain (built on demand)."""

    def __init__(self, torch, tls, inputs, dev):
        self.torch, self.tls, self.inputs, self.dev = torch, tls, inputs, dev
        self._mlp_w = None
        self._x = {}
        self._y = {}
        self._conv = None
        self._attn = {}
        self._sa_w = None
        self._sa_x = {}

    def _t(self, a):
        return self.torch.from_numpy(a).to(self.dev)

    def mlp(self, M, pol, bf16=False, tile_cfg=None):
        if self._mlp_w is None:
            W1, W2 = self.inputs.mlp_weights(H, F, seed=0)
            self._mlp_w = (self._t(W1), self._t(W2))
        if M not in self._x:
            self._x[M] = self._t(self.inputs.mlp_x(M, H, seed=0))
            self._y[M] = self.torch.empty((M, H), dtype=self.torch.float16, device=self.dev)
        W1, W2 = self._mlp_w
        X, Y = self._x[M], self._y[M]
        if bf16:  # the same values converted to bf16 (timing only)
            bf = self.torch.bfloat16
            W1, W2, X = W1.to(bf), W2.to(bf), X.to(bf)
            Y = self.torch.empty((M, H), dtype=bf, device=self.dev)
        tls = self.tls
        if pol == "sentinel_ring":
            # two rotating intermediates: the fill happens inside the previous call
            ring = tls.SentinelRing(M, F, slots=2, device=self.dev)
            return lambda: tls.chain_mlp(X, W1, W2, Y, policy="sentinel", ring=ring)
        return lambda **kw: tls.chain_mlp(X, W1, W2, Y, policy=pol, tile_cfg=tile_cfg, **kw)

    def conv(self, pol, batch=CONV["N"], side=CONV["Hh"], channels=CONV["C"], tile_cfg=None):
        key = (batch, side, channels)
        if self._conv is None or self._conv[0] != key:
            X, Wa, Wb = self.inputs.resnet_pair_inputs(batch, seed=0, side=side, channels=channels)
            Y = self.torch.empty((batch, side, side, channels), dtype=self.torch.float16,
                                 device=self.dev)
            self._conv = (key, (self._t(X), self._t(Wa), self._t(Wb), Y))
        X, Wa, Wb, Y = self._conv[1]
        tls = self.tls
        if pol == "sentinel_ring":
            ring = tls.SentinelRing(batch * side * side, channels, slots=2, device=self.dev)
            return lambda: tls.chain_conv(X, Wa, Wb, Y, policy="sentinel", ring=ring)
        return lambda **kw: tls.chain_conv(X, Wa, Wb, Y, policy=pol, tile_cfg=tile_cfg, **kw)

    def attn(self, B, S, pol):
        if (B, S) not in self._attn:
            # keep one attention shape resident at a time (B=4, S=1024 needs 1.2 GB)
            self._attn.clear()
            self.torch.cuda.empty_cache()
            Q, K, V = self.inputs.attn_inputs(B, HEADS, S, DHEAD, seed=0)
            O = self.torch.empty((B, HEADS, S, DHEAD), dtype=self.torch.float16, device=self.dev)
            self._attn[(B, S)] = (self._t(Q), self._t(K), self._t(V), O)
        Q, K, V, O = self._attn[(B, S)]
        tls = self.tls
        scale = 1.0 / DHEAD ** 0.5
        if pol == "sentinel_ring":
            ring = tls.SentinelRing(B * HEADS * S, S, slots=2, device=self.dev)
            return lambda: tls.chain_attn(Q, K, V, O, policy="sentinel", scale=scale, ring=ring)
        return lambda **kw: tls.chain_attn(Q, K, V, O, policy=pol, scale=scale, **kw)


    def selfattn(self, M, pol):
        if self._sa_w is None:
            _, Wqkv, W2 = self.inputs.selfattn_inputs(256, H, SA_HEADS, DHEAD, seed=0)
            self._sa_w = (self._t(Wqkv), self._t(W2))
        if M not in self._sa_x:
            # same X stream as selfattn_inputs; avoids regenerating the weights
            X = self.inputs.mlp_x(M, H, seed=0)
            Y = self.torch.empty((M, H), dtype=self.torch.float16, device=self.dev)
            self._sa_x[M] = (self._t(X), Y)
        Wqkv, W2 = self._sa_w
        X, Y = self._sa_x[M]
        tls = self.tls
        return lambda **kw: tls.chain_selfattn(X, Wqkv, W2, Y, policy=pol, heads=SA_HEADS, **kw)


def trace_detail(w, torch, tls):
    """One traced call per (M, policy) after warm-up: per-item records of the
    realtime counter, summarised into busy fraction, tail-wave idle (CU time
    between a CU's last item and the end of the call), the gap between the
    last producer and the first consumer, and consumer waits."""
    from tile_level_sync_amd import trace
    khz = tls.trace_clock_khz()
    ncu = torch.cuda.get_device_properties(w.dev).multi_processor_count
    out = []
    for M, pols in ((64, ("serial", "tilesync")), (256, ("serial", "tilesync")),
                    (2048, ("serial", "rowsync"))):
        plan = tls.chain_mlp_plan(M, H, F)
        P = plan["producer_tiles"] * plan["split_k1"]
        n = tls.mlp_work_items(M, H, F)
        for pol in pols:
            fn = w.mlp(M, pol)
            for _ in range(3):
                fn()
            buf = tls.trace_buffer(n, device=w.dev)
            fn(trace=buf)
            torch.cuda.synchronize()
            srec = trace.summarize(trace.decode(buf), P, khz, n_cu=ncu)
            row = {"M": M, "policy": pol, "work_items": n, "producer_items": P}
            row.update({k: round(v, 4) if isinstance(v, float) else v for k, v in srec.items()})
            out.append(row)
            print("[bench] trace M=%d %s: span %.1f us, busy %.3f, tail idle %.3f, gap %.1f us, "
                  "consumer wait mean %.1f us" % (M, pol, srec["span_us"], srec["busy_frac"],
                                                  srec["tail_idle_frac"],
                                                  srec.get("producer_consumer_gap_us", 0.0),
                                                  srec.get("consumer_wait_mean_us", 0.0)),
                  flush=True)
    # the conv pair (32 x 56 x 56 x 64)
    c = CONV
    plan = tls.chain_conv_plan(c["N"], c["Hh"], c["Ww"], c["C"], c["K"])
    P = plan["producer_tiles"] * plan["split_k1"]
    n = tls.conv_work_items(c["N"], c["Hh"], c["Ww"], c["C"], c["K"])
    for pol in ("serial", "conv2d_tilesync"):
        fn = w.conv(pol)
        for _ in range(3):
            fn()
        buf = tls.trace_buffer(n, device=w.dev)
        fn(trace=buf)
        torch.cuda.synchronize()
        srec = trace.summarize(trace.decode(buf), P, khz, n_cu=ncu)
        row = {"chain": "conv", "policy": pol, "work_items": n, "producer_items": P}
        row.update({k: round(v, 4) if isinstance(v, float) else v for k, v in srec.items()})
        out.append(row)
        print("[bench] trace conv %s: span %.1f us, busy %.3f, tail idle %.3f, gap %.1f us, "
              "consumer wait mean %.1f us" % (pol, srec["span_us"], srec["busy_frac"],
                                              srec["tail_idle_frac"],
                                              srec.get("producer_consumer_gap_us", 0.0),
                                              srec.get("consumer_wait_mean_us", 0.0)), flush=True)
    # the self-attention chain (GPT-3 shard, M = 2048): stage 1 items as producers
    M = 2048
    plan = tls.chain_selfattn_plan(M, H, SA_HEADS)
    n = plan["stage1_items"] + plan["stage2_items"] + plan["stage3_items"]
    for pol in ("serial", "tilesync"):
        fn = w.selfattn(M, pol)
        for _ in range(3):
            fn()
        buf = tls.trace_buffer(n, device=w.dev)
        fn(trace=buf)
        torch.cuda.synchronize()
        srec = trace.summarize(trace.decode(buf), plan["stage1_items"], khz, n_cu=ncu)
        row = {"chain": "selfattn M=%d" % M, "policy": pol, "work_items": n,
               "producer_items": plan["stage1_items"]}
        row.update({k: round(v, 4) if isinstance(v, float) else v for k, v in srec.items()})
        out.append(row)
        print("[bench] trace selfattn %s: span %.1f us, busy %.3f, tail idle %.3f, gap %.1f us, "
              "consumer wait mean %.1f us" % (pol, srec["span_us"], srec["busy_frac"],
                                              srec["tail_idle_frac"],
                                              srec.get("producer_consumer_gap_us", 0.0),
                                              srec.get("consumer_wait_mean_us", 0.0)), flush=True)
    # the attention chain (B = 4, S = 1024, 96 heads)
    B, S = 4, 1024
    n = tls.attn_work_items(B, 96, S)
    for pol in ("serial", "rowsync"):
        fn = w.attn(B, S, pol)
        for _ in range(3):
            fn()
        buf = tls.trace_buffer(n, device=w.dev)
        fn(trace=buf)
        torch.cuda.synchronize()
        srec = trace.summarize(trace.decode(buf), n // 2, khz, n_cu=ncu)
        row = {"chain": "attn B=%d S=%d" % (B, S), "policy": pol, "work_items": n,
               "producer_items": n // 2}
        row.update({k: round(v, 4) if isinstance(v, float) else v for k, v in srec.items()})
        out.append(row)
        print("[bench] trace attn %s: span %.1f us, busy %.3f, tail idle %.3f, gap %.1f us, "
              "consumer wait mean %.1f us" % (pol, srec["span_us"], srec["busy_frac"],
                                              srec["tail_idle_frac"],
                                              srec.get("producer_consumer_gap_us", 0.0),
                                              srec.get("consumer_wait_mean_us", 0.0)), flush=True)
    return out


def case_fn(w, case):
    """``mlp:M:policy[:tile_cfg]`` | ``conv:policy`` | ``conv:batch:side:channels:policy[:cfg]`` |
    ``attn:B:S:policy`` | ``sa:M:policy``."""
    parts = case.split(":")
    if parts[0] == "mlp" and len(parts) in (3, 4):
        cfg = int(parts[3]) if len(parts) == 4 else None
        return w.mlp(int(parts[1]), parts[2], tile_cfg=cfg)
    if parts[0] == "conv" and len(parts) == 2:
        return w.conv(parts[1])
    if parts[0] == "conv" and len(parts) in (5, 6):  # conv:batch:side:channels:policy[:cfg]
        cfg = int(parts[5]) if len(parts) == 6 else None
        return w.conv(parts[4], int(parts[1]), int(parts[2]), int(parts[3]), tile_cfg=cfg)
    if parts[0] == "attn" and len(parts) == 4:
        return w.attn(int(parts[1]), int(parts[2]), parts[3])
    if parts[0] == "sa" and len(parts) == 3:
        return w.selfattn(int(parts[1]), parts[2])
    raise SystemExit("bench.py: unknown --case %r" % case)




def run_case(args, torch, tls, w):
    fn = case_fn(w, args.case)
    for _ in range(args.warmup):
        fn()
    tls.chain_sync()
    r = _public(time_calls(fn, args.steps, 0))
    tls.chain_sync()
    print("[bench] case %s: %s" % (args.case, json.dumps(r)), flush=True)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=w.dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            tls.calibrate_copy(src, dst)
        torch.cuda.synchronize()
        print("[bench] copy calibration (copy16_kernel): %d launches of %d bytes read + %d "
              "written" % (args.steps, n, n), flush=True)


def _line(name, row, pols):
    print("[bench] %s: %s" % (name, ", ".join(
        "%s %.1f us (med %.1f)" % (p, row[p]["mean_us"], row[p]["median_us"]) for p in pols)),
        flush=True)


def detail_mlp(w, tls, reps, warmup):
    out = []
    for M in MS:
        row = {"M": M, "step_policy": step_policy(M), "flops": chain_flops(M),
               "alg_bytes": chain_bytes(M),
               "tile_cfg": tls.tile_configs()[tls.chain_mlp_plan(M, H, F)["tile_cfg"]]}
        pols = ["serial", "tilesync", "rowsync"] + (["sentinel", "sentinel_ring"]
                                                     if M == 512 else [])
        ts = time_policies({pol: w.mlp(M, pol) for pol in pols}, reps, warmup)
        for pol in pols:
            row[pol] = with_rates(ts[pol], chain_flops(M), chain_bytes(M), row.get("serial"))
        tls.chain_sync()
        out.append(row)
        _line("mlp M=%d" % M, row, pols)
    return out


def detail_tiny(w, torch, tls, inputs, reps, warmup):
    """The tiny chain X[64x256].W1[256x1024].W2[1024x256] (all N(0, 0.02))."""
    X, W1, W2 = (torch.from_numpy(a).to(w.dev) for a in inputs.tiny_mlp_inputs(seed=0))
    Y = torch.empty((64, 256), dtype=torch.float16, device=w.dev)
    fl = 4.0 * 64 * 256 * 1024
    nb = 2.0 * (2 * 256 * 1024 + 64 * 256 + 2 * 64 * 1024 + 64 * 256)
    row = {"shape": "64x256x1024", "flops": fl, "alg_bytes": nb}
    pols = ("serial", "tilesync", "rowsync")
    ts = time_policies({pol: (lambda pol=pol: tls.chain_mlp(X, W1, W2, Y, policy=pol))
                        for pol in pols}, reps, warmup)
    for pol in pols:
        row[pol] = with_rates(ts[pol], fl, nb, row.get("serial"))
    tls.chain_sync()
    _line("tiny mlp 64x256x1024", row, ("serial", "tilesync", "rowsync"))
    return row


def detail_small_and_bf16(w, tls, reps, warmup):
    small = []
    for M in MLP_SMALL_MS:
        row = {"M": M, "flops": chain_flops(M), "alg_bytes": chain_bytes(M)}
        pols = ("serial", "tilesync", "rowsync")
        ts = time_policies({pol: w.mlp(M, pol) for pol in pols}, reps, warmup)
        for pol in pols:
            row[pol] = with_rates(ts[pol], chain_flops(M), chain_bytes(M), row.get("serial"))
        tls.chain_sync()
        small.append(row)
        _line("mlp M=%d" % M, row, ("serial", "tilesync", "rowsync"))
    bf = []
    for M in (256, 2048):
        row = {"M": M, "dtype": "bf16", "flops": chain_flops(M), "alg_bytes": chain_bytes(M)}
        pols = ("serial", step_policy(M))
        ts = time_policies({pol: w.mlp(M, pol, bf16=True) for pol in pols}, reps, warmup)
        for pol in pols:
            row[pol] = with_rates(ts[pol], chain_flops(M), chain_bytes(M), row.get("serial"))
        tls.chain_sync()
        bf.append(row)
        _line("mlp bf16 M=%d" % M, row, pols)
    return small, bf


def detail_conv(w, tls, inputs, reps, warmup):
    pols = ("serial", "conv2d_tilesync", "rowsync", "sentinel", "sentinel_ring")
    row = {"shape": "NHWC [32,56,56,64] -> 64 -> 64, 3x3 pad 1", "flops": conv_flops(),
           "alg_bytes": conv_bytes()}
    ts = time_policies({pol: w.conv(pol) for pol in pols}, reps, warmup)
    for pol in pols:
        row[pol] = with_rates(ts[pol], conv_flops(), conv_bytes(), row.get("serial"))
    tls.chain_sync()
    _line("conv 32x56x56x64", row, pols)
    # the same pair in bf16 (values drawn as for the fp16 pair, rounded to bf16)
    import numpy as np
    import torch
    Xb, Wab, Wbb = (torch.from_numpy(a.view(np.int16)).to(w.dev).view(torch.bfloat16)
                    for a in inputs.conv_inputs_bf16(CONV["N"], CONV["Hh"], CONV["Ww"],
                                                     CONV["C"], CONV["K"], seed=0))
    Yb = torch.empty((CONV["N"], CONV["Hh"], CONV["Ww"], CONV["K"]), dtype=torch.bfloat16,
                     device=w.dev)
    bp = ("serial", "conv2d_tilesync")
    ts = time_policies({pol: (lambda pol=pol: tls.chain_conv(Xb, Wab, Wbb, Yb, policy=pol))
                        for pol in bp}, reps, warmup)
    row["bf16"] = {pol: with_rates(ts[pol], conv_flops(), conv_bytes()) for pol in bp}
    row["bf16"]["conv2d_tilesync"]["speedup_vs_serial"] = (ts["serial"]["mean_us"] /
                                                         ts["conv2d_tilesync"]["mean_us"])
    tls.chain_sync()
    _line("conv 32x56x56x64 bf16", row["bf16"], bp)
    sweep = []
    for side, ch in inputs.RESNET38_PAIRS:
        for b in RESNET_BATCHES:
            r = {"batch": b, "side": side, "channels": ch}
            cp = ("serial", "conv2d_tilesync", "rowsync")
            ts = time_policies({pol: w.conv(pol, b, side, ch) for pol in cp}, reps, warmup)
            for pol in cp:
                r[pol] = with_rates(ts[pol], conv_flops(b, side, ch), conv_bytes(b, side, ch),
                                    r.get("serial"))
            tls.chain_sync()
            sweep.append(r)
            _line("resnet38 %dx%dx%d b%d" % (side, side, ch, b), r,
                  ("serial", "conv2d_tilesync", "rowsync"))
    return row, sweep


def detail_attn(w, tls, reps, warmup):
    pols = ("serial", "tilesync", "rowsync", "sentinel", "sentinel_ring")
    out = []
    for B, S in ATTN:
        row = {"B": B, "S": S, "heads": HEADS, "d": DHEAD, "flops": attn_flops(B, S),
               "alg_bytes": attn_bytes(B, S)}
        ts = time_policies({pol: w.attn(B, S, pol) for pol in pols}, reps, warmup)
        for pol in pols:
            row[pol] = with_rates(ts[pol], attn_flops(B, S), attn_bytes(B, S), row.get("serial"))
        tls.chain_sync()
        out.append(row)
        _line("attn B=%d S=%d" % (B, S), row, pols)
    # the largest shape in bf16 (values drawn as for fp16, rounded to bf16)
    import numpy as np
    B, S = ATTN[-1]
    w._attn.clear()
    w.torch.cuda.empty_cache()
    Qb, Kb, Vb = (w.torch.from_numpy(a.view(np.int16)).to(w.dev).view(w.torch.bfloat16)
                  for a in w.inputs.attn_inputs_bf16(B, HEADS, S, DHEAD, seed=0))
    Ob = w.torch.empty_like(Qb)
    bp = ("serial", "rowsync")
    ts = time_policies({pol: (lambda pol=pol: tls.chain_attn(Qb, Kb, Vb, Ob, policy=pol,
                                                             scale=1.0 / DHEAD ** 0.5))
                        for pol in bp}, reps, warmup)
    row = {"B": B, "S": S, "heads": HEADS, "d": DHEAD, "dtype": "bf16"}
    for pol in bp:
        row[pol] = with_rates(ts[pol], attn_flops(B, S), attn_bytes(B, S), row.get("serial"))
    tls.chain_sync()
    del Qb, Kb, Vb, Ob
    w.torch.cuda.empty_cache()
    out.append(row)
    _line("attn B=%d S=%d bf16" % (B, S), row, bp)
    return out


def detail_selfattn(w, tls, reps, warmup):
    pols = ("serial", "stridedsync", "tilesync")
    out = []
    for M in SA_MS:
        row = {"M": M, "H": H, "heads": SA_HEADS, "d": DHEAD, "flops": sa_flops(M),
               "alg_bytes": sa_bytes(M)}
        ts = time_policies({pol: w.selfattn(M, pol) for pol in pols}, reps, warmup)
        for pol in pols:
            row[pol] = with_rates(ts[pol], sa_flops(M), sa_bytes(M), row.get("serial"))
        tls.chain_sync()
        out.append(row)
        _line("self-attention M=%d" % M, row, pols)
    # the largest M in bf16 (values drawn as for fp16, rounded to bf16)
    import numpy as np
    M = SA_MS[-1]
    Xb, Wqb, W2b = (w.torch.from_numpy(a.view(np.int16)).to(w.dev).view(w.torch.bfloat16)
                    for a in w.inputs.selfattn_inputs_bf16(M, H, SA_HEADS, DHEAD, seed=0))
    Yb = w.torch.empty((M, H), dtype=w.torch.bfloat16, device=w.dev)
    bp = ("serial", "stridedsync")
    ts = time_policies({pol: (lambda pol=pol: tls.chain_selfattn(Xb, Wqb, W2b, Yb, policy=pol,
                                                                 heads=SA_HEADS))
                        for pol in bp}, reps, warmup)
    row = {"M": M, "H": H, "heads": SA_HEADS, "d": DHEAD, "dtype": "bf16"}
    for pol in bp:
        row[pol] = with_rates(ts[pol], sa_flops(M), sa_bytes(M), row.get("serial"))
    tls.chain_sync()
    del Xb, Wqb, W2b, Yb
    out.append(row)
    _line("self-attention M=%d bf16" % M, row, bp)
    return out


def detail_orders(w, tls, reps, warmup):
    """Tile orders of the cuSync paper's "Tile Processing Order" against the
    default (per-XCD column slabs for the MLP, one global row-major counter
    for attention)."""
    out = []
    for M, pol in ((2048, "rowsync"), (512, "tilesync")):
        row = {"chain": "mlp M=%d" % M, "policy": pol}
        fn = w.mlp(M, pol)
        row.update(time_policies({order: (lambda order=order: fn(order=order))
                                  for order in ("xcd", "row_major", "col_major", "strided",
                                                "interleaved")}, reps, warmup))
        tls.chain_sync()
        out.append(row)
        _line("orders mlp M=%d %s" % (M, pol), row,
              ("xcd", "row_major", "col_major", "strided", "interleaved"))
    B, S = 4, 1024
    row = {"chain": "attn B=%d S=%d" % (B, S), "policy": "rowsync"}
    fn = w.attn(B, S, "rowsync")
    row.update(time_policies({order: (lambda order=order: fn(order=order))
                              for order in ("row_major", "col_major", "strided", "interleaved")},
                             reps, warmup))
    tls.chain_sync()
    out.append(row)
    _line("orders attn B=%d S=%d rowsync" % (B, S), row,
          ("row_major", "col_major", "strided", "interleaved"))
    return out


def vs_serial_summary(mlp_rows):
    """Per M: the step policy's chain latency against the stream-serialised
    pair (mean us of the interleaved detail run) and the speedup; where the
    sentinel protocol was timed (M = 512, config 5) its plain and ring
    latencies beside them."""
    out = {}
    for r in mlp_rows:
        pol = r["step_policy"]
        e = {"policy": pol, "chain_us": round(r[pol]["mean_us"], 1),
             "serial_us": round(r["serial"]["mean_us"], 1),
             "speedup": round(r["serial"]["mean_us"] / r[pol]["mean_us"], 3)}
        for k in ("sentinel", "sentinel_ring"):
            if k in r:
                e[k + "_us"] = round(r[k]["mean_us"], 1)
        out[str(r["M"])] = e
    return out


def contract_line(value, step_ms, steps, warmup, per_m_us, roofline, cpu, vs_serial):
    """The final JSON line (compact: every per-policy figure goes to the
    detail file and the earlier [bench] lines)."""
    def rnd(x, n=4):
        return round(x, n) if isinstance(x, float) else x
    out = {
        "metric": METRIC, "value": rnd(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": rnd(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "GPT-3 MLP slice chain X[M,12288].W1[12288,6144] -> GeLU -> "
                               ".W2[6144,12288], one chain per M in {256,512,1024,2048} per "
                               "step, fp16 storage / fp32 accumulation",
                   "H": H, "F": F, "M": list(MS),
                   "policy": {str(M): step_policy(M) for M in MS},
                   "per_chain_us": {str(M): rnd(per_m_us.get(M), 1) for M in MS},
                   "parallelism": "single GPU"},
        "roofline": {k: rnd(v) for k, v in roofline.items()},
        "cpu_baseline": cpu,
    }
    if vs_serial:
        out["vs_serial"] = vs_serial
    return json.dumps(out, separators=(",", ":"), ensure_ascii=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="timed calls per detail entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--detail-out", default=DETAIL_OUT,
                    help="file that receives the per-policy detail (JSON)")
    ap.add_argument("--case", default=None,
                    help="run only this chain call (mlp:M:policy, conv:policy, "
                         "conv:batch:side:channels:policy, attn:B:S:policy, sa:M:policy)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --case: then run a plain device copy of this many MiB")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the sustained dense fp16 MFMA rate and clock and exit")
    ap.add_argument("--oracle-times", action="store_true",
                    help="time the full-size oracle of every configuration on the host "
                         "and exit (no GPU)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the chain runs on a single "
              "MI355X); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.oracle_times:
        oracle_full_times()
        return

    import torch
    import tile_level_sync_amd as tls
    from tile_level_sync_amd import inputs

    tls.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = Workloads(torch, tls, inputs, dev)
    if args.case:
        run_case(args, torch, tls, w)
        return
    if args.calibrate:
        for wps in (1, 2):
            for rep in range(3):
                c = tls.calibrate_mfma(wps, 20000)
                print("[bench] calibrate waves/SIMD %d rep %d: %.1f TFLOP/s dense fp16 MFMA "
                      "(%.3f of %.1f), shader clock %.3f GHz, %.3f ms"
                      % (wps, rep, c["tflops"], c["tflops"] / PEAK_F16_TFLOPS, PEAK_F16_TFLOPS,
                         c["ghz"], c["ms"]), flush=True)
        return

    calls = [(M, w.mlp(M, step_policy(M))) for M in MS]
    print("[bench] inputs resident", flush=True)

    Mx = max(MS)

    def step(evs=None, only=None):
        # evs[i] brackets chain i with two events; with `only`, just that M.
        for i, (M, fn) in enumerate(calls):
            rec = evs is not None and (only is None or M == only)
            if rec:
                evs[i][0].record()
            fn()
            if rec:
                evs[i][1].record()

    for _ in range(args.warmup):
        step()
    tls.chain_sync()
    torch.cuda.synchronize()
    # Timed region: only the dominant chain's calls are bracketed by events
    # (the roofline needs its launch time); an event pair between two
    # back-to-back chains adds a few microseconds to the step.
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in MS]
          for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(args.steps):
        step(ev[s], only=Mx)
    t1.record()
    torch.cuda.synchronize()
    tls.chain_sync()
    step_ms = t0.elapsed_time(t1) / args.steps
    step_flops = sum(chain_flops(M) for M in MS)
    value = step_flops / (step_ms * 1e-3) / 1e12
    ix = MS.index(Mx)
    launch_us = statistics.fmean(ev[s][ix][0].elapsed_time(ev[s][ix][1]) * 1e3
                                 for s in range(args.steps))
    # The other chains' latencies come from the interleaved detail run (when
    # it runs); `value` is the timed region alone.
    per_m_us = {Mx: launch_us}
    print("[bench] timed %d steps: %.3f ms/step, %.1f TFLOP/s; M = %d launch %.1f us"
          % (args.steps, step_ms, value, Mx, launch_us), flush=True)

    # Roofline of the dominant kernel: the M = 2048 chain, one launch per call,
    # its duration from the events around it inside the timed region.
    ach = chain_flops(Mx) / (per_m_us[Mx] * 1e-6) / 1e12
    cfg = tls.chain_mlp_plan(Mx, H, F)["tile_cfg"]
    tc = tls.tile_configs()[cfg]
    roofline = {"bound": "mfma", "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_F16_TFLOPS, "traffic": load_traffic(),
                "launch_us": per_m_us[Mx],
                "kernel": "mlp_chain_kernel cfg %d: %dx%dx%d tile, %d threads, %s (M=%d, "
                          "one launch per call)" % (cfg, tc["bm"], tc["bn1"], tc["bk"],
                                                     tc["threads"], step_policy(Mx), Mx)}
    # The published peak assumes the top clock; the chip's sustained MFMA
    # rate under a pure MFMA load (calibration kernel, median of three
    # launches) says how much of it this device actually delivers.
    cal = sorted((tls.calibrate_mfma(2, 20000) for _ in range(3)), key=lambda c: c["tflops"])[1]
    roofline["sustained_mfma_tflops"] = cal["tflops"]
    roofline["sustained_mfma_ghz"] = cal["ghz"]
    roofline["frac_of_sustained"] = ach / cal["tflops"]
    print("[bench] roofline: %s" % json.dumps(roofline), flush=True)

    detail, vs_serial = {}, None
    if not args.no_detail:
        r, wu = args.reps, args.warmup
        detail["mlp"] = detail_mlp(w, tls, r, wu)
        vs_serial = vs_serial_summary(detail["mlp"])
        for row in detail["mlp"]:  # the step policy's latency for the other chains
            per_m_us.setdefault(row["M"], row[row["step_policy"]]["mean_us"])
        detail["tiny"] = detail_tiny(w, torch, tls, inputs, r, wu)
        detail["mlp_small_batch"], detail["mlp_bf16"] = detail_small_and_bf16(w, tls, r, wu)
        detail["trace"] = trace_detail(w, torch, tls)
        detail["conv"], detail["resnet38_pairs"] = detail_conv(w, tls, inputs, r, wu)
        detail["attn"] = detail_attn(w, tls, r, wu)
        detail["selfattn"] = detail_selfattn(w, tls, r, wu)
        detail["orders"] = detail_orders(w, tls, r, wu)
        try:
            os.makedirs(os.path.dirname(os.path.abspath(args.detail_out)), exist_ok=True)
            with open(args.detail_out, "w") as f:
                json.dump(detail, f, indent=1)
            print("[bench] detail written to %s" % args.detail_out, flush=True)
        except OSError as e:  # pragma: no cover
            print("[bench] detail not written: %s" % e, flush=True)

    cpu = None if args.no_cpu_baseline else cpu_baseline()
    print(contract_line(value, step_ms, args.steps, args.warmup, per_m_us, roofline, cpu,
                        vs_serial), flush=True)


if __name__ == "__main__":
    main()
