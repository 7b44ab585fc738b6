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
MLP_SOURCES = ("chain_mlp.h", "chain_mlp.hip", "chain_mlp_f16b.hip", "chain_mlp_bf16.hip",
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


def time_calls(fn, reps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in evs]  # us
    return {"mean_us": statistics.fmean(ts), "median_us": statistics.median(ts),
            "min_us": min(ts)}


def cpu_baseline(budget_s=12.0):
    """The oracle (float64 numpy, as committed) timed on the host on a bounded
    sample: whole chains at M = 256, 512, 1024, 2048 in turn, repeated until
    about ``budget_s`` seconds of oracle time have been spent."""
    import oracle
    from tile_level_sync_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    W1, W2 = inputs.mlp_weights(H, F, seed=0)
    Xs = {M: inputs.mlp_x(M, H, seed=0) for M in MS}
    done_flops, elapsed, chains = 0.0, 0.0, 0
    while elapsed < budget_s and chains < 64:
        M = MS[chains % len(MS)]
        t0 = time.perf_counter()
        oracle.mlp_chain(Xs[M], W1, W2)
        elapsed += time.perf_counter() - t0
        done_flops += chain_flops(M)
        chains += 1
    return {"value": done_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": "%d whole float64 oracle chains cycling M=256,512,1024,2048 (H=%d, F=%d), "
                      "%.1f s" % (chains, H, F, elapsed)}


def with_rates(r, flops, nbytes, serial=None):
    r["tflops"] = flops / (r["mean_us"] * 1e-6) / 1e12
    r["frac_peak"] = r["tflops"] / PEAK_F16_TFLOPS
    r["alg_gbs"] = nbytes / (r["mean_us"] * 1e-6) / 1e9
    r["frac_hbm"] = r["alg_gbs"] / PEAK_HBM_GBS
    if serial is not None:
        r["speedup_vs_serial"] = serial["mean_us"] / r["mean_us"]
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

    def mlp(self, M, pol, bf16=False):
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
        return lambda **kw: tls.chain_mlp(X, W1, W2, Y, policy=pol, **kw)

    def conv(self, pol, batch=CONV["N"], side=CONV["Hh"], channels=CONV["C"]):
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
        return lambda **kw: tls.chain_conv(X, Wa, Wb, Y, policy=pol, **kw)

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
    """``mlp:M:policy`` | ``conv:policy`` | ``conv:batch:side:channels:policy`` |
    ``attn:B:S:policy`` | ``sa:M:policy``."""
    parts = case.split(":")
    if parts[0] == "mlp" and len(parts) == 3:
        return w.mlp(int(parts[1]), parts[2])
    if parts[0] == "conv" and len(parts) == 2:
        return w.conv(parts[1])
    if parts[0] == "conv" and len(parts) == 5:  # conv:batch:side:channels:policy
        return w.conv(parts[4], int(parts[1]), int(parts[2]), int(parts[3]))
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
    r = time_calls(fn, args.steps, 0)
    tls.chain_sync()
    print("[bench] case %s: %s" % (args.case, json.dumps(r)), flush=True)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=w.dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: %d launches of %d bytes read + %d written"
              % (args.steps, n, n), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="timed calls per detail entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--case", default=None,
                    help="run only this chain call (mlp:M:policy, conv:policy, "
                         "conv:batch:side:channels:policy, attn:B:S:policy, sa:M:policy)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --case: then run a plain device copy of this many MiB")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the chain runs on a single "
              "MI355X); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

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

    calls = [(M, w.mlp(M, step_policy(M))) for M in MS]
    print("[bench] inputs resident", flush=True)

    def step(evs=None):
        for i, (M, fn) in enumerate(calls):
            if evs is not None:
                evs[i][0].record()
            fn()
            if evs is not None:
                evs[i][1].record()

    for _ in range(args.warmup):
        step()
    tls.chain_sync()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in MS]
          for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(args.steps):
        step(ev[s])
    t1.record()
    torch.cuda.synchronize()
    tls.chain_sync()
    step_ms = t0.elapsed_time(t1) / args.steps
    step_flops = sum(chain_flops(M) for M in MS)
    value = step_flops / (step_ms * 1e-3) / 1e12
    per_m_us = {M: statistics.fmean(ev[s][i][0].elapsed_time(ev[s][i][1]) * 1e3
                                    for s in range(args.steps))
                for i, M in enumerate(MS)}
    print("[bench] timed %d steps: %.3f ms/step; per chain (us): %s"
          % (args.steps, step_ms, {M: round(t, 1) for M, t in per_m_us.items()}), flush=True)

    # Roofline of the dominant kernel: the M = 2048 chain, one launch per call,
    # its duration from the events around it inside the timed region.
    Mx = max(MS)
    ach = chain_flops(Mx) / (per_m_us[Mx] * 1e-6) / 1e12
    cfg = tls.chain_mlp_plan(Mx, H, F)["tile_cfg"]
    tc = tls.tile_configs()[cfg]
    roofline = {"bound": "mfma", "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_F16_TFLOPS, "traffic": load_traffic(),
                "launch_us": per_m_us[Mx],
                "kernel": "mlp_chain_kernel<%d,%d,%d,...,%s> (M=%d, one launch per call)"
                          % (tc["bm"], tc["bn1"], tc["bn2"], step_policy(Mx), Mx)}

    detail = {}
    if not args.no_detail:
        mlp = []
        for M in MS:
            row = {"M": M, "step_policy": step_policy(M), "flops": chain_flops(M),
                   "alg_bytes": chain_bytes(M),
                   "tile_cfg": tls.tile_configs()[tls.chain_mlp_plan(M, H, F)["tile_cfg"]]}
            pols = ["serial", "tilesync", "rowsync"] + (["sentinel", "sentinel_ring"]
                                                         if M == 512 else [])
            for pol in pols:
                row[pol] = with_rates(time_calls(w.mlp(M, pol), args.reps, args.warmup),
                                      chain_flops(M), chain_bytes(M), row.get("serial"))
            tls.chain_sync()
            mlp.append(row)
            print("[bench] mlp M=%d: %s" % (M, ", ".join(
                "%s %.1f us" % (p, row[p]["mean_us"]) for p in pols)), flush=True)
        detail["mlp"] = mlp
        small = []
        for M in MLP_SMALL_MS:
            row = {"M": M, "flops": chain_flops(M), "alg_bytes": chain_bytes(M)}
            for pol in ("serial", "tilesync", "rowsync"):
                row[pol] = with_rates(time_calls(w.mlp(M, pol), args.reps, args.warmup),
                                      chain_flops(M), chain_bytes(M), row.get("serial"))
            tls.chain_sync()
            small.append(row)
            print("[bench] mlp M=%d: %s" % (M, ", ".join(
                "%s %.1f us" % (p, row[p]["mean_us"]) for p in ("serial", "tilesync", "rowsync"))),
                flush=True)
        detail["mlp_small_batch"] = small
        bf = []
        for M in (256, 2048):
            row = {"M": M, "dtype": "bf16", "flops": chain_flops(M), "alg_bytes": chain_bytes(M)}
            for pol in ("serial", step_policy(M)):
                row[pol] = with_rates(time_calls(w.mlp(M, pol, bf16=True), args.reps,
                                                 args.warmup),
                                      chain_flops(M), chain_bytes(M), row.get("serial"))
            tls.chain_sync()
            bf.append(row)
            print("[bench] mlp bf16 M=%d: %s" % (M, ", ".join(
                "%s %.1f us" % (p, row[p]["mean_us"]) for p in ("serial", step_policy(M)))),
                flush=True)
        detail["mlp_bf16"] = bf
        detail["trace"] = trace_detail(w, torch, tls)
        row = {"shape": "NHWC [32,56,56,64] -> 64 -> 64, 3x3 pad 1", "flops": conv_flops(),
               "alg_bytes": conv_bytes()}
        for pol in ("serial", "conv2d_tilesync", "rowsync", "sentinel", "sentinel_ring"):
            row[pol] = with_rates(time_calls(w.conv(pol), args.reps, args.warmup),
                                  conv_flops(), conv_bytes(), row.get("serial"))
        tls.chain_sync()
        detail["conv"] = row
        sweep = []
        for side, ch in inputs.RESNET38_PAIRS:
            for b in RESNET_BATCHES:
                r = {"batch": b, "side": side, "channels": ch}
                for pol in ("serial", "conv2d_tilesync", "rowsync"):
                    r[pol] = with_rates(time_calls(w.conv(pol, b, side, ch), args.reps, args.warmup),
                                        conv_flops(b, side, ch), conv_bytes(b, side, ch),
                                        r.get("serial"))
                tls.chain_sync()
                sweep.append(r)
        detail["resnet38_pairs"] = sweep
        print("[bench] resnet38 pairs: %s" % "; ".join(
            "%dx%dx%d b%d %.1f/%.1f/%.1f us" % (r["side"], r["side"], r["channels"], r["batch"],
                                                r["serial"]["mean_us"],
                                                r["conv2d_tilesync"]["mean_us"],
                                                r["rowsync"]["mean_us"]) for r in sweep),
              flush=True)
        print("[bench] conv: %s" % ", ".join("%s %.1f us" % (p, row[p]["mean_us"]) for p in
                                             ("serial", "conv2d_tilesync", "rowsync",
                                              "sentinel", "sentinel_ring")), flush=True)
        attn = []
        for B, S in ATTN:
            row = {"B": B, "S": S, "heads": HEADS, "d": DHEAD, "flops": attn_flops(B, S),
                   "alg_bytes": attn_bytes(B, S)}
            for pol in ("serial", "tilesync", "rowsync", "sentinel", "sentinel_ring"):
                row[pol] = with_rates(time_calls(w.attn(B, S, pol), args.reps, args.warmup),
                                      attn_flops(B, S), attn_bytes(B, S), row.get("serial"))
            tls.chain_sync()
            attn.append(row)
            print("[bench] attn B=%d S=%d: %s" % (B, S, ", ".join(
                "%s %.1f us" % (p, row[p]["mean_us"]) for p in
                ("serial", "tilesync", "rowsync", "sentinel", "sentinel_ring"))), flush=True)
        detail["attn"] = attn
        sa = []
        for M in SA_MS:
            row = {"M": M, "H": H, "heads": SA_HEADS, "d": DHEAD, "flops": sa_flops(M),
                   "alg_bytes": sa_bytes(M)}
            for pol in ("serial", "stridedsync", "tilesync"):
                row[pol] = with_rates(time_calls(w.selfattn(M, pol), args.reps, args.warmup),
                                      sa_flops(M), sa_bytes(M), row.get("serial"))
            tls.chain_sync()
            sa.append(row)
            print("[bench] self-attention M=%d: %s" % (M, ", ".join(
                "%s %.1f us" % (p, row[p]["mean_us"]) for p in
                ("serial", "stridedsync", "tilesync"))), flush=True)
        detail["selfattn"] = sa

    cpu = None if args.no_cpu_baseline else cpu_baseline()

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "GPT-3 MLP slice chain X[M,12288].W1[12288,6144] -> GeLU -> "
                               ".W2[6144,12288], one chain per M in {256,512,1024,2048} per "
                               "step, fp16 storage / fp32 accumulation",
                   "H": H, "F": F, "M": list(MS),
                   "policy": {str(M): step_policy(M) for M in MS},
                   "per_chain_us": {str(M): per_m_us[M] for M in MS},
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
