"""Decoding and summarising the optional per-item trace of a chain call.

Every work item of a traced call writes one record (``chain_trace_rec`` of the
C ABI): its index, the persistent workgroup that ran it, the CU it ran on, and
three times of the GPU's constant-rate realtime counter -- taken from the
scheduler, first dependency wait returned, finished.  ``summarize`` turns the
records of one call (one launch, or the two stream-ordered launches of the
serial baseline) into what the measurement reports: the span, the fraction of
CU time spent running items, the idle time each CU has between its last item
and the end of the call (tail-wave idle), the gap between the last producer
and the first consumer, and how long consumers waited for their producers.

Host-side numpy only; nothing here runs on the GPU.
"""

import numpy as np

REC = np.dtype([("item", "<u4"), ("wg", "<u2"), ("hw", "<u2"), ("t_start", "<u8"),
                ("t_ready", "<u8"), ("t_end", "<u8")])
assert REC.itemsize == 32


def decode(buf):
    """Records of a trace buffer (a uint8 tensor or bytes-like) that were
    written (t_end != 0), in item order."""
    if hasattr(buf, "cpu"):
        buf = buf.cpu().numpy()
    a = np.frombuffer(np.asarray(buf, dtype=np.uint8).tobytes(), dtype=REC)
    return a[a["t_end"] != 0]


def _covered(starts, ends):
    """Total length covered by the union of intervals [starts[i], ends[i])."""
    order = np.argsort(starts, kind="stable")
    total, cur_s, cur_e = 0, None, None
    for s, e in zip(starts[order], ends[order]):
        s, e = int(s), int(e)
        if cur_e is None or s > cur_e:
            if cur_e is not None:
                total += cur_e - cur_s
            cur_s, cur_e = s, e
        else:
            cur_e = max(cur_e, e)
    if cur_e is not None:
        total += cur_e - cur_s
    return total


def summarize(recs, producer_items, clock_khz, n_cu=None):
    """Summary of one call's records.  ``producer_items`` is the number of
    producer work items (items below it are producers); ``clock_khz`` the
    trace clock rate; ``n_cu`` the CUs of the device (default: those seen).
    Times in microseconds."""
    if len(recs) == 0:
        raise ValueError("no trace records")
    us = 1000.0 / float(clock_khz)
    t0 = int(recs["t_start"].min())
    t1 = int(recs["t_end"].max())
    span = t1 - t0
    cus = np.unique(recs["hw"])
    n = int(n_cu) if n_cu is not None else len(cus)
    busy = 0
    tail = 0
    for c in cus:
        r = recs[recs["hw"] == c]
        busy += _covered(r["t_start"], r["t_end"])
        tail += t1 - int(r["t_end"].max())
    tail += (n - len(cus)) * span  # CUs that ran nothing idle the whole call
    prod = recs[recs["item"] < producer_items]
    cons = recs[recs["item"] >= producer_items]
    out = {
        "span_us": span * us,
        "cus": n,
        "busy_frac": busy / (n * span) if span else 1.0,
        "tail_idle_frac": tail / (n * span) if span else 0.0,
        "items": int(len(recs)),
    }
    if len(prod):
        out["producer_phase_us"] = (int(prod["t_end"].max()) - t0) * us
    if len(cons):
        wait = (cons["t_ready"].astype(np.int64) - cons["t_start"].astype(np.int64)) * us
        out["consumer_wait_mean_us"] = float(wait.mean())
        out["consumer_wait_max_us"] = float(wait.max())
        out["consumer_wait_total_cu_frac"] = float(wait.sum() / us / (n * span)) if span else 0.0
    if len(prod) and len(cons):
        # positive: the consumers started only after the producers ended (a kernel boundary)
        out["producer_consumer_gap_us"] = (int(cons["t_start"].min()) -
                                           int(prod["t_end"].max())) * us
    return out
